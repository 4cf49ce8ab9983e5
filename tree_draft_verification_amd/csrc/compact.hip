// KV compaction: commit the accepted path into contiguous cache rows.
//
// After verification, sequence b keeps the K/V of its accepted nodes only,
// right after its own prefix: row L_b + j takes row L_b + path[j] for
// j < path_len, and L_b grows by path_len.  Each sequence of a ragged batch
// uses its own offset (EQSPEC/EXSPEC abstract, arXiv 2510.22876 on the RSS
// reader page: ragged acceptance must keep every sequence's KV state in step).
//
// Caches are contiguous planes [B][Hkv][Lcap][row] or pages of a pool
// [num_pages][Hkv][page_size][row] named by a block table (row r of sequence
// b in page block_table[b][r / page_size]); the moves are the same.
//
// One workgroup per sequence handles every plane (K and V of every KV head)
// and then updates that sequence's length itself, so one launch does the
// whole commit.  For the caches of every layer of a model ([layers][B][Hkv]
// [Lcap][row]), the planes of all layers are shared out among several
// workgroups per sequence; the last to finish updates the length.
//
// In-place hazard: the row a move reads can be another move's destination
// (path[j] == j' for a moved j'), only inside a plane.  An accepted path is
// increasing with path[j] >= j, so the serial order in increasing j reads
// every such row before overwriting it; the workgroup does the same by
// loading all moved rows of whole planes into registers (at most 64 KB per
// round), waiting at a barrier and only then writing.  Rows with
// path[j] == j are skipped.  Accesses are 16-byte vectors, consecutive
// threads on consecutive 16-byte pieces of a row, a thread's pieces of a
// round all in flight together.
//
// Fused with acceptance (ACCEPT): each workgroup first selects its sequence's
// accepted path itself (accept_core.h; a few LDS rounds over the tree, so
// the workgroups of one sequence need not wait for each other), workgroup 0
// of the sequence writes path, path_len and bonus, and the moves use the
// path from LDS: one launch instead of two.
#include <type_traits>

#include "accept_core.h"

namespace tv {
namespace {

constexpr int kThreads = 1024;
// s_waitcnt operand: vmcnt(0), expcnt and lgkmcnt left at their maxima
// (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kPer = 4;  // 16-byte pieces a thread holds per round (64 KB a workgroup)

struct PagedArgs {
  const int32_t* block_table;  // nullptr: contiguous planes
  int max_blocks, page_shift, num_pages;
};

struct AcceptArgs {  // inputs and outputs of the fused acceptance
  const int32_t* parent;
  const int32_t* draft;
  const int32_t* target;
  int32_t* bonus;
  int32_t* dev_status;
  int N;
};

// n / d for n * d < 2^32: one multiply-high by m = ceil(2^32 / d)
struct FastDiv {
  unsigned d, m;
};
__device__ __forceinline__ FastDiv make_fastdiv(unsigned d) {
  return {d, d == 1u ? 0u : 0xffffffffu / d + 1u};
}
__device__ __forceinline__ unsigned fast_div(unsigned n, FastDiv f) {
  return f.d == 1u ? n : __umulhi(n, f.m);
}

// Byte offset of row `row` of sequence b in KV head 0 of a cache plane set
// (head h adds h * head_stride), or -1 when a paged entry is outside the
// pool.
template <bool PAGED>
__device__ __forceinline__ long long row_part(const PagedArgs& pa, int b, int Hkv, int Lcap,
                                              int row, int row_bytes) {
  if constexpr (PAGED) {
    const int pg = pa.block_table[(size_t)b * pa.max_blocks + (row >> pa.page_shift)];
    if (pg < 0 || pg >= pa.num_pages) return -1;
    return (((long long)pg * Hkv << pa.page_shift) + (row & ((1 << pa.page_shift) - 1))) *
           row_bytes;
  } else {
    return ((long long)b * Hkv * Lcap + row) * row_bytes;
  }
}

template <bool PAGED, bool ACCEPT>
__global__ __launch_bounds__(kThreads, (PAGED || ACCEPT) ? 4 : 8) void compact_kernel(
    char* __restrict__ kc, char* __restrict__ vc, int32_t* __restrict__ seq_lens,
    int32_t* __restrict__ path, int32_t* __restrict__ path_len, int Hkv, int Lcap,
    int P, int row_bytes, PagedArgs pa, int layers, long long layer_bytes, int groups,
    unsigned* __restrict__ counters, AcceptArgs ac) {
  __shared__ long long s_src[64];  // row parts (head 0) of every move's source
  __shared__ long long s_dst[64];  // and destination, in increasing j
  __shared__ int s_nmove;
  __shared__ int s_last;
  struct NoAccept {};
  __shared__ std::conditional_t<ACCEPT, AcceptLds, NoAccept> s_acc;
  const int b = blockIdx.x / groups;
  const int grp = blockIdx.x - b * groups;
  const int tid = threadIdx.x;
  const int L = seq_lens[b];
  int n;
  int src = -1;  // path entry of lane tid (wavefront 0)
  if constexpr (ACCEPT) {
    // one wavefront selects the path (its LDS rounds need no workgroup
    // barriers); the workgroup waits once for the result
    const size_t r = (size_t)b * ac.N;
    if (tid < 64) accept_sequence<64>(s_acc, ac.parent + r, ac.draft + r, ac.target + r, ac.N, P);
    __syncthreads();
    if (grp == 0) accept_write<kThreads>(s_acc, b, P, path, path_len, ac.bonus, ac.dev_status);
    n = s_acc.res[0];
    if (tid < n) src = s_acc.path[tid];
  } else {
    // the path is read together with the lengths (P <= 64 entries)
    if (tid < P) src = path[(size_t)b * P + tid];
    n = path_len[b];
    n = n < 0 ? 0 : (n > P ? P : n);
  }
  // caller contract broken: touch nothing (the length is left as it was);
  // every workgroup of the sequence takes this branch together
  if (L < 0 || L + n > Lcap) return;
  // The rows that move, in increasing j: wavefront 0 locates both rows of
  // every move (a paged move whose source or destination page is outside
  // the pool is dropped) and ranks the moves with a ballot.
  if (tid < 64) {
    bool mv = tid < n && src != tid && src >= 0 && L + src < Lcap;
    long long ps = 0, pd = 0;
    if (mv) {
      ps = row_part<PAGED>(pa, b, Hkv, Lcap, L + src, row_bytes);
      pd = row_part<PAGED>(pa, b, Hkv, Lcap, L + tid, row_bytes);
      mv = ps >= 0 && pd >= 0;
    }
    const unsigned long long bal = __ballot(mv);
    if (mv) {
      const int pos = __popcll(bal & ((1ull << tid) - 1ull));
      s_src[pos] = ps;
      s_dst[pos] = pd;
    }
    if (tid == 0) s_nmove = __popcll(bal);
  }
  __syncthreads();
  const int m = s_nmove;
  const int chunks = row_bytes / 16;
  const int per_plane = m * chunks;  // pieces per plane
  const long long head_stride =
      PAGED ? (long long)row_bytes << pa.page_shift : (long long)Lcap * row_bytes;
  // planes (layer, K|V, head) of all layers, shared out among the groups
  const int planes_all = 2 * Hkv * layers;
  const int pb = (int)((long long)grp * planes_all / groups);
  const int pe = (int)((long long)(grp + 1) * planes_all / groups);
  if (per_plane > 0) {
    // a round takes whole planes, at most kPer pieces per thread; the
    // quotients below stay exact (pieces < 2^12 per round, and the host
    // bounds planes_all * 2 * Hkv below 2^32)
    const int group = kPer * kThreads / per_plane;  // >= 1: P * row_bytes <= 64 KB
    const FastDiv div_pp = make_fastdiv(per_plane);
    const FastDiv div_ch = make_fastdiv(chunks);
    const FastDiv div_kv = make_fastdiv(2 * Hkv);
    for (int p0 = pb; p0 < pe; p0 += group) {
      const int items = min(group, pe - p0) * per_plane;
      u32x4_t val[kPer];
      char* dst[kPer];
      // straight-line loads, all in flight together (a thread past the end
      // reloads the last piece and writes nothing)
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int it = min(tid + q * kThreads, items - 1);
        const int pl = (int)fast_div(it, div_pp);
        const int rem = it - pl * per_plane;
        const int k = (int)fast_div(rem, div_ch);
        const int x = rem - k * chunks;
        const int p = p0 + pl;
        const int ly = (int)fast_div(p, div_kv);
        const int qh = p - ly * 2 * Hkv;
        const int h = qh < Hkv ? qh : qh - Hkv;
        char* base = (qh < Hkv ? kc : vc) + ly * layer_bytes + h * head_stride + 16 * x;
        val[q] = *reinterpret_cast<const u32x4_t*>(base + s_src[k]);
        dst[q] = tid + q * kThreads < items ? base + s_dst[k] : nullptr;
      }
      // every read of these planes has returned before any write: each
      // thread waits for its own loads, then the barrier; the next round's
      // planes are others, so no barrier follows the writes
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        if (dst[q] != nullptr) *reinterpret_cast<u32x4_t*>(dst[q]) = val[q];
    }
  }
  // The new length: every workgroup of the sequence has read L (before its
  // barriers above).  With one workgroup it writes directly; otherwise the
  // last one to arrive at the counter writes it and clears the counter.  The
  // counter's return value orders the arrivals; no data passes through it.
  if (groups == 1) {
    if (tid == 0) seq_lens[b] = L + n;
    return;
  }
  if (tid == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(&counters[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)groups - 1u;
    if (s_last) {
      seq_lens[b] = L + n;
      __hip_atomic_store(&counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Commit on a slot table (one row per page): the tree window of the table
// is permuted, no row moves.  One workgroup per sequence, thread i for tree
// node i: node path[j] goes to position j, a rejected node i to path_len +
// (i minus the accepted nodes below i), counted by a binary search of the
// increasing path.  Every entry of the window is read before the barrier and
// written after it, so the in-place permutation needs no staging beyond one
// register per thread.
__global__ __launch_bounds__(TV_MAX_NODES) void commit_slots_kernel(
    int32_t* __restrict__ table, int32_t* __restrict__ seq_lens, const int32_t* __restrict__ path,
    const int32_t* __restrict__ path_len, int N, int P, int max_blocks,
    int32_t* __restrict__ dev_status) {
  __shared__ int s_path[64];
  __shared__ int s_bad;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = seq_lens[b];
  int n = path_len[b];
  n = n < 0 ? 0 : (n > P ? P : n);
  n = n > N ? N : n;
  if (L < 0 || (long long)L + N > max_blocks) {
    if (tid == 0 && dev_status != nullptr) atomicOr(&dev_status[b], TV_STATUS_BAD_LEN);
    return;
  }
  if (tid < 64) {
    // the path is increasing within [0, N): each entry checks itself and its
    // predecessor (from the lane below)
    const int pj = tid < n ? path[(size_t)b * P + tid] : 0x7fffffff;
    const int prev = __shfl_up(pj, 1, 64);
    const bool bad = tid < n && (pj < 0 || pj >= N || (tid > 0 && prev >= pj));
    const unsigned long long any_bad = __ballot(bad);
    s_path[tid] = pj;
    if (tid == 0) s_bad = any_bad != 0ull;
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0 && dev_status != nullptr) atomicOr(&dev_status[b], TV_STATUS_BAD_PATH);
    return;
  }
  int32_t* win = table + (size_t)b * max_blocks + L;
  int slot = 0, dest = 0;
  if (tid < N) {
    slot = win[tid];
    // accepted nodes below tid: entries of the increasing path that are < tid
    int lo = 0, hi = n;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_path[mid] < tid) lo = mid + 1;
      else hi = mid;
    }
    dest = (lo < n && s_path[lo] == tid) ? lo : n + (tid - lo);
  }
  // every entry of the window has been read (each thread waits for its own
  // load, then the barrier) before any is written
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (tid < N) win[dest] = slot;
  if (tid == 0) seq_lens[b] = L + n;
}

}  // namespace

hipError_t launch_kv_compact(void* k, void* v, int32_t* seq_lens, const int32_t* path,
                             const int32_t* path_len, int B, int Hkv, int D, int Lcap, int P,
                             int dtype, hipStream_t stream, const int32_t* block_table,
                             int max_blocks, int page_size, int num_pages) {
  const int row_bytes = D * (dtype == TV_F32 ? 4 : 2);
  PagedArgs pa{block_table, max_blocks, 0, num_pages};
  if (block_table != nullptr) {
    while ((1 << pa.page_shift) < page_size) ++pa.page_shift;
    Lcap = max_blocks << pa.page_shift;
    hipLaunchKernelGGL((compact_kernel<true, false>), dim3(B), dim3(kThreads), 0, stream,
                       static_cast<char*>(k), static_cast<char*>(v), seq_lens,
                       const_cast<int32_t*>(path), const_cast<int32_t*>(path_len), Hkv, Lcap, P,
                       row_bytes, pa, 1, 0LL, 1, nullptr, AcceptArgs{});
  } else {
    hipLaunchKernelGGL((compact_kernel<false, false>), dim3(B), dim3(kThreads), 0, stream,
                       static_cast<char*>(k), static_cast<char*>(v), seq_lens,
                       const_cast<int32_t*>(path), const_cast<int32_t*>(path_len), Hkv, Lcap, P,
                       row_bytes, pa, 1, 0LL, 1, nullptr, AcceptArgs{});
  }
  return hipGetLastError();
}

// Every layer in one launch: about eight planes per workgroup, at most 512
// workgroups in all (two 1024-thread workgroups fit a compute unit, so the
// grid is resident at once on 256 units and no workgroup waits for a slot).
hipError_t launch_kv_compact_layers(void* k, void* v, int32_t* seq_lens, const int32_t* path,
                                    const int32_t* path_len, int B, int Hkv, int D, int Lcap,
                                    int P, int layers, int dtype, unsigned* counters,
                                    hipStream_t stream) {
  const int row_bytes = D * (dtype == TV_F32 ? 4 : 2);
  const long long layer_bytes = (long long)B * Hkv * Lcap * row_bytes;
  const int planes = 2 * Hkv * layers;
  int groups = (planes + 7) / 8;
  const int cap = 512 / B > 1 ? 512 / B : 1;
  if (groups > cap) groups = cap;
  if (groups < 1) groups = 1;
  PagedArgs pa{nullptr, 0, 0, 0};
  hipLaunchKernelGGL((compact_kernel<false, false>), dim3(B * groups), dim3(kThreads), 0, stream,
                     static_cast<char*>(k), static_cast<char*>(v), seq_lens,
                     const_cast<int32_t*>(path), const_cast<int32_t*>(path_len), Hkv, Lcap, P,
                     row_bytes, pa, layers, layer_bytes, groups, counters, AcceptArgs{});
  return hipGetLastError();
}

// Acceptance and the compaction of a single-layer contiguous cache in one
// launch: one workgroup per sequence.
hipError_t launch_accept_compact(const int32_t* parent, const int32_t* draft,
                                 const int32_t* target, int32_t* path, int32_t* path_len,
                                 int32_t* bonus, void* k, void* v, int32_t* seq_lens, int B,
                                 int N, int P, int Hkv, int D, int Lcap, int dtype,
                                 int32_t* dev_status, hipStream_t stream) {
  const int row_bytes = D * (dtype == TV_F32 ? 4 : 2);
  PagedArgs pa{nullptr, 0, 0, 0};
  AcceptArgs ac{parent, draft, target, bonus, dev_status, N};
  hipLaunchKernelGGL((compact_kernel<false, true>), dim3(B), dim3(kThreads), 0, stream,
                     static_cast<char*>(k), static_cast<char*>(v), seq_lens, path, path_len, Hkv,
                     Lcap, P, row_bytes, pa, 1, 0LL, 1, nullptr, ac);
  return hipGetLastError();
}

hipError_t launch_kv_commit_slots(int32_t* block_table, int32_t* seq_lens, const int32_t* path,
                                  const int32_t* path_len, int B, int N, int P, int max_blocks,
                                  int32_t* dev_status, hipStream_t stream) {
  hipLaunchKernelGGL(commit_slots_kernel, dim3(B), dim3(TV_MAX_NODES), 0, stream, block_table,
                     seq_lens, path, path_len, N, P, max_blocks, dev_status);
  return hipGetLastError();
}

}  // namespace tv
