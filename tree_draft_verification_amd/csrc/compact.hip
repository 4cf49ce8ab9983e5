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
// In-place hazard: move j reads row L+path[j], which move j' < j may be
// writing when path[j] == j'; the hazard exists only inside a plane.  The workgroup therefore stages whole planes - all moved rows of a
// group of planes - in LDS, waits at a barrier and only then writes.  Rows
// with path[j] == j are skipped.  Accesses are 16-byte vectors, consecutive
// threads on consecutive 16-byte pieces of a row.
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
constexpr int kStageBytes = 64 * 1024;  // LDS staging per workgroup

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

// Byte offset of row `row` of plane (b, head) in a cache, or -1 when a
// paged entry is outside the pool.
template <bool PAGED>
__device__ __forceinline__ long long row_offset(const PagedArgs& pa, int b, int head, int Hkv,
                                                int Lcap, int row, int row_bytes) {
  if constexpr (PAGED) {
    const int pg = pa.block_table[(size_t)b * pa.max_blocks + (row >> pa.page_shift)];
    if (pg < 0 || pg >= pa.num_pages) return -1;
    return ((((long long)pg * Hkv + head) << pa.page_shift) + (row & ((1 << pa.page_shift) - 1))) *
           row_bytes;
  } else {
    return (((long long)b * Hkv + head) * Lcap + row) * row_bytes;
  }
}

template <bool PAGED, bool ACCEPT>
__global__ __launch_bounds__(kThreads) void compact_kernel(
    char* __restrict__ kc, char* __restrict__ vc, int32_t* __restrict__ seq_lens,
    int32_t* __restrict__ path, int32_t* __restrict__ path_len, int Hkv, int Lcap,
    int P, int row_bytes, PagedArgs pa, int layers, long long layer_bytes, int groups,
    unsigned* __restrict__ counters, AcceptArgs ac) {
  __shared__ uint4 stage[kStageBytes / 16];
  __shared__ int16_t s_move[64];  // j of every row that moves
  __shared__ int s_nmove;
  __shared__ int s_last;
  struct NoAccept {};
  __shared__ std::conditional_t<ACCEPT, AcceptLds, NoAccept> s_acc;
  const int b = blockIdx.x / groups;
  const int grp = blockIdx.x - b * groups;
  const int tid = threadIdx.x;
  const int L = seq_lens[b];
  int n;
  const int* pth;
  if constexpr (ACCEPT) {
    // one wavefront selects the path (its LDS rounds need no workgroup
    // barriers); the workgroup waits once for the result
    const size_t r = (size_t)b * ac.N;
    if (tid < 64) accept_sequence<64>(s_acc, ac.parent + r, ac.draft + r, ac.target + r, ac.N, P);
    __syncthreads();
    if (grp == 0) accept_write<kThreads>(s_acc, b, P, path, path_len, ac.bonus, ac.dev_status);
    n = s_acc.res[0];
    pth = s_acc.path;
  } else {
    n = path_len[b];
    n = n < 0 ? 0 : (n > P ? P : n);
    pth = path + (size_t)b * P;
  }
  // caller contract broken: touch nothing (the length is left as it was);
  // every workgroup of the sequence takes this branch together
  if (L < 0 || L + n > Lcap) return;
  if (tid == 0) {
    int m = 0;
    for (int j = 0; j < n; ++j) {
      const int src = pth[j];
      if (src != j && src >= 0 && L + src < Lcap) s_move[m++] = (int16_t)j;
    }
    s_nmove = m;
  }
  __syncthreads();
  const int m = s_nmove;
  const int chunks = row_bytes / 16;
  const int per_plane = m * chunks;  // staged pieces per plane
  // planes (layer, K|V, head) of all layers, shared out among the groups
  const int planes_all = 2 * Hkv * layers;
  const int pb = (int)((long long)grp * planes_all / groups);
  const int pe = (int)((long long)(grp + 1) * planes_all / groups);
  auto plane_base = [&](int p, int& h) -> char* {
    const int ly = p / (2 * Hkv);
    const int q = p - ly * 2 * Hkv;
    h = q < Hkv ? q : q - Hkv;
    return (q < Hkv ? kc : vc) + (long long)ly * layer_bytes;
  };
  if (per_plane > 0) {
    const int group = (kStageBytes / 16) / per_plane;  // >= 1: P * row_bytes <= 64 KB
    for (int p0 = pb; p0 < pe; p0 += group) {
      const int pn = min(group, pe - p0);
      const int items = pn * per_plane;
      for (int it = tid; it < items; it += kThreads) {
        const int p = p0 + it / per_plane;
        const int rem = it - (it / per_plane) * per_plane;
        const int k = rem / chunks;
        const int x = rem - k * chunks;
        const int j = s_move[k];
        int h;
        const char* base = plane_base(p, h);
        const long long off = row_offset<PAGED>(pa, b, h, Hkv, Lcap, L + pth[j], row_bytes);
        if (off >= 0) stage[it] = reinterpret_cast<const uint4*>(base + off)[x];
      }
      __syncthreads();
      for (int it = tid; it < items; it += kThreads) {
        const int p = p0 + it / per_plane;
        const int rem = it - (it / per_plane) * per_plane;
        const int k = rem / chunks;
        const int x = rem - k * chunks;
        const int j = s_move[k];
        int h;
        char* base = plane_base(p, h);
        const long long src = row_offset<PAGED>(pa, b, h, Hkv, Lcap, L + pth[j], row_bytes);
        const long long off = row_offset<PAGED>(pa, b, h, Hkv, Lcap, L + j, row_bytes);
        if (off >= 0 && src >= 0) reinterpret_cast<uint4*>(base + off)[x] = stage[it];
      }
      __syncthreads();
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

// Every layer in one launch: about eight planes per workgroup, at most 1024
// workgroups in all.
hipError_t launch_kv_compact_layers(void* k, void* v, int32_t* seq_lens, const int32_t* path,
                                    const int32_t* path_len, int B, int Hkv, int D, int Lcap,
                                    int P, int layers, int dtype, unsigned* counters,
                                    hipStream_t stream) {
  const int row_bytes = D * (dtype == TV_F32 ? 4 : 2);
  const long long layer_bytes = (long long)B * Hkv * Lcap * row_bytes;
  const int planes = 2 * Hkv * layers;
  int groups = (planes + 7) / 8;
  const int cap = 1024 / B > 1 ? 1024 / B : 1;
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

}  // namespace tv
