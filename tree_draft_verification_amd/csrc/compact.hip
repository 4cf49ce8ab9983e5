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
// whole commit.  In-place hazard: move j reads row L+path[j], which move
// j' < j may be writing when path[j] == j'; the hazard exists only inside a
// plane.  The workgroup therefore stages whole planes - all moved rows of a
// group of planes - in LDS, waits at a barrier and only then writes.  Rows
// with path[j] == j are skipped.  Accesses are 16-byte vectors, consecutive
// threads on consecutive 16-byte pieces of a row.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 1024;
constexpr int kStageBytes = 64 * 1024;  // LDS staging per workgroup

struct PagedArgs {
  const int32_t* block_table;  // nullptr: contiguous planes
  int max_blocks, page_shift, num_pages;
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

template <bool PAGED>
__global__ __launch_bounds__(kThreads) void compact_kernel(
    char* __restrict__ kc, char* __restrict__ vc, int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ path, const int32_t* __restrict__ path_len, int Hkv, int Lcap,
    int P, int row_bytes, PagedArgs pa) {
  __shared__ uint4 stage[kStageBytes / 16];
  __shared__ int16_t s_move[64];  // j of every row that moves
  __shared__ int s_nmove;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = seq_lens[b];
  int n = path_len[b];
  n = n < 0 ? 0 : (n > P ? P : n);
  // caller contract broken: touch nothing (the length is left as it was)
  if (L < 0 || L + n > Lcap) return;
  const int32_t* pth = path + (size_t)b * P;
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
  const int planes = 2 * Hkv;
  if (per_plane > 0) {
    const int group = (kStageBytes / 16) / per_plane;  // >= 1: P * row_bytes <= 64 KB
    for (int p0 = 0; p0 < planes; p0 += group) {
      const int pn = min(group, planes - p0);
      const int items = pn * per_plane;
      for (int it = tid; it < items; it += kThreads) {
        const int p = p0 + it / per_plane;
        const int rem = it - (it / per_plane) * per_plane;
        const int k = rem / chunks;
        const int x = rem - k * chunks;
        const int j = s_move[k];
        const long long off =
            row_offset<PAGED>(pa, b, p < Hkv ? p : p - Hkv, Hkv, Lcap, L + pth[j], row_bytes);
        if (off >= 0)
          stage[it] = reinterpret_cast<const uint4*>((p < Hkv ? kc : vc) + off)[x];
      }
      __syncthreads();
      for (int it = tid; it < items; it += kThreads) {
        const int p = p0 + it / per_plane;
        const int rem = it - (it / per_plane) * per_plane;
        const int k = rem / chunks;
        const int x = rem - k * chunks;
        const int j = s_move[k];
        const int h = p < Hkv ? p : p - Hkv;
        const long long src = row_offset<PAGED>(pa, b, h, Hkv, Lcap, L + pth[j], row_bytes);
        const long long off = row_offset<PAGED>(pa, b, h, Hkv, Lcap, L + j, row_bytes);
        if (off >= 0 && src >= 0)
          reinterpret_cast<uint4*>((p < Hkv ? kc : vc) + off)[x] = stage[it];
      }
      __syncthreads();
    }
  }
  if (tid == 0) seq_lens[b] = L + n;  // every thread read L before the barriers above
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
    hipLaunchKernelGGL(compact_kernel<true>, dim3(B), dim3(kThreads), 0, stream,
                       static_cast<char*>(k), static_cast<char*>(v), seq_lens, path, path_len,
                       Hkv, Lcap, P, row_bytes, pa);
  } else {
    hipLaunchKernelGGL(compact_kernel<false>, dim3(B), dim3(kThreads), 0, stream,
                       static_cast<char*>(k), static_cast<char*>(v), seq_lens, path, path_len,
                       Hkv, Lcap, P, row_bytes, pa);
  }
  return hipGetLastError();
}

}  // namespace tv
