// KV compaction: commit the accepted path into contiguous cache rows.
//
// After verification, sequence b keeps the K/V of its accepted nodes only,
// right after its own prefix: row L_b + j takes row L_b + path[j] for
// j < path_len, and L_b grows by path_len.  Each sequence of a ragged batch
// uses its own offset (EQSPEC/EXSPEC abstract, arXiv 2510.22876 on the RSS
// reader page: ragged acceptance must keep every sequence's KV state in step).
//
// In-place hazard: move j reads row L+path[j], which a parallel move j' < j
// may be writing when path[j] == j'.  Each workgroup owns one (sequence,
// head, K-or-V) plane, loads every moved row into LDS, waits at a barrier and
// only then writes, so the result equals the serial order.  The loads and
// stores are 16-byte vector accesses, consecutive threads on consecutive
// 16-byte pieces of a row.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void compact_kernel(
    char* __restrict__ kc, char* __restrict__ vc, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ path, const int32_t* __restrict__ path_len, int Hkv,
    int Lcap, int P, int row_bytes) {
  extern __shared__ uint4 stage[];  // [P][row_bytes / 16]
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  char* plane = (blockIdx.z ? vc : kc) + ((size_t)b * Hkv + h) * (size_t)Lcap * row_bytes;
  const int L = seq_lens[b];
  int n = path_len[b];
  n = n < 0 ? 0 : (n > P ? P : n);
  if (L < 0 || L + n > Lcap) return;  // caller contract broken: touch nothing
  const int32_t* pth = path + (size_t)b * P;
  const int chunks = row_bytes / 16;
  const int total = n * chunks;

  for (int c = threadIdx.x; c < total; c += kThreads) {
    const int j = c / chunks;
    const int x = c - j * chunks;
    const int src = pth[j];
    if (src != j && src >= 0 && L + src < Lcap)
      stage[c] = reinterpret_cast<const uint4*>(plane + (size_t)(L + src) * row_bytes)[x];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < total; c += kThreads) {
    const int j = c / chunks;
    const int x = c - j * chunks;
    const int src = pth[j];
    if (src != j && src >= 0 && L + src < Lcap)
      reinterpret_cast<uint4*>(plane + (size_t)(L + j) * row_bytes)[x] = stage[c];
  }
}

// Runs after every plane of the batch has read the old lengths.
__global__ void seqlen_kernel(int32_t* __restrict__ seq_lens,
                              const int32_t* __restrict__ path_len, int B, int P) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) {
    int n = path_len[b];
    n = n < 0 ? 0 : (n > P ? P : n);
    seq_lens[b] += n;
  }
}

}  // namespace

hipError_t launch_kv_compact(void* k, void* v, int32_t* seq_lens, const int32_t* path,
                             const int32_t* path_len, int B, int Hkv, int D, int Lcap,
                             int P, int dtype, hipStream_t stream) {
  const int row_bytes = D * (dtype == TV_F32 ? 4 : 2);
  const size_t lds = (size_t)P * row_bytes;
  hipLaunchKernelGGL(compact_kernel, dim3(Hkv, B, 2), dim3(kThreads), lds, stream,
                     static_cast<char*>(k), static_cast<char*>(v), seq_lens, path,
                     path_len, Hkv, Lcap, P, row_bytes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(seqlen_kernel, dim3((B + 255) / 256), dim3(256), 0, stream,
                     seq_lens, path_len, B, P);
  return hipGetLastError();
}

}  // namespace tv
