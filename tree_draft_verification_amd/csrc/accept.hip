// Greedy longest-accepted-path selection plus the bonus token: one 64-lane
// wavefront per sequence runs accept_sequence (accept_core.h, which states
// the rule and the pointer-jumping scheme).
#include "accept_core.h"

namespace tv {
namespace {

constexpr int kWave = 64;

__global__ __launch_bounds__(kWave) void accept_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ tgt, int32_t* __restrict__ path,
    int32_t* __restrict__ path_len, int32_t* __restrict__ bonus, int N, int P,
    int32_t* __restrict__ dev_status) {
  __shared__ AcceptLds s;
  const int b = blockIdx.x;
  accept_sequence<kWave>(s, parent + (size_t)b * N, draft + (size_t)b * N, tgt + (size_t)b * N,
                         N, P);
  accept_write<kWave>(s, b, P, path, path_len, bonus, dev_status);
}

}  // namespace

hipError_t launch_tree_accept(const int32_t* parent, const int32_t* draft,
                              const int32_t* tgt, int32_t* path, int32_t* path_len,
                              int32_t* bonus, int B, int N, int P,
                              int32_t* dev_status, hipStream_t stream) {
  hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(kWave), 0, stream, parent, draft,
                     tgt, path, path_len, bonus, N, P, dev_status);
  return hipGetLastError();
}

}  // namespace tv
