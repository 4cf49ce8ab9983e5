// Greedy longest-accepted-path selection plus the bonus token.
//
// Rule (JetSpec GitHub README, "JetSpec > Overview": the accepted path is
// chosen from the target's own logits, lossless by construction): node i >= 1
// is accepted when its parent is accepted and its draft token equals the
// target's greedy token at the parent; the emitted path runs from the root to
// the deepest accepted node (smallest index on ties), and the bonus token is
// the target's greedy token at that node.
//
// One 64-lane wavefront per sequence.  "Accepted" is an AND along the root
// path and the depth is a sum along it, so both come from pointer jumping
// over the parent array in LDS: after round r each node has folded in the
// 2^r nearest ancestors' values, so ceil(log2(depth)) rounds finish a tree
// (at most 10 for 1024 nodes) instead of a serial scan over N nodes.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kWave = 64;

__device__ __forceinline__ int wave_max_int(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off, kWave));
  return x;
}

__global__ __launch_bounds__(kWave) void accept_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ tgt, int32_t* __restrict__ path,
    int32_t* __restrict__ path_len, int32_t* __restrict__ bonus, int N, int P,
    int32_t* __restrict__ dev_status) {
  __shared__ int16_t s_ptr[2][TV_MAX_NODES];
  __shared__ int16_t s_dep[2][TV_MAX_NODES];
  __shared__ uint8_t s_ok[2][TV_MAX_NODES];
  __shared__ int16_t s_par[TV_MAX_NODES];

  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int32_t* par = parent + (size_t)b * N;
  const int32_t* dr = draft + (size_t)b * N;
  const int32_t* tg = tgt + (size_t)b * N;

  // Initial values: ptr = parent, ok = own match, dep = 1 (root: 0, 1, 0).
  int bad = 0;
  for (int i = lane; i < N; i += kWave) {
    const int p = par[i];
    int ptr = 0, ok = 1, dep = 0;
    if (i == 0) {
      bad |= (p != -1);
    } else {
      const bool valid = (p >= 0) && (p < i);
      bad |= !valid;
      ptr = valid ? p : 0;
      ok = valid && (dr[i] == tg[ptr]);
      dep = 1;
    }
    s_par[i] = (int16_t)ptr;
    s_ptr[0][i] = (int16_t)ptr;
    s_dep[0][i] = (int16_t)dep;
    s_ok[0][i] = (uint8_t)ok;
  }
  bad = wave_max_int(bad);
  __syncthreads();

  int cur = 0;
  for (int round = 0; round < 11; ++round) {
    const int nxt = cur ^ 1;
    int active = 0;
    for (int i = lane; i < N; i += kWave) {
      const int q = s_ptr[cur][i];
      const int np = s_ptr[cur][q];
      s_ok[nxt][i] = s_ok[cur][i] & s_ok[cur][q];
      s_dep[nxt][i] = (int16_t)(s_dep[cur][i] + s_dep[cur][q]);
      s_ptr[nxt][i] = (int16_t)np;
      active |= (np != 0);
    }
    __syncthreads();
    cur = nxt;
    if (wave_max_int(active) == 0) break;
  }

  // Deepest accepted node, smallest index on ties: maximise (dep, -index).
  int key = -1;
  for (int i = lane; i < N; i += kWave) {
    if (s_ok[cur][i]) key = max(key, (int)s_dep[cur][i] * 65536 + (65535 - i));
  }
  key = wave_max_int(key);  // the root is always accepted, so key >= 0
  const int best = 65535 - (key & 0xffff);
  const int depth = key >> 16;
  const bool too_deep = depth + 1 > P;

  int32_t* pth = path + (size_t)b * P;
  if (bad || too_deep) {
    for (int j = lane; j < P; j += kWave) pth[j] = -1;
    if (lane == 0) {
      path_len[b] = 0;
      bonus[b] = -1;
      if (dev_status) atomicOr(&dev_status[b], bad ? TV_STATUS_BAD_PARENT : TV_STATUS_DEPTH);
    }
    return;
  }
  for (int j = depth + 1 + lane; j < P; j += kWave) pth[j] = -1;
  if (lane == 0) {
    int node = best;
    for (int t = depth; t >= 0; --t) {
      pth[t] = node;
      node = s_par[node];
    }
    path_len[b] = depth + 1;
    bonus[b] = tg[best];
  }
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
