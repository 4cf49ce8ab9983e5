// Greedy longest-accepted-path selection for one sequence, computed by NT
// threads of the calling workgroup (shared by accept_kernel and the fused
// acceptance + compaction kernel).
//
// Rule (JetSpec GitHub README, "JetSpec > Overview": the accepted path is
// chosen from the target's own logits, lossless by construction): node i >= 1
// is accepted when its parent is accepted and its draft token equals the
// target's greedy token at the parent; the emitted path runs from the root to
// the deepest accepted node (smallest index on ties), and the bonus token is
// the target's greedy token at that node.
//
// "Accepted" is an AND along the root path and the depth is a sum along it,
// so both come from pointer jumping over the parent array in LDS: after
// round r each node has folded in the 2^r nearest ancestors' values, so
// ceil(log2(depth)) rounds finish a tree (at most 10 for 1024 nodes) instead
// of a serial scan over N nodes.
#pragma once

#include "tv_internal.h"

namespace tv {

struct AcceptLds {
  int16_t ptr[2][TV_MAX_NODES];
  int16_t dep[2][TV_MAX_NODES];
  uint8_t ok[2][TV_MAX_NODES];
  int16_t par[TV_MAX_NODES];
  int red[16];     // one slot per wavefront (NT <= 1024)
  int path[64];    // the accepted path (P <= 64)
  int res[3];      // path length (0: rejected), bonus, status flags
};

__device__ __forceinline__ int accept_wave_max(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off, 64));
  return x;
}

// Phase boundary among the NT threads that run accept_sequence: a
// workgroup barrier, or for one wavefront (NT == 64) only an LDS fence (a
// wavefront's LDS accesses are performed in order), so one wavefront of a
// larger workgroup can run it alone.
template <int NT>
__device__ __forceinline__ int accept_sync_or(int x) {
  if constexpr (NT == 64) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return __any(x) ? 1 : 0;
  } else {
    return __syncthreads_or(x);
  }
}

// Fills s.res (and s.path[0 .. length-1]) for sequence rows par/dr/tg of N
// nodes with at most P path entries.  Threads 0 .. NT-1 of the workgroup call
// it (NT == 64: one wavefront, which may be part of a larger workgroup); the
// results are visible to them on return (to the rest of a larger workgroup
// after its next barrier).
template <int NT>
__device__ void accept_sequence(AcceptLds& s, const int32_t* __restrict__ par,
                                const int32_t* __restrict__ dr, const int32_t* __restrict__ tg,
                                int N, int P) {
  const int tid = threadIdx.x;
  // initial values: ptr = parent, ok = own match, dep = 1 (root: 0, 1, 0).
  // Every thread's parent and draft loads go out together, then every
  // target load at those parents (clamped addresses, no branch around a
  // load): two memory latencies per thread, not two per node.
  constexpr int kPer = (TV_MAX_NODES + NT - 1) / NT;
  int pv[kPer], dv[kPer], tv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = min(tid + u * NT, N - 1);
    pv[u] = par[i];
    dv[u] = dr[i];
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) tv[u] = tg[min(max(pv[u], 0), N - 1)];
  int bad = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + u * NT;
    if (i >= N) break;
    const int p = pv[u];
    int ptr = 0, ok = 1, dep = 0;
    if (i == 0) {
      bad |= (p != -1);
    } else {
      const bool valid = (p >= 0) && (p < i);
      bad |= !valid;
      ptr = valid ? p : 0;
      ok = valid && (dv[u] == tv[u]);
      dep = 1;
    }
    s.par[i] = (int16_t)ptr;
    s.ptr[0][i] = (int16_t)ptr;
    s.dep[0][i] = (int16_t)dep;
    s.ok[0][i] = (uint8_t)ok;
  }
  bad = accept_sync_or<NT>(bad);

  int cur = 0;
  for (int round = 0; round < 11; ++round) {
    const int nxt = cur ^ 1;
    int active = 0;
    // the nodes of a thread are independent: unrolled, their LDS reads
    // overlap instead of costing two round trips each
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * NT;
      if (i >= N) break;
      const int q = s.ptr[cur][i];
      const int np = s.ptr[cur][q];
      s.ok[nxt][i] = s.ok[cur][i] & s.ok[cur][q];
      s.dep[nxt][i] = (int16_t)(s.dep[cur][i] + s.dep[cur][q]);
      s.ptr[nxt][i] = (int16_t)np;
      active |= (np != 0);
    }
    cur = nxt;
    if (accept_sync_or<NT>(active) == 0) break;
  }

  // deepest accepted node, smallest index on ties: maximise (dep, -index)
  int key = -1;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + u * NT;
    if (i >= N) break;
    if (s.ok[cur][i]) key = max(key, (int)s.dep[cur][i] * 65536 + (65535 - i));
  }
  key = accept_wave_max(key);
  if constexpr (NT > 64) {
    if ((tid & 63) == 0) s.red[tid >> 6] = key;
    __syncthreads();
    key = s.red[0];
    for (int w = 1; w < NT / 64; ++w) key = max(key, s.red[w]);
  }
  // the root is always accepted, so key >= 0
  const int best = 65535 - (key & 0xffff);
  const int depth = key >> 16;
  if (tid == 0) {
    if (bad || depth + 1 > P) {
      s.res[0] = 0;
      s.res[1] = -1;
      s.res[2] = bad ? TV_STATUS_BAD_PARENT : TV_STATUS_DEPTH;
    } else {
      int node = best;
      for (int t = depth; t >= 0; --t) {
        s.path[t] = node;
        node = s.par[node];
      }
      s.res[0] = depth + 1;
      s.res[1] = tg[best];
      s.res[2] = 0;
    }
  }
  accept_sync_or<NT>(0);
}

// Writes one sequence's outputs from s (P entries of path, -1 past its end).
template <int NT>
__device__ __forceinline__ void accept_write(const AcceptLds& s, int b, int P, int32_t* path,
                                             int32_t* path_len, int32_t* bonus,
                                             int32_t* dev_status) {
  const int n = s.res[0];
  int32_t* pth = path + (size_t)b * P;
  for (int j = threadIdx.x; j < P; j += NT) pth[j] = j < n ? s.path[j] : -1;
  if (threadIdx.x == 0) {
    path_len[b] = n;
    bonus[b] = s.res[1];
    if (s.res[2] && dev_status) atomicOr(&dev_status[b], s.res[2]);
  }
}

}  // namespace tv
