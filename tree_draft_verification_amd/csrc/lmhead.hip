// Target LM head fused with a per-row argmax.
//
// The accepted path must follow the target's own logits (JetSpec GitHub
// README, "JetSpec > Overview"); at temperature 0 (the README's "Quick Start"
// examples) that is the argmax of  logits[r][v] = sum_k hidden[r][k] w[v][k].
// The logits are never written on the hot path: each workgroup reduces its
// tile to one (value, index) key per row and folds it into a per-row 64-bit
// atomicMax; the last workgroup to finish turns the keys into indices and
// clears them.  Max over packed keys is order-independent, so the result is
// deterministic, with ties going to the smallest index.
//
// bf16 kernel: a workgroup owns 128 vocabulary rows x 64 hidden-state rows.
// Every vocabulary row is read from HBM by exactly one workgroup per 64-row
// slice of hidden states; it goes straight from HBM into MFMA A-operand
// registers - each lane streams 64 contiguous bytes of one row per 128-wide k
// chunk, so four lanes cover 256 contiguous bytes - with the next chunk in
// flight while the current one is multiplied.  The reduction index k is
// permuted identically in both operands, which is what lets a lane's 64 bytes
// serve four consecutive 32-wide MFMA k-steps.  The hidden-state slice, shared
// by all four wavefronts, is staged through double-buffered LDS.  Workgroups
// that share a vocabulary tile (different hidden-state slices) get adjacent
// logical ids, which the remap places on one die so the tile is read from HBM
// once and served from that die's L2 afterwards.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 256;
constexpr int kVT = 128;   // vocabulary rows per workgroup (32 per wavefront)
constexpr int kMT = 64;    // hidden-state rows per workgroup
constexpr int kKC = 128;   // k per pipeline stage
constexpr int kHRow = kKC + 8;  // LDS row of the hidden-state slice (bf16)

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long x, int off) {
  const uint32_t lo = __shfl_xor((uint32_t)x, off, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), off, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// Fold this workgroup's per-row keys into the global keys; the last
// workgroup converts them to indices and leaves the workspace zeroed.
__device__ __forceinline__ void argmax_commit(unsigned long long* keys, unsigned* counter,
                                              int32_t* argmax, int M, int total_blocks,
                                              int m0, int mt, const unsigned long long* s_rowkey) {
  const int tid = threadIdx.x;
  if (tid < mt && m0 + tid < M) atomicMax(&keys[m0 + tid], s_rowkey[tid]);
  __threadfence();
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0) {
    const unsigned prev = atomicAdd(counter, 1u);
    s_last = (prev == (unsigned)total_blocks - 1u);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int m = tid; m < M; m += blockDim.x) {
    const unsigned long long k = atomicExch(&keys[m], 0ull);
    argmax[m] = (int32_t)(~(uint32_t)(k & 0xffffffffull));
  }
  if (tid == 0) atomicExch(counter, 0u);
}

__global__ __launch_bounds__(kThreads, 2) void lmhead_bf16_kernel(
    const bf16_t* __restrict__ H, const bf16_t* __restrict__ W, int32_t* __restrict__ argmax,
    float* __restrict__ logits, unsigned long long* __restrict__ keys,
    unsigned* __restrict__ counter, int M, int K, int V, int nmt, int total_blocks) {
  __shared__ __attribute__((aligned(16))) bf16_t sH[2][kMT * kHRow];
  __shared__ unsigned long long s_wkey[4][kMT];
  __shared__ unsigned long long s_rowkey[kMT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int kg = lane >> 4;

  const int lid = xcd_remap(blockIdx.x, total_blocks);
  const int mt = lid % nmt;
  const int vt = lid / nmt;
  const int m0 = mt * kMT;
  const int v0 = vt * kVT;

  // this lane's two vocabulary rows (one per 16-row block)
  const bf16_t* wrow[2];
  bool wok[2];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb) {
    const int v = v0 + wave * 32 + vb * 16 + l16;
    wok[vb] = v < V;
    wrow[vb] = W + (size_t)(wok[vb] ? v : 0) * K + 32 * kg;
  }
  // this thread's four 16-byte pieces of each hidden-state stage
  const bf16_t* hsrc[4];
  bool hok[4];
  int hdst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + i * kThreads;
    const int r = c / (kKC / 8);
    const int x = c - r * (kKC / 8);
    hok[i] = m0 + r < M;
    hsrc[i] = H + (size_t)(hok[i] ? m0 + r : 0) * K + x * 8;
    hdst[i] = r * kHRow + x * 8;
  }

  const int nk = K / kKC;
  uint4 wcur[2][4], wnxt[2][4], hreg[4];
  const uint4 z = make_uint4(0, 0, 0, 0);

#pragma unroll
  for (int i = 0; i < 4; ++i) hreg[i] = hok[i] ? *reinterpret_cast<const uint4*>(hsrc[i]) : z;
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      wcur[vb][s] = wok[vb] ? *reinterpret_cast<const uint4*>(wrow[vb] + 8 * s) : z;
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&sH[0][hdst[i]]) = hreg[i];
  __syncthreads();

  f32x4_t acc[2][4];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[vb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int c = 0; c < nk; ++c) {
    const bool more = c + 1 < nk;
    if (more) {
      const int ko = (c + 1) * kKC;
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          wnxt[vb][s] = wok[vb] ? *reinterpret_cast<const uint4*>(wrow[vb] + ko + 8 * s) : z;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hreg[i] = hok[i] ? *reinterpret_cast<const uint4*>(hsrc[i] + ko) : z;
    }
    const bf16_t* sh = sH[c & 1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      Frag8 hf[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        hf[mb].u = *reinterpret_cast<const uint4*>(&sh[(mb * 16 + l16) * kHRow + 32 * kg + 8 * s]);
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        Frag8 wf;
        wf.u = wcur[vb][s];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[vb][mb] = mfma16x16x32(wf.v, hf[mb].v, acc[vb][mb]);
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&sH[(c + 1) & 1][hdst[i]]) = hreg[i];
    }
    __syncthreads();
    if (more) {
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int s = 0; s < 4; ++s) wcur[vb][s] = wnxt[vb][s];
    }
  }

  // ---- epilogue: lane holds rows v = v0 + wave*32 + vb*16 + 4*kg + r of
  // hidden-state row m = m0 + mb*16 + l16
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = m0 + mb * 16 + l16;
    unsigned long long best = 0ull;
#pragma unroll
    for (int vb = 0; vb < 2; ++vb) {
      const int vbase = v0 + wave * 32 + vb * 16 + 4 * kg;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = vbase + r;
        if (v < V) {
          const unsigned long long key = argmax_key(acc[vb][mb][r], (uint32_t)v);
          best = key > best ? key : best;
        }
      }
      if (logits != nullptr && m < M) {
        float* dst = logits + (size_t)m * V + vbase;
        if ((V & 3) == 0 && vbase + 3 < V) {
          *reinterpret_cast<f32x4_t*>(dst) = acc[vb][mb];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (vbase + r < V) dst[r] = acc[vb][mb][r];
        }
      }
    }
    unsigned long long o = shfl_xor_u64(best, 16);
    best = o > best ? o : best;
    o = shfl_xor_u64(best, 32);
    best = o > best ? o : best;
    if (kg == 0) s_wkey[wave][mb * 16 + l16] = best;
  }
  __syncthreads();
  if (tid < kMT) {
    unsigned long long k = s_wkey[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) k = s_wkey[w][tid] > k ? s_wkey[w][tid] : k;
    s_rowkey[tid] = k;
  }
  __syncthreads();
  argmax_commit(keys, counter, argmax, M, total_blocks, m0, kMT, s_rowkey);
}

// fp32 path: one thread per vocabulary row, 16 hidden-state rows per
// workgroup staged through LDS in 256-wide k chunks.
constexpr int kF32MT = 16;
constexpr int kF32KC = 256;

__global__ __launch_bounds__(kThreads) void lmhead_f32_kernel(
    const float* __restrict__ H, const float* __restrict__ W, int32_t* __restrict__ argmax,
    float* __restrict__ logits, unsigned long long* __restrict__ keys,
    unsigned* __restrict__ counter, int M, int K, int V, int nmt, int total_blocks) {
  __shared__ float sH[kF32MT][kF32KC];
  __shared__ unsigned long long s_wkey[4][kF32MT];
  __shared__ unsigned long long s_rowkey[kF32MT];
  const int tid = threadIdx.x;
  const int mt = blockIdx.x % nmt;
  const int vt = blockIdx.x / nmt;
  const int m0 = mt * kF32MT;
  const int v = vt * kThreads + tid;
  const bool vok = v < V;
  const float* wr = W + (size_t)(vok ? v : 0) * K;
  float acc[kF32MT];
#pragma unroll
  for (int i = 0; i < kF32MT; ++i) acc[i] = 0.f;
  for (int kc = 0; kc < K; kc += kF32KC) {
    const int kn = min(kF32KC, K - kc);
    __syncthreads();
    for (int x = tid; x < kF32MT * kF32KC; x += kThreads) {
      const int r = x / kF32KC, kk = x - r * kF32KC;
      sH[r][kk] = (m0 + r < M && kk < kn) ? H[(size_t)(m0 + r) * K + kc + kk] : 0.f;
    }
    __syncthreads();
    if (vok) {
      for (int kk = 0; kk < kn; ++kk) {
        const float wv = wr[kc + kk];
#pragma unroll
        for (int i = 0; i < kF32MT; ++i) acc[i] = fmaf(sH[i][kk], wv, acc[i]);
      }
    }
  }
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int i = 0; i < kF32MT; ++i) {
    unsigned long long best = vok ? argmax_key(acc[i], (uint32_t)v) : 0ull;
    if (logits != nullptr && vok && m0 + i < M) logits[(size_t)(m0 + i) * V + v] = acc[i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const unsigned long long o = shfl_xor_u64(best, off);
      best = o > best ? o : best;
    }
    if (lane == 0) s_wkey[wave][i] = best;
  }
  __syncthreads();
  if (tid < kF32MT) {
    unsigned long long k = s_wkey[0][tid];
    for (int w = 1; w < 4; ++w) k = s_wkey[w][tid] > k ? s_wkey[w][tid] : k;
    s_rowkey[tid] = k;
  }
  __syncthreads();
  argmax_commit(keys, counter, argmax, M, total_blocks, m0, kF32MT, s_rowkey);
}

}  // namespace

size_t lmhead_ws_bytes(int M, int /*K*/, int /*V*/, int /*dtype*/) {
  // per-row keys, then the completion counter on its own 256-byte line
  return ((size_t)M * 8 + 255) / 256 * 256 + 256;
}

hipError_t launch_lmhead_argmax(const void* hidden, const void* w, int32_t* argmax,
                                float* logits, int M, int K, int V, int dtype, void* ws,
                                hipStream_t stream) {
  unsigned long long* keys = static_cast<unsigned long long*>(ws);
  unsigned* counter = reinterpret_cast<unsigned*>(static_cast<char*>(ws) +
                                                  ((size_t)M * 8 + 255) / 256 * 256);
  if (dtype == TV_F32) {
    const int nmt = (M + kF32MT - 1) / kF32MT;
    const int nvt = (V + kThreads - 1) / kThreads;
    const int total = nmt * nvt;
    hipLaunchKernelGGL(lmhead_f32_kernel, dim3(total), dim3(kThreads), 0, stream,
                       static_cast<const float*>(hidden), static_cast<const float*>(w), argmax,
                       logits, keys, counter, M, K, V, nmt, total);
    return hipGetLastError();
  }
  const int nmt = (M + kMT - 1) / kMT;
  const int nvt = (V + kVT - 1) / kVT;
  const int total = nmt * nvt;
  hipLaunchKernelGGL(lmhead_bf16_kernel, dim3(total), dim3(kThreads), 0, stream,
                     static_cast<const bf16_t*>(hidden), static_cast<const bf16_t*>(w), argmax,
                     logits, keys, counter, M, K, V, nmt, total);
  return hipGetLastError();
}

}  // namespace tv
