// Products with many hidden-state rows (M > 64): out[m][v] = sum_k H[m][k] W[v][k].
//
// Used by the LM head with argmax (keys per (row, vocabulary tile), finished
// by argmax_reduce_kernel) and by the projections of the multi-layer pass
// (split-K partial sums, finished by the epilogue kernels).  At these sizes
// the product is bound by the matrix cores, not by reading W, so the tiling
// is built around operand reuse:
//   * v_mfma_f32_32x32x16_bf16: a 32 x 32 block per instruction, half the
//     operand bytes per flop of the 16 x 16 form;
//   * a workgroup owns 256 W rows x 128 H rows; each of its 4 wavefronts
//     owns 64 W rows (two 32-row blocks) against all 128 H rows (four
//     blocks), 128 fp32 accumulators per lane;
//   * W comes from the packed layout (the LM head's) straight into MFMA
//     operand registers through a two-chunk ring, each W byte read by one
//     wavefront; H is staged through double-buffered LDS and read by all
//     four (4 KB of LDS per wavefront per 16-wide k step, against 8 MFMAs);
//   * workgroups that share a W tile (up to four 128-row slices of H) get
//     adjacent logical ids, which the remap places on one die, so the tile
//     comes from HBM once per die and the slices' rows stay in its L2.
// Operand lane layout of the 32 x 32 x 16 form (measured): lane l holds
// row (or column) l % 32 and k values 8*(l/32) .. 8*(l/32)+7; result
// register i of lane l is row 8*(i/4) + 4*(l/32) + i%4, column l % 32.
#include "tv_internal.h"

namespace tv {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWT = 256;        // W rows per workgroup
constexpr int kPT = 128;        // W rows per packed tile
constexpr int kMT = 128;        // H rows per workgroup
constexpr int kKC = 128;        // k per pipeline stage (8 steps of 16)
constexpr int kHRow = kKC + 8;  // LDS row of the H stage (bf16); 272 bytes
constexpr int kHP = kMT * (kKC / 8) / kThreads;  // 16-byte H pieces per thread per stage

enum : int { kGemmArgmax = 0, kGemmStore = 1 };

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long x, int off) {
  const uint32_t lo = __shfl_xor((uint32_t)x, off, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), off, 64);
  return ((unsigned long long)hi << 32) | lo;
}

template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void gemm32_kernel(const bf16_t* __restrict__ H, const bf16_t* __restrict__ W,
                   unsigned long long* __restrict__ keys, float* __restrict__ logits,
                   float* __restrict__ part, int M, int K, int V, int nmt, int nsplit,
                   int total_blocks) {
  __shared__ __attribute__((aligned(16))) bf16_t sH[2][kMT * kHRow];
  __shared__ unsigned long long s_key[4][kMT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hh = lane >> 5;

  // Logical order (mi, ks, vt, group): groups of mg H slices; within a
  // group the mg slices of one W tile are adjacent, so they share the tile
  // through one die's L2, and a die works on few H slices at a time (their
  // rows stay in its L2).  mg = 4 measured 13% faster than all slices of a
  // W tile together at 4096 rows.
  const int lid = xcd_remap(blockIdx.x, total_blocks);
  const int nvt = total_blocks / (nmt * nsplit);
  const int mg = nmt % 4 == 0 ? 4 : (nmt % 2 == 0 ? 2 : 1);
  const int mi = lid % mg;
  const int r1 = lid / mg;
  const int ks = r1 % nsplit;
  const int r2 = r1 / nsplit;
  const int vt = r2 % nvt;
  const int mt = (r2 / nvt) * mg + mi;
  const int m0 = mt * kMT;
  const int nk = K / kKC;
  const int npair = nk / 2;
  const int cb = 2 * (ks * npair / nsplit);
  const int nkl = 2 * ((ks + 1) * npair / nsplit) - cb;

  // this wavefront's 64 W rows: packed tile pt, 16-row blocks jj0 .. jj0+3
  const int ntiles = (V + kPT - 1) / kPT;
  const int vrow0 = vt * kWT + wave * 64;  // first W row of the wavefront
  int pt = vrow0 / kPT;
  pt = pt < ntiles ? pt : ntiles - 1;  // past the last tile: read it, drop the rows
  const int jj0 = (vrow0 % kPT) / 16;
  // element offset of (chunk c, 32-row block b, k step t) for this lane
  auto woff = [&](int c, int b, int t) -> size_t {
    const int jj = jj0 + 2 * b + (r32 >> 4);
    const int s = 2 * (t & 1) + hh;
    const int L = (t >> 1) * 16 + (r32 & 15);
    return (((((size_t)pt * nk + c) * 8 + jj) * 4 + s) * 64 + L) * 8;
  };
  auto wload = [&](int c, int b, int t) -> u32x4_t {
    return *reinterpret_cast<const u32x4_t*>(W + woff(c, b, t));
  };

  // this thread's 16-byte pieces of each H stage (clamped rows)
  const bf16_t* hsrc[kHP];
  int hdst[kHP];
#pragma unroll
  for (int i = 0; i < kHP; ++i) {
    const int c = tid + i * kThreads;
    const int r = c >> 4;
    const int x = c & 15;
    hsrc[i] = H + (size_t)(m0 + r < M ? m0 + r : M - 1) * K + x * 8;
    hdst[i] = r * kHRow + x * 8;
  }

  u32x4_t wb[2][2][8];  // [ring slot][32-row block][k step]
  u32x4_t hreg[kHP];
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int t = 0; t < 8; ++t) wb[d][b][t] = wload(cb + min(d, nkl - 1), b, t);
#pragma unroll
  for (int i = 0; i < kHP; ++i) hreg[i] = *reinterpret_cast<const u32x4_t*>(hsrc[i] + cb * kKC);
#pragma unroll
  for (int i = 0; i < kHP; ++i) *reinterpret_cast<u32x4_t*>(&sH[0][hdst[i]]) = hreg[i];
  __syncthreads();

  f32x16_t acc[2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][mb][i] = 0.f;

  for (int c0 = 0; c0 < nkl; c0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + u;
      const int ch = cb + min(c + 1, nkl - 1);
#pragma unroll
      for (int i = 0; i < kHP; ++i) hreg[i] = *reinterpret_cast<const u32x4_t*>(hsrc[i] + ch * kKC);
      const bf16_t* sh = sH[u];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        Frag8 hf[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          hf[mb].q = *reinterpret_cast<const u32x4_t*>(&sh[(mb * 32 + r32) * kHRow + 16 * t + 8 * hh]);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          Frag8 wf;
          wf.q = wb[u][b][t];
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) acc[b][mb] = mfma32(wf.v, hf[mb].v, acc[b][mb]);
        }
      }
      const int cw = cb + min(c + 2, nkl - 1);
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int t = 0; t < 8; ++t) wb[u][b][t] = wload(cw, b, t);
#pragma unroll
      for (int i = 0; i < kHP; ++i) *reinterpret_cast<u32x4_t*>(&sH[u ^ 1][hdst[i]]) = hreg[i];
      __syncthreads();
    }
  }

  // ---- epilogue: acc[b][mb][i] is W row vrow0 + 32b + 8(i/4) + 4hh + i%4,
  // H row m0 + 32mb + r32
  if constexpr (MODE == kGemmStore) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + mb * 32 + r32;
      if (m >= M) continue;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int v = vrow0 + 32 * b + 8 * q + 4 * hh;
          float* dst = part + ((size_t)ks * M + m) * V + v;
          const f32x4_t val = {acc[b][mb][4 * q], acc[b][mb][4 * q + 1], acc[b][mb][4 * q + 2],
                               acc[b][mb][4 * q + 3]};
          if ((V & 3) == 0 && v + 3 < V) {
            *reinterpret_cast<f32x4_t*>(dst) = val;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (v + e < V) dst[e] = val[e];
          }
        }
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + mb * 32 + r32;
      unsigned long long best = 0ull;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int v = vrow0 + 32 * b + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (v < V) {
            const unsigned long long key = argmax_key(acc[b][mb][i], (uint32_t)v);
            best = key > best ? key : best;
          }
        }
      if (logits != nullptr && m < M) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int v = vrow0 + 32 * b + 8 * (i >> 2) + 4 * hh + (i & 3);
            if (v < V) logits[(size_t)m * V + v] = acc[b][mb][i];
          }
      }
      const unsigned long long o = shfl_xor_u64(best, 32);
      best = o > best ? o : best;
      if (hh == 0) s_key[wave][mb * 32 + r32] = best;
    }
    __syncthreads();
    if (tid < kMT && m0 + tid < M) {
      unsigned long long k = s_key[0][tid];
#pragma unroll
      for (int w = 1; w < 4; ++w) k = s_key[w][tid] > k ? s_key[w][tid] : k;
      keys[(size_t)(m0 + tid) * nvt + vt] = k;
    }
  }
}

}  // namespace

int gemm32_vtiles(int V) { return (V + kWT - 1) / kWT; }

int gemm32_splits(int M, int K, int Nout) {
  const int tiles = ((M + kMT - 1) / kMT) * gemm32_vtiles(Nout);
  const int npair = K / (2 * kKC);
  int best = 1;
  for (int s = 1; s <= npair; ++s)  // about two workgroups per CU at most
    if (npair % s == 0 && (long)s * tiles <= 512) best = s;
  return best;
}

hipError_t launch_gemm32_argmax(const void* hidden, const void* w_packed,
                                unsigned long long* keys, float* logits, int M, int K, int V,
                                hipStream_t stream) {
  const int nmt = (M + kMT - 1) / kMT;
  const int total = nmt * gemm32_vtiles(V);
  hipLaunchKernelGGL(gemm32_kernel<kGemmArgmax>, dim3(total), dim3(kThreads), 0, stream,
                     static_cast<const bf16_t*>(hidden), static_cast<const bf16_t*>(w_packed),
                     keys, logits, nullptr, M, K, V, nmt, 1, total);
  return hipGetLastError();
}

hipError_t launch_gemm32_store(const void* hidden, const void* w_packed, float* part, int M,
                               int K, int Nout, int nsplit, hipStream_t stream) {
  const int nmt = (M + kMT - 1) / kMT;
  const int total = nmt * gemm32_vtiles(Nout) * nsplit;
  hipLaunchKernelGGL(gemm32_kernel<kGemmStore>, dim3(total), dim3(kThreads), 0, stream,
                     static_cast<const bf16_t*>(hidden), static_cast<const bf16_t*>(w_packed),
                     nullptr, nullptr, part, M, K, Nout, nmt, nsplit, total);
  return hipGetLastError();
}

}  // namespace tv
