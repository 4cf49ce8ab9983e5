// Products with many hidden-state rows (M > 64): out[m][v] = sum_k H[m][k] W[v][k].
//
// Used by the LM head with argmax (keys per (row, vocabulary tile), finished
// by argmax_reduce_kernel) and by the projections of the multi-layer pass
// (split-K partial sums, finished by the epilogue kernels).  At these sizes
// the product is bound by the matrix cores, not by reading W, so the tiling
// is built around operand reuse:
//   * v_mfma_f32_32x32x16_bf16: a 32 x 32 block per instruction, half the
//     operand bytes per flop of the 16 x 16 form;
//   * a workgroup owns 256 W rows and 128 or 256 H rows; each of its 4
//     wavefronts owns 64 W rows (two 32-row blocks) against all of the H
//     rows, 128 or 256 fp32 accumulators per lane;
//   * W comes from the packed layout (the LM head's) straight into MFMA
//     operand registers through a two-chunk ring, each W byte read by one
//     wavefront; H is staged through double-buffered LDS and read by all
//     four;
//   * workgroups that share a W tile (up to four H slices) get adjacent
//     logical ids, which the remap places on one die, so the tile comes from
//     HBM once per die and the slices' rows stay in its L2.
// What bounds it is the rate at which a compute unit's vector memory path
// brings chunks in from L2 (about 74 cache lines in flight per CU, ~500
// cycles each).  For the LM head from 512 rows on, a 256-row H tile halves
// the H bytes per product and runs 6-14 % faster; it has no registers left
// for staging H, so H goes straight from memory into LDS.  At 256 rows it
// would leave most CUs with two tiles against three, and the split-K
// projections would need twice the splits, so both keep the 128-row tile.
// Operand lane layout of the 32 x 32 x 16 form (measured): lane l holds
// row (or column) l % 32 and k values 8*(l/32) .. 8*(l/32)+7; result
// register i of lane l is row 8*(i/4) + 4*(l/32) + i%4, column l % 32.
#include <type_traits>

#include "tv_internal.h"

namespace tv {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWT = 256;        // W rows per workgroup
constexpr int kPT = 128;        // W rows per packed tile
constexpr int kKC = 128;        // k per pipeline stage (8 steps of 16)
constexpr int kHRow = kKC + 8;  // LDS row of the register-staged H stage (bf16); 272 bytes
constexpr int kWideRows = 512;  // the 256-row H tile from this many rows on

enum : int { kGemmArgmax = 0, kGemmStore = 1 };

// s_waitcnt operand: vmcnt(0), expcnt and lgkmcnt left at their maxima
// (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long x, int off) {
  const uint32_t lo = __shfl_xor((uint32_t)x, off, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), off, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// Which (H slice, k split, W tile) a workgroup computes, and the W
// addressing of its wavefront.
struct Tile {
  int m0, ks, vt, nvt, cb, nkl, nk;  // first H row, split, W tile, chunks
  int vrow0, pt, jj0;                // first W row of the wavefront, packed tile, 16-row block
};

// Logical order (mi, ks, vt, group): groups of mg H slices; within a group
// the mg slices of one W tile are adjacent, so they share the tile through
// one die's L2, and a die works on few H slices at a time (their rows stay
// in its L2).  mg = 4 measured 13% faster than all slices of a W tile
// together at 4096 rows.
__device__ __forceinline__ Tile tile_of(int total_blocks, int nmt, int nsplit, int MT, int K,
                                        int V, int wave) {
  Tile t;
  const int lid = xcd_remap(blockIdx.x, total_blocks);
  t.nvt = total_blocks / (nmt * nsplit);
  const int mg = nmt % 4 == 0 ? 4 : (nmt % 2 == 0 ? 2 : 1);
  const int mi = lid % mg;
  const int r1 = lid / mg;
  t.ks = r1 % nsplit;
  const int r2 = r1 / nsplit;
  t.vt = r2 % t.nvt;
  t.m0 = ((r2 / t.nvt) * mg + mi) * MT;
  t.nk = K / kKC;
  const int npair = t.nk / 2;
  t.cb = 2 * (t.ks * npair / nsplit);
  t.nkl = 2 * ((t.ks + 1) * npair / nsplit) - t.cb;
  // this wavefront's 64 W rows: packed tile pt, 16-row blocks jj0 .. jj0+3
  const int ntiles = (V + kPT - 1) / kPT;
  t.vrow0 = t.vt * kWT + wave * 64;
  t.pt = t.vrow0 / kPT;
  t.pt = t.pt < ntiles ? t.pt : ntiles - 1;  // past the last tile: read it, drop the rows
  t.jj0 = (t.vrow0 % kPT) / 16;
  return t;
}

// Element offset in the packed W of (chunk c, 32-row block b, k step t) for
// this lane: lane l of piece s holds row l % 16 of its block at
// k = 32 (l / 16) + 8 s.
__device__ __forceinline__ size_t w_offset(const Tile& tl, int r32, int hh, int c, int b, int t) {
  const int jj = tl.jj0 + 2 * b + (r32 >> 4);
  const int s = 2 * (t & 1) + hh;
  const int L = (t >> 1) * 16 + (r32 & 15);
  return (((((size_t)tl.pt * tl.nk + c) * 8 + jj) * 4 + s) * 64 + L) * 8;
}

// acc[b][mb][i] is W row vrow0 + 32b + 8(i/4) + 4hh + i%4, H row
// m0 + 32mb + r32.  Store mode writes the split's fp32 partial sums; argmax
// mode writes one key per (row, W tile) (logits too, when asked).
template <int MODE, int MT>
__device__ __forceinline__ void epilogue(const f32x16_t (&acc)[2][MT / 32], const Tile& tl,
                                         unsigned long long (*s_key)[MT],
                                         unsigned long long* __restrict__ keys,
                                         float* __restrict__ logits, float* __restrict__ part,
                                         int M, int V) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hh = lane >> 5;
  if constexpr (MODE == kGemmStore) {
#pragma unroll
    for (int mb = 0; mb < MT / 32; ++mb) {
      const int m = tl.m0 + mb * 32 + r32;
      if (m >= M) continue;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int v = tl.vrow0 + 32 * b + 8 * q + 4 * hh;
          float* dst = part + ((size_t)tl.ks * M + m) * V + v;
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
    for (int mb = 0; mb < MT / 32; ++mb) {
      const int m = tl.m0 + mb * 32 + r32;
      unsigned long long best = 0ull;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int v = tl.vrow0 + 32 * b + 8 * (i >> 2) + 4 * hh + (i & 3);
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
            const int v = tl.vrow0 + 32 * b + 8 * (i >> 2) + 4 * hh + (i & 3);
            if (v < V) logits[(size_t)m * V + v] = acc[b][mb][i];
          }
      }
      const unsigned long long o = shfl_xor_u64(best, 32);
      best = o > best ? o : best;
      if (hh == 0) s_key[wave][mb * 32 + r32] = best;
    }
    __syncthreads();
    for (int r = tid; r < MT; r += kThreads) {
      if (tl.m0 + r >= M) break;
      unsigned long long k = s_key[0][r];
#pragma unroll
      for (int w = 1; w < 4; ++w) k = s_key[w][r] > k ? s_key[w][r] : k;
      keys[(size_t)(tl.m0 + r) * tl.nvt + tl.vt] = k;
    }
  }
}

// 128 H rows per workgroup; H staged through registers into padded LDS rows.
template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void gemm32_kernel(const bf16_t* __restrict__ H, const bf16_t* __restrict__ W,
                   unsigned long long* __restrict__ keys, float* __restrict__ logits,
                   float* __restrict__ part, int M, int K, int V, int nmt, int nsplit,
                   int total_blocks) {
  constexpr int MT = 128;
  constexpr int kHP = MT * (kKC / 8) / kThreads;  // 16-byte H pieces per thread per stage
  __shared__ __attribute__((aligned(16))) bf16_t sH[2][MT * kHRow];
  __shared__ unsigned long long s_key[4][MT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hh = lane >> 5;
  const Tile tl = tile_of(total_blocks, nmt, nsplit, MT, K, V, wave);
  const int m0 = tl.m0, cb = tl.cb, nkl = tl.nkl;
  auto wload = [&](int c, int b, int t) -> u32x4_t {
    return *reinterpret_cast<const u32x4_t*>(W + w_offset(tl, r32, hh, c, b, t));
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

  f32x16_t acc[2][MT / 32];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int mb = 0; mb < MT / 32; ++mb)
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
        Frag8 hf[MT / 32];
#pragma unroll
        for (int mb = 0; mb < MT / 32; ++mb)
          hf[mb].q = *reinterpret_cast<const u32x4_t*>(&sh[(mb * 32 + r32) * kHRow + 16 * t + 8 * hh]);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          Frag8 wf;
          wf.q = wb[u][b][t];
#pragma unroll
          for (int mb = 0; mb < MT / 32; ++mb) acc[b][mb] = mfma32(wf.v, hf[mb].v, acc[b][mb]);
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
  epilogue<MODE, MT>(acc, tl, s_key, keys, logits, part, M, V);
}

// 256 H rows per workgroup; H goes straight from memory into LDS (no
// registers are left for staging it next to 256 accumulators per lane).
template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void gemm32w_kernel(const bf16_t* __restrict__ H, const bf16_t* __restrict__ W,
                    unsigned long long* __restrict__ keys, float* __restrict__ logits,
                    float* __restrict__ part, int M, int K, int V, int nmt, int nsplit,
                    int total_blocks) {
  constexpr int MT = 256;
  constexpr int kDI = MT / 16;  // direct-to-LDS loads per wavefront per stage
  // Two stages as separate arrays, so that the reads of one never wait for
  // the loads filling the other.  Rows of 256 bytes; 16-byte piece x of row
  // r sits at position x ^ (r & 15), which keeps the fragment reads free of
  // bank conflicts.
  __shared__ __attribute__((aligned(1024))) bf16_t sH0[MT * kKC];
  __shared__ __attribute__((aligned(1024))) bf16_t sH1[MT * kKC];
  __shared__ unsigned long long s_key[4][MT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hh = lane >> 5;
  const Tile tl = tile_of(total_blocks, nmt, nsplit, MT, K, V, wave);
  const int cb = tl.cb, nkl = tl.nkl;
  auto wload = [&](int c, int b, int t) -> u32x4_t {
    return *reinterpret_cast<const u32x4_t*>(W + w_offset(tl, r32, hh, c, b, t));
  };

  // Wavefront w fills stage rows 64w .. 64w+63, four rows (1 KB) per
  // instruction: lane p of instruction i brings row 64w + 4i + p/16, piece
  // (p % 16) ^ (row & 15).  Rows past M read row M - 1.  Offsets are taken
  // from the slice's first row (at most 256 rows of K elements).
  const bf16_t* hslice = H + (size_t)tl.m0 * K;
  int hoff[kDI];
#pragma unroll
  for (int i = 0; i < kDI; ++i) {
    const int row = 64 * wave + 4 * i + (lane >> 4);
    const int x = (lane & 15) ^ (row & 15);
    const int rl = tl.m0 + row < M ? row : M - 1 - tl.m0;
    hoff[i] = rl * K + 8 * x;
  }
  auto hdma = [&](bf16_t* stage, int c) {
#pragma unroll
    for (int i = 0; i < kDI; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void*)(hslice + hoff[i] + (size_t)c * kKC),
          (__attribute__((address_space(3))) void*)(stage + (64 * wave + 4 * i) * kKC), 16, 0, 0);
  };
  // fragment of 32-row block mb, k step t: row 32mb + r32, piece 2t + hh
  auto frag = [&](const bf16_t* stage, int mb, int t) -> bf16x8_t {
    const int pos = (2 * t + hh) ^ (r32 & 15);
    Frag8 f;
    f.q = *reinterpret_cast<const u32x4_t*>(stage + (mb * 32 + r32) * kKC + pos * 8);
    return f.v;
  };

  u32x4_t wb[2][2][8];  // [ring slot][32-row block][k step]
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int t = 0; t < 8; ++t) wb[0][b][t] = wload(cb, b, t);
  hdma(sH0, cb);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __builtin_amdgcn_s_barrier();

  f32x16_t acc[2][MT / 32];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int mb = 0; mb < MT / 32; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][mb][i] = 0.f;

  // One chunk on stage U (a compile-time constant: each stage stays one
  // known LDS object in every instruction).  Chunk c + 1 goes into the other
  // stage and ring slot first (both last read in chunk c - 1, before the
  // last barrier; past the end, the last chunk again), so that any wait the
  // compiler places before this chunk's stage reads comes before those
  // loads; the chunk ends waiting for all of them, a chunk of products
  // after they were issued.
  auto chunk = [&](int c, auto stage_tag) {
    constexpr int U = decltype(stage_tag)::value;
    const bf16_t* sh = U ? sH1 : sH0;
    const int cn = cb + min(c + 1, nkl - 1);
    hdma(U ? sH0 : sH1, cn);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int t = 0; t < 8; ++t) wb[U ^ 1][b][t] = wload(cn, b, t);
    __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of the products
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      bf16x8_t hf[MT / 32];
#pragma unroll
      for (int mb = 0; mb < MT / 32; ++mb) hf[mb] = frag(sh, mb, t);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        Frag8 wf;
        wf.q = wb[U][b][t];
#pragma unroll
        for (int mb = 0; mb < MT / 32; ++mb) acc[b][mb] = mfma32(wf.v, hf[mb], acc[b][mb]);
      }
    }
    // chunk c + 1 is in this wavefront's registers and stage rows; after
    // the barrier, in everyone's
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_s_barrier();
  };
  for (int c0 = 0; c0 < nkl; c0 += 2) {
    chunk(c0, std::integral_constant<int, 0>{});
    chunk(c0 + 1, std::integral_constant<int, 1>{});
  }
  epilogue<MODE, MT>(acc, tl, s_key, keys, logits, part, M, V);
}

// The 256-row tile serves the LM head (one pass over k, argmax epilogue).
// The split-K projections stay on 128-row tiles: with half as many tiles
// they would take twice the splits, each with half the k range and twice
// the partial sums, and measured slower (a 36-layer pass at 512 rows: 13.4
// against 11.2 ms of projections).
bool use_wide(int M) { return M >= kWideRows; }

}  // namespace

int gemm32_vtiles(int V) { return (V + kWT - 1) / kWT; }

int gemm32_splits(int M, int K, int Nout) {
  const int tiles = ((M + 127) / 128) * gemm32_vtiles(Nout);
  const int npair = K / (2 * kKC);
  int best = 1;
  for (int s = 1; s <= npair; ++s)  // about two workgroups per CU at most
    if (npair % s == 0 && (long)s * tiles <= 512) best = s;
  return best;
}

hipError_t launch_gemm32_argmax(const void* hidden, const void* w_packed,
                                unsigned long long* keys, float* logits, int M, int K, int V,
                                hipStream_t stream) {
  const int rows = use_wide(M) ? 256 : 128;
  const int nmt = (M + rows - 1) / rows;
  const int total = nmt * gemm32_vtiles(V);
  const bf16_t* h = static_cast<const bf16_t*>(hidden);
  const bf16_t* w = static_cast<const bf16_t*>(w_packed);
  if (use_wide(M))
    hipLaunchKernelGGL(gemm32w_kernel<kGemmArgmax>, dim3(total), dim3(kThreads), 0, stream, h,
                       w, keys, logits, nullptr, M, K, V, nmt, 1, total);
  else
    hipLaunchKernelGGL(gemm32_kernel<kGemmArgmax>, dim3(total), dim3(kThreads), 0, stream, h, w,
                       keys, logits, nullptr, M, K, V, nmt, 1, total);
  return hipGetLastError();
}

hipError_t launch_gemm32_store(const void* hidden, const void* w_packed, float* part, int M,
                               int K, int Nout, int nsplit, hipStream_t stream) {
  const int nmt = (M + 127) / 128;
  const int total = nmt * gemm32_vtiles(Nout) * nsplit;
  hipLaunchKernelGGL(gemm32_kernel<kGemmStore>, dim3(total), dim3(kThreads), 0, stream,
                     static_cast<const bf16_t*>(hidden), static_cast<const bf16_t*>(w_packed),
                     nullptr, nullptr, part, M, K, Nout, nmt, nsplit, total);
  return hipGetLastError();
}

}  // namespace tv
