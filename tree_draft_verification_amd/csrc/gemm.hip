// Products with many hidden-state rows (M > 64): out[m][v] = sum_k H[m][k] W[v][k].
//
// Used by the LM head with argmax (keys per (row, vocabulary tile), finished
// by argmax_reduce_kernel) and by the projections of the multi-layer pass
// (split-K partial sums, finished by the epilogue kernels).  At these sizes
// the product is bound by the matrix cores, not by reading W, so the tiling
// is built around operand reuse (v_mfma_f32_32x32x16_bf16: a 32 x 32 block
// per instruction, half the operand bytes per flop of the 16 x 16 form):
//   * below 256 rows, gemm32_kernel: a workgroup of 4 wavefronts owns 256 W
//     rows and 128 H rows; each wavefront owns 64 W rows against all of the
//     H rows (128 accumulators per lane); W comes from the packed layout (the
//     LM head's) straight into MFMA operand registers through a two-chunk
//     ring, each W byte read by one wavefront; H is staged through
//     double-buffered LDS and read by all four;
//   * from 256 rows, the eight-wavefront kernels (gemm8_argmax_kernel for
//     the LM head, gemm8_store_kernel for the projections): 256 H rows and
//     256 or 384 W rows per workgroup, both operands copied from memory
//     straight into LDS;
//   * workgroups that share a W tile (up to four H slices) get adjacent
//     logical ids, which the remap places on one die, so the tile comes from
//     HBM once per die and the slices' rows stay in its L2.
// What bounds them is the rate at which a compute unit's vector memory path
// brings chunks in from L2 (about 74 cache lines in flight per CU, ~500
// cycles each), so the lever is bytes per product: the larger tiles of the
// eight-wavefront kernels.
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

enum : int { kGemmArgmax = 0, kGemmStore = 1 };

// s_waitcnt operand: vmcnt(0), expcnt and lgkmcnt left at their maxima
// (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kCpolNT = 2;  // cache-policy bits of a global load: non-temporal

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

// LM head with argmax from 256 rows on: eight wavefronts (two per SIMD),
// TW W rows (256 or 384) x 256 H rows per workgroup, both operands loaded
// straight from memory into LDS in 64-wide k chunks, two stages.  With two
// wavefronts per SIMD one wavefront's products run while the other waits at
// a barrier or on its fragment reads; each wavefront owns TW/4 W rows x 128
// H rows (TW/2 accumulators per lane, so two fit a SIMD's registers).
//   * W stage: half of a packed 128-wide chunk of TW/128 packed tiles,
//     copied verbatim: slot ((tile * 8 + block) * 4 + piece) * 32 + lane' of
//     16 bytes holds row lane' % 16 of that 16-row block at k = 8 piece +
//     32 (lane' / 16) of the half chunk, so a fragment read of 16 rows is 256
//     contiguous bytes;
//   * H stage: 256 rows of 128 bytes; 16-byte piece x of row r sits at
//     slot x ^ ((r / 2) % 8), which spreads the 16 rows of one fragment read
//     over all the banks.
// The 384-row tile takes all 160 KB of LDS (the epilogue's key table reuses
// the first W stage) and 256 VGPRs; it reads 17 % fewer operand bytes per
// product and 22 % fewer fragments per matrix instruction than the 256-row
// tile, which measured 4-5 % faster on the 4096 x 2048 x 151936 product.
// Store mode (the projections of the multi-layer pass from 256 rows): a
// workgroup owns one k range of nsplit and writes its fp32 partial sums
// part[split][M][V]; the splits of a tile share a die.
// WNT: W loads marked non-temporal, for a single H slice, where each W byte
// is read once (measured 2 % faster there; with several slices sharing W
// tiles on one die, 2-5 % slower).
template <int TW, int MODE, bool WNT>
__device__ __forceinline__ void gemm8_body(const bf16_t* __restrict__ H,
                                           const bf16_t* __restrict__ W,
                                           unsigned long long* __restrict__ keys,
                                           float* __restrict__ logits, float* __restrict__ part,
                                           int M, int K, int V, int nmt, int nsplit,
                                           int total_blocks, int v_base, int key_base, int nkeys) {
  constexpr int KC = 64;           // k per stage
  constexpr int TH = 256;
  constexpr int NWAVE = 8;
  constexpr int NT = NWAVE * 64;
  constexpr int NWV = 4, NWH = 2;  // wavefronts along W and along H
  constexpr int BW = TW / NWV / 32, BH = TH / NWH / 32;
  constexpr int DMA_W = TW * KC * 2 / 1024 / NWAVE;  // 1 KB loads per wavefront
  constexpr int DMA_H = TH * KC * 2 / 1024 / NWAVE;
  __shared__ __attribute__((aligned(1024))) bf16_t sW0[TW * KC];
  __shared__ __attribute__((aligned(1024))) bf16_t sW1[TW * KC];
  __shared__ __attribute__((aligned(1024))) bf16_t sH0[TH * KC];
  __shared__ __attribute__((aligned(1024))) bf16_t sH1[TH * KC];
  typedef unsigned long long KeyRow[TH];
  static_assert(TW * KC * 2 >= NWV * TH * 8, "the key table fits a W stage");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar addressing
  const int r32 = lane & 31, hh = lane >> 5;
  const int wv = wave / NWH, wh = wave % NWH;
  // which (H slice, k split, W tile): logical order (mi, ks, vt, group), so
  // groups of mg H slices and the splits of one W tile run on one die
  const int nvt = total_blocks / (nmt * nsplit);
  const int lid = xcd_remap(blockIdx.x, total_blocks);
  const int mg = nmt % 4 == 0 ? 4 : (nmt % 2 == 0 ? 2 : 1);
  const int r1 = lid / mg;
  const int ks = r1 % nsplit;
  const int r2 = r1 / nsplit;
  const int vt = r2 % nvt;
  const int m0 = ((r2 / nvt) * mg + lid % mg) * TH;
  const int nk128 = K / 128;
  const int ntp = (V + kPT - 1) / kPT;  // packed 128-row tiles

  // Addresses of the loads are formed per chunk (few VGPRs: the 384-row
  // tile has none to spare).  W: load q = wave * DMA_W + i copies 16-byte
  // slots 64q .. 64q + 63, the halves of segments 2q and 2q + 1 (segment =
  // (tile, block, piece)); the packed tile of a load is the same for the
  // whole wavefront, so its base is scalar.  Offsets in 16-byte units (below
  // 2^31 for any supported V and K).  H: load i of wavefront w fills rows
  // 8 (w * DMA_H + i) .. + 7, 8 pieces each.
  const uint32_t wlane = (uint32_t)hh * 64 + r32;
  auto dma = [&](bf16_t* sw, bf16_t* sh, int c) {
    const uint32_t wc = (uint32_t)(c >> 1) * 32 * 64 + (c & 1) * 32;
#pragma unroll
    for (int i = 0; i < DMA_W; ++i) {
      const int s0 = 2 * (wave * DMA_W + i);  // even: both halves in one packed tile
      int pt = v_base / kPT + (TW / kPT) * vt + (s0 >> 5);
      pt = pt < ntp ? pt : ntp - 1;           // past the last tile: read it, drop the rows
      const uint32_t off = ((uint32_t)pt * nk128 * 32 + (s0 & 31)) * 64 + wc + wlane;
      __builtin_amdgcn_global_load_lds((const void*)(W + (size_t)off * 8),
          (__attribute__((address_space(3))) void*)(sw + (wave * DMA_W + i) * 512), 16, 0,
          WNT ? kCpolNT : 0);
    }
#pragma unroll
    for (int i = 0; i < DMA_H; ++i) {
      const int row = (wave * DMA_H + i) * 8 + (lane >> 3);
      const int x = (lane & 7) ^ ((row >> 1) & 7);
      const int gr = m0 + row < M ? m0 + row : M - 1;
      __builtin_amdgcn_global_load_lds((const void*)(H + (size_t)gr * K + 8 * x + (size_t)c * KC),
          (__attribute__((address_space(3))) void*)(sh + (wave * DMA_H + i) * 512), 16, 0, 0);
    }
  };
  auto wfrag = [&](const bf16_t* st, int r, int t) -> bf16x8_t {
    const int x = 2 * t + hh;
    const int slot = (((r >> 7) * 8 + ((r >> 4) & 7)) * 4 + (x & 3)) * 32 + (x >> 2) * 16 + (r & 15);
    Frag8 f;
    f.q = *reinterpret_cast<const u32x4_t*>(st + slot * 8);
    return f.v;
  };
  auto hfrag = [&](const bf16_t* st, int r, int t) -> bf16x8_t {
    const int pos = (2 * t + hh) ^ ((r >> 1) & 7);
    Frag8 f;
    f.q = *reinterpret_cast<const u32x4_t*>(st + r * KC + pos * 8);
    return f.v;
  };

  f32x16_t acc[BW][BH];
#pragma unroll
  for (int i = 0; i < BW; ++i)
#pragma unroll
    for (int j = 0; j < BH; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // chunks [cb, cb + nkl) of this split, whole pairs (one per stage)
  const int npair = K / (2 * KC);
  const int cb = 2 * (ks * npair / nsplit);
  const int nkl = 2 * ((ks + 1) * npair / nsplit) - cb;
  dma(sW0, sH0, cb);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __builtin_amdgcn_s_barrier();
  // chunk c on stage U (compile-time: each stage one known LDS object); the
  // loads of chunk c + 1 into the other stage are issued among its products,
  // and the chunk ends waiting for them
  auto chunk = [&](int c, auto stage_tag) {
    constexpr int U = decltype(stage_tag)::value;
    const bf16_t* sw = U ? sW1 : sW0;
    const bf16_t* sh = U ? sH1 : sH0;
    dma(U ? sW0 : sW1, U ? sH0 : sH1, min(c + 1, cb + nkl - 1));
#pragma unroll
    for (int t = 0; t < KC / 16; ++t) {
      bf16x8_t wf[BW], hf[BH];
#pragma unroll
      for (int i = 0; i < BW; ++i) wf[i] = wfrag(sw, wv * (TW / NWV) + 32 * i + r32, t);
#pragma unroll
      for (int j = 0; j < BH; ++j) hf[j] = hfrag(sh, wh * (TH / NWH) + 32 * j + r32, t);
#pragma unroll
      for (int i = 0; i < BW; ++i)
#pragma unroll
        for (int j = 0; j < BH; ++j) acc[i][j] = mfma32(wf[i], hf[j], acc[i][j]);
    }
    // Schedule: one product, then each of the wavefront's copies for the
    // next chunk followed by four products.  Issued all at once ahead of the
    // products, the copies stalled the wavefront at issue while the memory
    // path drained them, and its products started late (7 % on the
    // 4096 x 2048 x 151936 product; 3 or 5 products per copy measured slower).
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // matrix instruction
#pragma unroll
    for (int k = 0; k < DMA_W + DMA_H; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // vector memory (a copy)
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_s_barrier();
  };
  for (int c0 = cb; c0 < cb + nkl; c0 += 2) {
    chunk(c0, std::integral_constant<int, 0>{});
    chunk(c0 + 1, std::integral_constant<int, 1>{});
  }

  // acc[i][j][e]: W row v0 + TW/4 wv + 32 i + 8 (e / 4) + 4 hh + e % 4,
  // H row m0 + 128 wh + 32 j + r32.  Every read of the stages is done (the
  // loop ends at a barrier), so the key table can take the first W stage.
  if constexpr (MODE == kGemmStore) {
    // lane: rows m0 + 128 wh + 32 j + r32, W rows vw0 + 32 i + 8 q + 4 hh .. + 3
    const int vw0 = v_base + vt * TW + wv * (TW / NWV) + 4 * hh;
#pragma unroll
    for (int j = 0; j < BH; ++j) {
      const int m = m0 + wh * (TH / NWH) + 32 * j + r32;
      if (m >= M) continue;
      float* dst = part + ((size_t)ks * M + m) * V + vw0;
#pragma unroll
      for (int i = 0; i < BW; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int v = vw0 + 32 * i + 8 * q;
          const f32x4_t val = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                               acc[i][j][4 * q + 3]};
          if ((V & 3) == 0 && v + 3 < V) {
            *reinterpret_cast<f32x4_t*>(dst + 32 * i + 8 * q) = val;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (v + e < V) dst[32 * i + 8 * q + e] = val[e];
          }
        }
    }
    return;
  }
  // Per row, a lane first takes the maximum of its 16 BW candidates, then the
  // first candidate (in increasing vocabulary order: i, then e) equal to it;
  // the index and the 64-bit key are formed once per row.  Only the last W
  // tile checks indices against V, with a strict compare in increasing order
  // that keeps the first of equal maxima.  Candidate pos = 16 i + e is row
  // vw0 + 4 hh + voff(pos) (voff a compile-time constant), in range while
  // voff(pos) < lim.
  constexpr int NC = 16 * BW;
  KeyRow* s_key = reinterpret_cast<KeyRow*>(sW0);
  const int vw0 = v_base + vt * TW + wv * (TW / NWV);
  const bool full = vw0 + TW / NWV <= V;
  const int lim = V - vw0 - 4 * hh;
  auto voff = [](int pos) { return 32 * (pos >> 4) + 8 * ((pos & 15) >> 2) + (pos & 3); };
#pragma unroll
  for (int j = 0; j < BH; ++j) {
    const int hrow = wh * (TH / NWH) + 32 * j + r32;
    const int m = m0 + hrow;
    float bv = -INFINITY;
    int bp = -1;
    if (full) {
      bv = acc[0][j][0];
#pragma unroll
      for (int pos = 1; pos + 1 < NC; pos += 2)
        bv = fmaxf(fmaxf(bv, acc[pos >> 4][j][pos & 15]), acc[(pos + 1) >> 4][j][(pos + 1) & 15]);
      if (NC % 2 == 0) bv = fmaxf(bv, acc[BW - 1][j][15]);
#pragma unroll
      for (int pos = NC - 1; pos >= 0; --pos) bp = acc[pos >> 4][j][pos & 15] == bv ? pos : bp;
    } else {
#pragma unroll
      for (int pos = 0; pos < NC; ++pos) {
        const float x = acc[pos >> 4][j][pos & 15];
        const bool take = voff(pos) < lim && x > bv;
        bv = take ? x : bv;
        bp = take ? pos : bp;
      }
    }
    if (logits != nullptr && m < M) {
      float* lrow = logits + (size_t)m * V + vw0 + 4 * hh;
#pragma unroll
      for (int pos = 0; pos < NC; ++pos)
        if (voff(pos) < lim) lrow[voff(pos)] = acc[pos >> 4][j][pos & 15];
    }
    unsigned long long best = bp >= 0 ? argmax_key(bv, (uint32_t)(vw0 + 4 * hh + voff(bp))) : 0ull;
    const unsigned long long o = shfl_xor_u64(best, 32);
    best = o > best ? o : best;
    if (hh == 0) s_key[wv][hrow] = best;
  }
  __syncthreads();
  for (int r = tid; r < TH; r += NT) {
    if (m0 + r >= M) break;
    unsigned long long k = s_key[0][r];
#pragma unroll
    for (int w = 1; w < NWV; ++w) k = s_key[w][r] > k ? s_key[w][r] : k;
    keys[(size_t)(m0 + r) * nkeys + key_base + vt] = k;
  }
}

template <int TW, bool WNT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void gemm8_argmax_kernel(const bf16_t* __restrict__ H, const bf16_t* __restrict__ W,
                         unsigned long long* __restrict__ keys, float* __restrict__ logits, int M,
                         int K, int V, int nmt, int total_blocks, int v_base, int key_base,
                         int nkeys) {
  gemm8_body<TW, kGemmArgmax, WNT>(H, W, keys, logits, nullptr, M, K, V, nmt, 1, total_blocks, v_base,
                              key_base, nkeys);
}

template <int TW>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void gemm8_store_kernel(const bf16_t* __restrict__ H, const bf16_t* __restrict__ W,
                        float* __restrict__ part, int M, int K, int Nout, int nmt, int nsplit,
                        int total_blocks) {
  gemm8_body<TW, kGemmStore, false>(H, W, nullptr, nullptr, part, M, K, Nout, nmt, nsplit, total_blocks,
                             0, 0, 0);
}

// The eight-wavefront LM head from this many rows on, and its W tiles.  One
// workgroup fits a CU, so a launch runs in rounds of 256 workgroups, and a
// round costs what its longest workgroup costs.  The vocabulary is split
// into a run of 384-row W tiles (about 5 % cheaper per product, 1.5x the
// work per workgroup) and a tail of 256-row tiles, in two launches, where
// that takes fewer rounds than one width alone: at 256 H rows and 151936
// vocabulary rows, 256 tiles of 384 rows (one round) and 210 of 256 rows
// (one round of two-thirds the work) against 396 tiles of 384 (two
// rounds).  Measured with one width: 256 rows (594 -> 396 workgroups, 3 ->
// 2 rounds) 393 -> 380 us; 512 rows (1188 -> 792, 5 -> 4 rounds of 1.5x
// work) 636 -> 687 us; 4096 rows 2238-2326 -> 2225 us.
constexpr int kGemm8Rows = 256;
constexpr int kCUs = 256;
bool use_gemm8(int M) { return M >= kGemm8Rows; }
struct Gemm8Plan {
  int n384, n256;  // W tiles of each width: rows [0, 384 n384) then the rest
};
Gemm8Plan gemm8_plan(int M, int V) {
  const long nmt = (M + 255) / 256;
  auto rounds = [&](long tiles) { return (nmt * tiles + kCUs - 1) / kCUs; };
  // cost in rounds of 256-row tiles; a second launch adds a little
  constexpr double k384 = 1.5 * 0.95, kLaunch = 0.05;
  Gemm8Plan best{0, (V + 255) / 256};
  double cost = (double)rounds(best.n256);
  const int all384 = (V + 383) / 384;
  if (rounds(all384) * k384 < cost) {
    best = Gemm8Plan{all384, 0};
    cost = rounds(all384) * k384;
  }
  for (int n = 1; 384L * n < V; ++n) {  // on equal cost, the most 384-row tiles
    const int tail = (V - 384 * n + 255) / 256;
    const double c = rounds(n) * k384 + rounds(tail) + kLaunch;
    if (c <= cost) {
      best = Gemm8Plan{n, tail};
      cost = c;
    }
  }
  return best;
}

// The store-mode product from 256 rows (the multi-layer pass's projections):
// the W tile width and the k split with the least modelled time, rounds of
// 256 workgroups x (chunks per split + 2 for the ramp and the epilogue) x
// 1.8 us per 256-row chunk (1.425x for 384 rows), plus the partial sums
// written and read back at 5 TB/s.
struct Gemm8StorePlan {
  int tw, nsplit;
};
Gemm8StorePlan gemm8_store_plan(int M, int K, int Nout) {
  const long nmt = (M + 255) / 256;
  const int npair = K / 128;
  Gemm8StorePlan best{256, 1};
  double cost = 1e300;
  for (int tw = 256; tw <= 384; tw += 128) {
    const long nvt = (Nout + tw - 1) / tw;
    const double unit = tw == 384 ? 1.425 : 1.0;
    for (int s = 1; s <= npair; ++s) {
      if (npair % s) continue;
      const long rounds = (nmt * nvt * s + kCUs - 1) / kCUs;
      const double t = rounds * (2.0 * npair / s + 2) * unit * 1.8 +
                       (double)s * M * Nout * 8 / 5e6;
      if (t < cost) {
        cost = t;
        best = Gemm8StorePlan{tw, s};
      }
    }
  }
  return best;
}

}  // namespace

int gemm32_vtiles(int V) { return (V + kWT - 1) / kWT; }

int gemm_argmax_vtiles(int M, int V) {
  if (use_gemm8(M)) {
    const Gemm8Plan p = gemm8_plan(M, V);
    return p.n384 + p.n256;
  }
  return (V + kWT - 1) / kWT;
}

int gemm32_splits(int M, int K, int Nout) {
  if (use_gemm8(M) && K % 128 == 0) return gemm8_store_plan(M, K, Nout).nsplit;
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
  if (use_gemm8(M)) {
    const int nmt = (M + 255) / 256;
    const Gemm8Plan p = gemm8_plan(M, V);
    const int nkeys = p.n384 + p.n256;
    const bf16_t* h = static_cast<const bf16_t*>(hidden);
    const bf16_t* w = static_cast<const bf16_t*>(w_packed);
    if (p.n384 > 0) {
      const int total = nmt * p.n384;
      if (nmt == 1)
        hipLaunchKernelGGL((gemm8_argmax_kernel<384, true>), dim3(total), dim3(512), 0, stream, h,
                           w, keys, logits, M, K, V, nmt, total, 0, 0, nkeys);
      else
        hipLaunchKernelGGL((gemm8_argmax_kernel<384, false>), dim3(total), dim3(512), 0, stream, h,
                           w, keys, logits, M, K, V, nmt, total, 0, 0, nkeys);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (p.n256 > 0) {
      const int total = nmt * p.n256;
      if (nmt == 1)
        hipLaunchKernelGGL((gemm8_argmax_kernel<256, true>), dim3(total), dim3(512), 0, stream, h,
                           w, keys, logits, M, K, V, nmt, total, 384 * p.n384, p.n384, nkeys);
      else
        hipLaunchKernelGGL((gemm8_argmax_kernel<256, false>), dim3(total), dim3(512), 0, stream, h,
                           w, keys, logits, M, K, V, nmt, total, 384 * p.n384, p.n384, nkeys);
    }
    return hipGetLastError();
  }
  const int nmt = (M + 127) / 128;
  const int total = nmt * gemm32_vtiles(V);
  hipLaunchKernelGGL(gemm32_kernel<kGemmArgmax>, dim3(total), dim3(kThreads), 0, stream,
                     static_cast<const bf16_t*>(hidden), static_cast<const bf16_t*>(w_packed), keys,
                     logits, nullptr, M, K, V, nmt, 1, total);
  return hipGetLastError();
}

hipError_t launch_gemm32_store(const void* hidden, const void* w_packed, float* part, int M,
                               int K, int Nout, int nsplit, hipStream_t stream) {
  if (use_gemm8(M) && K % 128 == 0) {
    const int nmt = (M + 255) / 256;
    const int tw = gemm8_store_plan(M, K, Nout).tw;
    const int total = nmt * ((Nout + tw - 1) / tw) * nsplit;
    const bf16_t* h = static_cast<const bf16_t*>(hidden);
    const bf16_t* w = static_cast<const bf16_t*>(w_packed);
    if (tw == 384)
      hipLaunchKernelGGL(gemm8_store_kernel<384>, dim3(total), dim3(512), 0, stream, h, w, part, M,
                         K, Nout, nmt, nsplit, total);
    else
      hipLaunchKernelGGL(gemm8_store_kernel<256>, dim3(total), dim3(512), 0, stream, h, w, part, M,
                         K, Nout, nmt, nsplit, total);
    return hipGetLastError();
  }
  const int nmt = (M + 127) / 128;
  const int total = nmt * gemm32_vtiles(Nout) * nsplit;
  hipLaunchKernelGGL(gemm32_kernel<kGemmStore>, dim3(total), dim3(kThreads), 0, stream,
                     static_cast<const bf16_t*>(hidden), static_cast<const bf16_t*>(w_packed),
                     nullptr, nullptr, part, M, K, Nout, nmt, nsplit, total);
  return hipGetLastError();
}

}  // namespace tv
