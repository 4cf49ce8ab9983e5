// Target LM head fused with a per-row argmax.
//
// The accepted path must follow the target's own logits (JetSpec GitHub
// README, "JetSpec > Overview"); at temperature 0 (the README's "Quick Start"
// examples) that is the argmax of  logits[r][v] = sum_k hidden[r][k] w[v][k].
// The logits are never written on the hot path: each workgroup reduces its
// tile to one packed (value, index) key per row and folds it into a per-row
// 64-bit atomic max; the last workgroup to finish turns the keys into indices
// and clears them.  A max over packed keys does not depend on the order of
// arrival, so the result is deterministic, with ties to the smallest index.
//
// bf16 streaming kernel (few hidden-state rows: the step is bound by reading
// the vocabulary matrix once from HBM):
//   * A workgroup owns 128 vocabulary rows x 64 hidden-state rows; each of
//     its 4 wavefronts owns 32 vocabulary rows (two 16-row MFMA blocks).
//   * The vocabulary rows go straight from HBM into MFMA A-operand registers
//     through a two-deep register ring (chunk c+2 is in flight while chunk c
//     is multiplied).  Every load is unconditional (addresses are clamped and
//     out-of-range rows are dropped in the epilogue): a lane-dependent branch
//     around a load would make the compiler wait for every outstanding load
//     at the next use, which serialises the stream.
//   * The reduction index k is permuted identically in both operands, so a
//     lane's 64 contiguous bytes of one row serve four 32-wide k-steps.
//   * The 64 hidden-state rows, shared by the 4 wavefronts, are staged
//     through double-buffered LDS, one 128-wide k chunk at a time.
//   * Packed vocabulary layout (tv_lmhead_pack_weights): the 4 KB that one
//     wavefront consumes for one 16-row block and one k chunk are stored
//     contiguously in lane order, and a workgroup's whole tile is contiguous,
//     so every load instruction reads 1 KB of consecutive bytes; the
//     row-major layout reads 16 rows x 64 bytes per instruction instead.
//   * Workgroups that share a vocabulary tile (different 64-row slices of
//     hidden states) get adjacent logical ids, which the remap places on one
//     die so that the tile comes from HBM once and from that die's L2 after.
//   * With the packed layout and M <= 64 (the LM head of a verification
//     step) the same products run as a persistent stream,
//     lmhead_stream_kernel: as many workgroups as stay resident, each
//     walking its share of the tiles as one stream of k chunks, so no
//     workgroup ramps up, drains or finishes per tile.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 256;
constexpr int kVT = 128;        // vocabulary rows per workgroup (32 per wavefront)
constexpr int kKC = 128;        // k per pipeline stage
constexpr int kHRow = kKC + 8;  // LDS row of the hidden-state slice (bf16)
// s_waitcnt operand: vmcnt(0), expcnt and lgkmcnt left at their maxima
// (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long x, int off) {
  const uint32_t lo = __shfl_xor((uint32_t)x, off, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), off, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// Fold a tile's per-row keys into the global keys.  The atomics return
// their old value and an empty asm statement takes it as an input, so the
// compiler waits for each one to complete before the thread goes on.
__device__ __forceinline__ void fold_row_keys(unsigned long long* keys, int M, int m0, int mt,
                                              const unsigned long long* s_rowkey) {
  const int tid = threadIdx.x;
  if (tid < mt && m0 + tid < M) {
    const unsigned long long old = __hip_atomic_fetch_max(
        &keys[m0 + tid], s_rowkey[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::"v"(old));
  }
}

// After every key update of the workgroup (a barrier past fold_row_keys):
// count the workgroup as done; the last of `total_blocks` converts the keys
// to indices and leaves the workspace zeroed.  Every key update of a
// workgroup has completed before its counter increment is issued, so no
// device-wide fence (and no L2 write-back) is needed.
__device__ __forceinline__ void finish_argmax(unsigned long long* keys, unsigned* counter,
                                              int32_t* argmax, int M, int total_blocks) {
  __shared__ int s_last;
  const int tid = threadIdx.x;
  if (tid == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)total_blocks - 1u;
  }
  __syncthreads();
  if (!s_last) return;
  for (int m = tid; m < M; m += blockDim.x) {
    const unsigned long long k =
        __hip_atomic_exchange(&keys[m], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    argmax[m] = (int32_t)(~(uint32_t)(k & 0xffffffffull));
  }
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup's keys folded, then the finish.
__device__ __forceinline__ void argmax_commit(unsigned long long* keys, unsigned* counter,
                                              int32_t* argmax, int M, int total_blocks, int m0,
                                              int mt, const unsigned long long* s_rowkey) {
  fold_row_keys(keys, M, m0, mt, s_rowkey);
  __syncthreads();
  finish_argmax(keys, counter, argmax, M, total_blocks);
}

// Address of piece s (16 bytes) of lane `lane` of 16-row block j of tile vt,
// k chunk c, in the packed layout (bf16 elements).
__device__ __forceinline__ size_t packed_offset(int vt, int c, int nk, int j, int s, int lane) {
  return (((((size_t)vt * nk + c) * 8 + j) * 4 + s) * 64 + lane) * 8;
}

// What a workgroup does with its tile of products.
enum : int {
  kArgmaxCommit = 0,   // fold per-row keys into the global keys (M <= 64)
  kArgmaxPartial = 1,  // write one key per (row, vocabulary tile)
  kStorePartial = 2,   // write the fp32 partial sums of its k range (projections)
  kSwiGLU = 3,         // gate/up projection, whole k range: write bf16 silu(gate) * up
};

// MODE kStorePartial computes out = H W^T for a linear layer (V = output
// features): workgroup (mt, vt, ks) covers k chunks [cb, ce) of the split ks
// of nsplit and writes its partial sums to part[ks][M][V]; an epilogue
// kernel adds the splits in a fixed order, so the result is deterministic.
//
// MODE kSwiGLU is the gate/up projection of a layer's MLP over the whole k
// range, with gate and up rows interleaved per tile (see pack_kernel): it
// writes bf16 silu(gate) * up for the tile's 64 features.
//
// RING is the depth of the register ring of W chunks (loads in flight per
// wavefront).  Every form uses 2: with several workgroups per CU (the LM
// head) a deeper ring only costs occupancy, and for the projections (about
// one workgroup per CU) a sweep of depth 2 and 4 found no gain from 4.
//
// HD is the depth of the H stage prefetch: 1 loads a chunk's H slice while
// the previous chunk is multiplied; deeper rings keep HD chunks in flight
// (projections: one workgroup per CU, so an H load's L2 latency is not
// hidden by other workgroups; 4 deep: 5 % on the multi-layer pass).  A trip
// covers max(RING, HD) chunks.
template <bool PACKED, int MB, int MODE, int RING = 2, int HD = 1>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(MB == 4 ? 2 : 1)))
void lmhead_bf16_kernel(const bf16_t* __restrict__ H, const bf16_t* __restrict__ W,
                        int32_t* __restrict__ argmax, float* __restrict__ logits,
                        unsigned long long* __restrict__ keys, unsigned* __restrict__ counter,
                        int M, int K, int V, int nmt, int total_blocks, float* __restrict__ part,
                        int nsplit, bf16_t* __restrict__ act, int inter) {
  constexpr int kRowsM = 16 * MB;                  // hidden-state rows per workgroup
  constexpr int HP = kRowsM * (kKC / 8) / kThreads;  // 16-byte H pieces per thread per stage
  __shared__ __attribute__((aligned(16))) bf16_t sH[2][kRowsM * kHRow];
  __shared__ unsigned long long s_wkey[4][kRowsM];
  __shared__ unsigned long long s_rowkey[kRowsM];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int kg = lane >> 4;

  const int lid = xcd_remap(blockIdx.x, total_blocks);
  const int mt = lid % nmt;
  const int vs = lid / nmt;
  const int ks = vs % nsplit;
  const int vt = vs / nsplit;
  const int m0 = mt * kRowsM;
  const int v0 = vt * kVT;
  const int nk = K / kKC;
  // this split's k chunks [cb, cb + nkl): whole groups of TRIP chunks
  constexpr int TRIP = RING > HD ? RING : HD;
  const int ngroup = nk / TRIP;
  const int cb = TRIP * (ks * ngroup / nsplit);
  const int nkl = TRIP * ((ks + 1) * ngroup / nsplit) - cb;

  // W source of this lane (clamped rows in the row-major layout; the packed
  // layout is zero-padded to whole tiles)
  const bf16_t* wrow[2];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb) {
    const int v = v0 + wave * 32 + vb * 16 + l16;
    wrow[vb] = W + (size_t)(v < V ? v : V - 1) * K + 32 * kg;
  }
  auto wload = [&](int c, int vb, int s) -> u32x4_t {
    if constexpr (PACKED && MB == 4) {
      // one row block (M <= 64): every W byte is read once, so the loads are
      // non-temporal (measured 6% faster on the packed layout, slower on the
      // row-major one)
      return __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(W + packed_offset(vt, c, nk, wave * 2 + vb, s, lane)));
    } else if constexpr (PACKED) {
      // several row blocks share each W tile (neighbouring workgroups on one
      // XCD): keep it cacheable so the re-reads hit L2
      return *reinterpret_cast<const u32x4_t*>(W + packed_offset(vt, c, nk, wave * 2 + vb, s, lane));
    } else {
      return *reinterpret_cast<const u32x4_t*>(wrow[vb] + c * kKC + 8 * s);
    }
  };
  // this thread's 16-byte pieces of each hidden-state stage (clamped rows)
  const bf16_t* hsrc[HP];
  int hdst[HP];
#pragma unroll
  for (int i = 0; i < HP; ++i) {
    const int c = tid + i * kThreads;
    const int r = c >> 4;
    const int x = c & 15;
    hsrc[i] = H + (size_t)(m0 + r < M ? m0 + r : M - 1) * K + x * 8;
    hdst[i] = r * kHRow + x * 8;
  }

  u32x4_t wb[RING][2][4];  // [ring slot][16-row block][piece]
  u32x4_t hreg[HD][HP];    // [H slot: chunk % HD][piece]
#pragma unroll
  for (int d = 0; d < RING; ++d)
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int s = 0; s < 4; ++s) wb[d][vb][s] = wload(cb + min(d, nkl - 1), vb, s);
#pragma unroll
  for (int d = 0; d < HD; ++d)
#pragma unroll
    for (int i = 0; i < HP; ++i)
      hreg[d][i] = *reinterpret_cast<const u32x4_t*>(hsrc[i] + (cb + min(d, nkl - 1)) * kKC);
#pragma unroll
  for (int i = 0; i < HP; ++i) *reinterpret_cast<u32x4_t*>(&sH[0][hdst[i]]) = hreg[0][i];
  if constexpr (HD > 1) {  // slot 0 is free again: chunk HD goes there
#pragma unroll
    for (int i = 0; i < HP; ++i)
      hreg[0][i] = *reinterpret_cast<const u32x4_t*>(hsrc[i] + (cb + min(HD, nkl - 1)) * kKC);
  }
  __syncthreads();

  f32x4_t acc[2][MB];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[vb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // nkl is a multiple of TRIP (K is a multiple of 256, splits take whole
  // groups): TRIP chunks per trip keep the ring slots and the LDS buffer
  // compile-time constants.
  for (int c0 = 0; c0 < nkl; c0 += TRIP) {
#pragma unroll
    for (int u = 0; u < TRIP; ++u) {
      const int c = c0 + u;
      if constexpr (HD == 1) {
        const int ch = cb + min(c + 1, nkl - 1);
#pragma unroll
        for (int i = 0; i < HP; ++i) hreg[0][i] = *reinterpret_cast<const u32x4_t*>(hsrc[i] + ch * kKC);
      }
      const bf16_t* sh = sH[u & 1];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          Frag8 hf;
          hf.u = *reinterpret_cast<const uint4*>(&sh[(mb * 16 + l16) * kHRow + 32 * kg + 8 * s]);
#pragma unroll
          for (int vb = 0; vb < 2; ++vb) {
            Frag8 wf;
            wf.q = wb[u % RING][vb][s];
            acc[vb][mb] = mfma16x16x32(wf.v, hf.v, acc[vb][mb]);
          }
        }
      }
      const int cw = cb + min(c + RING, nkl - 1);
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int s = 0; s < 4; ++s) wb[u % RING][vb][s] = wload(cw, vb, s);
      // chunk c+1's H slice (slot (c+1) % HD) into the other LDS buffer;
      // with HD > 1 that slot then takes chunk c+1+HD
      const int hs = HD == 1 ? 0 : (u + 1) % HD;  // constant once unrolled
#pragma unroll
      for (int i = 0; i < HP; ++i) *reinterpret_cast<u32x4_t*>(&sH[(u & 1) ^ 1][hdst[i]]) = hreg[hs][i];
      if constexpr (HD > 1) {
        const int cn = cb + min(c + 1 + HD, nkl - 1);
#pragma unroll
        for (int i = 0; i < HP; ++i) hreg[hs][i] = *reinterpret_cast<const u32x4_t*>(hsrc[i] + cn * kKC);
      }
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds rows v = v0 + wave*32 + vb*16 + 4*kg + r of
  // hidden-state row m = m0 + mb*16 + l16
  if constexpr (MODE == kSwiGLU) {
    // Gate/up rows are packed interleaved (each 128-row tile: gate rows of
    // features 64 vt .. 64 vt + 63, then the up rows of the same features),
    // so wavefronts 2 and 3 hold the up values matching wavefronts 0 and 1
    // lane for lane.  They pass them through LDS; 0 and 1 write
    // a[m][f] = bf16(silu(gate) * up), the expression of the split form's
    // epilogue kernel.
    float* su = reinterpret_cast<float*>(&sH[0][0]);  // [2][2][MB][64][4] floats
    __syncthreads();  // every wavefront is past its last read of sH
    if (wave >= 2) {
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          *reinterpret_cast<f32x4_t*>(&su[((((wave - 2) * 2 + vb) * MB + mb) * 64 + lane) * 4]) =
              acc[vb][mb];
    }
    __syncthreads();
    if (wave < 2) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = m0 + mb * 16 + l16;
        if (m >= M) continue;
#pragma unroll
        for (int vb = 0; vb < 2; ++vb) {
          const f32x4_t u =
              *reinterpret_cast<const f32x4_t*>(&su[(((wave * 2 + vb) * MB + mb) * 64 + lane) * 4]);
          const f32x4_t g = acc[vb][mb];
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = g[e] / (1.f + __expf(-g[e])) * u[e];
          const int f = 64 * vt + wave * 32 + vb * 16 + 4 * kg;
          u32x2_t pk;
          pk.x = f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16);
          pk.y = f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16);
          *reinterpret_cast<u32x2_t*>(act + (size_t)m * inter + f) = pk;
        }
      }
    }
    return;
  }
  if constexpr (MODE == kStorePartial) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + mb * 16 + l16;
      if (m >= M) continue;
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        const int vbase = v0 + wave * 32 + vb * 16 + 4 * kg;
        float* dst = part + ((size_t)ks * M + m) * V + vbase;
        if ((V & 3) == 0 && vbase + 3 < V) {
          *reinterpret_cast<f32x4_t*>(dst) = acc[vb][mb];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (vbase + r < V) dst[r] = acc[vb][mb][r];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
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
  if (tid < kRowsM) {
    unsigned long long k = s_wkey[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) k = s_wkey[w][tid] > k ? s_wkey[w][tid] : k;
    s_rowkey[tid] = k;
  }
  __syncthreads();
  if constexpr (MODE == kArgmaxPartial) {
    // one key per (row, vocabulary tile); argmax_reduce_kernel finishes
    const int nvt = total_blocks / nmt;
    if (tid < kRowsM && m0 + tid < M) keys[(size_t)(m0 + tid) * nvt + vt] = s_rowkey[tid];
  } else {
    argmax_commit(keys, counter, argmax, M, total_blocks, m0, kRowsM, s_rowkey);
  }
}

// Persistent form of the packed M <= 64 argmax (the LM head of a
// verification step).  Each workgroup walks the vocabulary tiles
// blockIdx.x, blockIdx.x + gridDim.x, ... as one stream of k chunks: the
// W ring runs across tile boundaries, so the next tile's first chunks are
// in flight while a tile's epilogue folds its keys, and no workgroup ramps
// up or drains per tile.  The grid is what stays resident at once (about
// 3 workgroups per CU), measured 5 % faster than one workgroup per tile.
// Products, operand layouts, the key fold and the last-workgroup finish
// are those of lmhead_bf16_kernel.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void lmhead_stream_kernel(const bf16_t* __restrict__ H, const bf16_t* __restrict__ W,
                          int32_t* __restrict__ argmax, float* __restrict__ logits,
                          unsigned long long* __restrict__ keys, unsigned* __restrict__ counter,
                          int M, int K, int V, int ntiles) {
  constexpr int MB = 4;
  constexpr int kRowsM = 16 * MB;
  constexpr int HP = kRowsM * (kKC / 8) / kThreads;
  __shared__ __attribute__((aligned(16))) bf16_t sH[2][kRowsM * kHRow];
  __shared__ unsigned long long s_wkey[4][kRowsM];
  __shared__ unsigned long long s_rowkey[kRowsM];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int kg = lane >> 4;
  const int nk = K / kKC;  // even: K is a multiple of 256
  const int ntl = (ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int G = ntl * nk;  // chunks of this workgroup's stream
  // chunk g of the stream: chunk g % nk of tile blockIdx.x + (g / nk) gridDim.x
  auto wload = [&](int g, int vb, int s) -> u32x4_t {
    const int j = g / nk;
    const int c = g - j * nk;
    const int vt = blockIdx.x + j * gridDim.x;
    return __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_t*>(W + packed_offset(vt, c, nk, wave * 2 + vb, s, lane)));
  };
  const bf16_t* hsrc[HP];
  int hdst[HP];
#pragma unroll
  for (int i = 0; i < HP; ++i) {
    const int c = tid + i * kThreads;
    const int r = c >> 4;
    const int x = c & 15;
    hsrc[i] = H + (size_t)(r < M ? r : M - 1) * K + x * 8;
    hdst[i] = r * kHRow + x * 8;
  }

  u32x4_t wb[2][2][4];  // [ring slot][16-row block][piece]
  u32x4_t hreg[HP];
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int s = 0; s < 4; ++s) wb[d][vb][s] = wload(min(d, G - 1), vb, s);
#pragma unroll
  for (int i = 0; i < HP; ++i) hreg[i] = *reinterpret_cast<const u32x4_t*>(hsrc[i]);
#pragma unroll
  for (int i = 0; i < HP; ++i) *reinterpret_cast<u32x4_t*>(&sH[0][hdst[i]]) = hreg[i];
  __syncthreads();

  f32x4_t acc[2][MB];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[vb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int g0 = 0; g0 < G; g0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int g = g0 + u;
      const int c = g % nk;
      // every tile uses the same H rows: the next chunk's slice is chunk
      // c + 1, or chunk 0 of the next tile
      const int ch = c + 1 == nk ? 0 : c + 1;
#pragma unroll
      for (int i = 0; i < HP; ++i) hreg[i] = *reinterpret_cast<const u32x4_t*>(hsrc[i] + ch * kKC);
      const bf16_t* sh = sH[u];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          Frag8 hf;
          hf.u = *reinterpret_cast<const uint4*>(&sh[(mb * 16 + l16) * kHRow + 32 * kg + 8 * s]);
#pragma unroll
          for (int vb = 0; vb < 2; ++vb) {
            Frag8 wf;
            wf.q = wb[u][vb][s];
            acc[vb][mb] = mfma16x16x32(wf.v, hf.v, acc[vb][mb]);
          }
        }
      }
      const int gw = min(g + 2, G - 1);  // past the end: reload the last chunk
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int s = 0; s < 4; ++s) wb[u][vb][s] = wload(gw, vb, s);
#pragma unroll
      for (int i = 0; i < HP; ++i) *reinterpret_cast<u32x4_t*>(&sH[u ^ 1][hdst[i]]) = hreg[i];
      __syncthreads();
      if (u == 1 && c == nk - 1) {
        // a tile is complete (its last chunk is odd): fold its per-row keys
        // (and write its logits, when asked), then start the next from zero
        const int v0 = (blockIdx.x + (g / nk) * gridDim.x) * kVT;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int m = mb * 16 + l16;
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
            acc[vb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
          unsigned long long o = shfl_xor_u64(best, 16);
          best = o > best ? o : best;
          o = shfl_xor_u64(best, 32);
          best = o > best ? o : best;
          if (kg == 0) s_wkey[wave][m] = best;
        }
        __syncthreads();
        if (tid < kRowsM) {
          unsigned long long k = s_wkey[0][tid];
#pragma unroll
          for (int w = 1; w < 4; ++w) k = s_wkey[w][tid] > k ? s_wkey[w][tid] : k;
          s_rowkey[tid] = k;
        }
        // (s_wkey and s_rowkey are rewritten only a whole tile of barriers
        // later).  The fold does not wait for its atomics, so the next
        // tile's W loads already in flight are not drained here.
        if (tid < kRowsM && tid < M)
          __hip_atomic_fetch_max(&keys[tid], s_rowkey[tid], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // every key atomic of this wavefront has completed (its acknowledgement
  // counts in vmcnt), then every wavefront's: only then the finish
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  finish_argmax(keys, counter, argmax, M, gridDim.x);
}

// Finish of the partial-key form: one wavefront per row takes the maximum
// over the row's per-tile keys.
__global__ __launch_bounds__(256) void argmax_reduce_kernel(const unsigned long long* __restrict__ part,
                                                            int32_t* __restrict__ argmax, int M,
                                                            int nvt) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= M) return;
  const unsigned long long* row = part + (size_t)m * nvt;
  unsigned long long best = 0ull;
  for (int i = lane; i < nvt; i += 64) best = row[i] > best ? row[i] : best;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long o = shfl_xor_u64(best, off);
    best = o > best ? o : best;
  }
  if (lane == 0) argmax[m] = (int32_t)(~(uint32_t)(best & 0xffffffffull));
}

// Row-major [V][K] -> packed layout; one thread per 16-byte packed piece,
// rows past V written as zeros.
// With inter > 0 the rows are a gate/up weight [2 inter][K] (gate rows, then
// up rows) and are packed interleaved: packed row 128 t + j is gate row
// 64 t + j (j < 64) or up row 64 t + j - 64 (j >= 64).
__global__ __launch_bounds__(256) void pack_kernel(const bf16_t* __restrict__ W,
                                                   bf16_t* __restrict__ P, int K, int V,
                                                   size_t pieces, int inter) {
  const int nk = K / kKC;
  for (size_t p = (size_t)blockIdx.x * blockDim.x + threadIdx.x; p < pieces;
       p += (size_t)gridDim.x * blockDim.x) {
    size_t t = p;
    const int lane = (int)(t % 64);
    t /= 64;
    const int s = (int)(t % 4);
    t /= 4;
    const int j = (int)(t % 8);
    t /= 8;
    const int c = (int)(t % nk);
    const size_t vt = t / nk;
    size_t row = vt * kVT + j * 16 + (lane & 15);
    const int col = c * kKC + 32 * (lane >> 4) + 8 * s;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (inter > 0) {
      const size_t jr = row % kVT;
      row = jr < 64 ? 64 * vt + jr : (size_t)inter + 64 * vt + (jr - 64);
    }
    if (row < (size_t)V) val = *reinterpret_cast<const uint4*>(W + row * K + col);
    reinterpret_cast<uint4*>(P)[p] = val;
  }
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

// Hidden-state rows per workgroup of the bf16 kernel: up to 64 rows keep the
// single-kernel argmax; larger M uses 128-row blocks (each vocabulary tile
// then feeds twice the products) and finishes with argmax_reduce_kernel.
// 256-row blocks measured slower: they fit only one workgroup per CU.
static int lmhead_mb(int M) { return M <= 64 ? 4 : 8; }

// Workspace: per-row keys, then the completion counter on its own 256-byte
// line (this region is zero between calls); for the partial-key form (M >
// 64), one key per (row, vocabulary tile) at the END of the caller's buffer,
// overwritten by every call.  At the end, a call's partial keys never land
// inside the zero region of a later call with more rows (the buffer holds
// that call's zero region plus at least as many partial keys).
size_t lmhead_zero_bytes(int M) { return ((size_t)M * 8 + 255) / 256 * 256 + 256; }

size_t lmhead_ws_bytes(int M, int /*K*/, int V, int dtype) {
  size_t bytes = lmhead_zero_bytes(M);
  if (dtype == TV_BF16 && lmhead_mb(M) != 4) bytes += (size_t)M * ((V + kVT - 1) / kVT) * 8;
  return bytes;
}

size_t lmhead_packed_bytes(int V, int K) {
  return (size_t)((V + kVT - 1) / kVT) * kVT * (size_t)K * sizeof(bf16_t);
}

hipError_t launch_lmhead_pack(const void* w, void* packed, int V, int K, hipStream_t stream) {
  const size_t pieces = lmhead_packed_bytes(V, K) / 16;
  hipLaunchKernelGGL(pack_kernel, dim3(4096), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(w), static_cast<bf16_t*>(packed), K, V, pieces, 0);
  return hipGetLastError();
}

hipError_t launch_pack_gate_up(const void* w, void* packed, int inter, int K,
                               hipStream_t stream) {
  const size_t pieces = lmhead_packed_bytes(2 * inter, K) / 16;
  hipLaunchKernelGGL(pack_kernel, dim3(4096), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(w), static_cast<bf16_t*>(packed), K, 2 * inter,
                     pieces, inter);
  return hipGetLastError();
}


// Workgroups of lmhead_stream_kernel resident at once on the current device
// (its grid), queried once per device.
static int stream_grid() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, lmhead_stream_kernel, kThreads, 0) !=
            hipSuccess || per_cu < 1)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
    cached[dev] = per_cu * cus;
  }
  return cached[dev];
}

hipError_t launch_lmhead_argmax(const void* hidden, const void* w, int32_t* argmax,
                                float* logits, int M, int K, int V, int dtype, int w_layout,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
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
  const int mb = lmhead_mb(M);
  const int nmt = (M + 16 * mb - 1) / (16 * mb);
  const int nvt = (V + kVT - 1) / kVT;
  const int total = nmt * nvt;
  const bf16_t* h = static_cast<const bf16_t*>(hidden);
  const bf16_t* wv = static_cast<const bf16_t*>(w);
  const bool pk = w_layout == TV_LAYOUT_PACKED;
  const dim3 grid(total), block(kThreads);
  if (mb != 4) {
    const size_t pbytes = (size_t)M * (pk ? gemm_argmax_vtiles(M, V) : nvt) * 8;
    keys = reinterpret_cast<unsigned long long*>(static_cast<char*>(ws) +
                                                 ((ws_bytes - pbytes) & ~(size_t)255));
  }
  if (mb != 4 && pk) {
    // many rows: the matrix-core tiling (256-row W tiles), then the reduce
    hipError_t e = launch_gemm32_argmax(h, wv, keys, logits, M, K, V, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(argmax_reduce_kernel, dim3((M + 3) / 4), dim3(256), 0, stream, keys,
                       argmax, M, gemm_argmax_vtiles(M, V));
    return hipGetLastError();
  }
#define TV_LM_LAUNCH(P, MBV, MODEV)                                                         \
  hipLaunchKernelGGL((lmhead_bf16_kernel<P, MBV, MODEV>), grid, block, 0, stream, h, wv, argmax, \
                     logits, keys, counter, M, K, V, nmt, total, nullptr, 1, nullptr, 0)
  if (mb == 4 && pk) {
    const int g = stream_grid();
    hipLaunchKernelGGL(lmhead_stream_kernel, dim3(nvt < g ? nvt : g), block, 0, stream, h, wv,
                       argmax, logits, keys, counter, M, K, V, nvt);
    return hipGetLastError();
  }
  if (mb == 4) {
    if (pk) TV_LM_LAUNCH(true, 4, kArgmaxCommit); else TV_LM_LAUNCH(false, 4, kArgmaxCommit);
  } else {
    if (pk) TV_LM_LAUNCH(true, 8, kArgmaxPartial); else TV_LM_LAUNCH(false, 8, kArgmaxPartial);
  }
#undef TV_LM_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || mb == 4) return e;
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3((M + 3) / 4), dim3(256), 0, stream, keys, argmax,
                     M, nvt);
  return hipGetLastError();
}

// Chunks per trip of the projection kernel (one row block): 4 (two-deep W
// ring, four-deep H prefetch) when K holds whole groups of four chunks,
// else 2 (both two-deep).
static int proj_ring(int M, int K) {
  return lmhead_mb(M) == 4 && (K / kKC) % 4 == 0 ? 4 : 2;
}

// Splits of a projection: the largest count that divides the k groups evenly
// and keeps the grid at one workgroup per CU or fewer (a partly doubled-up
// grid runs at the speed of its doubled CUs: measured 40% slower at 320
// workgroups than at 256 for the 4096 x 4096 case).
int proj_splits(int M, int K, int Nout) {
  if (lmhead_mb(M) != 4) return gemm32_splits(M, K, Nout);
  const int nmt = (M + 16 * lmhead_mb(M) - 1) / (16 * lmhead_mb(M));
  const int tiles = nmt * ((Nout + kVT - 1) / kVT);
  const int ngroup = K / (kKC * proj_ring(M, K));
  int best = 1;
  for (int s = 1; s <= ngroup; ++s)
    if (ngroup % s == 0 && (long)s * tiles <= 256) best = s;
  return best;
}

bool proj_swiglu_fused(int M, int K, int inter) {
  return lmhead_mb(M) == 4 && proj_splits(M, K, 2 * inter) == 1;
}

hipError_t launch_proj_swiglu(const void* hidden, const void* w_gu_packed, void* act, int M,
                              int K, int inter, hipStream_t stream) {
  const int total = (2 * inter + kVT - 1) / kVT;  // one row block, one split
  const bf16_t* h = static_cast<const bf16_t*>(hidden);
  const bf16_t* wv = static_cast<const bf16_t*>(w_gu_packed);
  bf16_t* a = static_cast<bf16_t*>(act);
  if (proj_ring(M, K) == 4)
    hipLaunchKernelGGL((lmhead_bf16_kernel<true, 4, kSwiGLU, 2, 4>), dim3(total), dim3(kThreads),
                       0, stream, h, wv, nullptr, nullptr, nullptr, nullptr, M, K, 2 * inter, 1,
                       total, nullptr, 1, a, inter);
  else
    hipLaunchKernelGGL((lmhead_bf16_kernel<true, 4, kSwiGLU, 2, 2>), dim3(total), dim3(kThreads),
                       0, stream, h, wv, nullptr, nullptr, nullptr, nullptr, M, K, 2 * inter, 1,
                       total, nullptr, 1, a, inter);
  return hipGetLastError();
}

hipError_t launch_proj(const void* hidden, const void* w_packed, float* part, int M, int K,
                       int Nout, int nsplit, hipStream_t stream) {
  const int mb = lmhead_mb(M);
  if (mb != 4) return launch_gemm32_store(hidden, w_packed, part, M, K, Nout, nsplit, stream);
  const int nmt = (M + 16 * mb - 1) / (16 * mb);
  const int total = nmt * ((Nout + kVT - 1) / kVT) * nsplit;
  const bf16_t* h = static_cast<const bf16_t*>(hidden);
  const bf16_t* wv = static_cast<const bf16_t*>(w_packed);
  if (mb == 4 && proj_ring(M, K) == 4)
    hipLaunchKernelGGL((lmhead_bf16_kernel<true, 4, kStorePartial, 2, 4>), dim3(total),
                       dim3(kThreads), 0, stream, h, wv, nullptr, nullptr, nullptr, nullptr, M,
                       K, Nout, nmt, total, part, nsplit, nullptr, 0);
  else if (mb == 4)
    hipLaunchKernelGGL((lmhead_bf16_kernel<true, 4, kStorePartial, 2, 2>), dim3(total),
                       dim3(kThreads), 0, stream, h, wv, nullptr, nullptr, nullptr, nullptr, M,
                       K, Nout, nmt, total, part, nsplit, nullptr, 0);
  else
    hipLaunchKernelGGL((lmhead_bf16_kernel<true, 8, kStorePartial, 2>), dim3(total),
                       dim3(kThreads), 0, stream, h, wv, nullptr, nullptr, nullptr, nullptr, M,
                       K, Nout, nmt, total, part, nsplit, nullptr, 0);
  return hipGetLastError();
}

}  // namespace tv
