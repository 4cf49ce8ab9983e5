// Tree-causal verification attention.
//
// Method (JetSpec GitHub README, "JetSpec > Overview"): the target verifies
// the whole draft tree in one forward pass under a tree-causal mask.  Node i
// of sequence b sees the prefix (cache rows 0..L_b-1) and the tree nodes on
// its own root path (rows L_b+j, j an ancestor of i or i itself):
//     out[b][i][h] = softmax(scale * q K_vis^T) V_vis,   KV head = h / G.
//
// bf16 kernel (gfx950 matrix cores), attn_bf16_kernel<D, QBW, NW>:
//   * A workgroup of NW wavefronts owns NW*QBW*16 query rows of one
//     (sequence, KV head); row r is node r / G, head r % G of the group, so
//     the G heads of a node - which share every key and the whole mask - are
//     adjacent, and each 64-key K/V tile staged in LDS serves every row.
//   * Per tile: S^T = K Q^T on 16x16x32 bf16 MFMA (Q^T fragments stay in
//     registers), online softmax, O^T += V^T P^T.  With the transposed
//     products each lane owns one query column in both results, so the
//     softmax state never moves between lanes and the probabilities feed the
//     second product straight from registers (the key order inside a 32-wide
//     k-step is permuted identically in V^T and P^T).
//   * D = 128: a tile's K and V rows go straight from memory into LDS
//     (global_load_lds), the next tile's into a second buffer pair while
//     this tile's products run; V stays row-major and the V^T operand comes
//     from the transposing LDS read of gfx950 (ds_read_b64_tr_b16).  D = 64:
//     tiles are staged through registers and V is transposed on its way
//     into LDS.  Loads are unconditional (rows past the valid range are
//     clamped to a valid row and masked out of the scores), so a tile's
//     loads are all in flight at once.
//   * Softmax in the exp2 domain: one FMA folds the scale and the running
//     max, then v_exp_f32; probabilities go to bf16 with v_cvt_pk_bf16_f32.
//     The running reference max moves only when a wavefront sees a score more
//     than 2^8 above it (rescaling O and the sum); until then probabilities up
//     to 2^8 accumulate exactly as they would after a rescale.
//   * Masking runs only on tree tiles and partial tiles.  The mask is one
//     64-bit ancestor word per (node, 64-key tree tile), built in LDS by
//     walking parent pointers (TV_STATUS_BAD_PARENT on a malformed tree);
//     tree tiles that no node of the block can see are skipped.
//   * Long prefixes can be split across workgroups (split-KV): each writes
//     fp32 (reference max, sum, unnormalised output) partials and a combine
//     kernel merges them; the tree keys then get the last split to
//     themselves.
//   * Workgroup ids are remapped so that the blocks reading the same K/V rows
//     run on the same die (shared L2).
// fp32 kernel: a plain VALU kernel for small fp32 problems.
#include <type_traits>

#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kKT = 64;     // keys per tile
constexpr int kKPad = 8;    // bf16 padding of a K row in LDS
// V^T rows in LDS are unpadded; the 4-key (8-byte) units of row d are
// XOR-swizzled by vt_swz(d), which makes both the transposing stores (16
// lanes on 16 rows 8 apart) and the PV operand reads (16 lanes on 16
// consecutive rows) free of bank conflicts.
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 3) ^ d) & 15; }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;  // rescale when a score exceeds the reference by 2^8
// s_waitcnt operand: every counter at zero (all loads and LDS operations
// of the wavefront complete)
constexpr int kWaitAll0 = 0x0000;

struct AttnArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const int32_t* seq_lens;
  const int32_t* parent;
  bf16_t* out;
  float* part_o;   // [B*Hkv][nqblk*rows][nsplit][D] fp32 (ragged: [item][Hkv][nqblk*rows][D])
  float* part_ml;  // [B*Hkv][nqblk*rows][nsplit][2] fp32 (ragged: [item][Hkv][nqblk*rows][2])
  int32_t* dev_status;
  int B, N, Hq, Hkv, G, Lcap, max_seq_len;
  int rows;        // query rows per workgroup
  int nqblk, nsplit, chunk_len, total_blocks;
  // ragged batches: per-sequence splits derived on the device from the
  // lengths (ragged_plan); nsplit and chunk_len above are then unused
  int ragged, want_blocks, min_tiles;
  int* ragged_start;  // [B + 1] (ragged): workgroup 0 publishes the plan here for the combine
  int anc_words;   // ceil(N / 64)
  float scale_log2;  // scale * log2(e)
  // paged caches (block_table != nullptr): pools [num_pages][Hkv][ps][D],
  // logical row r of sequence b in page block_table[b][r >> page_shift]
  const int32_t* block_table;
  int max_blocks, page_shift, num_pages;
};

__device__ __forceinline__ void flag(int32_t* st, int b, int f) {
  if (st) atomicOr(&st[b], f);
}

// Maxima of scores that are never NaN.  fmaxf must quiet signalling NaNs, so
// the compiler puts a v_max(x, x) in front of every operand it cannot prove
// canonical; v_max3_f32 written out takes three operands with no such step.
__device__ __forceinline__ float max3f(float x, float y, float z) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}
__device__ __forceinline__ float smax(float x, float y) { return max3f(x, y, y); }

// Reductions across the four 16-lane groups of a wavefront (lanes l, l^16,
// l^32, l^48) with the gfx950 row/half swaps: each swap returns both
// operands exchanged, so combining its two results pairs every lane with
// its partner without a trip through LDS.
__device__ __forceinline__ float max_across_groups(float x) {
  auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = smax(__uint_as_float(h[0]), __uint_as_float(h[1]));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return smax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_groups(float x) {
  auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Prefix splits of a ragged batch (at most kMaxRaggedB sequences), derived
// from the lengths so that every split holds about the same number of key
// tiles whatever the mix of lengths: chunk = max(min_tiles, ceil(total tiles
// x Hkv x query blocks / want_blocks)) tiles,
// nsplit_b = max(1, ceil(tiles_b / chunk)), and every sequence with more
// than one split gets one more for its tree keys while the whole grid stays
// within want_blocks.  Work items (b, split) are numbered sequence by
// sequence; start[b] is the first item of sequence b, start[B] the count.
// Every workgroup of a launch derives the same plan (wavefront 0 computes it,
// one sequence per lane; a barrier publishes it).  A length outside
// [0, max_seq_len] counts as no prefix (its workgroups flag it and return).
constexpr int kMaxRaggedB = kMaxRaggedBatch;

struct RaggedPlan {
  const int* start;  // [B + 1], in LDS
  int chunk_len;     // keys per prefix split
};

__device__ RaggedPlan ragged_plan(const AttnArgs& a) {
  __shared__ int sStart[kMaxRaggedB + 1];
  __shared__ int sChunk;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    int tiles = 0;
    if (lane < a.B) {
      const int L = a.seq_lens[lane];
      tiles = (L >= 0 && L <= a.max_seq_len) ? (L + kKT - 1) / kKT : 0;
    }
    int total = tiles, most = tiles;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      total += __shfl_xor(total, off, 64);
      most = max(most, __shfl_xor(most, off, 64));
    }
    const long hq = (long)a.Hkv * a.nqblk;
    auto items_at = [&](long c) {  // work items of the batch with chunks of c tiles
      int n = lane < a.B ? max(1, (int)((tiles + c - 1) / c)) : 0;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off, 64);
      return (long)n;
    };
    // the smallest chunk (at least the even share and min_tiles) whose items
    // fit the workgroup target: the per-sequence rounding up must not push
    // the grid into a second round
    long ct = ((long)total * hq + a.want_blocks - 1) / a.want_blocks;
    if (ct < a.min_tiles) ct = a.min_tiles;
    long hi = most > ct ? most : ct;
    while (ct < hi && items_at(ct) * hq > a.want_blocks) {  // non-increasing in ct
      const long mid = (ct + hi) / 2;
      if (items_at(mid) * hq <= a.want_blocks) hi = mid;
      else ct = mid + 1;
    }
    int ns = lane < a.B ? max(1, (int)((tiles + ct - 1) / ct)) : 0;
    const int with_tree = ns + (ns > 1 ? 1 : 0);
    int sum_tree = with_tree;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum_tree += __shfl_xor(sum_tree, off, 64);
    if ((long)sum_tree * hq <= a.want_blocks) ns = with_tree;
    int incl = ns;  // inclusive scan over the lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane < a.B) sStart[lane] = incl - ns;
    if (lane == a.B - 1) sStart[a.B] = incl;
    if (lane == 0) sChunk = (int)ct * kKT;
  }
  __syncthreads();
  return RaggedPlan{sStart, sChunk};
}

template <int D, int QBW, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int kThreads = NW * 64;
  constexpr int kRows = NW * QBW * 16;
  constexpr int DS = D / 32;  // k-steps of the QK^T product
  constexpr int DB = D / 16;  // 16-row output blocks of the PV product
  constexpr int KROW = D + kKPad;
  constexpr int VROW = kKT;
  constexpr int KP_TOTAL = kKT * D / 8;           // 16-byte pieces of a K tile
  constexpr int KP = (KP_TOTAL + kThreads - 1) / kThreads;
  constexpr int VI_TOTAL = (kKT / 4) * (D / 8);   // 4-key x 8-dim items of a V tile
  constexpr int VI = (VI_TOTAL + kThreads - 1) / kThreads;
  constexpr int kMaxAncNodes = kRows + 2;
  // D = 128: K and V tiles go straight from memory into two LDS buffers
  // each (unpadded, swizzled), and the ancestor words live in dynamic LDS
  // sized to the tree; D = 64: one padded K buffer and V^T, staged through
  // registers.
  constexpr bool kDma = (D == 128);
  __shared__ __attribute__((aligned(1024))) bf16_t sK0[kKT * (kDma ? D : KROW)];
  __shared__ __attribute__((aligned(1024))) bf16_t sK1[kDma ? kKT * D : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t sV0[kDma ? kKT * D : D * VROW];
  __shared__ __attribute__((aligned(1024))) bf16_t sV1[kDma ? kKT * D : 8];
  bf16_t* const sK = sK0;
  bf16_t* const sVt = sV0;
  __shared__ int16_t sPar[TV_MAX_NODES];
  __shared__ unsigned long long sAncStatic[kDma ? 1 : kMaxAncNodes * (TV_MAX_NODES / 64)];
  extern __shared__ unsigned long long sAncDyn[];
  unsigned long long* const sAnc = kDma ? sAncDyn : sAncStatic;
  __shared__ unsigned sTreeMask;
  __shared__ int8_t sTreeList[TV_MAX_NODES / 64];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS addresses
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int kg = lane >> 4;

  // ---- which (sequence, KV head, split, query block) this workgroup owns
  int t, qblk, b, g, split, nsplit, chunk_len, item = 0;
  if (a.ragged) {
    // the grid covers the most items any lengths can give; the first
    // `active` workgroup ids (dealt round-robin to the dies) do the work, and
    // the remap over that count keeps each die's share contiguous
    const RaggedPlan rp = ragged_plan(a);
    if (blockIdx.x == 0 && tid <= a.B) a.ragged_start[tid] = rp.start[tid];
    const int active = rp.start[a.B] * a.Hkv * a.nqblk;
    if ((int)blockIdx.x >= active) return;
    t = xcd_remap(blockIdx.x, active);
    qblk = t % a.nqblk;
    t /= a.nqblk;
    g = t % a.Hkv;
    item = t / a.Hkv;
    b = 0;
    while (b + 1 < a.B && rp.start[b + 1] <= item) ++b;
    split = item - rp.start[b];
    nsplit = rp.start[b + 1] - rp.start[b];
    chunk_len = rp.chunk_len;
  } else {
    t = xcd_remap(blockIdx.x, a.total_blocks);
    qblk = t % a.nqblk;
    t /= a.nqblk;
    split = t % a.nsplit;
    t /= a.nsplit;
    g = t % a.Hkv;
    b = t / a.Hkv;
    nsplit = a.nsplit;
    chunk_len = a.chunk_len;
  }

  const int N = a.N, G = a.G;
  const int R = N * G;
  const int L = a.seq_lens[b];
  if (L < 0 || L > a.max_seq_len || L + N > a.Lcap) {
    if (tid == 0) flag(a.dev_status, b, TV_STATUS_BAD_LEN);
    return;
  }
  const int row0 = qblk * kRows;
  const int node_lo = row0 / G;
  const int node_hi = (min(R, row0 + kRows) - 1) / G;
  const bool do_tree = (split == nsplit - 1);
  const int c0 = split * chunk_len;
  const int c1 = min(c0 + chunk_len, L);
  const int W = a.anc_words;

  // ---- ancestor words of the block's nodes and the tree tiles they touch
  int n_tree = 0;
  if (do_tree) {
    const int32_t* par = a.parent + (size_t)b * N;
    int bad = 0;
    for (int i = tid; i <= node_hi; i += kThreads) {
      const int p = par[i];
      const bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i);
      bad |= !ok;
      sPar[i] = (int16_t)(ok ? p : -1);
    }
    const int nn = node_hi - node_lo + 1;
    for (int x = tid; x < nn * W; x += kThreads) sAnc[x] = 0ull;
    if (tid == 0) sTreeMask = 0u;
    __syncthreads();
    for (int n = tid; n < nn; n += kThreads) {
      unsigned long long* w = sAnc + n * W;
      unsigned used = 0u;
      int j = node_lo + n;
      while (j >= 0) {  // parent[j] < j, so this ends within j + 1 steps
        w[j >> 6] |= 1ull << (j & 63);
        used |= 1u << (j >> 6);
        j = (j == 0) ? -1 : sPar[j];
      }
      atomicOr(&sTreeMask, used);
    }
    if (bad) flag(a.dev_status, b, TV_STATUS_BAD_PARENT);
    __syncthreads();
    const unsigned mask = sTreeMask;
    n_tree = __popc(mask);
    if (tid == 0) {
      int k = 0;
      for (int tt = 0; tt < W; ++tt)
        if (mask & (1u << tt)) sTreeList[k++] = (int8_t)tt;
    }
    // (published to the other threads by the first barrier of the tile loop)
  }

  // ---- where key/value rows live: one contiguous plane per (sequence, KV
  // head), or pages of a pool named by the block table.  For pages, the lanes
  // that load a row look up its page entry themselves (a 4-byte load; a
  // sequence's entries are read by all its query blocks, so they sit in L2;
  // a whole prefix tile with pages of 16 rows or more takes one entry per
  // wavefront):
  // no entries are staged in LDS, so neither the page size nor the length of
  // a split is bounded by LDS.  An entry outside the pool reads page 0 and
  // flags TV_STATUS_BAD_PAGE at the end.
  const size_t kv_plane = ((size_t)b * a.Hkv + g) * (size_t)a.Lcap * D;
  const int sh = a.page_shift;
  const int32_t* bt = PAGED ? a.block_table + (size_t)b * a.max_blocks : nullptr;
  int bad_page = 0;
  auto row_off = [&](int row, bool tree) -> size_t {
    (void)tree;
    if constexpr (PAGED) {
      int pg = bt[row >> sh];
      if ((unsigned)pg >= (unsigned)a.num_pages) {
        bad_page = 1;
        pg = 0;
      }
      return ((((size_t)pg * a.Hkv + g) << sh) + (row & ((1 << sh) - 1))) * D;
    } else {
      return kv_plane + (size_t)row * D;
    }
  };

  // ---- Q^T fragments of this lane's query columns
  bf16x8_t qf[QBW][DS];
  int qnode[QBW];
  bool qvalid[QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const int row = row0 + wave * QBW * 16 + qb * 16 + l16;
    qvalid[qb] = row < R;
    const int node = qvalid[qb] ? row / G : node_hi;
    const int hh = qvalid[qb] ? row - node * G : 0;
    qnode[qb] = node;
    const bf16_t* qrow = a.q + (((size_t)b * N + node) * a.Hq + (size_t)g * G + hh) * D;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      Frag8 f;
      f.u = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * kg);
      qf[qb][s] = f.v;
    }
  }

  float m_ref[QBW], l_run[QBW];
  f32x4_t o[QBW][DB];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    m_ref[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int n_pre = (c1 > c0) ? (c1 - c0 + kKT - 1) / kKT : 0;
  const int n_tiles = n_pre + n_tree;

  // Tile descriptor: first cache row and number of valid keys.
  auto tile_rows = [&](int it, int& krow0, int& nvalid, int& tt) {
    if (it < n_pre) {
      krow0 = c0 + it * kKT;
      nvalid = min(kKT, c1 - krow0);
      tt = -1;
    } else {
      tt = sTreeList[it - n_pre];
      krow0 = L + tt * kKT;
      nvalid = min(kKT, N - tt * kKT);
    }
  };

  // Register staging of one tile: K pieces and V 4-key items.
  u32x4_t kreg[KP];
  u32x4_t vreg[VI][4];
  auto load_tile = [&](int krow0, int nvalid, bool tree) {
    const int last = krow0 + nvalid - 1;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int c = min(tid + i * kThreads, KP_TOTAL - 1);
      const int r = c / (D / 8);
      const int x = c - r * (D / 8);
      kreg[i] = *reinterpret_cast<const u32x4_t*>(a.k + row_off(min(krow0 + r, last), tree) + x * 8);
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int c = min(tid + i * kThreads, VI_TOTAL - 1);
      const int kq = c / (D / 8);
      const int x = c - kq * (D / 8);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        vreg[i][e] = *reinterpret_cast<const u32x4_t*>(a.v + row_off(min(krow0 + kq * 4 + e, last), tree) + x * 8);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int c = min(tid + i * kThreads, KP_TOTAL - 1);
      const int r = c / (D / 8);
      const int x = c - r * (D / 8);
      *reinterpret_cast<u32x4_t*>(&sK[r * KROW + x * 8]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int c = min(tid + i * kThreads, VI_TOTAL - 1);
      const int kq = c / (D / 8);
      const int x = c - kq * (D / 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // element e of keys 4kq .. 4kq+3, packed as two bf16 pairs:
        // v_perm picks the low (e even) or high (e odd) halves of two words
        const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2_t pk;
        pk.x = __builtin_amdgcn_perm(vreg[i][1][e >> 1], vreg[i][0][e >> 1], sel);
        pk.y = __builtin_amdgcn_perm(vreg[i][3][e >> 1], vreg[i][2][e >> 1], sel);
        const int d = x * 8 + e;
        *reinterpret_cast<u32x2_t*>(&sVt[d * VROW + ((kq ^ vt_swz(d)) << 2)]) = pk;
      }
    }
  };

  // One tile's products once its K rows and V are in LDS (read through
  // kfrag and vfrag): S^T = K Q^T, mask, online softmax, O^T += V^T P^T.
  // All K fragments of the tile are read before the first product and all
  // V fragments before the softmax, so each phase waits on LDS once instead
  // of once per fragment.
  auto compute_tile = [&](int nvalid, int tt, auto kfrag, auto vfrag) {
    const bool tree = tt >= 0;
    const bool need_mask = tree || nvalid < kKT;
    Frag8 kf[4][DS];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int ks = 0; ks < DS; ++ks) kf[kb][ks].u = kfrag(kb, ks);
    // S^T = K Q^T: lane holds query column l16, keys kb*16 + 4*kg + r.  The
    // k step is the outer loop (and in O^T += V^T P^T below the key half u), so
    // eight independent products separate two into one accumulator and the
    // second half's exponentials can run under the first half's products;
    // each accumulator still sums in the same order.
    f32x4_t s[QBW][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) s[qb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) s[qb][kb] = mfma16x16x32(kf[kb][ks].v, qf[qb][ks], s[qb][kb]);
    if constexpr (kDma) {
      // The next tile's copies (issued just before, in this basic block) go
      // out among these products, one per QBW products after the K fragment
      // reads, instead of all ahead of them, where the wavefront waited at
      // issue while the memory path drained them (2-3 % on the long-prefix
      // workloads; one per 2 QBW products gained less).
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * DS, 0);  // LDS reads: K fragments
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // matrix instruction
#pragma unroll
      for (int k = 0; k < 2 * kKT / (4 * NW); ++k) {
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);     // vector memory (a copy)
        __builtin_amdgcn_sched_group_barrier(0x008, QBW, 0);
      }
    }
    // O^T += V^T P^T below reads these (the first half of the output rows'
    // fragments are in flight during the softmax, the second half during the
    // first half's products); k-slot e of lane group kg is key 32u + 4kg + e
    // (e < 4) or 32u + 16 + 4kg + e - 4 (e >= 4), in both operands.
    constexpr int DH = DB / 2;
    Frag8 vf[DB][2];
#pragma unroll
    for (int db = 0; db < DH; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u) vf[db][u].u = vfrag(db, u);

    // mask (only where needed), then the online softmax in the exp2 domain
    Frag8 pf[QBW][2];
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      if (need_mask) {
        // visible keys of this query as a 64-bit word (ancestor bits, keys
        // past the tile's valid rows cleared); this lane's keys kb*16 +
        // 4kg + r are bits kb*16 + r of the word shifted right by 4kg
        unsigned long long word = tree ? sAnc[(qnode[qb] - node_lo) * W + tt] : ~0ull;
        if (nvalid < kKT) word &= (1ull << nvalid) - 1ull;
        const uint32_t wlo = (uint32_t)(word >> (4 * kg));
        const uint32_t whi = (uint32_t)(word >> (32 + 4 * kg));
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // all ones where the key is visible: the score, else -inf
            const uint32_t keep =
                (uint32_t)__builtin_amdgcn_sbfe((int)(kb < 2 ? wlo : whi), (kb & 1) * 16 + r, 1);
            s[qb][kb][r] = __uint_as_float((__float_as_uint(s[qb][kb][r]) & keep) | (~keep & 0xff800000u));
          }
      }
      const float m0 = max3f(s[qb][0][0], s[qb][0][1], s[qb][0][2]);
      const float m1 = max3f(s[qb][0][3], s[qb][1][0], s[qb][1][1]);
      const float m2 = max3f(s[qb][1][2], s[qb][1][3], s[qb][2][0]);
      const float m3 = max3f(s[qb][2][1], s[qb][2][2], s[qb][2][3]);
      const float m4 = max3f(s[qb][3][0], s[qb][3][1], s[qb][3][2]);
      const float lmax = max3f(max3f(m0, m1, m2), max3f(m3, m4, s[qb][3][3]), -INFINITY);
      // a query's tile maximum exceeds the threshold exactly when one of its
      // four lane groups' maxima does, so the maximum across the groups is
      // only formed for a rescale
      if (__any(lmax * a.scale_log2 > m_ref[qb] + kLazy)) {
        const float tm = max_across_groups(lmax) * a.scale_log2;
        const float m_new = smax(m_ref[qb], tm);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref[qb] - m_new);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
        m_ref[qb] = m_new;
      }
      const float mu = (m_ref[qb] == -INFINITY) ? 0.f : m_ref[qb];
      float p[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][r], a.scale_log2, -mu));
      float ps[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) ps[kb] = (p[kb][0] + p[kb][1]) + (p[kb][2] + p[kb][3]);
      l_run[qb] += (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        pf[qb][u].u = make_uint4(pack_bf16x2(p[2 * u][0], p[2 * u][1]),
                                 pack_bf16x2(p[2 * u][2], p[2 * u][3]),
                                 pack_bf16x2(p[2 * u + 1][0], p[2 * u + 1][1]),
                                 pack_bf16x2(p[2 * u + 1][2], p[2 * u + 1][3]));
    }

#pragma unroll
    for (int db = DH; db < DB; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u) vf[db][u].u = vfrag(db, u);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) o[qb][db] = mfma16x16x32(vf[db][u].v, pf[qb][u].v, o[qb][db]);
  };

  if constexpr (kDma) {
    // Tiles go straight from memory into LDS, the next tile's into the
    // other buffer pair while this tile's products run; each tile ends
    // waiting for the next one's loads (issued a tile of products earlier)
    // and meeting at one barrier.  The buffers are separate LDS objects used
    // with compile-time indices, so no read of one waits for loads into the
    // other.  Layouts (16-byte pieces of a 256-byte row r):
    //   K: piece x at position x ^ (r & 15): the fragment reads (16 rows,
    //      one piece each) touch every bank once;
    //   V: piece x at position x ^ 2 (r & 3): the transposing reads (4 rows
    //      x 4 eight-byte units per 16 lanes) touch 32 distinct banks.
    auto tdma = [&](bf16_t* kbuf, bf16_t* vbuf, int krow0, int nvalid, bool tree) {
      if constexpr (PAGED) {
        if (!tree && nvalid == kKT && sh >= 4) {
          // a whole prefix tile (krow0 a multiple of 64): each wavefront's 16
          // rows lie in one page of at least 16 rows, one entry per wavefront
          const int r0 = (kKT / NW) * wave;
          int pg = bt[(krow0 + r0) >> sh];
          if ((unsigned)pg >= (unsigned)a.num_pages) {
            bad_page = 1;
            pg = 0;
          }
          const size_t pbase = (((size_t)pg * a.Hkv + g) << sh) * D;
#pragma unroll
          for (int i = 0; i < kKT / (4 * NW); ++i) {
            const int r = r0 + 4 * i + (lane >> 4);
            const size_t ro = pbase + (size_t)((krow0 + r) & ((1 << sh) - 1)) * D;
            const int xk = (lane & 15) ^ (r & 15);
            const int xv = (lane & 15) ^ (2 * (r & 3));
            const int dst = ((kKT / NW) * wave + 4 * i) * D;
            __builtin_amdgcn_global_load_lds((const void*)(a.k + ro + xk * 8),
                                             (__attribute__((address_space(3))) void*)(kbuf + dst),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(a.v + ro + xv * 8),
                                             (__attribute__((address_space(3))) void*)(vbuf + dst),
                                             16, 0, 0);
          }
          return;
        }
      }
      const int last = krow0 + nvalid - 1;
#pragma unroll
      for (int i = 0; i < kKT / (4 * NW); ++i) {
        const int r = (kKT / NW) * wave + 4 * i + (lane >> 4);
        const size_t ro = row_off(min(krow0 + r, last), tree);
        const int xk = (lane & 15) ^ (r & 15);
        const int xv = (lane & 15) ^ (2 * (r & 3));
        const int dst = ((kKT / NW) * wave + 4 * i) * D;
        __builtin_amdgcn_global_load_lds((const void*)(a.k + ro + xk * 8),
                                         (__attribute__((address_space(3))) void*)(kbuf + dst), 16,
                                         0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(a.v + ro + xv * 8),
                                         (__attribute__((address_space(3))) void*)(vbuf + dst), 16,
                                         0, 0);
      }
    };
    auto step = [&](int it, auto buf_tag) {
      constexpr int U = decltype(buf_tag)::value;
      const bf16_t* kb_lds = U ? sK1 : sK0;
      const bf16_t* vb_lds = U ? sV1 : sV0;
      int krow0, nvalid, tt;
      tile_rows(it, krow0, nvalid, tt);
      {
        // the next tile's copies; the last tile copies itself again into the
        // free buffers (never read: an L2 hit), so that the copies share a
        // basic block with the products they are spread among
        int k1r, n1, t1;
        tile_rows(min(it + 1, n_tiles - 1), k1r, n1, t1);
        tdma(U ? sK0 : sK1, U ? sV0 : sV1, k1r, n1, t1 >= 0);
      }
      // V^T operand rows d = db*16 + l16 for keys key0 .. key0+3: lane j of
      // a 16-lane group points at key key0 + j/4, dims db*16 + 4 (j % 4) ..
      // + 3, and the transposing read hands lane j dim db*16 + j of the four
      // keys.
      auto vtr = [&](int db, int key0) -> u32x2_t {
        const int r = key0 + (l16 >> 2);
        const int x = 2 * db + ((l16 & 3) >> 1);
        const bf16_t* ptr = vb_lds + r * D + ((x ^ (2 * (r & 3))) * 8) + (l16 & 1) * 4;
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        const v4i16 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)ptr);
        return __builtin_bit_cast(u32x2_t, t4);
      };
      compute_tile(
          nvalid, tt,
          [&](int kb, int ks) -> uint4 {
            const int pos = (4 * ks + kg) ^ l16;  // row kb*16 + l16: (row & 15) == l16
            return *reinterpret_cast<const uint4*>(kb_lds + (kb * 16 + l16) * D + pos * 8);
          },
          [&](int db, int u) -> uint4 {
            const u32x2_t lo = vtr(db, 32 * u + 4 * kg);
            const u32x2_t hi = vtr(db, 32 * u + 16 + 4 * kg);
            return make_uint4(lo.x, lo.y, hi.x, hi.y);
          });
      // the next tile is in this wavefront's part of the buffers and its LDS
      // reads of this tile are done; after the barrier, everyone's
      __builtin_amdgcn_s_waitcnt(kWaitAll0);
      __builtin_amdgcn_s_barrier();
    };
    __syncthreads();  // tree tile list (and page entries) visible
    if (n_tiles > 0) {
      int kr, nv, tq;
      tile_rows(0, kr, nv, tq);
      tdma(sK0, sV0, kr, nv, tq >= 0);
      __builtin_amdgcn_s_waitcnt(kWaitAll0);
      __builtin_amdgcn_s_barrier();
    }
    for (int it = 0; it < n_tiles; it += 2) {
      step(it, std::integral_constant<int, 0>{});
      if (it + 1 < n_tiles) step(it + 1, std::integral_constant<int, 1>{});
    }
  } else {
    // D = 64, tiles staged through registers.  The 128-row variant issues a
    // tile's loads back to back and does not hold them across the products
    // (with two workgroups per CU, one workgroup's loads overlap another's
    // products).  The 64-row variant runs at small sizes with few
    // workgroups per CU, so it issues the next tile's loads right after
    // staging the current one and hides their latency behind the products.
    constexpr bool kPrefetch = (QBW == 1);
    if constexpr (kPrefetch) {
      __syncthreads();  // tree tile list (and page entries) visible
      if (n_tiles > 0) {
        int k0r, n0, t0;
        tile_rows(0, k0r, n0, t0);
        load_tile(k0r, n0, t0 >= 0);
      }
    }
    for (int it = 0; it < n_tiles; ++it) {
      int krow0, nvalid, tt;
      __syncthreads();  // previous tile consumed (first trip: tree tile list visible)
      tile_rows(it, krow0, nvalid, tt);
      if constexpr (!kPrefetch) load_tile(krow0, nvalid, tt >= 0);
      store_tile();
      __syncthreads();  // this tile is in LDS
      if constexpr (kPrefetch) {
        if (it + 1 < n_tiles) {
          int k1r, n1, t1;
          tile_rows(it + 1, k1r, n1, t1);
          load_tile(k1r, n1, t1 >= 0);
        }
      }
      compute_tile(
          nvalid, tt,
          [&](int kb, int ks) -> uint4 {
            return *reinterpret_cast<const uint4*>(&sK[(kb * 16 + l16) * KROW + 32 * ks + 8 * kg]);
          },
          [&](int db, int u) -> uint4 {
            const int d = db * 16 + l16;
            const bf16_t* vrow = &sVt[d * VROW];
            const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (((8 * u + kg) ^ vt_swz(d)) << 2));
            const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (((8 * u + kg + 4) ^ vt_swz(d)) << 2));
            return make_uint4(lo.x, lo.y, hi.x, hi.y);
          });
    }
  }

  if constexpr (PAGED) {
    if (bad_page) flag(a.dev_status, b, TV_STATUS_BAD_PAGE);
  }

  // ---- epilogue: lane holds O^T rows d = db*16 + 4*kg + r of its query
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const float l_tot = sum_across_groups(l_run[qb]);
    if (!qvalid[qb]) continue;
    const int row = row0 + wave * QBW * 16 + qb * 16 + l16;
    if (nsplit == 1) {
      const int node = qnode[qb];
      const int hh = row - node * G;
      bf16_t* orow = a.out + (((size_t)b * N + node) * a.Hq + (size_t)g * G + hh) * D;
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        uint2 pk;
        pk.x = pack_bf16x2(o[qb][db][0] * inv, o[qb][db][1] * inv);
        pk.y = pack_bf16x2(o[qb][db][2] * inv, o[qb][db][3] * inv);
        *reinterpret_cast<uint2*>(orow + db * 16 + 4 * kg) = pk;
      }
    } else {
      const size_t prow =
          a.ragged ? ((size_t)item * a.Hkv + g) * ((size_t)a.nqblk * kRows) + row
                   : (((size_t)b * a.Hkv + g) * ((size_t)a.nqblk * kRows) + row) * a.nsplit + split;
      float* po = a.part_o + prow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4_t*>(po + db * 16 + 4 * kg) = o[qb][db];
      if (kg == 0) {
        a.part_ml[prow * 2 + 0] = m_ref[qb];
        a.part_ml[prow * 2 + 1] = l_tot;
      }
    }
  }
}

// Merge split partials: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// Ragged batches: sequence b's partials are items start[b] .. start[b+1]-1
// (the plan the attention kernel published); a sequence with one split wrote
// its output directly.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int D4 = D / 4;
  const int R = a.N * a.G;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)a.B * a.Hkv * R * D4;
  if (gid >= total) return;
  const int d4 = (int)(gid % D4);
  size_t t = gid / D4;
  const int row = (int)(t % R);
  t /= R;
  const int g = (int)(t % a.Hkv);
  const int b = (int)(t / a.Hkv);
  int ns = a.nsplit;
  size_t prow0, pstride;
  if (a.ragged) {
    const int s0 = a.ragged_start[b];
    ns = a.ragged_start[b + 1] - s0;
    if (ns == 1) return;
    pstride = (size_t)a.Hkv * a.nqblk * a.rows;
    prow0 = ((size_t)s0 * a.Hkv + g) * ((size_t)a.nqblk * a.rows) + row;
  } else {
    pstride = 1;
    prow0 = (((size_t)b * a.Hkv + g) * ((size_t)a.nqblk * a.rows) + row) * a.nsplit;
  }
  // up to kRegSplits splits: every load issued before the first use, the
  // same arithmetic in the same order as the general loop below
  constexpr int kRegSplits = 8;
  float mx = -INFINITY;
  float lsum = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (ns <= kRegSplits) {
    float2 ml[kRegSplits];
    f32x4_t vo[kRegSplits];
#pragma unroll
    for (int s = 0; s < kRegSplits; ++s) {
      const size_t pr = prow0 + (size_t)(s < ns ? s : 0) * pstride;
      ml[s] = *reinterpret_cast<const float2*>(a.part_ml + pr * 2);
      vo[s] = *reinterpret_cast<const f32x4_t*>(a.part_o + pr * D + d4 * 4);
    }
#pragma unroll
    for (int s = 0; s < kRegSplits; ++s)
      if (s < ns) mx = fmaxf(mx, ml[s].x);
    const float m_use = (mx == -INFINITY) ? 0.f : mx;
#pragma unroll
    for (int s = 0; s < kRegSplits; ++s)
      if (s < ns) {
        const float w = __builtin_amdgcn_exp2f(ml[s].x - m_use);
        lsum += w * ml[s].y;
        acc += w * vo[s];
      }
  } else {
    for (int s = 0; s < ns; ++s) mx = fmaxf(mx, a.part_ml[(prow0 + s * pstride) * 2]);
    const float m_use = (mx == -INFINITY) ? 0.f : mx;
    for (int s = 0; s < ns; ++s) {
      const size_t pr = prow0 + s * pstride;
      const float w = __builtin_amdgcn_exp2f(a.part_ml[pr * 2] - m_use);
      lsum += w * a.part_ml[pr * 2 + 1];
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(a.part_o + pr * D + d4 * 4);
      acc += w * v;
    }
  }
  const float inv = 1.f / lsum;
  const int node = row / a.G;
  const int hh = row - node * a.G;
  bf16_t* orow = a.out + (((size_t)b * a.N + node) * a.Hq + (size_t)g * a.G + hh) * D;
  uint2 pk;
  pk.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pk.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<uint2*>(orow + d4 * 4) = pk;
}

// ---------------------------------------------------------------- fp32 path
// One workgroup per (node, query head, sequence); each wavefront takes every
// fourth visible key, keeps an online softmax with the head dimension spread
// over its lanes, and the four partial states are merged through LDS.
__global__ __launch_bounds__(256) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ parent,
    float* __restrict__ out, int N, int Hq, int Hkv, int D, int Lcap, int max_seq_len,
    float scale, int32_t* __restrict__ dev_status) {
  __shared__ float s_m[4], s_l[4];
  __shared__ float s_o[4][128];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = Hq / Hkv, g = h / G;
  const int L = seq_lens[b];
  if (L < 0 || L > max_seq_len || L + N > Lcap) {
    if (threadIdx.x == 0 && h == 0 && i == 0) flag(dev_status, b, TV_STATUS_BAD_LEN);
    return;
  }
  const int32_t* par = parent + (size_t)b * N;
  // validate the root path of node i (bounded walk)
  {
    int j = i;
    bool ok = par[0] == -1;
    while (ok && j != 0) {
      const int p = par[j];
      ok = p >= 0 && p < j;
      j = ok ? p : 0;
    }
    if (!ok) {
      if (threadIdx.x == 0) flag(dev_status, b, TV_STATUS_BAD_PARENT);
      return;
    }
  }
  const float* qv = q + (((size_t)b * N + i) * Hq + h) * D;
  const float* kp = k + ((size_t)b * Hkv + g) * (size_t)Lcap * D;
  const float* vp = v + ((size_t)b * Hkv + g) * (size_t)Lcap * D;
  const float q0 = lane < D ? qv[lane] : 0.f;
  const float q1 = lane + 64 < D ? qv[lane + 64] : 0.f;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  auto visit = [&](int row) {
    const float* kr = kp + (size_t)row * D;
    float d = (lane < D ? q0 * kr[lane] : 0.f) + (lane + 64 < D ? q1 * kr[lane + 64] : 0.f);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) d += __shfl_xor(d, off, 64);
    const float sc = d * scale;
    const float mn = fmaxf(m, sc);
    const float al = expf(m - mn);
    const float p = expf(sc - mn);
    const float* vr = vp + (size_t)row * D;
    o0 = o0 * al + (lane < D ? p * vr[lane] : 0.f);
    o1 = o1 * al + (lane + 64 < D ? p * vr[lane + 64] : 0.f);
    l = l * al + p;
    m = mn;
  };
  for (int t = wave; t < L; t += 4) visit(t);
  {
    int j = i, c = 0;
    while (true) {
      if ((c & 3) == wave) visit(L + j);
      if (j == 0) break;
      j = par[j];
      ++c;
    }
  }
  if (lane == 0) {
    s_m[wave] = m;
    s_l[wave] = l;
  }
  if (lane < D) s_o[wave][lane] = o0;
  if (lane + 64 < D) s_o[wave][lane + 64] = o1;
  __syncthreads();
  if (wave == 0) {
    float mx = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    float lt = 0.f, a0 = 0.f, a1 = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float sc = (s_m[w] == -INFINITY) ? 0.f : expf(s_m[w] - mx);
      lt += sc * s_l[w];
      if (lane < D) a0 += sc * s_o[w][lane];
      if (lane + 64 < D) a1 += sc * s_o[w][lane + 64];
    }
    float* orow = out + (((size_t)b * N + i) * Hq + h) * D;
    if (lane < D) orow[lane] = a0 / lt;
    if (lane + 64 < D) orow[lane + 64] = a1 / lt;
  }
}

// Variant table: (query rows per wavefront / 16, wavefronts per workgroup).
template <int D, bool PAGED>
hipError_t launch_bf16(const AttnArgs& a, int qbw, hipStream_t stream) {
  const dim3 grid(a.total_blocks);
  // the D = 128 variants keep the ancestor words of their nodes (at most
  // (rows - 1) / G + 2 of them) in dynamic LDS
  const size_t anc_bytes = D == 128 ? (size_t)((a.rows - 1) / a.G + 2) * a.anc_words * 8 : 0;
  if (qbw == 2)
    hipLaunchKernelGGL((attn_bf16_kernel<D, 2, 4, PAGED>), grid, dim3(256), anc_bytes, stream, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, 1, 4, PAGED>), grid, dim3(256), anc_bytes, stream, a);
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int B, int N, int Hq, int Hkv, int D, int max_seq_len, int dtype,
                   int page_size) {
  AttnPlan p{};
  const int G = Hq / Hkv;
  const long R = (long)N * G;
  const int ntiles = (max_seq_len + kKT - 1) / kKT;
  const long target = 512;  // about two workgroups per CU
  // Query rows per workgroup and prefix splits.
  //  * Long prefixes (>= 32 tiles) keep 128-row blocks, where each K/V tile
  //    serves the most rows, and split the prefix (>= 8 tiles per split)
  //    until about two workgroups per CU exist.
  //  * Short prefixes use 64-row blocks and splits of >= 4 tiles, aiming at
  //    one workgroup per CU: there the cost is the latency of each tile, and
  //    a finer split would write more partial results than it reads.
  p.qbw = 2;
  p.nw = 4;
  p.rows = 128;
  int min_tiles = 8;
  long want_blocks = target;
  if (dtype == TV_BF16 && ntiles < 32) {
    p.qbw = 1, p.nw = 4, p.rows = 64;
    min_tiles = 4;
    want_blocks = target / 2;
  }
  p.nqblk = (int)((R + p.rows - 1) / p.rows);
  p.nsplit = 1;
  p.chunk_len = kKT * (ntiles > 0 ? ntiles : 1);
  if (dtype == TV_BF16 && ntiles > 1) {
    const long base = (long)B * Hkv * p.nqblk;
    if (base < want_blocks) {
      long want = (want_blocks + base - 1) / base;
      long cap = ntiles / min_tiles;
      if (cap < 1) cap = 1;
      if (want > cap) want = cap;
      const int per = (int)((ntiles + want - 1) / want);
      p.chunk_len = per * kKT;
      p.nsplit = (ntiles + per - 1) / per;
    }
  }
  (void)page_size;  // pages look up their entries per row: the plan is the contiguous one
  // With the prefix split, the tree keys get a split of their own (the last,
  // whose prefix range is empty) while the grid stays within the target:
  // otherwise the workgroup that owns the last prefix chunk also walks the
  // parents, builds the ancestor words and runs the tree tiles, and sets the
  // critical path (measured 10-13 % off the attention time at 512-2048-token
  // prefixes; past the target, the extra workgroups form a second wave).
  if (dtype == TV_BF16 && p.nsplit > 1 &&
      (long)B * Hkv * p.nqblk * (p.nsplit + 1) <= want_blocks)
    p.nsplit += 1;
  // A batch of several sequences whose prefixes want splitting takes its
  // splits from the actual lengths on the device (ragged_plan in the
  // kernels): one chunk length for the whole batch, so a long sequence gets
  // many splits and a short one few, instead of every sequence getting the
  // longest one's split count.  The grid covers the most work items any
  // lengths up to max_seq_len can give; workgroups past the actual count
  // return at once.
  p.ragged = 0;
  if (dtype == TV_BF16 && B > 1 && B <= kMaxRaggedBatch && p.nsplit > 1) {
    const long hq = (long)Hkv * p.nqblk;
    p.ragged = 1;
    p.want_blocks = (int)want_blocks;
    p.min_tiles = min_tiles;
    p.max_items = (int)(want_blocks / hq + 1 + 2L * B);
  }
  p.ws_bytes = 0;
  if (p.ragged) {
    const size_t rows = (size_t)p.max_items * Hkv * p.nqblk * p.rows;
    p.ws_bytes = rows * D * sizeof(float) + rows * 2 * sizeof(float) +
                 (kMaxRaggedBatch + 1) * sizeof(int);
  } else if (p.nsplit > 1) {
    const size_t rows = (size_t)B * Hkv * p.nqblk * p.rows * p.nsplit;
    p.ws_bytes = rows * D * sizeof(float) + rows * 2 * sizeof(float);
  }
  return p;
}

hipError_t launch_tree_attn(const void* q, const void* k, const void* v,
                            const int32_t* seq_lens, const int32_t* parent, void* out,
                            int B, int N, int Hq, int Hkv, int D, int Lcap,
                            int max_seq_len, float scale, int dtype, const AttnPlan& plan,
                            void* ws, int32_t* dev_status, hipStream_t stream,
                            const int32_t* block_table, int max_blocks, int page_size,
                            int num_pages) {
  if (dtype == TV_F32) {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(N, Hq, B), dim3(256), 0, stream,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), seq_lens, parent,
                       static_cast<float*>(out), N, Hq, Hkv, D, Lcap, max_seq_len, scale,
                       dev_status);
    return hipGetLastError();
  }
  AttnArgs a{};
  a.q = static_cast<const bf16_t*>(q);
  a.k = static_cast<const bf16_t*>(k);
  a.v = static_cast<const bf16_t*>(v);
  a.seq_lens = seq_lens;
  a.parent = parent;
  a.out = static_cast<bf16_t*>(out);
  a.dev_status = dev_status;
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.Lcap = Lcap;
  a.max_seq_len = max_seq_len;
  a.rows = plan.rows;
  a.nqblk = plan.nqblk;
  a.nsplit = plan.nsplit;
  a.chunk_len = plan.chunk_len;
  a.ragged = plan.ragged;
  a.want_blocks = plan.want_blocks;
  a.min_tiles = plan.min_tiles;
  a.total_blocks = plan.ragged ? plan.max_items * Hkv * plan.nqblk
                               : B * Hkv * plan.nqblk * plan.nsplit;
  a.anc_words = (N + 63) / 64;
  a.scale_log2 = scale * kLog2e;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.num_pages = num_pages;
  a.page_shift = 0;
  if (block_table != nullptr) {
    while ((1 << a.page_shift) < page_size) ++a.page_shift;
    a.Lcap = max_blocks << a.page_shift;  // logical capacity of a sequence
  }
  if (plan.ragged || plan.nsplit > 1) {
    const size_t rows = plan.ragged ? (size_t)plan.max_items * Hkv * plan.nqblk * plan.rows
                                    : (size_t)B * Hkv * plan.nqblk * plan.rows * plan.nsplit;
    a.part_o = static_cast<float*>(ws);
    a.part_ml = static_cast<float*>(ws) + rows * D;
    a.ragged_start = reinterpret_cast<int*>(a.part_ml + rows * 2);
  }
  hipError_t e;
  if (block_table != nullptr)
    e = (D == 128) ? launch_bf16<128, true>(a, plan.qbw, stream)
                   : launch_bf16<64, true>(a, plan.qbw, stream);
  else
    e = (D == 128) ? launch_bf16<128, false>(a, plan.qbw, stream)
                   : launch_bf16<64, false>(a, plan.qbw, stream);
  if (e != hipSuccess || (plan.nsplit == 1 && !plan.ragged)) return e;
  const size_t items = (size_t)B * Hkv * N * a.G * (D / 4);
  const dim3 grid((unsigned)((items + 255) / 256));
  if (D == 128)
    hipLaunchKernelGGL(attn_combine_kernel<128>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_combine_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tv
