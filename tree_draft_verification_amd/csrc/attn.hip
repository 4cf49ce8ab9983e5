// Tree-causal verification attention.
//
// Method (JetSpec GitHub README, "JetSpec > Overview"): the target verifies
// the whole draft tree in one forward pass under a tree-causal mask.  Node i
// of sequence b sees the prefix (cache rows 0..L_b-1) and the tree nodes on
// its own root path (rows L_b+j, j an ancestor of i or i itself):
//     out[b][i][h] = softmax(scale * q K_vis^T) V_vis,   KV head = h / G.
//
// bf16 kernel (gfx950 matrix cores):
//   * A workgroup (4 wavefronts) owns 128 query rows of one (sequence, KV
//     head).  Row r is node r / G, head r % G of the group, so the G heads of
//     one node - which share every key and the whole mask - are adjacent and
//     the key/value tiles staged in LDS are shared by all 128 rows.
//   * Per 64-key tile: S^T = K Q^T on 16x16x32 bf16 MFMA (K rows from LDS,
//     Q^T fragments held in registers for the whole loop), then an online
//     softmax in the exp2 domain, then O^T += V^T P^T on MFMA.  Computing the
//     transposed products leaves each lane with one query column in both
//     results, so the softmax state of a query never leaves its lane, and the
//     probabilities feed the second product straight from registers (the key
//     order inside the 32-wide k-step is permuted identically in V^T and
//     P^T).  V is stored transposed in LDS for that product.
//   * The mask is one 64-bit ancestor word per (node, 64-key tree tile),
//     built in LDS at kernel start by walking parent pointers from each node
//     of the block (TV_STATUS_BAD_PARENT on a malformed tree).  Tree tiles
//     past the block's last node are skipped: a node only sees lower indices.
//   * Long prefixes are split across workgroups (split-KV).  Each split writes
//     fp32 (max, sum, unnormalised output) partials and a combine kernel
//     merges them; with one split the kernel writes the output directly.
//     The tree keys are handled by the last split.
//   * Workgroup ids are remapped so that the query blocks and splits that read
//     the same key/value rows run on the same die (shared L2).
// fp32 kernel: a plain VALU kernel for small fp32 problems.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kKT = 64;          // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;  // two 16-query MFMA column blocks
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;  // 128
constexpr int kKPad = 8;         // bf16 padding of a K row in LDS
constexpr int kVPad = 4;         // bf16 padding of a V^T row in LDS
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const int32_t* seq_lens;
  const int32_t* parent;
  bf16_t* out;
  float* part_o;   // [B*Hkv][nqblk*128][nsplit][D] fp32
  float* part_ml;  // [B*Hkv][nqblk*128][nsplit][2] fp32
  int32_t* dev_status;
  int B, N, Hq, Hkv, G, Lcap, max_seq_len;
  int nqblk, nsplit, chunk_len, total_blocks;
  int anc_nodes;   // node slots of the ancestor table in LDS
  int anc_words;   // ceil(N / 64)
  float scale_log2;  // scale * log2(e)
};

__device__ __forceinline__ void flag(int32_t* st, int b, int f) {
  if (st) atomicOr(&st[b], f);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(AttnArgs a) {
  constexpr int DS = D / 32;  // k-steps of the QK^T product
  constexpr int DB = D / 16;  // 16-row output blocks of the PV product
  constexpr int KROW = D + kKPad;
  constexpr int VROW = kKT + kVPad;
  __shared__ __attribute__((aligned(16))) bf16_t sK[kKT * KROW];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[D * VROW];
  __shared__ int16_t sPar[TV_MAX_NODES];
  extern __shared__ unsigned long long sAnc[];  // [anc_nodes][anc_words]

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int kg = lane >> 4;

  // ---- which (sequence, KV head, split, query block) this workgroup owns
  int t = xcd_remap(blockIdx.x, a.total_blocks);
  const int qblk = t % a.nqblk;
  t /= a.nqblk;
  const int split = t % a.nsplit;
  t /= a.nsplit;
  const int g = t % a.Hkv;
  const int b = t / a.Hkv;

  const int N = a.N, G = a.G;
  const int R = N * G;
  const int L = a.seq_lens[b];
  if (L < 0 || L > a.max_seq_len || L + N > a.Lcap) {
    if (tid == 0) flag(a.dev_status, b, TV_STATUS_BAD_LEN);
    return;
  }
  const int row0 = qblk * kRowsPerBlock;
  const int node_lo = row0 / G;
  const int node_hi = (min(R, row0 + kRowsPerBlock) - 1) / G;
  const bool do_tree = (split == a.nsplit - 1);
  const int c0 = split * a.chunk_len;
  const int c1 = min(c0 + a.chunk_len, L);

  // ---- ancestor words of the block's nodes (tree split only)
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
    for (int x = tid; x < nn * a.anc_words; x += kThreads) sAnc[x] = 0ull;
    __syncthreads();
    for (int n = tid; n < nn; n += kThreads) {
      unsigned long long* w = sAnc + n * a.anc_words;
      int j = node_lo + n;
      while (j >= 0) {  // parent[j] < j, so this ends within j + 1 steps
        w[j >> 6] |= 1ull << (j & 63);
        j = (j == 0) ? -1 : sPar[j];
      }
    }
    if (bad) flag(a.dev_status, b, TV_STATUS_BAD_PARENT);
  }

  // ---- Q^T fragments of this lane's two query columns
  const size_t kv_plane = ((size_t)b * a.Hkv + g) * (size_t)a.Lcap * D;
  const bf16_t* kp = a.k + kv_plane;
  const bf16_t* vp = a.v + kv_plane;
  bf16x8_t qf[2][DS];
  int qnode[2];
  bool qvalid[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = row0 + wave * kRowsPerWave + qb * 16 + l16;
    qvalid[qb] = row < R;
    const int node = qvalid[qb] ? row / G : node_hi;
    const int hh = qvalid[qb] ? row - node * G : 0;
    qnode[qb] = node;
    const bf16_t* qrow = a.q + (((size_t)b * N + node) * a.Hq + (size_t)g * G + hh) * D;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      Frag8 f;
      f.u = qvalid[qb] ? *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * kg)
                       : make_uint4(0, 0, 0, 0);
      qf[qb][s] = f.v;
    }
  }

  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f32x4_t o[2][DB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int n_pre = (c1 > c0) ? (c1 - c0 + kKT - 1) / kKT : 0;
  const int n_tree = do_tree ? (node_hi / kKT + 1) : 0;

  for (int it = 0; it < n_pre + n_tree; ++it) {
    const bool tree = it >= n_pre;
    const int tt = it - n_pre;
    const int krow0 = tree ? L + tt * kKT : c0 + it * kKT;
    const int nvalid = tree ? min(kKT, N - tt * kKT) : min(kKT, c1 - krow0);

    __syncthreads();  // previous tile fully consumed (and ancestor table built)
    // K tile: rows krow0.. are contiguous in the plane; 16-byte pieces.
    for (int c = tid; c < kKT * (D / 8); c += kThreads) {
      const int r = c / (D / 8);
      const int x = c - r * (D / 8);
      uint4 val = make_uint4(0, 0, 0, 0);
      if (r < nvalid) val = *reinterpret_cast<const uint4*>(kp + (size_t)(krow0 + r) * D + x * 8);
      *reinterpret_cast<uint4*>(&sK[r * KROW + x * 8]) = val;
    }
    // V tile, transposed: a thread takes 4 keys x 8 dims and writes 8 rows
    // of V^T with 4 keys each.
    for (int c = tid; c < (kKT / 4) * (D / 8); c += kThreads) {
      const int kq = c / (D / 8);
      const int x = c - kq * (D / 8);
      uint4 rv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = kq * 4 + i;
        rv[i] = (r < nvalid) ? *reinterpret_cast<const uint4*>(vp + (size_t)(krow0 + r) * D + x * 8)
                             : make_uint4(0, 0, 0, 0);
      }
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&rv[0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&rv[1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&rv[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&rv[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        const uint32_t a0 = (w0[e >> 1] >> sh) & 0xffffu, a1 = (w1[e >> 1] >> sh) & 0xffffu;
        const uint32_t a2 = (w2[e >> 1] >> sh) & 0xffffu, a3 = (w3[e >> 1] >> sh) & 0xffffu;
        uint2 pk;
        pk.x = a0 | (a1 << 16);
        pk.y = a2 | (a3 << 16);
        *reinterpret_cast<uint2*>(&sVt[(x * 8 + e) * VROW + kq * 4]) = pk;
      }
    }
    __syncthreads();

    // S^T = K Q^T: lane holds query column l16, keys kb*16 + 4*kg + r.
    f32x4_t s[2][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[0][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      s[1][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DS; ++ks) {
        Frag8 kf;
        kf.u = *reinterpret_cast<const uint4*>(&sK[(kb * 16 + l16) * KROW + 32 * ks + 8 * kg]);
        s[0][kb] = mfma16x16x32(kf.v, qf[0][ks], s[0][kb]);
        s[1][kb] = mfma16x16x32(kf.v, qf[1][ks], s[1][kb]);
      }
    }

    // mask, online softmax (exp2 domain), probabilities to bf16
    Frag8 pf[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      unsigned long long word = ~0ull;
      if (tree) word = sAnc[(qnode[qb] - node_lo) * a.anc_words + tt];
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb * 16 + 4 * kg + r;
          const bool vis = key < nvalid && ((word >> key) & 1ull);
          const float x = vis ? s[qb][kb][r] * a.scale_log2 : -INFINITY;
          s[qb][kb][r] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run[qb], tmax);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run[qb] - m_use);
      m_run[qb] = m_new;
      float psum = 0.f;
      uint32_t pb[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = exp2f(s[qb][kb][r] - m_use);
          psum += p;
          pb[kb][r] = f32_to_bf16(p);
        }
      l_run[qb] = l_run[qb] * alpha + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        pf[qb][u].u = make_uint4(pb[2 * u][0] | (pb[2 * u][1] << 16),
                                 pb[2 * u][2] | (pb[2 * u][3] << 16),
                                 pb[2 * u + 1][0] | (pb[2 * u + 1][1] << 16),
                                 pb[2 * u + 1][2] | (pb[2 * u + 1][3] << 16));
      }
    }

    // O^T += V^T P^T; k-slot e of lane group kg is key 32u + 4kg + e (e < 4)
    // or 32u + 16 + 4kg + e - 4 (e >= 4), in both operands.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16_t* vrow = &sVt[(db * 16 + l16) * VROW + 32 * u + 4 * kg];
        Frag8 vf;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
        vf.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[0][db] = mfma16x16x32(vf.v, pf[0][u].v, o[0][db]);
        o[1][db] = mfma16x16x32(vf.v, pf[1][u].v, o[1][db]);
      }
    }
  }

  // ---- epilogue: lane holds O^T rows d = db*16 + 4*kg + r of its query
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l_tot = l_run[qb];
    l_tot += __shfl_xor(l_tot, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (!qvalid[qb]) continue;
    const int row = row0 + wave * kRowsPerWave + qb * 16 + l16;
    if (a.nsplit == 1) {
      const int node = qnode[qb];
      const int hh = row - node * G;
      bf16_t* orow = a.out + (((size_t)b * N + node) * a.Hq + (size_t)g * G + hh) * D;
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        uint2 pk;
        pk.x = f32_to_bf16(o[qb][db][0] * inv) | (f32_to_bf16(o[qb][db][1] * inv) << 16);
        pk.y = f32_to_bf16(o[qb][db][2] * inv) | (f32_to_bf16(o[qb][db][3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + db * 16 + 4 * kg) = pk;
      }
    } else {
      const size_t prow = (((size_t)b * a.Hkv + g) * ((size_t)a.nqblk * kRowsPerBlock) + row) * a.nsplit + split;
      float* po = a.part_o + prow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4_t*>(po + db * 16 + 4 * kg) = o[qb][db];
      if (kg == 0) {
        a.part_ml[prow * 2 + 0] = m_run[qb];
        a.part_ml[prow * 2 + 1] = l_tot;
      }
    }
  }
}

// Merge split partials: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
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
  const size_t prow0 = (((size_t)b * a.Hkv + g) * ((size_t)a.nqblk * kRowsPerBlock) + row) * a.nsplit;
  float mx = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) mx = fmaxf(mx, a.part_ml[(prow0 + s) * 2]);
  const float m_use = (mx == -INFINITY) ? 0.f : mx;
  float lsum = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.nsplit; ++s) {
    const float w = exp2f(a.part_ml[(prow0 + s) * 2] - m_use);
    lsum += w * a.part_ml[(prow0 + s) * 2 + 1];
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(a.part_o + (prow0 + s) * D + d4 * 4);
    acc += w * v;
  }
  const float inv = 1.f / lsum;
  const int node = row / a.G;
  const int hh = row - node * a.G;
  bf16_t* orow = a.out + (((size_t)b * a.N + node) * a.Hq + (size_t)g * a.G + hh) * D;
  uint2 pk;
  pk.x = f32_to_bf16(acc[0] * inv) | (f32_to_bf16(acc[1] * inv) << 16);
  pk.y = f32_to_bf16(acc[2] * inv) | (f32_to_bf16(acc[3] * inv) << 16);
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

}  // namespace

AttnPlan attn_plan(int B, int N, int Hq, int Hkv, int D, int max_seq_len, int dtype) {
  AttnPlan p{};
  const int G = Hq / Hkv;
  const int R = N * G;
  p.nqblk = (R + kRowsPerBlock - 1) / kRowsPerBlock;
  p.nsplit = 1;
  const int ntiles = (max_seq_len + kKT - 1) / kKT;
  p.chunk_len = kKT * (ntiles > 0 ? ntiles : 1);
  if (dtype == TV_BF16 && ntiles > 1) {
    const long base = (long)B * Hkv * p.nqblk;
    const long target = 512;  // two workgroups on each of the 256 CUs
    if (base < target) {
      long want = (target + base - 1) / base;
      long cap = ntiles / 2;  // at least two tiles per split
      if (cap < 1) cap = 1;
      if (want > cap) want = cap;
      const int per = (int)((ntiles + want - 1) / want);
      p.chunk_len = per * kKT;
      p.nsplit = (ntiles + per - 1) / per;
    }
  }
  p.ws_bytes = 0;
  if (p.nsplit > 1) {
    const size_t rows = (size_t)B * Hkv * p.nqblk * kRowsPerBlock * p.nsplit;
    p.ws_bytes = rows * D * sizeof(float) + rows * 2 * sizeof(float);
  }
  return p;
}

hipError_t launch_tree_attn(const void* q, const void* k, const void* v,
                            const int32_t* seq_lens, const int32_t* parent, void* out,
                            int B, int N, int Hq, int Hkv, int D, int Lcap,
                            int max_seq_len, float scale, int dtype, const AttnPlan& plan,
                            void* ws, int32_t* dev_status, hipStream_t stream) {
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
  a.nqblk = plan.nqblk;
  a.nsplit = plan.nsplit;
  a.chunk_len = plan.chunk_len;
  a.total_blocks = B * Hkv * plan.nqblk * plan.nsplit;
  a.anc_words = (N + 63) / 64;
  a.anc_nodes = kRowsPerBlock / a.G + 2;
  if (a.anc_nodes > N) a.anc_nodes = N;
  a.scale_log2 = scale * kLog2e;
  if (plan.nsplit > 1) {
    const size_t rows = (size_t)B * Hkv * plan.nqblk * kRowsPerBlock * plan.nsplit;
    a.part_o = static_cast<float*>(ws);
    a.part_ml = static_cast<float*>(ws) + rows * D;
  }
  const size_t lds = (size_t)a.anc_nodes * a.anc_words * sizeof(unsigned long long);
  if (D == 128)
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(a.total_blocks), dim3(kThreads), lds, stream, a);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(a.total_blocks), dim3(kThreads), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.nsplit == 1) return e;
  const size_t items = (size_t)B * Hkv * N * a.G * (D / 4);
  const dim3 grid((unsigned)((items + 255) / 256));
  if (D == 128)
    hipLaunchKernelGGL(attn_combine_kernel<128>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_combine_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tv
