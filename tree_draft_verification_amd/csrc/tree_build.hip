// Draft-tree construction by cumulative log-probability (accum_logp).
//
// The JetSpec README ("Evaluation") names accum_logp, a breadth-first
// cumulative-log-probability tree, as the default tree algorithm; its "Quick
// Start" shapes the tree by a depth, a width and a node budget.  From the
// draft head's normalised log-probabilities logp[b][d][V] (one row per depth):
//   * the candidate tokens of depth d are the `width` largest entries of row
//     d (ties to the smaller id);
//   * breadth first, every node of the level-(d-1) frontier gets one child
//     per candidate token, score = parent score + logp; the level-d frontier
//     is the `width` best children (score, then generation order); every
//     child is a candidate;
//   * the tree is the root plus the `budget` best candidates (score, then
//     depth, then generation), numbered by depth and generation.
// Scores are fp32 inputs summed in fp64, which is exact here, so every
// decision is exact.
//
// Top lists are kept per wavefront: lanes 0..W-1 hold the wavefront's best
// keys in order.  An element costs one compare against the wavefront's W-th
// key and a ballot; only the rare elements that beat it are inserted, all
// lanes shifting their entry in one step.
// Kernel 1 (data parallel, HBM bound): one workgroup per (row, vocabulary
// chunk) writes the chunk's sorted top-W packed (value, id) keys.
// Kernel 2 (one workgroup of 16 wavefronts per sequence, LDS resident):
// merges the chunk lists of every depth, runs the breadth-first levels in
// one wavefront, keeps the budget's best candidates (bitonic sort) and
// numbers the kept nodes by a scan.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kTopThreads = 256;    // kernel 1
constexpr int kTreeThreads = 1024;  // kernel 2
constexpr int kMaxW = 16;           // width limit (wavefront list)
constexpr int kMaxPool = 4096;      // candidate pool limit
constexpr int kMaxDepth = 64;

typedef unsigned long long u64;

__device__ __forceinline__ u64 shfl_up1_u64(u64 x) {
  const uint32_t lo = __shfl_up((uint32_t)x, 1, 64);
  const uint32_t hi = __shfl_up((uint32_t)(x >> 32), 1, 64);
  return ((u64)hi << 32) | lo;
}

__device__ __forceinline__ u64 readlane_u64(u64 x, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)x, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), lane);
  return ((u64)hi << 32) | lo;
}

// Order-preserving map of fp64 to u64 (larger value -> larger key; any
// non-NaN value maps above 0, the empty-slot key).
__device__ __forceinline__ u64 f64_order_key(double d) {
  const u64 u = (u64)__double_as_longlong(d);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Inverse of f32_order_key on the high half of an argmax key.
__device__ __forceinline__ float key_value(u64 k) {
  const uint32_t u = (uint32_t)(k >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
__device__ __forceinline__ int key_token(u64 k) { return (int)(~(uint32_t)(k & 0xffffffffull)); }

// A wavefront's sorted list: lane i < W holds its i-th best key L (0 when
// empty) and a payload P.  offer() inserts every lane's key k that beats the
// W-th entry, in lane order; an equal key never passes an entry already in
// the list, so among equal keys the earlier offered ranks first.
struct WaveList {
  u64 L = 0ull;
  int P = 0;
  u64 thr = 0ull;  // W-th key (wave uniform)

  __device__ __forceinline__ void offer(u64 k, int payload, int W, int lane) {
    u64 m = __ballot(k > thr);
    while (m) {
      const int src = __builtin_ctzll(m);
      m &= m - 1;
      const u64 kk = readlane_u64(k, src);
      if (kk <= thr) continue;  // the threshold rose since the ballot
      const int pp = __builtin_amdgcn_readlane(payload, src);
      const u64 up = shfl_up1_u64(L);
      const int upp = __shfl_up(P, 1, 64);
      if (lane < W && L < kk) {
        const bool here = lane == 0 || up >= kk;
        L = here ? kk : up;
        P = here ? pp : upp;
      }
      thr = readlane_u64(L, W - 1);
    }
  }
};

// The wavefront's 64 keys in descending order across the lanes (bitonic
// network over lane indices, exchanges by shuffles).
__device__ __forceinline__ u64 wave_sort_desc(u64 k, int lane) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int j = size >> 1; j > 0; j >>= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)k, j, 64);
      const uint32_t hi = __shfl_xor((uint32_t)(k >> 32), j, 64);
      const u64 o = ((u64)hi << 32) | lo;
      // the lower lane of a pair keeps the larger key in a descending
      // block ((lane & size) == 0), the smaller in an ascending one
      const bool lower = (lane & j) == 0;
      const bool desc = (lane & size) == 0;
      const u64 big = o > k ? o : k, small = o > k ? k : o;
      k = (lower == desc) ? big : small;
    }
  }
  return k;
}

// Rank of (v, i) among a[0..n) in LDS: entries greater than v, or equal to
// it at a smaller index.  Eight independent reads per trip (the count is
// bound by LDS latency otherwise; more would exceed the register budget of
// a 1024-thread workgroup).
template <typename T>
__device__ __forceinline__ int rank_among(const T* a, int n, T v, int i) {
  int r = 0, j = 0;
  for (; j + 8 <= n; j += 8) {
    T x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = a[j + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) r += (x[u] > v) | ((x[u] == v) & (j + u < i));
  }
  for (; j < n; ++j) r += (a[j] > v) | ((a[j] == v) & (j < i));
  return r;
}

// ---- kernel 1: sorted top-W keys of one vocabulary chunk of one row.
// Row r of the grid reads input row (r / rows_per_seq) * row_pitch +
// r % rows_per_seq: the first rows_per_seq rows of each sequence's block of
// row_pitch rows.
__global__ __launch_bounds__(kTopThreads) void draft_topk_kernel(
    const float* __restrict__ logp, int V, int W, int nch, int chunk_len, int rows_per_seq,
    int row_pitch, u64* __restrict__ part) {
  __shared__ u64 s_wl[kTopThreads / 64][kMaxW];
  const int row = blockIdx.x / nch;
  const int c = blockIdx.x - row * nch;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int v0 = c * chunk_len;
  const int v1 = min(V, v0 + chunk_len);
  const int in_row = (row / rows_per_seq) * row_pitch + row % rows_per_seq;
  const float* x = logp + (size_t)in_row * V;
  WaveList wl;
  // kBatch independent loads per trip (clamped addresses; one trip covers a
  // 6144-element chunk), then the offers; the trip count is uniform across
  // the wavefront (offer() uses ballots).  The list starts from the first
  // 64 keys sorted across the lanes, which fills it and sets its threshold
  // without one insertion per key; keys are unique, so the list ends the
  // same whatever the order of the offers.
  constexpr int kBatch = 24;
  bool first = true;
  for (int b0 = v0 + wave * 64; b0 < v1; b0 += kBatch * kTopThreads) {
    float val[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) val[u] = x[min(b0 + u * kTopThreads + lane, v1 - 1)];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int v = b0 + u * kTopThreads + lane;
      // + 0.0f turns -0.0 into +0.0, so equal values tie on the token id
      const u64 k = v < v1 ? argmax_key(val[u] + 0.0f, (uint32_t)v) : 0ull;
      if (u == 0 && first) {
        const u64 sk = wave_sort_desc(k, lane);
        wl.L = lane < W ? sk : 0ull;
        wl.thr = readlane_u64(sk, W - 1);
        first = false;
      } else {
        wl.offer(k, 0, W, lane);
      }
    }
  }
  if (lane < W) s_wl[wave][lane] = wl.L;
  __syncthreads();
  if (wave == 0) {  // merge the four lists (4 W <= 64 unique keys): sort them
    const int n = (kTopThreads / 64) * W;
    const u64 k = wave_sort_desc(lane < n ? s_wl[lane / W][lane % W] : 0ull, lane);
    if (lane < W) part[(size_t)blockIdx.x * kMaxW + lane] = k;
  }
}

// LDS arrays of a candidate pool (the tree kernels' shared memory).
struct PoolLds {
  double* score;    // pool scores, then sort keys
  int16_t* id;      // sort payload: pool index
  int16_t* par;     // parent pool index (-1: root)
  int32_t* tok;
  int8_t* dep;
  int16_t* node;    // node number of a kept entry, else -1
  float* kscore;    // fp32 score of a kept entry
  int* wsum;        // per-wavefront sums of the scan
};

// Stages C-E of a tree, for the workgroup of sequence blockIdx.x (all
// kTreeThreads threads call it; the pool's C entries are in LDS).
__device__ void cut_number_write(const PoolLds& pl, int C, int budget,
                                 const int32_t* __restrict__ root_tokens,
                                 int32_t* __restrict__ parent_out, int32_t* __restrict__ token_out,
                                 int32_t* __restrict__ depth_out, float* __restrict__ score_out) {
  double* s_score = pl.score;
  int16_t* s_id = pl.id;
  int16_t* s_par = pl.par;
  int32_t* s_tok = pl.tok;
  int8_t* s_dep = pl.dep;
  int16_t* s_node = pl.node;
  float* s_kscore = pl.kscore;
  int* s_wsum = pl.wsum;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  // C. keep the `budget` best candidates (score descending, then pool
  // index, i.e. depth and generation).  Only the kept set matters (the
  // nodes are numbered in pool order), so up to 1024 entries need no global
  // sort: each wavefront sorts its 64 entries across its lanes (shuffle
  // bitonic network), and an entry's rank is its place in its own list plus,
  // for every other list, the number of entries there that beat it (a binary
  // search; the lists are sorted by the same order).  Larger pools sort in
  // LDS.
  int P2 = 1;
  while (P2 < C) P2 <<= 1;
  if (C <= kTreeThreads) {
    double sc = tid < C ? s_score[tid] : -INFINITY;
    int id = tid;
    // entry (so, io) beats (sc, id): higher score, or equal and earlier
    for (int k = 2; k <= 64; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        const long long bits = __double_as_longlong(sc);
        const uint32_t lo = __shfl_xor((uint32_t)bits, j, 64);
        const uint32_t hi = __shfl_xor((uint32_t)((unsigned long long)bits >> 32), j, 64);
        const double so = __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
        const int io = __shfl_xor(id, j, 64);
        // the lower lane of a pair ends with the better entry in a
        // descending block ((lane & k) == 0), the worse in an ascending one
        const bool o_better = so > sc || (so == sc && io < id);
        const bool lower = (lane & j) == 0;
        const bool desc = (lane & k) == 0;
        if (lower == desc ? o_better : !o_better) {
          sc = so;
          id = io;
        }
      }
    }
    // each wavefront read only its own 64 entries: its sorted list replaces them
    s_score[tid] = sc;
    s_id[tid] = (int16_t)id;
    if (tid < C) s_node[tid] = -1;
    __syncthreads();
    const int nl = (C + 63) / 64;
    if (id < C) {
      int rank = lane;
      for (int w = 0; w < nl; ++w) {
        if (w == wave) continue;
        const double* ls = s_score + w * 64;
        const int16_t* li = s_id + w * 64;
        int lo = 0, hi = 64;  // entries [0, lo) beat (sc, id), [hi, 64) do not
#pragma unroll
        for (int step = 0; step < 7; ++step) {  // 65 possible counts
          if (lo < hi) {
            const int mid = (lo + hi) >> 1;
            const double sm = ls[mid];
            const bool beats = sm > sc || (sm == sc && li[mid] < id);
            lo = beats ? mid + 1 : lo;
            hi = beats ? hi : mid;
          }
        }
        rank += lo;
      }
      if (rank < budget) {
        s_node[id] = 1;
        s_kscore[id] = (float)sc;
      }
    }
    __syncthreads();
  } else {
    for (int i = tid; i < P2; i += kTreeThreads) {
      s_id[i] = (int16_t)i;
      if (i >= C) s_score[i] = -INFINITY;
    }
    __syncthreads();
    for (int k = 2; k <= P2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P2; i += kTreeThreads) {
          const int l = i ^ j;
          if (l > i) {
            const double si = s_score[i], sl = s_score[l];
            const int ii = s_id[i], il = s_id[l];
            const bool l_better = sl > si || (sl == si && il < ii);
            const bool swap = ((i & k) == 0) ? l_better : !l_better;
            if (swap) {
              s_score[i] = sl;
              s_score[l] = si;
              s_id[i] = (int16_t)il;
              s_id[l] = (int16_t)ii;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < C; i += kTreeThreads) s_node[i] = -1;
    __syncthreads();
    for (int r = tid; r < budget; r += kTreeThreads) {
      const int id = s_id[r];
      s_node[id] = 1;
      s_kscore[id] = (float)s_score[r];
    }
    __syncthreads();
  }

  // D. number the kept entries in pool order (block scan)
  const int per = (C + kTreeThreads - 1) / kTreeThreads;
  const int lo = min(C, tid * per), hi = min(C, lo + per);
  int cnt = 0;
  for (int i = lo; i < hi; ++i) cnt += s_node[i] > 0;
  int incl = cnt;  // inclusive scan within the wavefront
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int before = 1;  // node 0 is the root
  for (int w = 0; w < wave; ++w) before += s_wsum[w];
  int next = before + incl - cnt;
  for (int i = lo; i < hi; ++i)
    if (s_node[i] > 0) s_node[i] = (int16_t)next++;
  __syncthreads();

  // E. outputs
  const int N = budget + 1;
  int32_t* par = parent_out + (size_t)b * N;
  int32_t* tok = token_out + (size_t)b * N;
  if (tid == 0) {
    par[0] = -1;
    tok[0] = root_tokens[b];
    if (depth_out) depth_out[(size_t)b * N] = 0;
    if (score_out) score_out[(size_t)b * N] = 0.f;
  }
  for (int i = tid; i < C; i += kTreeThreads) {
    const int n = s_node[i];
    if (n <= 0) continue;
    const int pi = s_par[i];
    const int pn = pi < 0 ? 0 : s_node[pi];
    par[n] = pn < 0 ? 0 : pn;  // the kept set holds every kept node's parent
    tok[n] = s_tok[i];
    if (depth_out) depth_out[(size_t)b * N + n] = s_dep[i];
    if (score_out) score_out[(size_t)b * N + n] = s_kscore[i];
  }
}

// ---- kernel 2: the tree of one sequence.
__global__ __launch_bounds__(kTreeThreads) void tree_build_kernel(
    const u64* __restrict__ part, const int32_t* __restrict__ root_tokens, int D, int W,
    int nch, int budget, int32_t* __restrict__ parent_out, int32_t* __restrict__ token_out,
    int32_t* __restrict__ depth_out, float* __restrict__ score_out) {
  __shared__ double s_score[kMaxPool];       // chunk lists, then pool scores, then sort keys
  __shared__ int16_t s_id[kMaxPool];         // sort payload: pool index
  __shared__ int16_t s_par[kMaxPool];        // parent pool index (-1: root)
  __shared__ int32_t s_tok[kMaxPool];
  __shared__ int8_t s_dep[kMaxPool];
  __shared__ int16_t s_node[kMaxPool];       // node number of a kept entry, else -1
  __shared__ float s_kscore[kMaxPool];       // fp32 score of a kept entry
  __shared__ int32_t s_ctok[kMaxDepth][kMaxW];
  __shared__ float s_clp[kMaxDepth][kMaxW];
  __shared__ int s_fidx[kMaxW];
  __shared__ double s_fscore[kMaxW];
  __shared__ double s_escore[64];            // eligible children of a level (see B)
  __shared__ int s_eidx[64];
  __shared__ int s_wsum[kTreeThreads / 64];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  constexpr int kWaves = kTreeThreads / 64;

  // A. candidates of every depth: the chunks' sorted lists are staged in LDS
  // (D * nch * W <= kMaxPool) and merged into a wavefront list, one
  // wavefront per depth (keys are unique)
  u64* s_lists = reinterpret_cast<u64*>(s_score);
  for (int e = tid; e < D * nch * W; e += kTreeThreads) {
    const int r = e % W, dc = e / W;  // dc = d * nch + c
    s_lists[e] = part[((size_t)b * D * nch + dc) * kMaxW + r];
  }
  __syncthreads();
  const int nl = nch * W;
  for (int d = wave; d < D; d += kWaves) {
    const u64* lists = s_lists + (size_t)d * nl;
    // the first 64 keys sorted across the lanes start the list (as in
    // kernel 1), the rest are offered
    WaveList m;
    const u64 sk = wave_sort_desc(lane < nl ? lists[lane] : 0ull, lane);
    m.L = lane < W ? sk : 0ull;
    m.thr = readlane_u64(sk, W - 1);
    for (int i0 = 64; i0 < nl; i0 += 64)
      m.offer(i0 + lane < nl ? lists[i0 + lane] : 0ull, 0, W, lane);
    if (lane < W) {
      s_ctok[d][lane] = key_token(m.L);
      s_clp[d][lane] = key_value(m.L);
    }
  }
  __syncthreads();  // s_score is free again

  // B. breadth-first levels, all in wavefront 0 (LDS accesses of one
  // wavefront are ordered, so no barrier is needed between levels): the
  // children of the frontier in generation order, then the next frontier
  // by rank counting (score descending, then generation).
  // Only children (r, j) with (r + 1)(j + 1) <= W can reach the frontier:
  // the frontier (by rank) and the candidate log-probabilities are both in
  // descending order and fp64 addition is monotone, so the other children
  // (r', j') with r' <= r and j' <= j score at least as high and come
  // earlier in generation order, which puts (r, j) at rank >= (r+1)(j+1)-1.
  // The W best children are therefore all eligible, and every child that
  // beats an eligible child ranked below W is eligible too: ranks counted
  // among the eligible children (kept in generation order) are the true
  // ranks wherever they are below W, and at least W elsewhere.  At most
  // sum_r floor(W / (r + 1)) <= 50 children are eligible (W <= 16).
  if (wave == 0) {
    if (lane == 0) {
      s_fidx[0] = -1;
      s_fscore[0] = 0.0;
    }
    int base = 0, fsize = 1;
    for (int d = 1; d <= D; ++d) {
      const int lsz = fsize * W;
      for (int t = lane; t < lsz; t += 64) {
        const int r = t / W, j = t - (t / W) * W;
        s_score[base + t] = s_fscore[r] + (double)s_clp[d - 1][j];
        s_par[base + t] = (int16_t)s_fidx[r];
        s_tok[base + t] = s_ctok[d - 1][j];
        s_dep[base + t] = (int8_t)d;
      }
      int ne = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // lsz <= 256: up to four children per lane
        const int t = lane + 64 * q;
        const int r = t / W, j = t - (t / W) * W;
        const bool el = t < lsz && (r + 1) * (j + 1) <= W;
        const u64 m = __ballot(el);
        if (el) {
          const int k = ne + __popcll(m & ((1ull << lane) - 1ull));
          s_escore[k] = s_score[base + t];
          s_eidx[k] = base + t;
        }
        ne += __popcll(m);
      }
      int nrank = kMaxW, nidx = 0;
      double nsc = 0.0;
      if (lane < ne) {
        nsc = s_escore[lane];
        nidx = s_eidx[lane];
        nrank = rank_among(s_escore, ne, nsc, lane);
      }
      // every read of the old frontier is done before it is overwritten
      if (nrank < W) {
        s_fidx[nrank] = nidx;
        s_fscore[nrank] = nsc;
      }
      fsize = lsz < W ? lsz : W;
      base += lsz;
    }
    if (lane == 0) s_wsum[0] = base;
  }
  __syncthreads();
  const int C = s_wsum[0];
  __syncthreads();  // s_wsum is reused by the scan

  PoolLds pl{s_score, s_id, s_par, s_tok, s_dep, s_node, s_kscore, s_wsum};
  cut_number_write(pl, C, budget, root_tokens, parent_out, token_out, depth_out, score_out);
}


// ---- branch-conditioned construction, one level per launch pair.
//
// The draft head conditions each branch on its own path (JetSpec abstract:
// branch-wise causal conditioning), so the candidates below a frontier node
// come from that node's own row: logp[b][r][V] is the row of the token after
// the path of frontier node r (rank order; level 1: row 0, for the root).
// The per-sequence state between launches lives in the workspace: the
// candidate pool (score, parent pool index, token, depth) and the current
// frontier (pool index and score by rank).  Level d appends the F * W
// children of the F = (d == 1 ? 1 : W) frontier nodes at pool index
// W + (d - 2) W^2 (0 for d = 1); the finish kernel then runs the budget cut
// and numbering of the one-launch builder on that pool.

constexpr int kStateHdr = 256;  // frontier scores (16 x f64) and pool indices (16 x i32)

__host__ __device__ inline int level_pool_base(int level, int W) {
  return level == 1 ? 0 : W + (level - 2) * W * W;
}

struct LevelState {
  double* fscore;
  int* fidx;
  double* score;
  int* par;
  int* tok;
  int* dep;
};

__device__ __forceinline__ LevelState level_state(unsigned char* state, size_t stride, int pcap,
                                                  int b) {
  unsigned char* st = state + (size_t)b * stride;
  LevelState s;
  s.fscore = reinterpret_cast<double*>(st);
  s.fidx = reinterpret_cast<int*>(st + kMaxW * sizeof(double));
  s.score = reinterpret_cast<double*>(st + kStateHdr);
  s.par = reinterpret_cast<int*>(s.score + pcap);
  s.tok = s.par + pcap;
  s.dep = s.tok + pcap;
  return s;
}

// One workgroup per sequence: merge each frontier row's chunk lists into its
// `W` candidates (one wavefront per row), append the children to the pool,
// rank them (score descending, then generation order) and keep the W best as
// the next frontier.  frontier_src / frontier_tok [B][W] name, for each new
// frontier rank, the rank of its parent in the previous frontier and its
// token, so that the caller can extend the paths it conditions on.
__global__ __launch_bounds__(kTreeThreads) void tree_level_kernel(
    const u64* __restrict__ part, int nch, int W, int level, int pcap, size_t stride,
    unsigned char* __restrict__ state, int32_t* __restrict__ frontier_src,
    int32_t* __restrict__ frontier_tok) {
  __shared__ u64 s_lists[kMaxPool];          // F * nch * W <= kMaxPool
  __shared__ int32_t s_ctok[kMaxW][kMaxW];
  __shared__ float s_clp[kMaxW][kMaxW];
  __shared__ int s_fidx[kMaxW];
  __shared__ double s_fscore[kMaxW];
  __shared__ double s_esc[kMaxW * kMaxW];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int F = level == 1 ? 1 : W;
  const int base = level_pool_base(level, W);
  const LevelState g = level_state(state, stride, pcap, b);
  const int nl = nch * W;
  for (int e = tid; e < F * nl; e += kTreeThreads)
    s_lists[e] = part[((size_t)b * F * nch + e / W) * kMaxW + e % W];
  if (tid < F) {
    s_fidx[tid] = level == 1 ? -1 : g.fidx[tid];
    s_fscore[tid] = level == 1 ? 0.0 : g.fscore[tid];
  }
  __syncthreads();
  if (wave < F) {  // the candidates of frontier row `wave` (keys are unique)
    const u64* lists = s_lists + wave * nl;
    WaveList m;
    const u64 sk = wave_sort_desc(lane < nl ? lists[lane] : 0ull, lane);
    m.L = lane < W ? sk : 0ull;
    m.thr = readlane_u64(sk, W - 1);
    for (int i0 = 64; i0 < nl; i0 += 64)
      m.offer(i0 + lane < nl ? lists[i0 + lane] : 0ull, 0, W, lane);
    if (lane < W) {
      s_ctok[wave][lane] = key_token(m.L);
      s_clp[wave][lane] = key_value(m.L);
    }
  }
  __syncthreads();
  // children in generation order t = r * W + j; every read of the old
  // frontier (in LDS) precedes the writes of the new one
  const int nc = F * W;
  double sc = 0.0;
  int tok = 0, r = 0;
  if (tid < nc) {
    r = tid / W;
    const int j = tid - r * W;
    sc = s_fscore[r] + (double)s_clp[r][j];
    tok = s_ctok[r][j];
    s_esc[tid] = sc;
    g.score[base + tid] = sc;
    g.par[base + tid] = s_fidx[r];
    g.tok[base + tid] = tok;
    g.dep[base + tid] = level;
  }
  __syncthreads();
  if (tid < nc) {
    const int rank = rank_among(s_esc, nc, sc, tid);
    if (rank < W) {
      g.fidx[rank] = base + tid;
      g.fscore[rank] = sc;
      frontier_src[(size_t)b * W + rank] = r;
      frontier_tok[(size_t)b * W + rank] = tok;
    }
  }
}

// One workgroup per sequence: the pool of all levels into LDS, then the
// budget cut, numbering and outputs of the one-launch builder.
__global__ __launch_bounds__(kTreeThreads) void tree_finish_kernel(
    const int32_t* __restrict__ root_tokens, int C, int budget, int pcap, size_t stride,
    unsigned char* __restrict__ state, int32_t* __restrict__ parent_out,
    int32_t* __restrict__ token_out, int32_t* __restrict__ depth_out,
    float* __restrict__ score_out) {
  __shared__ double s_score[kMaxPool];
  __shared__ int16_t s_id[kMaxPool];
  __shared__ int16_t s_par[kMaxPool];
  __shared__ int32_t s_tok[kMaxPool];
  __shared__ int8_t s_dep[kMaxPool];
  __shared__ int16_t s_node[kMaxPool];
  __shared__ float s_kscore[kMaxPool];
  __shared__ int s_wsum[kTreeThreads / 64];
  const LevelState g = level_state(state, stride, pcap, blockIdx.x);
  for (int i = threadIdx.x; i < C; i += kTreeThreads) {
    s_score[i] = g.score[i];
    s_par[i] = (int16_t)g.par[i];
    s_tok[i] = g.tok[i];
    s_dep[i] = (int8_t)g.dep[i];
  }
  __syncthreads();
  PoolLds pl{s_score, s_id, s_par, s_tok, s_dep, s_node, s_kscore, s_wsum};
  cut_number_write(pl, C, budget, root_tokens, parent_out, token_out, depth_out, score_out);
}

// Vocabulary chunks per row: about 512 workgroups in all, chunks of at least
// 4096 entries, and few enough that every depth's lists fit the tree
// kernel's LDS staging.
int tb_chunks(int B, int D, int V, int W) {
  int nch = (512 + B * D - 1) / (B * D);
  const int max_by_len = V / 4096 > 0 ? V / 4096 : 1;
  if (nch > max_by_len) nch = max_by_len;
  if (nch > kMaxPool / (D * W)) nch = kMaxPool / (D * W);
  return nch < 1 ? 1 : nch;
}

}  // namespace

int tree_build_pool(int D, int W) { return W + (D - 1) * W * W; }

size_t tree_build_ws_bytes(int B, int D, int V, int W) {
  return (size_t)B * D * tb_chunks(B, D, V, W) * kMaxW * sizeof(u64);
}

hipError_t launch_tree_build(const float* logp, const int32_t* root_tokens, int B, int D, int V,
                             int W, int budget, int32_t* parent, int32_t* tokens,
                             int32_t* node_depth, float* score, void* ws, hipStream_t stream) {
  const int nch = tb_chunks(B, D, V, W);
  const int chunk_len = (V + nch - 1) / nch;
  u64* part = static_cast<u64*>(ws);
  hipLaunchKernelGGL(draft_topk_kernel, dim3(B * D * nch), dim3(kTopThreads), 0, stream, logp,
                     V, W, nch, chunk_len, D, D, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tree_build_kernel, dim3(B), dim3(kTreeThreads), 0, stream, part,
                     root_tokens, D, W, nch, budget, parent, tokens, node_depth, score);
  return hipGetLastError();
}


namespace {

// Vocabulary chunks per frontier row of a level: about 512 workgroups in all,
// chunks of at least 4096 entries, and at most W * W * nch <= kMaxPool keys
// staged by the level kernel.
int tb_level_chunks(int B, int V, int W) {
  int nch = (512 + B * W - 1) / (B * W);
  const int max_by_len = V / 4096 > 0 ? V / 4096 : 1;
  if (nch > max_by_len) nch = max_by_len;
  if (nch > kMaxPool / (W * W)) nch = kMaxPool / (W * W);
  return nch < 1 ? 1 : nch;
}

size_t level_state_stride(int D, int W) {
  const size_t pcap = (size_t)tree_build_pool(D, W);
  const size_t bytes = kStateHdr + pcap * (sizeof(double) + 3 * sizeof(int));
  return (bytes + 255) / 256 * 256;
}

size_t level_part_bytes(int B, int V, int W) {
  return (size_t)B * W * tb_level_chunks(B, V, W) * kMaxW * sizeof(u64);
}

}  // namespace

size_t tree_level_ws_bytes(int B, int D, int V, int W) {
  return level_part_bytes(B, V, W) + (size_t)B * level_state_stride(D, W);
}

hipError_t launch_tree_level(const float* logp, int level, int B, int D, int V, int W,
                             int32_t* frontier_src, int32_t* frontier_tok, void* ws,
                             hipStream_t stream) {
  const int nch = tb_level_chunks(B, V, W);
  const int chunk_len = (V + nch - 1) / nch;
  const int F = level == 1 ? 1 : W;
  u64* part = static_cast<u64*>(ws);
  unsigned char* state = static_cast<unsigned char*>(ws) + level_part_bytes(B, V, W);
  hipLaunchKernelGGL(draft_topk_kernel, dim3(B * F * nch), dim3(kTopThreads), 0, stream, logp,
                     V, W, nch, chunk_len, F, W, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tree_level_kernel, dim3(B), dim3(kTreeThreads), 0, stream, part, nch, W,
                     level, tree_build_pool(D, W), level_state_stride(D, W), state,
                     frontier_src, frontier_tok);
  return hipGetLastError();
}

hipError_t launch_tree_finish(const int32_t* root_tokens, int B, int D, int V, int W, int budget,
                              int32_t* parent, int32_t* tokens, int32_t* node_depth, float* score,
                              void* ws, hipStream_t stream) {
  unsigned char* state = static_cast<unsigned char*>(ws) + level_part_bytes(B, V, W);
  const int pcap = tree_build_pool(D, W);
  hipLaunchKernelGGL(tree_finish_kernel, dim3(B), dim3(kTreeThreads), 0, stream, root_tokens,
                     pcap, budget, pcap, level_state_stride(D, W), state, parent, tokens,
                     node_depth, score);
  return hipGetLastError();
}

}  // namespace tv
