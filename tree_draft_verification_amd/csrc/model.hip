// Multi-layer verification pass: a dense Qwen3-style decoder stack run over
// every node of the draft trees in one pass, then the LM head with argmax.
//
// The target model verifies the whole draft tree in one forward pass under a
// tree-causal mask (JetSpec GitHub README, "JetSpec > Overview"); the pages'
// targets are dense and MoE Qwen3 models (JetSpec abstract), and the serving
// engine compiles verification and replays it as a graph (README, "Quick
// Start").  Per layer, with x the fp32 residual stream of the B*N nodes:
//
//   h = bf16(rmsnorm(x) * ln1)                       (fused into the epilogue
//                                                     that produced x)
//   qkv = h Wqkv^T                                   split-K projection
//   q, k = rope(rmsnorm(q|k) * q_norm|k_norm, L_b + depth), v as is
//          q -> Q buffer, k and v -> cache rows L_b + i of this layer
//   o = tree_attention(Q, cache)                     (the single-layer kernel)
//   x += o Wo^T ; h = bf16(rmsnorm(x) * ln2)         split-K + fused epilogue
//   a = bf16(silu(h Wg^T) * (h Wu^T))                split-K + fused epilogue
//   x += a Wd^T ; h = bf16(rmsnorm(x) * next norm)   split-K + fused epilogue
//
// and after the last layer the LM-head kernel takes argmax over h Wlm^T.
//
// Projections stream their packed bf16 weights with the LM-head kernel in its
// split-K store mode: a workgroup writes the fp32 partial sums of its k range
// and the epilogue kernels below add the splits in a fixed order (so the pass
// is deterministic) and apply the elementwise and row-wise steps on the way.
// Every buffer between kernels lives in the caller's workspace; nothing is
// allocated and nothing is cleared with a memset, so the pass can be captured
// in a HIP graph and replayed.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr float kTwoPi = 6.283185307179586f;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over a 256-thread workgroup (every thread gets the result).
__device__ __forceinline__ float block_sum256(float v, float* s_red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // s_red free from any earlier use
  if ((threadIdx.x & 63) == 0) s_red[wave] = v;
  __syncthreads();
  return s_red[0] + s_red[1] + s_red[2] + s_red[3];
}

__device__ __forceinline__ void flag(int32_t* st, int b, int f) {
  if (st) atomicOr(&st[b], f);
}

// ---- positions, embedding and the first layer's input norm (one workgroup
// per node row m = b*N + i).  pos[m] = L_b + depth(i), or -1 when the length
// of sequence b or the root path of node i is malformed (a row with pos -1 is
// never written to the caches).
// Workgroup 0 also clears the LM head's key region of the workspace (the LM
// head needs it zero and leaves it zero; clearing it here makes the pass
// independent of what earlier calls with other shapes left in the buffer).
__global__ __launch_bounds__(256) void prep_kernel(
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ seq_lens, const bf16_t* __restrict__ embed,
    const bf16_t* __restrict__ ln1, float* __restrict__ x, bf16_t* __restrict__ h,
    int32_t* __restrict__ pos, int32_t* __restrict__ dev_status, int N, int hidden, int V,
    int Lcap, int max_seq_len, float eps, uint32_t* __restrict__ lm_zero, int lm_zero_words) {
  __shared__ float s_red[4];
  const int m = blockIdx.x;
  const int b = m / N;
  const int i = m - b * N;
  const int tid = threadIdx.x;
  if (m == 0)
    for (int w = tid; w < lm_zero_words; w += 256) lm_zero[w] = 0u;
  if (tid == 0) {
    const int32_t* par = parent + (size_t)b * N;
    const int L = seq_lens[b];
    bool ok = L >= 0 && L <= max_seq_len && L + N <= Lcap;
    if (!ok) flag(dev_status, b, TV_STATUS_BAD_LEN);
    // depth by walking parents; every step must go to a smaller index
    int d = 0, j = i;
    bool tree_ok = (par[0] == -1);
    while (j > 0 && tree_ok) {
      const int p = par[j];
      tree_ok = p >= 0 && p < j;
      j = p;
      ++d;
    }
    if (!tree_ok) flag(dev_status, b, TV_STATUS_BAD_PARENT);
    pos[m] = (ok && tree_ok) ? L + d : -1;
  }
  int tok = tokens[m];
  if (tok < 0 || tok >= V) {
    if (tid == 0) flag(dev_status, b, TV_STATUS_BAD_TOKEN);
    tok = 0;
  }
  const bf16_t* e = embed + (size_t)tok * hidden;
  float* xr = x + (size_t)m * hidden;
  float ss = 0.f;
  for (int n = tid; n < hidden; n += 256) {
    const float v = bf16_to_f32(e[n]);
    xr[n] = v;
    ss += v * v;
  }
  const float r = rsqrtf(block_sum256(ss, s_red) / (float)hidden + eps);
  bf16_t* hr = h + (size_t)m * hidden;
  for (int n = tid; n < hidden; n += 256)
    hr[n] = (bf16_t)f32_to_bf16(xr[n] * r * bf16_to_f32(ln1[n]));
}

// ---- after the QKV projection: one wavefront per (row, head).  Lane j < D/2
// holds the rotary pair (j, j + D/2).  Query heads: per-head RMSNorm, rotary
// embedding, stored to Q [M][Hq][D].  Key heads: the same with k_norm, stored
// to cache row L_b + i.  Value heads: stored as they are.
__global__ __launch_bounds__(256) void epi_qkv_kernel(
    const float* __restrict__ part, int nsplit, int M, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ seq_lens, const bf16_t* __restrict__ q_norm,
    const bf16_t* __restrict__ k_norm, bf16_t* __restrict__ Q, bf16_t* __restrict__ kc,
    bf16_t* __restrict__ vc, int N, int Hq, int Hkv, int D, int Lcap, float eps,
    float log2_theta) {
  const int heads = Hq + 2 * Hkv;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= M * heads) return;
  const int lane = threadIdx.x & 63;
  const int m = item / heads;
  const int hd = item - m * heads;
  const int half = D >> 1;
  const bool act = lane < half;
  const int d0 = act ? lane : 0;
  const int ncol = heads * D;
  const float* src = part + (size_t)m * ncol + (size_t)hd * D;
  float v0 = 0.f, v1 = 0.f;
  for (int s = 0; s < nsplit; ++s) {  // fixed order: deterministic
    v0 += src[(size_t)s * M * ncol + d0];
    v1 += src[(size_t)s * M * ncol + d0 + half];
  }
  if (!act) v0 = v1 = 0.f;
  const int p = pos[m];
  const int b = m / N;
  const int i = m - b * N;
  if (hd < Hq + Hkv) {
    const bf16_t* w = (hd < Hq) ? q_norm : k_norm;
    const float r = rsqrtf(wave_sum(v0 * v0 + v1 * v1) / (float)D + eps);
    v0 *= r * bf16_to_f32(w[d0]);
    v1 *= r * bf16_to_f32(w[d0 + half]);
    // angle p * theta^(-2 d0 / D), formed and reduced in fp64 so that long
    // positions keep full fp32 accuracy in the sine and cosine
    const double inv = exp2(-(2.0 * d0 / D) * (double)log2_theta);
    double ang = (double)(p < 0 ? 0 : p) * inv;
    ang -= (double)kTwoPi * rint(ang / (double)kTwoPi);
    float sn, cs;
    sincosf((float)ang, &sn, &cs);
    const float r0 = v0 * cs - v1 * sn;
    const float r1 = v1 * cs + v0 * sn;
    v0 = r0;
    v1 = r1;
  }
  if (!act || p < 0) return;
  bf16_t* dst;
  if (hd < Hq) {
    dst = Q + ((size_t)m * Hq + hd) * D;
  } else {
    const int hk = (hd < Hq + Hkv) ? hd - Hq : hd - Hq - Hkv;
    bf16_t* cache = (hd < Hq + Hkv) ? kc : vc;
    const int L = seq_lens[b];
    dst = cache + (((size_t)b * Hkv + hk) * Lcap + (L + i)) * D;
  }
  dst[d0] = (bf16_t)f32_to_bf16(v0);
  dst[d0 + half] = (bf16_t)f32_to_bf16(v1);
}

// ---- after the output and down projections: x += sum of splits, then
// h = bf16(rmsnorm(x) * w) for the next projection (and, for the last layer,
// the fp32 normalised row to hout when requested).  One workgroup of up to
// 1024 threads per row, four columns per thread per trip; every split's
// loads of a trip are issued before they are added (in split order).
constexpr int kNormThreads = 1024;

__device__ __forceinline__ float block_sum(float v, float* s_red, int nwaves) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nwaves; ++i) t += s_red[i];
  return t;
}

__global__ __launch_bounds__(kNormThreads) void epi_resid_norm_kernel(
    const float* __restrict__ part, int nsplit, int M, int hidden, float* __restrict__ x,
    const bf16_t* __restrict__ w, bf16_t* __restrict__ h, float* __restrict__ hout, float eps) {
  __shared__ float s_red[kNormThreads / 64];
  constexpr int kMaxTrips = 4;  // hidden <= 4 * 4 * 1024
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  float* xr = x + (size_t)m * hidden;
  f32x4_t v[kMaxTrips];
  float ss = 0.f;
#pragma unroll
  for (int t = 0; t < kMaxTrips; ++t) {
    const int n = 4 * (tid + t * nt);
    if (n >= hidden) break;
    f32x4_t a = *reinterpret_cast<const f32x4_t*>(xr + n);
    const float* pp = part + (size_t)m * hidden + n;
    const size_t sstride = (size_t)M * hidden;
    int s = 0;
    for (; s + 4 <= nsplit; s += 4) {
      const f32x4_t p0 = *reinterpret_cast<const f32x4_t*>(pp + (s + 0) * sstride);
      const f32x4_t p1 = *reinterpret_cast<const f32x4_t*>(pp + (s + 1) * sstride);
      const f32x4_t p2 = *reinterpret_cast<const f32x4_t*>(pp + (s + 2) * sstride);
      const f32x4_t p3 = *reinterpret_cast<const f32x4_t*>(pp + (s + 3) * sstride);
      a += p0;
      a += p1;
      a += p2;
      a += p3;
    }
    for (; s < nsplit; ++s) a += *reinterpret_cast<const f32x4_t*>(pp + s * sstride);
    *reinterpret_cast<f32x4_t*>(xr + n) = a;
    ss += a[0] * a[0] + a[1] * a[1] + a[2] * a[2] + a[3] * a[3];
    v[t] = a;
  }
  const float r = rsqrtf(block_sum(ss, s_red, nt >> 6) / (float)hidden + eps);
#pragma unroll
  for (int t = 0; t < kMaxTrips; ++t) {
    const int n = 4 * (tid + t * nt);
    if (n >= hidden) break;
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = v[t][e] * r * bf16_to_f32(w[n + e]);
    u32x2_t pk;
    pk.x = f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16);
    pk.y = f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16);
    *reinterpret_cast<u32x2_t*>(h + (size_t)m * hidden + n) = pk;
    if (hout) *reinterpret_cast<f32x4_t*>(hout + (size_t)m * hidden + n) = f32x4_t{o[0], o[1], o[2], o[3]};
  }
}

// Threads per row of epi_resid_norm_kernel: hidden/4 up to 1024 (a multiple
// of 64, since hidden is a multiple of 256).
int norm_threads(int hidden) { return hidden / 4 < kNormThreads ? hidden / 4 : kNormThreads; }

// ---- after the gate/up projection when it runs split: a = bf16(silu(gate) *
// up), four columns per thread.  The weight is packed interleaved, so the
// gate value of feature f = 64 t + j is column 128 t + j of the partial sums
// and its up value column 128 t + 64 + j.
__global__ __launch_bounds__(256) void epi_swiglu_kernel(const float* __restrict__ part,
                                                         int nsplit, int M, int I,
                                                         bf16_t* __restrict__ a) {
  const int q4 = I >> 2;
  const size_t total = (size_t)M * q4;
  for (size_t t = (size_t)blockIdx.x * 256 + threadIdx.x; t < total;
       t += (size_t)gridDim.x * 256) {
    const int m = (int)(t / q4);
    const int j = (int)(t - (size_t)m * q4) * 4;
    const int cg = 128 * (j >> 6) + (j & 63);
    f32x4_t g = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nsplit; ++s) {
      const float* row = part + ((size_t)s * M + m) * (2 * (size_t)I);
      g += *reinterpret_cast<const f32x4_t*>(row + cg);
      u += *reinterpret_cast<const f32x4_t*>(row + cg + 64);
    }
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = g[e] / (1.f + __expf(-g[e])) * u[e];
    u32x2_t pk;
    pk.x = f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16);
    pk.y = f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16);
    *reinterpret_cast<u32x2_t*>(a + (size_t)m * I + j) = pk;
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

PassPlan pass_plan(const tv_model_dims& d, int B, int N, int max_seq_len) {
  PassPlan p{};
  const int M = B * N;
  const int qkv = (d.Hq + 2 * d.Hkv) * d.D;
  p.s_qkv = proj_splits(M, d.hidden, qkv);
  p.s_o = proj_splits(M, d.Hq * d.D, d.hidden);
  p.s_gu = proj_splits(M, d.hidden, 2 * d.inter);
  p.s_down = proj_splits(M, d.inter, d.hidden);
  p.attn = attn_plan(B, N, d.Hq, d.Hkv, d.D, max_seq_len, TV_BF16, 0);
  size_t part = 0;
  auto upd = [&](size_t v) { part = v > part ? v : part; };
  upd((size_t)p.s_qkv * qkv);
  upd((size_t)p.s_o * d.hidden);
  upd((size_t)p.s_gu * 2 * d.inter);
  upd((size_t)p.s_down * d.hidden);
  size_t gin = (size_t)d.hidden;  // normalised hidden rows or attention output
  if ((size_t)d.Hq * d.D > gin) gin = (size_t)d.Hq * d.D;
  size_t off = 0;
  p.off_lm = off;
  off += align256(lmhead_ws_bytes(M, d.hidden, d.vocab, TV_BF16));
  p.off_pos = off;
  off += align256((size_t)M * 4);
  p.off_x = off;
  off += align256((size_t)M * d.hidden * 4);
  p.off_gin = off;
  off += align256((size_t)M * gin * 2);
  p.off_q = off;
  off += align256((size_t)M * d.Hq * d.D * 2);
  p.off_act = off;
  off += align256((size_t)M * d.inter * 2);
  p.off_part = off;
  off += align256((size_t)M * part * 4);
  p.off_attn = off;
  off += align256(p.attn.ws_bytes);
  p.ws_bytes = off;
  return p;
}

size_t packed_layer_bytes(int rows, int K) { return lmhead_packed_bytes(rows, K); }

hipError_t launch_verify_pass(const tv_model_dims& d, const tv_model_weights& w,
                              const PassPlan& p, const int32_t* tokens, const int32_t* parent,
                              const int32_t* seq_lens, void* k_cache, void* v_cache, int B,
                              int N, int Lcap, int max_seq_len, int32_t* argmax, float* logits,
                              float* hidden_out, void* ws, int32_t* dev_status,
                              hipStream_t stream) {
  const int M = B * N;
  char* base = static_cast<char*>(ws);
  int32_t* pos = reinterpret_cast<int32_t*>(base + p.off_pos);
  float* x = reinterpret_cast<float*>(base + p.off_x);
  bf16_t* gin = reinterpret_cast<bf16_t*>(base + p.off_gin);
  bf16_t* Q = reinterpret_cast<bf16_t*>(base + p.off_q);
  bf16_t* act = reinterpret_cast<bf16_t*>(base + p.off_act);
  const bool fused_mlp = proj_swiglu_fused(M, d.hidden, d.inter);
  float* part = reinterpret_cast<float*>(base + p.off_part);
  void* attn_ws = base + p.off_attn;
  const int qkv = (d.Hq + 2 * d.Hkv) * d.D;
  const size_t pb_qkv = packed_layer_bytes(qkv, d.hidden);
  const size_t pb_o = packed_layer_bytes(d.hidden, d.Hq * d.D);
  const size_t pb_gu = packed_layer_bytes(2 * d.inter, d.hidden);
  const size_t pb_down = packed_layer_bytes(d.hidden, d.inter);
  const size_t layer_elems = (size_t)B * d.Hkv * Lcap * d.D;
  const bf16_t* ln1 = static_cast<const bf16_t*>(w.ln1);
  const bf16_t* ln2 = static_cast<const bf16_t*>(w.ln2);
  const bf16_t* qn = static_cast<const bf16_t*>(w.q_norm);
  const bf16_t* kn = static_cast<const bf16_t*>(w.k_norm);
  const char* wqkv = static_cast<const char*>(w.w_qkv);
  const char* wo = static_cast<const char*>(w.w_o);
  const char* wgu = static_cast<const char*>(w.w_gu);
  const char* wdown = static_cast<const char*>(w.w_down);
  const float log2_theta = log2f(d.rope_theta);
  const float scale = 1.0f / sqrtf((float)d.D);
  hipError_t e;

  hipLaunchKernelGGL(prep_kernel, dim3(M), dim3(256), 0, stream, tokens, parent, seq_lens,
                     static_cast<const bf16_t*>(w.embed), ln1, x, gin, pos, dev_status, N,
                     d.hidden, d.vocab, Lcap, max_seq_len, d.rms_eps,
                     reinterpret_cast<uint32_t*>(base + p.off_lm), (int)(lmhead_zero_bytes(M) / 4));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int heads = d.Hq + 2 * d.Hkv;
  for (int ly = 0; ly < d.layers; ++ly) {
    bf16_t* kc = static_cast<bf16_t*>(k_cache) + ly * layer_elems;
    bf16_t* vc = static_cast<bf16_t*>(v_cache) + ly * layer_elems;
    if ((e = launch_proj(gin, wqkv + ly * pb_qkv, part, M, d.hidden, qkv, p.s_qkv, stream)))
      return e;
    hipLaunchKernelGGL(epi_qkv_kernel, dim3((M * heads + 3) / 4), dim3(256), 0, stream, part,
                       p.s_qkv, M, pos, seq_lens, qn + (size_t)ly * d.D, kn + (size_t)ly * d.D,
                       Q, kc, vc, N, d.Hq, d.Hkv, d.D, Lcap, d.rms_eps, log2_theta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_tree_attn(Q, kc, vc, seq_lens, parent, gin, B, N, d.Hq, d.Hkv, d.D, Lcap,
                              max_seq_len, scale, TV_BF16, p.attn, attn_ws, dev_status, stream)))
      return e;
    if ((e = launch_proj(gin, wo + ly * pb_o, part, M, d.Hq * d.D, d.hidden, p.s_o, stream)))
      return e;
    hipLaunchKernelGGL(epi_resid_norm_kernel, dim3(M), dim3(norm_threads(d.hidden)), 0, stream,
                       part, p.s_o, M, d.hidden, x, ln2 + (size_t)ly * d.hidden, gin, nullptr,
                       d.rms_eps);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (fused_mlp) {
      if ((e = launch_proj_swiglu(gin, wgu + ly * pb_gu, act, M, d.hidden, d.inter, stream)))
        return e;
    } else {
      if ((e = launch_proj(gin, wgu + ly * pb_gu, part, M, d.hidden, 2 * d.inter, p.s_gu,
                           stream)))
        return e;
      const size_t sw_items = (size_t)M * (d.inter / 4);
      const unsigned sw_grid =
          (unsigned)((sw_items + 255) / 256 < 2048 ? (sw_items + 255) / 256 : 2048);
      hipLaunchKernelGGL(epi_swiglu_kernel, dim3(sw_grid), dim3(256), 0, stream, part, p.s_gu,
                         M, d.inter, act);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = launch_proj(act, wdown + ly * pb_down, part, M, d.inter, d.hidden, p.s_down,
                         stream)))
      return e;
    const bool last = ly + 1 == d.layers;
    const bf16_t* wn = last ? static_cast<const bf16_t*>(w.final_norm)
                            : ln1 + (size_t)(ly + 1) * d.hidden;
    hipLaunchKernelGGL(epi_resid_norm_kernel, dim3(M), dim3(norm_threads(d.hidden)), 0, stream,
                       part, p.s_down, M, d.hidden, x, wn, gin, last ? hidden_out : nullptr,
                       d.rms_eps);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return launch_lmhead_argmax(gin, w.lm_head, argmax, logits, M, d.hidden, d.vocab, TV_BF16,
                              TV_LAYOUT_PACKED, base + p.off_lm, p.off_pos - p.off_lm, stream);
}

}  // namespace tv
