// Public C ABI (include/treeverify.h): host-side validation, then launches.
// Every check here runs before any HIP call, so a rejected call has no
// effect on the device or the stream.
#include <math.h>
#include <stdio.h>

#include "tv_internal.h"

namespace {

thread_local char g_hip_msg[256];

bool dtype_ok(int dtype) { return dtype == TV_BF16 || dtype == TV_F32; }

}  // namespace

namespace tv {

int hip_status(hipError_t e) {
  if (e == hipSuccess) return TV_OK;
  snprintf(g_hip_msg, sizeof(g_hip_msg), "HIP launch failed: %s (%d)", hipGetErrorString(e),
           (int)e);
  return TV_EHIP;
}

int lmhead_check(const void* hidden, const void* w, const int32_t* argmax, int M, int K, int V,
                 int dtype, int w_layout) {
  if (!hidden || !w || !argmax) return TV_EINVAL;
  if (M < 1 || K < 1 || V < 1) return TV_EINVAL;
  if (w_layout != TV_LAYOUT_ROWMAJOR && w_layout != TV_LAYOUT_PACKED) return TV_EINVAL;
  if (!dtype_ok(dtype)) return TV_ENOTSUP;
  if (dtype == TV_BF16 && K % 256) return TV_ENOTSUP;
  if (dtype == TV_F32 && w_layout != TV_LAYOUT_ROWMAJOR) return TV_ENOTSUP;
  const long long blocks = dtype == TV_BF16
                               ? (long long)((M + 63) / 64) * ((V + 127) / 128)
                               : (long long)((M + 15) / 16) * ((V + 255) / 256);
  if (blocks > 2147483647LL) return TV_ENOTSUP;
  return TV_OK;
}

}  // namespace tv

using tv::hip_status;

extern "C" {

int tv_abi_version(void) { return 10000; }

const char* tv_status_string(int status) {
  switch (status) {
    case TV_OK: return "ok";
    case TV_EINVAL: return "invalid argument (shape, size or null pointer)";
    case TV_ENOTSUP: return "unsupported configuration (head dim, dtype, layout, node count or width)";
    case TV_EWORKSPACE: return "workspace missing or too small";
    case TV_EHIP: return g_hip_msg[0] ? g_hip_msg : "HIP launch failed";
    case TV_ESCRATCH:
      return "problem larger than the static scratch of the allocation-free call";
    default: return "unknown status";
  }
}

size_t tv_tree_verify_attn_workspace(int B, int N, int Hq, int Hkv, int D, int max_seq_len,
                                     int dtype) {
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || max_seq_len < 0) return 0;
  return tv::attn_plan(B, N, Hq, Hkv, D, max_seq_len, dtype, 0).ws_bytes;
}

int tv_tree_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seq_lens, const int32_t* parent, void* out, int B,
                        int N, int Hq, int Hkv, int D, int Lcap, int max_seq_len, float scale,
                        int dtype, void* workspace, size_t ws_bytes, int32_t* dev_status,
                        void* stream) {
  if (!q || !k_cache || !v_cache || !seq_lens || !parent || !out) return TV_EINVAL;
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || D < 1 || Lcap < 1 || max_seq_len < 0)
    return TV_EINVAL;
  if (Hq % Hkv) return TV_EINVAL;
  if ((long long)max_seq_len + N > Lcap) return TV_EINVAL;
  if (!isfinite(scale)) return TV_EINVAL;
  if (!dtype_ok(dtype)) return TV_ENOTSUP;
  if (D != 64 && D != 128) return TV_ENOTSUP;
  if (N > TV_MAX_NODES) return TV_ENOTSUP;
  if (dtype == TV_F32 && ((long long)N * Hq > 2147483647LL || B > 65535 || Hq > 65535))
    return TV_ENOTSUP;
  const tv::AttnPlan plan = tv::attn_plan(B, N, Hq, Hkv, D, max_seq_len, dtype, 0);
  if ((long long)B * Hkv * plan.nqblk * plan.nsplit > 2147483647LL) return TV_ENOTSUP;
  if (plan.ws_bytes > 0 && (!workspace || ws_bytes < plan.ws_bytes)) return TV_EWORKSPACE;
  return hip_status(tv::launch_tree_attn(q, k_cache, v_cache, seq_lens, parent, out, B, N, Hq,
                                         Hkv, D, Lcap, max_seq_len, scale, dtype, plan,
                                         workspace, dev_status,
                                         static_cast<hipStream_t>(stream)));
}

static bool page_size_ok(int ps) { return ps >= 1 && ps <= 4096 && (ps & (ps - 1)) == 0; }

size_t tv_tree_verify_attn_paged_workspace(int B, int N, int Hq, int Hkv, int D,
                                           int max_seq_len, int page_size, int dtype) {
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || max_seq_len < 0 ||
      !page_size_ok(page_size))
    return 0;
  return tv::attn_plan(B, N, Hq, Hkv, D, max_seq_len, dtype, page_size).ws_bytes;
}

int tv_tree_verify_attn_paged(const void* q, const void* k_pages, const void* v_pages,
                              const int32_t* block_table, int max_blocks, int page_size,
                              int num_pages, const int32_t* seq_lens, const int32_t* parent,
                              void* out, int B, int N, int Hq, int Hkv, int D, int max_seq_len,
                              float scale, int dtype, void* workspace, size_t ws_bytes,
                              int32_t* dev_status, void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !parent || !out)
    return TV_EINVAL;
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || D < 1 || max_blocks < 1 || num_pages < 1 ||
      max_seq_len < 0)
    return TV_EINVAL;
  if (Hq % Hkv) return TV_EINVAL;
  if (!page_size_ok(page_size)) return TV_EINVAL;
  if ((long long)max_seq_len + N > (long long)max_blocks * page_size) return TV_EINVAL;
  if ((long long)max_blocks * page_size > 2147483647LL) return TV_EINVAL;
  if (!isfinite(scale)) return TV_EINVAL;
  if (dtype != TV_BF16) return TV_ENOTSUP;  // paged caches: bf16 kernel only
  if (D != 64 && D != 128) return TV_ENOTSUP;
  if (N > TV_MAX_NODES) return TV_ENOTSUP;
  const tv::AttnPlan plan = tv::attn_plan(B, N, Hq, Hkv, D, max_seq_len, dtype, page_size);
  if ((long long)B * Hkv * plan.nqblk * plan.nsplit > 2147483647LL) return TV_ENOTSUP;
  if (plan.ws_bytes > 0 && (!workspace || ws_bytes < plan.ws_bytes)) return TV_EWORKSPACE;
  return hip_status(tv::launch_tree_attn(
      q, k_pages, v_pages, seq_lens, parent, out, B, N, Hq, Hkv, D, 0, max_seq_len, scale,
      dtype, plan, workspace, dev_status, static_cast<hipStream_t>(stream), block_table,
      max_blocks, page_size, num_pages));
}

int tv_kv_compact_paged(void* k_pages, void* v_pages, const int32_t* block_table, int max_blocks,
                        int page_size, int num_pages, int32_t* seq_lens, const int32_t* path,
                        const int32_t* path_len, int B, int Hkv, int D, int P, int dtype,
                        void* stream) {
  if (!k_pages || !v_pages || !block_table || !seq_lens || !path || !path_len) return TV_EINVAL;
  if (B < 1 || Hkv < 1 || D < 1 || P < 1 || max_blocks < 1 || num_pages < 1) return TV_EINVAL;
  if (!page_size_ok(page_size)) return TV_EINVAL;
  if ((long long)max_blocks * page_size > 2147483647LL) return TV_EINVAL;
  if (!dtype_ok(dtype)) return TV_ENOTSUP;
  const int esz = dtype == TV_F32 ? 4 : 2;
  if ((D * esz) % 16 || P > 64 || (long long)P * D * esz > 65536) return TV_ENOTSUP;
  if (B > 65535) return TV_ENOTSUP;
  return hip_status(tv::launch_kv_compact(k_pages, v_pages, seq_lens, path, path_len, B, Hkv, D,
                                          0, P, dtype, static_cast<hipStream_t>(stream),
                                          block_table, max_blocks, page_size, num_pages));
}

int tv_kv_commit_slots(int32_t* block_table, int32_t* seq_lens, const int32_t* path,
                       const int32_t* path_len, int B, int N, int P, int max_blocks,
                       int32_t* dev_status, void* stream) {
  if (!block_table || !seq_lens || !path || !path_len) return TV_EINVAL;
  if (B < 1 || N < 1 || P < 1 || max_blocks < 1) return TV_EINVAL;
  if (N > TV_MAX_NODES || P > 64 || N > max_blocks) return TV_ENOTSUP;
  if (B > 65535) return TV_ENOTSUP;
  return hip_status(tv::launch_kv_commit_slots(block_table, seq_lens, path, path_len, B, N, P,
                                               max_blocks, dev_status,
                                               static_cast<hipStream_t>(stream)));
}

size_t tv_lmhead_argmax_workspace(int M, int K, int V, int dtype) {
  if (M < 1) return 0;
  return tv::lmhead_ws_bytes(M, K, V, dtype);
}

size_t tv_lmhead_packed_bytes(int V, int K, int dtype) {
  if (V < 1 || K < 1 || dtype != TV_BF16 || K % 256) return 0;
  return tv::lmhead_packed_bytes(V, K);
}

int tv_lmhead_pack_weights(const void* w, void* w_packed, int V, int K, int dtype,
                           void* stream) {
  if (!w || !w_packed || w == w_packed) return TV_EINVAL;
  if (V < 1 || K < 1) return TV_EINVAL;
  if (dtype != TV_BF16 || K % 256) return TV_ENOTSUP;
  return hip_status(tv::launch_lmhead_pack(w, w_packed, V, K, static_cast<hipStream_t>(stream)));
}

int tv_pack_gate_up_weights(const void* w, void* w_packed, int inter, int K, int dtype,
                            void* stream) {
  if (!w || !w_packed || w == w_packed) return TV_EINVAL;
  if (inter < 1 || K < 1) return TV_EINVAL;
  if (dtype != TV_BF16 || K % 256 || inter % 64) return TV_ENOTSUP;
  return hip_status(
      tv::launch_pack_gate_up(w, w_packed, inter, K, static_cast<hipStream_t>(stream)));
}

int tv_lmhead_argmax(const void* hidden, const void* w, int32_t* argmax, float* logits, int M,
                     int K, int V, int dtype, int w_layout, void* workspace, size_t ws_bytes,
                     void* stream) {
  const int st = tv::lmhead_check(hidden, w, argmax, M, K, V, dtype, w_layout);
  if (st != TV_OK) return st;
  if (!workspace || ws_bytes < tv::lmhead_ws_bytes(M, K, V, dtype)) return TV_EWORKSPACE;
  return hip_status(tv::launch_lmhead_argmax(hidden, w, argmax, logits, M, K, V, dtype, w_layout,
                                             workspace, ws_bytes,
                                             static_cast<hipStream_t>(stream)));
}

int tv_tree_accept(const int32_t* parent, const int32_t* draft_tokens,
                   const int32_t* target_tokens, int32_t* path, int32_t* path_len,
                   int32_t* bonus, int B, int N, int P, int32_t* dev_status, void* stream) {
  if (!parent || !draft_tokens || !target_tokens || !path || !path_len || !bonus)
    return TV_EINVAL;
  if (B < 1 || N < 1 || P < 1) return TV_EINVAL;
  if (N > TV_MAX_NODES || P > 64 || B > 2147483647) return TV_ENOTSUP;
  return hip_status(tv::launch_tree_accept(parent, draft_tokens, target_tokens, path, path_len,
                                           bonus, B, N, P, dev_status,
                                           static_cast<hipStream_t>(stream)));
}

int tv_kv_compact(void* k_cache, void* v_cache, int32_t* seq_lens, const int32_t* path,
                  const int32_t* path_len, int B, int Hkv, int D, int Lcap, int P, int dtype,
                  void* stream) {
  if (!k_cache || !v_cache || !seq_lens || !path || !path_len) return TV_EINVAL;
  if (B < 1 || Hkv < 1 || D < 1 || Lcap < 1 || P < 1) return TV_EINVAL;
  if (!dtype_ok(dtype)) return TV_ENOTSUP;
  const int esz = dtype == TV_F32 ? 4 : 2;
  if ((D * esz) % 16 || P > 64 || (long long)P * D * esz > 65536) return TV_ENOTSUP;
  if (B > 65535 || Hkv > 2147483647) return TV_ENOTSUP;
  return hip_status(tv::launch_kv_compact(k_cache, v_cache, seq_lens, path, path_len, B, Hkv, D,
                                          Lcap, P, dtype, static_cast<hipStream_t>(stream)));
}

int tv_accept_compact(const int32_t* parent, const int32_t* draft_tokens,
                      const int32_t* target_tokens, int32_t* path, int32_t* path_len,
                      int32_t* bonus, void* k_cache, void* v_cache, int32_t* seq_lens, int B,
                      int N, int P, int Hkv, int D, int Lcap, int dtype, int32_t* dev_status,
                      void* stream) {
  if (!parent || !draft_tokens || !target_tokens || !path || !path_len || !bonus || !k_cache ||
      !v_cache || !seq_lens)
    return TV_EINVAL;
  if (B < 1 || N < 1 || P < 1 || Hkv < 1 || D < 1 || Lcap < 1) return TV_EINVAL;
  if (!dtype_ok(dtype)) return TV_ENOTSUP;
  const int esz = dtype == TV_F32 ? 4 : 2;
  if (N > TV_MAX_NODES || P > 64 || (D * esz) % 16 || (long long)P * D * esz > 65536)
    return TV_ENOTSUP;
  if (B > 65535) return TV_ENOTSUP;
  return hip_status(tv::launch_accept_compact(parent, draft_tokens, target_tokens, path, path_len,
                                              bonus, k_cache, v_cache, seq_lens, B, N, P, Hkv, D,
                                              Lcap, dtype, dev_status,
                                              static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------- multi-layer pass

namespace {

// 0 when the dims are usable, else the status to return.
int dims_status(const tv_model_dims* d) {
  if (!d) return TV_EINVAL;
  if (d->layers < 1 || d->hidden < 1 || d->Hq < 1 || d->Hkv < 1 || d->D < 1 || d->inter < 1 ||
      d->vocab < 1 || d->Hq % d->Hkv)
    return TV_EINVAL;
  if (!isfinite(d->rms_eps) || d->rms_eps < 0.f || !isfinite(d->rope_theta) ||
      d->rope_theta <= 1.f)
    return TV_EINVAL;
  if (d->D != 64 && d->D != 128) return TV_ENOTSUP;
  if (d->hidden % 256 || d->inter % 256 || (d->Hq * d->D) % 256) return TV_ENOTSUP;
  if (d->hidden > 16384) return TV_ENOTSUP;  // one row per norm workgroup
  if ((long long)d->vocab * d->hidden > (1LL << 40)) return TV_ENOTSUP;
  return TV_OK;
}

bool weights_ok(const tv_model_weights* w) {
  return w && w->embed && w->ln1 && w->w_qkv && w->q_norm && w->k_norm && w->w_o && w->ln2 &&
         w->w_gu && w->w_down && w->final_norm && w->lm_head;
}

}  // namespace

extern "C" {

size_t tv_verify_pass_workspace(const tv_model_dims* dims, int B, int N, int max_seq_len) {
  if (dims_status(dims) != TV_OK || B < 1 || N < 1 || N > TV_MAX_NODES || max_seq_len < 0 ||
      (long long)B * N > 65536)
    return 0;
  return tv::pass_plan(*dims, B, N, max_seq_len).ws_bytes;
}

int tv_verify_pass(const tv_model_dims* dims, const tv_model_weights* weights,
                   const int32_t* tokens, const int32_t* parent, const int32_t* seq_lens,
                   void* k_cache, void* v_cache, int B, int N, int Lcap, int max_seq_len,
                   int32_t* argmax, float* logits, float* hidden_out, void* workspace,
                   size_t ws_bytes, int32_t* dev_status, void* stream) {
  const int ds = dims_status(dims);
  if (ds != TV_OK) return ds;
  if (!weights_ok(weights) || !tokens || !parent || !seq_lens || !k_cache || !v_cache ||
      !argmax)
    return TV_EINVAL;
  if (B < 1 || N < 1 || max_seq_len < 0 || Lcap < 1) return TV_EINVAL;
  if ((long long)max_seq_len + N > Lcap) return TV_EINVAL;
  if (N > TV_MAX_NODES || (long long)B * N > 65536) return TV_ENOTSUP;
  if ((long long)dims->layers * B * dims->Hkv * Lcap * dims->D > (1LL << 40)) return TV_ENOTSUP;
  const tv::PassPlan plan = tv::pass_plan(*dims, B, N, max_seq_len);
  if ((long long)B * dims->Hkv * plan.attn.nqblk * plan.attn.nsplit > 2147483647LL)
    return TV_ENOTSUP;
  if (!workspace || ws_bytes < plan.ws_bytes) return TV_EWORKSPACE;
  return hip_status(tv::launch_verify_pass(*dims, *weights, plan, tokens, parent, seq_lens,
                                           k_cache, v_cache, B, N, Lcap, max_seq_len, argmax,
                                           logits, hidden_out, workspace, dev_status,
                                           static_cast<hipStream_t>(stream)));
}

size_t tv_kv_compact_layers_workspace(int B) {
  return B < 1 ? 0 : ((size_t)B * 4 + 255) / 256 * 256;
}

int tv_kv_compact_layers(void* k_cache, void* v_cache, int32_t* seq_lens, const int32_t* path,
                         const int32_t* path_len, int B, int Hkv, int D, int Lcap, int P,
                         int layers, int dtype, void* workspace, size_t ws_bytes, void* stream) {
  if (!k_cache || !v_cache || !seq_lens || !path || !path_len) return TV_EINVAL;
  if (B < 1 || Hkv < 1 || D < 1 || Lcap < 1 || P < 1 || layers < 1) return TV_EINVAL;
  if (!dtype_ok(dtype)) return TV_ENOTSUP;
  const int esz = dtype == TV_F32 ? 4 : 2;
  if ((D * esz) % 16 || P > 64 || (long long)P * D * esz > 65536) return TV_ENOTSUP;
  // planes (layer, K|V, head) are indexed in 32 bits with quotients by 2 * Hkv
  if (B > 65535 || (long long)layers * 4 * Hkv * Hkv >= 4294967296LL) return TV_ENOTSUP;
  if (!workspace || ws_bytes < tv_kv_compact_layers_workspace(B)) return TV_EWORKSPACE;
  return hip_status(tv::launch_kv_compact_layers(k_cache, v_cache, seq_lens, path, path_len, B,
                                                 Hkv, D, Lcap, P, layers, dtype,
                                                 static_cast<unsigned*>(workspace),
                                                 static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- graphs

struct tv_graph {
  hipGraphExec_t exec;
};

int tv_graph_begin(void* stream) {
  if (!stream) return TV_EINVAL;  // the null stream cannot be captured
  return hip_status(
      hipStreamBeginCapture(static_cast<hipStream_t>(stream), hipStreamCaptureModeThreadLocal));
}

int tv_graph_end(void* stream, tv_graph** graph) {
  if (!stream || !graph) return TV_EINVAL;
  *graph = nullptr;
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(static_cast<hipStream_t>(stream), &g);
  if (e != hipSuccess) return hip_status(e);
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
  hipGraphDestroy(g);
  if (e != hipSuccess) return hip_status(e);
  *graph = new tv_graph{exec};
  return TV_OK;
}

int tv_graph_launch(const tv_graph* graph, void* stream) {
  if (!graph) return TV_EINVAL;
  return hip_status(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)));
}

int tv_graph_destroy(tv_graph* graph) {
  if (!graph) return TV_EINVAL;
  const hipError_t e = hipGraphExecDestroy(graph->exec);
  delete graph;
  return hip_status(e);
}

}  // extern "C"

// ---------------------------------------------------------------- tree construction

extern "C" {

size_t tv_tree_build_workspace(int B, int depth, int V, int width) {
  if (B < 1 || depth < 1 || V < 1 || width < 1) return 0;
  return tv::tree_build_ws_bytes(B, depth, V, width);
}

int tv_tree_build(const float* draft_logp, const int32_t* root_tokens, int B, int depth, int V,
                  int width, int budget, int32_t* parent, int32_t* tokens, int32_t* node_depth,
                  float* score, void* workspace, size_t ws_bytes, void* stream) {
  if (!draft_logp || !root_tokens || !parent || !tokens) return TV_EINVAL;
  if (B < 1 || depth < 1 || V < 1 || width < 1 || budget < 1 || V < width) return TV_EINVAL;
  if (width > 16 || depth > 64 || budget + 1 > TV_MAX_NODES || B > 65535) return TV_ENOTSUP;
  if ((long long)width + (long long)(depth - 1) * width * width > 4096) return TV_ENOTSUP;
  if (budget > tv::tree_build_pool(depth, width)) return TV_EINVAL;
  if ((long long)B * depth * V > (1LL << 40)) return TV_ENOTSUP;
  if (!workspace || ws_bytes < tv::tree_build_ws_bytes(B, depth, V, width)) return TV_EWORKSPACE;
  return hip_status(tv::launch_tree_build(draft_logp, root_tokens, B, depth, V, width, budget,
                                          parent, tokens, node_depth, score, workspace,
                                          static_cast<hipStream_t>(stream)));
}


size_t tv_tree_build_level_workspace(int B, int depth, int V, int width) {
  if (B < 1 || depth < 1 || V < 1 || width < 1 || width > 16) return 0;
  return tv::tree_level_ws_bytes(B, depth, V, width);
}

static int tree_level_shape_ok(int B, int depth, int V, int width) {
  if (B < 1 || depth < 1 || V < 1 || width < 1 || V < width) return TV_EINVAL;
  if (width > 16 || depth > 64 || B > 65535) return TV_ENOTSUP;
  if ((long long)width + (long long)(depth - 1) * width * width > 4096) return TV_ENOTSUP;
  if ((long long)B * width * V > (1LL << 40)) return TV_ENOTSUP;
  return TV_OK;
}

int tv_tree_build_level(const float* draft_logp, int level, int B, int depth, int V, int width,
                        int32_t* frontier_src, int32_t* frontier_tok, void* workspace,
                        size_t ws_bytes, void* stream) {
  if (!draft_logp || !frontier_src || !frontier_tok) return TV_EINVAL;
  const int st = tree_level_shape_ok(B, depth, V, width);
  if (st != TV_OK) return st;
  if (level < 1 || level > depth) return TV_EINVAL;
  if (!workspace || ws_bytes < tv::tree_level_ws_bytes(B, depth, V, width)) return TV_EWORKSPACE;
  return hip_status(tv::launch_tree_level(draft_logp, level, B, depth, V, width, frontier_src,
                                          frontier_tok, workspace,
                                          static_cast<hipStream_t>(stream)));
}

int tv_tree_build_finish(const int32_t* root_tokens, int B, int depth, int V, int width,
                         int budget, int32_t* parent, int32_t* tokens, int32_t* node_depth,
                         float* score, void* workspace, size_t ws_bytes, void* stream) {
  if (!root_tokens || !parent || !tokens) return TV_EINVAL;
  const int st = tree_level_shape_ok(B, depth, V, width);
  if (st != TV_OK) return st;
  if (budget < 1 || budget > tv::tree_build_pool(depth, width)) return TV_EINVAL;
  if (budget + 1 > TV_MAX_NODES) return TV_ENOTSUP;
  if (!workspace || ws_bytes < tv::tree_level_ws_bytes(B, depth, V, width)) return TV_EWORKSPACE;
  return hip_status(tv::launch_tree_finish(root_tokens, B, depth, V, width, budget, parent, tokens,
                                           node_depth, score, workspace,
                                           static_cast<hipStream_t>(stream)));
}

}  // extern "C"
