// Internal declarations of the gfx950 tree-verification library.
// Nothing here is part of the public C ABI (include/treeverify.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "treeverify.h"

namespace tv {

// ---------------------------------------------------------------- bf16 bits

typedef uint16_t bf16_t;  // bf16 storage: raw bit pattern

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even, NaN kept quiet.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------- MFMA types

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// 16-byte register payload.  A native vector, not HIP's uint4 struct: arrays
// of the struct are copied with memcpy and can stay in scratch memory.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

union Frag8 {  // eight bf16 values as one MFMA operand or one 16-byte load
  uint4 u;
  u32x4_t q;
  bf16x8_t v;
};

// D = A(16x32) * B(32x16) + C on the matrix cores.  Lane l holds row/column
// l % 16 and the eight k values 8*(l/16)..8*(l/16)+7 of each operand; the
// result lane l holds column l % 16, rows 4*(l/16)..4*(l/16)+3.
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- launch helpers

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

// The dispatcher hands workgroup `bid` to die bid % 8.  Returns a logical index
// such that consecutive logical indices run on the same die (so workgroups that
// share data share that die's L2).  A bijection on [0, total).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int xcd = bid % kXcds;
  const int slot = bid / kXcds;
  const int per = total / kXcds;
  const int rem = total % kXcds;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Order-preserving map of fp32 to uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Packed (value, index) key: the maximum key is the largest value, and among
// equal values (-0 and +0 included: f + 0 is +0 for both) the smallest index.
__device__ __forceinline__ unsigned long long argmax_key(float f, uint32_t idx) {
  return ((unsigned long long)f32_order_key(f + 0.0f) << 32) | (unsigned long long)(~idx);
}

// ---------------------------------------------------------------- launchers

struct AttnPlan {
  int qbw, nw;    // 16-row query blocks per wavefront, wavefronts per workgroup
  int rows;       // query rows per workgroup (16 * qbw * nw)
  int nqblk;      // query blocks per (sequence, KV head)
  int nsplit;     // workgroups along the prefix per query block
  int chunk_len;  // prefix keys per split (multiple of 64)
  // ragged batches: splits derived on the device from the lengths
  int ragged, want_blocks, min_tiles, max_items;
  size_t ws_bytes;
};

// Largest batch whose splits are derived on the device from its lengths.
constexpr int kMaxRaggedBatch = 64;


// page_size 0 = contiguous caches
AttnPlan attn_plan(int B, int N, int Hq, int Hkv, int D, int max_seq_len, int dtype,
                   int page_size);

hipError_t launch_tree_attn(const void* q, const void* k, const void* v,
                            const int32_t* seq_lens, const int32_t* parent,
                            void* out, int B, int N, int Hq, int Hkv, int D,
                            int Lcap, int max_seq_len, float scale, int dtype,
                            const AttnPlan& plan, void* ws, int32_t* dev_status,
                            hipStream_t stream, const int32_t* block_table = nullptr,
                            int max_blocks = 0, int page_size = 0, int num_pages = 0);

size_t lmhead_ws_bytes(int M, int K, int V, int dtype);
// Host checks of tv_lmhead_argmax's arguments other than the workspace.
int lmhead_check(const void* hidden, const void* w, const int32_t* argmax, int M, int K, int V,
                 int dtype, int w_layout);
// TV_OK, or TV_EHIP with the error's text kept for tv_status_string.
int hip_status(hipError_t e);
size_t lmhead_packed_bytes(int V, int K);

hipError_t launch_lmhead_pack(const void* w, void* packed, int V, int K, hipStream_t stream);
// A gate/up weight [2 inter][K] packed with gate and up rows interleaved per
// 128-row tile (64 gate rows, then the 64 up rows of the same features).
hipError_t launch_pack_gate_up(const void* w, void* packed, int inter, int K,
                               hipStream_t stream);

// The first lmhead_zero_bytes(M) bytes of ws must be zero and are left zero.
size_t lmhead_zero_bytes(int M);
hipError_t launch_lmhead_argmax(const void* hidden, const void* w, int32_t* argmax,
                                float* logits, int M, int K, int V, int dtype, int w_layout,
                                void* ws, size_t ws_bytes, hipStream_t stream);

hipError_t launch_tree_accept(const int32_t* parent, const int32_t* draft,
                              const int32_t* tgt, int32_t* path, int32_t* path_len,
                              int32_t* bonus, int B, int N, int P,
                              int32_t* dev_status, hipStream_t stream);

hipError_t launch_kv_commit_slots(int32_t* block_table, int32_t* seq_lens, const int32_t* path,
                                  const int32_t* path_len, int B, int N, int P, int max_blocks,
                                  int32_t* dev_status, hipStream_t stream);
hipError_t launch_kv_compact(void* k, void* v, int32_t* seq_lens, const int32_t* path,
                             const int32_t* path_len, int B, int Hkv, int D,
                             int Lcap, int P, int dtype, hipStream_t stream,
                             const int32_t* block_table = nullptr, int max_blocks = 0,
                             int page_size = 0, int num_pages = 0);
hipError_t launch_accept_compact(const int32_t* parent, const int32_t* draft,
                                 const int32_t* target, int32_t* path, int32_t* path_len,
                                 int32_t* bonus, void* k, void* v, int32_t* seq_lens, int B,
                                 int N, int P, int Hkv, int D, int Lcap, int dtype,
                                 int32_t* dev_status, hipStream_t stream);

// ---------------------------------------------------------------- products with M > 64 rows

int gemm32_vtiles(int V);                  // 256-row W tiles
int gemm_argmax_vtiles(int M, int V);      // W tiles (keys per row) of the M > 64 argmax product
int gemm32_splits(int M, int K, int Nout);
hipError_t launch_gemm32_argmax(const void* hidden, const void* w_packed,
                                unsigned long long* keys, float* logits, int M, int K, int V,
                                hipStream_t stream);
hipError_t launch_gemm32_store(const void* hidden, const void* w_packed, float* part, int M,
                               int K, int Nout, int nsplit, hipStream_t stream);

// ---------------------------------------------------------------- projections

// Split count of a packed-weight projection out[M][Nout] = H[M][K] W^T.
int proj_splits(int M, int K, int Nout);
// The gate/up projection with silu(gate) * up in its epilogue (one row block
// of M <= 64 rows whose split count is 1): a[M][inter] bf16.
bool proj_swiglu_fused(int M, int K, int inter);
hipError_t launch_proj_swiglu(const void* hidden, const void* w_gu_packed, void* act, int M,
                              int K, int inter, hipStream_t stream);

// fp32 partial sums part[nsplit][M][Nout] (W packed as by launch_lmhead_pack).
hipError_t launch_proj(const void* hidden, const void* w_packed, float* part, int M, int K,
                       int Nout, int nsplit, hipStream_t stream);

// ---------------------------------------------------------------- multi-layer pass

struct PassPlan {
  int s_qkv, s_o, s_gu, s_down;  // split-K factors of the four projections
  AttnPlan attn;
  size_t off_lm, off_pos, off_x, off_gin, off_q, off_act, off_part, off_attn;  // workspace offsets
  size_t ws_bytes;
};

PassPlan pass_plan(const tv_model_dims& d, int B, int N, int max_seq_len);
size_t packed_layer_bytes(int rows, int K);

hipError_t launch_verify_pass(const tv_model_dims& d, const tv_model_weights& w,
                              const PassPlan& p, const int32_t* tokens, const int32_t* parent,
                              const int32_t* seq_lens, void* k_cache, void* v_cache, int B,
                              int N, int Lcap, int max_seq_len, int32_t* argmax, float* logits,
                              float* hidden_out, void* ws, int32_t* dev_status,
                              hipStream_t stream);

hipError_t launch_kv_compact_layers(void* k, void* v, int32_t* seq_lens, const int32_t* path,
                                    const int32_t* path_len, int B, int Hkv, int D, int Lcap,
                                    int P, int layers, int dtype, unsigned* counters,
                                    hipStream_t stream);

// ---------------------------------------------------------------- tree construction

int tree_build_pool(int depth, int width);  // candidate nodes of a tree
size_t tree_build_ws_bytes(int B, int depth, int V, int width);
size_t tree_level_ws_bytes(int B, int depth, int V, int width);
hipError_t launch_tree_level(const float* logp, int level, int B, int depth, int V, int width,
                             int32_t* frontier_src, int32_t* frontier_tok, void* ws,
                             hipStream_t stream);
hipError_t launch_tree_finish(const int32_t* root_tokens, int B, int depth, int V, int width,
                              int budget, int32_t* parent, int32_t* tokens, int32_t* node_depth,
                              float* score, void* ws, hipStream_t stream);
hipError_t launch_tree_build(const float* logp, const int32_t* root_tokens, int B, int depth,
                             int V, int width, int budget, int32_t* parent, int32_t* tokens,
                             int32_t* node_depth, float* score, void* ws, hipStream_t stream);

}  // namespace tv
