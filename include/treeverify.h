/*
 * treeverify.h - C ABI of the tree-verification step of tree speculative
 * decoding, for AMD Instinct MI355X (gfx950).
 *
 * Source of the method: JetSpec GitHub README, section "JetSpec > Overview":
 * a draft head proposes a token tree, the frozen target model verifies the
 * whole tree in one forward pass under a tree-causal attention mask, and the
 * accepted path is chosen from the target's own logits, so decoding stays
 * lossless.  The README's "Quick Start" runs at temperature 0.  The
 * EQSPEC/EXSPEC abstract (arXiv 2510.22876, on the RSS reader page) names
 * output equivalence with plain autoregressive decoding as the correctness
 * criterion and the per-sequence KV-cache state of a ragged batch.
 *
 * One step is four calls on one stream, in this order:
 *   tv_tree_verify_attn -> tv_lmhead_argmax -> tv_tree_accept -> tv_kv_compact
 *
 * Conventions shared by every call
 *   - Every array pointer is a DEVICE pointer owned by the caller; the library
 *     allocates nothing and keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls validate their arguments on the host, enqueue their kernels on
 *     `stream` and return at once; results are ready when the stream is.
 *   - Return value: TV_OK (0), or a negative TV_E* code.  On a negative
 *     return nothing was enqueued, except TV_EHIP, whose text is available
 *     from tv_status_string() of that code until the next call on the thread.
 *   - dtype: TV_BF16 (bfloat16 storage, fp32 accumulation on MFMA) or TV_F32
 *     (fp32 storage and arithmetic).
 *   - dev_status (nullable): device int32[B] that the caller zeroes; kernels
 *     OR TV_STATUS_* flags into entry b when sequence b is malformed; the
 *     outputs of such a sequence are then unspecified.
 *   - Calls that share a workspace, or that write the same cache, must not
 *     overlap in time (same stream, or ordered by events).
 *
 * Two arguments go beyond the bare problem statement, on purpose: the
 * workspace queries take `dtype` (the fp32 kernels tile differently and need
 * other scratch than the bf16 ones), and tv_lmhead_argmax takes `w_layout`
 * (the vocabulary projection is a static weight, repacked once into the
 * layout the matrix-core kernels stream fastest; the row-major layout stays
 * accepted).
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TV_OK          0
#define TV_EINVAL     -1 /* bad shape, size or null pointer                  */
#define TV_ENOTSUP    -2 /* valid but unsupported: head dim, dtype, N, ...   */
#define TV_EWORKSPACE -3 /* workspace null or smaller than the query result  */
#define TV_EHIP       -4 /* a HIP launch failed                              */
#define TV_ESCRATCH   -5 /* larger than the allocation-free call's scratch   */

/* Bytes of the device array behind tv_lmhead_argmax_noalloc (per device). */
#define TV_NOALLOC_SCRATCH_BYTES (64u << 20)

#define TV_BF16 0
#define TV_F32  1

#define TV_LAYOUT_ROWMAJOR 0 /* w is [V][K], one row per vocabulary entry     */
#define TV_LAYOUT_PACKED   1 /* w as written by tv_lmhead_pack_weights        */

#define TV_STATUS_BAD_PARENT 1 /* parent[0] != -1 or parent[i] not in [0, i) */
#define TV_STATUS_BAD_LEN    2 /* L_b < 0, L_b > max_seq_len or L_b+N > Lcap */
#define TV_STATUS_DEPTH      4 /* accepted path longer than P                */
#define TV_STATUS_BAD_PAGE   8 /* a block-table entry outside [0, num_pages) */
#define TV_STATUS_BAD_TOKEN 16 /* a draft token outside [0, vocab)           */
#define TV_STATUS_BAD_PATH  32 /* path not increasing within [0, N)          */

#define TV_MAX_NODES 1024 /* N limit of every call                           */

/*
 * Tree-causal attention (JetSpec GitHub README, "JetSpec > Overview": the
 * whole tree is verified in one pass under a tree-causal mask).
 *
 * For sequence b, node i (0 <= i < N) and query head h (KV head g = h / G,
 * G = Hq / Hkv), with L = seq_lens[b]:
 *   visible keys = cache rows 0..L-1 (the prefix) and rows L + j for every
 *                  tree node j on the root-to-i path, i included;
 *   out[b][i][h] = sum_t softmax_t(scale * q . k_t) v_t over those keys.
 * Node 0 is the last accepted token; the tree is topologically ordered:
 * parent[b][0] = -1 and 0 <= parent[b][i] < i.
 *
 * q        [B][N][Hq][D]         dtype
 * k_cache  [B][Hkv][Lcap][D]     dtype; rows L..L+N-1 hold the tree nodes'
 * v_cache  [B][Hkv][Lcap][D]     keys/values in node order (read only)
 * seq_lens [B] int32             prefix length of each sequence
 * parent   [B][N] int32
 * out      [B][N][Hq][D]         dtype (written)
 * max_seq_len   host-side upper bound of seq_lens (sizes the split of the
 *               prefix across workgroups); needs max_seq_len + N <= Lcap
 * scale         softmax scale, normally 1/sqrt(D)
 * workspace     device scratch of at least tv_tree_verify_attn_workspace()
 *               bytes for the same shapes (may be NULL when that is 0); no
 *               initial contents needed.  Long prefixes are split across
 *               workgroups; for a batch of 2..64 sequences the splits are
 *               derived on the device from seq_lens (one chunk length for
 *               the batch), so the workspace covers any lengths up to
 *               max_seq_len.
 * Supported: D in {64, 128}, 1 <= N <= TV_MAX_NODES, Hq % Hkv == 0.
 * Device-side checks: TV_STATUS_BAD_PARENT, TV_STATUS_BAD_LEN.
 */
size_t tv_tree_verify_attn_workspace(int B, int N, int Hq, int Hkv, int D,
                                     int max_seq_len, int dtype);
int tv_tree_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seq_lens, const int32_t* parent,
                        void* out, int B, int N, int Hq, int Hkv, int D,
                        int Lcap, int max_seq_len, float scale, int dtype,
                        void* workspace, size_t ws_bytes, int32_t* dev_status,
                        void* stream);

/*
 * Tree-causal attention over paged key/value caches (the engine of the
 * JetSpec GitHub README, "Quick Start", keeps its KV cache in pages).
 * Same computation as tv_tree_verify_attn; only where rows live differs:
 *
 * k_pages, v_pages  [num_pages][Hkv][page_size][D] bf16 pools (read only)
 * block_table       [B][max_blocks] int32: logical row r of sequence b is
 *                   row r % page_size of page block_table[b][r / page_size]
 *                   (prefix rows 0..L-1, then the N tree rows L..L+N-1)
 * page_size         power of two, 1..4096 (1: a slot table, one row per
 *                   page; see tv_kv_commit_slots); max_seq_len + N must fit in
 *                   max_blocks * page_size
 * workspace         at least tv_tree_verify_attn_paged_workspace() bytes
 * Device-side checks add TV_STATUS_BAD_PAGE (an entry outside the pool;
 * it is never dereferenced).  bf16 only (TV_ENOTSUP otherwise).
 */
size_t tv_tree_verify_attn_paged_workspace(int B, int N, int Hq, int Hkv, int D,
                                           int max_seq_len, int page_size, int dtype);
int tv_tree_verify_attn_paged(const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* block_table,
                              int max_blocks, int page_size, int num_pages,
                              const int32_t* seq_lens, const int32_t* parent,
                              void* out, int B, int N, int Hq, int Hkv, int D,
                              int max_seq_len, float scale, int dtype,
                              void* workspace, size_t ws_bytes,
                              int32_t* dev_status, void* stream);

/*
 * Target LM head fused with a per-row argmax (the accepted path follows the
 * target's own logits; temperature 0 makes that the argmax).
 *
 *   logits[r][v] = sum_k hidden[r][k] * w[v][k]   (fp32 accumulation)
 *   argmax[r]    = smallest v attaining max_v logits[r][v]
 *
 * hidden  [M][K] dtype, row r = b*N + i for node i of sequence b
 * w       the vocabulary projection in layout `w_layout`:
 *         TV_LAYOUT_ROWMAJOR: [V][K] dtype, one row per vocabulary entry;
 *         TV_LAYOUT_PACKED:   the buffer written by tv_lmhead_pack_weights
 *                             (bf16 only), the faster form for a weight that
 *                             is reused across steps
 * argmax  [M] int32 (written)
 * logits  [M][V] fp32 or NULL; written only when non-NULL (for checking:
 *         the step itself never materialises the logits)
 * workspace  at least tv_lmhead_argmax_workspace() bytes.  It must be
 *         zero-filled before its first use; every call leaves its first
 *         8*M (rounded up to 256) + 256 bytes zero-filled again when it
 *         completes.  When M > 64 a call also uses scratch at the end of the
 *         buffer (ws_bytes counts), never inside the zero region of any M the
 *         buffer was sized for; so one buffer serves any number of calls in
 *         stream order, of any M up to the size it was queried for (calls
 *         sharing it must not overlap).
 * Supported: bf16 needs K % 256 == 0; M >= 1, V >= 1.
 */
size_t tv_lmhead_argmax_workspace(int M, int K, int V, int dtype);
int tv_lmhead_argmax(const void* hidden, const void* w, int32_t* argmax,
                     float* logits, int M, int K, int V, int dtype,
                     int w_layout, void* workspace, size_t ws_bytes,
                     void* stream);

/*
 * tv_lmhead_argmax without a workspace, for callers that cannot allocate
 * device memory: code under stream capture, tight serving loops, harnesses
 * that forbid allocation.  Arguments, results and checks as for
 * tv_lmhead_argmax; the same kernels run.  Their scratch is one device array
 * of TV_NOALLOC_SCRATCH_BYTES per device, held from first use until the
 * process ends: a shape whose tv_lmhead_argmax_workspace() exceeds it
 * returns TV_ESCRATCH with nothing enqueued (64 MiB covers 4096 rows at
 * V = 151936, K = 2048).  The call allocates nothing.  Each call clears the
 * part that must start at zero, on `stream`, before its kernels; every call
 * on a device shares that device's array, so calls that may overlap on one
 * device (other streams, other threads) race and must be ordered by the
 * caller.
 */
int tv_lmhead_argmax_noalloc(const void* hidden, const void* w, int32_t* argmax,
                             float* logits, int M, int K, int V, int dtype, int w_layout,
                             void* stream);

/*
 * Repack a row-major bf16 vocabulary projection [V][K] into the layout the
 * LM-head kernel streams fastest: for every tile of 128 rows and every
 * 128-wide k chunk, the 32 KB the kernel reads are stored contiguously in
 * the order its lanes consume them (rows past V are zero).  Done once per
 * weight; `w_packed` (device, tv_lmhead_packed_bytes() bytes, caller-owned)
 * must not overlap `w`.  Returns TV_ENOTSUP unless dtype is TV_BF16 and
 * K % 256 == 0 (tv_lmhead_packed_bytes then returns 0).
 */
size_t tv_lmhead_packed_bytes(int V, int K, int dtype);
int tv_lmhead_pack_weights(const void* w, void* w_packed, int V, int K,
                           int dtype, void* stream);

/*
 * Pack a gate/up weight of the multi-layer pass's MLP (the SwiGLU of the
 * Qwen3 targets named in the JetSpec abstract): w is [2 inter][K] bf16
 * row-major, the inter gate rows, then the inter up rows.  The result has
 * the tv_lmhead_pack_weights layout of a [2 inter][K] weight whose rows are
 * interleaved per 128-row tile: packed rows 128 t .. 128 t + 63 are gate
 * rows 64 t .. 64 t + 63 and packed rows 128 t + 64 .. 128 t + 127 the up
 * rows of the same features, so one workgroup holds both halves of the
 * features it produces.  w_packed: tv_lmhead_packed_bytes(2 inter, K, dtype)
 * bytes, caller-owned, not overlapping w.  Returns TV_ENOTSUP unless dtype is
 * TV_BF16, K % 256 == 0 and inter % 64 == 0.
 */
int tv_pack_gate_up_weights(const void* w, void* w_packed, int inter, int K,
                            int dtype, void* stream);

/*
 * Greedy longest-accepted-path selection plus the bonus token (JetSpec GitHub
 * README, "JetSpec > Overview": lossless by construction).
 *
 * Node i >= 1 is accepted when its parent is accepted and
 * draft_tokens[b][i] == target_tokens[b][parent[i]]; the root is always
 * accepted.  best = deepest accepted node, smallest index on ties.
 *   path[b][0..path_len-1] = root .. best (node indices), rest = -1
 *   path_len[b]            = depth(best) + 1
 *   bonus[b]               = target_tokens[b][best]
 * Emitting draft_tokens[path[1..]] followed by bonus equals what greedy
 * decoding with the same target tokens would emit.
 *
 * parent, draft_tokens, target_tokens  [B][N] int32
 * path [B][P] int32, path_len [B] int32, bonus [B] int32 (written)
 * Device-side checks: TV_STATUS_BAD_PARENT, TV_STATUS_DEPTH; a flagged
 * sequence gets path_len 0, bonus -1 and path all -1.
 * Supported: 1 <= N <= TV_MAX_NODES, 1 <= P <= 64.
 */
int tv_tree_accept(const int32_t* parent, const int32_t* draft_tokens,
                   const int32_t* target_tokens, int32_t* path,
                   int32_t* path_len, int32_t* bonus, int B, int N, int P,
                   int32_t* dev_status, void* stream);

/*
 * KV compaction: commit the accepted path into contiguous cache rows
 * (EQSPEC/EXSPEC abstract: each sequence of a ragged batch keeps its own KV
 * state).  For every b, KV head and j < path_len[b]:
 *   row L_b + j  <-  row L_b + path[b][j]     (in k_cache and v_cache)
 * then seq_lens[b] += path_len[b].  Rows are moved as stored bits; the moves
 * of one (b, head) are staged before any is written, so the in-place update
 * is exact.  Rows past the new length keep unspecified contents.
 *
 * k_cache, v_cache [B][Hkv][Lcap][D] dtype (updated in place)
 * seq_lens [B] int32 (updated in place); path [B][P], path_len [B] int32
 * The caller guarantees L_b + path_len[b] <= Lcap and path entries in
 * [0, Lcap - L_b); rows are not read past that.
 * Supported: D * sizeof(dtype) % 16 == 0, P <= 64.
 */
int tv_kv_compact(void* k_cache, void* v_cache, int32_t* seq_lens,
                  const int32_t* path, const int32_t* path_len, int B, int Hkv,
                  int D, int Lcap, int P, int dtype, void* stream);

/*
 * Acceptance and compaction in one launch: exactly tv_tree_accept followed
 * by tv_kv_compact on the same arguments (the same outputs, bit for bit),
 * for the end of a verification step (JetSpec GitHub README, "JetSpec >
 * Overview": the accepted path follows the target's own logits; EQSPEC/EXSPEC
 * abstract, arXiv 2510.22876 on the RSS reader page: each sequence's KV state
 * stays in step).  Arguments as for those two calls: parent, draft_tokens,
 * target_tokens [B][N] int32; path [B][P], path_len [B], bonus [B] int32
 * (written); k_cache, v_cache [B][Hkv][Lcap][D] dtype and seq_lens [B]
 * (updated in place, seq_lens[b] += path_len[b]).  A sequence whose tree is
 * malformed or whose path is longer than P gets path_len 0 and a status flag,
 * and its cache and length are left as they are.
 * Supported: N <= TV_MAX_NODES, P <= 64, D * sizeof(dtype) % 16 == 0.
 */
int tv_accept_compact(const int32_t* parent, const int32_t* draft_tokens,
                      const int32_t* target_tokens, int32_t* path,
                      int32_t* path_len, int32_t* bonus, void* k_cache,
                      void* v_cache, int32_t* seq_lens, int B, int N, int P,
                      int Hkv, int D, int Lcap, int dtype, int32_t* dev_status,
                      void* stream);

/*
 * KV compaction on paged caches (layout as for tv_tree_verify_attn_paged):
 * the same row moves as tv_kv_compact, through the block table; a move
 * whose page entry is outside the pool is skipped.  bf16 or fp32 pools,
 * updated in place, with seq_lens[b] += path_len[b].  The caller guarantees
 * L_b + path_len[b] <= max_blocks * page_size (else sequence b is left
 * untouched) and that the pages holding rows L_b .. L_b+P-1 of a sequence
 * belong to that sequence alone (pages of a shared prefix may be shared;
 * tree rows may not).
 */
int tv_kv_compact_paged(void* k_pages, void* v_pages, const int32_t* block_table,
                        int max_blocks, int page_size, int num_pages,
                        int32_t* seq_lens, const int32_t* path,
                        const int32_t* path_len, int B, int Hkv, int D, int P,
                        int dtype, void* stream);

/*
 * Commit of the accepted path on a slot table: a block table whose pages
 * hold one row each (page_size 1 in tv_tree_verify_attn_paged and
 * tv_kv_compact_paged).  The serving engine keeps its KV cache in pages
 * (JetSpec GitHub README, "Quick Start"); with one row per page the commit
 * moves table entries instead of K/V rows, so no cache row is read or
 * written.  Per sequence b, the window block_table[b][L_b .. L_b+N-1] (the
 * tree rows) is permuted: position L_b + j takes the slot of node path[j]
 * for j < path_len[b], and the slots of the rejected nodes follow in node
 * order at L_b + path_len[b] .. L_b + N - 1, free for the next tree (whose N
 * rows need path_len[b] more slots, appended by the caller).  Then
 * seq_lens[b] += path_len[b].
 *
 * block_table [B][max_blocks] int32, updated in place; seq_lens [B] int32,
 *             updated in place; path [B][P] int32 and path_len [B] int32 as
 *             written by tv_tree_accept (path_len clamped to [0, min(P, N)]).
 * Device-side checks (dev_status nullable): TV_STATUS_BAD_LEN (L_b < 0 or
 * L_b + N > max_blocks), TV_STATUS_BAD_PATH (an entry outside [0, N) or not
 * increasing); a flagged sequence is left unchanged.  Supported: 1 <= N <=
 * TV_MAX_NODES, 1 <= P <= 64.
 */
int tv_kv_commit_slots(int32_t* block_table, int32_t* seq_lens, const int32_t* path,
                       const int32_t* path_len, int B, int N, int P, int max_blocks,
                       int32_t* dev_status, void* stream);

/*
 * Multi-layer verification pass: the target model run over every node of
 * the draft trees in one pass, ending in the LM-head argmax (JetSpec GitHub
 * README, "JetSpec > Overview": one forward pass of the target under the
 * tree-causal mask; its "Quick Start" compiles that verification and
 * replays it as a graph; the JetSpec abstract names dense and MoE Qwen3
 * targets).  The model is a dense Qwen3-style decoder stack (pre-norm
 * RMSNorm, grouped-query attention with per-head RMSNorm of queries and keys
 * before rotary embedding, SwiGLU MLP).  Node i of sequence b is token
 * tokens[b][i] at position L_b + depth(i); its key and value rows go to row
 * L_b + i of every layer's cache, and it attends as in tv_tree_verify_attn.
 *
 * dims     host struct: layers, hidden, Hq, Hkv, D, inter (MLP width),
 *          vocab, rms_eps, rope_theta (rotary pairs (d, d + D/2) turned by
 *          pos * rope_theta^(-2d/D))
 * weights  host struct of device pointers, all bf16:
 *            embed      [vocab][hidden] row-major
 *            ln1, ln2   [layers][hidden]
 *            q_norm, k_norm [layers][D]
 *            w_qkv      layers x packed([(Hq + 2 Hkv) D] rows, K = hidden):
 *                       q rows (head-major), then k rows, then v rows
 *            w_o        layers x packed([hidden] rows, K = Hq D)
 *            w_gu       layers x packed_gu([2 inter] rows, K = hidden): the
 *                       tv_pack_gate_up_weights layout (gate and up rows
 *                       interleaved per 128-row tile)
 *            w_down     layers x packed([hidden] rows, K = inter)
 *            final_norm [hidden]
 *            lm_head    packed([vocab] rows, K = hidden)
 *          "packed(r, K)" is the tv_lmhead_pack_weights layout of an [r][K]
 *          row-major weight, tv_lmhead_packed_bytes(r, K, TV_BF16) bytes
 *          (packed_gu the same size); the layers' blocks follow each other
 *          without gaps.
 * tokens, parent  [B][N] int32; seq_lens [B] (read only: the caller runs
 *          tv_tree_accept and tv_kv_compact_layers afterwards)
 * k_cache, v_cache  [layers][B][Hkv][Lcap][D] bf16: prefix rows read, tree
 *          rows L_b .. L_b+N-1 written
 * argmax   [B*N] int32, row b*N + i
 * logits   [B*N][vocab] fp32 or NULL (for checking; not on the hot path)
 * hidden_out [B*N][hidden] fp32 or NULL: the final normalised hidden states
 * workspace  tv_verify_pass_workspace() bytes of scratch (no initial
 *          contents needed; one buffer serves passes of any shape up to the
 *          size it was queried for, in stream order).  Nothing is allocated
 *          or memset: the pass may be captured with tv_graph_begin/end.
 * Supported: D in {64, 128}; hidden, inter and Hq*D multiples of 256;
 *          hidden <= 16384; 1 <= N <= TV_MAX_NODES.  Device-side checks: TV_STATUS_BAD_PARENT,
 *          TV_STATUS_BAD_LEN, TV_STATUS_BAD_TOKEN (the token is read as 0).
 */
typedef struct {
  int layers, hidden, Hq, Hkv, D, inter, vocab;
  float rms_eps, rope_theta;
} tv_model_dims;

typedef struct {
  const void* embed;
  const void* ln1;
  const void* w_qkv;
  const void* q_norm;
  const void* k_norm;
  const void* w_o;
  const void* ln2;
  const void* w_gu;
  const void* w_down;
  const void* final_norm;
  const void* lm_head;
} tv_model_weights;

size_t tv_verify_pass_workspace(const tv_model_dims* dims, int B, int N, int max_seq_len);
int tv_verify_pass(const tv_model_dims* dims, const tv_model_weights* weights,
                   const int32_t* tokens, const int32_t* parent,
                   const int32_t* seq_lens, void* k_cache, void* v_cache, int B,
                   int N, int Lcap, int max_seq_len, int32_t* argmax,
                   float* logits, float* hidden_out, void* workspace,
                   size_t ws_bytes, int32_t* dev_status, void* stream);

/*
 * KV compaction of every layer in one launch: the row moves of
 * tv_kv_compact applied to caches [layers][B][Hkv][Lcap][D], then
 * seq_lens[b] += path_len[b] once.  The workgroups of a sequence share its
 * planes; the last of them to finish updates the length through a counter in
 * `workspace` (tv_kv_compact_layers_workspace() bytes, zero-filled before
 * its first use and left zero by every call).
 * Supported: as tv_kv_compact, with B <= 65535 and
 * layers * (2 * Hkv)^2 < 2^32.
 */
size_t tv_kv_compact_layers_workspace(int B);
int tv_kv_compact_layers(void* k_cache, void* v_cache, int32_t* seq_lens,
                         const int32_t* path, const int32_t* path_len, int B,
                         int Hkv, int D, int Lcap, int P, int layers, int dtype,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * Graph capture of a sequence of calls (the README's "Quick Start" engine
 * replays verification as a graph).  tv_graph_begin starts capturing the
 * work later enqueued on `stream` (a stream created by the caller, not the
 * null stream); tv_graph_end stops, instantiates the captured work and
 * returns it in *graph (owned by the caller, freed with tv_graph_destroy).
 * tv_graph_launch replays it on a stream: the same kernels with the same
 * pointers, reading whatever the buffers hold at that time.  Between begin
 * and end the thread must not allocate or synchronise device memory.
 */
typedef struct tv_graph tv_graph;
int tv_graph_begin(void* stream);
int tv_graph_end(void* stream, tv_graph** graph);
int tv_graph_launch(const tv_graph* graph, void* stream);
int tv_graph_destroy(tv_graph* graph);

/*
 * Draft-tree construction by cumulative log-probability: the accum_logp
 * algorithm of the JetSpec README ("Evaluation": breadth-first
 * cumulative-log-probability tree, the default), shaped by depth, width and
 * budget as in its "Quick Start".  Reading of the steps:
 *   - candidates of depth d (1..depth): the `width` largest entries of
 *     draft_logp[b][d-1][:], ties to the smaller token id;
 *   - breadth first from the root (score 0): each node of the level-(d-1)
 *     frontier gets one child per candidate of depth d, score = parent score
 *     + logp (summed in fp64), generated in (frontier rank, token rank)
 *     order; the level-d frontier is the `width` best children (score
 *     descending, then generation order); every child is a candidate;
 *   - the tree: the root plus the `budget` best candidates (score
 *     descending, then shallower, then generation order), numbered by depth
 *     and generation, so parent[i] < i.
 *
 * This one-launch form serves a draft head whose row depends only on the
 * depth (every branch gets the same candidates); tv_tree_build_level below
 * takes one row per frontier node (branch-conditioned).
 * draft_logp   [B][depth][V] fp32 normalised log-probabilities of the draft
 *              head (no NaN)
 * root_tokens  [B] int32: token of node 0 (the last accepted token)
 * parent, tokens [B][budget+1] int32 (written): the trees, in the layout the
 *              verification calls read
 * node_depth   [B][budget+1] int32 or NULL; score [B][budget+1] fp32 or
 *              NULL (cumulative log-probability, rounded from fp64)
 * workspace    tv_tree_build_workspace() bytes (scratch)
 * Supported: width <= 16, depth <= 64, width + (depth-1)*width^2 <= 4096
 * candidates, budget + 1 <= TV_MAX_NODES, V >= width, budget <= candidates.
 */
size_t tv_tree_build_workspace(int B, int depth, int V, int width);
int tv_tree_build(const float* draft_logp, const int32_t* root_tokens, int B,
                  int depth, int V, int width, int budget, int32_t* parent,
                  int32_t* tokens, int32_t* node_depth, float* score,
                  void* workspace, size_t ws_bytes, void* stream);

/*
 * Branch-conditioned tree construction, one level per call.  The JetSpec
 * abstract describes the draft head as causal and parallel: it conditions
 * every branch on its own path ("branch-wise causal conditioning"), so that
 * the tree's scores follow the target's autoregressive factorisation.  The
 * candidates below a frontier node therefore come from that node's own
 * row.  The algorithm is the accum_logp reading above with one change: the
 * candidates of a child of frontier node r at level d are the `width`
 * largest entries of row r of that level's call, and the child's score is
 * its parent's score + that row's log-probability of its token.
 *
 * Call order, on one stream (or otherwise ordered), with one workspace:
 * tv_tree_build_level for level = 1, 2, ..., depth, then
 * tv_tree_build_finish.  Between two level calls the caller runs its draft
 * head on the paths the previous call reported.
 *
 * tv_tree_build_level:
 *   draft_logp     [B][width][V] fp32 normalised log-probabilities (no NaN);
 *                  row r of sequence b is the draft head's distribution of
 *                  the token after the root path of frontier node r (rank
 *                  order of the previous call's frontier).  Level 1 reads
 *                  row 0 only (the root's row).
 *   level          1..depth
 *   frontier_src   [B][width] int32 (written): for each rank r' of the new
 *                  frontier (best first), the rank of its parent in the
 *                  previous frontier (0 at level 1, whose parent is the root)
 *   frontier_tok   [B][width] int32 (written): the token of that node
 *   So the path of new frontier node r' is the path of previous node
 *   frontier_src[b][r'] followed by frontier_tok[b][r'].
 * tv_tree_build_finish:
 *   root_tokens, parent, tokens, node_depth, score as for tv_tree_build; the
 *   root plus the `budget` best candidates of every level's pool.
 * workspace        tv_tree_build_level_workspace() bytes; it carries the
 *                  candidate pool and the frontier from call to call (no
 *                  initial contents needed: level 1 starts a new tree).
 * Supported: as tv_tree_build.  Rejected calls (TV_EINVAL, TV_ENOTSUP,
 * TV_EWORKSPACE) enqueue nothing and leave the workspace's tree unchanged.
 */
size_t tv_tree_build_level_workspace(int B, int depth, int V, int width);
int tv_tree_build_level(const float* draft_logp, int level, int B, int depth, int V,
                        int width, int32_t* frontier_src, int32_t* frontier_tok,
                        void* workspace, size_t ws_bytes, void* stream);
int tv_tree_build_finish(const int32_t* root_tokens, int B, int depth, int V, int width,
                         int budget, int32_t* parent, int32_t* tokens, int32_t* node_depth,
                         float* score, void* workspace, size_t ws_bytes, void* stream);

/* Text of a status code (TV_EHIP: the HIP error text of the failed launch). */
const char* tv_status_string(int status);

/* Version of this ABI: major * 10000 + minor * 100 + patch. */
int tv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TREEVERIFY_H */
