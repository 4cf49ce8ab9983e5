"""fp64 oracle of a multi-layer verification pass.  TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module (see the package docstring).

The target model verifies the whole draft tree in one forward pass under a
tree-causal mask (JetSpec GitHub README, "JetSpec > Overview"); the pages'
targets are dense and MoE Qwen3 models (JetSpec abstract, catalyzex author
page).  The layer below is the standard dense Qwen3 decoder layer, written
from its public definition (pre-norm RMSNorm, grouped-query attention with a
per-head RMSNorm of queries and keys before rotary embedding, SwiGLU MLP):

    h = rmsnorm(x) * ln1
    q, k, v = h Wq^T, h Wk^T, h Wv^T                (split by heads)
    q = rope(rmsnorm(q) * q_norm, pos),  k = rope(rmsnorm(k) * k_norm, pos)
    k, v -> the layer's cache at row L_b + i        (node i of sequence b)
    x = x + tree_attention(q, cache) Wo^T
    h = rmsnorm(x) * ln2
    x = x + (silu(h Wg^T) * (h Wu^T)) Wd^T

Tree node i sits at position L_b + depth(i): it continues the prefix along
its own root path (a reading; the pages do not state positions).  Rotary
embedding pairs element d with element d + D/2 ("rotate half") and turns the
pair by the angle pos * theta^(-2d/D).

Weights are the bf16 values of the synthetic model, decoded exactly; every
step is computed in fp64 with matmul as the only library primitive.
Weight layout (rows are output features, as in a linear layer):
  embed [V][hidden], w_qkv [layers][(Hq + 2 Hkv) D][hidden] (q, then k, then
  v rows), w_o [layers][hidden][Hq D], w_gu [layers][2 I][hidden] (gate rows,
  then up rows), w_down [layers][hidden][I], ln1/ln2 [layers][hidden],
  q_norm/k_norm [layers][D], final_norm [hidden], lm_head [V][hidden].
"""
from __future__ import annotations

import numpy as np

from .verify import ancestors, decode, kv_compact, round_bf16, tree_attention


def rms_norm(x, w, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotary embedding of the last axis (length D) at positions ``pos``
    (broadcast against x's leading axes): element d and d + D/2 form a pair
    turned by the angle pos * theta^(-2d/D)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    inv = theta ** (-2.0 * np.arange(half) / D)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def node_positions(parent, seq_lens) -> np.ndarray:
    """pos[b][i] = L_b + depth(i), depth(i) = number of proper ancestors."""
    parent = np.asarray(parent)
    B, N = parent.shape
    pos = np.empty((B, N), dtype=np.int64)
    for b in range(B):
        for i in range(N):
            pos[b, i] = int(seq_lens[b]) + len(ancestors(parent[b], i)) - 1
    return pos


def verify_pass(dims: dict, weights: dict, tokens, parent, seq_lens, k_cache, v_cache,
                logit_rows=None, v_chunk: int = 8192, bf16_points: bool = False) -> dict:
    """The multi-layer pass over one draft tree per sequence.

    dims: layers, hidden, Hq, Hkv, D, inter, V, eps, theta.
    weights: bf16 bit patterns (uint16) in the layout of the module docstring.
    tokens, parent [B][N]; seq_lens [B]; k_cache, v_cache
    [layers][B][Hkv][Lcap][D] with the prefix rows filled: bf16 bit patterns,
    or fp64 values (as returned by an earlier pass).
    Returns the final normalised hidden states [B*N][hidden], the argmax and
    top-2 gap of every row, the logits of ``logit_rows`` (all rows if None),
    and fp64 copies of the caches with the tree rows written.

    bf16_points=True is not the definition but a model of a pipeline that
    stores its activations in bf16: every normalised input of a product (h
    after each norm), q, the k and v rows written to the caches, the
    attention output, the MLP activation silu(g) * u, the probabilities that
    multiply V, and the LM head's input are rounded to bf16 where they are
    produced; the residual stream, all sums and the returned (fp32-stored)
    final hidden states stay exact.  The distance between the two modes
    sizes the tolerance of a bf16 implementation.
    """
    Ly, Hd = dims["layers"], dims["hidden"]
    Hq, Hkv, D, I = dims["Hq"], dims["Hkv"], dims["D"], dims["inter"]
    eps, theta = dims["eps"], dims["theta"]
    tokens = np.asarray(tokens)
    B, N = tokens.shape
    M = B * N
    pos = node_positions(parent, seq_lens)                      # [B][N]
    cdt = "bf16" if np.asarray(k_cache).dtype == np.uint16 else "f64"
    Kc = decode(k_cache, cdt)
    Vc = decode(v_cache, cdt)
    emb = np.asarray(weights["embed"])
    x = decode(emb[tokens.reshape(-1)], "bf16")                 # [M][hidden]
    scale = 1.0 / np.sqrt(D)
    rnd = round_bf16 if bf16_points else (lambda t: t)
    for ly in range(Ly):
        h = rnd(rms_norm(x, decode(weights["ln1"][ly], "bf16"), eps))
        qkv = h @ decode(weights["w_qkv"][ly], "bf16").T         # [M][(Hq+2Hkv)D]
        q = qkv[:, :Hq * D].reshape(B, N, Hq, D)
        k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(B, N, Hkv, D)
        v = qkv[:, (Hq + Hkv) * D:].reshape(B, N, Hkv, D)
        q = rnd(rope(rms_norm(q, decode(weights["q_norm"][ly], "bf16"), eps), pos[:, :, None], theta))
        k = rnd(rope(rms_norm(k, decode(weights["k_norm"][ly], "bf16"), eps), pos[:, :, None], theta))
        v = rnd(v)
        for b in range(B):
            L = int(seq_lens[b])
            Kc[ly, b, :, L:L + N] = k[b].transpose(1, 0, 2)
            Vc[ly, b, :, L:L + N] = v[b].transpose(1, 0, 2)
        o = rnd(tree_attention(q, Kc[ly], Vc[ly], seq_lens, parent, scale, "f64",
                               p_round=round_bf16 if bf16_points else None))
        x = x + o.reshape(M, Hq * D) @ decode(weights["w_o"][ly], "bf16").T
        h = rnd(rms_norm(x, decode(weights["ln2"][ly], "bf16"), eps))
        gu = h @ decode(weights["w_gu"][ly], "bf16").T           # [M][2I]
        x = x + rnd(silu(gu[:, :I]) * gu[:, I:]) @ decode(weights["w_down"][ly], "bf16").T
    hf = rms_norm(x, decode(weights["final_norm"], "bf16"), eps)
    hl = rnd(hf)                                                # the LM head's input
    V = dims["V"]
    lm = np.asarray(weights["lm_head"])
    top1 = np.full(M, -np.inf)
    top2 = np.full(M, -np.inf)
    arg = np.zeros(M, dtype=np.int64)
    rows = np.arange(M) if logit_rows is None else np.asarray(logit_rows, dtype=np.int64)
    logits = np.empty((len(rows), V))
    for v0 in range(0, V, v_chunk):
        lg = hl @ decode(lm[v0:v0 + v_chunk], "bf16").T          # [M][chunk]
        logits[:, v0:v0 + lg.shape[1]] = lg[rows]
        # merge this chunk's two largest values into the running top-2
        part = np.sort(np.partition(lg, -2, axis=1)[:, -2:] if lg.shape[1] > 1
                       else np.concatenate([lg, np.full_like(lg, -np.inf)], axis=1), axis=1)
        a = v0 + np.argmax(lg, axis=1)
        c1, c2 = part[:, 1], part[:, 0]
        new_top = c1 > top1
        top2 = np.where(new_top, np.maximum(top1, c2), np.maximum(top2, c1))
        arg = np.where(new_top, a, arg)
        top1 = np.where(new_top, c1, top1)
    return dict(hidden=hf, argmax=arg, top1=top1, gap=top1 - top2, logits=logits,
                logit_rows=rows, k_cache=Kc, v_cache=Vc, pos=pos)


def kv_compact_layers(k_cache, v_cache, seq_lens, path, path_len):
    """kv_compact applied to every layer's cache with the same lengths, then
    one length update (caches [layers][B][Hkv][Lcap][D])."""
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    lens = None
    for ly in range(k.shape[0]):
        k[ly], v[ly], lens = kv_compact(k[ly], v[ly], seq_lens, path, path_len)
    return k, v, lens


def ar_decode(dims: dict, weights: dict, k_cache, v_cache, seq_lens, root_tokens,
              n_tokens: int) -> dict:
    """Independent greedy decoding of every sequence, one token per pass.

    Sequence b starts from its cached prefix (rows 0..L_b-1) and the token
    root_tokens[b], whose key/value row is not cached yet (node 0 of a
    verification tree).  Each step runs a one-node pass at the current
    length, appends that token's rows and emits the argmax.  Returns the
    emitted tokens [B][n_tokens], the top-2 gap of each choice, and the
    caches after the last step (fp64).
    """
    B = len(seq_lens)
    toks = np.asarray(root_tokens, dtype=np.int64).reshape(B, 1)
    lens = np.asarray(seq_lens, dtype=np.int64).copy()
    kc, vc = k_cache, v_cache
    out = np.empty((B, n_tokens), dtype=np.int64)
    gap = np.empty((B, n_tokens))
    for t in range(n_tokens):
        r = verify_pass(dims, weights, toks, np.full((B, 1), -1), lens, kc, vc, logit_rows=[])
        out[:, t] = r["argmax"]
        gap[:, t] = r["gap"]
        kc, vc = r["k_cache"], r["v_cache"]
        lens = lens + 1
        toks = r["argmax"].reshape(B, 1)
    return dict(tokens=out, gap=gap, k_cache=kc, v_cache=vc, seq_lens=lens)
