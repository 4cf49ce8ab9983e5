"""Pins of the multi-layer pass oracle (oracle.model) against independent
constructions: hand-computed norms and rotations, invariants of rotary
embedding, a dense causal forward of each node's root path written here from
scratch (np.tril mask over the concatenated sequence), and token-by-token
decoding."""
import numpy as np
import pytest

import oracle
from workloads import MODELS, WORKLOADS, model_inputs, model_weights

CFG = MODELS["tiny_d64"]
WL = WORKLOADS["qwen3_8b_ragged8_N64"].replace(B=2, Hq=4, Hkv=2, D=64, N=12, L_lo=20,
                                              L_hi=70, seed=5)


def _dec(x):
    return oracle.decode(x, "bf16")


# ---------------------------------------------------------------- building blocks


def test_m1_rms_norm_hand_values_and_invariants():
    x = np.array([3.0, 4.0])
    np.testing.assert_allclose(oracle.rms_norm(x, 1.0, 0.0), [3 / np.sqrt(12.5), 4 / np.sqrt(12.5)],
                               rtol=1e-15)
    np.testing.assert_allclose(oracle.rms_norm(x, np.array([2.0, -1.0]), 0.0),
                               [6 / np.sqrt(12.5), -4 / np.sqrt(12.5)], rtol=1e-15)
    rng = np.random.default_rng(1)
    y = rng.standard_normal((5, 33))
    r = oracle.rms_norm(y, 1.0, 0.0)
    np.testing.assert_allclose(np.sqrt((r ** 2).mean(axis=1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(oracle.rms_norm(7.5 * y, 1.0, 0.0), r, rtol=1e-13)
    # eps enters under the root: a zero row stays zero, a tiny row is damped
    np.testing.assert_array_equal(oracle.rms_norm(np.zeros(4), 1.0, 1e-6), np.zeros(4))


def test_m2_rope_hand_values():
    # D = 2: one pair, frequency theta^0 = 1, angle = pos radians
    for pos in (0, 1, 5, 1000):
        np.testing.assert_allclose(oracle.rope(np.array([1.0, 0.0]), pos, 1e6),
                                   [np.cos(pos), np.sin(pos)], atol=1e-12)
    # D = 4, theta = 100: pairs (0, 2) at angle pos and (1, 3) at angle pos / 10
    x = np.array([1.0, 2.0, 3.0, 4.0])
    pos = 3
    a, b = 3.0, 0.3
    want = [1 * np.cos(a) - 3 * np.sin(a), 2 * np.cos(b) - 4 * np.sin(b),
            3 * np.cos(a) + 1 * np.sin(a), 4 * np.cos(b) + 2 * np.sin(b)]
    np.testing.assert_allclose(oracle.rope(x, pos, 100.0), want, atol=1e-12)


def test_m2_rope_invariants():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((2, 64))
    np.testing.assert_array_equal(oracle.rope(q, 0, 1e6), q)
    half = 32
    rq = oracle.rope(q, 77, 1e6)
    np.testing.assert_allclose(rq[:half] ** 2 + rq[half:] ** 2, q[:half] ** 2 + q[half:] ** 2,
                               rtol=1e-12)
    # scores depend on the position difference only
    for m, n, t in ((5, 2, 100), (1000, 999, 7), (0, 40, 12345)):
        s1 = oracle.rope(q, m, 1e6) @ oracle.rope(k, n, 1e6)
        s2 = oracle.rope(q, m + t, 1e6) @ oracle.rope(k, n + t, 1e6)
        assert abs(s1 - s2) < 1e-9


def test_m2b_silu_hand_values():
    """silu(x) = x * logistic(x): the logistic function's known values at
    0, +-1 and +-2, the far negative tail and the positive
    saturation, where the correction falls below fp64 spacing (values to
    40 digits from a decimal evaluation of x / (1 + e^-x))."""
    x = np.array([0.0, 1.0, -1.0, 2.0, -2.0, -30.0, 40.0])
    want = np.array([0.0,
                     0.7310585786300049,      # logistic(1)
                     -0.2689414213699951,     # -logistic(-1) = -(1 - logistic(1))
                     1.7615941559557646,      # 2 * logistic(2)
                     -0.2384058440442351,     # -2 * logistic(-2)
                     -2.807286890651790e-12,   # -30 / (1 + e^30)
                     40.0])
    np.testing.assert_allclose(oracle.silu(x), want, rtol=1e-15, atol=0)
    # odd part: silu(x) - silu(-x) = x for every x
    y = np.linspace(-8, 8, 33)
    np.testing.assert_allclose(oracle.silu(y) - oracle.silu(-y), y, rtol=0, atol=1e-14)


def test_m3_node_positions_hand_tree():
    parent = np.array([[-1, 0, 0, 1, 3, 2]])
    np.testing.assert_array_equal(oracle.node_positions(parent, [10]),
                                  [[10, 11, 11, 12, 13, 12]])


def test_m4_zero_output_projections_leave_the_embedding():
    w = model_weights(CFG)
    x = model_inputs(CFG, WL)
    w = dict(w, w_o=np.zeros_like(w["w_o"]), w_down=np.zeros_like(w["w_down"]))
    r = oracle.verify_pass(CFG.dims(), w, x["tokens"], x["parent"], x["seq_lens"],
                           x["k_cache"], x["v_cache"])
    e = _dec(w["embed"])[x["tokens"].reshape(-1)]
    h = e / np.sqrt((e ** 2).mean(axis=1, keepdims=True) + CFG.eps) * _dec(w["final_norm"])
    np.testing.assert_allclose(r["hidden"], h, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(r["argmax"], np.argmax(h @ _dec(w["lm_head"]).T, axis=1))


# ---------------------------------------------------------------- dense causal forward


def _dense_path_logits(cfg, w, kc, vc, b, L, path_tokens, ly_count):
    """Logits of the last token of ``path_tokens`` (positions L, L+1, ...)
    by a plain causal forward over the prefix cache plus the path."""
    Hq, Hkv, D, I = cfg.Hq, cfg.Hkv, cfg.D, cfg.inter
    G = Hq // Hkv
    T = len(path_tokens)
    x = _dec(w["embed"])[np.asarray(path_tokens)]
    pos = L + np.arange(T)
    for ly in range(ly_count):
        h = oracle.rms_norm(x, _dec(w["ln1"][ly]), cfg.eps)
        wq = _dec(w["w_qkv"][ly])
        q = (h @ wq[:Hq * D].T).reshape(T, Hq, D)
        k = (h @ wq[Hq * D:(Hq + Hkv) * D].T).reshape(T, Hkv, D)
        v = (h @ wq[(Hq + Hkv) * D:].T).reshape(T, Hkv, D)
        q = oracle.rope(oracle.rms_norm(q, _dec(w["q_norm"][ly]), cfg.eps), pos[:, None], cfg.theta)
        k = oracle.rope(oracle.rms_norm(k, _dec(w["k_norm"][ly]), cfg.eps), pos[:, None], cfg.theta)
        att = np.empty((T, Hq, D))
        mask = np.concatenate([np.ones((T, L), bool), np.tril(np.ones((T, T), bool))], axis=1)
        for hh in range(Hq):
            g = hh // G
            keys = np.concatenate([_dec(kc[ly, b, g, :L]), k[:, g]], axis=0)
            vals = np.concatenate([_dec(vc[ly, b, g, :L]), v[:, g]], axis=0)
            s = np.where(mask, q[:, hh] @ keys.T / np.sqrt(D), -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            att[:, hh] = (p / p.sum(axis=1, keepdims=True)) @ vals
        x = x + att.reshape(T, Hq * D) @ _dec(w["w_o"][ly]).T
        h = oracle.rms_norm(x, _dec(w["ln2"][ly]), cfg.eps)
        g_ = h @ _dec(w["w_gu"][ly][:I]).T
        u_ = h @ _dec(w["w_gu"][ly][I:]).T
        x = x + (g_ / (1 + np.exp(-g_)) * u_) @ _dec(w["w_down"][ly]).T
    hf = oracle.rms_norm(x[-1], _dec(w["final_norm"]), cfg.eps)
    return hf @ _dec(w["lm_head"]).T


def test_m5_every_tree_node_equals_a_dense_causal_forward_of_its_root_path():
    w = model_weights(CFG)
    x = model_inputs(CFG, WL)
    r = oracle.verify_pass(CFG.dims(), w, x["tokens"], x["parent"], x["seq_lens"],
                           x["k_cache"], x["v_cache"])
    N = WL.N
    for b in range(WL.B):
        L = int(x["seq_lens"][b])
        for i in range(N):
            path = oracle.ancestors(x["parent"][b], i)[::-1]
            ref = _dense_path_logits(CFG, w, x["k_cache"], x["v_cache"], b, L,
                                     x["tokens"][b, path], CFG.layers)
            np.testing.assert_allclose(r["logits"][b * N + i], ref, rtol=0, atol=1e-10)


def test_m6_chain_tree_equals_token_by_token_decoding():
    w = model_weights(CFG)
    wl = WL.replace(B=1, N=6, L_lo=30, L_hi=30)
    x = model_inputs(CFG, wl)
    chain = np.arange(-1, wl.N - 1, dtype=np.int32)[None]
    r = oracle.verify_pass(CFG.dims(), w, x["tokens"], chain, x["seq_lens"], x["k_cache"],
                           x["v_cache"])
    kc = oracle.decode(x["k_cache"], "bf16")
    vc = oracle.decode(x["v_cache"], "bf16")
    L = int(x["seq_lens"][0])
    for j in range(wl.N):
        # one token at a time at the growing length: the cache holds the
        # earlier tokens' rows as the previous one-token pass wrote them
        step = oracle.verify_pass(CFG.dims(), w, x["tokens"][:, j:j + 1], np.array([[-1]]),
                                  np.array([L + j]), kc, vc)
        np.testing.assert_allclose(step["logits"][0], r["logits"][j], rtol=0, atol=1e-10)
        kc, vc = step["k_cache"], step["v_cache"]
    np.testing.assert_allclose(kc[:, :, :, L:L + wl.N], r["k_cache"][:, :, :, L:L + wl.N],
                               rtol=0, atol=1e-12)


def _consistent_draft(w, x, every=3, rounds=16):
    """Draft tokens that copy the target's greedy token at the parent for
    nodes i with i % every != 0, iterated until the tokens stop changing
    (each round fixes one more tree level)."""
    tokens = x["tokens"].copy()
    B, N = tokens.shape
    for _ in range(rounds):
        r = oracle.verify_pass(CFG.dims(), w, tokens, x["parent"], x["seq_lens"],
                               x["k_cache"], x["v_cache"])
        tgt = r["argmax"].reshape(B, N).astype(np.int32)
        new = tokens.copy()
        for b in range(B):
            for i in range(1, N):
                if i % every:
                    new[b, i] = tgt[b, x["parent"][b, i]]
        if (new == tokens).all():
            return tokens, r
        tokens = new
    raise AssertionError("draft did not settle")


def test_m7_compaction_then_bonus_token_continues_the_accepted_path():
    """After the accepted path is compacted into every layer's cache, a one-node
    pass of the bonus token at the new length equals the dense forward of
    prefix + path tokens + bonus (cross-step invariant)."""
    w = model_weights(CFG)
    x = model_inputs(CFG, WL)
    tokens, r = _consistent_draft(w, x)
    tgt = r["argmax"].reshape(WL.B, WL.N).astype(np.int32)
    acc = oracle.tree_accept(x["parent"], tokens, tgt, P=16)
    assert acc["path_len"].min() >= 3
    k2, v2, lens2 = oracle.kv_compact_layers(r["k_cache"], r["v_cache"], x["seq_lens"],
                                             acc["path"], acc["path_len"])
    for ly in range(CFG.layers):
        ka, va, la = oracle.kv_compact(r["k_cache"][ly], r["v_cache"][ly], x["seq_lens"],
                                       acc["path"], acc["path_len"])
        np.testing.assert_array_equal(k2[ly], ka)
        np.testing.assert_array_equal(v2[ly], va)
        np.testing.assert_array_equal(lens2, la)
    np.testing.assert_array_equal(lens2, x["seq_lens"] + acc["path_len"])
    nxt = oracle.verify_pass(CFG.dims(), w, acc["bonus"][:, None], np.full((WL.B, 1), -1),
                             lens2, k2, v2)
    for b in range(WL.B):
        n = int(acc["path_len"][b])
        toks = list(tokens[b, acc["path"][b, :n]]) + [int(acc["bonus"][b])]
        ref = _dense_path_logits(CFG, w, x["k_cache"], x["v_cache"], b, int(x["seq_lens"][b]),
                                 toks, CFG.layers)
        np.testing.assert_allclose(nxt["logits"][b], ref, rtol=0, atol=1e-10)


def test_m8_greedy_decoding_is_consistent_with_one_chain_pass():
    """n one-token steps of greedy decoding against one pass over the chain
    [root, t1, .., t_{n-1}]: the chain's argmax at node i is t_{i+1}, and the
    caches agree (independent formulations: n sequential passes, one tree
    pass)."""
    w = model_weights(CFG)
    wl = WL.replace(B=2, N=1, L_lo=25, L_hi=60)
    x = model_inputs(CFG, wl)
    n = 7
    ar = oracle.ar_decode(CFG.dims(), w, x["k_cache"], x["v_cache"], x["seq_lens"],
                          x["tokens"][:, 0], n)
    chain_tok = np.concatenate([x["tokens"][:, :1], ar["tokens"][:, :n - 1]], axis=1)
    chain = np.tile(np.arange(-1, n - 1), (wl.B, 1))
    r = oracle.verify_pass(CFG.dims(), w, chain_tok, chain, x["seq_lens"], x["k_cache"],
                           x["v_cache"])
    np.testing.assert_array_equal(r["argmax"].reshape(wl.B, n), ar["tokens"])
    np.testing.assert_array_equal(ar["seq_lens"], x["seq_lens"] + n)
    for b in range(wl.B):
        L = int(x["seq_lens"][b])
        np.testing.assert_allclose(ar["k_cache"][:, b, :, L:L + n], r["k_cache"][:, b, :, L:L + n],
                                   rtol=0, atol=1e-11)


# ---------------------------------------------------------------- bf16 storage model


def test_m9_round_bf16_hand_values_and_invariants():
    """Round to nearest, ties to even, at 7 fraction bits (spacing 2^-7 at 1)."""
    r = oracle.round_bf16
    e = 2.0 ** -8
    cases = [(1.0, 1.0), (1 + e, 1.0),                    # tie -> even (1.0)
             (1 + 3 * e, 1 + 4 * e),                       # tie -> even (1 + 2^-6)
             (1 + e + 2.0 ** -20, 1 + 2 * e),              # above the tie
             (-(1 + 3 * e), -(1 + 4 * e)), (65535.0, 65536.0),
             (3.14159265358979, 3.140625), (0.1, 0.10009765625), (0.0, 0.0)]
    for x, want in cases:
        assert r(np.array([x]))[0] == want, x
    assert np.isinf(r(np.array([np.inf]))[0]) and np.isnan(r(np.array([np.nan]))[0])
    # every finite bf16 value is its own rounding; relative error <= 2^-8
    bits = np.arange(1 << 16, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        vals = oracle.decode(bits, "bf16")
    fin = np.isfinite(vals)
    np.testing.assert_array_equal(r(vals[fin]), vals[fin])
    x = np.random.default_rng(3).standard_normal(100_000) * 10.0 ** np.random.default_rng(4).uniform(-20, 20, 100_000)
    y = r(x)
    np.testing.assert_array_equal(r(y), y)
    assert np.all(np.abs(y - x) <= 2.0 ** -8 * np.abs(x))


def test_m10_bf16_storage_model_rounds_what_it_names_and_only_perturbs():
    """With bf16_points the written cache rows are bf16 values; the pass moves by about the rounding size (2^-9 relative per
    stored value), not by more, and the prefix rows stay as they were."""
    w = model_weights(CFG)
    x = model_inputs(CFG, WL)
    args = (CFG.dims(), w, x["tokens"], x["parent"], x["seq_lens"], x["k_cache"], x["v_cache"])
    ex = oracle.verify_pass(*args)
    rd = oracle.verify_pass(*args, bf16_points=True)
    for b, L in enumerate(x["seq_lens"]):
        L = int(L)
        for c in ("k_cache", "v_cache"):
            t = rd[c][:, b, :, L:L + WL.N]
            np.testing.assert_array_equal(oracle.round_bf16(t), t)
            np.testing.assert_array_equal(rd[c][:, b, :, :L], ex[c][:, b, :, :L])
    rel = np.linalg.norm(rd["hidden"] - ex["hidden"]) / np.linalg.norm(ex["hidden"])
    assert 2.0 ** -12 < rel < 2.0 ** -6
    # the probability rounding alone moves attention by no more than its size
    q = x["k_cache"][0, :, :, :WL.N].transpose(0, 2, 1, 3)        # any bf16 [B][N][H][D]
    q = np.repeat(q, WL.Hq // WL.Hkv, axis=2)
    kc, vc = x["k_cache"][0].copy(), x["v_cache"][0].copy()
    for b, L in enumerate(x["seq_lens"]):
        kc[b, :, int(L):int(L) + WL.N] = x["k_cache"][0, b, :, :WL.N]
        vc[b, :, int(L):int(L) + WL.N] = x["v_cache"][0, b, :, :WL.N]
    a0 = oracle.tree_attention(q, kc, vc, x["seq_lens"], x["parent"], 0.1, "bf16")
    a1 = oracle.tree_attention(q, kc, vc, x["seq_lens"], x["parent"], 0.1, "bf16",
                               p_round=oracle.round_bf16)
    # |sum_t (p~_t - p_t) v_t| / sum_t p_t <= 2^-8 max |v| when |p~ - p| <= 2^-8 p
    d = np.abs(a1 - a0)
    vmax = np.nanmax(np.abs(oracle.decode(vc, "bf16")))
    assert 0 < d.max() <= 2.0 ** -8 * vmax
