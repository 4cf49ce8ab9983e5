"""Pins that tie the fp64 oracle to the pages' definitions and to mathematics.

None of these re-types the oracle's own formula: each compares it with an
independent construction (dense causal attention built from np.tril, a mask
from a transitive closure, closed forms, exact integer arithmetic, exhaustive
enumeration, a path-functional greedy decoder, a hand-worked fixture).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from workloads import bf16_bits_from_f32

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand_f32(rng, shape, scale=1.0):
    return (scale * rng.standard_normal(shape)).astype(np.float32)


def _softmax_rows(s):
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def _caches(rng, B, Hkv, L, N, D, extra=5):
    Lcap = L + N + extra
    k = _rand_f32(rng, (B, Hkv, Lcap, D))
    v = _rand_f32(rng, (B, Hkv, Lcap, D))
    return k, v


def _random_tree(rng, N):
    parent = np.full(N, -1, dtype=np.int32)
    for i in range(1, N):
        parent[i] = rng.integers(0, i)
    return parent


# ---------------------------------------------------------------- attention


@pytest.mark.parametrize("G", [1, 4])
def test_p1_chain_tree_equals_causal_attention(G):
    """Chain tree (parent[i] = i-1) == ordinary causal attention."""
    rng = np.random.default_rng(11)
    B, Hkv, L, N, D = 2, 2, 13, 9, 16
    Hq = Hkv * G
    k, v = _caches(rng, B, Hkv, L, N, D)
    q = _rand_f32(rng, (B, N, Hq, D))
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    seq = np.array([L, L - 4], dtype=np.int32)
    scale = 0.3
    got = oracle.tree_attention(q, k, v, seq, parent, scale, "f32")
    for b in range(B):
        Lb = int(seq[b])
        T = Lb + N
        causal = np.tril(np.ones((T, T), dtype=bool))[Lb:]      # rows of the tree
        for h in range(Hq):
            g = h // G
            Kb = k[b, g, :T].astype(np.float64)
            Vb = v[b, g, :T].astype(np.float64)
            s = scale * q[b, :, h].astype(np.float64) @ Kb.T      # [N, T]
            s = np.where(causal, s, -np.inf)
            ref = _softmax_rows(s) @ Vb
            np.testing.assert_allclose(got[b, :, h], ref, rtol=0, atol=1e-12)


def _closure_mask(parent):
    """Ancestor-or-self matrix by boolean transitive closure of the parent edges."""
    N = len(parent)
    A = np.eye(N, dtype=bool)
    E = np.zeros((N, N), dtype=bool)
    for i in range(1, N):
        E[i, parent[i]] = True
    R = A | E
    while True:
        R2 = R | ((R.astype(np.int64) @ R.astype(np.int64)) > 0)
        if (R2 == R).all():
            return R
        R = R2


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_p2_brute_force_dense_mask(seed):
    """Every node == plain masked attention over prefix + its closure ancestors."""
    rng = np.random.default_rng(100 + seed)
    B, Hkv, G, N, D = 2, 2, 2, 17, 8
    Hq = Hkv * G
    seq = np.array([5, 0], dtype=np.int32)       # includes an empty prefix
    k, v = _caches(rng, B, Hkv, 5, N, D)
    q = _rand_f32(rng, (B, N, Hq, D))
    parent = np.stack([_random_tree(rng, N) for _ in range(B)])
    scale = 1 / np.sqrt(D)
    got = oracle.tree_attention(q, k, v, seq, parent, scale, "f32")
    for b in range(B):
        Lb = int(seq[b])
        mask = np.concatenate(
            [np.ones((N, Lb), dtype=bool), _closure_mask(parent[b])], axis=1)
        for h in range(Hq):
            g = h // G
            for i in range(N):
                keys = np.nonzero(mask[i])[0]
                kk = k[b, g, keys].astype(np.float64)
                vv = v[b, g, keys].astype(np.float64)
                s = scale * kk @ q[b, i, h].astype(np.float64)
                p = np.exp(s - s.max())
                ref = (p / p.sum()) @ vv
                np.testing.assert_allclose(got[b, i, h], ref, rtol=0, atol=1e-12)


def test_p3_single_node_equals_decode_attention():
    rng = np.random.default_rng(3)
    B, Hkv, G, L, D = 1, 2, 4, 40, 32
    Hq = Hkv * G
    k, v = _caches(rng, B, Hkv, L, 1, D)
    q = _rand_f32(rng, (B, 1, Hq, D))
    parent = np.array([[-1]], dtype=np.int32)
    got = oracle.tree_attention(q, k, v, np.array([L], np.int32), parent, 0.2, "f32")
    for h in range(Hq):
        K = k[0, h // G, :L + 1].astype(np.float64)
        V = v[0, h // G, :L + 1].astype(np.float64)
        w = _softmax_rows(0.2 * (K @ q[0, 0, h].astype(np.float64))[None])[0]
        np.testing.assert_allclose(got[0, 0, h], w @ V, rtol=0, atol=1e-12)


def test_p4_closed_forms():
    rng = np.random.default_rng(4)
    B, Hkv, G, L, N, D = 1, 1, 2, 6, 7, 4
    Hq = Hkv * G
    k, v = _caches(rng, B, Hkv, L, N, D)
    parent = np.array([[-1, 0, 0, 1, 1, 2, 2]], dtype=np.int32)
    seq = np.array([L], np.int32)
    q = _rand_f32(rng, (B, N, Hq, D))
    # constant V rows -> output is that constant
    c = np.array([1.5, -2.0, 0.25, 3.0], dtype=np.float32)
    vc = np.broadcast_to(c, v.shape).copy()
    got = oracle.tree_attention(q, k, vc, seq, parent, 0.7, "f32")
    np.testing.assert_allclose(got, np.broadcast_to(c, got.shape), atol=1e-12)
    # q = 0 -> uniform weights: mean of the visible V rows
    got = oracle.tree_attention(np.zeros_like(q), k, v, seq, parent, 0.7, "f32")
    vis = {0: [0], 1: [0, 1], 2: [0, 2], 3: [0, 1, 3], 4: [0, 1, 4],
           5: [0, 2, 5], 6: [0, 2, 6]}
    for i, anc in vis.items():
        rows = list(range(L)) + [L + j for j in anc]
        ref = v[0, 0, rows].astype(np.float64).mean(axis=0)
        for h in range(Hq):
            np.testing.assert_allclose(got[0, i, h], ref, atol=1e-12)
    # one prefix key: the root output is a two-term weighted average
    q1 = _rand_f32(rng, (1, 1, 1, D))
    k1, v1 = _caches(rng, 1, 1, 1, 1, D)
    got = oracle.tree_attention(q1, k1, v1, np.array([1], np.int32),
                                np.array([[-1]], np.int32), 0.5, "f32")
    qd = q1[0, 0, 0].astype(np.float64)
    s0 = 0.5 * qd @ k1[0, 0, 0].astype(np.float64)
    sr = 0.5 * qd @ k1[0, 0, 1].astype(np.float64)
    ref = (v1[0, 0, 0] * np.exp(s0) + v1[0, 0, 1] * np.exp(sr)) / (np.exp(s0) + np.exp(sr))
    np.testing.assert_allclose(got[0, 0, 0], ref, atol=1e-12)


def _random_topological_relabel(rng, parent):
    """A random order of the nodes in which every parent precedes its children."""
    N = len(parent)
    children = {i: [] for i in range(N)}
    for i in range(1, N):
        children[int(parent[i])].append(i)
    order, avail = [], [0]
    while avail:
        j = avail.pop(rng.integers(0, len(avail)))
        order.append(j)
        avail.extend(children[j])
    return np.array(order)          # new index t holds old node order[t]


def test_p5_relabeling_invariance():
    rng = np.random.default_rng(5)
    Hkv, G, L, N, D = 2, 2, 9, 23, 8
    Hq = Hkv * G
    k, v = _caches(rng, 1, Hkv, L, N, D)
    q = _rand_f32(rng, (1, N, Hq, D))
    parent = _random_tree(rng, N)
    order = _random_topological_relabel(rng, parent)
    new_of_old = np.empty(N, dtype=np.int64)
    new_of_old[order] = np.arange(N)
    parent2 = np.array([-1] + [new_of_old[parent[o]] for o in order[1:]], dtype=np.int32)
    q2 = q[:, order]
    k2, v2 = k.copy(), v.copy()
    k2[:, :, L:L + N] = k[:, :, L + order]
    v2[:, :, L:L + N] = v[:, :, L + order]
    seq = np.array([L], np.int32)
    a = oracle.tree_attention(q, k, v, seq, parent[None], 0.35, "f32")
    b = oracle.tree_attention(q2, k2, v2, seq, parent2[None], 0.35, "f32")
    np.testing.assert_allclose(b[0], a[0, order], atol=1e-12)


def test_attention_reads_bf16_bits_exactly():
    """bf16 bit patterns decode to their exact values (e.g. 0x3F80 = 1.0)."""
    x = np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x7F80], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.decode(x, "bf16"),
                                  [1.0, -2.0, 0.25, 0.0, np.inf])


# ---------------------------------------------------------------- LM head


def test_p6_lm_head_exact_small_integers_and_ties():
    rng = np.random.default_rng(6)
    M, Hd, V = 9, 24, 61
    Hi = rng.integers(-3, 4, size=(M, Hd))
    Wi = rng.integers(-3, 4, size=(V, Hd))
    Wi[40] = Wi[7]              # exact duplicate rows -> exact logit ties
    Wi[41] = Wi[7]
    Wi[13] = Wi[12]
    exact = Hi.astype(np.int64) @ Wi.T.astype(np.int64)   # integer arithmetic
    for dtype, enc in (("bf16", bf16_bits_from_f32), ("f32", lambda a: a.astype(np.float32))):
        h = enc(Hi.astype(np.float32))
        w = enc(Wi.astype(np.float32))
        np.testing.assert_array_equal(oracle.lm_logits(h, w, dtype), exact)
        for chunk in (7, 8, 64, 8192):
            r = oracle.lm_head_argmax(h, w, dtype, v_chunk=chunk)
            np.testing.assert_array_equal(r["argmax"], np.argmax(exact, axis=1))
            srt = np.sort(exact, axis=1)
            np.testing.assert_array_equal(r["top1"], srt[:, -1])
            np.testing.assert_array_equal(r["gap"], srt[:, -1] - srt[:, -2])
    # a row whose maximum is attained twice has gap 0 and the smaller index wins
    h = np.zeros((1, Hd), np.float32)
    h[0, 0] = 1.0
    w = np.zeros((V, Hd), np.float32)
    w[30, 0] = 5.0
    w[10, 0] = 5.0
    r = oracle.lm_head_argmax(h, w, "f32", v_chunk=16)
    assert r["argmax"][0] == 10 and r["gap"][0] == 0.0


def test_lm_head_row_subset_matches_full():
    rng = np.random.default_rng(66)
    h = bf16_bits_from_f32(rng.standard_normal((12, 32)))
    w = bf16_bits_from_f32(0.02 * rng.standard_normal((300, 32)))
    full = oracle.lm_head_argmax(h, w, "bf16", v_chunk=64)
    rows = np.array([3, 7, 11])
    sub = oracle.lm_head_argmax(h, w, "bf16", rows=rows, v_chunk=64)
    np.testing.assert_array_equal(sub["argmax"], full["argmax"][rows])


# ---------------------------------------------------------------- acceptance


def _brute_accept(parent, draft, tgt):
    """Enumerate every node, check its whole root path, keep the deepest."""
    N = len(parent)
    best, best_d = 0, 0
    for i in range(N):
        path = [i]
        while path[-1] != 0:
            path.append(int(parent[path[-1]]))
        path = path[::-1]
        ok = all(draft[path[t]] == tgt[path[t - 1]] for t in range(1, len(path)))
        if ok and len(path) - 1 > best_d:
            best, best_d = i, len(path) - 1
    path = [best]
    while path[-1] != 0:
        path.append(int(parent[path[-1]]))
    return path[::-1], tgt[best]


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7])
def test_p7_accept_brute_force_all_topologies(N):
    rng = np.random.default_rng(70 + N)
    for choice in itertools.product(*[range(i) for i in range(1, N)]):
        parent = np.array([-1] + list(choice), dtype=np.int32)
        for _ in range(3):
            draft = rng.integers(0, 3, size=N).astype(np.int32)
            tgt = rng.integers(0, 3, size=N).astype(np.int32)
            r = oracle.tree_accept(parent[None], draft[None], tgt[None], P=8)
            path, bonus = _brute_accept(parent, draft, tgt)
            n = int(r["path_len"][0])
            assert n == len(path)
            assert list(r["path"][0, :n]) == path
            assert (r["path"][0, n:] == -1).all()
            assert r["bonus"][0] == bonus


def _path_hash(tokens, V):
    h = 1469598103934665603
    for t in tokens:
        h = ((h ^ int(t)) * 1099511628211) & ((1 << 64) - 1)
    return int(h % V)


@pytest.mark.parametrize("seed", range(6))
def test_p8_ar_equivalence_path_functional_target(seed):
    """Emitted tokens == the first path_len tokens of greedy AR decoding.

    The target is path-functional: its greedy token after a token sequence is
    a hash of that sequence, so greedy decoding from the root is a fixed
    token stream independent of the tree.
    """
    rng = np.random.default_rng(800 + seed)
    V, N = 5, 40
    parent = _random_tree(rng, N)
    draft = np.zeros(N, dtype=np.int32)
    draft[0] = rng.integers(0, V)
    toks = {0: [int(draft[0])]}
    for i in range(1, N):
        p = int(parent[i])
        want = _path_hash(toks[p], V)
        draft[i] = want if rng.random() < 0.85 else rng.integers(0, V)
        toks[i] = toks[p] + [int(draft[i])]
    tgt = np.array([_path_hash(toks[i], V) for i in range(N)], dtype=np.int32)
    r = oracle.tree_accept(parent[None], draft[None], tgt[None], P=N + 1)
    n = int(r["path_len"][0])
    path = r["path"][0, :n]
    emitted = [int(draft[j]) for j in path[1:]] + [int(r["bonus"][0])]
    ar = [int(draft[0])]
    for _ in range(n):
        ar.append(_path_hash(ar, V))
    assert emitted == ar[1:n + 1]
    # maximality: no tree node reproduces a longer AR prefix
    for i in range(N):
        if toks[i] == ar[:len(toks[i])]:
            assert len(toks[i]) <= n


def test_p9_special_cases():
    N = 9
    chain = np.arange(-1, N - 1, dtype=np.int32)[None]
    tgt = np.arange(100, 100 + N, dtype=np.int32)[None]
    draft = np.concatenate([[7], tgt[0, :-1]]).astype(np.int32)[None]
    r = oracle.tree_accept(chain, draft, tgt, P=16)
    assert r["path_len"][0] == N and r["bonus"][0] == tgt[0, N - 1]
    assert list(r["path"][0, :N]) == list(range(N))
    r = oracle.tree_accept(chain, np.full((1, N), 5, np.int32), tgt, P=16)
    assert r["path_len"][0] == 1 and r["bonus"][0] == 100 and r["path"][0, 0] == 0
    r = oracle.tree_accept(np.array([[-1]], np.int32), np.array([[3]], np.int32),
                           np.array([[42]], np.int32), P=4)
    assert r["path_len"][0] == 1 and r["bonus"][0] == 42
    with pytest.raises(ValueError):
        oracle.tree_accept(np.array([[-1, 1]], np.int32), np.zeros((1, 2), np.int32),
                           np.zeros((1, 2), np.int32))


def test_golden_worked_example():
    with open(os.path.join(HERE, "golden", "accept_worked_example.json")) as f:
        g = json.load(f)
    parent = np.array([g["parent"]], np.int32)
    draft = np.array([g["draft"]], np.int32)
    tgt = np.array([g["tgt"]], np.int32)
    r = oracle.tree_accept(parent, draft, tgt, P=8)
    n = int(r["path_len"][0])
    assert n == g["path_len"]
    assert list(r["path"][0, :n]) == g["path"]
    assert r["bonus"][0] == g["bonus"]
    assert [int(draft[0, j]) for j in r["path"][0, 1:n]] + [int(r["bonus"][0])] == g["emitted"]
    N, D, L = 8, 4, g["prefix_len"]
    k = np.arange(1 * 2 * (L + N + 3) * D, dtype=np.float32).reshape(1, 2, L + N + 3, D)
    v = -k
    k2, v2, lens = oracle.kv_compact(k, v, np.array([L], np.int32), r["path"], r["path_len"])
    assert lens[0] == g["new_len"]
    moved = {dst: src for dst, src in g["row_moves"]}
    for row in range(L + N + 3):
        src = moved.get(row, row)
        np.testing.assert_array_equal(k2[0, :, row], k[0, :, src])
        np.testing.assert_array_equal(v2[0, :, row], v[0, :, src])


# ---------------------------------------------------------------- compaction


@pytest.mark.parametrize("seed", range(4))
def test_compaction_moves_path_rows(seed):
    """Row L+j of the result holds original row L+path[j]; nothing else moves."""
    rng = np.random.default_rng(900 + seed)
    B, Hkv, N, D = 3, 2, 30, 4
    seq = rng.integers(0, 20, size=B).astype(np.int32)
    Lcap = 20 + N + 4
    k = rng.integers(0, 60000, size=(B, Hkv, Lcap, D)).astype(np.uint16)
    v = rng.integers(0, 60000, size=(B, Hkv, Lcap, D)).astype(np.uint16)
    parent = np.stack([_random_tree(rng, N) for _ in range(B)])
    # accept a random deep chain: choose a node, its root path is "accepted"
    P = N + 1
    path = np.full((B, P), -1, np.int32)
    plen = np.zeros(B, np.int32)
    for b in range(B):
        node = int(rng.integers(0, N))
        walk = oracle.ancestors(parent[b], node)[::-1]
        path[b, :len(walk)] = walk
        plen[b] = len(walk)
    k2, v2, lens = oracle.kv_compact(k, v, seq, path, plen)
    np.testing.assert_array_equal(lens, seq + plen)
    for b in range(B):
        L = int(seq[b])
        for row in range(Lcap):
            j = row - L
            src = L + int(path[b, j]) if 0 <= j < plen[b] else row
            np.testing.assert_array_equal(k2[b, :, row], k[b, :, src])
            np.testing.assert_array_equal(v2[b, :, row], v[b, :, src])


def test_p10_cross_step_invariant():
    """After compaction, causal attention of node path[j] over rows [0, L+j]
    equals its tree output; prefix rows are bit-identical."""
    rng = np.random.default_rng(10)
    B, Hkv, G, L, N, D = 2, 2, 2, 11, 25, 8
    Hq = Hkv * G
    k, v = _caches(rng, B, Hkv, L, N, D)
    q = _rand_f32(rng, (B, N, Hq, D))
    parent = np.stack([_random_tree(rng, N) for _ in range(B)])
    seq = np.array([L, L - 3], np.int32)
    tree_out = oracle.tree_attention(q, k, v, seq, parent, 0.4, "f32")
    tgt = rng.integers(0, 3, size=(B, N)).astype(np.int32)
    draft = np.take_along_axis(tgt, np.maximum(parent, 0), axis=1)
    draft[:, 0] = 0
    flip = rng.random((B, N)) < 0.2
    draft = np.where(flip, (draft + 1) % 3, draft).astype(np.int32)
    acc = oracle.tree_accept(parent, draft, tgt, P=N + 1)
    k2, v2, lens = oracle.kv_compact(k, v, seq, acc["path"], acc["path_len"])
    for b in range(B):
        Lb = int(seq[b])
        np.testing.assert_array_equal(k2[b, :, :Lb], k[b, :, :Lb])
        np.testing.assert_array_equal(v2[b, :, :Lb], v[b, :, :Lb])
        for j in range(int(acc["path_len"][b])):
            node = int(acc["path"][b, j])
            for h in range(Hq):
                K = k2[b, h // G, :Lb + j + 1].astype(np.float64)
                V = v2[b, h // G, :Lb + j + 1].astype(np.float64)
                w = _softmax_rows(0.4 * (K @ q[b, node, h].astype(np.float64))[None])[0]
                np.testing.assert_allclose(w @ V, tree_out[b, node, h], atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_verify_step_composes_the_pinned_parts(seed):
    """The whole-step oracle against independent checks of each part's
    result: the LM head's greedy tokens against a dense argmax of the exact
    logits, the accepted path and bonus against brute-force enumeration, the
    emitted chain against the greedy tokens it must follow, the caches
    against the row moves the path names, and every accepted node's tree
    output against causal attention over the compacted rows (the cross-step
    invariant)."""
    rng = np.random.default_rng(1200 + seed)
    B, Hkv, G, L, N, D, hid, V = 2, 2, 2, 9, 14, 8, 6, 5
    Hq = Hkv * G
    k, v = _caches(rng, B, Hkv, L, N, D)
    att = dict(q=_rand_f32(rng, (B, N, Hq, D)), k_cache=k, v_cache=v,
               seq_lens=np.array([L, L - 4], np.int32),
               parent=np.stack([_random_tree(rng, N) for _ in range(B)]), scale=0.3)
    lm = dict(hidden=rng.integers(-3, 4, size=(B * N, hid)).astype(np.float32),
              w=rng.integers(-3, 4, size=(V, hid)).astype(np.float32))
    # exact small-integer logits: the greedy token is the first maximum
    logits = lm["hidden"].astype(np.int64) @ lm["w"].astype(np.int64).T
    tgt = np.array([int(np.flatnonzero(r == r.max())[0]) for r in logits]).reshape(B, N)
    draft = np.take_along_axis(tgt, np.maximum(att["parent"], 0), axis=1)
    draft = np.where(rng.random((B, N)) < 0.25, rng.integers(0, V, size=(B, N)), draft)
    draft = draft.astype(np.int32)
    res = oracle.verify_step(att, lm, draft, "f32", P=N + 1)
    np.testing.assert_array_equal(res["tgt"], tgt)
    for b in range(B):
        Lb = int(att["seq_lens"][b])
        path, bonus = _brute_accept(att["parent"][b], draft[b], tgt[b])
        n = int(res["accept"]["path_len"][b])
        assert list(res["accept"]["path"][b, :n]) == path
        assert int(res["accept"]["bonus"][b]) == int(bonus)
        for j in range(1, n):   # every emitted draft is the greedy token of its parent
            assert draft[b, path[j]] == tgt[b, path[j - 1]]
        assert res["seq_lens"][b] == Lb + n
        for row in range(k.shape[2]):
            src = Lb + path[row - Lb] if 0 <= row - Lb < n else row
            np.testing.assert_array_equal(res["k_cache"][b, :, row], k[b, :, src])
            np.testing.assert_array_equal(res["v_cache"][b, :, row], v[b, :, src])
        for j, node in enumerate(path):
            for h in range(Hq):
                K = res["k_cache"][b, h // G, :Lb + j + 1].astype(np.float64)
                Vv = res["v_cache"][b, h // G, :Lb + j + 1].astype(np.float64)
                q = att["q"][b, node, h].astype(np.float64)
                w = _softmax_rows(0.3 * (K @ q)[None])[0]
                np.testing.assert_allclose(w @ Vv, res["out"][b, node, h], atol=1e-12)


# ---------------------------------------------------------------- paged caches


def test_paged_oracle_matches_contiguous_under_any_page_placement():
    """Pages placed by a random permutation hold the same logical rows: paged
    attention and paged compaction equal the (pinned) contiguous results."""
    from workloads import WORKLOADS, attn_inputs, paged_layout
    wl = WORKLOADS["qwen3_8b_ragged8_N64"].replace(B=3, L_lo=40, L_hi=150, N=20, Hq=4, Hkv=2,
                                                   D=16, seed=71)
    a = attn_inputs(wl)
    for ps in (16, 64):
        pg = paged_layout(a["k_cache"], a["v_cache"], ps, seed=ps)
        np.testing.assert_array_equal(
            oracle.paged_to_contiguous(pg["k_pages"], pg["block_table"], ps, a["Lcap"]),
            a["k_cache"])
        got = oracle.tree_attention_paged(a["q"], pg["k_pages"], pg["v_pages"],
                                          pg["block_table"], ps, a["seq_lens"], a["parent"],
                                          a["scale"], "bf16")
        ref = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], a["seq_lens"],
                                    a["parent"], a["scale"], "bf16")
        np.testing.assert_array_equal(got, ref)
        rng = np.random.default_rng(ps)
        P = 16
        path = np.full((wl.B, P), -1, np.int32)
        plen = np.zeros(wl.B, np.int32)
        for b in range(wl.B):
            walk = oracle.ancestors(a["parent"][b], int(rng.integers(0, wl.N)))[::-1]
            path[b, :len(walk)] = walk
            plen[b] = len(walk)
        k2, v2, l2 = oracle.kv_compact_paged(pg["k_pages"], pg["v_pages"], pg["block_table"], ps,
                                             a["seq_lens"], path, plen)
        kc, vc, lc = oracle.kv_compact(a["k_cache"], a["v_cache"], a["seq_lens"], path, plen)
        np.testing.assert_array_equal(l2, lc)
        np.testing.assert_array_equal(
            oracle.paged_to_contiguous(k2, pg["block_table"], ps, a["Lcap"]), kc)
        np.testing.assert_array_equal(
            oracle.paged_to_contiguous(v2, pg["block_table"], ps, a["Lcap"]), vc)


def test_commit_slots_hand_example():
    """Sequence 0 (prefix 2, tree of 5 nodes in slots 102..106) accepts nodes
    0, 2, 4: its window becomes the accepted slots, then the rejected ones in
    node order; sequence 1 accepts 0, 1 and keeps its order."""
    bt = np.arange(20, dtype=np.int32).reshape(2, 10) + 100
    path = np.array([[0, 2, 4, -1], [0, 1, -1, -1]], np.int32)
    nbt, lens = oracle.kv_commit_slots(bt, np.array([2, 3]), path, np.array([3, 2]), 5)
    np.testing.assert_array_equal(nbt[0], [100, 101, 102, 104, 106, 103, 105, 107, 108, 109])
    np.testing.assert_array_equal(nbt[1], bt[1])
    np.testing.assert_array_equal(lens, [5, 5])
    with pytest.raises(ValueError):
        oracle.kv_commit_slots(bt, np.array([2, 3]), np.array([[0, 3, 2, -1], [0, 1, -1, -1]]),
                               np.array([3, 2]), 5)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_commit_slots_equals_row_compaction(seed):
    """With one row per page, the committed table names, at every logical row
    below the new length, the row that the (pinned) row-moving compaction puts
    there; the tree window is a permutation of the old one (no slot lost or
    doubled) and nothing outside it changes."""
    from workloads import WORKLOADS, attn_inputs, paged_layout
    wl = WORKLOADS["qwen3_8b_ragged8_N64"].replace(B=4, L_lo=3, L_hi=60, N=24, Hq=2, Hkv=2, D=8,
                                                   seed=80 + seed)
    a = attn_inputs(wl)
    pg = paged_layout(a["k_cache"], a["v_cache"], 1, seed=seed)
    rng = np.random.default_rng(seed)
    P = 16
    path = np.full((wl.B, P), -1, np.int32)
    plen = np.zeros(wl.B, np.int32)
    for b in range(wl.B):
        walk = oracle.ancestors(a["parent"][b], int(rng.integers(0, wl.N)))[::-1][:P]
        path[b, :len(walk)] = walk
        plen[b] = len(walk)
    nbt, lens = oracle.kv_commit_slots(pg["block_table"], a["seq_lens"], path, plen, wl.N)
    kc, vc, lc = oracle.kv_compact(a["k_cache"], a["v_cache"], a["seq_lens"], path, plen)
    np.testing.assert_array_equal(lens, lc)
    gk = oracle.paged_to_contiguous(pg["k_pages"], nbt, 1, a["Lcap"])
    gv = oracle.paged_to_contiguous(pg["v_pages"], nbt, 1, a["Lcap"])
    for b in range(wl.B):
        n = int(lens[b])
        np.testing.assert_array_equal(gk[b, :, :n], kc[b, :, :n])
        np.testing.assert_array_equal(gv[b, :, :n], vc[b, :, :n])
        L = int(a["seq_lens"][b])
        old, new = pg["block_table"][b], nbt[b]
        assert sorted(new[L:L + wl.N]) == sorted(old[L:L + wl.N])
        np.testing.assert_array_equal(new[:L], old[:L])
        np.testing.assert_array_equal(new[L + wl.N:], old[L + wl.N:])
        # the rejected slots follow in node order
        kept = set(int(x) for x in path[b, :plen[b]])
        rej = [int(old[L + i]) for i in range(wl.N) if i not in kept]
        np.testing.assert_array_equal(new[L + plen[b]:L + wl.N], rej)


def test_commit_slots_brute_force_small_trees():
    """Every increasing path through tiny windows (N <= 5), against a table
    built by explicit position moves."""
    N = 5
    bt = np.array([[7, 11, 3, 9, 5, 13, 2, 8]], np.int32)
    L = 2
    for n in range(1, N + 1):
        for rest in itertools.combinations(range(1, N), n - 1):
            walk = (0,) + rest
            path = np.full((1, N), -1, np.int32)
            path[0, :n] = walk
            nbt, lens = oracle.kv_commit_slots(bt, np.array([L]), path, np.array([n]), N)
            want = list(bt[0])
            window = [int(x) for x in bt[0, L:L + N]]
            order = list(walk) + [i for i in range(N) if i not in walk]
            for pos, node in enumerate(order):
                want[L + pos] = window[node]
            np.testing.assert_array_equal(nbt[0], want)
            assert int(lens[0]) == L + n
