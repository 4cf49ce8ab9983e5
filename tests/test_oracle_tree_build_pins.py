"""Pins of the draft-tree construction oracle (oracle.tree_build): hand-worked
examples (one row per depth, and a path-conditioned draft head whose two
level-1 nodes get different candidates), the width-1 chain, brute-force
enumeration where no level is pruned, and invariants on random inputs
(scores as sums of path-conditioned log-probabilities along each path)."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _logp(rng, B, D, V, scale=3.0):
    x = scale * rng.standard_normal((B, D, V))
    x = x - x.max(axis=-1, keepdims=True)
    return (x - np.log(np.exp(x).sum(axis=-1, keepdims=True))).astype(np.float32)


GOLDEN = json.load(open(os.path.join(HERE, "golden", "tree_build_worked_example.json")))


@pytest.mark.parametrize("ex", GOLDEN["examples"], ids=lambda e: e["name"])
def test_t1_hand_worked_examples(ex):
    logp = np.array(ex["logp"], dtype=np.float32)[None]
    r = oracle.accum_logp_tree(logp, [ex["root_token"]], ex["width"], ex["budget"])
    for k in ("parent", "token", "depth"):
        assert r[k][0].tolist() == ex[k], k
    assert r["score"][0].tolist() == ex["score"]


def test_t2_width_one_is_the_argmax_chain():
    rng = np.random.default_rng(1)
    logp = _logp(rng, 2, 9, 50)
    r = oracle.accum_logp_tree(logp, [3, 4], width=1, budget=6)
    for b in range(2):
        assert r["parent"][b].tolist() == [-1, 0, 1, 2, 3, 4, 5]
        assert r["depth"][b].tolist() == list(range(7))
        want = [int(np.argmax(logp[b, d])) for d in range(6)]
        assert r["token"][b, 1:].tolist() == want
        np.testing.assert_allclose(r["score"][b, 1:],
                                   np.cumsum([float(logp[b, d, want[d]]) for d in range(6)]), rtol=0,
                                   atol=1e-12)


@pytest.mark.parametrize("width,budget", [(3, 5), (4, 12), (5, 30)])
def test_t3_two_levels_match_brute_force_enumeration(width, budget):
    """With depth 2 nothing is pruned: the candidates are every path of one
    or two tokens over the per-depth top tokens."""
    rng = np.random.default_rng(width)
    V = 40
    logp = _logp(rng, 1, 2, V)
    # per-depth candidate lists by an independent sort (value desc, id asc)
    tops = [sorted(range(V), key=lambda t: (-float(logp[0, d, t]), t))[:width] for d in range(2)]
    paths = []   # (score, depth, generation, tokens)
    for j in range(width):
        paths.append((float(logp[0, 0, tops[0][j]]), 1, j, (tops[0][j],)))
    for j1, j2 in itertools.product(range(width), range(width)):
        s = float(logp[0, 0, tops[0][j1]]) + float(logp[0, 1, tops[1][j2]])
        paths.append((s, 2, j1 * width + j2, (tops[0][j1], tops[1][j2])))
    kept = sorted(paths, key=lambda p: (-p[0], p[1], p[2]))[:budget]
    kept = sorted(kept, key=lambda p: (p[1], p[2]))
    r = oracle.accum_logp_tree(logp, [0], width, budget)
    got = []
    for n in range(1, budget + 1):
        toks, i = [], n
        while i != 0:
            toks.append(int(r["token"][0, i]))
            i = int(r["parent"][0, i])
        got.append(tuple(toks[::-1]))
    assert got == [p[3] for p in kept]


def test_t4_invariants_on_random_trees():
    rng = np.random.default_rng(4)
    B, D, V, W, budget = 3, 20, 500, 7, 128
    logp = _logp(rng, B, D, V)
    r = oracle.accum_logp_tree(logp, [1, 2, 3], W, budget)
    for b in range(B):
        par, tok, dep, sc = (r[k][b] for k in ("parent", "token", "depth", "score"))
        assert par[0] == -1 and dep[0] == 0 and sc[0] == 0.0
        for i in range(1, budget + 1):
            p = par[i]
            assert 0 <= p < i and dep[i] == dep[p] + 1
            assert tok[i] in oracle.topk_tokens(logp[b, dep[i] - 1], W)
            assert sc[i] == sc[p] + float(logp[b, dep[i] - 1, tok[i]])
        assert (np.diff(dep) >= 0).all()                      # breadth-first order
        kids = np.bincount(par[1:], minlength=budget + 1)
        assert kids.max() <= W
        # children of one parent carry distinct tokens
        for p in range(budget + 1):
            t = tok[1:][par[1:] == p]
            assert len(set(t.tolist())) == len(t)


# ---------------------------------------------------------------- path-conditioned draft head

def _path_rows(seed, V, scale=3.0, quantum=None):
    """A synthetic path-conditioned draft head: the row after a path is the
    log-softmax of normal logits seeded by (seed, b, path)."""
    cache = {}

    def row(b, path):
        key = (b,) + tuple(int(t) for t in path)
        if key not in cache:
            rng = np.random.default_rng([seed, len(key)] + list(key))
            x = scale * rng.standard_normal(V)
            if quantum:
                x = np.round(x / quantum) * quantum
            x = x - x.max()
            cache[key] = (x - np.log(np.exp(x).sum())).astype(np.float32)
        return cache[key]
    return row


GOLDEN_PATHS = json.load(open(os.path.join(HERE, "golden", "tree_build_branch_conditioned.json")))


def test_t5_hand_worked_branch_conditioned_example():
    g = GOLDEN_PATHS
    rows = {tuple(int(t) for t in k.split(",")): np.array(v, np.float32)
            for k, v in g["rows"].items()}
    asked = []

    def row(b, path):
        asked.append(tuple(path))
        return rows[tuple(path)]
    r = oracle.accum_logp_tree_paths(row, [g["root_token"]], g["levels"], g["width"], g["budget"])
    for k in ("parent", "token", "depth"):
        assert r[k][0].tolist() == g[k], k
    assert r["score"][0].tolist() == g["score"]
    assert r["frontier_src"][0].tolist() == g["frontier_src"]
    assert r["frontier_tok"][0].tolist() == g["frontier_tok"]
    # one row per frontier node of levels 0 .. depth-1, each for its own path
    assert sorted(asked) == sorted(rows)


@pytest.mark.parametrize("width,budget", [(3, 5), (4, 12), (5, 30)])
def test_t6_two_levels_path_conditioned_match_brute_force(width, budget):
    """Depth 2 prunes nothing: the candidates are every one-token path over
    the root row's top tokens and every two-token path whose second token is
    among the top tokens of the row conditioned on the first."""
    V = 40
    row = _path_rows(60 + width, V)
    root = 3

    def top(r):   # independent sort: value descending, id ascending
        return sorted(range(V), key=lambda t: (-float(r[t]), t))[:width]
    r0 = row(0, (root,))
    paths = [(float(r0[t]), 1, j, (t,)) for j, t in enumerate(top(r0))]
    for j1, t1 in enumerate(top(r0)):
        r1 = row(0, (root, t1))
        for j2, t2 in enumerate(top(r1)):
            paths.append((float(r0[t1]) + float(r1[t2]), 2, j1 * width + j2, (t1, t2)))
    kept = sorted(paths, key=lambda p: (-p[0], p[1], p[2]))[:budget]
    kept = sorted(kept, key=lambda p: (p[1], p[2]))
    r = oracle.accum_logp_tree_paths(row, [root], 2, width, budget)
    got = []
    for n in range(1, budget + 1):
        toks, i = [], n
        while i != 0:
            toks.append(int(r["token"][0, i]))
            i = int(r["parent"][0, i])
        got.append(tuple(toks[::-1]))
    assert got == [p[3] for p in kept]
    # at least one pair of level-1 nodes draws different candidates
    firsts = {p[3][0] for p in paths if p[1] == 2}
    seconds = [frozenset(p[3][1] for p in paths if p[1] == 2 and p[3][0] == f) for f in firsts]
    assert len(set(seconds)) > 1


@pytest.mark.parametrize("quantum", [None, 0.5])
def test_t7_scores_follow_the_path_conditioned_factorisation(quantum):
    """On deep random trees (with exact ties when quantised): every node's
    token is among the top tokens of the row conditioned on its parent's
    path, its score is the sum of those rows' log-probabilities along the
    path, the level frontiers name kept-or-pruned paths consistently, and
    the tree is breadth-first with distinct sibling tokens."""
    V, W, depth, budget = 300, 5, 9, 60
    row = _path_rows(70, V, quantum=quantum)
    roots = [11, 12]
    r = oracle.accum_logp_tree_paths(row, roots, depth, W, budget)
    for b in range(2):
        par, tok, dep, sc = (r[k][b] for k in ("parent", "token", "depth", "score"))
        paths = {0: (roots[b],)}
        for i in range(1, budget + 1):
            p = int(par[i])
            assert 0 <= p < i and dep[i] == dep[p] + 1
            prow = row(b, paths[p])
            assert tok[i] in oracle.topk_tokens(prow, W)
            paths[i] = paths[p] + (int(tok[i]),)
            want = sum(float(row(b, paths[i][:k])[paths[i][k]]) for k in range(1, len(paths[i])))
            assert sc[i] == want
            assert sc[i] <= sc[p]
        assert (np.diff(dep) >= 0).all()
        for p in range(budget + 1):
            t = tok[1:][par[1:] == p]
            assert len(t) <= W and len(set(t.tolist())) == len(t)
        # frontier records: rebuild each level's frontier paths from the
        # (source rank, token) pairs; their scores descend and every kept
        # node of that depth scoring above the last one is in the frontier
        front = [(roots[b],)]
        for d in range(depth):
            src, ft = r["frontier_src"][b, d], r["frontier_tok"][b, d]
            front = [front[int(s)] + (int(t),) for s, t in zip(src, ft)]
            fsc = [sum(float(row(b, f[:k])[f[k]]) for k in range(1, len(f))) for f in front]
            assert all(x >= y for x, y in zip(fsc, fsc[1:]))
            kept_d = [paths[i] for i in range(1, budget + 1) if dep[i] == d + 1]
            for pth, s in ((pth, sc[list(paths.values()).index(pth)]) for pth in kept_d):
                if s > fsc[-1]:
                    assert pth in front
