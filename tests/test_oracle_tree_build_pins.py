"""Pins of the draft-tree construction oracle (oracle.tree_build): a
hand-worked example, the width-1 chain, brute-force enumeration where no
level is pruned, and invariants on random inputs."""
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
