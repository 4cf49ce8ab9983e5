"""GPU parity of draft-tree construction against the fp64 oracle: bit-exact
trees (parent, token, depth) and fp32 scores, at the README's settings, at
the limits, and on quantised log-probabilities full of exact score ties.
tv_tree_build takes one draft row per depth; tv_tree_build_level /
tv_tree_build_finish take one row per frontier node (a path-conditioned
draft head), and their level frontiers are checked too."""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import TREE_BUILDS, PathDrafter, TreeBuildConfig, draft_logp

from _helpers import i32_dev

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))

CASES = dict(TREE_BUILDS)
CASES.update({
    "b4_d12_w8_n300_V5000": TreeBuildConfig("b4", B=4, depth=12, width=8, budget=300, V=5000,
                                            seed=11),
    "b2_d64_w8_n1023_V1000": TreeBuildConfig("d64", B=2, depth=64, width=8, budget=1023,
                                             V=1000, seed=12),
    "b2_d16_w16_n1023_V3000": TreeBuildConfig("w16", B=2, depth=16, width=16, budget=1023,
                                              V=3000, seed=13),
    "b3_d9_w1_n9_chain": TreeBuildConfig("w1", B=3, depth=9, width=1, budget=9, V=777, seed=14),
    "b3_d10_w6_n200_ties": TreeBuildConfig("ties", B=3, depth=10, width=6, budget=200, V=64,
                                           scale=1.0, quantum=0.5, seed=15),
    "b1_d2_w3_n3_V3": TreeBuildConfig("tiny", B=1, depth=2, width=3, budget=3, V=3, seed=16),
    # widest frontier with a pool under 1024 (register sort): 50 eligible
    # children per level, the most the level step handles
    "b2_d3_w16_n400_V4000": TreeBuildConfig("w16s", B=2, depth=3, width=16, budget=400, V=4000,
                                            seed=17),
    # tie-heavy log-probabilities at width 16 (equal scores across parents)
    "b2_d4_w16_n500_ties": TreeBuildConfig("w16t", B=2, depth=4, width=16, budget=500, V=300,
                                           scale=1.0, quantum=0.25, seed=18),
})


def _run(logp, root, width, budget):
    import torch
    import tree_draft_verification_amd as tv
    B, D, V = logp.shape
    lp = torch.from_numpy(np.ascontiguousarray(logp)).cuda()
    dep = torch.empty((B, budget + 1), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, budget + 1), dtype=torch.float32, device="cuda")
    par, tok = tv.tv_tree_build(lp, i32_dev(root), width, budget, node_depth=dep, score=sc)
    return par.cpu().numpy(), tok.cpu().numpy(), dep.cpu().numpy(), sc.cpu().numpy()


def _check(ref, got):
    par, tok, dep, sc = got
    np.testing.assert_array_equal(par, ref["parent"])
    np.testing.assert_array_equal(tok, ref["token"])
    np.testing.assert_array_equal(dep, ref["depth"])
    np.testing.assert_array_equal(sc.view(np.uint32),
                                  ref["score"].astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("name", list(CASES))
def test_tree_build_bit_exact(name):
    cfg = CASES[name]
    x = draft_logp(cfg)
    print(f"[tree] {name}: B={cfg.B} depth={cfg.depth} width={cfg.width} budget={cfg.budget} "
          f"V={cfg.V}", flush=True)
    ref = oracle.accum_logp_tree(x["logp"], x["root_tokens"], cfg.width, cfg.budget)
    _check(ref, _run(x["logp"], x["root_tokens"], cfg.width, cfg.budget))


def test_tree_build_hand_worked_examples():
    g = json.load(open(os.path.join(HERE, "golden", "tree_build_worked_example.json")))
    for ex in g["examples"]:
        logp = np.array(ex["logp"], dtype=np.float32)[None]
        par, tok, dep, sc = _run(logp, np.array([ex["root_token"]], np.int32), ex["width"],
                                 ex["budget"])
        assert par[0].tolist() == ex["parent"], ex["name"]
        assert tok[0].tolist() == ex["token"], ex["name"]
        assert dep[0].tolist() == ex["depth"], ex["name"]
        assert sc[0].tolist() == ex["score"], ex["name"]


def test_tree_build_trees_feed_verification():
    """Built trees are valid inputs of the accept call: with the target's
    greedy token at every node set to the token of its best-scored child,
    the GPU acceptance equals the oracle's and follows best children."""
    import tree_draft_verification_amd as tv
    cfg = TREE_BUILDS["quickstart_d20_w7_n128"]
    x = draft_logp(cfg)
    par, tok, dep, sc = _run(x["logp"], x["root_tokens"], cfg.width, cfg.budget)
    N = cfg.budget + 1
    tgt = np.zeros((1, N), np.int32)
    best = {}
    for i in range(1, N):
        p = int(par[0, i])
        if p not in best or sc[0, i] > sc[0, best[p]]:
            best[p] = i
    for p, i in best.items():
        tgt[0, p] = tok[0, i]
    acc = oracle.tree_accept(par, tok, tgt, P=32)
    path, plen, bonus = tv.tv_tree_accept(i32_dev(par), i32_dev(tok), i32_dev(tgt), 32)
    np.testing.assert_array_equal(path.cpu().numpy(), acc["path"])
    np.testing.assert_array_equal(plen.cpu().numpy(), acc["path_len"])
    n = int(acc["path_len"][0])
    assert n >= 2
    for j in range(1, n):
        assert acc["path"][0, j] == best[int(acc["path"][0, j - 1])]



# ---------------------------------------------------------------- branch-conditioned, level by level

def _run_levels(row_fn, roots, depth, width, budget, V, ws=None):
    """Drive the level calls: before each level, the draft rows of the
    current frontier's paths (as the GPU reported them) go to the device."""
    import torch
    import tree_draft_verification_amd as tv
    B = len(roots)
    if ws is None:
        ws = torch.zeros(tv.tv_tree_build_level_workspace(B, depth, V, width),
                         dtype=torch.uint8, device="cuda")
    paths = [[(int(roots[b]),)] for b in range(B)]
    fsrc = np.zeros((B, depth, width), np.int32)
    ftok = np.zeros((B, depth, width), np.int32)
    rows = np.zeros((B, width, V), np.float32)
    for level in range(1, depth + 1):
        for b in range(B):
            for r, pth in enumerate(paths[b]):
                rows[b, r] = row_fn(b, pth)
        fs, ft = tv.tv_tree_build_level(torch.from_numpy(rows).cuda(), level, depth, workspace=ws)
        fs, ft = fs.cpu().numpy(), ft.cpu().numpy()
        fsrc[:, level - 1], ftok[:, level - 1] = fs, ft
        paths = [[paths[b][int(fs[b, r])] + (int(ft[b, r]),) for r in range(width)]
                 for b in range(B)]
    dep = torch.empty((B, budget + 1), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, budget + 1), dtype=torch.float32, device="cuda")
    par, tok = tv.tv_tree_build_finish(i32_dev(np.asarray(roots, np.int32)), depth, V, width,
                                       budget, node_depth=dep, score=sc, workspace=ws)
    return (par.cpu().numpy(), tok.cpu().numpy(), dep.cpu().numpy(), sc.cpu().numpy()), fsrc, ftok


# (B, depth, width, budget, V, scale, quantum, seed)
LEVEL_CASES = {
    "quickstart_d20_w7_n128": (1, 20, 7, 128, 151936, 3.0, None, 4001),
    "b8_d20_w7_n128_V151936": (8, 20, 7, 128, 151936, 3.0, None, 4002),
    "b3_d12_w8_n300_V5000": (3, 12, 8, 300, 5000, 3.0, None, 4003),
    "b2_d16_w16_n1023_V3000": (2, 16, 16, 1023, 3000, 3.0, None, 4004),
    "b2_d64_w8_n1023_V1000": (2, 64, 8, 1023, 1000, 3.0, None, 4005),
    "b3_d9_w1_n9_chain": (3, 9, 1, 9, 777, 3.0, None, 4006),
    "b3_d10_w6_n200_ties": (3, 10, 6, 200, 64, 1.0, 0.5, 4007),
    "b2_d4_w16_n500_ties": (2, 4, 16, 500, 300, 1.0, 0.25, 4008),
    "b1_d2_w3_n3_V3": (1, 2, 3, 3, 3, 3.0, None, 4009),
}


@pytest.mark.parametrize("name", list(LEVEL_CASES))
def test_tree_build_levels_bit_exact(name):
    B, depth, W, budget, V, scale, quantum, seed = LEVEL_CASES[name]
    print(f"[tree-levels] {name}", flush=True)
    d = PathDrafter(V, seed, scale=scale, quantum=quantum)
    roots = d.roots(B)
    ref = oracle.accum_logp_tree_paths(d.row, roots, depth, W, budget)
    got, fsrc, ftok = _run_levels(d.row, roots, depth, W, budget, V)
    np.testing.assert_array_equal(fsrc, ref["frontier_src"])
    np.testing.assert_array_equal(ftok, ref["frontier_tok"])
    _check(ref, got)


def test_tree_build_levels_hand_worked_example():
    g = json.load(open(os.path.join(HERE, "golden", "tree_build_branch_conditioned.json")))
    rows = {tuple(int(t) for t in k.split(",")): np.array(v, np.float32)
            for k, v in g["rows"].items()}
    V = len(next(iter(rows.values())))
    (par, tok, dep, sc), fsrc, ftok = _run_levels(lambda b, p: rows[tuple(p)], [g["root_token"]],
                                                  g["levels"], g["width"], g["budget"], V)
    assert par[0].tolist() == g["parent"]
    assert tok[0].tolist() == g["token"]
    assert dep[0].tolist() == g["depth"]
    assert sc[0].tolist() == g["score"]
    assert fsrc[0].tolist() == g["frontier_src"]
    assert ftok[0].tolist() == g["frontier_tok"]


@pytest.mark.parametrize("name", ["quickstart_d20_w7_n128", "b3_d10_w6_n200_ties"])
def test_tree_build_levels_with_depth_rows_equal_the_one_launch_build(name):
    """A draft head whose row depends only on the depth: the level calls give
    the one-launch tv_tree_build's tree."""
    cfg = CASES[name]
    x = draft_logp(cfg)
    one = _run(x["logp"], x["root_tokens"], cfg.width, cfg.budget)
    lv, _, _ = _run_levels(lambda b, p: x["logp"][b, len(p) - 1], x["root_tokens"], cfg.depth,
                           cfg.width, cfg.budget, cfg.V)
    for a, c in zip(one, lv):
        np.testing.assert_array_equal(a, c)


def test_tree_build_levels_restart_and_two_sizes():
    """A workspace reused for a second tree (level 1 starts over) after a
    larger one: the second tree is the oracle's."""
    import torch
    import tree_draft_verification_amd as tv
    d1 = PathDrafter(2000, 4010)
    d2 = PathDrafter(2000, 4011, quantum=0.5, scale=1.0)
    ws = torch.zeros(tv.tv_tree_build_level_workspace(2, 12, 2000, 8), dtype=torch.uint8,
                     device="cuda")
    assert ws.numel() >= tv.tv_tree_build_level_workspace(2, 5, 2000, 4)
    for d, (depth, W, budget) in ((d1, (12, 8, 200)), (d2, (5, 4, 40))):
        roots = d.roots(2)
        ref = oracle.accum_logp_tree_paths(d.row, roots, depth, W, budget)
        got, fsrc, ftok = _run_levels(d.row, roots, depth, W, budget, 2000, ws=ws)
        np.testing.assert_array_equal(ftok, ref["frontier_tok"])
        _check(ref, got)
