"""fp64 oracle of draft-tree construction by cumulative log-probability.
TEST INFRASTRUCTURE (see the package docstring).

The JetSpec README ("Evaluation": the tree algorithms of its reference
benchmark) names accum_logp, a breadth-first cumulative-log-probability tree
and its default, shaped by a depth, a width and a node budget (its "Quick
Start" passes tree_depth, tree_width and budget).  The pages give no more
detail; the reading written out here (listed with the other readings in the
design notes):

  * the draft head's output for sequence b is one normalised log-probability
    row per depth d = 1..depth over the vocabulary, logp[b][d-1][:];
  * the candidate tokens at depth d are the `width` largest entries of that
    row (ties to the smaller token id), best first;
  * breadth first: level 0 is the root (cumulative score 0).  Every node of
    the level-(d-1) frontier gets one child per candidate token of depth d,
    child score = parent score + logp of its token.  Children are generated
    in (frontier rank, token rank) order.  The level-d frontier is the
    `width` best children (score descending, then generation order);
  * every generated child is a candidate node; the tree keeps the root and
    the `budget` best candidates (score descending, then shallower depth,
    then generation order).  Scores never increase along a path, so the kept
    set contains the parent of every kept node;
  * node order: the root, then the kept nodes by depth and generation order
    (parents precede children).

Scores are sums of fp32 inputs accumulated in fp64: exact for these ranges,
so every comparison is exact.
"""
from __future__ import annotations

import numpy as np


def topk_tokens(row, k: int) -> np.ndarray:
    """Indices of the k largest entries, largest first, ties to smaller id."""
    row = np.asarray(row)
    order = np.lexsort((np.arange(row.shape[0]), -row.astype(np.float64)))
    return order[:k]


def accum_logp_tree(logp, root_tokens, width: int, budget: int) -> dict:
    """Trees of budget + 1 nodes for every sequence.

    logp [B][depth][V] fp32 log-probabilities; root_tokens [B].
    Returns parent, token, depth [B][budget+1] int32 and score [B][budget+1]
    (fp64 cumulative log-probability; 0 for the root).
    """
    logp = np.asarray(logp)
    B, Dmax, V = logp.shape
    N = budget + 1
    out = dict(parent=np.empty((B, N), np.int32), token=np.empty((B, N), np.int32),
               depth=np.empty((B, N), np.int32), score=np.empty((B, N), np.float64))
    for b in range(B):
        cand = [topk_tokens(logp[b, d], width) for d in range(Dmax)]
        # pool entries: (score, depth, gen, parent pool index or -1, token)
        pool = []
        frontier = [(-1, 0.0)]                      # (pool index, score) of level 0
        for d in range(1, Dmax + 1):
            level = []
            for r, (pidx, pscore) in enumerate(frontier):
                for j, tok in enumerate(cand[d - 1]):
                    s = pscore + float(logp[b, d - 1, tok])
                    level.append((s, d, r * width + j, pidx, int(tok)))
            base = len(pool)
            pool.extend(level)
            best = sorted(range(len(level)), key=lambda t: (-level[t][0], level[t][2]))[:width]
            frontier = [(base + t, level[t][0]) for t in best]
        if len(pool) < budget:
            raise ValueError("fewer candidates than the budget")
        kept = sorted(range(len(pool)), key=lambda t: (-pool[t][0], pool[t][1], t))[:budget]
        kept_set = set(kept)
        order = sorted(kept, key=lambda t: (pool[t][1], t))      # depth, generation
        node_of = {t: n + 1 for n, t in enumerate(order)}
        out["parent"][b, 0], out["token"][b, 0] = -1, int(root_tokens[b])
        out["depth"][b, 0], out["score"][b, 0] = 0, 0.0
        for n, t in enumerate(order, start=1):
            s, d, _, pidx, tok = pool[t]
            if pidx >= 0 and pidx not in kept_set:
                raise AssertionError("kept set not closed under parents")
            out["parent"][b, n] = 0 if pidx < 0 else node_of[pidx]
            out["token"][b, n] = tok
            out["depth"][b, n] = d
            out["score"][b, n] = s
    return out
