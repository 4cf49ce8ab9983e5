"""fp64 oracle of draft-tree construction by cumulative log-probability.
TEST INFRASTRUCTURE (see the package docstring).

The JetSpec README ("Evaluation": the tree algorithms of its reference
benchmark) names accum_logp, a breadth-first cumulative-log-probability tree
and its default, shaped by a depth, a width and a node budget (its "Quick
Start" passes tree_depth, tree_width and budget).  The JetSpec abstract says
what the scores are: the causal parallel draft head conditions every branch
on its own path ("branch-wise causal conditioning", as opposed to
"branch-agnostic marginals"), so that a tree's scores follow the target's
autoregressive factorisation.  The reading written out here (listed with the
other readings in the design notes):

  * the draft head's output for a tree node is one normalised
    log-probability row over the vocabulary for the token that follows that
    node's root path: next_logp(b, path), path = the tokens from the root
    (the last accepted token) to the node;
  * the candidate tokens below a node are the `width` largest entries of
    its row (ties to the smaller token id), best first;
  * breadth first: level 0 is the root (cumulative score 0).  Every node of
    the level-(d-1) frontier gets one child per candidate token of its own
    row, child score = parent score + that row's log-probability of the
    token, i.e. the sum of log p(token_k | path before k) along the path.
    Children are generated in (frontier rank, token rank) order.  The
    level-d frontier is the `width` best children (score descending, then
    generation order);
  * every generated child is a candidate node; the tree keeps the root and
    the `budget` best candidates (score descending, then shallower depth,
    then generation order).  Log-probabilities are <= 0, so scores never
    increase along a path and the kept set contains the parent of every
    kept node;
  * node order: the root, then the kept nodes by depth and generation order
    (parents precede children).

A draft head whose row depends only on the depth (the same row for every
branch) is the special case accum_logp_tree(logp[B][depth][V]).

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


def accum_logp_tree_paths(next_logp, root_tokens, depth: int, width: int,
                          budget: int) -> dict:
    """Trees of budget + 1 nodes for every sequence, from a path-conditioned
    draft head.

    next_logp(b, path) returns the fp32 row [V] of normalised log-
    probabilities of the token after `path` (a tuple of token ids, root
    token first) in sequence b; it is called once per frontier node.
    Returns parent, token, depth [B][budget+1] int32, score [B][budget+1]
    (fp64 cumulative log-probability; 0 for the root), and the frontier of
    every level: frontier_src [B][depth][width] (the rank, in the previous
    level's frontier, of each new frontier node's parent; 0 at level 1) and
    frontier_tok [B][depth][width] (its token), best first.
    """
    root_tokens = [int(t) for t in root_tokens]
    B = len(root_tokens)
    N = budget + 1
    out = dict(parent=np.empty((B, N), np.int32), token=np.empty((B, N), np.int32),
               depth=np.empty((B, N), np.int32), score=np.empty((B, N), np.float64),
               frontier_src=np.full((B, depth, width), -1, np.int32),
               frontier_tok=np.full((B, depth, width), -1, np.int32))
    for b in range(B):
        # pool entries: (score, depth, gen, parent pool index or -1, token)
        pool = []
        frontier = [(-1, 0.0, (root_tokens[b],))]   # (pool index, score, path)
        for d in range(1, depth + 1):
            level = []                               # + (frontier rank, path)
            for r, (pidx, pscore, path) in enumerate(frontier):
                row = np.asarray(next_logp(b, path))
                for j, tok in enumerate(topk_tokens(row, width)):
                    tok = int(tok)
                    s = pscore + float(row[tok])
                    level.append((s, d, r * width + j, pidx, tok, r, path + (tok,)))
            base = len(pool)
            pool.extend(e[:5] for e in level)
            best = sorted(range(len(level)), key=lambda t: (-level[t][0], level[t][2]))[:width]
            frontier = [(base + t, level[t][0], level[t][6]) for t in best]
            for rank, t in enumerate(best):
                out["frontier_src"][b, d - 1, rank] = level[t][5]
                out["frontier_tok"][b, d - 1, rank] = level[t][4]
        if len(pool) < budget:
            raise ValueError("fewer candidates than the budget")
        kept = sorted(range(len(pool)), key=lambda t: (-pool[t][0], pool[t][1], t))[:budget]
        kept_set = set(kept)
        order = sorted(kept, key=lambda t: (pool[t][1], t))      # depth, generation
        node_of = {t: n + 1 for n, t in enumerate(order)}
        out["parent"][b, 0], out["token"][b, 0] = -1, root_tokens[b]
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


def accum_logp_tree(logp, root_tokens, width: int, budget: int) -> dict:
    """The special case of a draft head whose row depends only on the depth:
    logp [B][depth][V] fp32, row d - 1 for every node of level d - 1."""
    logp = np.asarray(logp)
    return accum_logp_tree_paths(lambda b, path: logp[b, len(path) - 1], root_tokens,
                                 logp.shape[1], width, budget)
