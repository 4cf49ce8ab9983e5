"""fp64 oracle functions (test infrastructure; see the package docstring).

Readings of points the pages leave open (each one is listed in the design
notes with its justification):
  * softmax scale is a caller argument (1/sqrt(D) by default);
  * query head h reads KV head h // (Hq/Hkv) (contiguous GQA groups);
  * node 0 is the last accepted token; its K/V sit at cache row L_b, it sees
    the prefix and itself, and it is always accepted;
  * nodes are topologically ordered (parent[i] < i, parent[0] = -1) and the
    tree rows of sequence b are cache rows L_b .. L_b+N-1 in node order;
  * the accepted path is the deepest node whose whole root path matches the
    target's greedy tokens, ties to the smallest node index; the bonus token
    is the target's greedy token at that node;
  * argmax ties go to the smallest vocabulary index.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# input decoding

def decode(x, dtype: str) -> np.ndarray:
    """Exact fp64 value of stored inputs: bf16 bit patterns (uint16), fp32, or
    values already in fp64 (dtype "f64")."""
    x = np.asarray(x)
    if dtype == "bf16":
        if x.dtype != np.uint16:
            raise TypeError("bf16 inputs are expected as uint16 bit patterns")
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype in ("f32", "f64"):
        return x.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_bf16(x) -> np.ndarray:
    """The fp64 value of x stored as bf16: binary32's sign, exponent and top 7
    fraction bits, rounded to nearest with ties to even (x is first rounded
    to binary32).  Not used by the functions below unless a caller asks for a
    model of bf16 storage (``p_round`` and the pass's ``bf16_points``), which
    only sizes tolerances."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    finite = np.isfinite(f)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    r = np.where(finite, r, u & 0xFFFF0000)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# tree topology

def ancestors(parent_row, i: int) -> list[int]:
    """Node i and every ancestor up to the root, by walking parent pointers.

    The draft tree is topologically ordered: parent[0] == -1 and
    0 <= parent[j] < j for j >= 1.
    """
    out = [i]
    j = i
    while j != 0:
        p = int(parent_row[j])
        if not 0 <= p < j:
            raise ValueError(f"malformed tree: parent[{j}] = {p}")
        out.append(p)
        j = p
    if int(parent_row[0]) != -1:
        raise ValueError("malformed tree: parent[0] must be -1")
    return out


# ----------------------------------------------------------------------------
# step 1: tree-causal attention

def tree_attention(q, k_cache, v_cache, seq_lens, parent, scale, dtype,
                   node_chunk: int = 128, nodes=None, p_round=None) -> np.ndarray:
    """Output of every (sequence b, node i, query head h), in fp64.

    Definition (JetSpec GitHub README, "JetSpec > Overview": the whole tree
    is verified in one forward pass under a tree-causal mask): node i of
    sequence b sees the prefix keys, cache rows 0..L_b-1, and the tree keys
    of its own root path, cache rows L_b + j for j in ancestors(i) (i itself
    included).  With s_t = scale * q.k_t over that visible set,
        o = sum_t softmax(s)_t v_t.
    Query head h reads KV head h // G.  The prefix scores of a chunk of nodes
    are one matmul; the softmax is taken over the union of both key sets.
    ``nodes`` restricts the work to those node indices (in every sequence);
    the other outputs are left as NaN.  ``p_round``, if given, is applied to
    the unnormalised probabilities that multiply V (not to their sum): a
    model of a kernel that feeds them to the second product in a narrower
    type, used only to size tolerances.
    """
    Q = decode(q, dtype)
    K = decode(k_cache, dtype)
    Vv = decode(v_cache, dtype)
    B, N, Hq, D = Q.shape
    Hkv = K.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    out = np.full((B, N, Hq, D), np.nan)
    todo = np.arange(N) if nodes is None else np.unique(np.asarray(nodes, dtype=np.int64))
    for b in range(B):
        L = int(seq_lens[b])
        anc = {int(i): np.array(ancestors(parent[b], int(i)), dtype=np.int64) for i in todo}
        for g in range(Hkv):
            Kp, Vp = K[b, g, :L], Vv[b, g, :L]
            for c0 in range(0, len(todo), node_chunk):
                sel = todo[c0:c0 + node_chunk]
                Qc = Q[b, sel, g * G:(g + 1) * G, :]            # [n, G, D]
                s_pre = (Qc @ Kp.T) * scale                       # [n, G, L]
                for n, i in enumerate(sel):
                    i = int(i)
                    rows = L + anc[i]
                    Ka, Va = K[b, g, rows], Vv[b, g, rows]        # [a, D]
                    s_anc = (Q[b, i, g * G:(g + 1) * G] @ Ka.T) * scale  # [G, a]
                    sp = s_pre[n]
                    m = np.maximum(sp.max(axis=1) if L else -np.inf,
                                   s_anc.max(axis=1))[:, None]
                    p_pre = np.exp(sp - m)
                    p_anc = np.exp(s_anc - m)
                    den = p_pre.sum(axis=1) + p_anc.sum(axis=1)
                    if p_round is not None:
                        p_pre, p_anc = p_round(p_pre), p_round(p_anc)
                    o = p_pre @ Vp + p_anc @ Va
                    out[b, i, g * G:(g + 1) * G] = o / den[:, None]
    return out


# ----------------------------------------------------------------------------
# step 2: LM head + argmax

def lm_logits(hidden, w, dtype, rows=None) -> np.ndarray:
    """logits[r][v] = sum_k hidden[r][k] * w[v][k] in fp64 (small cases)."""
    H = decode(hidden if rows is None else np.asarray(hidden)[rows], dtype)
    return H @ decode(w, dtype).T


def lm_head_argmax(hidden, w, dtype, rows=None, v_chunk: int = 8192) -> dict:
    """Greedy (temperature 0) token of every row, from fp64 logits.

    The accepted path must follow the target's own logits (JetSpec GitHub
    README, "JetSpec > Overview"); at temperature 0 (the README's quick-start
    examples) the target's token is the argmax, ties to the smallest index.
    Also returns the top-1 value and the gap to the best other index, which
    the GPU comparison uses to exempt near-ties.  Streams the vocabulary in
    chunks so that fp64 copies of a 150k x 4k matrix are never formed whole.
    """
    H = decode(hidden if rows is None else np.asarray(hidden)[rows], dtype)
    M = H.shape[0]
    V = np.asarray(w).shape[0]
    best = np.full(M, -np.inf)
    second = np.full(M, -np.inf)
    arg = np.zeros(M, dtype=np.int64)
    ar = np.arange(M)
    for v0 in range(0, V, v_chunk):
        v1 = min(V, v0 + v_chunk)
        lg = H @ decode(np.asarray(w)[v0:v1], dtype).T      # [M, v1-v0]
        ci = np.argmax(lg, axis=1)                         # first max in chunk
        c1 = lg[ar, ci]
        if v1 - v0 >= 2:
            c2 = np.partition(lg, -2, axis=1)[:, -2]       # 2nd largest value
        else:
            c2 = np.full(M, -np.inf)
        take = c1 > best                                   # earlier chunk wins ties
        new_second = np.where(take, np.maximum(best, c2), np.maximum(second, c1))
        best = np.where(take, c1, best)
        arg = np.where(take, ci + v0, arg)
        second = new_second
    return dict(argmax=arg.astype(np.int32), top1=best, top2=second,
                gap=best - second)


# ----------------------------------------------------------------------------
# step 3: greedy longest-accepted-path selection + bonus token

def tree_accept(parent, draft, tgt, P: int = 32) -> dict:
    """Accepted path, its length and the bonus token of every sequence.

    A node is accepted when its parent is accepted and its draft token equals
    the target's greedy token at the parent (the root, the last accepted
    token, is always accepted).  The emitted path runs from the root to the
    deepest accepted node (smallest index on ties); the bonus token is the
    target's greedy token at that node.  Emitting token[path[1:]] + [bonus]
    reproduces step-by-step greedy decoding (JetSpec GitHub README,
    "JetSpec > Overview": lossless by construction; EQSPEC/EXSPEC abstract:
    output equivalence is the criterion).
    """
    parent = np.asarray(parent)
    draft = np.asarray(draft)
    tgt = np.asarray(tgt).reshape(parent.shape)
    B, N = parent.shape
    path = np.full((B, P), -1, dtype=np.int32)
    path_len = np.zeros(B, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    for b in range(B):
        if parent[b, 0] != -1:
            raise ValueError("malformed tree: parent[0] must be -1")
        acc = [False] * N
        depth = [0] * N
        acc[0] = True
        for i in range(1, N):
            p = int(parent[b, i])
            if not 0 <= p < i:
                raise ValueError(f"malformed tree: parent[{i}] = {p}")
            depth[i] = depth[p] + 1
            acc[i] = acc[p] and int(draft[b, i]) == int(tgt[b, p])
        best = 0
        for i in range(N):
            if acc[i] and depth[i] > depth[best]:
                best = i
        walk = ancestors(parent[b], best)[::-1]
        if len(walk) > P:
            raise ValueError("accepted path longer than P")
        path[b, :len(walk)] = walk
        path_len[b] = len(walk)
        bonus[b] = int(tgt[b, best])
    return dict(path=path, path_len=path_len, bonus=bonus)


# ----------------------------------------------------------------------------
# step 4: KV compaction

def kv_compact(k_cache, v_cache, seq_lens, path, path_len):
    """Cache after committing the accepted path (copies; inputs untouched).

    The accepted nodes' K/V move to contiguous rows right after the prefix:
    row L_b + j takes row L_b + path[j] for j < path_len, and the sequence
    length grows by path_len.  Each sequence uses its own offset L_b (the
    ragged-batch KV state of the EQSPEC/EXSPEC abstract).  Rows are moved one
    at a time in increasing j; that order never reads a row it has already
    overwritten because path[j] >= j and path is increasing.  Values are
    moved as stored bits.
    """
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    lens = np.array(seq_lens, dtype=np.int32, copy=True)
    B = k.shape[0]
    for b in range(B):
        L = int(lens[b])
        n = int(path_len[b])
        for j in range(n):
            s = int(path[b, j])
            if s != j:
                k[b, :, L + j, :] = k[b, :, L + s, :]
                v[b, :, L + j, :] = v[b, :, L + s, :]
        lens[b] = L + n
    return k, v, lens


# ----------------------------------------------------------------------------
# paged caches

def paged_to_contiguous(pages, block_table, page_size, rows):
    """Logical rows 0..rows-1 of every sequence, gathered from a page pool.

    pages [num_pages][Hkv][page_size][D]; logical row r of sequence b lives
    at pages[block_table[b][r // page_size], :, r % page_size].
    """
    pages = np.asarray(pages)
    bt = np.asarray(block_table)
    B = bt.shape[0]
    Hkv, D = pages.shape[1], pages.shape[3]
    out = np.empty((B, Hkv, rows, D), dtype=pages.dtype)
    for b in range(B):
        for r in range(rows):
            out[b, :, r, :] = pages[bt[b, r // page_size], :, r % page_size, :]
    return out


def tree_attention_paged(q, k_pages, v_pages, block_table, page_size, seq_lens, parent,
                         scale, dtype, nodes=None) -> np.ndarray:
    """tree_attention on the logical rows that a block table names."""
    rows = int(np.max(seq_lens)) + np.asarray(parent).shape[1]
    k = paged_to_contiguous(k_pages, block_table, page_size, rows)
    v = paged_to_contiguous(v_pages, block_table, page_size, rows)
    return tree_attention(q, k, v, seq_lens, parent, scale, dtype, nodes=nodes)


def kv_compact_paged(k_pages, v_pages, block_table, page_size, seq_lens, path, path_len):
    """kv_compact on paged caches: the same serial row moves, each row found
    through the block table (copies; inputs untouched)."""
    k = np.array(k_pages, copy=True)
    v = np.array(v_pages, copy=True)
    bt = np.asarray(block_table)
    lens = np.array(seq_lens, dtype=np.int32, copy=True)
    for b in range(bt.shape[0]):
        L = int(lens[b])
        n = int(path_len[b])
        for j in range(n):
            s = int(path[b, j])
            if s != j:
                ps, pd = bt[b, (L + s) // page_size], bt[b, (L + j) // page_size]
                k[pd, :, (L + j) % page_size, :] = k[ps, :, (L + s) % page_size, :]
                v[pd, :, (L + j) % page_size, :] = v[ps, :, (L + s) % page_size, :]
        lens[b] = L + n
    return k, v, lens


def kv_commit_slots(block_table, seq_lens, path, path_len, N: int):
    """Commit of the accepted path on a slot table (a block table whose pages
    hold one row each): the table entries move, not the rows.

    The serving engine keeps its KV cache in pages (JetSpec GitHub README,
    "Quick Start") and each sequence of a ragged batch keeps its own KV state
    (EQSPEC/EXSPEC abstract).  Reading used here: with one row per page, the
    compaction of kv_compact becomes a permutation of the table window
    L_b .. L_b + N - 1 of each sequence.  Position L_b + j takes the slot of
    tree node path[j] for j < path_len; the slots of the rejected nodes follow,
    in node order, at L_b + path_len .. L_b + N - 1 (free for the next tree
    rows, which need path_len more slots appended by the caller); seq_lens[b]
    grows by path_len.  Returns the new table and lengths (inputs untouched).
    """
    bt = np.array(block_table, dtype=np.int32, copy=True)
    lens = np.array(seq_lens, dtype=np.int32, copy=True)
    for b in range(bt.shape[0]):
        L = int(lens[b])
        n = int(path_len[b])
        window = [int(x) for x in bt[b, L:L + N]]
        taken = [int(path[b, j]) for j in range(n)]
        if any(not 0 <= t < N for t in taken) or any(x >= y for x, y in zip(taken, taken[1:])):
            raise ValueError(f"path of sequence {b} is not increasing within the tree")
        rejected = [window[i] for i in range(N) if i not in taken]
        new = [window[i] for i in taken] + rejected
        bt[b, L:L + N] = new
        lens[b] = L + n
    return bt, lens


# ----------------------------------------------------------------------------
# the whole step

def verify_step(att: dict, lm: dict, draft, dtype: str, P: int = 32,
                with_attention: bool = True) -> dict:
    """All four parts in order, as one verification step."""
    res = {}
    if with_attention:
        res["out"] = tree_attention(att["q"], att["k_cache"], att["v_cache"],
                                    att["seq_lens"], att["parent"],
                                    att["scale"], dtype)
    lmres = lm_head_argmax(lm["hidden"], lm["w"], dtype)
    B, N = np.asarray(att["parent"]).shape
    tgt = lmres["argmax"].reshape(B, N)
    acc = tree_accept(att["parent"], draft, tgt, P)
    k, v, lens = kv_compact(att["k_cache"], att["v_cache"], att["seq_lens"],
                            acc["path"], acc["path_len"])
    res.update(lm=lmres, tgt=tgt, accept=acc, k_cache=k, v_cache=v,
               seq_lens=lens)
    return res
