"""Seeded synthetic inputs for one tree-verification step.

What the inputs stand for (JetSpec GitHub README, "JetSpec > Overview"): a
draft head proposes a token tree, and the frozen target verifies the whole
tree in one forward pass under a tree-causal mask.  The pages measure on
public math/code/chat suites with trained draft heads; none of those are used
here.  Every tensor below is drawn from a seeded generator with the shapes of
Qwen3-style GQA layers, and draft tokens come from a simulated drafter that
copies the target's greedy token at the node's parent with a depth-dependent
probability.

Layouts (shared by every consumer):
  q        [B][N][Hq][D]            query of node i, head h
  k_cache  [B][Hkv][Lcap][D]        rows [0, L_b) prefix, [L_b, L_b+N) tree
  v_cache  same as k_cache          rows past L_b+N hold NaN on purpose
  parent   [B][N] int32             parent[b][0] = -1, parent[b][i] < i
  hidden   [B*N][hidden]            row b*N+i is node i of sequence b
  w        [V][hidden]              vocabulary projection (row per token)

bf16 tensors are returned as uint16 bit patterns; fp32 tensors as float32.

Random streams: numpy SeedSequence(seed).spawn gives one independent stream
per tensor, so drawing one tensor never shifts another.  Large normal tensors
are filled chunk by chunk (fixed chunk size, one spawned child per chunk, so
the bytes do not depend on the thread count) by mapping 16 random bits to a
quantile table of the normal law: value = bf16(std * Phi^-1((u + 0.5)/65536)).
That is a 65536-level discretisation of N(0, std^2), finer than bf16 spacing
except within about 5e-3 of zero, and it fills 1.2 GB in about a second.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BF16_QNAN = 0x7FC0
_CHUNK = 1 << 22  # elements per independently seeded chunk of a big tensor

# Stream indices of SeedSequence(seed).spawn(_NSTREAMS).
_S_TREE, _S_LENS, _S_Q, _S_K, _S_V, _S_H, _S_W, _S_COIN, _S_TOK, _S_PMATCH = range(10)
_NSTREAMS = 10


@dataclass(frozen=True)
class Workload:
    """One verification-step workload.

    tree: "binary"  - complete binary tree (N = 2^levels - 1)
          "uniform" - parent[i] uniform over earlier nodes of depth < depth_cap
          "bfs"     - breadth-first growth, each node gets U{lo..hi} children,
                      nodes at depth_cap get none, stop at N nodes
    p0, decay: a node at depth d >= 1 copies the target's greedy token at its
          parent with probability p0 * decay**(d-1).  If p0_range is set, p0
          is drawn per sequence uniformly from that range instead.
    """
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    hidden: int
    V: int
    N: int
    L_lo: int
    L_hi: int
    tree: str
    depth_cap: int
    branch_lo: int = 1
    branch_hi: int = 1
    p0: float = 0.8
    p0_range: tuple | None = None
    decay: float = 1.0
    dtype: str = "bf16"
    w_std: float = 0.02
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def M(self) -> int:
        return self.B * self.N

    @property
    def Lcap(self) -> int:
        need = self.L_hi + self.N
        return (need + 63) // 64 * 64

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: the tiny fp32 case, Qwen3-8B-shaped layers (prefix 1024
# with 64 nodes; prefix 16384 with 256 nodes; a ragged batch of 8) and
# Qwen3-30B-A3B-shaped attention with a 1024-node budget.
WORKLOADS = {
    "tiny_fp32": Workload(
        name="tiny_fp32", B=1, Hq=1, Hkv=1, D=64, hidden=64, V=1000, N=7,
        L_lo=32, L_hi=32, tree="binary", depth_cap=2, p0=0.8, dtype="f32",
        seed=1001),
    "qwen3_8b_L1024_N64": Workload(
        name="qwen3_8b_L1024_N64", B=1, Hq=32, Hkv=8, D=128, hidden=4096,
        V=151936, N=64, L_lo=1024, L_hi=1024, tree="uniform", depth_cap=16,
        p0=0.8, seed=1002),
    "qwen3_8b_L16384_N256": Workload(
        name="qwen3_8b_L16384_N256", B=1, Hq=32, Hkv=8, D=128, hidden=4096,
        V=151936, N=256, L_lo=16384, L_hi=16384, tree="bfs", depth_cap=16,
        branch_lo=1, branch_hi=4, p0=0.8, decay=0.95, seed=1003),
    "qwen3_8b_ragged8_N64": Workload(
        name="qwen3_8b_ragged8_N64", B=8, Hq=32, Hkv=8, D=128, hidden=4096,
        V=151936, N=64, L_lo=512, L_hi=8192, tree="uniform", depth_cap=12,
        p0_range=(0.5, 0.95), seed=1004),
    "qwen3_30b_a3b_B4_L4096_N1024": Workload(
        name="qwen3_30b_a3b_B4_L4096_N1024", B=4, Hq=32, Hkv=4, D=128,
        hidden=2048, V=151936, N=1024, L_lo=4096, L_hi=4096, tree="bfs",
        depth_cap=24, branch_lo=1, branch_hi=8, p0=0.8, decay=0.97,
        seed=1005),
}


# ----------------------------------------------------------------------------
# bit-level helpers (input encoding only)

def bf16_bits_from_f32(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even; NaN -> 0x7FC0."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[np.isnan(x32)] = BF16_QNAN
    return r


_TABLE_CACHE: dict = {}


def _normal_table_bf16(std: float) -> np.ndarray:
    key = ("bf16", std)
    if key not in _TABLE_CACHE:
        from scipy.special import ndtri
        u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        _TABLE_CACHE[key] = bf16_bits_from_f32((std * ndtri(u)).astype(np.float32))
    return _TABLE_CACHE[key]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_bf16(ss: np.random.SeedSequence, n: int, std: float) -> np.ndarray:
    """n bf16 draws of N(0, std^2) as uint16 bits (see module docstring)."""
    table = _normal_table_bf16(std)
    nchunks = max(1, -(-n // _CHUNK))
    kids = ss.spawn(nchunks)
    out = np.empty(n, dtype=np.uint16)

    def fill(c):
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        m = hi - lo
        raw = np.random.PCG64(kids[c]).random_raw(-(-m // 4))
        idx = raw.view(np.uint16)[:m].astype(np.intp)
        out[lo:hi] = table[idx]

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def _normal_f32(ss: np.random.SeedSequence, n: int, std: float) -> np.ndarray:
    rng = np.random.default_rng(ss)
    return (std * rng.standard_normal(n)).astype(np.float32)


def _normal(wl: Workload, ss, shape, std=1.0) -> np.ndarray:
    n = int(np.prod(shape))
    if wl.dtype == "bf16":
        return _normal_bf16(ss, n, std).reshape(shape)
    if wl.dtype == "f32":
        return _normal_f32(ss, n, std).reshape(shape)
    raise ValueError(f"unknown dtype {wl.dtype!r}")


def _streams(seed: int):
    return np.random.SeedSequence(seed).spawn(_NSTREAMS)


# ----------------------------------------------------------------------------
# trees

def _tree_binary(N: int):
    parent = np.full(N, -1, dtype=np.int32)
    depth = np.zeros(N, dtype=np.int32)
    for i in range(1, N):
        parent[i] = (i - 1) // 2
        depth[i] = depth[parent[i]] + 1
    return parent, depth


def _tree_uniform(rng, N: int, cap: int):
    parent = np.full(N, -1, dtype=np.int32)
    depth = np.zeros(N, dtype=np.int32)
    for i in range(1, N):
        cand = np.nonzero(depth[:i] < cap)[0]
        p = int(cand[rng.integers(0, len(cand))])
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent, depth


def _tree_bfs(rng, N: int, lo: int, hi: int, cap: int):
    parent = np.full(N, -1, dtype=np.int32)
    depth = np.zeros(N, dtype=np.int32)
    count = 1
    u = 0
    while count < N:
        if u >= count:
            raise ValueError("tree growth stalled below the node budget")
        if depth[u] < cap:
            k = int(rng.integers(lo, hi + 1))
            for _ in range(min(k, N - count)):
                parent[count] = u
                depth[count] = depth[u] + 1
                count += 1
        u += 1
    return parent, depth


def make_tree(wl: Workload, rng) -> tuple[np.ndarray, np.ndarray]:
    if wl.tree == "binary":
        return _tree_binary(wl.N)
    if wl.tree == "uniform":
        return _tree_uniform(rng, wl.N, wl.depth_cap)
    if wl.tree == "bfs":
        return _tree_bfs(rng, wl.N, wl.branch_lo, wl.branch_hi, wl.depth_cap)
    raise ValueError(f"unknown tree rule {wl.tree!r}")


# ----------------------------------------------------------------------------
# public generators

def attn_inputs(wl: Workload, seed: int | None = None) -> dict:
    """Inputs of the tree-attention call plus the trees (and their depths)."""
    s = _streams(wl.seed if seed is None else seed)
    rt = np.random.default_rng(s[_S_TREE])
    parent = np.empty((wl.B, wl.N), dtype=np.int32)
    depth = np.empty((wl.B, wl.N), dtype=np.int32)
    for b in range(wl.B):
        parent[b], depth[b] = make_tree(wl, rt)
    rl = np.random.default_rng(s[_S_LENS])
    if wl.L_lo == wl.L_hi:
        seq_lens = np.full(wl.B, wl.L_lo, dtype=np.int32)
    else:
        seq_lens = rl.integers(wl.L_lo, wl.L_hi + 1, size=wl.B).astype(np.int32)
    Lcap = wl.Lcap
    q = _normal(wl, s[_S_Q], (wl.B, wl.N, wl.Hq, wl.D))
    k = _normal(wl, s[_S_K], (wl.B, wl.Hkv, Lcap, wl.D))
    v = _normal(wl, s[_S_V], (wl.B, wl.Hkv, Lcap, wl.D))
    nan = BF16_QNAN if wl.dtype == "bf16" else np.float32(np.nan)
    for b in range(wl.B):
        end = int(seq_lens[b]) + wl.N
        k[b, :, end:, :] = nan
        v[b, :, end:, :] = nan
    return dict(q=q, k_cache=k, v_cache=v, seq_lens=seq_lens, parent=parent,
                depth=depth, Lcap=Lcap, scale=wl.scale)


def lmhead_inputs(wl: Workload, seed: int | None = None) -> dict:
    """Hidden states of every node (row b*N+i) and the vocab projection."""
    s = _streams(wl.seed if seed is None else seed)
    h = _normal(wl, s[_S_H], (wl.M, wl.hidden), 1.0)
    w = _normal(wl, s[_S_W], (wl.V, wl.hidden), wl.w_std)
    return dict(hidden=h, w=w)


def draft_coins(wl: Workload, depth: np.ndarray, seed: int | None = None) -> dict:
    """Random draws of the simulated drafter.

    u[b][i]        uniform [0,1) coin of node i
    rand_tok[b][i] uniform token in [0, V) used when the coin says "miss"
    p[b][i]        copy probability p0 * decay**(depth-1) (0 for the root)
    """
    s = _streams(wl.seed if seed is None else seed)
    u = np.random.default_rng(s[_S_COIN]).random((wl.B, wl.N))
    rand_tok = np.random.default_rng(s[_S_TOK]).integers(
        0, wl.V, size=(wl.B, wl.N)).astype(np.int32)
    if wl.p0_range is not None:
        p0 = np.random.default_rng(s[_S_PMATCH]).uniform(
            wl.p0_range[0], wl.p0_range[1], size=wl.B)
    else:
        p0 = np.full(wl.B, wl.p0)
    d = depth.astype(np.float64)
    p = p0[:, None] * np.power(wl.decay, np.maximum(d - 1.0, 0.0))
    p[:, 0] = 0.0
    return dict(u=u, rand_tok=rand_tok, p=p)


def draft_tokens(parent: np.ndarray, coins: dict, tgt: np.ndarray) -> np.ndarray:
    """Draft token of every node of the simulated drafter.

    token[b][0] is the last accepted token (a random id); for i >= 1 the node
    copies tgt[b][parent[b][i]] (the target's greedy token at its parent,
    supplied by the caller) when u < p, otherwise it takes rand_tok (which can
    coincide with that token by chance).
    """
    parent = np.asarray(parent)
    tgt = np.asarray(tgt).reshape(parent.shape)
    par = np.maximum(parent, 0)
    at_parent = np.take_along_axis(tgt, par, axis=1)
    copy = coins["u"] < coins["p"]
    tok = np.where(copy, at_parent, coins["rand_tok"]).astype(np.int32)
    tok[:, 0] = coins["rand_tok"][:, 0]
    return tok


def paged_layout(k_cache, v_cache, page_size: int, seed: int, extra_pages: int = 3) -> dict:
    """The same caches laid out in pages of a shared pool.

    Every sequence's logical rows 0..Lcap-1 are cut into blocks of
    page_size rows (ceil(Lcap / page_size) blocks); the blocks of all sequences are placed on pages chosen by
    a seeded random permutation of the pool, which also holds extra_pages
    unused pages filled with NaN.  Pool layout [num_pages][Hkv][page_size][D].
    """
    k_cache = np.asarray(k_cache)
    B, Hkv, Lcap, D = k_cache.shape
    nblk = -(-Lcap // page_size)      # a partial last block is padded with NaN rows
    num_pages = B * nblk + extra_pages
    perm = np.random.default_rng(seed).permutation(num_pages)
    block_table = perm[:B * nblk].reshape(B, nblk).astype(np.int32)
    nan = BF16_QNAN if k_cache.dtype == np.uint16 else np.float32(np.nan)
    pools = []
    for cache in (k_cache, np.asarray(v_cache)):
        pool = np.full((num_pages, Hkv, page_size, D), nan, dtype=cache.dtype)
        if nblk * page_size != Lcap:
            pad = np.full((B, Hkv, nblk * page_size - Lcap, D), nan, dtype=cache.dtype)
            cache = np.concatenate([cache, pad], axis=2)
        blocks = cache.reshape(B, Hkv, nblk, page_size, D).transpose(0, 2, 1, 3, 4)
        pool[block_table.reshape(-1)] = blocks.reshape(B * nblk, Hkv, page_size, D)
        pools.append(pool)
    return dict(k_pages=pools[0], v_pages=pools[1], block_table=block_table,
                page_size=page_size, num_pages=num_pages)


# ----------------------------------------------------------------------------
# draft-head log-probabilities for tree construction

@dataclass(frozen=True)
class TreeBuildConfig:
    """Tree construction from the draft head's per-depth log-probabilities
    (depth, width and budget as in the JetSpec README's "Quick Start" and
    "Evaluation" commands)."""
    name: str
    B: int
    depth: int
    width: int
    budget: int
    V: int
    scale: float = 3.0             # std of the synthetic draft logits
    quantum: float | None = None   # round logits to this step (makes exact ties)
    seed: int = 0


TREE_BUILDS = {
    "quickstart_d20_w7_n128": TreeBuildConfig("quickstart_d20_w7_n128", B=1, depth=20, width=7,
                                              budget=128, V=151936, seed=3001),
    "bench_d20_w7_n256": TreeBuildConfig("bench_d20_w7_n256", B=1, depth=20, width=7,
                                         budget=256, V=151936, seed=3002),
    "batch8_d20_w7_n128": TreeBuildConfig("batch8_d20_w7_n128", B=8, depth=20, width=7,
                                          budget=128, V=151936, seed=3003),
}


def draft_logp(cfg: TreeBuildConfig) -> dict:
    """logp [B][depth][V] fp32: log-softmax (fp64, then rounded to fp32) of
    seeded logits ~ N(0, scale^2), optionally rounded to multiples of
    `quantum` first; root_tokens [B] uniform ids.  These stand for the draft
    head's output, which lies outside the tree construction."""
    s = np.random.SeedSequence(cfg.seed).spawn(2)
    rng = np.random.default_rng(s[0])
    logits = cfg.scale * rng.standard_normal((cfg.B, cfg.depth, cfg.V))
    if cfg.quantum:
        logits = np.round(logits / cfg.quantum) * cfg.quantum
    m = logits.max(axis=-1, keepdims=True)
    lse = m + np.log(np.exp(logits - m).sum(axis=-1, keepdims=True))
    logp = (logits - lse).astype(np.float32)
    root = np.random.default_rng(s[1]).integers(0, cfg.V, size=cfg.B).astype(np.int32)
    return dict(logp=logp, root_tokens=root)


class PathDrafter:
    """A synthetic branch-conditioned draft head: the row after a token path
    (root token first) of sequence b is the log-softmax (fp64, rounded to
    fp32) of logits ~ N(0, scale^2) drawn from a generator seeded by (seed,
    b, path), optionally rounded to multiples of `quantum` first (exact
    ties).  Every branch therefore gets its own distribution, as the JetSpec
    abstract's causal parallel draft head conditions each branch on its own
    path.  It stands for the draft head's output, which lies outside tree
    construction; rows are cached per path."""

    def __init__(self, V: int, seed: int, scale: float = 3.0, quantum: float | None = None):
        self.V, self.seed, self.scale, self.quantum = V, seed, scale, quantum
        self._rows: dict = {}

    def row(self, b: int, path) -> np.ndarray:
        key = (int(b),) + tuple(int(t) for t in path)
        r = self._rows.get(key)
        if r is None:
            rng = np.random.default_rng(np.random.SeedSequence([self.seed, len(key)] + list(key)))
            x = self.scale * rng.standard_normal(self.V)
            if self.quantum:
                x = np.round(x / self.quantum) * self.quantum
            x = x - x.max()
            r = (x - np.log(np.exp(x).sum())).astype(np.float32)
            self._rows[key] = r
        return r

    def roots(self, B: int) -> np.ndarray:
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, 0xC0FFEE]))
        return rng.integers(0, self.V, size=B).astype(np.int32)
