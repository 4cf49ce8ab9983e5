"""Seeded synthetic decoder stacks for the multi-layer verification pass.

Inputs only (no arithmetic of the method): bf16 weights of a dense
Qwen3-style decoder stack, prefix key/value caches of every layer, and the
draft trees, lengths and tokens of a Workload.  Layouts follow the oracle's
model module: rows of a projection are its output features; stacked tensors
lead with the layer index; caches are [layers][B][Hkv][Lcap][D].

Weight values: projections, LM head ~ N(0, w_std^2) (w_std = 0.02, as for the
single-layer LM head); embeddings ~ N(0, 1); norm weights 1 + 0.1 N(0, 1),
so that a weight applied to the wrong element shows.  Prefix cache rows
~ N(0, 1) (keys stand for post-rotary keys of earlier tokens); tree rows and
rows past them hold NaN until the pass writes the tree rows.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .gen import (BF16_QNAN, Workload, _normal_bf16, _streams, bf16_bits_from_f32, make_tree,
                  _S_LENS, _S_TREE)


@dataclass(frozen=True)
class ModelConfig:
    name: str
    layers: int
    hidden: int
    Hq: int
    Hkv: int
    D: int
    inter: int
    V: int
    eps: float = 1e-6
    theta: float = 1e6
    w_std: float = 0.02
    lm_std: float | None = None   # LM-head std (w_std when None)
    seed: int = 0

    def dims(self, layers: int | None = None) -> dict:
        return dict(layers=self.layers if layers is None else layers, hidden=self.hidden,
                    Hq=self.Hq, Hkv=self.Hkv, D=self.D, inter=self.inter, V=self.V,
                    eps=self.eps, theta=self.theta)


# Qwen3-8B geometry (36 layers, hidden 4096, 32/8 heads of 128, MLP 12288,
# vocabulary 151936, rotary base 1e6) and two small stacks for parity tests.
MODELS = {
    "qwen3_8b": ModelConfig("qwen3_8b", layers=36, hidden=4096, Hq=32, Hkv=8, D=128,
                            inter=12288, V=151936, seed=2001),
    "tiny_d64": ModelConfig("tiny_d64", layers=2, hidden=256, Hq=4, Hkv=2, D=64, inter=512,
                            V=1000, seed=2002),
    "small_d128": ModelConfig("small_d128", layers=3, hidden=512, Hq=8, Hkv=2, D=128,
                              inter=768, V=3000, seed=2003),
    # a small stack whose larger LM head spreads the logits (std about 4.5),
    # so greedy choices are rarely near-ties: for multi-step decoding checks
    "loop_d128": ModelConfig("loop_d128", layers=3, hidden=512, Hq=8, Hkv=2, D=128,
                             inter=768, V=3000, lm_std=0.2, seed=2004),
    # a wide MLP (128 gate/up tiles of 128 rows over a short k range), the
    # shape at which the gate/up projection runs unsplit with silu(gate) * up
    # in its own epilogue, as at Qwen3-8B scale
    "wide_mlp": ModelConfig("wide_mlp", layers=2, hidden=256, Hq=2, Hkv=1, D=128, inter=8192,
                            V=1000, seed=2005),
    # one Qwen3-8B-shaped layer with a small vocabulary: the projections at
    # their full widths (QKV 6144, O 4096, gate/up 24576, down 4096 over
    # k = 12288), which from 256 rows run split-K on both W tile widths
    "qwen3_8b_layer": ModelConfig("qwen3_8b_layer", layers=1, hidden=4096, Hq=32, Hkv=8, D=128,
                                  inter=12288, V=3000, seed=2006),
}


def _model_cases():
    from .gen import WORKLOADS
    q8 = WORKLOADS["qwen3_8b_L1024_N64"]
    r8 = WORKLOADS["qwen3_8b_ragged8_N64"]
    return {
        "tiny_d64_B2_ragged": ("tiny_d64", r8.replace(B=2, Hq=4, Hkv=2, D=64, N=12, L_lo=20,
                                                      L_hi=70, seed=5)),
        "small_d128_L300_N64": ("small_d128", q8.replace(Hq=8, Hkv=2, L_lo=300, L_hi=300, seed=61)),
        "small_d128_B3_N40_M120": ("small_d128", r8.replace(B=3, Hq=8, Hkv=2, N=40, L_lo=10,
                                                            L_hi=200, seed=62)),
        # unsplit gate/up projection with the fused silu(gate) * up epilogue
        "wide_mlp_N64_L200": ("wide_mlp", q8.replace(Hq=2, Hkv=1, L_lo=200, L_hi=200, seed=63)),
        # 256 rows: one H slice (the LM head's non-temporal W loads, the
        # projections' splits with no slice group)
        "small_d128_B4_N64_M256": ("small_d128", r8.replace(B=4, Hq=8, Hkv=2, N=64, L_lo=10,
                                                            L_hi=150, seed=67)),
        # 512 and 640 rows: the products with 256-row H tiles (the last slice
        # of 640 rows half empty)
        "small_d128_B8_N64_M512": ("small_d128", r8.replace(B=8, Hq=8, Hkv=2, N=64, L_lo=10,
                                                            L_hi=120, seed=64)),
        "small_d128_B10_N64_M640": ("small_d128", r8.replace(B=10, Hq=8, Hkv=2, N=64, L_lo=10,
                                                             L_hi=90, seed=65)),
        # one full-width Qwen3-8B layer at 512 rows (8 ragged sequences of 64
        # nodes): gate/up on 384-row W tiles in 2 splits, the others on 256-row
        # tiles in 4 or 8
        "qwen3_8b_layer_B8_N64_M512": ("qwen3_8b_layer", r8.replace(B=8, N=64, L_lo=16, L_hi=200,
                                                                    seed=66)),
        # the full Qwen3-8B-shaped stack on one 64-node tree over 1024 tokens
        "qwen3_8b_L1024_N64": ("qwen3_8b", q8),
    }


# Multi-layer pass cases: name -> (model, workload).
MODEL_CASES = _model_cases()

_W_KEYS = ("embed", "ln1", "w_qkv", "q_norm", "k_norm", "w_o", "ln2", "w_gu", "w_down",
           "final_norm", "lm_head")


def _norm_weight(ss, shape):
    rng = np.random.default_rng(ss)
    return bf16_bits_from_f32((1.0 + 0.1 * rng.standard_normal(shape)).astype(np.float32))


def model_weights(cfg: ModelConfig, layers: int | None = None) -> dict:
    """bf16 bit patterns of every weight (layers: the first n layers only;
    a layer's values do not depend on how many layers are drawn)."""
    Ly = cfg.layers if layers is None else layers
    top = np.random.SeedSequence(cfg.seed).spawn(4 + cfg.layers)
    Hd, I = cfg.hidden, cfg.inter
    qkv_rows = (cfg.Hq + 2 * cfg.Hkv) * cfg.D
    w = {}
    w["embed"] = _normal_bf16(top[0], cfg.V * Hd, 1.0).reshape(cfg.V, Hd)
    lm_std = cfg.w_std if cfg.lm_std is None else cfg.lm_std
    w["lm_head"] = _normal_bf16(top[1], cfg.V * Hd, lm_std).reshape(cfg.V, Hd)
    w["final_norm"] = _norm_weight(top[2], (Hd,))
    per = {k: [] for k in ("ln1", "w_qkv", "q_norm", "k_norm", "w_o", "ln2", "w_gu", "w_down")}
    for ly in range(Ly):
        s = top[4 + ly].spawn(8)
        per["ln1"].append(_norm_weight(s[0], (Hd,)))
        per["w_qkv"].append(_normal_bf16(s[1], qkv_rows * Hd, cfg.w_std).reshape(qkv_rows, Hd))
        per["q_norm"].append(_norm_weight(s[2], (cfg.D,)))
        per["k_norm"].append(_norm_weight(s[3], (cfg.D,)))
        per["w_o"].append(_normal_bf16(s[4], Hd * cfg.Hq * cfg.D, cfg.w_std)
                          .reshape(Hd, cfg.Hq * cfg.D))
        per["ln2"].append(_norm_weight(s[5], (Hd,)))
        per["w_gu"].append(_normal_bf16(s[6], 2 * I * Hd, cfg.w_std).reshape(2 * I, Hd))
        per["w_down"].append(_normal_bf16(s[7], Hd * I, cfg.w_std).reshape(Hd, I))
    for k, v in per.items():
        w[k] = np.stack(v)
    return w


def model_inputs(cfg: ModelConfig, wl: Workload, layers: int | None = None) -> dict:
    """Trees, prefix lengths, draft tokens (uniform ids) and the prefix caches
    of every layer for one pass of ``cfg`` over ``wl``'s batch."""
    if (wl.Hq, wl.Hkv, wl.D) != (cfg.Hq, cfg.Hkv, cfg.D):
        raise ValueError("workload and model disagree on the attention geometry")
    Ly = cfg.layers if layers is None else layers
    s = _streams(wl.seed)
    rt = np.random.default_rng(s[_S_TREE])
    parent = np.empty((wl.B, wl.N), dtype=np.int32)
    depth = np.empty((wl.B, wl.N), dtype=np.int32)
    for b in range(wl.B):
        parent[b], depth[b] = make_tree(wl, rt)
    if wl.L_lo == wl.L_hi:
        seq_lens = np.full(wl.B, wl.L_lo, dtype=np.int32)
    else:
        seq_lens = np.random.default_rng(s[_S_LENS]).integers(
            wl.L_lo, wl.L_hi + 1, size=wl.B).astype(np.int32)
    Lcap = wl.Lcap
    extra = np.random.SeedSequence(wl.seed + 7919).spawn(1 + 2 * cfg.layers)
    tokens = np.random.default_rng(extra[0]).integers(0, cfg.V, size=(wl.B, wl.N)).astype(np.int32)
    shape = (wl.B, cfg.Hkv, Lcap, cfg.D)
    n = int(np.prod(shape))
    k = np.empty((Ly,) + shape, dtype=np.uint16)
    v = np.empty((Ly,) + shape, dtype=np.uint16)
    for ly in range(Ly):
        k[ly] = _normal_bf16(extra[1 + 2 * ly], n, 1.0).reshape(shape)
        v[ly] = _normal_bf16(extra[2 + 2 * ly], n, 1.0).reshape(shape)
    for b in range(wl.B):
        L = int(seq_lens[b])
        k[:, b, :, L:, :] = BF16_QNAN
        v[:, b, :, L:, :] = BF16_QNAN
    return dict(tokens=tokens, parent=parent, depth=depth, seq_lens=seq_lens, k_cache=k,
                v_cache=v, Lcap=Lcap)
