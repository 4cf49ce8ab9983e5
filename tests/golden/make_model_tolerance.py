"""Writes model_tolerance.json: how far a pipeline that stores its activations
in bf16 lands from the exact fp64 pass, per synthetic model and workload.

Both passes are the oracle's (oracle.verify_pass, exact and with
bf16_points=True, which rounds every activation the pass stores to bf16 where
it is produced and keeps sums and the residual stream exact).  A bf16
implementation that accumulates in fp32 carries the same rounding noise (its
realisation differs, its size does not) plus far smaller fp32 terms, so these
distances size the GPU pass's tolerances.  Nothing here runs on a GPU.

    python tests/golden/make_model_tolerance.py [case ...]

Cases are those of workloads.MODEL_CASES (default: all of them, the small
stacks of the multi-layer tests and the 36-layer Qwen3-8B-shaped model on 64
nodes over a 1024-token prefix).  Recorded per case:
rel-L2 of the final hidden states, of the written cache rows and of the
logits, and the largest absolute logit change over every row and vocabulary
entry.
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from workloads import MODEL_CASES, MODELS, model_inputs, model_weights  # noqa: E402

OUT = os.path.join(HERE, "model_tolerance.json")


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def tree_rows(cache, seq_lens, N):
    """The tree rows L_b .. L_b + N - 1 of every layer, sequence and KV head."""
    return np.concatenate([cache[:, b, :, int(L):int(L) + N].ravel()
                           for b, L in enumerate(seq_lens)])


def measure(case):
    model_name, wl = MODEL_CASES[case]
    cfg = MODELS[model_name]
    t0 = time.time()
    w = model_weights(cfg)
    x = model_inputs(cfg, wl)
    args = (cfg.dims(), w, x["tokens"], x["parent"], x["seq_lens"], x["k_cache"], x["v_cache"])
    ex = oracle.verify_pass(*args)
    rd = oracle.verify_pass(*args, bf16_points=True)
    N = x["tokens"].shape[1]
    kr = _rel(tree_rows(rd["k_cache"], x["seq_lens"], N), tree_rows(ex["k_cache"], x["seq_lens"], N))
    vr = _rel(tree_rows(rd["v_cache"], x["seq_lens"], N), tree_rows(ex["v_cache"], x["seq_lens"], N))
    dl = np.abs(rd["logits"] - ex["logits"])
    rec = {
        "model": model_name, "layers": cfg.layers, "rows": int(ex["hidden"].shape[0]),
        "hidden_rel_l2": _rel(rd["hidden"], ex["hidden"]),
        "cache_rel_l2": max(kr, vr),
        "logits_rel_l2": _rel(rd["logits"], ex["logits"]),
        "logit_max_abs_change": float(dl.max()),
        "logit_rms_change": float(np.sqrt(np.mean(dl * dl))),
        "argmax_changes": int((rd["argmax"] != ex["argmax"]).sum()),
        "min_top2_gap": float(ex["gap"].min()),
    }
    print(f"{case} {rec} ({time.time() - t0:.0f} s)", flush=True)
    return rec


def main(cases):
    table = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            table = json.load(f)
    for c in cases:
        table[c] = measure(c)
        with open(OUT, "w") as f:
            json.dump(table, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:] or list(MODEL_CASES))
