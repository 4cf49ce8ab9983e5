"""Shared helpers of the parity tests: host<->device copies and tolerances."""
from __future__ import annotations

import numpy as np

# Tolerances of the GPU path against the fp64 oracle.
ATTN_MAX_ABS = 2e-2     # attention output, max |delta|
ATTN_REL_L2 = 1e-2      # attention output, ||delta|| / ||ref||
LOGITS_REL_L2 = 5e-3    # LM-head logits, ||delta|| / ||ref||
ARGMAX_GAP_EXEMPT = 1e-3  # argmax may differ where the oracle top-2 gap is below this


def to_dev(x: np.ndarray, dtype: str):
    import torch
    x = np.ascontiguousarray(x)
    if dtype == "bf16":
        assert x.dtype == np.uint16
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    if x.dtype == np.float32:
        return torch.from_numpy(x).cuda()
    return torch.from_numpy(x).cuda()


def i32_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def to_host_bits(t) -> np.ndarray:
    """Stored bits of a device tensor: uint16 for bf16, float32 for fp32."""
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_host_f64(t) -> np.ndarray:
    x = to_host_bits(t)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def attn_errors(got: np.ndarray, ref: np.ndarray):
    """(max |delta|, relative L2) over the entries where ref is defined."""
    sel = ~np.isnan(ref)
    d = got[sel] - ref[sel]
    return float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref[sel]))


def assert_attn_close(got, ref, what=""):
    assert not np.isnan(got[~np.isnan(ref)]).any(), f"{what}: NaN in GPU output"
    mx, rel = attn_errors(got, ref)
    assert mx <= ATTN_MAX_ABS and rel <= ATTN_REL_L2, f"{what}: max|d|={mx:.3e} rel={rel:.3e}"
    return mx, rel


def assert_argmax_ok(got_arg, ref: dict, what=""):
    """Argmax agrees with the oracle except where the oracle's top-2 gap < 1e-3."""
    got_arg = np.asarray(got_arg)
    bad = (got_arg != ref["argmax"]) & (ref["gap"] >= ARGMAX_GAP_EXEMPT)
    assert not bad.any(), (f"{what}: argmax differs at rows {np.nonzero(bad)[0][:10]} "
                           f"(gaps {ref['gap'][bad][:10]})")
    return int((got_arg != ref["argmax"]).sum())
