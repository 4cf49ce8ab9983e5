"""The allocation-free LM head (tv_lmhead_argmax_noalloc) through the C ABI
against tv_lmhead_argmax with a workspace of its own: argmax and logits bit
for bit, on calls in a row whose second input is smaller (the device array
keeps the previous call's contents), across the dtypes and layouts, and a
shape beyond the array rejected with TV_ESCRATCH before anything runs."""
import ctypes

import numpy as np
import pytest

from workloads import WORKLOADS, lmhead_inputs

from _helpers import to_dev

pytestmark = pytest.mark.gpu

Q8 = WORKLOADS["qwen3_8b_L1024_N64"]


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _pair(wl, packed):
    """(argmax, logits) of the allocation-free call and of the workspace call."""
    import torch
    import tree_draft_verification_amd as tv
    from tree_draft_verification_amd import _lib
    lib = tv._lib_handle()
    lm = lmhead_inputs(wl)
    h = to_dev(lm["hidden"], wl.dtype)
    w = to_dev(lm["w"], wl.dtype)
    dt = _lib.TV_BF16 if wl.dtype == "bf16" else _lib.TV_F32
    layout = _lib.TV_LAYOUT_PACKED if packed else _lib.TV_LAYOUT_ROWMAJOR
    wt = tv.tv_lmhead_pack_weights(w) if packed else w
    wptr = _ptr(wt.data if packed else wt)
    M, K = h.shape
    V = w.shape[0]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for noalloc in (True, False):
        arg = torch.full((M,), -7, dtype=torch.int32, device="cuda")
        logits = torch.full((M, V), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            st = lib.tv_lmhead_argmax_noalloc(_ptr(h), wptr, _ptr(arg), _ptr(logits), M, K, V, dt,
                                              layout, stream)
        else:
            ws = torch.zeros(tv.tv_lmhead_argmax_workspace(M, K, V, dt), dtype=torch.uint8,
                             device="cuda")
            st = lib.tv_lmhead_argmax(_ptr(h), wptr, _ptr(arg), _ptr(logits), M, K, V, dt, layout,
                                      _ptr(ws), ws.numel(), stream)
        assert st == 0, tv.tv_status_string(st)
        # the argmax alone (no logits), as the verification step calls it
        arg2 = torch.full((M,), -7, dtype=torch.int32, device="cuda")
        if noalloc:
            st = lib.tv_lmhead_argmax_noalloc(_ptr(h), wptr, _ptr(arg2), None, M, K, V, dt,
                                              layout, stream)
            assert st == 0, tv.tv_status_string(st)
        torch.cuda.synchronize()
        if noalloc:
            assert torch.equal(arg, arg2)
        out.append((arg.cpu().numpy(), logits.cpu().numpy()))
    return out


# each sequence: calls in a row on the shared device array, larger first
SEQUENCES = {
    "bf16_packed_300_then_40": [(Q8.replace(B=1, N=300, hidden=512, V=5000, seed=71), True),
                                (Q8.replace(B=1, N=40, hidden=512, V=5000, seed=72), True)],
    "bf16_rowmajor_130_then_17": [(Q8.replace(B=1, N=130, hidden=256, V=3001, seed=73), False),
                                  (Q8.replace(B=1, N=17, hidden=256, V=3001, seed=74), False)],
    "bf16_600_then_f32_50": [(Q8.replace(B=1, N=600, hidden=256, V=2000, seed=75), True),
                             (Q8.replace(B=1, N=50, hidden=96, V=777, dtype="f32", seed=76), False)],
}


@pytest.mark.parametrize("name", list(SEQUENCES))
def test_noalloc_lmhead_equals_the_workspace_call(name):
    for wl, packed in SEQUENCES[name]:
        print(f"[noalloc] {name}: M={wl.M} K={wl.hidden} V={wl.V} {wl.dtype} "
              f"{'packed' if packed else 'row-major'}", flush=True)
        (a1, l1), (a2, l2) = _pair(wl, packed)
        np.testing.assert_array_equal(a1, a2)
        np.testing.assert_array_equal(l1.view(np.uint32), l2.view(np.uint32))
        assert (a1 >= 0).all() and (a1 < wl.V).all()


def test_noalloc_lmhead_rejects_shapes_beyond_its_array():
    import torch
    import tree_draft_verification_amd as tv
    from tree_draft_verification_amd import _lib
    lib = tv._lib_handle()
    M, K, V = 8192, 2048, 151936            # 8192 rows of partial keys exceed 64 MiB
    assert tv.tv_lmhead_argmax_workspace(M, K, V, _lib.TV_BF16) > _lib.TV_NOALLOC_SCRATCH_BYTES
    arg = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    fake = ctypes.c_void_p(0x1000)           # never dereferenced: rejected on the host
    st = lib.tv_lmhead_argmax_noalloc(fake, fake, _ptr(arg), None, M, K, V, _lib.TV_BF16,
                                      _lib.TV_LAYOUT_PACKED, None)
    assert st == _lib.TV_ESCRATCH
    assert "allocation-free" in tv.tv_status_string(st)
    torch.cuda.synchronize()
    assert (arg.cpu().numpy() == -7).all()
