"""GPU parity of the multi-layer verification pass against the fp64 oracle
(oracle.model), of the one-launch multi-layer compaction, and of graph
replay of the whole step against its eager run."""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import MODEL_CASES, MODELS, WORKLOADS, model_inputs, model_weights

from _helpers import i32_dev, to_dev, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu

# Tolerances of the pass (bf16 activations between kernels, fp32 accumulation)
# against the fp64 oracle.  tests/golden/model_tolerance.json holds, per case,
# how far the oracle itself moves when every activation the pass stores is
# rounded to bf16 (oracle.verify_pass(..., bf16_points=True), written by
# tests/golden/make_model_tolerance.py).  The GPU pass carries rounding noise
# of that size in another realisation, plus fp32 accumulation terms orders of
# magnitude smaller: its rel-L2 distances may be up to REL_MARGIN times the
# model's.  A greedy token may differ from the oracle's only if the token the
# GPU picked has an exact logit within twice the largest logit change the GPU
# may make (REL_MARGIN times the model's) of the exact maximum: a flip needs
# the two logits to move apart by their gap.
REL_MARGIN = 2.0
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                       "model_tolerance.json")) as _f:
    TOL = json.load(_f)


def _bounds(name):
    t = TOL[name]
    return dict(hidden=REL_MARGIN * t["hidden_rel_l2"], cache=REL_MARGIN * t["cache_rel_l2"],
                logits=REL_MARGIN * t["logits_rel_l2"],
                gap=2 * REL_MARGIN * t["logit_max_abs_change"])


CASES = {k: v for k, v in MODEL_CASES.items() if v[0] != "qwen3_8b"}


def _bad_argmax(got, ref, bound):
    """Rows whose GPU token differs from the oracle's and whose exact logit is
    further than ``bound`` below the exact maximum (ref holds every row's
    logits)."""
    rows = np.arange(len(got))
    picked = ref["logits"][rows, got]
    return (got != ref["argmax"]) & (picked < ref["top1"] - bound)


def _tree_rows(cache, seq_lens, N):
    return np.concatenate([cache[:, b, :, int(L):int(L) + N].ravel()
                           for b, L in enumerate(seq_lens)])


def _cache_rel(gk, gv, ref, x, N):
    return max(_rel(_tree_rows(gk, x["seq_lens"], N), _tree_rows(ref["k_cache"], x["seq_lens"], N)),
               _rel(_tree_rows(gv, x["seq_lens"], N), _tree_rows(ref["v_cache"], x["seq_lens"], N)))


def _dims_torch(cfg):
    return cfg.dims()


def _model_dev(cfg, w):
    import tree_draft_verification_amd as tv
    wd = {k: to_dev(v, "bf16") for k, v in w.items()}
    return tv.tv_model_pack(cfg.dims(), wd)


def _rel(a, b):
    sel = ~np.isnan(b)
    return float(np.linalg.norm(a[sel] - b[sel]) / np.linalg.norm(b[sel]))


def _run_pass(model, x, wl, logits=True):
    import torch
    import tree_draft_verification_amd as tv
    k, v = to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16")
    M = wl.B * wl.N
    lg = torch.empty((M, model.dims["V"]), dtype=torch.float32, device="cuda") if logits else None
    hid = torch.empty((M, model.dims["hidden"]), dtype=torch.float32, device="cuda")
    st = torch.zeros(wl.B, dtype=torch.int32, device="cuda")
    arg = tv.tv_verify_pass(model, i32_dev(x["tokens"]), i32_dev(x["parent"]),
                            i32_dev(x["seq_lens"]), k, v, max_seq_len=int(x["seq_lens"].max()),
                            logits=lg, hidden_out=hid, dev_status=st)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [0] * wl.B
    return arg, lg, hid, k, v


@pytest.mark.parametrize("name", list(CASES))
def test_pass_matches_oracle(name):
    mname, wl = CASES[name]
    cfg = MODELS[mname]
    w = model_weights(cfg)
    x = model_inputs(cfg, wl)
    print(f"[pass] {name}: layers={cfg.layers} hidden={cfg.hidden} B={wl.B} N={wl.N} "
          f"L={list(x['seq_lens'])}", flush=True)
    model = _model_dev(cfg, w)
    arg, lg, hid, k, v = _run_pass(model, x, wl)
    ref = oracle.verify_pass(cfg.dims(), w, x["tokens"], x["parent"], x["seq_lens"],
                             x["k_cache"], x["v_cache"])
    bd = _bounds(name)
    rl = _rel(lg.cpu().numpy().astype(np.float64), ref["logits"])
    rh = _rel(hid.cpu().numpy().astype(np.float64), ref["hidden"])
    gk, gv = to_host_f64(k), to_host_f64(v)
    rc = _cache_rel(gk, gv, ref, x, wl.N)
    got = arg.cpu().numpy()
    bad = _bad_argmax(got, ref, bd["gap"])
    print(f"[pass] {name}: logits rel={rl:.2e} hidden rel={rh:.2e} cache rel={rc:.2e} "
          f"argmax diffs={(got != ref['argmax']).sum()} (non-exempt {bad.sum()}); bounds {bd}",
          flush=True)
    assert rl <= bd["logits"] and rh <= bd["hidden"] and rc <= bd["cache"]
    assert not bad.any(), f"argmax differs at rows {np.nonzero(bad)[0]}"
    # rows the pass must not touch: prefix bits and the NaN rows past the tree
    kb = to_host_bits(k)
    for b in range(wl.B):
        L = int(x["seq_lens"][b])
        np.testing.assert_array_equal(kb[:, b, :, :L], x["k_cache"][:, b, :, :L])
        np.testing.assert_array_equal(kb[:, b, :, L + wl.N:], x["k_cache"][:, b, :, L + wl.N:])


def test_pass_flags_bad_tokens_and_trees():
    import torch
    import tree_draft_verification_amd as tv
    mname, wl = CASES["tiny_d64_B2_ragged"]
    cfg = MODELS[mname]
    x = model_inputs(cfg, wl)
    model = _model_dev(cfg, model_weights(cfg))
    tokens = x["tokens"].copy()
    tokens[0, 3] = cfg.V                       # out of the vocabulary
    parent = x["parent"].copy()
    parent[1, 4] = 7                           # parent[i] >= i
    st = torch.zeros(wl.B, dtype=torch.int32, device="cuda")
    k, v = to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16")
    tv.tv_verify_pass(model, i32_dev(tokens), i32_dev(parent), i32_dev(x["seq_lens"]), k, v,
                      max_seq_len=int(x["seq_lens"].max()), dev_status=st)
    torch.cuda.synchronize()
    s = st.cpu().tolist()
    assert s[0] == tv.TV_STATUS_BAD_TOKEN
    assert s[1] & tv.TV_STATUS_BAD_PARENT
    # a flagged sequence's outputs are unspecified, but nothing outside its
    # tree rows is ever written
    kb = to_host_bits(k)
    L = int(x["seq_lens"][1])
    np.testing.assert_array_equal(kb[:, 1, :, :L], x["k_cache"][:, 1, :, :L])
    np.testing.assert_array_equal(kb[:, 1, :, L + wl.N:], x["k_cache"][:, 1, :, L + wl.N:])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_compact_layers_bit_exact_and_reusable(dtype):
    import torch
    import tree_draft_verification_amd as tv
    rng = np.random.default_rng(71)
    Ly, B, Hkv, Lcap, D, P = 5, 3, 4, 96, 64 if dtype == "f32" else 128, 16
    if dtype == "bf16":
        kc = rng.integers(0, 65535, size=(Ly, B, Hkv, Lcap, D)).astype(np.uint16)
        vc = rng.integers(0, 65535, size=(Ly, B, Hkv, Lcap, D)).astype(np.uint16)
    else:
        kc = rng.standard_normal((Ly, B, Hkv, Lcap, D)).astype(np.float32)
        vc = rng.standard_normal((Ly, B, Hkv, Lcap, D)).astype(np.float32)
    lens = np.array([5, 30, 0], np.int32)
    path = np.full((B, P), -1, np.int32)
    path[0, :6] = [0, 2, 4, 6, 8, 9]
    path[1, :16] = np.concatenate([[0], np.arange(1, 16) + 20])
    path[2, :1] = [0]
    plen = np.array([6, 16, 1], np.int32)
    k2, v2, l2 = oracle.kv_compact_layers(kc, vc, lens, path, plen)
    k, v, sl = to_dev(kc, dtype), to_dev(vc, dtype), i32_dev(lens)
    ws = torch.zeros(tv.tv_kv_compact_layers_workspace(B), dtype=torch.uint8, device="cuda")
    tv.tv_kv_compact_layers(k, v, sl, i32_dev(path), i32_dev(plen), workspace=ws)
    gk, gv = to_host_bits(k), to_host_bits(v)
    if dtype == "f32":
        gk, gv, k2, v2 = (a.view(np.uint32) for a in (gk, gv, k2, v2))
    np.testing.assert_array_equal(gk, k2)
    np.testing.assert_array_equal(gv, v2)
    np.testing.assert_array_equal(sl.cpu().numpy(), l2)
    assert int(ws.sum()) == 0                  # counters left at zero
    # a second call on the same workspace (lengths advanced)
    tv.tv_kv_compact_layers(k, v, sl, i32_dev(path), i32_dev(plen), workspace=ws)
    k3, v3, l3 = oracle.kv_compact_layers(k2 if dtype == "bf16" else k2.view(np.float32),
                                          v2 if dtype == "bf16" else v2.view(np.float32),
                                          l2, path, plen)
    gk = to_host_bits(k)
    if dtype == "f32":
        gk, k3 = gk.view(np.uint32), k3.view(np.uint32)
    np.testing.assert_array_equal(gk, k3)
    np.testing.assert_array_equal(sl.cpu().numpy(), l3)
    assert int(ws.sum()) == 0


def test_compact_layers_many_planes_per_workgroup():
    """64 sequences over 32 layers of 4 KV heads: eight workgroups per
    sequence, each moving 32 planes in several rounds.  Paths whose moves
    read rows that later moves write (path[j] = 2j), long runs of moved
    rows, and random paths."""
    import torch
    import tree_draft_verification_amd as tv
    rng = np.random.default_rng(72)
    Ly, B, Hkv, Lcap, D, P = 32, 64, 4, 80, 64, 32
    kc = rng.integers(0, 65535, size=(Ly, B, Hkv, Lcap, D)).astype(np.uint16)
    vc = rng.integers(0, 65535, size=(Ly, B, Hkv, Lcap, D)).astype(np.uint16)
    lens = rng.integers(0, 8, size=B).astype(np.int32)
    path = np.full((B, P), -1, np.int32)
    plen = np.zeros(B, np.int32)
    for b in range(B):
        if b % 3 == 0:
            n = 32
            path[b, :n] = np.arange(n) * 2            # every move reads a later destination
        elif b % 3 == 1:
            n = 32
            path[b, :n] = np.concatenate([[0], np.arange(1, n) + 30])
        else:
            n = int(rng.integers(1, 33))
            path[b, :n] = np.concatenate([[0], np.sort(rng.choice(np.arange(1, 70), n - 1, replace=False))])
        plen[b] = n
    k2, v2, l2 = oracle.kv_compact_layers(kc, vc, lens, path, plen)
    k, v, sl = to_dev(kc, "bf16"), to_dev(vc, "bf16"), i32_dev(lens)
    ws = torch.zeros(tv.tv_kv_compact_layers_workspace(B), dtype=torch.uint8, device="cuda")
    tv.tv_kv_compact_layers(k, v, sl, i32_dev(path), i32_dev(plen), workspace=ws)
    np.testing.assert_array_equal(to_host_bits(k), k2)
    np.testing.assert_array_equal(to_host_bits(v), v2)
    np.testing.assert_array_equal(sl.cpu().numpy(), l2)
    assert int(ws.sum()) == 0


def test_graph_replay_of_the_whole_step_matches_eager():
    """pass -> accept -> multi-layer compaction captured once and replayed;
    every replay (restored inputs, eager work in between) is bit-identical
    to the eager step."""
    import torch
    import tree_draft_verification_amd as tv
    mname, wl = CASES["small_d128_L300_N64"]
    cfg = MODELS[mname]
    x = model_inputs(cfg, wl)
    model = _model_dev(cfg, model_weights(cfg))
    k0, v0 = to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16")
    lens0 = i32_dev(x["seq_lens"])
    k, v, lens = k0.clone(), v0.clone(), lens0.clone()
    tokens, parent = i32_dev(x["tokens"]), i32_dev(x["parent"])
    msl = int(x["seq_lens"].max())
    M, P = wl.B * wl.N, 32
    arg = torch.empty(M, dtype=torch.int32, device="cuda")
    path = torch.empty((wl.B, P), dtype=torch.int32, device="cuda")
    plen = torch.empty(wl.B, dtype=torch.int32, device="cuda")
    bonus = torch.empty(wl.B, dtype=torch.int32, device="cuda")
    ws = torch.zeros(tv.tv_verify_pass_workspace(model, wl.B, wl.N, msl), dtype=torch.uint8,
                     device="cuda")
    cws = torch.zeros(tv.tv_kv_compact_layers_workspace(wl.B), dtype=torch.uint8, device="cuda")

    def step():
        tv.tv_verify_pass(model, tokens, parent, lens, k, v, arg, max_seq_len=msl, workspace=ws)
        tv.tv_tree_accept(parent, tokens, arg, P, path=path, path_len=plen, bonus=bonus)
        tv.tv_kv_compact_layers(k, v, lens, path, plen, workspace=cws)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    s.synchronize()
    want = [t.clone() for t in (arg, path, plen, bonus, k, v, lens)]
    with torch.cuda.stream(s):
        k.copy_(k0), v.copy_(v0), lens.copy_(lens0)
        s.synchronize()
        tv.tv_graph_begin(s)
        step()
        g = tv.tv_graph_end(s)
    for rep in range(3):
        with torch.cuda.stream(s):
            k.copy_(k0), v.copy_(v0), lens.copy_(lens0)
            arg.fill_(-5)
            g.launch(s)
        s.synchronize()
        got = (arg, path, plen, bonus, k, v, lens)
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), rep
        # eager work between replays
        _ = (k0.float().sum() + 1).item()
    tv.tv_graph_destroy(g)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wname", ["qwen3_8b_L1024_N64"])
def test_pass_full_size_qwen3_8b(wname):
    """All 36 Qwen3-8B-shaped layers over the full workload, every row, in
    the launch configuration the benchmark times."""
    import time
    mname, wl = MODEL_CASES[wname]
    cfg = MODELS[mname]
    bd = _bounds(wname)
    t0 = time.time()
    w = model_weights(cfg)
    x = model_inputs(cfg, wl)
    print(f"[pass-full] {wname}: inputs drawn in {time.time() - t0:.0f} s", flush=True)
    model = _model_dev(cfg, w)
    arg, lg, hid, k, v = _run_pass(model, x, wl, logits=False)
    gk, gv, got_h, got = to_host_f64(k), to_host_f64(v), hid.cpu().numpy(), arg.cpu().numpy()
    del model, k, v
    print(f"[pass-full] {wname}: GPU pass done at {time.time() - t0:.0f} s", flush=True)
    ref = oracle.verify_pass(cfg.dims(), w, x["tokens"], x["parent"], x["seq_lens"],
                             x["k_cache"], x["v_cache"])
    print(f"[pass-full] {wname}: oracle done at {time.time() - t0:.0f} s", flush=True)
    rh = _rel(got_h.astype(np.float64), ref["hidden"])
    rc = _cache_rel(gk, gv, ref, x, wl.N)
    bad = _bad_argmax(got, ref, bd["gap"])
    print(f"[pass-full] {wname}: hidden rel={rh:.2e} cache rel={rc:.2e} argmax diffs="
          f"{(got != ref['argmax']).sum()} (non-exempt {bad.sum()}), min gap "
          f"{ref['gap'].min():.3e}; bounds {bd}", flush=True)
    assert rh <= bd["hidden"] and rc <= bd["cache"]
    assert not bad.any()


def test_pass_workspace_needs_no_initial_contents():
    """One workspace, filled with 0xFF bytes, serves passes of different
    shapes in turn (small then larger row counts and back)."""
    import torch
    import tree_draft_verification_amd as tv
    runs = []
    for name in ("small_d128_L300_N64", "small_d128_B3_N40_M120", "small_d128_L300_N64"):
        mname, wl = CASES[name]
        cfg = MODELS[mname]
        runs.append((name, cfg, wl, model_weights(cfg), model_inputs(cfg, wl)))
    model = _model_dev(runs[0][1], runs[0][3])
    need = max(tv.tv_verify_pass_workspace(model, wl.B, wl.N, int(x["seq_lens"].max()))
               for _, _, wl, _, x in runs)
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    for name, cfg, wl, w, x in runs:
        k, v = to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16")
        arg = tv.tv_verify_pass(model, i32_dev(x["tokens"]), i32_dev(x["parent"]),
                                i32_dev(x["seq_lens"]), k, v,
                                max_seq_len=int(x["seq_lens"].max()), workspace=ws)
        ref = oracle.verify_pass(cfg.dims(), w, x["tokens"], x["parent"], x["seq_lens"],
                                 x["k_cache"], x["v_cache"])
        got = arg.cpu().numpy()
        bad = _bad_argmax(got, ref, _bounds(name)["gap"])
        assert not bad.any(), f"{wl.B}x{wl.N}: argmax differs at rows {np.nonzero(bad)[0]}"
