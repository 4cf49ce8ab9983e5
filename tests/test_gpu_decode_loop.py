"""Multi-step ragged speculative decoding on the GPU against independent
greedy decoding (fp64 oracle): every sequence of a ragged batch must emit
exactly the tokens plain autoregressive greedy decoding emits (output
equivalence, EQSPEC/EXSPEC abstract, arXiv 2510.22876 on the RSS reader
page; lossless by construction, JetSpec GitHub README, "JetSpec >
Overview"), with each step's trees built level by level from a
path-conditioned draft head (tv_tree_build_level / tv_tree_build_finish),
verified by the multi-layer pass, accepted and compacted per sequence at its
own length."""
import numpy as np
import pytest

import oracle
from workloads import MODELS, WORKLOADS, model_inputs, model_weights

from _helpers import i32_dev, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

GAP_EXEMPT = 5e-2   # a reference choice closer than this may legitimately differ


def _drafter_row(rng, ref_b, e_b, path, V, hit=0.9, boost=8.0):
    """The simulated draft head's row after `path` (root token first): a
    frontier node whose drafted tokens follow the reference continuation
    from emitted index e_b favours the next reference token with probability
    `hit`; any other node favours a token of its own."""
    x = rng.standard_normal(V)
    d = len(path) - 1                      # drafted tokens on the path
    on_ref = list(path[1:]) == [int(t) for t in ref_b[e_b:e_b + d]]
    i = e_b + d
    tok = ref_b[i] if (on_ref and i < len(ref_b) and rng.random() < hit) else rng.integers(0, V)
    x[tok] += boost
    x -= x.max()
    return (x - np.log(np.exp(x).sum())).astype(np.float32)


def test_multi_step_ragged_decoding_equals_independent_greedy_decoding():
    import torch
    import tree_draft_verification_amd as tv
    cfg = MODELS["loop_d128"]
    steps, depth, width, budget = 8, 6, 3, 24
    N = budget + 1
    room = N + steps * (depth + 1)
    wl = WORKLOADS["qwen3_8b_ragged8_N64"].replace(B=3, Hq=8, Hkv=2, N=room, L_lo=20,
                                                  L_hi=150, seed=81)
    w = model_weights(cfg)
    x = model_inputs(cfg, wl)
    B, V = wl.B, cfg.V
    L0 = x["seq_lens"].copy()
    root0 = x["tokens"][:, 0].copy()
    n_ref = steps * (depth + 1) + 2
    ref = oracle.ar_decode(cfg.dims(), w, x["k_cache"], x["v_cache"], L0, root0, n_ref)
    print(f"[loop] L0={L0.tolist()} reference of {n_ref} tokens; min gap "
          f"{ref['gap'].min():.3e}", flush=True)

    wd = {k: to_dev(v, "bf16") for k, v in w.items()}
    model = tv.tv_model_pack(cfg.dims(), wd)
    del wd
    kc, vc = to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16")
    Lcap = kc.shape[3]
    lens = i32_dev(L0)
    emitted = [[] for _ in range(B)]
    root = root0.copy()
    rng = np.random.default_rng(5)
    plens = []
    for s in range(steps):
        cur = lens.cpu().numpy()
        e = cur - L0
        paths = [[(int(root[b]),)] for b in range(B)]
        for level in range(1, depth + 1):
            rows = np.zeros((B, width, V), np.float32)
            for b in range(B):
                for r, pth in enumerate(paths[b]):
                    rows[b, r] = _drafter_row(rng, ref["tokens"][b], int(e[b]), pth, V)
            fs, ft = tv.tv_tree_build_level(torch.from_numpy(rows).cuda(), level, depth)
            fs, ft = fs.cpu().numpy(), ft.cpu().numpy()
            paths = [[paths[b][int(fs[b, r])] + (int(ft[b, r]),) for r in range(width)]
                     for b in range(B)]
        par, tok = tv.tv_tree_build_finish(i32_dev(root), depth, V, width, budget)
        st = torch.zeros(B, dtype=torch.int32, device="cuda")
        arg = tv.tv_verify_pass(model, tok, par, lens, kc, vc,
                                max_seq_len=int(cur.max()), dev_status=st)
        path, plen, bonus = tv.tv_tree_accept(par, tok, arg, 32, dev_status=st)
        tv.tv_kv_compact_layers(kc, vc, lens, path, plen)
        torch.cuda.synchronize()
        assert st.cpu().tolist() == [0] * B
        path_h, plen_h, bonus_h, tok_h = (t.cpu().numpy() for t in (path, plen, bonus, tok))
        plens.append(plen_h.tolist())
        for b in range(B):
            n = int(plen_h[b])
            emitted[b] += [int(t) for t in tok_h[b, path_h[b, 1:n]]] + [int(bonus_h[b])]
            root[b] = bonus_h[b]
        assert int(cur.max()) + int(plen_h.max()) + N <= Lcap
    print(f"[loop] path lengths per step: {plens}", flush=True)
    assert max(max(p) for p in plens) >= 5                         # deep drafts were accepted
    assert any(len(set(p)) > 1 for p in plens)                      # acceptance was ragged

    final = lens.cpu().numpy()
    gk = to_host_f64(kc)
    checked = 0
    for b in range(B):
        got = np.array(emitted[b])
        assert final[b] == L0[b] + len(got)
        want = ref["tokens"][b, :len(got)]
        near = np.nonzero(ref["gap"][b, :len(got)] < GAP_EXEMPT)[0]
        upto = int(near[0]) if len(near) else len(got)   # up to the first near-tie choice
        diff = np.nonzero(got != want)[0]
        if len(diff):
            print(f"[loop] sequence {b}: first difference at {diff[0]} (reference gap "
                  f"{ref['gap'][b, diff[0]]:.3e}), first near-tie at {upto}", flush=True)
        np.testing.assert_array_equal(got[:upto], want[:upto], err_msg=f"sequence {b}")
        checked += upto
        if upto == len(got):
            # the committed cache rows match independent decoding's rows
            L, n = int(L0[b]), len(got)
            sl = (slice(None), b, slice(None), slice(L, L + n))
            a, r = gk[sl], ref["k_cache"][sl]
            rel = np.linalg.norm(a - r) / np.linalg.norm(r)
            assert rel < 5e-3, f"sequence {b}: committed K rows rel {rel:.2e}"
    print(f"[loop] emitted {[len(e) for e in emitted]} tokens, {checked} compared", flush=True)
    assert checked >= 30
