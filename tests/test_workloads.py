"""The seeded input generator: determinism, encodings and tree rules."""
import numpy as np
import pytest

from workloads import (BF16_QNAN, WORKLOADS, attn_inputs, bf16_bits_from_f32,
                       draft_coins, draft_tokens, lmhead_inputs)


def test_bf16_round_to_nearest_even_hand_cases():
    f = np.array([
        1.0,                      # exact
        1.0 + 2.0 ** -8,          # exact tie between 1.0 and 1+2^-7 -> even (1.0)
        1.0 + 3 * 2.0 ** -8,      # tie -> even (1 + 2^-6)
        1.0 + 2.0 ** -8 + 2.0 ** -20,   # just above the tie -> up
        -2.5, 65504.0, 3.0e38, np.inf, -0.0,
    ], dtype=np.float32)
    got = bf16_bits_from_f32(f)
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x4780, 0x7F62, 0x7F80, 0x8000]
    assert list(got) == want
    assert bf16_bits_from_f32(np.array([np.nan], np.float32))[0] == BF16_QNAN


def test_generation_is_deterministic_and_streams_independent():
    wl = WORKLOADS["qwen3_8b_L1024_N64"].replace(V=1000, hidden=256)
    a = attn_inputs(wl)
    b = attn_inputs(wl)
    for key in ("q", "k_cache", "v_cache", "parent", "seq_lens"):
        np.testing.assert_array_equal(a[key], b[key])
    l1 = lmhead_inputs(wl)
    l2 = lmhead_inputs(wl.replace(V=2000))     # W changes shape, H must not
    np.testing.assert_array_equal(l1["hidden"], l2["hidden"])
    c = attn_inputs(wl, seed=77)
    assert not np.array_equal(a["q"], c["q"])


def test_normal_draws_have_requested_spread():
    wl = WORKLOADS["qwen3_8b_L1024_N64"].replace(V=4096, hidden=512)
    w = lmhead_inputs(wl)["w"]
    x = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(x.mean()) < 2e-4
    assert abs(x.std() - 0.02) < 2e-4


def test_unused_cache_rows_are_nan_and_used_rows_finite():
    wl = WORKLOADS["qwen3_8b_ragged8_N64"].replace(L_hi=700)
    a = attn_inputs(wl)
    k = a["k_cache"]
    assert a["Lcap"] % 64 == 0 and a["Lcap"] >= 700 + 64
    for b in range(wl.B):
        end = int(a["seq_lens"][b]) + wl.N
        assert (k[b, :, end:] == BF16_QNAN).all()
        assert not (k[b, :, :end] == BF16_QNAN).any()
    assert a["seq_lens"].min() >= 512 and a["seq_lens"].max() <= 700


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_tree_rules(name):
    wl = WORKLOADS[name]
    a = attn_inputs(wl.replace(L_lo=min(wl.L_lo, 64), L_hi=min(wl.L_hi, 64), D=8,
                               Hq=wl.Hq // wl.Hkv, Hkv=1))
    parent, depth = a["parent"], a["depth"]
    assert parent.shape == (wl.B, wl.N)
    assert (parent[:, 0] == -1).all()
    idx = np.arange(1, wl.N)
    assert ((parent[:, 1:] >= 0) & (parent[:, 1:] < idx)).all()
    assert (depth[:, 1:] == np.take_along_axis(depth, parent[:, 1:], 1) + 1).all()
    if wl.tree == "binary":
        assert list(parent[0]) == [-1, 0, 0, 1, 1, 2, 2]
    else:
        assert depth.max() <= wl.depth_cap
    if wl.tree == "bfs":
        for b in range(wl.B):
            counts = np.bincount(parent[b, 1:], minlength=wl.N)
            last = parent[b, -1]
            # every node before the last expanded one got lo..hi children
            # (the last expanded node may be cut by the budget)
            for u in range(last):
                if depth[b, u] < wl.depth_cap:
                    assert wl.branch_lo <= counts[u] <= wl.branch_hi
            # children come in breadth-first order
            assert (np.diff(parent[b, 1:]) >= 0).all()


def test_draft_tokens_follow_coins():
    wl = WORKLOADS["qwen3_8b_L16384_N256"]
    parent = np.array([[-1, 0, 0, 1, 2, 4]], np.int32)
    depth = np.array([[0, 1, 1, 2, 2, 3]], np.int32)
    wl1 = wl.replace(N=6)
    coins = draft_coins(wl1, depth)
    np.testing.assert_allclose(coins["p"][0], [0, 0.8, 0.8, 0.76, 0.76, 0.722])
    tgt = np.array([[10, 11, 12, 13, 14, 15]], np.int32)
    tok = draft_tokens(parent, coins, tgt)
    for i in range(1, 6):
        if coins["u"][0, i] < coins["p"][0, i]:
            assert tok[0, i] == tgt[0, parent[0, i]]
        else:
            assert tok[0, i] == coins["rand_tok"][0, i]
    assert tok[0, 0] == coins["rand_tok"][0, 0]


def test_ragged_match_probability_is_per_sequence():
    wl = WORKLOADS["qwen3_8b_ragged8_N64"]
    depth = np.ones((wl.B, wl.N), np.int32)
    p = draft_coins(wl, depth)["p"]
    assert np.ptp(p[:, 1]) > 0.05
    assert ((p[:, 1:] >= 0.5) & (p[:, 1:] <= 0.95)).all()
    assert (p[:, 1:] == p[:, 1:2]).all()
