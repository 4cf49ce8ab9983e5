"""GPU parity at sizes the oracle finishes in seconds: element by element.

Every call goes through the C-ABI library (via the thin binding).  Inputs
are the seeded workloads; expected values come from the fp64 oracle only.
"""
import numpy as np
import pytest

import oracle
from workloads import (WORKLOADS, attn_inputs, draft_coins, draft_tokens, lmhead_inputs,
                       paged_layout)

from _helpers import (LOGITS_REL_L2, assert_argmax_ok, assert_attn_close, i32_dev,
                      to_dev, to_host_bits, to_host_f64)

pytestmark = pytest.mark.gpu

Q8 = WORKLOADS["qwen3_8b_L1024_N64"]
A3B = WORKLOADS["qwen3_30b_a3b_B4_L4096_N1024"]

# Small attention cases: several key tiles, ragged tails, GQA 1/3/4/8, D 64/128.
ATTN_CASES = {
    "tiny_fp32": WORKLOADS["tiny_fp32"],
    "q8_L300_N64": Q8.replace(L_lo=300, L_hi=300, seed=11),
    "q8_bfs_L1000_N256": WORKLOADS["qwen3_8b_L16384_N256"].replace(L_lo=1000, L_hi=1000, seed=12),
    "q8_ragged3_N64": WORKLOADS["qwen3_8b_ragged8_N64"].replace(B=3, L_lo=100, L_hi=700, seed=13),
    "a3b_B2_L257_N200": A3B.replace(B=2, L_lo=257, L_hi=257, N=200, seed=14),
    "d64_bf16_L129_N33": Q8.replace(Hq=8, Hkv=2, D=64, L_lo=129, L_hi=129, N=33, seed=15),
    "g3_L70_N50": Q8.replace(Hq=12, Hkv=4, L_lo=70, L_hi=70, N=50, seed=16),
    "g1_L64_N130": Q8.replace(Hq=4, Hkv=4, L_lo=64, L_hi=64, N=130, seed=17),
    "empty_prefix_N20": Q8.replace(L_lo=0, L_hi=0, N=20, seed=18),
    "single_node_L77": Q8.replace(L_lo=77, L_hi=77, N=1, seed=19),
    "f32_gqa_L90_N20": Q8.replace(dtype="f32", Hq=8, Hkv=2, L_lo=90, L_hi=90, N=20, seed=20),
    # prefixes of 32 tiles and more: 128-row query blocks, K loaded straight
    # into LDS, split prefixes with a ragged last tile
    "q8_L2100_N64": Q8.replace(L_lo=2100, L_hi=2100, seed=21),
    "q8_ragged2_L2000_3100_N64": WORKLOADS["qwen3_8b_ragged8_N64"].replace(
        B=2, L_lo=2000, L_hi=3100, seed=22),
    "q8_bfs_L2049_N256": WORKLOADS["qwen3_8b_L16384_N256"].replace(L_lo=2049, L_hi=2049, seed=23),
    # one query head per KV head: a 128-row block spans 128 nodes, whose
    # ancestor words (3 per node) fill the most dynamic LDS
    "g1_L2100_N130": Q8.replace(Hq=4, Hkv=4, L_lo=2100, L_hi=2100, N=130, seed=24),
    # ragged batches whose splits come from the lengths on the device: empty
    # to 3000-token prefixes; the most sequences that path takes (64) with
    # 64-row blocks; one more (65) on the uniform split
    "q8_ragged8_L0_3000_N64": WORKLOADS["qwen3_8b_ragged8_N64"].replace(L_lo=0, L_hi=3000,
                                                                        seed=25),
    "q8_ragged64_L0_700_N16": WORKLOADS["qwen3_8b_ragged8_N64"].replace(
        B=64, N=16, Hq=8, Hkv=2, L_lo=0, L_hi=700, seed=26),
    "q8_ragged65_L100_900_N8": WORKLOADS["qwen3_8b_ragged8_N64"].replace(
        B=65, N=8, Hq=4, Hkv=1, L_lo=100, L_hi=900, seed=27),
}


def _run_attn(a, wl, parent=None, max_seq_len=None):
    import tree_draft_verification_amd as tv
    par = a["parent"] if parent is None else parent
    q = to_dev(a["q"], wl.dtype)
    k = to_dev(a["k_cache"], wl.dtype)
    v = to_dev(a["v_cache"], wl.dtype)
    out = tv.tv_tree_verify_attn(q, k, v, i32_dev(a["seq_lens"]), i32_dev(par),
                                 max_seq_len=int(a["seq_lens"].max()) if max_seq_len is None
                                 else max_seq_len, scale=a["scale"])
    return out


@pytest.mark.parametrize("name", list(ATTN_CASES))
def test_attention_elementwise(name):
    wl = ATTN_CASES[name]
    a = attn_inputs(wl)
    print(f"[attn] {name} B={wl.B} N={wl.N} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} "
          f"L={list(a['seq_lens'])}", flush=True)
    out = _run_attn(a, wl)
    ref = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], a["seq_lens"],
                                a["parent"], a["scale"], wl.dtype)
    got = to_host_f64(out)
    mx, rel = assert_attn_close(got, ref, name)
    if wl.dtype == "f32":
        assert mx < 1e-5, f"fp32 path should be near-exact, max|d|={mx}"


@pytest.mark.parametrize("shape", ["chain", "star"])
def test_attention_chain_and_star_trees(shape):
    """Chain tree == causal attention and star tree (every node a root child)."""
    wl = Q8.replace(L_lo=200, L_hi=200, N=100, seed=21)
    a = attn_inputs(wl)
    N = wl.N
    if shape == "chain":
        parent = np.arange(-1, N - 1, dtype=np.int32)[None]
    else:
        parent = np.zeros((1, N), np.int32)
        parent[0, 0] = -1
    out = _run_attn(a, wl, parent=parent)
    ref = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], a["seq_lens"],
                                parent, a["scale"], wl.dtype)
    assert_attn_close(to_host_f64(out), ref, shape)


@pytest.mark.parametrize("hq,hkv,L", [(8, 1, 40), (2, 2, 2100)],
                         ids=["g8_L40", "g1_L2100"])
def test_attention_deep_chain_1024_nodes(hq, hkv, L):
    """A 1024-node chain: every tree tile visible to the deepest nodes; with
    one query head per KV head and a long prefix, each 128-row block spans
    128 nodes with 16 ancestor words each (the largest ancestor table)."""
    wl = A3B.replace(B=1, Hq=hq, Hkv=hkv, L_lo=L, L_hi=L, N=1024, seed=22)
    a = attn_inputs(wl)
    parent = np.arange(-1, 1023, dtype=np.int32)[None]
    out = _run_attn(a, wl, parent=parent)
    nodes = [0, 1, 63, 64, 65, 500, 1022, 1023]
    ref = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], a["seq_lens"], parent,
                                a["scale"], wl.dtype, nodes=nodes)
    assert_attn_close(to_host_f64(out), ref, "chain1024")


def test_attention_flags_bad_trees_and_lengths():
    import torch
    import tree_draft_verification_amd as tv
    wl = Q8.replace(B=2, L_lo=100, L_hi=100, N=16, seed=23)
    a = attn_inputs(wl)
    parent = a["parent"].copy()
    parent[1, 5] = 9                                    # parent[i] >= i in sequence 1
    st = torch.zeros(2, dtype=torch.int32, device="cuda")
    q, k, v = (to_dev(a[x], "bf16") for x in ("q", "k_cache", "v_cache"))
    tv.tv_tree_verify_attn(q, k, v, i32_dev(a["seq_lens"]), i32_dev(parent),
                           max_seq_len=100, dev_status=st)
    assert st.cpu().tolist() == [0, tv.TV_STATUS_BAD_PARENT]
    st.zero_()
    lens = a["seq_lens"].copy()
    lens[0] = 101                                       # above max_seq_len
    tv.tv_tree_verify_attn(q, k, v, i32_dev(lens), i32_dev(a["parent"]),
                           max_seq_len=100, dev_status=st)
    assert st.cpu().tolist() == [tv.TV_STATUS_BAD_LEN, 0]


def test_attention_ragged_batch_flags_one_bad_length():
    """A ragged batch (splits derived from the lengths on the device) with
    one length above max_seq_len: that sequence is flagged and counts as no
    prefix in the plan; the others equal the oracle."""
    import torch
    import tree_draft_verification_amd as tv
    wl = WORKLOADS["qwen3_8b_ragged8_N64"].replace(B=4, L_lo=1500, L_hi=2500, seed=29)
    a = attn_inputs(wl)
    msl = int(a["seq_lens"].max())
    lens = a["seq_lens"].copy()
    lens[2] = msl + 1
    st = torch.zeros(wl.B, dtype=torch.int32, device="cuda")
    q, k, v = (to_dev(a[x], "bf16") for x in ("q", "k_cache", "v_cache"))
    out = tv.tv_tree_verify_attn(q, k, v, i32_dev(lens), i32_dev(a["parent"]),
                                 max_seq_len=msl, scale=a["scale"], dev_status=st)
    assert st.cpu().tolist() == [0, 0, tv.TV_STATUS_BAD_LEN, 0]
    ref = oracle.tree_attention(a["q"], a["k_cache"], a["v_cache"], a["seq_lens"],
                                a["parent"], a["scale"], wl.dtype)
    got = to_host_f64(out)
    for b in (0, 1, 3):
        assert_attn_close(got[b], ref[b], f"sequence {b}")


def test_attention_deterministic():
    wl = ATTN_CASES["q8_bfs_L1000_N256"]
    a = attn_inputs(wl)
    o1 = to_host_bits(_run_attn(a, wl))
    o2 = to_host_bits(_run_attn(a, wl))
    np.testing.assert_array_equal(o1, o2)


# ---------------------------------------------------------------- LM head

LM_CASES = {
    "tiny_fp32": WORKLOADS["tiny_fp32"],
    "M64_K4096_V8192": Q8.replace(V=8192, seed=31),
    "M100_K256_V1001": Q8.replace(B=1, N=100, hidden=256, V=1001, seed=32),
    "M1_K256_V130": Q8.replace(N=1, hidden=256, V=130, seed=33),
    "M256_K512_V4163": Q8.replace(N=256, hidden=512, V=4163, seed=34),
    "M513_K256_V2000": Q8.replace(B=1, N=513, hidden=256, V=2000, seed=35),
    "f32_M40_K100_V777": Q8.replace(dtype="f32", N=40, hidden=100, V=777, seed=36),
    # more 128-row tiles than resident workgroups, so each workgroup of the
    # persistent M <= 64 kernel walks several tiles; the shortest k stream
    "M64_K256_V151936": Q8.replace(N=64, hidden=256, V=151936, seed=37),
    # ragged last tile (33 rows) after 781 whole ones
    "M17_K512_V100001": Q8.replace(B=1, N=17, hidden=512, V=100001, seed=38),
    # the eight-wavefront product: 128 W tiles of 384 rows (one round of 256
    # workgroups), then 66 of 256 rows with a partial last one, and a partial
    # last H slice
    "M300_K256_V66000": Q8.replace(B=1, N=300, hidden=256, V=66000, seed=39),
    # one width: 17 W tiles of 256 rows
    "M256_K256_V4163": Q8.replace(N=256, hidden=256, V=4163, seed=40),
}


# (case, packed layout): the packed layout exists for bf16 only
LM_LAYOUT_CASES = [(n, p) for n, wl in LM_CASES.items()
                   for p in ((False, True) if wl.dtype == "bf16" else (False,))]


@pytest.mark.parametrize("name,packed", LM_LAYOUT_CASES,
                         ids=[f"{n}-{'packed' if p else 'rowmajor'}" for n, p in LM_LAYOUT_CASES])
def test_lmhead_elementwise(name, packed):
    import torch
    import tree_draft_verification_amd as tv
    wl = LM_CASES[name]
    lm = lmhead_inputs(wl)
    M, V = wl.M, wl.V
    print(f"[lmhead] {name} M={M} K={wl.hidden} V={V}", flush=True)
    h = to_dev(lm["hidden"], wl.dtype)
    w = to_dev(lm["w"], wl.dtype)
    if packed:
        w = tv.tv_lmhead_pack_weights(w)
    logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
    ws = torch.zeros(tv.tv_lmhead_argmax_workspace(M, wl.hidden, V), dtype=torch.uint8,
                     device="cuda")
    arg = tv.tv_lmhead_argmax(h, w, logits=logits, workspace=ws)
    got_l = logits.cpu().numpy().astype(np.float64)
    ref_l = oracle.lm_logits(lm["hidden"], lm["w"], wl.dtype)
    rel = np.linalg.norm(got_l - ref_l) / np.linalg.norm(ref_l)
    assert rel <= LOGITS_REL_L2, f"logits rel L2 {rel:.3e}"
    ref = oracle.lm_head_argmax(lm["hidden"], lm["w"], wl.dtype)
    assert_argmax_ok(arg.cpu().numpy(), ref, name)
    # the zero region of the workspace is left zeroed, and a second call
    # (no logits) agrees
    zero_bytes = (M * 8 + 255) // 256 * 256 + 256
    assert int(ws[:zero_bytes].count_nonzero()) == 0
    arg2 = tv.tv_lmhead_argmax(h, w, workspace=ws)
    np.testing.assert_array_equal(arg2.cpu().numpy(), arg.cpu().numpy())


def test_lmhead_calls_of_different_m_share_one_workspace():
    """Single-kernel (M <= 64) and partial-key (M > 64) calls in any order on
    one workspace sized for the largest M."""
    import torch
    import tree_draft_verification_amd as tv
    wl = Q8.replace(B=1, N=300, hidden=512, V=3000, seed=39)
    lm = lmhead_inputs(wl)
    h_all = to_dev(lm["hidden"], "bf16")
    w = to_dev(lm["w"], "bf16")
    ref = oracle.lm_head_argmax(lm["hidden"], lm["w"], "bf16")
    ws = torch.zeros(tv.tv_lmhead_argmax_workspace(300, 512, 3000), dtype=torch.uint8,
                     device="cuda")
    wp = tv.tv_lmhead_pack_weights(w)
    for M in (300, 64, 100, 7, 300, 129):
        for wt in (w, wp):
            arg = tv.tv_lmhead_argmax(h_all[:M].contiguous(), wt, workspace=ws).cpu().numpy()
            sub = {k: v[:M] for k, v in ref.items()}
            assert_argmax_ok(arg, sub, f"M={M}")


def test_pack_layout_matches_definition():
    """Packed bytes = W (zero-padded to 128-row tiles) permuted to
    [tile][k chunk][16-row block][16-byte piece][lane][8 values]."""
    import tree_draft_verification_amd as tv
    rng = np.random.default_rng(38)
    V, K = 300, 512
    w = rng.integers(0, 65535, size=(V, K)).astype(np.uint16)
    got = tv.tv_lmhead_pack_weights(to_dev(w, "bf16")).data.cpu().numpy().view(np.uint16)
    nvt, nk = -(-V // 128), K // 128
    wp = np.zeros((nvt * 128, K), np.uint16)
    wp[:V] = w
    # row = vt*128 + j*16 + l16; col = c*128 + 32*kg + 8*s + e; lane = kg*16 + l16
    want = wp.reshape(nvt, 8, 16, nk, 4, 4, 8).transpose(0, 3, 1, 5, 4, 2, 6).reshape(-1)
    np.testing.assert_array_equal(got, want)


def test_lmhead_ties_go_to_smallest_index():
    import tree_draft_verification_amd as tv
    from workloads import bf16_bits_from_f32
    rng = np.random.default_rng(37)
    M, K, V = 70, 512, 3000
    Hi = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    Wi = rng.integers(-2, 3, size=(V, K)).astype(np.float32)
    Wi[2500] = Wi[11]          # duplicate rows -> exact ties across workgroups
    Wi[1234] = Wi[11]
    Wi[129] = Wi[128]          # a tie inside one workgroup tile
    h = bf16_bits_from_f32(Hi)
    w = bf16_bits_from_f32(Wi)
    exact = Hi.astype(np.int64) @ Wi.T.astype(np.int64)
    wd = to_dev(w, "bf16")
    for wt in (wd, tv.tv_lmhead_pack_weights(wd)):
        arg = tv.tv_lmhead_argmax(to_dev(h, "bf16"), wt).cpu().numpy()
        np.testing.assert_array_equal(arg, np.argmax(exact, axis=1))


def test_lmhead_stream_kernel_ties_across_its_tiles():
    """Up to 64 rows the persistent kernel walks 128-row vocabulary tiles
    b, b + grid, ...; duplicate W rows farther apart than one grid's worth
    of tiles tie across the tiles one workgroup walks and across workgroups:
    the smallest index wins."""
    import tree_draft_verification_amd as tv
    from workloads import bf16_bits_from_f32
    rng = np.random.default_rng(38)
    M, K, V = 17, 256, 150000
    Hi = rng.integers(1, 3, size=(M, K)).astype(np.float32)     # positive
    Wi = rng.integers(-1, 2, size=(V, K)).astype(np.float32)
    # all-ones rows score sum(H[m]), above every random row: exact ties at
    # the maximum, in tiles 5 and 5 + 768 (one workgroup's first and second
    # tile with a resident grid of 768), and farther apart than any grid of
    # at most 1024 tiles
    dup = [98947, 643, 131079, 140001, 65539]
    Wi[dup] = 1.0
    h = bf16_bits_from_f32(Hi)
    w = bf16_bits_from_f32(Wi)
    exact = Hi.astype(np.int64) @ Wi.T.astype(np.int64)
    want = np.argmax(exact, axis=1)
    assert (want == min(dup)).all()
    wd = to_dev(w, "bf16")
    for wt in (wd, tv.tv_lmhead_pack_weights(wd)):
        arg = tv.tv_lmhead_argmax(to_dev(h, "bf16"), wt).cpu().numpy()
        np.testing.assert_array_equal(arg, want)


def test_lmhead_ties_across_the_two_tile_widths():
    """From 256 rows the vocabulary is split into 384-row then 256-row W
    tiles, launched separately: duplicate W rows in the first tile, the last
    384-row tile, the 256-row tail and its partial last tile tie exactly at
    the maximum; the smallest index wins."""
    import tree_draft_verification_amd as tv
    from workloads import bf16_bits_from_f32
    rng = np.random.default_rng(41)
    M, K, V = 300, 256, 66000          # 128 tiles of 384 rows, then 66 of 256
    Hi = rng.integers(1, 3, size=(M, K)).astype(np.float32)
    Wi = rng.integers(-1, 2, size=(V, K)).astype(np.float32)
    for dup in ([49151, 49152, 65999], [65999, 50000], [11, 65999, 49151]):
        Wd = Wi.copy()
        Wd[dup] = 1.0
        exact = Hi.astype(np.int64) @ Wd.T.astype(np.int64)
        want = np.argmax(exact, axis=1)
        assert (want == min(dup)).all()
        wd = to_dev(bf16_bits_from_f32(Wd), "bf16")
        arg = tv.tv_lmhead_argmax(to_dev(bf16_bits_from_f32(Hi), "bf16"),
                                  tv.tv_lmhead_pack_weights(wd)).cpu().numpy()
        np.testing.assert_array_equal(arg, want, err_msg=f"duplicates at {dup}")


def test_lmhead_cached_workspaces_of_mixed_dtypes_and_sizes():
    """The binding's own workspaces: a bf16 call with M > 64 (which leaves
    partial keys behind), then fp32 calls with more rows, then the bf16 call
    again, each equal to the oracle."""
    import tree_draft_verification_amd as tv
    for wl in (Q8.replace(B=1, N=100, hidden=256, V=3001, seed=61),
               Q8.replace(B=1, N=200, hidden=96, V=3001, dtype="f32", seed=62),
               Q8.replace(B=1, N=300, hidden=96, V=2000, dtype="f32", seed=63),
               Q8.replace(B=1, N=100, hidden=256, V=3001, seed=61)):
        lm = lmhead_inputs(wl)
        arg = tv.tv_lmhead_argmax(to_dev(lm["hidden"], wl.dtype), to_dev(lm["w"], wl.dtype))
        ref = oracle.lm_head_argmax(lm["hidden"], lm["w"], wl.dtype)
        assert_argmax_ok(arg.cpu().numpy(), ref, f"M={wl.M} {wl.dtype}")


# ---------------------------------------------------------------- accept + compact

def _accept_gpu(parent, draft, tgt, P):
    import tree_draft_verification_amd as tv
    path, plen, bonus = tv.tv_tree_accept(i32_dev(parent), i32_dev(draft), i32_dev(tgt), P)
    return path.cpu().numpy(), plen.cpu().numpy(), bonus.cpu().numpy()


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_accept_bit_exact_on_workload_trees(name):
    wl = WORKLOADS[name]
    small = wl.replace(L_lo=min(wl.L_lo, 64), L_hi=min(wl.L_hi, 64), Hq=1, Hkv=1, D=64)
    a = attn_inputs(small)
    rng = np.random.default_rng(41)
    for trial in range(4):
        tgt = rng.integers(0, 50, size=(wl.B, wl.N)).astype(np.int32)
        draft = draft_tokens(a["parent"], draft_coins(wl, a["depth"], seed=wl.seed + trial), tgt)
        ref = oracle.tree_accept(a["parent"], draft, tgt, P=32)
        path, plen, bonus = _accept_gpu(a["parent"], draft, tgt, 32)
        np.testing.assert_array_equal(plen, ref["path_len"])
        np.testing.assert_array_equal(path, ref["path"])
        np.testing.assert_array_equal(bonus, ref["bonus"])


def test_accept_exhaustive_small_trees():
    import itertools
    rng = np.random.default_rng(42)
    parents, drafts, tgts = [], [], []
    for choice in itertools.product(*[range(i) for i in range(1, 6)]):
        parents.append([-1, *choice])
        drafts.append(rng.integers(0, 2, size=6))
        tgts.append(rng.integers(0, 2, size=6))
    parent = np.array(parents, np.int32)
    draft = np.array(drafts, np.int32)
    tgt = np.array(tgts, np.int32)
    ref = oracle.tree_accept(parent, draft, tgt, P=8)
    path, plen, bonus = _accept_gpu(parent, draft, tgt, 8)
    np.testing.assert_array_equal(path, ref["path"])
    np.testing.assert_array_equal(plen, ref["path_len"])
    np.testing.assert_array_equal(bonus, ref["bonus"])


def test_accept_edge_cases_and_flags():
    import torch
    import tree_draft_verification_amd as tv
    N = 40
    chain = np.arange(-1, N - 1, dtype=np.int32)
    tgt = np.arange(500, 500 + N, dtype=np.int32)
    all_match = np.concatenate([[3], tgt[:-1]]).astype(np.int32)
    no_match = np.full(N, 7, np.int32)
    star = np.zeros(N, np.int32)
    star[0] = -1
    parent = np.stack([chain, chain, star, chain, chain])
    draft = np.stack([all_match, no_match, np.full(N, 500, np.int32), all_match, all_match])
    tgts = np.stack([tgt] * 5)
    parent[3, 7] = 12                                   # malformed
    st = torch.zeros(5, dtype=torch.int32, device="cuda")
    path, plen, bonus = tv.tv_tree_accept(i32_dev(parent), i32_dev(draft), i32_dev(tgts), 48,
                                          dev_status=st)
    plen, bonus, path = plen.cpu().numpy(), bonus.cpu().numpy(), path.cpu().numpy()
    assert plen[0] == N and bonus[0] == tgt[N - 1] and list(path[0, :N]) == list(range(N))
    assert plen[1] == 1 and bonus[1] == 500 and path[1, 0] == 0 and (path[1, 1:] == -1).all()
    assert plen[2] == 2 and path[2, 1] == 1 and bonus[2] == tgt[1]   # first of equal siblings
    assert plen[3] == 0 and bonus[3] == -1 and (path[3] == -1).all()
    assert st.cpu().tolist() == [0, 0, 0, tv.TV_STATUS_BAD_PARENT, 0]
    # accepted path longer than P
    st.zero_()
    path, plen, bonus = tv.tv_tree_accept(i32_dev(chain[None]), i32_dev(all_match[None]),
                                          i32_dev(tgt[None]), 16, dev_status=st[:1])
    assert plen.item() == 0 and st[0].item() == tv.TV_STATUS_DEPTH
    # single node
    path, plen, bonus = _accept_gpu(np.array([[-1]], np.int32), np.array([[4]], np.int32),
                                    np.array([[99]], np.int32), 4)
    assert plen[0] == 1 and bonus[0] == 99 and list(path[0]) == [0, -1, -1, -1]


@pytest.mark.parametrize("name", ["tiny_fp32", "qwen3_8b_ragged8_N64", "qwen3_30b_a3b_B4_L4096_N1024"])
def test_compact_bit_exact(name):
    import tree_draft_verification_amd as tv
    wl = WORKLOADS[name]
    if name != "tiny_fp32":
        wl = wl.replace(L_lo=min(wl.L_lo, 300), L_hi=min(wl.L_hi, 900))
    a = attn_inputs(wl)
    rng = np.random.default_rng(43)
    tgt = rng.integers(0, 20, size=(wl.B, wl.N)).astype(np.int32)
    draft = draft_tokens(a["parent"], draft_coins(wl, a["depth"]), tgt)
    acc = oracle.tree_accept(a["parent"], draft, tgt, P=32)
    k2, v2, lens2 = oracle.kv_compact(a["k_cache"], a["v_cache"], a["seq_lens"],
                                      acc["path"], acc["path_len"])
    k = to_dev(a["k_cache"], wl.dtype)
    v = to_dev(a["v_cache"], wl.dtype)
    lens = i32_dev(a["seq_lens"])
    tv.tv_kv_compact(k, v, lens, i32_dev(acc["path"]), i32_dev(acc["path_len"]))
    np.testing.assert_array_equal(lens.cpu().numpy(), lens2)
    gk, gv = to_host_bits(k), to_host_bits(v)
    if wl.dtype == "f32":   # NaN-poisoned rows: compare bits
        gk, gv, k2, v2 = (x.view(np.uint32) for x in (gk, gv, k2, v2))
    np.testing.assert_array_equal(gk, k2)
    np.testing.assert_array_equal(gv, v2)


def test_compact_hazard_every_row_moves():
    """path = [0, 2, 4, 6, ...]: every move j reads the row a later move... and
    an earlier move writes row path[j'] = j; staging must keep it exact."""
    import tree_draft_verification_amd as tv
    B, Hkv, D, L, N, P = 2, 3, 128, 5, 64, 32
    rng = np.random.default_rng(44)
    kc = rng.integers(0, 65535, size=(B, Hkv, L + N + 8, D)).astype(np.uint16)
    vc = rng.integers(0, 65535, size=(B, Hkv, L + N + 8, D)).astype(np.uint16)
    path = np.full((B, P), -1, np.int32)
    path[0, :20] = np.arange(0, 40, 2)
    path[1, :32] = np.concatenate([[0], np.arange(1, 32) + 30])
    plen = np.array([20, 32], np.int32)
    lens = np.array([L, L], np.int32)
    k2, v2, lens2 = oracle.kv_compact(kc, vc, lens, path, plen)
    k, v, sl = to_dev(kc, "bf16"), to_dev(vc, "bf16"), i32_dev(lens)
    tv.tv_kv_compact(k, v, sl, i32_dev(path), i32_dev(plen))
    np.testing.assert_array_equal(to_host_bits(k), k2)
    np.testing.assert_array_equal(to_host_bits(v), v2)
    np.testing.assert_array_equal(sl.cpu().numpy(), lens2)


# ---------------------------------------------------------------- whole step

@pytest.mark.parametrize("name", ["tiny_fp32", "q8_ragged3_N64", "a3b_B2_L257_N200"])
def test_step_end_to_end_small(name):
    import tree_draft_verification_amd as tv
    wl = ATTN_CASES[name]
    if wl.dtype == "bf16":
        wl = wl.replace(V=5000, hidden=512)
    a = attn_inputs(wl)
    lm = lmhead_inputs(wl)
    ref_lm = oracle.lm_head_argmax(lm["hidden"], lm["w"], wl.dtype)
    tgt_ref = ref_lm["argmax"].reshape(wl.B, wl.N)
    draft = draft_tokens(a["parent"], draft_coins(wl, a["depth"]), tgt_ref)
    ref = oracle.verify_step(a, lm, draft, wl.dtype)

    q, k, v = (to_dev(a[x], wl.dtype) for x in ("q", "k_cache", "v_cache"))
    lens = i32_dev(a["seq_lens"])
    par = i32_dev(a["parent"])
    out = tv.tv_tree_verify_attn(q, k, v, lens, par, max_seq_len=int(a["seq_lens"].max()),
                                 scale=a["scale"])
    arg = tv.tv_lmhead_argmax(to_dev(lm["hidden"], wl.dtype), to_dev(lm["w"], wl.dtype))
    path, plen, bonus = tv.tv_tree_accept(par, i32_dev(draft), arg, 32)
    tv.tv_kv_compact(k, v, lens, path, plen)

    assert_attn_close(to_host_f64(out), ref["out"], name)
    got_arg = arg.cpu().numpy()
    assert_argmax_ok(got_arg, ref_lm, name)
    # acceptance is checked against the oracle run on the GPU's argmax, which
    # equals the oracle's own argmax except at exempt near-ties
    acc = oracle.tree_accept(a["parent"], draft, got_arg.reshape(wl.B, wl.N), 32)
    np.testing.assert_array_equal(plen.cpu().numpy(), acc["path_len"])
    np.testing.assert_array_equal(path.cpu().numpy(), acc["path"])
    np.testing.assert_array_equal(bonus.cpu().numpy(), acc["bonus"])
    k2, v2, lens2 = oracle.kv_compact(a["k_cache"], a["v_cache"], a["seq_lens"],
                                      acc["path"], acc["path_len"])
    np.testing.assert_array_equal(lens.cpu().numpy(), lens2)
    gk = to_host_bits(k)
    if wl.dtype == "f32":
        gk, k2 = gk.view(np.uint32), k2.view(np.uint32)
    np.testing.assert_array_equal(gk, k2)


# ---------------------------------------------------------------- paged caches

PAGED_CASES = {
    "q8_ragged3_N64_ps16": ("q8_ragged3_N64", 16),
    "a3b_B2_L257_N200_ps64": ("a3b_B2_L257_N200", 64),
    "q8_bfs_L1000_N256_ps256": ("q8_bfs_L1000_N256", 256),
    "d64_bf16_L129_N33_ps32": ("d64_bf16_L129_N33", 32),
    "empty_prefix_N20_ps16": ("empty_prefix_N20", 16),
    "g1_L64_N130_ps128": ("g1_L64_N130", 128),
    "q8_ragged2_L2000_3100_N64_ps16": ("q8_ragged2_L2000_3100_N64", 16),
    "g1_L2100_N130_ps64": ("g1_L2100_N130", 64),
    "q8_ragged8_L0_3000_N64_ps16": ("q8_ragged8_L0_3000_N64", 16),
    # 16-row pages and prefixes past 510 tiles (long splits of the ragged
    # plan, every row through its page entry)
    "ragged2_L33500_36000_N16_ps16": ("ragged2_L33500_36000_N16", 16),
    # slot tables (one row per page): every row through its own entry
    "q8_ragged3_N64_ps1": ("q8_ragged3_N64", 1),
    "a3b_B2_L257_N200_ps1": ("a3b_B2_L257_N200", 1),
    "empty_prefix_N20_ps1": ("empty_prefix_N20", 1),
    "g1_L2100_N130_ps1": ("g1_L2100_N130", 1),
    "q8_ragged8_L0_3000_N64_ps1": ("q8_ragged8_L0_3000_N64", 1),
    "q8_bfs_L1000_N256_ps4": ("q8_bfs_L1000_N256", 4),
}
ATTN_CASES["ragged2_L33500_36000_N16"] = WORKLOADS["qwen3_8b_ragged8_N64"].replace(
    B=2, N=16, Hq=2, Hkv=1, L_lo=33500, L_hi=36000, seed=28)


def _paged_dev(pg, dtype):
    return (to_dev(pg["k_pages"], dtype), to_dev(pg["v_pages"], dtype),
            i32_dev(pg["block_table"]))


@pytest.mark.parametrize("name", list(PAGED_CASES))
def test_attention_paged_elementwise(name):
    """Paged attention == the oracle on the gathered rows; with no plan change
    it also reproduces the contiguous kernel's bits."""
    import torch
    import tree_draft_verification_amd as tv
    case, ps = PAGED_CASES[name]
    wl = ATTN_CASES[case]
    a = attn_inputs(wl)
    pg = paged_layout(a["k_cache"], a["v_cache"], ps, seed=wl.seed + ps)
    print(f"[attn-paged] {name} B={wl.B} N={wl.N} L={list(a['seq_lens'])} "
          f"pages={pg['num_pages']}", flush=True)
    kp, vp, bt = _paged_dev(pg, wl.dtype)
    st = torch.zeros(wl.B, dtype=torch.int32, device="cuda")
    msl = int(a["seq_lens"].max())
    out = tv.tv_tree_verify_attn_paged(to_dev(a["q"], wl.dtype), kp, vp, bt,
                                       i32_dev(a["seq_lens"]), i32_dev(a["parent"]),
                                       max_seq_len=msl, scale=a["scale"], dev_status=st)
    assert st.cpu().tolist() == [0] * wl.B
    ref = oracle.tree_attention_paged(a["q"], pg["k_pages"], pg["v_pages"], pg["block_table"],
                                      ps, a["seq_lens"], a["parent"], a["scale"], wl.dtype)
    assert_attn_close(to_host_f64(out), ref, name)
    if (tv.tv_tree_verify_attn_paged_workspace(wl.B, wl.N, wl.Hq, wl.Hkv, wl.D, msl, ps)
            == tv.tv_tree_verify_attn_workspace(wl.B, wl.N, wl.Hq, wl.Hkv, wl.D, msl)):
        np.testing.assert_array_equal(to_host_bits(out), to_host_bits(_run_attn(a, wl)))


def test_attention_paged_flags_bad_page():
    """A block-table entry outside the pool flags its sequence only."""
    import torch
    import tree_draft_verification_amd as tv
    wl = ATTN_CASES["q8_ragged3_N64"]
    a = attn_inputs(wl)
    pg = paged_layout(a["k_cache"], a["v_cache"], 16, seed=5)
    bt = pg["block_table"].copy()
    bt[1, 0] = pg["num_pages"]               # first prefix block of sequence 1
    bt[2, int(a["seq_lens"][2]) // 16] = -7   # first tree block of sequence 2
    kp, vp, _ = _paged_dev(pg, "bf16")
    st = torch.zeros(wl.B, dtype=torch.int32, device="cuda")
    out = tv.tv_tree_verify_attn_paged(to_dev(a["q"], "bf16"), kp, vp, i32_dev(bt),
                                       i32_dev(a["seq_lens"]), i32_dev(a["parent"]),
                                       max_seq_len=int(a["seq_lens"].max()), scale=a["scale"],
                                       dev_status=st)
    assert st.cpu().tolist() == [0, tv.TV_STATUS_BAD_PAGE, tv.TV_STATUS_BAD_PAGE]
    ref = oracle.tree_attention(a["q"][:1], a["k_cache"][:1], a["v_cache"][:1],
                                a["seq_lens"][:1], a["parent"][:1], a["scale"], "bf16")
    assert_attn_close(to_host_f64(out)[:1], ref, "bad-page seq 0")


@pytest.mark.parametrize("name,ps", [("tiny_fp32", 16), ("qwen3_8b_ragged8_N64", 16),
                                     ("qwen3_30b_a3b_B4_L4096_N1024", 64),
                                     ("qwen3_8b_ragged8_N64", 1)])
def test_compact_paged_bit_exact(name, ps):
    import tree_draft_verification_amd as tv
    wl = WORKLOADS[name]
    if name != "tiny_fp32":
        wl = wl.replace(L_lo=min(wl.L_lo, 300), L_hi=min(wl.L_hi, 900))
    a = attn_inputs(wl)
    pg = paged_layout(a["k_cache"], a["v_cache"], ps, seed=wl.seed + 7)
    rng = np.random.default_rng(45)
    tgt = rng.integers(0, 20, size=(wl.B, wl.N)).astype(np.int32)
    draft = draft_tokens(a["parent"], draft_coins(wl, a["depth"]), tgt)
    acc = oracle.tree_accept(a["parent"], draft, tgt, P=32)
    k2, v2, lens2 = oracle.kv_compact_paged(pg["k_pages"], pg["v_pages"], pg["block_table"], ps,
                                            a["seq_lens"], acc["path"], acc["path_len"])
    kp, vp, bt = _paged_dev(pg, wl.dtype)
    lens = i32_dev(a["seq_lens"])
    tv.tv_kv_compact_paged(kp, vp, bt, lens, i32_dev(acc["path"]), i32_dev(acc["path_len"]))
    np.testing.assert_array_equal(lens.cpu().numpy(), lens2)
    gk, gv = to_host_bits(kp), to_host_bits(vp)
    if wl.dtype == "f32":
        gk, gv, k2, v2 = (x.view(np.uint32) for x in (gk, gv, k2, v2))
    np.testing.assert_array_equal(gk, k2)
    np.testing.assert_array_equal(gv, v2)


@pytest.mark.parametrize("name", ["qwen3_8b_ragged8_N64", "qwen3_30b_a3b_B4_L4096_N1024",
                                  "tiny_fp32"])
def test_commit_slots_bit_exact(name):
    """The committed slot table and lengths equal the oracle's, on acceptance
    paths of the workload's trees (ragged lengths, 1024-node trees)."""
    import tree_draft_verification_amd as tv
    wl = WORKLOADS[name]
    a = attn_inputs(wl.replace(Hq=wl.Hkv, D=8))   # trees and lengths only
    Lcap = a["Lcap"]
    rng = np.random.default_rng(46)
    bt = np.stack([rng.permutation(wl.B * Lcap)[:Lcap] for _ in range(wl.B)]).astype(np.int32)
    tgt = rng.integers(0, 20, size=(wl.B, wl.N)).astype(np.int32)
    draft = draft_tokens(a["parent"], draft_coins(wl, a["depth"]), tgt)
    acc = oracle.tree_accept(a["parent"], draft, tgt, P=32)
    want_bt, want_lens = oracle.kv_commit_slots(bt, a["seq_lens"], acc["path"], acc["path_len"],
                                                wl.N)
    print(f"[commit-slots] {name} B={wl.B} N={wl.N} path_len={list(acc['path_len'])}", flush=True)
    d_bt, lens = i32_dev(bt), i32_dev(a["seq_lens"])
    st = i32_dev(np.zeros(wl.B, np.int32))
    tv.tv_kv_commit_slots(d_bt, lens, i32_dev(acc["path"]), i32_dev(acc["path_len"]), wl.N,
                          dev_status=st)
    assert st.cpu().tolist() == [0] * wl.B
    np.testing.assert_array_equal(d_bt.cpu().numpy(), want_bt)
    np.testing.assert_array_equal(lens.cpu().numpy(), want_lens)


def test_commit_slots_flags_bad_paths_and_lengths():
    """A path that is not increasing within the tree, or a window past the
    table, flags its sequence and leaves it unchanged; the others commit."""
    import tree_draft_verification_amd as tv
    B, N, P, mb = 4, 16, 8, 40
    rng = np.random.default_rng(47)
    bt = rng.permutation(B * mb).reshape(B, mb).astype(np.int32)
    lens = np.array([3, 5, 30, 2], np.int32)          # sequence 2: 30 + 16 > 40
    path = np.full((B, P), -1, np.int32)
    plen = np.array([3, 3, 2, 4], np.int32)
    path[0, :3] = [0, 4, 9]
    path[1, :3] = [0, 7, 7]                            # not increasing
    path[2, :2] = [0, 1]
    path[3, :4] = [0, 2, 16, 17]                       # past the tree
    st = i32_dev(np.zeros(B, np.int32))
    d_bt, d_lens = i32_dev(bt), i32_dev(lens)
    tv.tv_kv_commit_slots(d_bt, d_lens, i32_dev(path), i32_dev(plen), N, dev_status=st)
    assert st.cpu().tolist() == [0, tv.TV_STATUS_BAD_PATH, tv.TV_STATUS_BAD_LEN,
                                 tv.TV_STATUS_BAD_PATH]
    want_bt, want_lens = oracle.kv_commit_slots(bt[:1], lens[:1], path[:1], plen[:1], N)
    got_bt, got_lens = d_bt.cpu().numpy(), d_lens.cpu().numpy()
    np.testing.assert_array_equal(got_bt[0], want_bt[0])
    np.testing.assert_array_equal(got_bt[1:], bt[1:])
    np.testing.assert_array_equal(got_lens, [want_lens[0], 5, 30, 2])


def test_slot_table_step_reads_the_committed_rows():
    """A step on slot tables: attention through the table, acceptance on the
    GPU, the commit as a table permutation; the rows the committed table
    names equal the row-moving compaction's rows, and a second attention
    (the next step's prefixes) through the new table equals the oracle's."""
    import tree_draft_verification_amd as tv
    wl = ATTN_CASES["q8_ragged3_N64"]
    a = attn_inputs(wl)
    pg = paged_layout(a["k_cache"], a["v_cache"], 1, seed=48)
    kp, vp, bt = _paged_dev(pg, "bf16")
    lens = i32_dev(a["seq_lens"])
    par = i32_dev(a["parent"])
    msl = int(a["seq_lens"].max())
    tv.tv_tree_verify_attn_paged(to_dev(a["q"], "bf16"), kp, vp, bt, lens, par,
                                 max_seq_len=msl, scale=a["scale"])
    rng = np.random.default_rng(49)
    tgt = rng.integers(0, 20, size=(wl.B, wl.N)).astype(np.int32)
    draft = draft_tokens(a["parent"], draft_coins(wl, a["depth"]), tgt)
    P = 32
    path = i32_dev(np.zeros((wl.B, P), np.int32))
    plen = i32_dev(np.zeros(wl.B, np.int32))
    bonus = i32_dev(np.zeros(wl.B, np.int32))
    tv.tv_tree_accept(par, i32_dev(draft), i32_dev(tgt), P, path=path, path_len=plen, bonus=bonus)
    tv.tv_kv_commit_slots(bt, lens, path, plen, wl.N)
    acc = oracle.tree_accept(a["parent"], draft, tgt, P=P)
    kc, vc, lc = oracle.kv_compact(a["k_cache"], a["v_cache"], a["seq_lens"], acc["path"],
                                   acc["path_len"])
    np.testing.assert_array_equal(lens.cpu().numpy(), lc)
    new_bt = bt.cpu().numpy()
    gk = oracle.paged_to_contiguous(pg["k_pages"], new_bt, 1, a["Lcap"])
    gv = oracle.paged_to_contiguous(pg["v_pages"], new_bt, 1, a["Lcap"])
    for b in range(wl.B):
        n = int(lc[b])
        np.testing.assert_array_equal(gk[b, :, :n], kc[b, :, :n])
        np.testing.assert_array_equal(gv[b, :, :n], vc[b, :, :n])
    # the next step: prefixes of the new lengths, trees on the rows after
    # them (the caller's slots for those rows: the rejected ones, then fresh
    # ones past the tree window, as laid out by the pool)
    n_next = 8
    par2 = np.tile(np.arange(-1, n_next - 1, dtype=np.int32), (wl.B, 1))
    q2 = a["q"][:, :n_next]
    out = tv.tv_tree_verify_attn_paged(to_dev(q2, "bf16"), kp, vp, bt, lens, i32_dev(par2),
                                       max_seq_len=int(lc.max()), scale=a["scale"])
    ref = oracle.tree_attention_paged(q2, pg["k_pages"], pg["v_pages"], new_bt, 1, lc, par2,
                                      a["scale"], "bf16")
    assert_attn_close(to_host_f64(out), ref, "slot-table next step")


def test_compact_paged_hazard_rows_cross_pages():
    """Moves whose source and destination rows sit on different pages, with
    every row of the path moving (page size 16, path of stride 2)."""
    import tree_draft_verification_amd as tv
    B, Hkv, D, L, N, P, ps = 2, 3, 128, 13, 64, 32, 16
    rng = np.random.default_rng(46)
    kc = rng.integers(0, 65535, size=(B, Hkv, 96, D)).astype(np.uint16)
    vc = rng.integers(0, 65535, size=(B, Hkv, 96, D)).astype(np.uint16)
    pg = paged_layout(kc, vc, ps, seed=47)
    path = np.full((B, P), -1, np.int32)
    path[0, :20] = np.arange(0, 40, 2)
    path[1, :32] = np.concatenate([[0], np.arange(1, 32) + 30])
    plen = np.array([20, 32], np.int32)
    lens = np.array([L, L + 1], np.int32)
    k2, v2, lens2 = oracle.kv_compact_paged(pg["k_pages"], pg["v_pages"], pg["block_table"], ps,
                                            lens, path, plen)
    kp, vp, bt = _paged_dev(pg, "bf16")
    sl = i32_dev(lens)
    tv.tv_kv_compact_paged(kp, vp, bt, sl, i32_dev(path), i32_dev(plen))
    np.testing.assert_array_equal(to_host_bits(kp), k2)
    np.testing.assert_array_equal(to_host_bits(vp), v2)
    np.testing.assert_array_equal(sl.cpu().numpy(), lens2)


# ---------------------------------------------------------------- graph replay

def test_step_graph_replay_matches_eager():
    """The four calls of a step captured once as a HIP graph (as bench.py times
    them) replay bit for bit like the same calls launched one by one, on every
    replay, with the caches and lengths restored in between by ordinary work."""
    import torch
    import tree_draft_verification_amd as tv
    wl = ATTN_CASES["q8_ragged3_N64"].replace(V=5000, hidden=512)
    a = attn_inputs(wl)
    lm = lmhead_inputs(wl)
    tgt = oracle.lm_head_argmax(lm["hidden"], lm["w"], wl.dtype)["argmax"].reshape(wl.B, wl.N)
    draft = i32_dev(draft_tokens(a["parent"], draft_coins(wl, a["depth"]), tgt))
    q = to_dev(a["q"], "bf16")
    k0, v0 = to_dev(a["k_cache"], "bf16"), to_dev(a["v_cache"], "bf16")
    k, v = k0.clone(), v0.clone()
    lens0 = i32_dev(a["seq_lens"])
    lens = lens0.clone()
    par = i32_dev(a["parent"])
    hid = to_dev(lm["hidden"], "bf16")
    w = tv.tv_lmhead_pack_weights(to_dev(lm["w"], "bf16"))
    msl = int(a["seq_lens"].max())
    out = torch.empty_like(q)
    arg = torch.empty(wl.B * wl.N, dtype=torch.int32, device="cuda")
    P = 32
    path = torch.empty((wl.B, P), dtype=torch.int32, device="cuda")
    plen = torch.empty(wl.B, dtype=torch.int32, device="cuda")
    bonus = torch.empty(wl.B, dtype=torch.int32, device="cuda")
    aws = torch.zeros(max(256, tv.tv_tree_verify_attn_workspace(wl.B, wl.N, wl.Hq, wl.Hkv, wl.D,
                                                                msl, tv.TV_BF16)),
                      dtype=torch.uint8, device="cuda")
    lws = torch.zeros(tv.tv_lmhead_argmax_workspace(wl.B * wl.N, wl.hidden, wl.V, tv.TV_BF16),
                      dtype=torch.uint8, device="cuda")

    def step():
        tv.tv_tree_verify_attn(q, k, v, lens, par, out, max_seq_len=msl, scale=a["scale"],
                               workspace=aws)
        tv.tv_lmhead_argmax(hid, w, arg, workspace=lws)
        tv.tv_tree_accept(par, draft, arg, P, path=path, path_len=plen, bonus=bonus)
        tv.tv_kv_compact(k, v, lens, path, plen)

    def state():
        return [t.clone() for t in (out, arg, path, plen, bonus, k, v, lens)]

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
        s.synchronize()
        eager = state()
        k.copy_(k0), v.copy_(v0), lens.copy_(lens0)
        tv.tv_graph_begin(s)
        step()
        graph = tv.tv_graph_end(s)
        for rep in range(3):
            k.copy_(k0), v.copy_(v0), lens.copy_(lens0)
            out.zero_(), arg.zero_(), plen.zero_()
            graph.launch(s)
            s.synchronize()
            for i, (x, y) in enumerate(zip(state(), eager)):
                assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                                   y.view(torch.int16) if y.dtype == torch.bfloat16 else y), \
                    f"replay {rep}: output {i} differs from the eager step"
    assert int(plen.min()) >= 1


@pytest.mark.parametrize("name", ["tiny_fp32", "q8_ragged3_N64", "a3b_B2_L257_N200",
                                  "g1_L64_N130"])
def test_accept_compact_equals_the_two_calls(name):
    """tv_accept_compact gives bit for bit what tv_tree_accept then
    tv_kv_compact give, on workload trees with the GPU's own argmax as the
    target and with planted bad trees and too-long paths."""
    import torch
    import tree_draft_verification_amd as tv
    wl = ATTN_CASES[name]
    a = attn_inputs(wl)
    rng = np.random.default_rng(wl.seed + 99)
    tgt = rng.integers(0, 50, size=(wl.B, wl.N)).astype(np.int32)
    draft = draft_tokens(a["parent"], draft_coins(wl, a["depth"]), tgt)
    parent = a["parent"].copy()
    if wl.B > 1:
        parent[1, min(3, wl.N - 1)] = wl.N + 5 if wl.N > 3 else parent[1, 0]  # malformed tree
    for P in (32, 2):  # 2: paths longer than P are rejected with a flag
        ref_k, ref_v = to_dev(a["k_cache"], wl.dtype), to_dev(a["v_cache"], wl.dtype)
        got_k, got_v = ref_k.clone(), ref_v.clone()
        ref_l, got_l = i32_dev(a["seq_lens"]), i32_dev(a["seq_lens"])
        st_ref = torch.zeros(wl.B, dtype=torch.int32, device="cuda")
        st_got = torch.zeros(wl.B, dtype=torch.int32, device="cuda")
        par, dr, tg = i32_dev(parent), i32_dev(draft), i32_dev(tgt)
        p1, l1, b1 = tv.tv_tree_accept(par, dr, tg, P, dev_status=st_ref)
        tv.tv_kv_compact(ref_k, ref_v, ref_l, p1, l1)
        p2, l2, b2 = tv.tv_accept_compact(par, dr, tg, got_k, got_v, got_l, P, dev_status=st_got)
        torch.cuda.synchronize()
        for x, y in ((p1, p2), (l1, l2), (b1, b2), (ref_l, got_l), (st_ref, st_got)):
            assert torch.equal(x, y), name
        for x, y in ((ref_k, got_k), (ref_v, got_v)):  # caches bit for bit
            assert np.array_equal(x.cpu().view(torch.int16 if wl.dtype == "bf16" else torch.int32),
                                  y.cpu().view(torch.int16 if wl.dtype == "bf16" else torch.int32))
        # and against the oracle, on every sequence the call did not flag
        # (a flagged sequence's outputs are unspecified)
        st_h = st_got.cpu().numpy()
        gk, gv = to_host_bits(got_k), to_host_bits(got_v)
        p_h, l_h, b_h, len_h = (t.cpu().numpy() for t in (p2, l2, b2, got_l))
        checked = 0
        for b in range(wl.B):
            if st_h[b]:
                continue
            acc = oracle.tree_accept(parent[b:b + 1], draft[b:b + 1], tgt[b:b + 1], 64)
            n = int(acc["path_len"][0])
            assert l_h[b] == n and b_h[b] == acc["bonus"][0], (name, b)
            np.testing.assert_array_equal(p_h[b], acc["path"][0, :P])
            k2, v2, lens2 = oracle.kv_compact(a["k_cache"][b:b + 1], a["v_cache"][b:b + 1],
                                              a["seq_lens"][b:b + 1], acc["path"],
                                              acc["path_len"])
            assert len_h[b] == lens2[0]
            np.testing.assert_array_equal(gk[b], k2[0])
            np.testing.assert_array_equal(gv[b], v2[0])
            checked += 1
        if P == 32:
            assert checked >= max(1, wl.B - 1), name
