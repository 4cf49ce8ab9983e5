"""CPU checks of the C-ABI library: it loads, exports every declared symbol,
and rejects bad arguments on the host before touching the GPU.

Only calls that fail host validation are made here (no GPU is needed); the
library is built first if it is not there yet.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "treeverify.h")


def _lib_path():
    from tree_draft_verification_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from tree_draft_verification_amd.build import build
        build()
    return _lib.LIB_PATH


@pytest.fixture(scope="module")
def lib():
    from tree_draft_verification_amd import _lib
    return _lib.load(_lib_path())


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tv_\w+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for n in ("tv_tree_verify_attn", "tv_lmhead_argmax", "tv_tree_accept", "tv_kv_compact",
              "tv_tree_verify_attn_workspace", "tv_lmhead_argmax_workspace",
              "tv_lmhead_packed_bytes", "tv_lmhead_pack_weights", "tv_pack_gate_up_weights",
              "tv_accept_compact",
              "tv_tree_verify_attn_paged", "tv_tree_verify_attn_paged_workspace",
              "tv_kv_compact_paged", "tv_kv_commit_slots", "tv_verify_pass",
              "tv_verify_pass_workspace",
              "tv_kv_compact_layers", "tv_kv_compact_layers_workspace", "tv_graph_begin",
              "tv_graph_end", "tv_graph_launch", "tv_graph_destroy", "tv_tree_build",
              "tv_tree_build_workspace", "tv_status_string", "tv_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (tv_\w+)", out))
    missing = [n for n in _declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    from tree_draft_verification_amd import _lib
    assert set(_lib.SIGNATURES) == set(_declared_functions())


def test_status_strings_and_version(lib):
    assert lib.tv_abi_version() == 10000
    for code in (0, -1, -2, -3, -4):
        assert lib.tv_status_string(code)
    assert lib.tv_status_string(-99) == b"unknown status"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def _attn(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sl=FAKE, par=FAKE, out=FAKE, B=1, N=64, Hq=32, Hkv=8,
             D=128, Lcap=2048, msl=1024, scale=0.088, dtype=0, ws=FAKE, wsb=1 << 30,
             st=None, stream=None)
    a.update(kw)
    return lib.tv_tree_verify_attn(a["q"], a["k"], a["v"], a["sl"], a["par"], a["out"],
                                   a["B"], a["N"], a["Hq"], a["Hkv"], a["D"], a["Lcap"],
                                   a["msl"], a["scale"], a["dtype"], a["ws"], a["wsb"],
                                   a["st"], a["stream"])


def test_attention_host_validation(lib):
    assert _attn(lib, q=None) == -1
    assert _attn(lib, out=None) == -1
    assert _attn(lib, Hq=30) == -1                       # Hq % Hkv
    assert _attn(lib, msl=2000) == -1                    # max_seq_len + N > Lcap
    assert _attn(lib, N=0) == -1
    assert _attn(lib, scale=float("nan")) == -1
    assert _attn(lib, D=96) == -2
    assert _attn(lib, dtype=7) == -2
    assert _attn(lib, N=1025, Lcap=4096) == -2
    need = lib.tv_tree_verify_attn_workspace(1, 64, 32, 8, 128, 1024, 0)
    assert need > 0                                      # the prefix is split
    assert _attn(lib, ws=None) == -3
    assert _attn(lib, wsb=need - 1) == -3
    assert lib.tv_tree_verify_attn_workspace(4, 1024, 32, 4, 128, 4096, 0) == 0


def test_lmhead_host_validation(lib):
    ws = lib.tv_lmhead_argmax_workspace(64, 4096, 151936, 0)
    assert ws >= 64 * 8
    f = lib.tv_lmhead_argmax
    assert f(None, FAKE, FAKE, None, 64, 4096, 151936, 0, 0, FAKE, ws, None) == -1
    assert f(FAKE, FAKE, None, None, 64, 4096, 151936, 0, 0, FAKE, ws, None) == -1
    assert f(FAKE, FAKE, FAKE, None, 0, 4096, 151936, 0, 0, FAKE, ws, None) == -1
    assert f(FAKE, FAKE, FAKE, None, 64, 4096, 151936, 0, 2, FAKE, ws, None) == -1   # layout
    assert f(FAKE, FAKE, FAKE, None, 64, 4000, 151936, 0, 0, FAKE, ws, None) == -2
    assert f(FAKE, FAKE, FAKE, None, 64, 4224, 151936, 0, 1, FAKE, ws, None) == -2   # K % 256
    assert f(FAKE, FAKE, FAKE, None, 64, 4096, 151936, 5, 0, FAKE, ws, None) == -2
    assert f(FAKE, FAKE, FAKE, None, 64, 4096, 151936, 1, 1, FAKE, ws, None) == -2   # f32 packed
    assert f(FAKE, FAKE, FAKE, None, 64, 4096, 151936, 0, 0, None, ws, None) == -3
    assert f(FAKE, FAKE, FAKE, None, 64, 4096, 151936, 0, 0, FAKE, ws - 1, None) == -3


def test_lmhead_noalloc_host_validation(lib):
    """The allocation-free LM head checks its arguments as the workspace
    call does, and rejects shapes beyond its device array before any HIP
    call (TV_ESCRATCH)."""
    from tree_draft_verification_amd import _lib
    f = lib.tv_lmhead_argmax_noalloc
    assert f(None, FAKE, FAKE, None, 64, 4096, 151936, 0, 1, None) == -1
    assert f(FAKE, FAKE, None, None, 64, 4096, 151936, 0, 1, None) == -1
    assert f(FAKE, FAKE, FAKE, None, 0, 4096, 151936, 0, 1, None) == -1
    assert f(FAKE, FAKE, FAKE, None, 64, 4096, 151936, 0, 7, None) == -1   # layout
    assert f(FAKE, FAKE, FAKE, None, 64, 100, 151936, 0, 1, None) == -2    # K % 256
    assert f(FAKE, FAKE, FAKE, None, 64, 4096, 151936, 1, 1, None) == -2   # f32 packed
    assert f(FAKE, FAKE, FAKE, None, 8192, 2048, 151936, 0, 1, None) == _lib.TV_ESCRATCH
    assert lib.tv_lmhead_argmax_workspace(8192, 2048, 151936, 0) > _lib.TV_NOALLOC_SCRATCH_BYTES
    assert lib.tv_lmhead_argmax_workspace(4096, 2048, 151936, 0) <= _lib.TV_NOALLOC_SCRATCH_BYTES
    assert b"allocation-free" in lib.tv_status_string(_lib.TV_ESCRATCH)


def test_pack_host_validation(lib):
    assert lib.tv_lmhead_packed_bytes(151936, 4096, 0) == 151936 * 4096 * 2
    assert lib.tv_lmhead_packed_bytes(1000, 256, 0) == 1024 * 256 * 2      # whole 128-row tiles
    assert lib.tv_lmhead_packed_bytes(1000, 384, 0) == 0
    assert lib.tv_lmhead_packed_bytes(1000, 256, 1) == 0
    p = lib.tv_lmhead_pack_weights
    assert p(None, FAKE, 1000, 256, 0, None) == -1
    assert p(FAKE, FAKE, 1000, 256, 0, None) == -1                         # in place
    assert p(FAKE, ctypes.c_void_p(0x2000), 0, 256, 0, None) == -1
    assert p(FAKE, ctypes.c_void_p(0x2000), 1000, 384, 0, None) == -2
    assert p(FAKE, ctypes.c_void_p(0x2000), 1000, 256, 1, None) == -2
    g = lib.tv_pack_gate_up_weights
    assert g(None, FAKE, 512, 256, 0, None) == -1
    assert g(FAKE, FAKE, 512, 256, 0, None) == -1                          # in place
    assert g(FAKE, ctypes.c_void_p(0x2000), 0, 256, 0, None) == -1
    assert g(FAKE, ctypes.c_void_p(0x2000), 500, 256, 0, None) == -2        # inter % 64
    assert g(FAKE, ctypes.c_void_p(0x2000), 512, 384, 0, None) == -2
    assert g(FAKE, ctypes.c_void_p(0x2000), 512, 256, 1, None) == -2


def test_accept_and_compact_host_validation(lib):
    a = lib.tv_tree_accept
    assert a(None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 32, None, None) == -1
    assert a(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 32, None, None) == -1
    assert a(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2048, 32, None, None) == -2
    assert a(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 65, None, None) == -2
    c = lib.tv_kv_compact
    assert c(None, FAKE, FAKE, FAKE, FAKE, 1, 8, 128, 2048, 32, 0, None) == -1
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 128, 2048, 0, 0, None) == -1
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 4, 2048, 32, 0, None) == -2   # 8-byte rows
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 128, 2048, 32, 3, None) == -2
    ac = lib.tv_accept_compact
    # valid arguments apart from the one changed in each case (no call reaches the device)
    args = [FAKE] * 9 + [2, 64, 32, 8, 128, 2048, 0, None, None]
    bad = list(args); bad[0] = None
    assert ac(*bad) == -1
    bad = list(args); bad[8] = None
    assert ac(*bad) == -1                       # seq_lens
    bad = list(args); bad[10] = 0
    assert ac(*bad) == -1                       # N
    bad = list(args); bad[10] = 1025
    assert ac(*bad) == -2                       # N > TV_MAX_NODES
    bad = list(args); bad[11] = 65
    assert ac(*bad) == -2                       # P > 64
    bad = list(args); bad[13] = 4
    assert ac(*bad) == -2                       # 8-byte rows
    bad = list(args); bad[15] = 7
    assert ac(*bad) == -2                       # dtype


def _attn_paged(lib, **kw):
    a = dict(q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, mb=68, ps=16, npg=100, sl=FAKE, par=FAKE,
             out=FAKE, B=1, N=64, Hq=32, Hkv=8, D=128, msl=1024, scale=0.088, dtype=0, ws=FAKE,
             wsb=1 << 30, st=None, stream=None)
    a.update(kw)
    return lib.tv_tree_verify_attn_paged(
        a["q"], a["kp"], a["vp"], a["bt"], a["mb"], a["ps"], a["npg"], a["sl"], a["par"],
        a["out"], a["B"], a["N"], a["Hq"], a["Hkv"], a["D"], a["msl"], a["scale"], a["dtype"],
        a["ws"], a["wsb"], a["st"], a["stream"])


def test_paged_host_validation(lib):
    assert _attn_paged(lib, bt=None) == -1
    assert _attn_paged(lib, ps=24) == -1                 # not a power of two
    assert _attn_paged(lib, ps=0) == -1                  # below one row
    assert _attn_paged(lib, ps=8192) == -1               # above 4096 rows
    assert _attn_paged(lib, mb=67) == -1                 # 67 * 16 < 1024 + 64
    assert _attn_paged(lib, npg=0) == -1
    assert _attn_paged(lib, Hq=30) == -1
    assert _attn_paged(lib, dtype=1) == -2               # paged attention: bf16 only
    assert _attn_paged(lib, D=96) == -2
    assert _attn_paged(lib, N=1025, mb=200) == -2
    need = lib.tv_tree_verify_attn_paged_workspace(1, 64, 32, 8, 128, 1024, 16, 0)
    assert need > 0
    assert _attn_paged(lib, ws=None) == -3
    assert _attn_paged(lib, wsb=need - 1) == -3
    assert lib.tv_tree_verify_attn_paged_workspace(1, 64, 32, 8, 128, 1024, 12, 0) == 0
    # pages look up their entries per row, so the split plan (and the
    # workspace) does not depend on the page size
    long_c = lib.tv_tree_verify_attn_workspace(1, 64, 32, 8, 128, 1 << 20, 0)
    for ps in (1, 16, 4096):
        assert lib.tv_tree_verify_attn_paged_workspace(1, 64, 32, 8, 128, 1 << 20, ps, 0) == long_c > 0
    c = lib.tv_kv_compact_paged
    assert c(None, FAKE, FAKE, 68, 16, 100, FAKE, FAKE, FAKE, 1, 8, 128, 32, 0, None) == -1
    assert c(FAKE, FAKE, FAKE, 68, 20, 100, FAKE, FAKE, FAKE, 1, 8, 128, 32, 0, None) == -1
    assert c(FAKE, FAKE, FAKE, 0, 16, 100, FAKE, FAKE, FAKE, 1, 8, 128, 32, 0, None) == -1
    assert c(FAKE, FAKE, FAKE, 68, 16, 100, FAKE, FAKE, FAKE, 1, 8, 4, 32, 0, None) == -2
    assert c(FAKE, FAKE, FAKE, 68, 16, 100, FAKE, FAKE, FAKE, 1, 8, 128, 65, 0, None) == -2
    c = lib.tv_kv_commit_slots   # table, lens, path, path_len, B, N, P, max_blocks, status, stream
    assert c(None, FAKE, FAKE, FAKE, 2, 64, 32, 2048, None, None) == -1
    assert c(FAKE, FAKE, FAKE, FAKE, 0, 64, 32, 2048, None, None) == -1
    assert c(FAKE, FAKE, FAKE, FAKE, 2, 0, 32, 2048, None, None) == -1
    assert c(FAKE, FAKE, FAKE, FAKE, 2, 64, 0, 2048, None, None) == -1
    assert c(FAKE, FAKE, FAKE, FAKE, 2, 1025, 32, 2048, None, None) == -2
    assert c(FAKE, FAKE, FAKE, FAKE, 2, 64, 65, 2048, None, None) == -2
    assert c(FAKE, FAKE, FAKE, FAKE, 2, 64, 32, 63, None, None) == -2


def _pass(lib, dims=None, weights=None, **kw):
    from tree_draft_verification_amd import _lib
    d = dims or _lib.ModelDims(2, 256, 4, 2, 64, 512, 1000, 1e-6, 1e6)
    w = weights or _lib.ModelWeights(*([0x1000] * 11))
    a = dict(tok=FAKE, par=FAKE, sl=FAKE, k=FAKE, v=FAKE, B=2, N=12, Lcap=128, msl=100,
             arg=FAKE, lg=None, hid=None, ws=FAKE, wsb=1 << 30, st=None, stream=None)
    a.update(kw)
    return lib.tv_verify_pass(ctypes.byref(d), ctypes.byref(w), a["tok"], a["par"], a["sl"],
                              a["k"], a["v"], a["B"], a["N"], a["Lcap"], a["msl"], a["arg"],
                              a["lg"], a["hid"], a["ws"], a["wsb"], a["st"], a["stream"])


def test_pass_host_validation(lib):
    from tree_draft_verification_amd import _lib
    D = _lib.ModelDims
    d = D(2, 256, 4, 2, 64, 512, 1000, 1e-6, 1e6)
    need = lib.tv_verify_pass_workspace(ctypes.byref(d), 2, 12, 100)
    assert need > 0
    assert _pass(lib, tok=None) == -1
    assert _pass(lib, weights=_lib.ModelWeights(*([0x1000] * 10 + [0]))) == -1  # lm_head NULL
    assert _pass(lib, msl=120) == -1                      # max_seq_len + N > Lcap
    assert _pass(lib, dims=D(2, 256, 3, 2, 64, 512, 1000, 1e-6, 1e6)) == -1    # Hq % Hkv
    assert _pass(lib, dims=D(2, 256, 4, 2, 64, 512, 1000, 1e-6, 1.0)) == -1    # rope_theta
    assert _pass(lib, dims=D(2, 256, 4, 2, 96, 512, 1000, 1e-6, 1e6)) == -2    # D
    assert _pass(lib, dims=D(2, 320, 4, 2, 64, 512, 1000, 1e-6, 1e6)) == -2    # hidden % 256
    assert _pass(lib, dims=D(2, 256, 4, 2, 64, 640, 1000, 1e-6, 1e6)) == -2    # inter % 256
    assert _pass(lib, N=1025, Lcap=2048) == -2
    assert _pass(lib, ws=None) == -3
    assert _pass(lib, wsb=need - 1) == -3
    c = lib.tv_kv_compact_layers
    cw = lib.tv_kv_compact_layers_workspace(3)
    assert cw >= 12
    assert c(None, FAKE, FAKE, FAKE, FAKE, 3, 8, 128, 2048, 32, 36, 0, FAKE, cw, None) == -1
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 8, 128, 2048, 32, 0, 0, FAKE, cw, None) == -1
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 8, 128, 2048, 65, 36, 0, FAKE, cw, None) == -2
    # plane indexing: layers * (2 Hkv)^2 must stay below 2^32
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 64, 128, 2048, 32, 262144, 0, FAKE, cw, None) == -2
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 8, 128, 2048, 32, 36, 0, None, cw, None) == -3
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 8, 128, 2048, 32, 36, 0, FAKE, cw - 1, None) == -3
    # graphs: the null stream cannot be captured; null handles are rejected
    assert lib.tv_graph_begin(None) == -1
    assert lib.tv_graph_end(None, None) == -1
    assert lib.tv_graph_launch(None, None) == -1
    assert lib.tv_graph_destroy(None) == -1


def test_tree_build_host_validation(lib):
    f = lib.tv_tree_build
    ws = lib.tv_tree_build_workspace(1, 20, 151936, 7)
    assert ws > 0
    ok = dict(lp=FAKE, root=FAKE, B=1, D=20, V=151936, W=7, n=128, par=FAKE, tok=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["lp"], a["root"], a["B"], a["D"], a["V"], a["W"], a["n"], a["par"], a["tok"],
                 None, None, FAKE if "ws" not in kw else kw["ws"], ws, None)
    assert call(lp=None) == -1
    assert call(tok=None) == -1
    assert call(V=5) == -1                       # V < width
    assert call(W=17) == -2                      # width limit
    assert call(D=65) == -2                      # depth limit
    assert call(n=1024) == -2                    # budget + 1 > TV_MAX_NODES
    assert call(W=16, D=17) == -2                # 16 + 16 * 256 > 4096 candidates
    assert call(W=2, D=2, n=7) == -1             # budget above the 6 candidates
    assert call(ws=None) == -3


def test_tree_build_level_host_validation(lib):
    ws = lib.tv_tree_build_level_workspace(1, 20, 151936, 7)
    assert ws > 0
    assert lib.tv_tree_build_level_workspace(1, 20, 151936, 17) == 0
    ok = dict(lp=FAKE, level=1, B=1, D=20, V=151936, W=7, fs=FAKE, ft=FAKE, ws=FAKE, n=ws)

    def lv(**kw):
        a = dict(ok, **kw)
        return lib.tv_tree_build_level(a["lp"], a["level"], a["B"], a["D"], a["V"], a["W"],
                                       a["fs"], a["ft"], a["ws"], a["n"], None)
    assert lv(lp=None) == -1
    assert lv(fs=None) == -1
    assert lv(ft=None) == -1
    assert lv(level=0) == -1
    assert lv(level=21) == -1                    # beyond depth
    assert lv(V=5) == -1                         # V < width
    assert lv(W=17) == -2
    assert lv(D=65) == -2
    assert lv(W=16, D=17) == -2                  # pool above 4096 candidates
    assert lv(ws=None) == -3
    assert lv(n=ws - 1) == -3

    def fin(**kw):
        a = dict(ok, root=FAKE, budget=128, par=FAKE, tok=FAKE)
        a.update(kw)
        return lib.tv_tree_build_finish(a["root"], a["B"], a["D"], a["V"], a["W"], a["budget"],
                                        a["par"], a["tok"], None, None, a["ws"], a["n"], None)
    assert fin(root=None) == -1
    assert fin(par=None) == -1
    assert fin(budget=0) == -1
    assert fin(W=2, D=2, budget=7) == -1         # budget above the 6 candidates
    assert fin(W=8, budget=1024) == -2           # budget + 1 > TV_MAX_NODES (pool 1224)
    assert fin(ws=None) == -3


def test_binding_names_match_the_c_calls():
    import tree_draft_verification_amd as tv
    for n in ("tv_tree_verify_attn", "tv_lmhead_argmax", "tv_tree_accept", "tv_kv_compact",
              "tv_tree_verify_attn_workspace", "tv_lmhead_argmax_workspace",
              "tv_lmhead_packed_bytes", "tv_lmhead_pack_weights", "tv_pack_gate_up_weights",
              "tv_accept_compact",
              "tv_tree_verify_attn_paged", "tv_tree_verify_attn_paged_workspace",
              "tv_kv_compact_paged", "tv_kv_commit_slots", "tv_verify_pass",
              "tv_verify_pass_workspace",
              "tv_kv_compact_layers", "tv_kv_compact_layers_workspace", "tv_graph_begin",
              "tv_graph_end", "tv_graph_launch", "tv_graph_destroy", "tv_status_string",
              "tv_abi_version", "tv_tree_build", "tv_tree_build_workspace",
              "tv_tree_build_level", "tv_tree_build_level_workspace", "tv_tree_build_finish"):
        assert callable(getattr(tv, n))
    assert tv.tv_status_string(-3) == "workspace missing or too small"
