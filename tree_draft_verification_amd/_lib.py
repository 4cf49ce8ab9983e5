"""ctypes handle on libtreeverify.so with the C signatures of include/treeverify.h."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libtreeverify.so")

TV_OK, TV_EINVAL, TV_ENOTSUP, TV_EWORKSPACE, TV_EHIP, TV_ESCRATCH = 0, -1, -2, -3, -4, -5
TV_NOALLOC_SCRATCH_BYTES = 64 << 20
TV_BF16, TV_F32 = 0, 1
TV_LAYOUT_ROWMAJOR, TV_LAYOUT_PACKED = 0, 1
TV_STATUS_BAD_PARENT, TV_STATUS_BAD_LEN, TV_STATUS_DEPTH, TV_STATUS_BAD_PAGE = 1, 2, 4, 8
TV_STATUS_BAD_TOKEN = 16
TV_STATUS_BAD_PATH = 32
TV_MAX_NODES = 1024

_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_f = ctypes.c_float


class ModelDims(ctypes.Structure):
    """tv_model_dims"""
    _fields_ = [("layers", _i), ("hidden", _i), ("Hq", _i), ("Hkv", _i), ("D", _i),
                ("inter", _i), ("vocab", _i), ("rms_eps", _f), ("rope_theta", _f)]


class ModelWeights(ctypes.Structure):
    """tv_model_weights (device pointers)"""
    _fields_ = [(n, _p) for n in ("embed", "ln1", "w_qkv", "q_norm", "k_norm", "w_o", "ln2",
                                  "w_gu", "w_down", "final_norm", "lm_head")]


_pd = ctypes.POINTER(ModelDims)
_pw = ctypes.POINTER(ModelWeights)

SIGNATURES = {
    "tv_tree_verify_attn_workspace": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "tv_tree_verify_attn": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i,
                                 _p, _sz, _p, _p]),
    "tv_tree_verify_attn_paged_workspace": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "tv_tree_verify_attn_paged": (_i, [_p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _i, _i, _i, _i,
                                       _i, _i, _f, _i, _p, _sz, _p, _p]),
    "tv_kv_compact_paged": (_i, [_p, _p, _p, _i, _i, _i, _p, _p, _p, _i, _i, _i, _i, _i, _p]),
    "tv_kv_commit_slots": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _p, _p]),
    "tv_lmhead_argmax_workspace": (_sz, [_i, _i, _i, _i]),
    "tv_lmhead_argmax": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _sz, _p]),
    "tv_lmhead_argmax_noalloc": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p]),
    "tv_lmhead_packed_bytes": (_sz, [_i, _i, _i]),
    "tv_lmhead_pack_weights": (_i, [_p, _p, _i, _i, _i, _p]),
    "tv_pack_gate_up_weights": (_i, [_p, _p, _i, _i, _i, _p]),
    "tv_tree_accept": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _p, _p]),
    "tv_kv_compact": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p]),
    "tv_accept_compact": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i,
                               _p, _p]),
    "tv_verify_pass_workspace": (_sz, [_pd, _i, _i, _i]),
    "tv_verify_pass": (_i, [_pd, _pw, _p, _p, _p, _p, _p, _i, _i, _i, _i, _p, _p, _p, _p, _sz,
                            _p, _p]),
    "tv_kv_compact_layers_workspace": (_sz, [_i]),
    "tv_kv_compact_layers": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _sz, _p]),
    "tv_tree_build_workspace": (_sz, [_i, _i, _i, _i]),
    "tv_tree_build": (_i, [_p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _sz, _p]),
    "tv_tree_build_level_workspace": (_sz, [_i, _i, _i, _i]),
    "tv_tree_build_level": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, _p, _sz, _p]),
    "tv_tree_build_finish": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _sz, _p]),
    "tv_graph_begin": (_i, [_p]),
    "tv_graph_end": (_i, [_p, ctypes.POINTER(_p)]),
    "tv_graph_launch": (_i, [_p, _p]),
    "tv_graph_destroy": (_i, [_p]),
    "tv_status_string": (ctypes.c_char_p, [_i]),
    "tv_abi_version": (_i, []),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -m tree_draft_verification_amd.build); there is no fallback")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib
