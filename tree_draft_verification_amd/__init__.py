"""Tree-verification step of tree speculative decoding on MI355X (gfx950).

Thin Python binding over the C-ABI library libtreeverify.so (declared in
include/treeverify.h).  Functions carry the C names; they check tensor
shapes, pass raw device pointers and the current HIP stream, and raise
TreeVerifyError on a negative status.  Every step of the computation runs in
the library's HIP kernels; torch only provides device memory and streams.
There is no CPU fallback: the first call raises ImportError if the library
is not built.

One verification step (JetSpec GitHub README, "JetSpec > Overview"):
    out        = tv_tree_verify_attn(q, k_cache, v_cache, seq_lens, parent, ...)
    tgt        = tv_lmhead_argmax(hidden, w_vocab)
    path, n, b = tv_tree_accept(parent, draft_tokens, tgt)
    tv_kv_compact(k_cache, v_cache, seq_lens, path, n)
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import (TV_BF16, TV_F32, TV_LAYOUT_PACKED, TV_LAYOUT_ROWMAJOR,  # noqa: F401
                   TV_MAX_NODES, TV_STATUS_BAD_LEN, TV_STATUS_BAD_PAGE, TV_STATUS_BAD_PARENT,
                   TV_STATUS_BAD_PATH, TV_STATUS_BAD_TOKEN, TV_STATUS_DEPTH)

_LIB_HANDLE = None


def _lib_handle():
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _LIB_HANDLE
    if _LIB_HANDLE is None:
        _LIB_HANDLE = _lib.load()
    return _LIB_HANDLE

__all__ = [
    "TreeVerifyError", "tv_tree_verify_attn", "tv_tree_verify_attn_workspace",
    "tv_lmhead_argmax", "tv_lmhead_argmax_workspace", "tv_lmhead_packed_bytes",
    "tv_lmhead_pack_weights", "tv_pack_gate_up_weights", "PackedWeights", "tv_tree_accept",
    "tv_kv_compact", "tv_accept_compact", "tv_status_string", "tv_abi_version", "library_path",
    "tv_tree_verify_attn_paged", "tv_tree_verify_attn_paged_workspace", "tv_kv_compact_paged",
    "tv_kv_commit_slots",
    "Model", "tv_model_pack", "tv_verify_pass", "tv_verify_pass_workspace",
    "tv_kv_compact_layers", "tv_kv_compact_layers_workspace", "Graph", "tv_graph_begin",
    "tv_graph_end", "tv_graph_launch", "tv_graph_destroy", "tv_tree_build",
    "tv_tree_build_workspace", "tv_tree_build_level", "tv_tree_build_level_workspace",
    "tv_tree_build_finish",
]


class TreeVerifyError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {tv_status_string(status)}")
        self.status = status


def library_path() -> str:
    return _lib.LIB_PATH


def tv_status_string(status: int) -> str:
    return _lib_handle().tv_status_string(int(status)).decode()


def tv_abi_version() -> int:
    return int(_lib_handle().tv_abi_version())


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise TreeVerifyError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TV_BF16
    if t.dtype == torch.float32:
        return TV_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _i32(t: torch.Tensor, shape, name: str):
    if t.dtype != torch.int32 or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be int32 of shape {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)}")


_WS_CACHE: dict = {}


def _cached_workspace(kind, nbytes: int, dev: torch.device) -> torch.Tensor:
    """Zero-initialised device scratch reused across calls (grown on demand).

    Calls that share it must be ordered on one stream.  `kind` names what
    may share a buffer: LM-head buffers are kept per (dtype, M, K, V), since
    a call leaves only the part its own shape uses zeroed (at most eight such
    buffers are kept; the least recently used goes first).
    """
    key = (kind, dev)
    buf = _WS_CACHE.pop(key, None)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _WS_CACHE[key] = buf                      # most recently used last
    if isinstance(kind, tuple):
        same = [k for k in _WS_CACHE if isinstance(k[0], tuple) and k[0][0] == kind[0]]
        for k in same[:-8]:
            del _WS_CACHE[k]
    return buf


# ---------------------------------------------------------------- attention

def tv_tree_verify_attn_workspace(B, N, Hq, Hkv, D, max_seq_len, dtype=TV_BF16) -> int:
    return int(_lib_handle().tv_tree_verify_attn_workspace(B, N, Hq, Hkv, D, max_seq_len, dtype))


def tv_tree_verify_attn(q, k_cache, v_cache, seq_lens, parent, out=None, *,
                        max_seq_len: int, scale: float | None = None,
                        workspace: torch.Tensor | None = None,
                        dev_status: torch.Tensor | None = None) -> torch.Tensor:
    """Tree-causal attention.  q [B,N,Hq,D]; caches [B,Hkv,Lcap,D]."""
    B, N, Hq, D = q.shape
    Bk, Hkv, Lcap, Dk = k_cache.shape
    if (Bk, Dk) != (B, D) or v_cache.shape != k_cache.shape:
        raise ValueError("q, k_cache and v_cache shapes disagree")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share a dtype")
    _i32(seq_lens, (B,), "seq_lens")
    _i32(parent, (B, N), "parent")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = tv_tree_verify_attn_workspace(B, N, Hq, Hkv, D, max_seq_len, dt)
    if workspace is None and need > 0:
        workspace = _cached_workspace("attn", need, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib_handle().tv_tree_verify_attn(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(parent), _ptr(out),
        B, N, Hq, Hkv, D, Lcap, int(max_seq_len), float(scale), dt,
        _ptr(workspace), ws_bytes, _ptr(dev_status), _stream(q.device))
    _check("tv_tree_verify_attn", st)
    return out


def tv_tree_verify_attn_paged_workspace(B, N, Hq, Hkv, D, max_seq_len, page_size,
                                        dtype=TV_BF16) -> int:
    return int(_lib_handle().tv_tree_verify_attn_paged_workspace(B, N, Hq, Hkv, D, max_seq_len,
                                                                  page_size, dtype))


def tv_tree_verify_attn_paged(q, k_pages, v_pages, block_table, seq_lens, parent, out=None, *,
                              max_seq_len: int, scale: float | None = None,
                              workspace: torch.Tensor | None = None,
                              dev_status: torch.Tensor | None = None) -> torch.Tensor:
    """Tree-causal attention over paged caches.  q [B,N,Hq,D];
    pools [num_pages,Hkv,page_size,D]; block_table [B,max_blocks] int32."""
    B, N, Hq, D = q.shape
    num_pages, Hkv, page_size, Dk = k_pages.shape
    if Dk != D or v_pages.shape != k_pages.shape:
        raise ValueError("q and the page pools disagree")
    if k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise TypeError("q and the page pools must share a dtype")
    Bt, max_blocks = block_table.shape
    _i32(block_table, (B, max_blocks), "block_table")
    _i32(seq_lens, (B,), "seq_lens")
    _i32(parent, (B, N), "parent")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = tv_tree_verify_attn_paged_workspace(B, N, Hq, Hkv, D, max_seq_len, page_size, dt)
    if workspace is None and need > 0:
        workspace = _cached_workspace("attn", need, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib_handle().tv_tree_verify_attn_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), max_blocks, page_size,
        num_pages, _ptr(seq_lens), _ptr(parent), _ptr(out), B, N, Hq, Hkv, D, int(max_seq_len),
        float(scale), dt, _ptr(workspace), ws_bytes, _ptr(dev_status), _stream(q.device))
    _check("tv_tree_verify_attn_paged", st)
    return out


# ---------------------------------------------------------------- LM head

class PackedWeights:
    """A vocabulary projection repacked by tv_lmhead_pack_weights.

    Holds the packed device buffer and the original shape; pass it to
    tv_lmhead_argmax in place of the [V, K] tensor.
    """

    def __init__(self, data: torch.Tensor, V: int, K: int, dtype: torch.dtype):
        self.data, self.V, self.K, self.dtype = data, V, K, dtype
        self.shape = (V, K)
        self.device = data.device


def tv_lmhead_argmax_workspace(M, K, V, dtype=TV_BF16) -> int:
    return int(_lib_handle().tv_lmhead_argmax_workspace(M, K, V, dtype))


def tv_lmhead_packed_bytes(V, K, dtype=TV_BF16) -> int:
    return int(_lib_handle().tv_lmhead_packed_bytes(V, K, dtype))


def tv_lmhead_pack_weights(w: torch.Tensor) -> PackedWeights:
    """Repack a [V, K] bf16 vocabulary projection once for the fast layout."""
    V, K = w.shape
    dt = _dtype_code(w)
    nbytes = tv_lmhead_packed_bytes(V, K, dt)
    if nbytes == 0:
        raise TreeVerifyError("tv_lmhead_pack_weights", _lib.TV_ENOTSUP)
    out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    st = _lib_handle().tv_lmhead_pack_weights(_ptr(w), _ptr(out), V, K, dt, _stream(w.device))
    _check("tv_lmhead_pack_weights", st)
    return PackedWeights(out, V, K, w.dtype)


def tv_pack_gate_up_weights(w: torch.Tensor) -> torch.Tensor:
    """Pack a [2 inter, K] bf16 gate/up weight (gate rows, then up rows) with
    gate and up rows interleaved per 128-row tile; returns the uint8 buffer."""
    R, K = w.shape
    if R % 2:
        raise ValueError("a gate/up weight has an even number of rows")
    dt = _dtype_code(w)
    nbytes = tv_lmhead_packed_bytes(R, K, dt)
    if nbytes == 0:
        raise TreeVerifyError("tv_pack_gate_up_weights", _lib.TV_ENOTSUP)
    out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    st = _lib_handle().tv_pack_gate_up_weights(_ptr(w.contiguous()), _ptr(out), R // 2, K, dt,
                                               _stream(w.device))
    _check("tv_pack_gate_up_weights", st)
    return out


def tv_lmhead_argmax(hidden, w, argmax=None, logits=None, *,
                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """argmax[r] = argmax_v sum_k hidden[r,k] w[v,k].  hidden [M,K]; w [V,K]
    (a tensor, row-major) or a PackedWeights.

    A caller-supplied workspace must be zero-filled before its first use.
    """
    M, K = hidden.shape
    V, Kw = w.shape
    if Kw != K or w.dtype != hidden.dtype:
        raise ValueError("hidden and w disagree in width or dtype")
    dt = _dtype_code(hidden)
    if isinstance(w, PackedWeights):
        layout, wptr = TV_LAYOUT_PACKED, _ptr(w.data)
    else:
        layout, wptr = TV_LAYOUT_ROWMAJOR, _ptr(w)
    if argmax is None:
        argmax = torch.empty(M, dtype=torch.int32, device=hidden.device)
    _i32(argmax, (M,), "argmax")
    if logits is not None and (logits.dtype != torch.float32 or tuple(logits.shape) != (M, V)):
        raise ValueError("logits must be float32 of shape (M, V)")
    need = tv_lmhead_argmax_workspace(M, K, V, dt)
    if workspace is None:
        workspace = _cached_workspace(("lmhead", dt, M, K, V), need, hidden.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib_handle().tv_lmhead_argmax(_ptr(hidden), wptr, _ptr(argmax), _ptr(logits), M, K, V, dt,
                               layout, _ptr(workspace), ws_bytes, _stream(hidden.device))
    _check("tv_lmhead_argmax", st)
    return argmax


# ---------------------------------------------------------------- accept

def tv_tree_accept(parent, draft_tokens, target_tokens, P: int = 32, *, path=None,
                   path_len=None, bonus=None, dev_status=None):
    """Longest accepted path + bonus token; returns (path [B,P], path_len [B], bonus [B])."""
    B, N = parent.shape
    _i32(parent, (B, N), "parent")
    _i32(draft_tokens, (B, N), "draft_tokens")
    target_tokens = target_tokens.reshape(B, N)
    _i32(target_tokens, (B, N), "target_tokens")
    dev = parent.device
    if path is None:
        path = torch.empty((B, P), dtype=torch.int32, device=dev)
    if path_len is None:
        path_len = torch.empty(B, dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty(B, dtype=torch.int32, device=dev)
    _i32(path, (B, P), "path")
    _i32(path_len, (B,), "path_len")
    _i32(bonus, (B,), "bonus")
    st = _lib_handle().tv_tree_accept(_ptr(parent), _ptr(draft_tokens), _ptr(target_tokens),
                             _ptr(path), _ptr(path_len), _ptr(bonus), B, N, P,
                             _ptr(dev_status), _stream(dev))
    _check("tv_tree_accept", st)
    return path, path_len, bonus


# ---------------------------------------------------------------- compaction

def tv_kv_compact(k_cache, v_cache, seq_lens, path, path_len) -> None:
    """Move the accepted rows to L_b + j in place and add path_len to seq_lens."""
    B, Hkv, Lcap, D = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache disagree")
    dt = _dtype_code(k_cache)
    _i32(seq_lens, (B,), "seq_lens")
    P = path.shape[1]
    _i32(path, (B, P), "path")
    _i32(path_len, (B,), "path_len")
    st = _lib_handle().tv_kv_compact(_ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(path),
                            _ptr(path_len), B, Hkv, D, Lcap, P, dt, _stream(k_cache.device))
    _check("tv_kv_compact", st)


def tv_accept_compact(parent, draft_tokens, target_tokens, k_cache, v_cache, seq_lens,
                      P: int = 32, *, path=None, path_len=None, bonus=None, dev_status=None):
    """tv_tree_accept then tv_kv_compact in one launch; returns (path, path_len, bonus)."""
    B, N = parent.shape
    _i32(parent, (B, N), "parent")
    _i32(draft_tokens, (B, N), "draft_tokens")
    target_tokens = target_tokens.reshape(B, N)
    _i32(target_tokens, (B, N), "target_tokens")
    Bk, Hkv, Lcap, D = k_cache.shape
    if Bk != B or v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache disagree with each other or with the batch")
    _i32(seq_lens, (B,), "seq_lens")
    dev = parent.device
    if path is None:
        path = torch.empty((B, P), dtype=torch.int32, device=dev)
    if path_len is None:
        path_len = torch.empty(B, dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty(B, dtype=torch.int32, device=dev)
    _i32(path, (B, P), "path")
    _i32(path_len, (B,), "path_len")
    _i32(bonus, (B,), "bonus")
    st = _lib_handle().tv_accept_compact(
        _ptr(parent), _ptr(draft_tokens), _ptr(target_tokens), _ptr(path), _ptr(path_len),
        _ptr(bonus), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), B, N, P, Hkv, D, Lcap,
        _dtype_code(k_cache), _ptr(dev_status), _stream(dev))
    _check("tv_accept_compact", st)
    return path, path_len, bonus


def tv_kv_compact_paged(k_pages, v_pages, block_table, seq_lens, path, path_len) -> None:
    """Paged compaction: the moves of tv_kv_compact through the block table."""
    num_pages, Hkv, page_size, D = k_pages.shape
    if v_pages.shape != k_pages.shape or v_pages.dtype != k_pages.dtype:
        raise ValueError("k_pages and v_pages disagree")
    dt = _dtype_code(k_pages)
    B, max_blocks = block_table.shape
    _i32(block_table, (B, max_blocks), "block_table")
    _i32(seq_lens, (B,), "seq_lens")
    P = path.shape[1]
    _i32(path, (B, P), "path")
    _i32(path_len, (B,), "path_len")
    st = _lib_handle().tv_kv_compact_paged(
        _ptr(k_pages), _ptr(v_pages), _ptr(block_table), max_blocks, page_size, num_pages,
        _ptr(seq_lens), _ptr(path), _ptr(path_len), B, Hkv, D, P, dt, _stream(k_pages.device))
    _check("tv_kv_compact_paged", st)


def tv_kv_commit_slots(block_table, seq_lens, path, path_len, N: int, dev_status=None) -> None:
    """Commit on a slot table (one row per page): permutes each sequence's
    tree window of the table and advances the lengths; no K/V row moves."""
    B, max_blocks = block_table.shape
    _i32(block_table, (B, max_blocks), "block_table")
    _i32(seq_lens, (B,), "seq_lens")
    P = path.shape[1]
    _i32(path, (B, P), "path")
    _i32(path_len, (B,), "path_len")
    if dev_status is not None:
        _i32(dev_status, (B,), "dev_status")
    st = _lib_handle().tv_kv_commit_slots(
        _ptr(block_table), _ptr(seq_lens), _ptr(path), _ptr(path_len), B, int(N), P, max_blocks,
        _ptr(dev_status) if dev_status is not None else None, _stream(block_table.device))
    _check("tv_kv_commit_slots", st)


# ---------------------------------------------------------------- multi-layer pass

_PACKED = ("w_qkv", "w_o", "w_gu", "w_down")


class Model:
    """Device-resident weights of a decoder stack in the layout tv_verify_pass
    reads (see tv_model_pack); holds the buffers the C structs point to."""

    def __init__(self, dims: dict, bufs: dict):
        self.dims = dict(dims)
        self.bufs = bufs
        self.c_dims = _lib.ModelDims(dims["layers"], dims["hidden"], dims["Hq"], dims["Hkv"],
                                     dims["D"], dims["inter"], dims["V"], dims["eps"],
                                     dims["theta"])
        self.c_weights = _lib.ModelWeights(*[bufs[n].data_ptr() for n, _ in
                                             _lib.ModelWeights._fields_])
        self.device = bufs["embed"].device


def tv_model_pack(dims: dict, w: dict) -> Model:
    """Stack a model's bf16 device weights for tv_verify_pass.

    dims: layers, hidden, Hq, Hkv, D, inter, V, eps, theta.  w: bf16 tensors
    embed [V,hidden], ln1/ln2 [layers,hidden], q_norm/k_norm [layers,D],
    w_qkv [layers,(Hq+2Hkv)D,hidden], w_o [layers,hidden,Hq D],
    w_gu [layers,2 inter,hidden], w_down [layers,hidden,inter],
    final_norm [hidden], lm_head [V,hidden].  Each projection of each layer is
    repacked with tv_lmhead_pack_weights (w_gu with tv_pack_gate_up_weights)
    into one buffer per projection.
    """
    bufs = {k: w[k].contiguous() for k in ("embed", "ln1", "ln2", "q_norm", "k_norm",
                                            "final_norm")}
    for k in _PACKED:
        t = w[k]
        Ly, R, K = t.shape
        per = tv_lmhead_packed_bytes(R, K, TV_BF16)
        if per == 0:
            raise TreeVerifyError("tv_model_pack", _lib.TV_ENOTSUP)
        out = torch.empty(Ly * per, dtype=torch.uint8, device=t.device)
        for ly in range(Ly):
            src = t[ly].contiguous()
            if k == "w_gu":
                st = _lib_handle().tv_pack_gate_up_weights(_ptr(src), out.data_ptr() + ly * per,
                                                           R // 2, K, TV_BF16, _stream(t.device))
                _check("tv_pack_gate_up_weights", st)
            else:
                st = _lib_handle().tv_lmhead_pack_weights(_ptr(src), out.data_ptr() + ly * per,
                                                          R, K, TV_BF16, _stream(t.device))
                _check("tv_lmhead_pack_weights", st)
        bufs[k] = out
    bufs["lm_head"] = tv_lmhead_pack_weights(w["lm_head"]).data
    return Model(dims, bufs)


def tv_verify_pass_workspace(model: Model, B: int, N: int, max_seq_len: int) -> int:
    return int(_lib_handle().tv_verify_pass_workspace(model.c_dims, B, N, max_seq_len))


def tv_verify_pass(model: Model, tokens, parent, seq_lens, k_cache, v_cache, argmax=None, *,
                   max_seq_len: int, logits=None, hidden_out=None, workspace=None,
                   dev_status=None) -> torch.Tensor:
    """The multi-layer pass; caches [layers,B,Hkv,Lcap,D] bf16.  Returns argmax [B*N]."""
    B, N = tokens.shape
    d = model.dims
    Ly, Bk, Hkv, Lcap, D = k_cache.shape
    if (Ly, Bk, Hkv, D) != (d["layers"], B, d["Hkv"], d["D"]) or v_cache.shape != k_cache.shape:
        raise ValueError("caches do not match the model and batch")
    if k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise TypeError("caches must be bfloat16")
    _i32(tokens, (B, N), "tokens")
    _i32(parent, (B, N), "parent")
    _i32(seq_lens, (B,), "seq_lens")
    M = B * N
    dev = tokens.device
    if argmax is None:
        argmax = torch.empty(M, dtype=torch.int32, device=dev)
    _i32(argmax, (M,), "argmax")
    if logits is not None and (logits.dtype != torch.float32
                               or tuple(logits.shape) != (M, d["V"])):
        raise ValueError("logits must be float32 of shape (B*N, V)")
    if hidden_out is not None and (hidden_out.dtype != torch.float32
                                   or tuple(hidden_out.shape) != (M, d["hidden"])):
        raise ValueError("hidden_out must be float32 of shape (B*N, hidden)")
    need = tv_verify_pass_workspace(model, B, N, max_seq_len)
    if workspace is None:
        workspace = _cached_workspace("pass", need, dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib_handle().tv_verify_pass(
        ctypes.byref(model.c_dims), ctypes.byref(model.c_weights), _ptr(tokens), _ptr(parent),
        _ptr(seq_lens), _ptr(k_cache), _ptr(v_cache), B, N, Lcap, int(max_seq_len),
        _ptr(argmax), _ptr(logits), _ptr(hidden_out), _ptr(workspace), ws_bytes,
        _ptr(dev_status), _stream(dev))
    _check("tv_verify_pass", st)
    return argmax


def tv_kv_compact_layers_workspace(B: int) -> int:
    return int(_lib_handle().tv_kv_compact_layers_workspace(B))


def tv_kv_compact_layers(k_cache, v_cache, seq_lens, path, path_len, *, workspace=None) -> None:
    """tv_kv_compact on every layer of [layers,B,Hkv,Lcap,D] caches in one launch."""
    Ly, B, Hkv, Lcap, D = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache disagree")
    dt = _dtype_code(k_cache)
    _i32(seq_lens, (B,), "seq_lens")
    P = path.shape[1]
    _i32(path, (B, P), "path")
    _i32(path_len, (B,), "path_len")
    need = tv_kv_compact_layers_workspace(B)
    if workspace is None:
        workspace = _cached_workspace("compact_layers", need, k_cache.device)
    st = _lib_handle().tv_kv_compact_layers(
        _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(path), _ptr(path_len), B, Hkv, D, Lcap,
        P, Ly, dt, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(k_cache.device))
    _check("tv_kv_compact_layers", st)


# ---------------------------------------------------------------- graphs

class Graph:
    """A captured and instantiated sequence of calls (tv_graph_end)."""

    def __init__(self, handle):
        self.handle = handle

    def launch(self, stream=None):
        tv_graph_launch(self, stream)

    def __del__(self):
        if getattr(self, "handle", None):
            try:
                tv_graph_destroy(self)
            except Exception:  # pragma: no cover - interpreter shutdown
                pass


def _stream_handle(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def tv_graph_begin(stream) -> None:
    """Start capturing the calls enqueued on ``stream`` (a torch.cuda.Stream
    other than the default one)."""
    _check("tv_graph_begin", _lib_handle().tv_graph_begin(_stream_handle(stream)))


def tv_graph_end(stream) -> Graph:
    out = ctypes.c_void_p()
    _check("tv_graph_end", _lib_handle().tv_graph_end(_stream_handle(stream), ctypes.byref(out)))
    return Graph(out.value)


def tv_graph_launch(graph: Graph, stream=None) -> None:
    _check("tv_graph_launch", _lib_handle().tv_graph_launch(graph.handle, _stream_handle(stream)))


def tv_graph_destroy(graph: Graph) -> None:
    h, graph.handle = graph.handle, None
    if h:
        _check("tv_graph_destroy", _lib_handle().tv_graph_destroy(h))


# ---------------------------------------------------------------- tree construction

def tv_tree_build_workspace(B: int, depth: int, V: int, width: int) -> int:
    return int(_lib_handle().tv_tree_build_workspace(B, depth, V, width))


def tv_tree_build(draft_logp, root_tokens, width: int, budget: int, *, parent=None, tokens=None,
                  node_depth=None, score=None, workspace=None):
    """Draft trees by cumulative log-probability.  draft_logp [B,depth,V] fp32;
    root_tokens [B] int32.  Returns (parent, tokens) [B, budget+1] int32
    (node_depth / score are filled when given)."""
    B, D, V = draft_logp.shape
    if draft_logp.dtype != torch.float32:
        raise TypeError("draft_logp must be float32")
    _i32(root_tokens, (B,), "root_tokens")
    N = budget + 1
    dev = draft_logp.device
    if parent is None:
        parent = torch.empty((B, N), dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    _i32(parent, (B, N), "parent")
    _i32(tokens, (B, N), "tokens")
    if node_depth is not None:
        _i32(node_depth, (B, N), "node_depth")
    if score is not None and (score.dtype != torch.float32 or tuple(score.shape) != (B, N)):
        raise ValueError("score must be float32 of shape (B, budget+1)")
    need = tv_tree_build_workspace(B, D, V, width)
    if workspace is None:
        workspace = _cached_workspace("tree_build", need, dev)
    st = _lib_handle().tv_tree_build(
        _ptr(draft_logp), _ptr(root_tokens), B, D, V, width, budget, _ptr(parent), _ptr(tokens),
        _ptr(node_depth), _ptr(score), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev))
    _check("tv_tree_build", st)
    return parent, tokens


def tv_tree_build_level_workspace(B: int, depth: int, V: int, width: int) -> int:
    return int(_lib_handle().tv_tree_build_level_workspace(B, depth, V, width))


def tv_tree_build_level(draft_logp, level: int, depth: int, *, frontier_src=None,
                        frontier_tok=None, workspace=None):
    """One level of a branch-conditioned tree.  draft_logp [B, width, V] fp32:
    row r is the draft head's row after the path of frontier node r (level 1
    reads row 0).  Returns (frontier_src, frontier_tok) [B, width] int32.
    Calls for levels 1..depth and tv_tree_build_finish share one workspace
    (by default one cached per device: build one tree at a time with it)."""
    B, W, V = draft_logp.shape
    if draft_logp.dtype != torch.float32:
        raise TypeError("draft_logp must be float32")
    dev = draft_logp.device
    if frontier_src is None:
        frontier_src = torch.empty((B, W), dtype=torch.int32, device=dev)
    if frontier_tok is None:
        frontier_tok = torch.empty((B, W), dtype=torch.int32, device=dev)
    _i32(frontier_src, (B, W), "frontier_src")
    _i32(frontier_tok, (B, W), "frontier_tok")
    need = tv_tree_build_level_workspace(B, depth, V, W)
    if workspace is None:
        workspace = _cached_workspace("tree_level", need, dev)
    st = _lib_handle().tv_tree_build_level(
        _ptr(draft_logp), level, B, depth, V, W, _ptr(frontier_src), _ptr(frontier_tok),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    _check("tv_tree_build_level", st)
    return frontier_src, frontier_tok


def tv_tree_build_finish(root_tokens, depth: int, V: int, width: int, budget: int, *,
                         parent=None, tokens=None, node_depth=None, score=None, workspace=None):
    """Budget cut and numbering of the tree built by tv_tree_build_level
    calls.  Returns (parent, tokens) [B, budget+1] int32 (node_depth /
    score are filled when given)."""
    B = root_tokens.shape[0]
    _i32(root_tokens, (B,), "root_tokens")
    N = budget + 1
    dev = root_tokens.device
    if parent is None:
        parent = torch.empty((B, N), dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    _i32(parent, (B, N), "parent")
    _i32(tokens, (B, N), "tokens")
    if node_depth is not None:
        _i32(node_depth, (B, N), "node_depth")
    if score is not None and (score.dtype != torch.float32 or tuple(score.shape) != (B, N)):
        raise ValueError("score must be float32 of shape (B, budget+1)")
    need = tv_tree_build_level_workspace(B, depth, V, width)
    if workspace is None:
        workspace = _cached_workspace("tree_level", need, dev)
    st = _lib_handle().tv_tree_build_finish(
        _ptr(root_tokens), B, depth, V, width, budget, _ptr(parent), _ptr(tokens),
        _ptr(node_depth), _ptr(score), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev))
    _check("tv_tree_build_finish", st)
    return parent, tokens
