"""Thin ctypes binding of libinfllmv2.so.

Functions carry the C names (infllmv2_compress_keys, ...) and take torch
tensors that live on the GPU; they only check and marshal arguments (data
pointers, sizes, the current HIP stream) and call the library.  Every step of
the computation runs in the library's HIP kernels.  There is no fallback: if
the library is missing or was not built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# INFLLMV2_LIB selects another build of the same library (same ABI)
LIB_PATH = os.environ.get("INFLLMV2_LIB") or os.path.join(_HERE, "libinfllmv2.so")

F32, BF16 = 0, 1
OP_DECODE, OP_TREE, OP_PREFILL_BWD = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 8 << 20          # INFLLMV2_NOALLOC_SCRATCH_BYTES
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
          3: "workspace missing, misaligned or too small", 4: "HIP launch failed"}


class InfLLMv2Error(RuntimeError):
    pass


class Params(ctypes.Structure):
    """Mirror of infllmv2_params (include/infllmv2.h)."""
    _fields_ = [("block_size", ctypes.c_int32), ("kernel_size", ctypes.c_int32),
                ("kernel_stride", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("init_blocks", ctypes.c_int32), ("local_blocks", ctypes.c_int32),
                ("dense_len", ctypes.c_int32), ("scale", ctypes.c_float),
                ("score_mode", ctypes.c_int32)]


DEBUG_LIB_PATH = os.path.join(_HERE, "libinfllmv2_debug.so")


def _load(path=None):
    """The library at `path` (default: the one this module binds) with its
    functions' argument and result types set."""
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with "
            "`python -m block_sparse_long_infllmv2_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    PP = ctypes.POINTER(Params)
    sigs = {
        "infllmv2_default_params": (None, [PP]),
        "infllmv2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "infllmv2_version": (ctypes.c_int, []),
        "infllmv2_compress_keys": (ctypes.c_int, [ctypes.c_int, P, i32, i32, i64, i32, P, i64,
                                                  i64, P, i64, PP, P]),
        "infllmv2_block_scores": (ctypes.c_int, [ctypes.c_int, P, i32, P, P, i32, i32, i32, P,
                                                 i32, i64, P, P, i64, i32, PP, P]),
        "infllmv2_select_topk": (ctypes.c_int, [P, i32, P, P, i32, i64, P, i32, P, PP, P]),
        "infllmv2_sparse_attn_prefill": (ctypes.c_int, [ctypes.c_int, P, i32, P, P, i64, i64,
                                                        i32, i32, i32, P, P, P, PP, P]),
        "infllmv2_sparse_attn_decode": (ctypes.c_int, [ctypes.c_int, P, i32, P, P, i64, P, i32,
                                                       i32, i32, i32, P, P, P, P, sz, PP, P]),
        "infllmv2_sparse_attn_decode_noalloc": (ctypes.c_int, [ctypes.c_int, P, i32, P, P, i64,
                                                               P, i32, i32, i32, i32, P, P, P,
                                                               PP, P]),
        "infllmv2_sparse_attn_decode_topk": (ctypes.c_int, [ctypes.c_int, P, i32, P, P, i64, P,
                                                            i32, i32, i32, i32, P, i64, P, P,
                                                            P, P, sz, PP, P]),
        "infllmv2_tree_verify": (ctypes.c_int, [ctypes.c_int, P, i32, P, P, i64, i64, P, P, P,
                                                i32, i32, i32, P, P, P, P, sz, PP, P]),
        "infllmv2_tree_verify_topk": (ctypes.c_int, [ctypes.c_int, P, i32, P, P, i64, i64, P, P,
                                                     P, i32, i32, i32, P, i64, P, P, P, P, sz,
                                                     PP, P]),
        "infllmv2_sparse_attn_prefill_backward": (ctypes.c_int, [ctypes.c_int, P, i32, P, P,
                                                                 i64, i64, i32, i32, i32, P,
                                                                 P, P, P, P, P, P, P, sz, PP,
                                                                 P]),
        "infllmv2_workspace_size": (sz, [ctypes.c_int, i32, i32, i32, i32, i64, PP]),
        "infllmv2_debug_check": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int),
                                                ctypes.POINTER(ctypes.c_int), P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def default_params(**over) -> Params:
    p = Params()
    LIB.infllmv2_default_params(ctypes.byref(p))
    for k, v in over.items():
        setattr(p, k, v)
    return p


def to_params(p) -> Params:
    """Params from a ctypes Params or any object with the same attributes."""
    if isinstance(p, Params):
        return p
    q = default_params()
    for name, _ in Params._fields_:
        if hasattr(p, name):
            setattr(q, name, getattr(p, name))
    return q


def _check(st: int, what: str):
    if st != 0:
        raise InfLLMv2Error(f"{what}: {LIB.infllmv2_status_string(st).decode()} ({st})")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _i32(t, name):
    if t is not None and t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return _ptr(t)


def _need(t, name, shape, dtype=None, optional=False):
    """The library sees raw pointers only: a buffer of another shape or dtype
    than the call's sizes imply would be read or written out of bounds, so
    it is rejected here, before any launch."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


# ---------------------------------------------------------------- C calls --
def infllmv2_compress_keys(k_cache, seqlens, m_begin, m_end, ck_cache, params):
    """k_cache [batch][h_kv][cap][d] -> ck_cache [batch][h_kv][nc_cap][d]."""
    batch, h_kv, cap, d = k_cache.shape
    _need(ck_cache, "ck_cache", (batch, h_kv, ck_cache.shape[2], d), k_cache.dtype)
    _need(seqlens, "seqlens", (batch,), torch.int32)
    p = to_params(params)
    _check(LIB.infllmv2_compress_keys(_dt(k_cache), _ptr(k_cache), batch, h_kv, cap, d,
                                      _i32(seqlens, "seqlens"), int(m_begin), int(m_end),
                                      _ptr(ck_cache), ck_cache.shape[2], ctypes.byref(p),
                                      _stream()), "infllmv2_compress_keys")


def infllmv2_block_scores(q, row_seq, row_pos, ck_cache, seqlens, scores, max_pos, params,
                          h_kv=None):
    """q [rows][h_q][d], ck [batch][h_kv][nc_cap][d] -> scores [rows][h_kv][nb_cap]."""
    rows, h_q, d = q.shape
    batch, hk, nc_cap, _ = ck_cache.shape
    _need(ck_cache, "ck_cache", (batch, hk, nc_cap, d), q.dtype)
    _need(scores, "scores", (rows, hk, scores.shape[2]), torch.float32)
    _need(row_seq, "row_seq", (rows,), torch.int32, optional=True)
    _need(row_pos, "row_pos", (rows,), torch.int32, optional=True)
    _need(seqlens, "seqlens", (batch,), torch.int32)
    p = to_params(params)
    _check(LIB.infllmv2_block_scores(_dt(q), _ptr(q), rows, _i32(row_seq, "row_seq"),
                                     _i32(row_pos, "row_pos"), h_q, hk, d, _ptr(ck_cache),
                                     batch, nc_cap, _i32(seqlens, "seqlens"), _ptr(scores),
                                     scores.shape[2], int(max_pos), ctypes.byref(p), _stream()),
           "infllmv2_block_scores")


def infllmv2_select_topk(scores, row_seq, row_pos, seqlens, block_idx, params):
    """scores [rows][h_kv][nb_cap] -> block_idx [rows][h_kv][topk] int32."""
    rows, h_kv, nb_cap = scores.shape
    p = to_params(params)
    if scores.dtype != torch.float32:
        raise TypeError("scores must be float32")
    _need(block_idx, "block_idx", (rows, h_kv, p.topk), torch.int32)
    _need(row_seq, "row_seq", (rows,), torch.int32, optional=True)
    _need(row_pos, "row_pos", (rows,), torch.int32, optional=True)
    _need(seqlens, "seqlens", (seqlens.shape[0],), torch.int32)
    _check(LIB.infllmv2_select_topk(_ptr(scores), rows, _i32(row_seq, "row_seq"),
                                    _i32(row_pos, "row_pos"), h_kv, nb_cap,
                                    _i32(seqlens, "seqlens"), seqlens.shape[0],
                                    _ptr(block_idx), ctypes.byref(p), _stream()),
           "infllmv2_select_topk")


def infllmv2_sparse_attn_prefill(q, k_cache, v_cache, n_k, block_idx, out, lse, params):
    """q [n_q][h_q][d]; k/v [h_kv][cap][d]; out like q; lse [n_q][h_q] or None."""
    n_q, h_q, d = q.shape
    h_kv, cap, _ = k_cache.shape
    p = to_params(params)
    _need(k_cache, "k_cache", (h_kv, cap, d), q.dtype)
    _need(v_cache, "v_cache", (h_kv, cap, d), q.dtype)
    _need(out, "out", (n_q, h_q, d), q.dtype)
    _need(lse, "lse", (n_q, h_q), torch.float32, optional=True)
    _need(block_idx, "block_idx", (n_q, h_kv, p.topk), torch.int32, optional=True)
    _check(LIB.infllmv2_sparse_attn_prefill(_dt(q), _ptr(q), n_q, _ptr(k_cache),
                                            _ptr(v_cache), cap, int(n_k), h_q, h_kv, d,
                                            _i32(block_idx, "block_idx"), _ptr(out), _ptr(lse),
                                            ctypes.byref(p), _stream()),
           "infllmv2_sparse_attn_prefill")


def infllmv2_workspace_size(op, n, h_q, h_kv, d, max_len, params) -> int:
    p = to_params(params)
    return int(LIB.infllmv2_workspace_size(op, n, h_q, h_kv, d, int(max_len), ctypes.byref(p)))


def infllmv2_sparse_attn_decode(q, k_cache, v_cache, seqlens, max_seqlen, block_idx, out, lse,
                                ws, params):
    """q [batch][h_q][d]; k/v [batch][h_kv][cap][d]; ws: uint8 workspace."""
    batch, h_q, d = q.shape
    _, h_kv, cap, _ = k_cache.shape
    p = to_params(params)
    _need(k_cache, "k_cache", (batch, h_kv, cap, d), q.dtype)
    _need(v_cache, "v_cache", (batch, h_kv, cap, d), q.dtype)
    _need(seqlens, "seqlens", (batch,), torch.int32)
    _need(out, "out", (batch, h_q, d), q.dtype)
    _need(lse, "lse", (batch, h_q), torch.float32, optional=True)
    _need(block_idx, "block_idx", (batch, h_kv, p.topk), torch.int32, optional=True)
    _need(ws, "ws", (ws.numel(),), torch.uint8)
    _check(LIB.infllmv2_sparse_attn_decode(_dt(q), _ptr(q), batch, _ptr(k_cache),
                                           _ptr(v_cache), cap, _i32(seqlens, "seqlens"),
                                           int(max_seqlen), h_q, h_kv, d,
                                           _i32(block_idx, "block_idx"), _ptr(out), _ptr(lse),
                                           _ptr(ws), ws.numel() * ws.element_size(),
                                           ctypes.byref(p), _stream()),
           "infllmv2_sparse_attn_decode")


def infllmv2_sparse_attn_decode_topk(q, k_cache, v_cache, seqlens, max_seqlen, scores,
                                     block_idx, out, lse, ws, params):
    """infllmv2_select_topk (row b = sequence b, at its last position) and
    infllmv2_sparse_attn_decode in one call: scores [batch][h_kv][nb_cap]
    float32 in, the selection out in block_idx [batch][h_kv][topk]."""
    batch, h_q, d = q.shape
    _, h_kv, cap, _ = k_cache.shape
    p = to_params(params)
    _need(k_cache, "k_cache", (batch, h_kv, cap, d), q.dtype)
    _need(v_cache, "v_cache", (batch, h_kv, cap, d), q.dtype)
    _need(seqlens, "seqlens", (batch,), torch.int32)
    _need(out, "out", (batch, h_q, d), q.dtype)
    _need(lse, "lse", (batch, h_q), torch.float32, optional=True)
    nb_cap = 0
    if scores is not None:
        nb_cap = scores.shape[2]
        _need(scores, "scores", (batch, h_kv, nb_cap), torch.float32)
    _need(block_idx, "block_idx", (batch, h_kv, p.topk), torch.int32, optional=True)
    _need(ws, "ws", (ws.numel(),), torch.uint8)
    _check(LIB.infllmv2_sparse_attn_decode_topk(_dt(q), _ptr(q), batch, _ptr(k_cache),
                                                _ptr(v_cache), cap, _i32(seqlens, "seqlens"),
                                                int(max_seqlen), h_q, h_kv, d, _ptr(scores),
                                                nb_cap, _i32(block_idx, "block_idx"),
                                                _ptr(out), _ptr(lse), _ptr(ws),
                                                ws.numel() * ws.element_size(),
                                                ctypes.byref(p), _stream()),
           "infllmv2_sparse_attn_decode_topk")


def infllmv2_sparse_attn_decode_noalloc(q, k_cache, v_cache, seqlens, max_seqlen, block_idx,
                                        out, lse, params):
    """infllmv2_sparse_attn_decode with the library's fixed scratch array in
    place of a workspace (NOALLOC_SCRATCH_BYTES per GPU): nothing is
    allocated; calls on one GPU must not overlap."""
    batch, h_q, d = q.shape
    _, h_kv, cap, _ = k_cache.shape
    p = to_params(params)
    _need(k_cache, "k_cache", (batch, h_kv, cap, d), q.dtype)
    _need(v_cache, "v_cache", (batch, h_kv, cap, d), q.dtype)
    _need(seqlens, "seqlens", (batch,), torch.int32)
    _need(out, "out", (batch, h_q, d), q.dtype)
    _need(lse, "lse", (batch, h_q), torch.float32, optional=True)
    _need(block_idx, "block_idx", (batch, h_kv, p.topk), torch.int32, optional=True)
    _check(LIB.infllmv2_sparse_attn_decode_noalloc(_dt(q), _ptr(q), batch, _ptr(k_cache),
                                                   _ptr(v_cache), cap, _i32(seqlens, "seqlens"),
                                                   int(max_seqlen), h_q, h_kv, d,
                                                   _i32(block_idx, "block_idx"), _ptr(out),
                                                   _ptr(lse), ctypes.byref(p), _stream()),
           "infllmv2_sparse_attn_decode_noalloc")


def infllmv2_tree_verify(q, k_cache, v_cache, n_ctx, k_draft, v_draft, tree_mask, block_idx,
                         out, lse, ws, params):
    """q [T][h_q][d]; k/v [h_kv][cap][d]; k/v_draft [h_kv][T][d]; tree_mask int64/uint64 [T]."""
    T, h_q, d = q.shape
    h_kv, cap, _ = k_cache.shape
    p = to_params(params)
    if tree_mask.dtype not in (torch.int64, torch.uint64):
        raise TypeError("tree_mask must be a 64-bit integer tensor")
    _need(tree_mask, "tree_mask", (T,))
    _need(k_cache, "k_cache", (h_kv, cap, d), q.dtype)
    _need(v_cache, "v_cache", (h_kv, cap, d), q.dtype)
    _need(k_draft, "k_draft", (h_kv, T, d), q.dtype)
    _need(v_draft, "v_draft", (h_kv, T, d), q.dtype)
    _need(out, "out", (T, h_q, d), q.dtype)
    _need(lse, "lse", (T, h_q), torch.float32, optional=True)
    _need(block_idx, "block_idx", (T, h_kv, p.topk), torch.int32, optional=True)
    _need(ws, "ws", (ws.numel(),), torch.uint8)
    _check(LIB.infllmv2_tree_verify(_dt(q), _ptr(q), T, _ptr(k_cache), _ptr(v_cache), cap,
                                    int(n_ctx), _ptr(k_draft), _ptr(v_draft), _ptr(tree_mask),
                                    h_q, h_kv, d, _i32(block_idx, "block_idx"), _ptr(out),
                                    _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                    ctypes.byref(p), _stream()),
           "infllmv2_tree_verify")


def infllmv2_tree_verify_topk(q, k_cache, v_cache, n_ctx, k_draft, v_draft, tree_mask, scores,
                              block_idx, out, lse, ws, params):
    """infllmv2_select_topk (every draft at position n_ctx - 1) and
    infllmv2_tree_verify in one call: scores [T][h_kv][nb_cap] float32 in,
    the selection out in block_idx [T][h_kv][topk]."""
    T, h_q, d = q.shape
    h_kv, cap, _ = k_cache.shape
    p = to_params(params)
    if tree_mask.dtype not in (torch.int64, torch.uint64):
        raise TypeError("tree_mask must be a 64-bit integer tensor")
    _need(tree_mask, "tree_mask", (T,))
    _need(k_cache, "k_cache", (h_kv, cap, d), q.dtype)
    _need(v_cache, "v_cache", (h_kv, cap, d), q.dtype)
    _need(k_draft, "k_draft", (h_kv, T, d), q.dtype)
    _need(v_draft, "v_draft", (h_kv, T, d), q.dtype)
    _need(out, "out", (T, h_q, d), q.dtype)
    _need(lse, "lse", (T, h_q), torch.float32, optional=True)
    nb_cap = 0
    if scores is not None:
        nb_cap = scores.shape[2]
        _need(scores, "scores", (T, h_kv, nb_cap), torch.float32)
    _need(block_idx, "block_idx", (T, h_kv, p.topk), torch.int32, optional=True)
    _need(ws, "ws", (ws.numel(),), torch.uint8)
    _check(LIB.infllmv2_tree_verify_topk(_dt(q), _ptr(q), T, _ptr(k_cache), _ptr(v_cache), cap,
                                         int(n_ctx), _ptr(k_draft), _ptr(v_draft),
                                         _ptr(tree_mask), h_q, h_kv, d, _ptr(scores), nb_cap,
                                         _i32(block_idx, "block_idx"), _ptr(out), _ptr(lse),
                                         _ptr(ws), ws.numel() * ws.element_size(),
                                         ctypes.byref(p), _stream()),
           "infllmv2_tree_verify_topk")


def infllmv2_sparse_attn_prefill_backward(q, k_cache, v_cache, n_k, block_idx, out, lse, d_out,
                                          dq, dk, dv, ws, params):
    """Gradients of the prefill attention, kept blocks fixed.  q, out, d_out,
    dq [n_q][h_q][d] (bf16); k/v [h_kv][cap][d]; lse float32 [n_q][h_q];
    dk, dv float32 [h_kv][cap][d] are accumulated into; ws: uint8 workspace."""
    n_q, h_q, d = q.shape
    h_kv, cap, _ = k_cache.shape
    p = to_params(params)
    _need(k_cache, "k_cache", (h_kv, cap, d), q.dtype)
    _need(v_cache, "v_cache", (h_kv, cap, d), q.dtype)
    for name, t in (("out", out), ("d_out", d_out), ("dq", dq)):
        _need(t, name, (n_q, h_q, d), q.dtype)
    _need(lse, "lse", (n_q, h_q), torch.float32)
    _need(dk, "dk", (h_kv, cap, d), torch.float32)
    _need(dv, "dv", (h_kv, cap, d), torch.float32)
    _need(block_idx, "block_idx", (n_q, h_kv, p.topk), torch.int32, optional=True)
    _need(ws, "ws", (ws.numel(),), torch.uint8)
    _check(LIB.infllmv2_sparse_attn_prefill_backward(
        _dt(q), _ptr(q), n_q, _ptr(k_cache), _ptr(v_cache), cap, int(n_k), h_q, h_kv, d,
        _i32(block_idx, "block_idx"), _ptr(out), _ptr(lse), _ptr(d_out), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(ws), ws.numel() * ws.element_size(), ctypes.byref(p), _stream()),
        "infllmv2_sparse_attn_prefill_backward")
