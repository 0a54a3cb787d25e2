"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, and rejects invalid calls on the host before launching
anything (only argument validation runs; no kernel is queued)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "infllmv2.h")
LIBPATH = os.path.join(ROOT, "block_sparse_long_infllmv2_amd", "libinfllmv2.so")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(infllmv2_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIBPATH):
        pytest.fail(f"{LIBPATH} not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIBPATH)
    from block_sparse_long_infllmv2_amd.binding import Params
    P = ctypes.c_void_p
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    PP = ctypes.POINTER(Params)
    lib.infllmv2_default_params.argtypes = [PP]
    lib.infllmv2_status_string.restype = ctypes.c_char_p
    lib.infllmv2_workspace_size.restype = sz
    lib.infllmv2_workspace_size.argtypes = [ctypes.c_int, i32, i32, i32, i32, i64, PP]
    lib.infllmv2_compress_keys.argtypes = [ctypes.c_int, P, i32, i32, i64, i32, P, i64, i64, P,
                                           i64, PP, P]
    lib.infllmv2_block_scores.argtypes = [ctypes.c_int, P, i32, P, P, i32, i32, i32, P, i32,
                                          i64, P, P, i64, i32, PP, P]
    lib.infllmv2_select_topk.argtypes = [P, i32, P, P, i32, i64, P, i32, P, PP, P]
    lib.infllmv2_sparse_attn_prefill.argtypes = [ctypes.c_int, P, i32, P, P, i64, i64, i32,
                                                 i32, i32, P, P, P, PP, P]
    lib.infllmv2_sparse_attn_decode.argtypes = [ctypes.c_int, P, i32, P, P, i64, P, i32, i32,
                                                i32, i32, P, P, P, P, sz, PP, P]
    lib.infllmv2_sparse_attn_decode_noalloc.argtypes = [ctypes.c_int, P, i32, P, P, i64, P,
                                                        i32, i32, i32, i32, P, P, P, PP, P]
    lib.infllmv2_debug_check.argtypes = [ctypes.POINTER(ctypes.c_int),
                                         ctypes.POINTER(ctypes.c_int), P]
    lib.infllmv2_tree_verify.argtypes = [ctypes.c_int, P, i32, P, P, i64, i64, P, P, P, i32,
                                         i32, i32, P, P, P, P, sz, PP, P]
    lib.infllmv2_sparse_attn_decode_topk.argtypes = [ctypes.c_int, P, i32, P, P, i64, P, i32,
                                                     i32, i32, i32, P, i64, P, P, P, P, sz, PP,
                                                     P]
    lib.infllmv2_tree_verify_topk.argtypes = [ctypes.c_int, P, i32, P, P, i64, i64, P, P, P,
                                              i32, i32, i32, P, i64, P, P, P, P, sz, PP, P]
    lib.infllmv2_sparse_attn_prefill_backward.argtypes = [ctypes.c_int, P, i32, P, P, i64, i64,
                                                          i32, i32, i32, P, P, P, P, P, P, P,
                                                          P, sz, PP, P]
    lib.Params = Params
    return lib


def params(lib, **kw):
    p = lib.Params()
    lib.infllmv2_default_params(ctypes.byref(p))
    for k, v in kw.items():
        setattr(p, k, v)
    return ctypes.byref(p)


FAKE = ctypes.c_void_p(0x10000)     # aligned, never dereferenced by the host


def test_header_declares_the_six_calls():
    fns = declared_functions()
    for name in ["infllmv2_compress_keys", "infllmv2_block_scores", "infllmv2_select_topk",
                 "infllmv2_sparse_attn_prefill", "infllmv2_sparse_attn_decode",
                 "infllmv2_tree_verify"]:
        assert name in fns


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in the header but not exported"


def test_defaults_status_version(lib):
    p = lib.Params()
    lib.infllmv2_default_params(ctypes.byref(p))
    assert (p.block_size, p.kernel_size, p.kernel_stride, p.topk, p.init_blocks,
            p.local_blocks, p.dense_len, p.scale, p.score_mode) == (64, 32, 16, 64, 1, 2,
                                                                    8192, 0.0, 0)
    assert lib.infllmv2_status_string(0) == b"ok"
    assert b"workspace" in lib.infllmv2_status_string(3)
    assert lib.infllmv2_status_string(99) == b"unknown status"
    assert lib.infllmv2_version() >= 100


def test_workspace_sizes(lib):
    ws = lib.infllmv2_workspace_size
    dec = ws(0, 8, 32, 2, 128, 131072, params(lib))
    # 8 rows x 32 heads x 16 splits (256 waves over 16 (row, KV head) pairs)
    # x (128 + 2) floats
    assert dec == 8 * 32 * 16 * 130 * 4
    dec_short = ws(0, 1, 32, 2, 128, 640, params(lib))   # 10 blocks -> 10 splits
    assert dec_short == ((1 * 32 * 10 * 130 * 4 + 255) // 256) * 256
    tree = ws(1, 16, 32, 2, 128, 131072, params(lib))
    assert tree > 16 * 32 * 130 * 4
    assert ws(1, 65, 32, 2, 128, 131072, params(lib)) == 0      # > 64 drafts
    assert ws(0, 8, 32, 3, 128, 131072, params(lib)) == 0       # 32 % 3 != 0
    assert ws(0, 8, 32, 2, 96, 131072, params(lib)) == 0        # head_dim 96
    assert ws(7, 8, 32, 2, 128, 131072, params(lib)) == 0       # unknown op


def test_compress_validation(lib):
    f = lib.infllmv2_compress_keys
    seq = FAKE
    assert f(1, None, 1, 2, 1024, 128, seq, 0, 10, FAKE, 63, params(lib), None) == INVALID
    assert f(5, FAKE, 1, 2, 1024, 128, seq, 0, 10, FAKE, 63, params(lib), None) == INVALID
    assert f(1, FAKE, 1, 2, 1024, 96, seq, 0, 10, FAKE, 63, params(lib), None) == UNSUPPORTED
    assert f(1, FAKE, 1, 2, 1024, 128, seq, 0, 64, FAKE, 63, params(lib), None) == INVALID
    assert f(1, FAKE, 1, 2, 100, 128, seq, 0, 10, FAKE, 63, params(lib), None) == INVALID
    assert f(1, FAKE, 1, 2, 1024, 128, seq, 0, 10, FAKE, 63,
             params(lib, topk=2, init_blocks=1, local_blocks=2), None) == INVALID
    assert f(1, FAKE, 1, 2, 1024, 128, seq, 0, 10, FAKE, 63,
             params(lib, kernel_stride=64), None) == UNSUPPORTED
    assert f(1, FAKE, 1, 2, 1024, 128, seq, 0, 10, FAKE, 63,
             params(lib, score_mode=2), None) == INVALID
    assert f(1, FAKE, 1, 2, 1024, 128, seq, 5, 5, FAKE, 63, params(lib), None) == OK  # empty


def test_scores_and_topk_validation(lib):
    s = lib.infllmv2_block_scores
    assert s(1, FAKE, 4, None, FAKE, 32, 3, 128, FAKE, 1, 100, FAKE, FAKE, 32, 1000,
             params(lib), None) == INVALID                           # 32 % 3
    assert s(1, FAKE, 4, None, FAKE, 32, 2, 128, FAKE, 1, 100, FAKE, FAKE, 8, 1000,
             params(lib), None) == INVALID                           # nb_cap too small
    assert s(1, FAKE, 4, None, FAKE, 32, 2, 128, FAKE, 1, 50, FAKE, FAKE, 32, 1000,
             params(lib), None) == INVALID                           # nc_cap too small
    assert s(1, FAKE, 0, None, FAKE, 32, 2, 128, FAKE, 1, 100, FAKE, FAKE, 32, 1000,
             params(lib), None) == OK                                # no rows
    t = lib.infllmv2_select_topk
    assert t(None, 4, None, FAKE, 2, 32, FAKE, 1, FAKE, params(lib), None) == INVALID
    assert t(FAKE, 4, None, FAKE, 2, 32, FAKE, 1, FAKE, params(lib, topk=200),
             None) == UNSUPPORTED
    assert t(FAKE, 0, None, FAKE, 2, 32, FAKE, 1, FAKE, params(lib), None) == OK


def test_attention_validation(lib):
    pre = lib.infllmv2_sparse_attn_prefill
    # sparse (n_k >= dense_len) without block_idx
    assert pre(1, FAKE, 8, FAKE, FAKE, 10000, 10000, 32, 2, 128, None, FAKE, None,
               params(lib), None) == INVALID
    # group size 3 has no matrix-core tiling
    assert pre(1, FAKE, 8, FAKE, FAKE, 10000, 10000, 6, 2, 128, FAKE, FAKE, None,
               params(lib), None) == UNSUPPORTED
    assert pre(1, FAKE, 8, FAKE, FAKE, 100, 1000, 32, 2, 128, FAKE, FAKE, None,
               params(lib), None) == INVALID                         # cap < n_k
    dec = lib.infllmv2_sparse_attn_decode
    need = lib.infllmv2_workspace_size(0, 2, 32, 2, 128, 20000, params(lib))
    assert dec(1, FAKE, 2, FAKE, FAKE, 20000, FAKE, 20000, 32, 2, 128, FAKE, FAKE, None,
               FAKE, need - 1, params(lib), None) == WORKSPACE
    assert dec(1, FAKE, 2, FAKE, FAKE, 20000, FAKE, 20000, 32, 2, 128, FAKE, FAKE, None,
               None, need, params(lib), None) == WORKSPACE
    assert dec(1, FAKE, 2, FAKE, FAKE, 20000, FAKE, 20000, 32, 2, 128, None, FAKE, None,
               FAKE, need, params(lib), None) == INVALID             # sparse needs idx
    tv = lib.infllmv2_tree_verify
    assert tv(1, FAKE, 65, FAKE, FAKE, 20000, 20000, FAKE, FAKE, FAKE, 32, 2, 128, FAKE, FAKE,
              None, FAKE, 1 << 30, params(lib), None) == INVALID     # > 64 drafts
    tneed = lib.infllmv2_workspace_size(1, 16, 32, 2, 128, 20000, params(lib))
    assert tv(1, FAKE, 16, FAKE, FAKE, 20000, 20000, FAKE, FAKE, FAKE, 32, 2, 128, FAKE,
              FAKE, None, FAKE, tneed - 256, params(lib), None) == WORKSPACE
    assert tv(1, FAKE, 16, FAKE, FAKE, 20000, 20000, FAKE, None, FAKE, 32, 2, 128, FAKE,
              FAKE, None, FAKE, tneed, params(lib), None) == INVALID  # no draft V


def test_select_in_attend_validation(lib):
    """The decode / tree calls that select from block scores check the scores
    and the selection output on the host (sparse rows need both, and a score
    row must cover every block of the longest sequence)."""
    dec = lib.infllmv2_sparse_attn_decode_topk
    need = lib.infllmv2_workspace_size(0, 2, 32, 2, 128, 20000, params(lib))
    nb = (20000 + 63) // 64

    def dcall(scores=FAKE, nb_cap=nb, idx=FAKE, ws_bytes=need, batch=2, h_q=32):
        return dec(1, FAKE, batch, FAKE, FAKE, 20000, FAKE, 20000, h_q, 2, 128, scores, nb_cap,
                   idx, FAKE, None, FAKE, ws_bytes, params(lib), None)
    assert dcall(scores=None) == INVALID
    assert dcall(idx=None) == INVALID
    assert dcall(nb_cap=nb - 1) == INVALID
    assert dcall(ws_bytes=need - 1) == WORKSPACE
    assert dcall(h_q=6) == UNSUPPORTED          # group size 3 (bf16)
    assert dcall(batch=0) == OK                 # nothing to do
    tv = lib.infllmv2_tree_verify_topk
    tneed = lib.infllmv2_workspace_size(1, 16, 32, 2, 128, 20000, params(lib))

    def tcall(scores=FAKE, nb_cap=nb, idx=FAKE, ws_bytes=tneed, n_draft=16):
        return tv(1, FAKE, n_draft, FAKE, FAKE, 20000, 20000, FAKE, FAKE, FAKE, 32, 2, 128,
                  scores, nb_cap, idx, FAKE, None, FAKE, ws_bytes, params(lib), None)
    assert tcall(scores=None) == INVALID
    assert tcall(idx=None) == INVALID
    assert tcall(nb_cap=nb - 1) == INVALID
    assert tcall(ws_bytes=tneed - 256) == WORKSPACE
    assert tcall(n_draft=65) == INVALID
    assert tcall(n_draft=0) == OK


def test_backward_validation(lib):
    bwd = lib.infllmv2_sparse_attn_prefill_backward
    ws = lib.infllmv2_workspace_size
    need = ws(2, 64, 32, 2, 128, 20000, params(lib))
    assert need > 64 * 32 * 8                                       # (lse, do.o) per pair
    assert ws(2, 20001, 32, 2, 128, 20000, params(lib)) == 0        # n_q > n_k
    dense_need = ws(2, 64, 32, 2, 128, 4000, params(lib))           # dense: no bitmap
    assert 0 < dense_need < need

    def call(dtype=1, n_q=64, n_k=20000, cap=20000, h_q=32, h_kv=2, d=128, idx=FAKE,
             lse=FAKE, ws_ptr=FAKE, ws_bytes=None, p=None):
        return bwd(dtype, FAKE, n_q, FAKE, FAKE, cap, n_k, h_q, h_kv, d, idx, FAKE, lse, FAKE,
                   FAKE, FAKE, FAKE, ws_ptr, need if ws_bytes is None else ws_bytes,
                   p if p is not None else params(lib), None)
    assert call(dtype=7) == INVALID                                  # unknown dtype
    assert call(lse=None) == INVALID                                 # lse is required
    assert call(idx=None) == INVALID                                 # sparse needs block_idx
    assert call(n_q=20001) == INVALID                                # more queries than keys
    assert call(cap=100) == INVALID                                  # cap < n_k
    assert call(h_q=6) == UNSUPPORTED                                # group size 3 (bf16)
    assert call(p=params(lib, block_size=96)) == UNSUPPORTED         # block not 64-aligned
    assert call(ws_bytes=need - 1) == WORKSPACE
    assert call(ws_ptr=None) == WORKSPACE
    assert call(ws_ptr=ctypes.c_void_p(0x10010)) == WORKSPACE        # not 256-byte aligned
    assert call(n_q=0) == OK                                         # nothing to do


def test_decode_noalloc_host_checks(lib):
    """The no-allocation decode rejects on the host what the decode call
    rejects, and any request whose workspace exceeds the fixed scratch
    array (8 MiB), before touching the GPU."""
    big = 1 << 14
    assert lib.infllmv2_workspace_size(0, big, 32, 2, 128, 4096, params(lib)) > 8 << 20
    args = lambda batch, hq=32, hkv=2, d=128, ml=4096: (
        1, FAKE, batch, FAKE, FAKE, 4096, FAKE, ml, hq, hkv, d, None, FAKE, None)
    assert lib.infllmv2_sparse_attn_decode_noalloc(*args(big), params(lib), None) == WORKSPACE
    assert lib.infllmv2_sparse_attn_decode_noalloc(*args(4, hq=30, hkv=4), params(lib),
                                                   None) == INVALID
    assert lib.infllmv2_sparse_attn_decode_noalloc(*args(4, d=96), params(lib),
                                                   None) == UNSUPPORTED
    assert lib.infllmv2_sparse_attn_decode_noalloc(*args(4, ml=0), params(lib), None) == INVALID


def test_debug_check_unsupported_without_debug_build(lib):
    """The normal library has no input checks compiled in: the call says so
    and touches nothing (no GPU needed)."""
    code, where = ctypes.c_int(7), ctypes.c_int(7)
    assert lib.infllmv2_debug_check(ctypes.byref(code), ctypes.byref(where), None) == UNSUPPORTED
    assert (code.value, where.value) == (7, 7)
