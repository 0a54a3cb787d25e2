"""The debug build (libinfllmv2_debug.so, -DINFLLMV2_DEBUG) through the C ABI:
valid calls report no violation and return the same results as the normal
library; kept-block rows and tree masks that break the selection's form are
reported with their code and row.  Such inputs are safe for the kernels (a
list is cut at its first id out of range, unions are sorted, mask bits past
the draft count are dropped), so nothing here can read out of bounds."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_long_infllmv2_amd.workloads import Params, make_decode, make_tree

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def D():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_long_infllmv2_amd import binding
    return binding, binding._load(binding.DEBUG_LIB_PATH)


def _check(lib):
    code, where = ctypes.c_int(-1), ctypes.c_int(-1)
    st = lib.infllmv2_debug_check(ctypes.byref(code), ctypes.byref(where),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    return code.value, where.value


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def test_debug_build_decode_rows(D):
    B, dbg = D
    _say("debug build: decode kept-block rows")
    p = Params(dense_len=2048, topk=16)
    c = make_decode(51, [9001, 3000, 1500, 12000], h_q=32, h_kv=2, d=128, params=p,
                    dtype="bf16", planted_per_token=1 / 512)
    lens = np.asarray(c.seqlens)
    cap = ((lens.max() + 63) // 64) * 64
    k = torch.zeros((4, 2, cap, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    for i, L in enumerate(lens):
        k[i, :, :L] = torch.from_numpy(c.k[i]).cuda().to(torch.bfloat16)
        v[i, :, :L] = torch.from_numpy(c.v[i]).cuda().to(torch.bfloat16)
    q = torch.from_numpy(c.q).cuda().to(torch.bfloat16)
    seqlens = torch.from_numpy(lens.astype(np.int32)).cuda()
    nc = O.num_windows(cap, 32, 16)
    ck = torch.zeros((4, 2, nc, 128), dtype=torch.bfloat16, device="cuda")
    B.infllmv2_compress_keys(k, seqlens, 0, nc, ck, p)
    from block_sparse_long_infllmv2_amd import pipeline as PL
    plan = PL.DecodePlan(4, int(lens.max()), 32, 2, 128, torch.bfloat16, p)
    plan.run(q, k, v, ck, seqlens)
    torch.cuda.synchronize()
    pp = B.to_params(p)
    out = torch.empty_like(plan.out)
    lse = torch.empty_like(plan.lse)
    ws = torch.empty_like(plan.ws)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def decode(idx):
        st = dbg.infllmv2_sparse_attn_decode(1, _p(q), 4, _p(k), _p(v), cap, _p(seqlens),
                                             int(lens.max()), 32, 2, 128, _p(idx), _p(out),
                                             _p(lse), _p(ws), ws.numel(), ctypes.byref(pp),
                                             stream)
        assert st == 0, st
        return _check(dbg)

    assert _check(dbg) == (0, 0)
    assert decode(plan.block_idx) == (0, 0)
    assert torch.equal(out, plan.out) and torch.equal(lse, plan.lse)
    good = plan.block_idx.clone()
    n_b3 = (12000 + 63) // 64
    cases = []
    bad = good.clone(); bad[3, 1, 7] = n_b3 + 5                      # id past the eligible blocks
    cases.append((bad, 1, 3 * 2 + 1))
    bad = good.clone(); bad[0, 0, [4, 5]] = bad[0, 0, [5, 4]]         # two ids swapped
    cases.append((bad, 2, 0))
    bad = good.clone(); bad[0, 1, 6] = -1                            # padding inside the list
    cases.append((bad, 3, 1))
    row = good[3, 0].cpu().numpy()
    free = sorted(set(range(1, n_b3 - 2)) - set(row.tolist()))[0]
    fixed = np.sort(np.concatenate([row[1:], [free]]))               # block 0 replaced
    bad = good.clone(); bad[3, 0] = torch.from_numpy(fixed.astype(np.int32)).cuda()
    cases.append((bad, 4, 3 * 2 + 0))
    for idx, code, where in cases:
        _say(f"  malformed row: expect code {code} at {where}")
        assert decode(idx) == (code, where)
    # rows of dense sequences are not read, so they are not checked
    bad = good.clone(); bad[2, :, :] = 999
    assert decode(bad) == (0, 0)


def test_debug_build_tree_masks_and_prefill_rows(D):
    B, dbg = D
    _say("debug build: tree masks and rows, prefill rows")
    p = Params(dense_len=0, topk=16)
    T, n_ctx = 8, 5000
    c = make_tree(52, n_ctx=n_ctx, n_draft=T, h_q=32, h_kv=2, d=128, params=p, dtype="bf16",
                  n_planted=2)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    q, k, v, kd, vd = bf(c.q), bf(c.k), bf(c.v), bf(c.k_draft), bf(c.v_draft)
    nc = O.num_windows(n_ctx, 32, 16)
    ck = torch.zeros((2, nc, 128), dtype=torch.bfloat16, device="cuda")
    B.infllmv2_compress_keys(k.unsqueeze(0), torch.tensor([n_ctx], dtype=torch.int32,
                                                          device="cuda"), 0, nc,
                             ck.unsqueeze(0), p)
    from block_sparse_long_infllmv2_amd import pipeline as PL
    plan = PL.TreePlan(T, n_ctx, 32, 2, 128, torch.bfloat16, p)
    mask = torch.from_numpy(c.mask.astype(np.int64)).cuda()
    plan.run(q, k, v, ck, kd, vd, mask)
    torch.cuda.synchronize()
    pp = B.to_params(p)
    out, lse, ws = torch.empty_like(plan.out), torch.empty_like(plan.lse), torch.empty_like(plan.ws)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def tree(m, idx):
        st = dbg.infllmv2_tree_verify(1, _p(q), T, _p(k), _p(v), n_ctx, n_ctx, _p(kd), _p(vd),
                                      _p(m), 32, 2, 128, _p(idx), _p(out), _p(lse), _p(ws),
                                      ws.numel(), ctypes.byref(pp), stream)
        assert st == 0, st
        return _check(dbg)

    assert tree(mask, plan.block_idx) == (0, 0)
    assert torch.equal(out, plan.out)
    high = c.mask.copy(); high[5] |= np.uint64(1) << np.uint64(40)
    assert tree(torch.from_numpy(high.view(np.int64)).cuda(), plan.block_idx) == (6, 5)
    later = c.mask.copy(); later[2] |= np.uint64(1) << np.uint64(6)
    assert tree(torch.from_numpy(later.view(np.int64)).cuda(), plan.block_idx) == (7, 2)
    bad = plan.block_idx.clone(); bad[6, 1, 3] = 100000
    assert tree(mask, bad) == (1, 6 * 2 + 1)
    # prefill: the drafts' rows read as the last 8 queries of the context
    # (positions n_ctx-8 .. n_ctx-1), selected for those positions
    pf = PL.PrefillPlan(T, n_ctx, 32, 2, 128, torch.bfloat16, p)
    pf.select(q, ck)
    torch.cuda.synchronize()

    def prefill(idx):
        st = dbg.infllmv2_sparse_attn_prefill(1, _p(q), T, _p(k), _p(v), n_ctx, n_ctx, 32, 2,
                                              128, _p(idx), _p(out), _p(lse), ctypes.byref(pp),
                                              stream)
        assert st == 0, st
        return _check(dbg)

    assert prefill(pf.block_idx) == (0, 0)
    bad = pf.block_idx.clone(); bad[4, 0, 2] = bad[4, 0, 1]           # a duplicate
    assert prefill(bad) == (2, 4 * 2)


def test_normal_build_has_no_checks(D):
    B, _ = D
    code, where = ctypes.c_int(), ctypes.c_int()
    assert B.LIB.infllmv2_debug_check(ctypes.byref(code), ctypes.byref(where), None) == 2
