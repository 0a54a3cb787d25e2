"""infllmv2_sparse_attn_decode_noalloc (decode with the library's fixed
scratch array in place of a workspace) against infllmv2_sparse_attn_decode
with a workspace of the caller's, through the C ABI, and against the oracle:
two calls in a row, the second on a smaller batch with shorter sequences, so
the shared scratch keeps the first call's contents when the second starts."""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_long_infllmv2_amd.workloads import Params, make_decode
from parity import check_close, check_selection

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _run_pair(B, PL, c, dtype):
    """One decode through a plan (its own workspace) and one through the
    no-allocation entry point, on the same inputs and selections."""
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    p = c.params
    lens = np.asarray(c.seqlens)
    batch = len(lens)
    h_kv, _, d = c.k[0].shape
    h_q = c.q.shape[1]
    cap = int(((lens.max() + 63) // 64) * 64)
    k = torch.zeros((batch, h_kv, cap, d), dtype=tdt, device=dev)
    v = torch.zeros_like(k)
    for i, L in enumerate(lens):
        k[i, :, :L] = torch.from_numpy(c.k[i]).to(dev, tdt)
        v[i, :, :L] = torch.from_numpy(c.v[i]).to(dev, tdt)
    q = torch.from_numpy(c.q).to(dev, tdt)
    seqlens = torch.from_numpy(lens.astype(np.int32)).to(dev)
    nc = O.num_windows(cap, p.kernel_size, p.kernel_stride)
    ck = torch.zeros((batch, h_kv, nc, d), dtype=tdt, device=dev)
    B.infllmv2_compress_keys(k, seqlens, 0, nc, ck, p)
    plan = PL.DecodePlan(batch, int(lens.max()), h_q, h_kv, d, tdt, p, device=dev)
    plan.run(q, k, v, ck, seqlens)
    out = torch.full_like(plan.out, float("nan"))
    lse = torch.full_like(plan.lse, float("nan"))
    B.infllmv2_sparse_attn_decode_noalloc(q, k, v, seqlens, int(lens.max()), plan.block_idx,
                                          out, lse, p)
    torch.cuda.synchronize()
    return plan, out, lse


def _check_against_oracle(c, plan, out, lse, dtype):
    p = c.params
    res = O.decode(c.q, c.k, c.v, c.seqlens, p, dtype)
    got = out.float().cpu().numpy().astype(np.float64)
    gl = lse.cpu().numpy()
    sel = plan.block_idx.cpu().numpy()
    for i, L in enumerate(c.seqlens):
        pos = int(L) - 1
        if res["dense"][i]:
            o, l = res["o"][i], res["lse"][i]
        else:
            P = [check_selection(sel[i, g], res["S"][i][g], res["sel"][i][g], pos, p,
                                 f"seq {i} g {g}") for g in range(c.k[0].shape[0])]
            o, l = O.attend_selected(c.q[i], c.k[i], c.v[i], P, pos, p)
        check_close(got[i], o, dtype, f"seq {i} (L={int(L)})")
        np.testing.assert_allclose(gl[i], l, atol=2e-3 if dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("dtype,h_q,h_kv,d", [("bf16", 32, 2, 128), ("bf16", 8, 2, 64),
                                              ("f32", 4, 2, 64)])
def test_decode_noalloc_matches_workspace_call_twice(dtype, h_q, h_kv, d):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_long_infllmv2_amd import binding as B
    from block_sparse_long_infllmv2_amd import pipeline as PL
    p = Params(dense_len=8192, topk=16 if dtype == "f32" else 64)
    first = make_decode(41, [20000, 9000, 5000, 13001], h_q=h_q, h_kv=h_kv, d=d, params=p,
                        dtype=dtype, planted_per_token=1.0 / 2048)
    second = make_decode(42, [8500, 3000], h_q=h_q, h_kv=h_kv, d=d, params=p, dtype=dtype,
                         planted_per_token=1.0 / 2048)
    for name, c in (("first call", first), ("second, smaller call", second)):
        _say(f"decode no-alloc {dtype} h_q={h_q} h_kv={h_kv} d={d}: {name}, "
             f"seqlens {list(map(int, c.seqlens))}")
        plan, out, lse = _run_pair(B, PL, c, dtype)
        assert torch.equal(out, plan.out), f"{name}: output differs from the workspace call"
        assert torch.equal(lse, plan.lse), f"{name}: lse differs from the workspace call"
        _check_against_oracle(c, plan, out, lse, dtype)


def test_decode_noalloc_rejects_requests_beyond_the_scratch():
    from block_sparse_long_infllmv2_amd import binding as B
    p = B.default_params()
    big = 1 << 14                      # 16384 rows x 32 heads x 130 floats > 8 MiB
    assert B.infllmv2_workspace_size(B.OP_DECODE, big, 32, 2, 128, 4096, p) > \
        B.NOALLOC_SCRATCH_BYTES
    fake = 0x10000                     # never dereferenced: rejected on the host
    import ctypes
    st = B.LIB.infllmv2_sparse_attn_decode_noalloc(
        1, ctypes.c_void_p(fake), big, ctypes.c_void_p(fake), ctypes.c_void_p(fake), 4096,
        ctypes.c_void_p(fake), 4096, 32, 2, 128, None, ctypes.c_void_p(fake), None,
        ctypes.byref(p), None)
    assert st == 3, st                 # INFLLMV2_ERR_WORKSPACE, nothing queued
