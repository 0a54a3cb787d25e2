"""GPU parity at the full workload sizes, in the exact launch configuration
bench.py times (its Workload class builds the inputs and plans and runs one
step).  Outputs are checked on sampled rows that the oracle computes one by
one: chunk edges, tile edges and seeded random rows for the 128K prefill
chunk; every sequence, draft and head for the decode and tree workloads."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from parity import check_close, check_selection

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _workload(wid):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bench
    wl = bench.Workload(wid, torch)
    wl.step()
    torch.cuda.synchronize()
    return wl


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_full_prefill_128k_chunk_sampled_rows():
    _say("full prefill 128K, final 8192-query chunk")
    wl = _workload(2)
    c, p = wl.case, wl.p
    rng = np.random.default_rng(123)
    rows = sorted(set([0, 1, 7, 8, 9, 63, 64, 4095, 4096, 8183, 8184, 8190, 8191] +
                      list(rng.integers(0, c.n_q, 11))))
    ck = O.compress_keys(c.k, p, "bf16")
    gck = _host(wl.ck)
    assert np.count_nonzero(gck != ck) <= max(1, ck.size // 10000)
    res = O.prefill(c.q, c.k, c.v, p, "bf16", rows=rows, ck=ck)
    out = _host(wl.plan.out)
    lse = wl.plan.lse.cpu().numpy()
    sel = wl.plan.block_idx.cpu().numpy()
    for i in rows:
        pos = c.n_k - c.n_q + i
        P = [check_selection(sel[i, g], res["S"][i][g], res["sel"][i][g], pos, p,
                             f"row {i} g {g}") for g in range(2)]
        o, l = O.attend_selected(c.q[i], c.k, c.v, P, pos, p)
        check_close(out[i], o, "bf16", f"row {i}")
        np.testing.assert_allclose(lse[i], l, atol=2e-3)
    # every row of the chunk: a valid selection (forced blocks, ascending, full)
    for g in range(2):
        s = sel[:, g]
        assert np.all(s[:, 0] == 0)
        assert np.all(np.diff(s, axis=1) > 0)
        own = (c.n_k - c.n_q + np.arange(c.n_q)) // p.block_size
        assert np.all(s[:, -1] == own) and np.all(s[:, -2] == own - 1)


@pytest.mark.parametrize("wid", [1, 5, 4])
def test_full_decode(wid):
    _say(f"full decode workload {wid}")
    wl = _workload(wid)
    c, p = wl.case, wl.p
    res = O.decode(c.q, c.k, c.v, c.seqlens, p, "bf16")
    out = _host(wl.plan.out)
    lse = wl.plan.lse.cpu().numpy()
    sel = wl.plan.block_idx.cpu().numpy()
    for i, L in enumerate(c.seqlens):
        pos = int(L) - 1
        if res["dense"][i]:
            o, l = res["o"][i], res["lse"][i]
        else:
            P = [check_selection(sel[i, g], res["S"][i][g], res["sel"][i][g], pos, p,
                                 f"seq {i} g {g}") for g in range(2)]
            o, l = O.attend_selected(c.q[i], c.k[i], c.v[i], P, pos, p)
        check_close(out[i], o, "bf16", f"seq {i} (L={int(L)})")
        np.testing.assert_allclose(lse[i], l, atol=2e-3)


def test_full_tree_verify_128k():
    _say("full tree verification 128K, 16 drafts")
    wl = _workload(3)
    c, p = wl.case, wl.p
    res = O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, c.mask, p, "bf16")
    out = _host(wl.plan.out)
    lse = wl.plan.lse.cpu().numpy()
    sel = wl.plan.block_idx.cpu().numpy()
    T = c.q.shape[0]
    pos = c.n_ctx - 1
    for i in range(T):
        anc = [j for j in range(T) if (int(c.mask[i]) >> j) & 1]
        P = [check_selection(sel[i, g], res["S"][i][g], res["sel"][i][g], pos, p,
                             f"draft {i} g {g}") for g in range(2)]
        o, l = O.attend_selected(c.q[i], c.k, c.v, P, pos, p,
                                 (c.k_draft[:, anc], c.v_draft[:, anc]))
        check_close(out[i], o, "bf16", f"draft {i}")
        np.testing.assert_allclose(lse[i], l, atol=2e-3)
