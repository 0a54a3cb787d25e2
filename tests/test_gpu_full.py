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
from parity import check_close, check_grad, check_selection

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


@pytest.mark.parametrize("wid", [2, 8])      # 8: 128-token blocks, top-6
def test_full_prefill_128k_chunk_sampled_rows(wid):
    """Outputs, log-sum-exp and selections of 590 rows of the final chunk
    against the oracle: one contiguous band of 512 rows (every edge of the
    8-token tiles inside it, and a 64-row band edge), the chunk's first and
    last rows and tile edges at its ends, and 64 seeded random rows."""
    from oracle_pool import prefill_rows
    _say(f"full prefill 128K, final 8192-query chunk (workload {wid})")
    wl = _workload(wid)
    c, p = wl.case, wl.p
    rng = np.random.default_rng(123)
    band = list(range(4064, 4576))
    rows = sorted(set([0, 1, 7, 8, 9, 15, 16, 63, 64, 8183, 8184, 8190, 8191] + band +
                      list(rng.integers(0, c.n_q, 64))))
    assert len(rows) >= 256
    ck = O.compress_keys(c.k, p, "bf16")
    gck = _host(wl.ck)
    assert np.count_nonzero(gck != ck) <= max(1, ck.size // 10000)
    res = prefill_rows(c.q, c.k, c.v, p, "bf16", ck, rows)
    _say(f"oracle done for {len(rows)} rows")
    out = _host(wl.plan.out)
    lse = wl.plan.lse.cpu().numpy()
    sel = wl.plan.block_idx.cpu().numpy()
    swaps = 0
    worst = 0.0
    for i in rows:
        pos = c.n_k - c.n_q + i
        o_ref, l_ref, S, osel = res[i]
        P = [check_selection(sel[i, g], S[g], osel[g], pos, p, f"row {i} g {g}")
             for g in range(2)]
        if any(set(P[g].tolist()) != set(int(b) for b in osel[g]) for g in range(2)):
            swaps += 1                      # a tie-band swap: the oracle on the GPU's set
            o_ref, l_ref = O.attend_selected(c.q[i], c.k, c.v, P, pos, p)
        mx, _ = check_close(out[i], o_ref, "bf16", f"row {i}")
        worst = max(worst, mx)
        np.testing.assert_allclose(lse[i], l_ref, atol=2e-3)
    _say(f"{len(rows)} rows: max-abs {worst:.3g}, {swaps} tie-band swaps")
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


def test_full_prefill_whole_prompt_sampled_rows():
    """The whole 131072-token prompt in 16 chunks of 8192 (bench workload 7):
    the compressed-key cache after the last chunk, and sampled rows of five
    chunks against the oracle's prefill of each row's prefix."""
    _say("full prefill: whole 128K prompt in 16 chunks")
    wl = _workload(7)
    c, p = wl.case, wl.p
    ck = O.compress_keys(c.k, p, "bf16")
    gck = _host(wl.ck)
    assert np.count_nonzero(gck != ck) <= max(1, ck.size // 10000)
    chunk = 8192
    rows = [0, 8191, 8192, 40000, 65535, 65536 + 4096, 131071]
    out = _host(wl.cp.out)
    lse = wl.cp.lse.cpu().numpy()
    for i in rows:
        ci = i // chunk
        pl = wl.cp.plans[ci]
        # the shared selection scratch holds the last chunk's selections:
        # select this chunk again (same inputs, same result)
        pl.select(wl.q[ci * chunk:(ci + 1) * chunk], wl.ck)
        torch.cuda.synchronize()
        sel = pl.block_idx.cpu().numpy()[i - ci * chunk]
        nw = O.num_windows(i + 1, p.kernel_size, p.kernel_stride)
        res = O.prefill(c.q[i:i + 1], c.k[:, :i + 1], c.v[:, :i + 1], p, "bf16", rows=[0],
                        ck=ck[:, :nw])
        if res["dense"]:
            o, l = res["o"][0], res["lse"][0]
        else:
            P = [check_selection(sel[g], res["S"][0][g], res["sel"][0][g], i, p,
                                 f"row {i} g {g}") for g in range(2)]
            o, l = O.attend_selected(c.q[i], c.k[:, :i + 1], c.v[:, :i + 1], P, i, p)
        check_close(out[i], o, "bf16", f"row {i}")
        np.testing.assert_allclose(lse[i], l, atol=2e-3)


def test_full_decode_128k_batch32():
    """Bench workload 6: 32 copies of the 128K sequence, each in its own
    memory (8 splits per row): row 0 against the oracle, every other row
    identical to it (same inputs, deterministic kernels)."""
    _say("full decode 128K batch 32")
    wl = _workload(6)
    c, p = wl.case, wl.p
    res = O.decode(c.q, c.k, c.v, c.seqlens, p, "bf16")
    out = _host(wl.plan.out)
    lse = wl.plan.lse.cpu().numpy()
    sel = wl.plan.block_idx.cpu().numpy()
    pos = int(c.seqlens[0]) - 1
    P = [check_selection(sel[0, g], res["S"][0][g], res["sel"][0][g], pos, p, f"g {g}")
         for g in range(2)]
    o, l = O.attend_selected(c.q[0], c.k[0], c.v[0], P, pos, p)
    check_close(out[0], o, "bf16", "row 0")
    np.testing.assert_allclose(lse[0], l, atol=2e-3)
    for i in range(1, out.shape[0]):
        assert np.array_equal(out[i], out[0]) and np.array_equal(sel[i], sel[0]), f"row {i}"


def test_full_prefill_backward_sampled():
    _say("full prefill backward 128K, final 8192-query chunk (workload 9)")
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bench
    wl = bench.Workload(9, torch)
    wl.dk.zero_()
    wl.dv.zero_()
    wl.backward()
    torch.cuda.synchronize()
    c, p = wl.case, wl.p
    sel = wl.plan.block_idx.cpu().numpy()
    d_out = wl.d_out.float().cpu().numpy().astype(np.float64)
    dq = _host(wl.dq)
    dk = wl.dk.cpu().numpy().astype(np.float64)
    dv = wl.dv.cpu().numpy().astype(np.float64)
    sel_rows = [[s[s >= 0] for s in row] for row in sel]
    rng = np.random.default_rng(321)
    rows = sorted(set([0, 1, 63, 64, 4095, 8190, 8191] + list(rng.integers(0, c.n_q, 5))))
    rq, _, _ = O.prefill_backward(c.q, c.k, c.v, sel_rows, p, d_out, rows=rows)
    check_grad(dq[rows], rq[rows], "dq sampled rows")
    # dk / dv at one scored (not forced) block of KV head 0: all rows that kept
    # it (the oracle takes ~0.7 s per row here, so a block kept by few rows)
    counts = np.bincount(sel[:, 0][sel[:, 0] >= 0].ravel(), minlength=c.n_k // p.block_size)
    own0 = (c.n_k - c.n_q) // p.block_size
    cand = [b for b in range(1, own0 - 1) if 8 <= counts[b] <= 48]
    if not cand:
        cand = [b for b in range(1, own0 - 1) if counts[b] > 0]
    b = max(cand, key=lambda x: counts[x]) if counts[cand].max() <= 48 else \
        min(cand, key=lambda x: counts[x])
    krows = list(np.nonzero((sel[:, 0] == b).any(axis=1))[0])
    _say(f"dk/dv of block {b} (kept by {len(krows)} rows)")
    _, rk, rv = O.prefill_backward(c.q, c.k, c.v, sel_rows, p, d_out, rows=krows)
    span = slice(b * p.block_size, (b + 1) * p.block_size)
    check_grad(dk[0, span], rk[0, span], f"dk block {b}")
    check_grad(dv[0, span], rv[0, span], f"dv block {b}")
    # invariants over every key of the context: each row's weights sum to 1,
    # so summing dV over keys gives the group's summed upstream gradient; each
    # row's dS sums to 0, so dK summed over keys vanishes
    G = c.q.shape[1] // c.k.shape[0]
    for g in range(c.k.shape[0]):
        want = d_out[:, g * G:(g + 1) * G].sum(axis=(0, 1))
        got = dv[g].sum(axis=0)
        err = np.abs(got - want).max() / np.abs(want).max()
        print(f"  sum of dv over keys, group {g}: relative max error {err:.2e}", flush=True)
        assert err <= 1e-3
        kmag = np.abs(dk[g]).sum(axis=0).max()
        resid = np.abs(dk[g].sum(axis=0)).max() / kmag
        print(f"  sum of dk over keys, group {g}: {resid:.2e} of sum |dk|", flush=True)
        assert resid <= 1e-3
