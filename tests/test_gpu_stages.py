"""GPU parity, stage by stage and end to end, at sizes the oracle finishes in
seconds (several tiles, ragged tails, dense/sparse mixes).  Every case calls
the HIP library through its C ABI (ctypes binding) and compares with the CPU
oracle on the same seeded inputs."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_long_infllmv2_amd.workloads import Params, config, make_decode, \
    make_prefill, make_tree
from parity import check_close, check_selection

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_long_infllmv2_amd import binding
    return binding


@pytest.fixture(scope="module")
def PL():
    from block_sparse_long_infllmv2_amd import pipeline
    return pipeline


def dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


# ------------------------------------------------------------- compress ----
def _check_ck(got, ref, dtype, where):
    """bf16: the float32 sum of 32 bf16 keys rounds only when their exponents
    spread widely, so the stored mean matches the oracle's float64 mean
    rounded once, except in rare cases where the float32 rounding (or a
    double rounding) moves the last bf16 bit.  float32: the sum itself
    rounds; allow a few float32 ulps."""
    if dtype == "bf16":
        mism = np.count_nonzero(got != ref)
        assert mism <= max(1, ref.size // 10000), f"{where}: {mism} of {ref.size} differ"
        np.testing.assert_allclose(got, ref, rtol=2 ** -7, atol=1e-30)
    else:
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("dtype,d,ks,s", [("bf16", 128, 32, 16), ("f32", 64, 32, 16),
                                         ("bf16", 64, 32, 16), ("bf16", 128, 64, 32),
                                         ("f32", 64, 48, 16), ("bf16", 128, 32, 32)])
def test_compress_keys(B, dtype, d, ks, s):
    _say(f"compress {dtype} d={d} kernel {ks}/{s}")
    p = Params(kernel_size=ks, kernel_stride=s)
    rng = np.random.default_rng(1)
    lens = [1000, 333, 31]
    cap = 1024
    h_kv = 2
    k = np.zeros((3, h_kv, cap, d), np.float32)
    for i, L in enumerate(lens):
        k[i, :, :L] = rng.standard_normal((h_kv, L, d))
    kk = dev(k, dtype)
    host_k = host(kk)
    nc_cap = O.num_windows(cap, ks, s)
    ck = torch.full((3, h_kv, nc_cap, d), 7.0, dtype=tdt(dtype), device="cuda")
    B.infllmv2_compress_keys(kk, torch.tensor(lens, dtype=torch.int32, device="cuda"), 0,
                             nc_cap, ck, p)
    torch.cuda.synchronize()
    got = host(ck)
    for i, L in enumerate(lens):
        ref = O.compress_keys(host_k[i, :, :L], p, dtype)
        n_c = ref.shape[1]
        _check_ck(got[i, :, :n_c], ref, dtype, f"seq {i}")
        assert np.all(got[i, :, n_c:] == 7.0), "windows past the sequence were written"


# --------------------------------------------------------------- scores ----
@pytest.mark.parametrize("dtype,d,h_q,h_kv,rows,bs,mode", [
    ("bf16", 128, 32, 2, 12, 64, 0),
    ("f32", 64, 2, 1, 12, 64, 0),
    ("bf16", 64, 8, 2, 12, 64, 0),
    ("bf16", 128, 32, 2, 300, 64, 0),    # MFMA
    ("bf16", 64, 4, 1, 100, 64, 0),      # MFMA
    ("bf16", 128, 32, 2, 300, 128, 0),   # MFMA
    ("bf16", 64, 4, 1, 100, 128, 0),     # MFMA
    ("bf16", 128, 32, 2, 12, 128, 0),
    # score_mode 1: per-head softmax over the visible windows, summed
    ("bf16", 128, 32, 2, 40, 64, 1),
    ("bf16", 64, 8, 2, 12, 128, 1),
    ("f32", 64, 2, 1, 12, 64, 1),
    ("f32", 128, 12, 2, 12, 64, 1)])
def test_block_scores_on_oracle_ck(B, dtype, d, h_q, h_kv, rows, bs, mode):
    _say(f"scores {dtype} d={d} h_q={h_q} h_kv={h_kv} rows={rows} block={bs} mode={mode}")
    _scores_case(B, dtype, d, h_q, h_kv, rows, Params(dense_len=0, block_size=bs,
                                                      score_mode=mode))


@pytest.mark.parametrize("ks,s,bs,rows", [
    (64, 32, 128, 300),   # ks = 2s, B = 4s: matrix-core kernel at stride 32
    (64, 32, 256, 300),   # B = 8s
    (64, 32, 128, 12),    # streaming kernel
    (32, 32, 64, 12),     # windows that do not overlap (ks = s)
    (48, 16, 64, 300),    # ks = 3s: the streaming kernel also for many rows
])
def test_block_scores_window_geometries(B, ks, s, bs, rows):
    _say(f"scores bf16 kernel {ks}/{s} block={bs} rows={rows}")
    _scores_case(B, "bf16", 128, 32, 2, rows,
                 Params(dense_len=0, block_size=bs, kernel_size=ks, kernel_stride=s))


def _scores_case(B, dtype, d, h_q, h_kv, rows, p):
    mode, bs = p.score_mode, p.block_size
    n_k = 5000
    c = make_prefill(3, n_k=n_k, n_q=1, h_q=h_q, h_kv=h_kv, d=d, params=p, dtype=dtype,
                     n_planted=5, alpha=1.5, beta=1.5)
    ck = O.compress_keys(c.k, p, dtype)
    rng = np.random.default_rng(2)
    edge = [0, 15, 30, 31, 63, 64, 78, 79, 200, 4095, 4999, 2500]
    pos = np.array(edge + list(rng.integers(0, n_k, rows - len(edge))), np.int32)
    q = dev(rng.standard_normal((len(pos), h_q, d)), dtype)
    nb = n_k // bs + 1
    scores = torch.full((len(pos), h_kv, nb), 123.0, dtype=torch.float32, device="cuda")
    B.infllmv2_block_scores(q, None, torch.from_numpy(pos).cuda(), dev(ck[None], dtype),
                            torch.tensor([n_k], dtype=torch.int32, device="cuda"), scores,
                            int(pos.max()), p)
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    qh = host(q)
    for r, ps in enumerate(pos):
        sig = O.kernel_scores(qh[r], ck, int(ps), p, h_kv)
        S = O.block_scores(sig, int(ps), p)
        ne = S.shape[1]
        g = got[r, :, :ne]
        inf = np.isinf(S)
        assert np.array_equal(np.isinf(g), inf), f"row {r}: -inf pattern differs"
        # mode 1: sums of float32 softmax shares (normalisers over thousands
        # of windows) -- a few 1e-6 relative
        np.testing.assert_allclose(g[~inf], S[~inf], rtol=2e-5 if mode == 0 else 1e-4,
                                   atol=2e-5 if mode == 0 else 1e-7)
        assert np.all(got[r, :, ne:] == 123.0), "scores beyond eligible blocks written"


# ----------------------------------------------------------------- topk ----
@pytest.mark.parametrize("rows", [24, 300])   # a few decode-sized rows, and many
def test_select_topk_matches_oracle_exactly(B, rows):
    _say(f"topk exact rows={rows}")
    rng = np.random.default_rng(4)
    cases = []
    for topk, init, local, nb, ties in [(8, 1, 2, 40, True), (64, 1, 2, 2048, False),
                                        (64, 1, 2, 2048, True), (6, 0, 0, 30, True),
                                        (16, 2, 3, 700, False), (64, 1, 2, 65, False),
                                        (64, 1, 2, 3000, True), (64, 1, 2, 10000, False)]:
        cases.append((Params(topk=topk, init_blocks=init, local_blocks=local, dense_len=0),
                      nb, ties))
    for p, nb, ties in cases:
        n_k = nb * 64
        pos = rng.integers(0, n_k, rows).astype(np.int32)
        pos[0] = n_k - 1
        pos[1] = 0
        S = rng.standard_normal((rows, 2, nb)).astype(np.float32)
        if ties:
            S = np.round(S * 2).astype(np.float32)
            S[2] = 1.0                      # a row of equal scores
        S[rng.random(S.shape) < 0.05] = -np.inf
        s_t = torch.from_numpy(S).cuda()
        idx = torch.full((rows, 2, p.topk), -7, dtype=torch.int32, device="cuda")
        B.infllmv2_select_topk(s_t, None, torch.from_numpy(pos).cuda(),
                               torch.tensor([n_k], dtype=torch.int32, device="cuda"), idx, p)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        for r in range(rows):
            for g in range(2):
                ne = pos[r] // 64 + 1
                want = O.select_blocks(S[r, g, :ne].astype(np.float64), int(pos[r]), p)
                row = got[r, g]
                assert list(row[:len(want)]) == list(want), (p, r, g)
                assert np.all(row[len(want):] == -1)


def test_select_topk_dense_rows_get_minus_one(B):
    _say("topk dense rows")
    p = Params()
    S = torch.zeros((3, 2, 200), dtype=torch.float32, device="cuda")
    idx = torch.zeros((3, 2, 64), dtype=torch.int32, device="cuda")
    seqlens = torch.tensor([8191, 8192, 12000], dtype=torch.int32, device="cuda")
    row_seq = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    B.infllmv2_select_topk(S, row_seq, None, seqlens, idx, p)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    assert np.all(got[0] == -1)
    assert np.all(got[1] >= 0) and np.all(got[2] >= 0)


# -------------------------------------------------------------- prefill ----
def _run_prefill(B, PL, c, rows_check=None):
    p = c.params
    h_kv, n_k, d = c.k.shape
    n_q, h_q, _ = c.q.shape
    q = dev(c.q, c.dtype)
    k = dev(c.k, c.dtype)
    v = dev(c.v, c.dtype)
    nc = max(1, O.num_windows(n_k, p.kernel_size, p.kernel_stride))
    ck = torch.zeros((h_kv, nc, d), dtype=tdt(c.dtype), device="cuda")
    plan = PL.PrefillPlan(n_q, n_k, h_q, h_kv, d, tdt(c.dtype), p)
    plan.run(q, k, v, ck, m_begin=0)
    torch.cuda.synchronize()
    return plan, ck


def _check_prefill(plan, ck_gpu, c, rows):
    p = c.params
    n_q = c.n_q
    res = O.prefill(c.q, c.k, c.v, p, c.dtype, rows=rows)
    out = host(plan.out)
    lse = plan.lse.cpu().numpy()
    if not res["dense"]:
        _check_ck(host(ck_gpu), res["ck"], c.dtype, "compressed keys")
        sel = plan.block_idx.cpu().numpy()
    for i in rows:
        pos = c.n_k - n_q + i
        if res["dense"]:
            ref_o, ref_l = res["o"][i], res["lse"][i]
        else:
            P = [check_selection(sel[i, g], res["S"][i][g], res["sel"][i][g], pos, p,
                                 f"row {i} g {g}") for g in range(c.k.shape[0])]
            ref_o, ref_l = O.attend_selected(c.q[i], c.k, c.v, P, pos, p)
        check_close(out[i], ref_o, c.dtype, f"row {i}")
        np.testing.assert_allclose(lse[i], ref_l, atol=2e-3 if c.dtype == "bf16" else 1e-4)


def test_prefill_tiny_f32_config(B, PL):
    """The tiny float32 workload at full size: N=2048, 2 q heads / 1 KV head."""
    _say("prefill cfg0 f32 n=2048")
    c = config(0)
    plan, ck = _run_prefill(B, PL, c)
    _check_prefill(plan, ck, c, rows=list(range(0, 2048, 7)) + [2047, 2046, 64, 63])


@pytest.mark.parametrize("n_k,n_q,h_q,h_kv,d,topk", [
    (4096, 300, 32, 2, 128, 16),     # several tiles, ragged last tile
    (9000, 133, 32, 2, 128, 64),     # ragged last KV block (9000 % 64 = 40)
    (3000, 200, 16, 2, 64, 8),       # G = 8, d = 64
    (2600, 64, 8, 2, 128, 8),        # G = 4: 32-token tiles
    (5000, 150, 32, 2, 64, 16),      # G = 16, d = 64
])
def test_prefill_bf16_end_to_end(B, PL, n_k, n_q, h_q, h_kv, d, topk):
    _say(f"prefill bf16 n_k={n_k} n_q={n_q} h_q={h_q} h_kv={h_kv} d={d} topk={topk}")
    p = Params(topk=topk, dense_len=0)
    c = make_prefill(5, n_k=n_k, n_q=n_q, h_q=h_q, h_kv=h_kv, d=d, params=p, dtype="bf16",
                     n_planted=max(1, n_k // 2048), alpha=1.5, beta=1.5)
    plan, ck = _run_prefill(B, PL, c)
    rows = sorted(set(list(range(0, n_q, 5)) + [n_q - 1, n_q - 2, 0, 7, 8, 9]))
    _check_prefill(plan, ck, c, rows)


def test_prefill_bf16_block128(B, PL):
    # 128-token blocks: two 64-key chunks per kept block, ragged last block
    _say("prefill bf16 block_size=128")
    p = Params(block_size=128, topk=8, dense_len=0)
    c = make_prefill(9, n_k=7000, n_q=120, h_q=32, h_kv=2, d=128, params=p, dtype="bf16",
                     n_planted=3, alpha=1.5, beta=1.5)
    plan, ck = _run_prefill(B, PL, c)
    _check_prefill(plan, ck, c, rows=list(range(0, 120, 4)) + [119])


@pytest.mark.parametrize("bs,topk,rising", [
    (64, 32, True),      # the ring loop; later blocks score up to 16x higher
    (64, 32, False),     # the first blocks score highest: the running max never moves
    (128, 6, True),      # small top-k: ring and each token's own pass
])
def test_prefill_running_max_moves(B, PL, bs, topk, rising):
    """Keys scaled by powers of two per fifth of the context (exact in bf16),
    so that the kept blocks' scores rise by more than the softmax's rescale
    slack several times along a row (or only fall): the loop's full step
    with the row maximum and the O rescale, and its step that keeps the
    running maximum, both against the oracle."""
    _say(f"prefill bf16 running max moves: block={bs} topk={topk} rising={rising}")
    p = Params(block_size=bs, topk=topk, dense_len=0)
    n_k, n_q = 4096, 100
    c = make_prefill(23, n_k=n_k, n_q=n_q, h_q=32, h_kv=2, d=128, params=p, dtype="bf16",
                     n_planted=2, alpha=1.5, beta=1.5)
    level = np.minimum(np.arange(n_k) * 5 // n_k, 4)
    f = 2.0 ** (level if rising else 4 - level)
    c.k *= f[None, :, None]
    plan, ck = _run_prefill(B, PL, c)
    _check_prefill(plan, ck, c, rows=sorted(set(list(range(0, n_q, 3)) + [n_q - 1])))


@pytest.mark.parametrize("bs,n_k,n_q,h_q,h_kv,d,topk,dtype", [
    (96, 5000, 150, 32, 2, 128, 8, "bf16"),   # 16-head groups; last block 8 keys
    (96, 3030, 100, 8, 2, 64, 8, "bf16"),     # G = 4 (32-row tiles); last block 54 keys
    (32, 2500, 120, 32, 2, 128, 24, "bf16"),  # one 32-key chunk per block
    (32, 2000, 80, 16, 2, 64, 16, "bf16"),    # G = 8
    (96, 2000, 100, 2, 1, 64, 8, "f32"),
])
def test_prefill_blocks_not_multiple_of_64(B, PL, bs, n_k, n_q, h_q, h_kv, d, topk, dtype):
    # a 96-token block is a full and a half 64-key chunk, a 32-token block a
    # half chunk; chunks past the context hold no keys
    _say(f"prefill {dtype} block_size={bs} n_k={n_k} n_q={n_q} h_q={h_q} h_kv={h_kv} d={d}")
    p = Params(block_size=bs, topk=topk, dense_len=0)
    c = make_prefill(17, n_k=n_k, n_q=n_q, h_q=h_q, h_kv=h_kv, d=d, params=p, dtype=dtype,
                     n_planted=3, alpha=1.5, beta=1.5)
    plan, ck = _run_prefill(B, PL, c)
    _check_prefill(plan, ck, c, rows=sorted(set(list(range(0, n_q, 4)) + [n_q - 1, n_q - 2])))


def test_prefill_bf16_dense_below_dense_len(B, PL):
    _say("prefill bf16 dense")
    p = Params(dense_len=4096)
    c = make_prefill(6, n_k=4095, n_q=150, h_q=32, h_kv=2, d=128, params=p, dtype="bf16",
                     n_planted=2, alpha=1.5, beta=1.5)
    plan, ck = _run_prefill(B, PL, c)
    assert plan.dense
    _check_prefill(plan, ck, c, rows=list(range(0, 150, 3)) + [149])


# --------------------------------------------------------------- decode ----
def _run_decode(B, PL, c, cap=None):
    p = c.params
    bsz = len(c.seqlens)
    h_kv, _, d = c.k[0].shape
    h_q = c.q.shape[1]
    maxL = int(max(c.seqlens))
    cap = cap or ((maxL + 63) // 64) * 64
    kc = np.zeros((bsz, h_kv, cap, d), np.float32)
    vc = np.zeros((bsz, h_kv, cap, d), np.float32)
    for i, L in enumerate(c.seqlens):
        kc[i, :, :L] = c.k[i]
        vc[i, :, :L] = c.v[i]
    k = dev(kc, c.dtype)
    v = dev(vc, c.dtype)
    q = dev(c.q, c.dtype)
    seqlens = torch.from_numpy(np.asarray(c.seqlens, np.int32)).cuda()
    nc_cap = max(1, O.num_windows(cap, p.kernel_size, p.kernel_stride))
    ck = torch.zeros((bsz, h_kv, nc_cap, d), dtype=tdt(c.dtype), device="cuda")
    B.infllmv2_compress_keys(k, seqlens, 0, nc_cap, ck, p)
    plan = PL.DecodePlan(bsz, maxL, h_q, h_kv, d, tdt(c.dtype), p)
    plan.run(q, k, v, ck, seqlens)
    torch.cuda.synchronize()
    plan.inputs = (q, k, v, ck, seqlens)
    return plan


def _check_decode(plan, c):
    p = c.params
    res = O.decode(c.q, c.k, c.v, c.seqlens, p, c.dtype)
    out = host(plan.out)
    lse = plan.lse.cpu().numpy()
    sel = plan.block_idx.cpu().numpy()
    for i, L in enumerate(c.seqlens):
        pos = int(L) - 1
        if res["dense"][i]:
            ref_o, ref_l = res["o"][i], res["lse"][i]
        else:
            P = [check_selection(sel[i, g], res["S"][i][g], res["sel"][i][g], pos, p,
                                 f"seq {i} g {g}") for g in range(c.k[i].shape[0])]
            ref_o, ref_l = O.attend_selected(c.q[i], c.k[i], c.v[i], P, pos, p)
        check_close(out[i], ref_o, c.dtype, f"seq {i}")
        np.testing.assert_allclose(lse[i], ref_l, atol=2e-3 if c.dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("dtype,d,h_q,h_kv", [("bf16", 128, 32, 2), ("f32", 64, 4, 2),
                                              ("bf16", 64, 8, 1), ("bf16", 64, 16, 1)])
def test_decode_ragged(B, PL, dtype, d, h_q, h_kv):
    _say(f"decode ragged {dtype} d={d} h_q={h_q} h_kv={h_kv}")
    p = Params(dense_len=2048, topk=16)
    c = make_decode(7, [100, 2047, 2048, 5000, 9001, 64, 1], h_q=h_q, h_kv=h_kv, d=d, params=p,
                    dtype=dtype, planted_per_token=1 / 512)
    plan = _run_decode(B, PL, c)
    _check_decode(plan, c)


def test_decode_score_mode1(B, PL):
    # selection from the per-head-softmax group score, end to end
    _say("decode bf16 score_mode=1")
    p = Params(dense_len=2048, topk=16, score_mode=1)
    c = make_decode(14, [100, 3000, 9001, 5000], h_q=32, h_kv=2, d=128, params=p,
                    dtype="bf16", planted_per_token=1 / 512)
    plan = _run_decode(B, PL, c)
    _check_decode(plan, c)


def test_prefill_score_mode1(B, PL):
    _say("prefill bf16 score_mode=1")
    p = Params(topk=16, dense_len=0, score_mode=1)
    c = make_prefill(15, n_k=5000, n_q=150, h_q=32, h_kv=2, d=128, params=p, dtype="bf16",
                     n_planted=3, alpha=1.5, beta=1.5)
    plan, ck = _run_prefill(B, PL, c)
    _check_prefill(plan, ck, c, rows=list(range(0, 150, 7)) + [149])


def test_decode_block128(B, PL):
    # 128-token blocks: two 64-key chunks per kept block in the split ranges
    _say("decode bf16 block_size=128")
    p = Params(block_size=128, topk=8, dense_len=2048)
    c = make_decode(12, [100, 2047, 2048, 5000, 9001, 200], h_q=32, h_kv=2, d=128, params=p,
                    dtype="bf16", planted_per_token=1 / 512)
    plan = _run_decode(B, PL, c)
    _check_decode(plan, c)


@pytest.mark.parametrize("bs,topk", [(96, 8), (32, 24)])
def test_decode_blocks_not_multiple_of_64(B, PL, bs, topk):
    _say(f"decode bf16 block_size={bs} topk={topk}")
    p = Params(block_size=bs, topk=topk, dense_len=2048)
    c = make_decode(16, [100, 2047, 2048, 5000, 9001, 200, 4130], h_q=32, h_kv=2, d=128,
                    params=p, dtype="bf16", planted_per_token=1 / 512)
    plan = _run_decode(B, PL, c)
    _check_decode(plan, c)


def test_decode_large_batch_fewer_splits(B, PL):
    # 40 sequences x 2 KV heads: the split count falls to ceil(256 / 80) = 4
    _say("decode bf16 batch 40")
    p = Params(dense_len=2048, topk=16)
    lens = [int(x) for x in np.random.default_rng(13).integers(1, 9000, 40)]
    c = make_decode(13, lens, h_q=32, h_kv=2, d=128, params=p, dtype="bf16",
                    planted_per_token=1 / 512)
    plan = _run_decode(B, PL, c)
    _check_decode(plan, c)


def test_decode_repeated_calls_reuse_workspace(B, PL):
    # a workspace holds nothing across calls: reusing it gives the same result
    _say("decode repeated calls")
    p = Params(dense_len=2048, topk=16)
    c = make_decode(11, [3000, 9001, 64], h_q=32, h_kv=2, d=128, params=p, dtype="bf16",
                    planted_per_token=1 / 512)
    plan = _run_decode(B, PL, c)
    first = plan.out.clone()
    plan.ws.fill_(0xAB)
    for _ in range(3):
        plan.run(*plan.inputs)
        torch.cuda.synchronize()
        assert torch.equal(plan.out, first)
    _check_decode(plan, c)


# ----------------------------------------------------------------- tree ----
@pytest.mark.parametrize("dtype,n_ctx,T,dense_len,bs,heads", [
    ("bf16", 12000, 16, 8192, 64, (32, 2, 128)),
    ("bf16", 5000, 16, 8192, 64, (32, 2, 128)),
    ("bf16", 9000, 40, 0, 64, (32, 2, 128)),
    ("bf16", 9000, 16, 0, 128, (32, 2, 128)),
    ("bf16", 9000, 16, 0, 96, (32, 2, 128)),
    # other group sizes: union planner and the 32-row tile kernel
    ("bf16", 9000, 16, 0, 64, (8, 2, 64)),       # G = 4
    ("bf16", 6000, 20, 0, 64, (16, 2, 128)),     # G = 8
    ("bf16", 7000, 16, 8192, 64, (8, 2, 128)),   # G = 4, dense
    ("f32", 3000, 7, 0, 64, (4, 2, 64))])
def test_tree_verify(B, PL, dtype, n_ctx, T, dense_len, bs, heads):
    h_q, h_kv, d = heads
    _say(f"tree {dtype} n_ctx={n_ctx} T={T} dense_len={dense_len} block={bs} "
         f"h_q={h_q} h_kv={h_kv} d={d}")
    p = Params(dense_len=dense_len, topk=16 if bs == 64 else 8, block_size=bs)
    c = make_tree(8, n_ctx=n_ctx, n_draft=T, h_q=h_q, h_kv=h_kv, d=d, params=p, dtype=dtype,
                  n_planted=max(1, n_ctx // 2048))
    q = dev(c.q, dtype)
    k = dev(c.k, dtype)
    v = dev(c.v, dtype)
    kd = dev(c.k_draft, dtype)
    vd = dev(c.v_draft, dtype)
    mask = torch.from_numpy(c.mask.astype(np.int64)).cuda()
    nc = O.num_windows(n_ctx, 32, 16)
    ck = torch.zeros((h_kv, nc, d), dtype=tdt(dtype), device="cuda")
    B.infllmv2_compress_keys(k.unsqueeze(0), torch.tensor([n_ctx], dtype=torch.int32,
                                                          device="cuda"), 0, nc,
                             ck.unsqueeze(0), p)
    plan = PL.TreePlan(T, n_ctx, h_q, h_kv, d, tdt(dtype), p)
    plan.run(q, k, v, ck, kd, vd, mask)
    torch.cuda.synchronize()
    res = O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, c.mask, p, dtype)
    out = host(plan.out)
    lse = plan.lse.cpu().numpy()
    pos = n_ctx - 1
    for i in range(T):
        anc = [j for j in range(T) if (int(c.mask[i]) >> j) & 1]
        extra = (c.k_draft[:, anc], c.v_draft[:, anc])
        if res["dense"]:
            ref_o, ref_l = res["o"][i], res["lse"][i]
        else:
            sel = plan.block_idx.cpu().numpy()
            P = [check_selection(sel[i, g], res["S"][i][g], res["sel"][i][g], pos, p,
                                 f"draft {i} g {g}") for g in range(h_kv)]
            ref_o, ref_l = O.attend_selected(c.q[i], c.k, c.v, P, pos, p, extra)
        check_close(out[i], ref_o, dtype, f"draft {i}")
        np.testing.assert_allclose(lse[i], ref_l, atol=2e-3 if dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("dtype,n_ctx,dense_len,heads", [
    ("bf16", 9000, 0, (32, 2, 128)),      # 16-head groups: drafts as decode rows
    ("bf16", 5000, 8192, (32, 2, 128)),   # dense context
    ("bf16", 9000, 0, (8, 2, 64)),        # G = 4: union planner + 32-row tiles
    ("f32", 3000, 0, (4, 2, 64)),         # float32 path
])
def test_tree_verify_mask_self_bit_and_high_bits(B, PL, dtype, n_ctx, dense_len, heads):
    """A draft always attends itself and mask bits at or above the draft count
    name no draft: masks with every self bit cleared and high bits set give
    the oracle's result (which follows the same reading) and exactly the
    result of the plain ancestor masks."""
    h_q, h_kv, d = heads
    T = 12
    _say(f"tree odd masks {dtype} n_ctx={n_ctx} dense_len={dense_len} h_q={h_q} h_kv={h_kv}")
    p = Params(dense_len=dense_len, topk=16)
    c = make_tree(9, n_ctx=n_ctx, n_draft=T, h_q=h_q, h_kv=h_kv, d=d, params=p, dtype=dtype,
                  n_planted=max(1, n_ctx // 2048))
    odd = c.mask.copy()
    for i in range(T):
        odd[i] = np.uint64((int(odd[i]) & ~(1 << i)) | (0xF << (60 - i % 8)) | (1 << (T + i)))
    assert all(not (int(odd[i]) >> i) & 1 for i in range(T))
    q, k, v = dev(c.q, dtype), dev(c.k, dtype), dev(c.v, dtype)
    kd, vd = dev(c.k_draft, dtype), dev(c.v_draft, dtype)
    nc = O.num_windows(n_ctx, 32, 16)
    ck = torch.zeros((h_kv, nc, d), dtype=tdt(dtype), device="cuda")
    B.infllmv2_compress_keys(k.unsqueeze(0), torch.tensor([n_ctx], dtype=torch.int32,
                                                          device="cuda"), 0, nc,
                             ck.unsqueeze(0), p)
    plan = PL.TreePlan(T, n_ctx, h_q, h_kv, d, tdt(dtype), p)
    plan.run(q, k, v, ck, kd, vd, torch.from_numpy(c.mask.astype(np.int64)).cuda())
    torch.cuda.synchronize()
    plain_out, plain_lse = plan.out.clone(), plan.lse.clone()
    plan.run(q, k, v, ck, kd, vd, torch.from_numpy(odd.view(np.int64)).cuda())
    torch.cuda.synchronize()
    assert torch.equal(plan.out, plain_out) and torch.equal(plan.lse, plain_lse)
    res = O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, odd, p, dtype)
    out = host(plan.out)
    lse = plan.lse.cpu().numpy()
    pos = n_ctx - 1
    for i in range(T):
        anc = sorted({i} | {j for j in range(T) if (int(odd[i]) >> j) & 1})
        extra = (c.k_draft[:, anc], c.v_draft[:, anc])
        if res["dense"]:
            ref_o, ref_l = res["o"][i], res["lse"][i]
        else:
            sel = plan.block_idx.cpu().numpy()
            P = [check_selection(sel[i, g], res["S"][i][g], res["sel"][i][g], pos, p,
                                 f"draft {i} g {g}") for g in range(h_kv)]
            ref_o, ref_l = O.attend_selected(c.q[i], c.k, c.v, P, pos, p, extra)
        check_close(out[i], ref_o, dtype, f"draft {i}")
        np.testing.assert_allclose(lse[i], ref_l, atol=2e-3 if dtype == "bf16" else 1e-4)


# ------------------------------------------------------ whole-prompt prefill ----
def test_chunked_prefill_whole_prompt(B, PL):
    """A 2560-token prompt prefilled in 5 chunks of 512 (the first, with fewer
    keys than dense_len, dense): the compressed-key cache grows chunk by
    chunk and every chunk's sampled rows match the oracle's prefill of the
    whole prompt."""
    _say("chunked prefill: 2560 tokens in chunks of 512, dense_len 1024")
    p = Params(topk=8, dense_len=1024)
    n, chunk = 2560, 512
    c = make_prefill(31, n_k=n, n_q=n, h_q=32, h_kv=2, d=128, params=p, dtype="bf16",
                     n_planted=3, alpha=1.5, beta=1.5)
    q, k, v = dev(c.q, "bf16"), dev(c.k, "bf16"), dev(c.v, "bf16")
    nc = O.num_windows(n, p.kernel_size, p.kernel_stride)
    ck = torch.full((2, nc, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    cp = PL.ChunkedPrefill(n, chunk, 32, 2, 128, torch.bfloat16, p)
    cp.run(q, k, v, ck)
    torch.cuda.synchronize()
    assert [pl.dense for pl in cp.plans] == [True, False, False, False, False]
    # every window written once the whole prompt has passed
    _check_ck(host(ck), O.compress_keys(c.k, p, "bf16"), "bf16", "compressed keys")
    rows = sorted(set(r for q0 in range(0, n, chunk)
                      for r in (q0, q0 + 1, q0 + 63, q0 + 64, q0 + 255, q0 + chunk - 1)))
    res = O.prefill(c.q, c.k, c.v, p, "bf16", rows=rows)
    out = host(cp.out)
    lse = cp.lse.cpu().numpy()
    for i in rows:
        ci = i // chunk
        pl = cp.plans[ci]
        if pl.dense:
            ref_o, ref_l = O.dense_attend(c.q[i], c.k, c.v, i, p)
        else:
            # selections of the chunk's rows are in the shared scratch of the
            # last run only for the last chunk: recompute this chunk's selection
            pl.select(q[ci * chunk:(ci + 1) * chunk], ck)
            torch.cuda.synchronize()
            sel = pl.block_idx.cpu().numpy()[i - ci * chunk]
            P = [check_selection(sel[g], res["S"][i][g], res["sel"][i][g], i, p,
                                 f"row {i} g {g}") for g in range(2)]
            ref_o, ref_l = O.attend_selected(c.q[i], c.k, c.v, P, i, p)
        check_close(out[i], ref_o, "bf16", f"row {i}")
        np.testing.assert_allclose(lse[i], ref_l, atol=2e-3)


def test_chunked_prefill_overlap_matches_one_stream(B, PL):
    """The overlapped schedule (each chunk's selection on a second stream,
    alternating selection buffers) gives the one-stream run's outputs, bit
    for bit, on a prompt of 6 chunks (more than the two buffers)."""
    _say("chunked prefill: overlapped schedule vs one stream, 3072 tokens in 6 chunks")
    p = Params(topk=8, dense_len=1024)
    n, chunk = 3072, 512
    c = make_prefill(32, n_k=n, n_q=n, h_q=32, h_kv=2, d=128, params=p, dtype="bf16",
                     n_planted=3, alpha=1.5, beta=1.5)
    q, k, v = dev(c.q, "bf16"), dev(c.k, "bf16"), dev(c.v, "bf16")
    nc = O.num_windows(n, p.kernel_size, p.kernel_stride)
    outs = []
    for overlap in (False, True):
        ck = torch.zeros((2, nc, 128), dtype=torch.bfloat16, device="cuda")
        cp = PL.ChunkedPrefill(n, chunk, 32, 2, 128, torch.bfloat16, p, overlap=overlap)
        cp.run(q, k, v, ck)
        torch.cuda.synchronize()
        outs.append((cp.out.clone(), cp.lse.clone(), ck.clone()))
    for a, b, what in zip(outs[0], outs[1], ("out", "lse", "compressed keys")):
        assert torch.equal(a, b), f"{what} differ"
