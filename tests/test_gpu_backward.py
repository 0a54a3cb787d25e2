"""GPU parity of the prefill backward (infllmv2_sparse_attn_prefill_backward)
against the oracle's prefill_backward, with the kept blocks fixed.

Selections are seeded random valid lists (forced initial and local blocks,
the rest drawn from the eligible blocks, ascending, -1 padded) so that every
kernel path sees irregular patterns; the full-size case uses the selections
of the forward pipeline.  The forward's own output and log-sum-exp feed the
backward, as in training.

Tolerance (parity.check_grad): the bf16 output bars of the forward, applied
relative to the reference gradient's largest magnitude.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_long_infllmv2_amd.workloads import Params, make_prefill, make_upstream_grad
from parity import check_grad

pytestmark = pytest.mark.gpu

def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_long_infllmv2_amd import binding
    return binding


def dev(x, dtype="bf16"):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def random_selection(seed, n_q, n_k, h_kv, p):
    """Valid kept-block lists [n_q][h_kv][topk]: forced blocks plus random
    eligible ones, ascending, -1 padded."""
    rng = np.random.default_rng(seed)
    B = p.block_size
    out = np.full((n_q, h_kv, p.topk), -1, np.int32)
    for i in range(n_q):
        pos = n_k - n_q + i
        own = pos // B
        forced = set(range(min(p.init_blocks, own + 1)))
        forced |= set(range(max(0, own - p.local_blocks + 1), own + 1))
        want = min(p.topk, own + 1)
        for g in range(h_kv):
            rest = [b for b in range(own + 1) if b not in forced]
            extra = rng.choice(rest, size=want - len(forced), replace=False) if rest else []
            sel = sorted(forced | set(int(b) for b in extra))
            out[i, g, :len(sel)] = sel
    return out


def run_backward(B, c, sel, d_out, dk0=None, dv0=None):
    """Forward then backward on the GPU; returns (dq, dk, dv) on the host."""
    p = c.params
    n_q, h_q, d = c.q.shape
    h_kv, n_k, _ = c.k.shape
    q, k, v = dev(c.q, c.dtype), dev(c.k, c.dtype), dev(c.v, c.dtype)
    bi = torch.from_numpy(sel).cuda() if sel is not None else None
    out = torch.empty_like(q)
    lse = torch.empty((n_q, h_q), dtype=torch.float32, device="cuda")
    B.infllmv2_sparse_attn_prefill(q, k, v, n_k, bi, out, lse, p)
    do = dev(d_out, c.dtype)
    dq = torch.empty_like(q)
    dk = torch.zeros((h_kv, n_k, d), dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    if dk0 is not None:
        dk.copy_(torch.from_numpy(dk0))
        dv.copy_(torch.from_numpy(dv0))
    nbytes = B.infllmv2_workspace_size(B.OP_PREFILL_BWD, n_q, h_q, h_kv, d, n_k, p)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    B.infllmv2_sparse_attn_prefill_backward(q, k, v, n_k, bi, out, lse, do, dq, dk, dv, ws, p)
    torch.cuda.synchronize()
    return host(dq), dk.cpu().numpy().astype(np.float64), dv.cpu().numpy().astype(np.float64)


def oracle_sel_rows(sel, dense):
    if dense:
        return [None] * sel_len(sel)
    return [[s[s >= 0] for s in row] for row in sel]


def sel_len(sel):
    return sel if isinstance(sel, int) else len(sel)


def case(seed, n_k, n_q, h_q, h_kv, d, dtype="bf16", **pover):
    p = Params(**pover)
    return make_prefill(seed, n_k, n_q, h_q, h_kv, d, p, dtype, n_planted=4, alpha=1.0,
                        beta=1.5, name="bwd")


def compare(B, c, sel, where, dense=False):
    d_out = make_upstream_grad(7, c.n_q, c.q.shape[1], c.q.shape[2], c.dtype)
    dq, dk, dv = run_backward(B, c, None if dense else sel, d_out)
    rows = [None] * c.n_q if dense else [[s[s >= 0] for s in row] for row in sel]
    rq, rk, rv = O.prefill_backward(c.q, c.k, c.v, rows, c.params, d_out)
    check_grad(dq, rq, f"{where} dq", c.dtype)
    check_grad(dk, rk, f"{where} dk", c.dtype)
    check_grad(dv, rv, f"{where} dv", c.dtype)
    return dq, dk, dv, d_out


def test_backward_sparse_g16_d128(B):
    _say("backward sparse G=16 d=128 n_k=4096 n_q=200 topk=16")
    c = case(1, 4096, 200, 32, 2, 128, topk=16, dense_len=0)
    sel = random_selection(11, c.n_q, c.n_k, 2, c.params)
    compare(B, c, sel, "sparse g16")


def test_backward_dense_g16_d128(B):
    _say("backward dense G=16 d=128 n_k=n_q=300")
    c = case(2, 300, 300, 32, 2, 128)
    compare(B, c, None, "dense g16", dense=True)


def test_backward_dense_chunk_after_context(B):
    _say("backward dense chunk: 150 queries after 500 keys, G=8 d=64")
    c = case(3, 650, 150, 8, 1, 64)
    compare(B, c, None, "dense chunk", dense=True)


@pytest.mark.parametrize("G,h_kv,d", [(1, 2, 64), (2, 2, 64), (4, 2, 128), (8, 2, 64),
                                      (32, 1, 64)])
def test_backward_groups(B, G, h_kv, d):
    _say(f"backward sparse G={G} h_kv={h_kv} d={d} n_k=2048 n_q=100 topk=8")
    c = case(4 + G, 2048, 100, G * h_kv, h_kv, d, topk=8, dense_len=0)
    sel = random_selection(20 + G, c.n_q, c.n_k, h_kv, c.params)
    compare(B, c, sel, f"G={G}")


def test_backward_block128_ragged_keys(B):
    _say("backward block 128, n_k=4000 (ragged last chunk), n_q=150, topk=8")
    c = case(30, 4000, 150, 32, 2, 128, block_size=128, topk=8, dense_len=0)
    sel = random_selection(31, c.n_q, c.n_k, 2, c.params)
    compare(B, c, sel, "block128")


def test_backward_many_segments(B):
    _say("backward: 700 rows keep block 0 (several dK/dV segments per chunk), G=16")
    c = case(40, 3000, 700, 32, 2, 64, topk=6, dense_len=0)
    sel = random_selection(41, c.n_q, c.n_k, 2, c.params)
    compare(B, c, sel, "segments")


def test_backward_accumulates_into_dk_dv(B):
    _say("backward adds into dk/dv that already hold values")
    c = case(50, 1024, 64, 16, 2, 64, topk=4, dense_len=0)
    sel = random_selection(51, c.n_q, c.n_k, 2, c.params)
    d_out = make_upstream_grad(52, c.n_q, 16, 64, "bf16")
    rng = np.random.default_rng(53)
    dk0 = rng.standard_normal((2, c.n_k, 64)).astype(np.float32)
    dv0 = rng.standard_normal((2, c.n_k, 64)).astype(np.float32)
    dq, dk, dv = run_backward(B, c, sel, d_out, dk0, dv0)
    rows = [[s[s >= 0] for s in row] for row in sel]
    rq, rk, rv = O.prefill_backward(c.q, c.k, c.v, rows, c.params, d_out)
    check_grad(dk - dk0, rk, "dk added")
    check_grad(dv - dv0, rv, "dv added")
    # keys no row attends keep their values exactly
    attended = np.zeros((2, c.n_k), bool)
    for i in range(c.n_q):
        pos = c.n_k - c.n_q + i
        for g in range(2):
            for b in rows[i][g]:
                attended[g, b * 64:min((b + 1) * 64, pos + 1)] = True
    assert np.array_equal(dk[~attended], dk0[~attended].astype(np.float64))
    assert np.array_equal(dv[~attended], dv0[~attended].astype(np.float64))


def test_backward_rejects_small_workspace(B):
    _say("backward argument checks")
    p = Params(dense_len=0, topk=4)
    n_q, n_k, h_q, h_kv, d = 8, 256, 4, 2, 64
    q = torch.zeros((n_q, h_q, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((h_kv, n_k, d), dtype=torch.bfloat16, device="cuda")
    bi = torch.zeros((n_q, h_kv, 4), dtype=torch.int32, device="cuda")
    lse = torch.zeros((n_q, h_q), dtype=torch.float32, device="cuda")
    dk = torch.zeros((h_kv, n_k, d), dtype=torch.float32, device="cuda")
    nbytes = B.infllmv2_workspace_size(B.OP_PREFILL_BWD, n_q, h_q, h_kv, d, n_k, p)
    small = torch.empty(max(256, nbytes - 512), dtype=torch.uint8, device="cuda")
    with pytest.raises(B.InfLLMv2Error, match="workspace"):
        B.infllmv2_sparse_attn_prefill_backward(q, k, k, n_k, bi, q, lse, q, q, dk, dk, small, p)


@pytest.mark.parametrize("n_k,n_q,h_q,h_kv,d,bs,dense_len", [
    (2048, 128, 2, 1, 64, 64, 0),          # the tiny float32 configuration's shape
    (200, 200, 8, 2, 128, 64, 8192),       # dense
    (1500, 90, 6, 3, 64, 32, 0),           # 32-token blocks, group of 2, three KV heads
])
def test_backward_f32(B, n_k, n_q, h_q, h_kv, d, bs, dense_len):
    _say(f"backward float32 n_k={n_k} n_q={n_q} h_q={h_q} h_kv={h_kv} d={d} B={bs}")
    c = case(90 + n_k, n_k, n_q, h_q, h_kv, d, dtype="f32", topk=8, block_size=bs,
             dense_len=dense_len)
    dense = n_k < dense_len
    sel = None if dense else random_selection(91, n_q, n_k, h_kv, c.params)
    compare(B, c, sel, f"f32 {n_k}x{n_q}", dense=dense)


def test_backward_block192(B):
    _say("backward block 192 (three 64-key chunks per block), n_k=3000, n_q=120, topk=6")
    c = case(60, 3000, 120, 16, 2, 64, block_size=192, topk=6, dense_len=0)
    sel = random_selection(61, c.n_q, c.n_k, 2, c.params)
    compare(B, c, sel, "block192")


@pytest.mark.parametrize("overlap", [False, True])
def test_backward_whole_prompt_in_chunks(B, overlap):
    """A 2500-token prompt run forward and backward in chunks of 1000 (the
    first chunk dense, the others sparse): every chunk adds its dk/dv into the
    same buffers, and the result equals the oracle's backward of the whole
    prompt with each row's selection as the forward made it.  overlap: the
    forward's two-stream schedule (selections under the previous chunk's
    attention) with every chunk's selection kept."""
    _say(f"chunked backward: 2500 tokens in chunks of 1000, dense_len 1500, overlap={overlap}")
    from block_sparse_long_infllmv2_amd import pipeline as PL
    p = Params(topk=8, dense_len=1500)
    n, chunk, h_q, h_kv, d = 2500, 1000, 16, 1, 64
    c = make_prefill(70, n_k=n, n_q=n, h_q=h_q, h_kv=h_kv, d=d, params=p, dtype="bf16",
                     n_planted=3, alpha=1.5, beta=1.5)
    q, k, v = dev(c.q), dev(c.k), dev(c.v)
    nc = O.num_windows(n, p.kernel_size, p.kernel_stride)
    ck = torch.zeros((h_kv, nc, d), dtype=torch.bfloat16, device="cuda")
    cp = PL.ChunkedPrefill(n, chunk, h_q, h_kv, d, torch.bfloat16, p, keep_selections=True,
                           overlap=overlap)
    cp.run(q, k, v, ck)
    d_out = make_upstream_grad(71, n, h_q, d, "bf16")
    dq = torch.empty_like(q)
    dk = torch.zeros((h_kv, n, d), dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    cp.backward(q, k, v, dev(d_out), dq, dk, dv)
    torch.cuda.synchronize()
    assert [pl.dense for pl in cp.plans] == [True, False, False]
    sel = cp.idx_buf.view(n, h_kv, p.topk).cpu().numpy()
    rows = [None if cp.plans[i // chunk].dense else [s[s >= 0] for s in sel[i]]
            for i in range(n)]
    rq, rk, rv = O.prefill_backward(c.q, c.k, c.v, rows, p, d_out)
    check_grad(host(dq), rq, "chunked dq")
    check_grad(dk.cpu().numpy(), rk, "chunked dk")
    check_grad(dv.cpu().numpy(), rv, "chunked dv")


@pytest.mark.parametrize("n_k,n_q,dense_len", [(1, 1, 8192), (40, 40, 8192), (700, 1, 0),
                                               (63, 17, 0)])
def test_backward_tiny_shapes(B, n_k, n_q, dense_len):
    _say(f"backward tiny shape n_k={n_k} n_q={n_q} dense_len={dense_len}")
    c = case(80 + n_k, n_k, n_q, 16, 2, 64, topk=4, dense_len=dense_len)
    dense = n_k < dense_len
    sel = None if dense else random_selection(81, n_q, n_k, 2, c.params)
    compare(B, c, sel, f"tiny {n_k}x{n_q}", dense=dense)


def test_backward_cache_larger_than_context(B):
    """K/V caches with cap > n_k (room for later tokens), 4 KV heads: keys
    past n_k are never read as data nor written in dk/dv."""
    _say("backward with cap = n_k + 100, h_kv = 4, G = 4, d = 128")
    p = Params(topk=6, dense_len=0)
    n_k, n_q, h_q, h_kv, d, cap = 1900, 70, 16, 4, 128, 2000
    c = make_prefill(95, n_k, n_q, h_q, h_kv, d, p, "bf16", n_planted=2, alpha=1.0, beta=1.5)
    sel = random_selection(96, n_q, n_k, h_kv, p)
    d_out = make_upstream_grad(97, n_q, h_q, d, "bf16")
    kc = torch.full((h_kv, cap, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    kc[:, :n_k] = dev(c.k)
    vc[:, :n_k] = dev(c.v)
    q = dev(c.q)
    bi = torch.from_numpy(sel).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((n_q, h_q), dtype=torch.float32, device="cuda")
    B.infllmv2_sparse_attn_prefill(q, kc, vc, n_k, bi, out, lse, p)
    dq = torch.empty_like(q)
    dk = torch.zeros((h_kv, cap, d), dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    ws = torch.empty(B.infllmv2_workspace_size(B.OP_PREFILL_BWD, n_q, h_q, h_kv, d, n_k, p),
                     dtype=torch.uint8, device="cuda")
    B.infllmv2_sparse_attn_prefill_backward(q, kc, vc, n_k, bi, out, lse, dev(d_out), dq, dk, dv,
                                            ws, p)
    torch.cuda.synchronize()
    dkh = dk.cpu().numpy().astype(np.float64)
    dvh = dv.cpu().numpy().astype(np.float64)
    assert np.all(dkh[:, n_k:] == 0) and np.all(dvh[:, n_k:] == 0), "keys past n_k written"
    rows = [[s[s >= 0] for s in row] for row in sel]
    rq, rk, rv = O.prefill_backward(c.q, c.k, c.v, rows, p, d_out)
    check_grad(host(dq), rq, "cap dq")
    check_grad(dkh[:, :n_k], rk, "cap dk")
    check_grad(dvh[:, :n_k], rv, "cap dv")


def test_backward_more_blocks_than_the_lds_bitmap_column(B):
    """n_b = 16401 blocks, more than the 16384-word LDS column of the row
    bitmap: the bitmap is cleared and marked with global atomics instead."""
    n_k = 64 * 16400 + 37
    _say(f"backward n_k={n_k} (16401 blocks) n_q=40 G=2 d=64 topk=4")
    c = case(70, n_k, 40, 2, 1, 64, topk=4, dense_len=0)
    sel = random_selection(71, c.n_q, n_k, 1, c.params)
    compare(B, c, sel, "16401 blocks")
