"""GPU: the decode and tree-verification calls that make their own top-k
selection from block scores (infllmv2_sparse_attn_decode_topk,
infllmv2_tree_verify_topk) give, bit for bit, what the top-k call followed by
the plain attention call gives on the same scores: outputs, log-sum-exps and
the selection they write.  Cases cover the selection inside the 16-head
kernels (rows of up to 1024, 2048 and 4096 blocks), the shapes that run the
top-k kernel first (longer rows, other group sizes, float32), dense rows in a
sparse batch, and scores with many ties.  Inputs: seeded normal K/V/Q drawn
on the device (no oracle here: the two-call path is checked against the
oracle by the stage tests)."""
import sys

import pytest
import torch

from block_sparse_long_infllmv2_amd.workloads import Params

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


def _n_windows(n, ks, s):
    return 0 if n < ks else (n - ks) // s + 1


def _tie(scores):
    # few distinct values: many equal scores, ranked by block index
    scores.copy_(torch.round(scores * 2.0) / 2.0)


def _same(a, b, what):
    assert a.shape == b.shape, what
    if a.dtype.is_floating_point:
        eq = (a == b) | (torch.isnan(a) & torch.isnan(b))
    else:
        eq = a == b
    bad = int((~eq).sum())
    assert bad == 0, f"{what}: {bad} of {a.numel()} differ"


@pytest.mark.parametrize("lens,h_q,h_kv,d,bs,topk,dtype,ties", [
    # selection inside the 16-head kernel: rows of <= 1024 / 2048 / 4096 blocks
    ([100, 2047, 2048, 5000, 9001, 64, 1], 32, 2, 128, 64, 16, "bf16", False),
    ([100, 2047, 2048, 5000, 9001, 64, 1], 32, 2, 128, 64, 16, "bf16", True),
    ([70000, 130000, 3000], 32, 2, 128, 64, 64, "bf16", False),
    ([250000, 9001], 16, 1, 64, 64, 64, "bf16", True),
    ([2047, 5000, 9001, 200, 30000], 32, 2, 128, 128, 8, "bf16", False),
    ([2047, 5000, 9001, 4130], 32, 2, 128, 96, 8, "bf16", False),
    # the top-k kernel first: 4688 blocks, 8-head groups, float32
    ([300000], 16, 1, 128, 64, 64, "bf16", False),
    ([100, 5000, 9001], 16, 2, 64, 64, 16, "bf16", True),
    ([100, 5000, 9001], 4, 2, 64, 64, 16, "f32", False),
])
def test_decode_select_in_attend_matches_two_calls(B, PL, lens, h_q, h_kv, d, bs, topk, dtype,
                                                   ties):
    _say(f"decode select-in-attend lens={lens} h_q={h_q} h_kv={h_kv} d={d} block={bs} "
         f"topk={topk} {dtype} ties={ties}")
    p = Params(block_size=bs, topk=topk, dense_len=2048)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(sum(lens) + h_q + bs)
    bsz, maxL = len(lens), max(lens)
    cap = ((maxL + 63) // 64) * 64
    k = torch.randn((bsz, h_kv, cap, d), generator=g, device="cuda").to(tdt)
    v = torch.randn((bsz, h_kv, cap, d), generator=g, device="cuda").to(tdt)
    q = (torch.randn((bsz, h_q, d), generator=g, device="cuda") * 2.0).to(tdt)
    seqlens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    nc = max(1, _n_windows(cap, p.kernel_size, p.kernel_stride))
    ck = torch.zeros((bsz, h_kv, nc, d), dtype=tdt, device="cuda")
    B.infllmv2_compress_keys(k, seqlens, 0, nc, ck, p)
    two = PL.DecodePlan(bsz, maxL, h_q, h_kv, d, tdt, p, select_in_attend=False)
    one = PL.DecodePlan(bsz, maxL, h_q, h_kv, d, tdt, p, select_in_attend=True)
    two.select(q, ck, seqlens)
    if ties:
        _tie(two.scores)
        B.infllmv2_select_topk(two.scores, two.row_seq, None, seqlens, two.block_idx, p)
    two.attend(q, k, v, seqlens)
    one.scores.copy_(two.scores)
    one.block_idx.fill_(-7)
    one.ws.fill_(0x5A)
    one.attend(q, k, v, seqlens)
    torch.cuda.synchronize()
    _same(one.block_idx, two.block_idx, "selection")
    _same(one.out, two.out, "out")
    _same(one.lse, two.lse, "lse")


@pytest.mark.parametrize("n_ctx,T,h_q,h_kv,d,bs,topk,dtype,ties", [
    (12000, 16, 32, 2, 128, 64, 16, "bf16", False),
    (9000, 40, 32, 2, 128, 64, 16, "bf16", True),
    (131072, 16, 32, 2, 128, 64, 64, "bf16", False),
    (9000, 16, 32, 2, 128, 128, 8, "bf16", False),
    (9000, 16, 8, 2, 64, 64, 16, "bf16", False),       # 4-head groups: top-k kernel first
    (3000, 7, 4, 2, 64, 64, 16, "f32", False),
])
def test_tree_select_in_attend_matches_two_calls(B, PL, n_ctx, T, h_q, h_kv, d, bs, topk,
                                                 dtype, ties):
    _say(f"tree select-in-attend n_ctx={n_ctx} T={T} h_q={h_q} h_kv={h_kv} d={d} block={bs} "
         f"topk={topk} {dtype} ties={ties}")
    p = Params(block_size=bs, topk=topk, dense_len=0)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(n_ctx + T + bs)
    k = torch.randn((h_kv, n_ctx, d), generator=g, device="cuda").to(tdt)
    v = torch.randn((h_kv, n_ctx, d), generator=g, device="cuda").to(tdt)
    kd = torch.randn((h_kv, T, d), generator=g, device="cuda").to(tdt)
    vd = torch.randn((h_kv, T, d), generator=g, device="cuda").to(tdt)
    q = (torch.randn((T, h_q, d), generator=g, device="cuda") * 2.0).to(tdt)
    # chain-with-branches ancestry: parent of i is (i - 1) // 2
    masks = []
    for i in range(T):
        m, j = 1 << i, i
        while j > 0:
            j = (j - 1) // 2
            m |= 1 << j
        masks.append(m - (1 << 64) if m >= 1 << 63 else m)
    mask = torch.tensor(masks, dtype=torch.int64, device="cuda")
    nc = _n_windows(n_ctx, p.kernel_size, p.kernel_stride)
    ck = torch.zeros((h_kv, nc, d), dtype=tdt, device="cuda")
    B.infllmv2_compress_keys(k.unsqueeze(0), torch.tensor([n_ctx], dtype=torch.int32,
                                                          device="cuda"), 0, nc,
                             ck.unsqueeze(0), p)
    two = PL.TreePlan(T, n_ctx, h_q, h_kv, d, tdt, p, select_in_attend=False)
    one = PL.TreePlan(T, n_ctx, h_q, h_kv, d, tdt, p, select_in_attend=True)
    two.select(q, ck)
    if ties:
        _tie(two.scores)
        B.infllmv2_select_topk(two.scores, None, two.row_pos, two.seqlens, two.block_idx, p)
    two.attend(q, k, v, kd, vd, mask)
    one.scores.copy_(two.scores)
    one.block_idx.fill_(-7)
    one.attend(q, k, v, kd, vd, mask)
    torch.cuda.synchronize()
    _same(one.block_idx, two.block_idx, "selection")
    _same(one.out, two.out, "out")
    _same(one.lse, two.lse, "lse")


def test_select_in_attend_dense_calls_need_no_scores(B, PL):
    """Below dense_len nothing is selected: the selecting calls accept NULL
    scores and selection and give the list-taking calls' dense results."""
    _say("select-in-attend: dense decode and tree without scores")
    p = Params(dense_len=8192, topk=16)
    g = torch.Generator(device="cuda").manual_seed(77)
    lens = [100, 3000, 8191]
    bsz, cap, d = len(lens), 8192, 128
    k = torch.randn((bsz, 2, cap, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((bsz, 2, cap, d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((bsz, 32, d), generator=g, device="cuda").to(torch.bfloat16)
    seqlens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    plan = PL.DecodePlan(bsz, max(lens), 32, 2, d, torch.bfloat16, p)
    out2, lse2 = torch.empty_like(plan.out), torch.empty_like(plan.lse)
    B.infllmv2_sparse_attn_decode(q, k, v, seqlens, max(lens), None, plan.out, plan.lse,
                                  plan.ws, p)
    B.infllmv2_sparse_attn_decode_topk(q, k, v, seqlens, max(lens), None, None, out2, lse2,
                                       plan.ws, p)
    torch.cuda.synchronize()
    _same(out2, plan.out, "decode out")
    _same(lse2, plan.lse, "decode lse")
    T, n_ctx = 7, 5000
    kc = torch.randn((2, n_ctx, d), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((2, n_ctx, d), generator=g, device="cuda").to(torch.bfloat16)
    kd = torch.randn((2, T, d), generator=g, device="cuda").to(torch.bfloat16)
    vd = torch.randn((2, T, d), generator=g, device="cuda").to(torch.bfloat16)
    qt = torch.randn((T, 32, d), generator=g, device="cuda").to(torch.bfloat16)
    mask = torch.tensor([(1 << (i + 1)) - 1 for i in range(T)], dtype=torch.int64,
                        device="cuda")
    tp = PL.TreePlan(T, n_ctx, 32, 2, d, torch.bfloat16, p)
    assert tp.dense
    out3, lse3 = torch.empty_like(tp.out), torch.empty_like(tp.lse)
    B.infllmv2_tree_verify(qt, kc, vc, n_ctx, kd, vd, mask, None, tp.out, tp.lse, tp.ws, p)
    B.infllmv2_tree_verify_topk(qt, kc, vc, n_ctx, kd, vd, mask, None, None, out3, lse3,
                                tp.ws, p)
    torch.cuda.synchronize()
    _same(out3, tp.out, "tree out")
    _same(lse3, tp.lse, "tree lse")
