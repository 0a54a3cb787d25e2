"""HIP graph capture of whole steps (chunked prefill, ragged decode, tree
verification, prefill forward + backward).  The library only launches kernels on the caller's stream and
allocates nothing, so a step captures whole; bench.py times steps as graph
replays.  Each test captures a step, then replays it several times with the
program's own eager work in between (the same plan run eagerly on other
queries, other torch work, synchronisations) and checks every replay against
the eager result bit for bit (the kernels are deterministic; the backward's
dk and dv are sums of float32 atomics, whose order may vary, so they are
compared to 1e-5 of their largest magnitude)."""
import sys

import numpy as np
import pytest
import torch

from block_sparse_long_infllmv2_amd.workloads import Params, make_decode, make_prefill, \
    make_tree

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


def up(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).cuda()


def _nwin(n, p):
    return 0 if n < p.kernel_size else (n - p.kernel_size) // p.kernel_stride + 1


def _replay_check(run, outputs, other_run):
    """run(): one step; outputs(): tensors to compare; other_run(): the same
    plan on other inputs (eager work between replays)."""
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(4):
        other_run()                                      # eager, different inputs
        torch.cuda.synchronize()
        assert any(not torch.equal(a, b) for a, b in zip(outputs(), ref)), \
            "the eager work in between should change the outputs"
        scratch = torch.randn(1 << 16, device="cuda")
        (scratch * 2.0).sum().item()                     # unrelated eager torch work
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs(), ref):
            assert torch.equal(a, b), f"replay {i} differs from the eager step"


def test_graph_prefill_step(B, PL):
    _say("graph: prefill step")
    p = Params(topk=16, dense_len=0)
    c = make_prefill(21, n_k=9000, n_q=133, h_q=32, h_kv=2, d=128, params=p, dtype="bf16",
                     n_planted=4, alpha=1.5, beta=1.5)
    q, k, v = up(c.q), up(c.k), up(c.v)
    q2 = up(np.flip(c.q, axis=0).copy())
    h_kv, n_k, d = c.k.shape
    plan = PL.PrefillPlan(c.n_q, n_k, c.q.shape[1], h_kv, d, torch.bfloat16, p)
    ck = torch.zeros((h_kv, _nwin(n_k, p), d), dtype=torch.bfloat16, device="cuda")
    plan.compress(k, ck, m_begin=0)
    _replay_check(lambda: plan.run(q, k, v, ck),
                  lambda: [plan.out, plan.lse, plan.block_idx],
                  lambda: plan.run(q2, k, v, ck))


def test_graph_chunked_prefill_overlap(B, PL):
    """A whole prompt in 4 chunks with the overlapped schedule (two streams)
    captured as one graph: every replay equals the eager run."""
    _say("graph: chunked prefill, overlapped schedule")
    p = Params(topk=8, dense_len=1024)
    n, chunk = 2048, 512
    c = make_prefill(33, n_k=n, n_q=n, h_q=32, h_kv=2, d=128, params=p, dtype="bf16",
                     n_planted=3, alpha=1.5, beta=1.5)
    q, k, v = up(c.q), up(c.k), up(c.v)
    q2 = up(np.flip(c.q, axis=0).copy())
    cp = PL.ChunkedPrefill(n, chunk, 32, 2, 128, torch.bfloat16, p, overlap=True)
    ck = torch.zeros((2, _nwin(n, p), 128), dtype=torch.bfloat16, device="cuda")
    _replay_check(lambda: cp.run(q, k, v, ck),
                  lambda: [cp.out, cp.lse],
                  lambda: cp.run(q2, k, v, ck))


def test_graph_decode_step(B, PL):
    _say("graph: decode step")
    p = Params(dense_len=2048, topk=16)
    c = make_decode(22, [3000, 9001, 100, 6000], h_q=32, h_kv=2, d=128, params=p,
                    dtype="bf16", planted_per_token=1 / 512)
    bsz = len(c.seqlens)
    maxL = int(max(c.seqlens))
    cap = ((maxL + 63) // 64) * 64
    kc = torch.zeros((bsz, 2, cap, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for i, L in enumerate(c.seqlens):
        kc[i, :, :L] = up(c.k[i])
        vc[i, :, :L] = up(c.v[i])
    q = up(c.q)
    q2 = up(-c.q)
    seqlens = torch.from_numpy(np.asarray(c.seqlens, np.int32)).cuda()
    ck = torch.zeros((bsz, 2, _nwin(cap, p), 128), dtype=torch.bfloat16, device="cuda")
    B.infllmv2_compress_keys(kc, seqlens, 0, ck.shape[2], ck, p)
    plan = PL.DecodePlan(bsz, maxL, 32, 2, 128, torch.bfloat16, p)
    _replay_check(lambda: plan.run(q, kc, vc, ck, seqlens),
                  lambda: [plan.out, plan.lse, plan.block_idx],
                  lambda: plan.run(q2, kc, vc, ck, seqlens))


def test_graph_tree_step(B, PL):
    _say("graph: tree step")
    p = Params(topk=16, dense_len=8192)
    c = make_tree(23, n_ctx=12000, n_draft=16, h_q=32, h_kv=2, d=128, params=p,
                  dtype="bf16", max_depth=6, n_planted=8, alpha=1.5, beta=1.5)
    q, k, v = up(c.q), up(c.k), up(c.v)
    q2 = up(-c.q)
    kd, vd = up(c.k_draft), up(c.v_draft)
    mask = torch.from_numpy(c.mask.astype(np.int64)).cuda()
    h_kv, n_ctx, d = c.k.shape
    ck = torch.zeros((1, h_kv, _nwin(n_ctx, p), d), dtype=torch.bfloat16, device="cuda")
    B.infllmv2_compress_keys(k.unsqueeze(0), torch.tensor([n_ctx], dtype=torch.int32,
                                                          device="cuda"),
                             0, ck.shape[2], ck, p)
    plan = PL.TreePlan(c.q.shape[0], n_ctx, c.q.shape[1], h_kv, d, torch.bfloat16, p)
    _replay_check(lambda: plan.run(q, k, v, ck[0], kd, vd, mask),
                  lambda: [plan.out, plan.lse, plan.block_idx],
                  lambda: plan.run(q2, k, v, ck[0], kd, vd, mask))


def test_graph_forward_backward_step(B, PL):
    _say("graph: prefill forward + backward step")
    from block_sparse_long_infllmv2_amd.workloads import make_upstream_grad
    p = Params(topk=12, dense_len=0)
    c = make_prefill(24, n_k=5000, n_q=300, h_q=32, h_kv=2, d=128, params=p, dtype="bf16",
                     n_planted=4, alpha=1.5, beta=1.5)
    q, k, v = up(c.q), up(c.k), up(c.v)
    q2 = up(np.flip(c.q, axis=0).copy())
    do = up(make_upstream_grad(24, c.n_q, 32, 128, "bf16"))
    h_kv, n_k, d = c.k.shape
    plan = PL.PrefillPlan(c.n_q, n_k, c.q.shape[1], h_kv, d, torch.bfloat16, p)
    ck = torch.zeros((h_kv, _nwin(n_k, p), d), dtype=torch.bfloat16, device="cuda")
    plan.compress(k, ck, m_begin=0)
    dq = torch.empty_like(q)
    dk = torch.zeros((h_kv, n_k, d), dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)

    def step(qq):
        dk.zero_()
        dv.zero_()
        plan.run(qq, k, v, ck)
        plan.backward(qq, k, v, do, dq, dk, dv)

    step(q)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (plan.out, plan.block_idx, dq, dk, dv)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(q)
    for i in range(4):
        step(q2)                                          # eager, different queries
        torch.cuda.synchronize()
        assert not torch.equal(dq, ref[2]), "the eager work in between should change dq"
        (torch.randn(1 << 16, device="cuda") * 2.0).sum().item()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "block_idx", "dq"), (plan.out, plan.block_idx, dq),
                              ref[:3]):
            assert torch.equal(a, b), f"replay {i}: {name} differs from the eager step"
        for name, a, b in zip(("dk", "dv"), (dk, dv), ref[3:]):
            tol = 1e-5 * float(b.abs().max())
            assert float((a - b).abs().max()) <= tol, f"replay {i}: {name} differs"
