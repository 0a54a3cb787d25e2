"""Throughput of the InfLLM v2 block-sparse attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N]

Default workload (2): the final 8192-query chunk of a 131072-token context
(bf16, 32 query heads / 2 KV heads, d=128, 64-token blocks, 32/16 kernels,
top-64, dense_len 8192) -- the long-context prefill the pages quote 128K
throughput for.  One step = compress the windows this chunk completes ->
block scores -> top-k -> sparse attention, i.e. every stage of the path.
Other workloads (for reports): 1 = 32K decode, 3 = 128K tree verification
with 16 drafts, 4 = ragged decode of 8 sequences up to 128K, 5 = 128K decode,
6 = 128K decode of a batch of 32 sequences (copies of workload 5's sequence),
7 = the whole 131072-token prompt prefilled in 16 chunks of 8192 (each chunk:
its new windows -> scores -> top-k -> attention over the keys so far), 8 = the
final chunk with 128-token blocks and top-6, 9 = the backward of workload 2's
attention (dQ, dK, dV through the kept blocks, selections and forward
outputs resident), one training step's attention gradient for the chunk,
10 = the backward of workload 7's whole 131072-token prompt (16 chunk
backwards adding into one dK/dV).

Prints one JSON line.  Timing: each of the K timed iterations flushes the
caches (a read-modify-write of 1 GiB, 4x the Infinity Cache) and then replays
the whole step, captured once as a HIP graph, between two HIP events;
ms_per_step is the median, with p10 / p90 / mean beside it.  The dominant
call (the attention call; for decode and tree verification the attention
call that also makes the top-k selection) is timed the same way on its own
after the step's earlier stages, and its mean duration gives the roofline fraction
(algorithmic FLOP or bytes per launch over that time).  Other workloads of
the metric (--also: ragged decode, 128K decode at batch 1, tree
verification) are timed the same way and reported in the same line.  The
CPU oracle is timed on a bounded sample of the headline workload, its rows
spread over the host cores (worker processes forked before the GPU is used).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "InfLLMv2 attn tokens/s at 128K (decode, prefill); % of HBM/MFMA roofline"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E peak
PROFILE_DIR = os.path.join(ROOT, "profiles")


def _n_windows(n, ks, s):
    return 0 if n < ks else (n - ks) // s + 1


def _visible_selected_keys(pos, p, n_sel_blocks):
    """Keys attended by a sparse query at `pos` that keeps n_sel_blocks blocks,
    its own (partial) block among them: full blocks + the own block's prefix."""
    B = p.block_size
    return (n_sel_blocks - 1) * B + (pos % B) + 1


def _kept_keys(pos, p):
    """Keys attended by the query at `pos`: every key up to it while its
    eligible blocks fit in topk, else topk - 1 full blocks + its own prefix."""
    if pos // p.block_size + 1 <= p.topk:
        return pos + 1
    return _visible_selected_keys(pos, p, p.topk)


def _kernel_sha(path):
    """Hash of a kernel source and every header of the library (the kernels
    include them), so a counter figure goes stale when any of them changes."""
    csrc = os.path.dirname(path)
    h = hashlib.sha256()
    for f in [path] + sorted(os.path.join(csrc, n) for n in os.listdir(csrc) if n.endswith(".h")):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(kernel_name, src_file, workload):
    """HBM bytes per call from committed rocprofv3 PMC summaries of this
    workload, if they were taken on the current kernel source (else None)."""
    path = os.path.join(PROFILE_DIR, f"traffic_{kernel_name}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != _kernel_sha(src_file):
        return None
    return t.get("hbm_bytes_per_launch")


def build_case(wid, seed=0, score_mode=None):
    """The seeded inputs of a workload, on the host: (case, name, rep).

    rep > 1 (workload 6): decode at 128K for `rep` copies of one
    131072-token sequence, each in its own HBM (same values, separate
    addresses, so every sequence's K/V is really read)."""
    from block_sparse_long_infllmv2_amd.workloads import CONFIG_NAMES, Params, config
    rep = 1
    if wid == 7:
        # the whole 128K prompt: queries at every position, 16 chunks of 8192
        case, name = config(2, seed=seed, n_q=131072), "sparse_prefill_bf16_128k_whole_16x8192"
    elif wid == 8:
        # the final chunk with the other variant the pages describe:
        # 128-token blocks, top-6
        case = config(2, seed=seed, params=Params(block_size=128, topk=6))
        name = "sparse_prefill_bf16_128k_chunk8192_block128_top6"
    elif wid == 9:
        case, name = config(2, seed=seed), "sparse_prefill_backward_bf16_128k_chunk8192"
    elif wid == 10:
        case = config(2, seed=seed, n_q=131072)
        name = "sparse_prefill_backward_bf16_128k_whole_16x8192"
    elif wid == 5:
        case, name = config(1, seed=seed, seqlen=131072, n_planted=64), "decode_bf16_128k"
    elif wid == 6:
        case = config(1, seed=seed, seqlen=131072, n_planted=64)
        name, rep = "decode_bf16_128k_batch32", 32
    elif wid in CONFIG_NAMES and wid != 0:
        case, name = config(wid, seed=seed), CONFIG_NAMES[wid]
    else:
        raise SystemExit(f"workload {wid} is a parity case, not a bench workload")
    if score_mode is not None:
        case.params = case.params.replace(score_mode=score_mode)
    return case, name, rep


# ----------------------------------------------------------------------------
class Workload:
    """Builds inputs on the GPU and exposes step() plus algorithmic work."""

    def __init__(self, wid, torch, seed=0, score_mode=None, case=None):
        from block_sparse_long_infllmv2_amd import binding as B
        from block_sparse_long_infllmv2_amd import pipeline as PL
        self.torch, self.B, self.PL = torch, B, PL
        self.wid = wid
        dev = torch.device("cuda:0")
        self.dev = dev
        if case is None:
            case = build_case(wid, seed, score_mode)
        self.case, self.name, self.rep = case
        c = self.case
        p = c.params
        self.p = p
        bf = torch.bfloat16
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev, bf)
        if wid == 7:
            self.q, self.k, self.v = up(c.q), up(c.k), up(c.v)
            h_kv, n_k, d = c.k.shape
            # each chunk's selection overlaps the previous chunk's attention
            self.cp = PL.ChunkedPrefill(n_k, 8192, c.q.shape[1], h_kv, d, bf, p, device=dev,
                                        overlap=True)
            self.plan = self.cp.plans[-1]
            nc = _n_windows(n_k, p.kernel_size, p.kernel_stride)
            self.ck = torch.zeros((h_kv, nc, d), dtype=bf, device=dev)
            torch.cuda.synchronize()
            self.tokens = n_k
            self.kind = "prefill_whole"
        elif wid == 10:
            from block_sparse_long_infllmv2_amd.workloads import make_upstream_grad
            self.q, self.k, self.v = up(c.q), up(c.k), up(c.v)
            h_kv, n_k, d = c.k.shape
            self.cp = PL.ChunkedPrefill(n_k, 8192, c.q.shape[1], h_kv, d, bf, p, device=dev,
                                        keep_selections=True)
            self.plan = self.cp.plans[-1]
            nc = _n_windows(n_k, p.kernel_size, p.kernel_stride)
            self.ck = torch.zeros((h_kv, nc, d), dtype=bf, device=dev)
            # the whole prompt's forward (selections, outputs, log-sum-exp)
            self.cp.run(self.q, self.k, self.v, self.ck)
            self.d_out = up(make_upstream_grad(seed, n_k, c.q.shape[1], d, "bf16"))
            self.dq = torch.empty_like(self.q)
            self.dk = torch.zeros((h_kv, n_k, d), dtype=torch.float32, device=dev)
            self.dv = torch.zeros_like(self.dk)
            torch.cuda.synchronize()
            self.tokens = n_k
            self.kind = "prefill_bwd_whole"
        elif wid == 9:
            from block_sparse_long_infllmv2_amd.workloads import make_upstream_grad
            self.q, self.k, self.v = up(c.q), up(c.k), up(c.v)
            h_kv, n_k, d = c.k.shape
            self.plan = PL.PrefillPlan(c.n_q, n_k, c.q.shape[1], h_kv, d, bf, p, device=dev)
            nc = _n_windows(n_k, p.kernel_size, p.kernel_stride)
            self.ck = torch.zeros((h_kv, nc, d), dtype=bf, device=dev)
            # the forward of the chunk (selections, output, log-sum-exp) is
            # resident, as after a training forward pass
            self.plan.run(self.q, self.k, self.v, self.ck, m_begin=0)
            self.d_out = up(make_upstream_grad(seed, c.n_q, c.q.shape[1], d, "bf16"))
            self.dq = torch.empty_like(self.q)
            self.dk = torch.zeros((h_kv, n_k, d), dtype=torch.float32, device=dev)
            self.dv = torch.zeros_like(self.dk)
            torch.cuda.synchronize()
            self.tokens = c.n_q
            self.kind = "prefill_bwd"
        elif wid in (2, 8):
            self.q, self.k, self.v = up(c.q), up(c.k), up(c.v)
            h_kv, n_k, d = c.k.shape
            self.plan = PL.PrefillPlan(c.n_q, n_k, c.q.shape[1], h_kv, d, bf, p, device=dev)
            nc = _n_windows(n_k, p.kernel_size, p.kernel_stride)
            self.ck = torch.zeros((h_kv, nc, d), dtype=bf, device=dev)
            # compressed keys of the context before this chunk already exist
            self.plan.compress(self.k, self.ck, m_begin=0)
            torch.cuda.synchronize()
            self.tokens = c.n_q
            self.kind = "prefill"
        elif wid in (1, 4, 5, 6):
            lens = np.tile(np.asarray(c.seqlens), self.rep)
            bsz = len(lens)
            n0 = len(c.seqlens)
            h_kv, _, d = c.k[0].shape
            cap = int(((lens.max() + 63) // 64) * 64)
            self.k = torch.zeros((bsz, h_kv, cap, d), dtype=bf, device=dev)
            self.v = torch.zeros_like(self.k)
            for i, L in enumerate(lens):
                self.k[i, :, :L] = up(c.k[i % n0])
                self.v[i, :, :L] = up(c.v[i % n0])
            self.q = up(np.tile(c.q, (self.rep, 1, 1)))
            self.seqlens = torch.from_numpy(lens.astype(np.int32)).to(dev)
            nc = _n_windows(cap, p.kernel_size, p.kernel_stride)
            self.ck = torch.zeros((bsz, h_kv, nc, d), dtype=bf, device=dev)
            B.infllmv2_compress_keys(self.k, self.seqlens, 0, nc, self.ck, p)
            self.plan = PL.DecodePlan(bsz, int(lens.max()), c.q.shape[1], h_kv, d, bf, p,
                                      device=dev)
            torch.cuda.synchronize()
            self.tokens = bsz
            self.kind = "decode"
        elif wid == 3:
            self.q, self.k, self.v = up(c.q), up(c.k), up(c.v)
            self.kd, self.vd = up(c.k_draft), up(c.v_draft)
            self.mask = torch.from_numpy(c.mask.astype(np.int64)).to(dev)
            h_kv, n_ctx, d = c.k.shape
            nc = _n_windows(n_ctx, p.kernel_size, p.kernel_stride)
            self.ck = torch.zeros((h_kv, nc, d), dtype=bf, device=dev)
            B.infllmv2_compress_keys(self.k.unsqueeze(0),
                                     torch.tensor([n_ctx], dtype=torch.int32, device=dev), 0,
                                     nc, self.ck.unsqueeze(0), p)
            self.plan = PL.TreePlan(c.q.shape[0], n_ctx, c.q.shape[1], h_kv, d, bf, p,
                                    device=dev)
            torch.cuda.synchronize()
            self.tokens = c.q.shape[0]
            self.kind = "tree"

    # one step, with optional per-stage event recording; skip_dominant leaves
    # out the attention call (to time that call inside real steps by difference)
    def step(self, ev=None, skip_dominant=False):
        def mark(name):
            if ev is not None:
                e = self.torch.cuda.Event(enable_timing=True)
                e.record()
                ev.append((name, e))
        pl = self.plan
        if self.kind == "prefill_whole" and ev is None:
            # the timed step: the plan's own schedule (selections on a second
            # stream, overlapping the previous chunk's attention)
            self.cp.run(self.q, self.k, self.v, self.ck, skip_attention=skip_dominant)
        elif self.kind == "prefill_whole":
            # stage times: the same calls one after another on one stream
            mark("start")
            cp = self.cp
            for (q0, q1, _, m0, m1), pc in zip(cp.sched, cp.plans):
                qc = self.q[q0:q1]
                if m1 > m0:
                    pc.compress(self.k, self.ck, m_begin=m0)
                mark("compress_keys")
                if not pc.dense:
                    pc.score(qc, self.ck)
                    mark("block_scores")
                    pc.topk()
                    mark("select_topk")
                if not skip_dominant:
                    pc.attend(qc, self.k, self.v)
                mark("sparse_attn_prefill")
        elif self.kind in ("prefill_bwd", "prefill_bwd_whole"):
            mark("start")
            if not skip_dominant:
                self.backward()
            mark("sparse_attn_prefill_backward")
        elif self.kind == "prefill":
            mark("start")
            pl.compress(self.k, self.ck)
            mark("compress_keys")
            pl.score(self.q, self.ck)
            mark("block_scores")
            pl.topk()
            mark("select_topk")
            if not skip_dominant:
                pl.attend(self.q, self.k, self.v)
            mark("sparse_attn_prefill")
        elif self.kind == "decode":
            mark("start")
            pl.select(self.q, self.ck, self.seqlens)
            mark("block_scores")
            if not skip_dominant:
                pl.attend(self.q, self.k, self.v, self.seqlens)
            mark("sparse_attn_decode_topk")
        else:
            mark("start")
            pl.select(self.q, self.ck)
            mark("block_scores")
            if not skip_dominant:
                pl.attend(self.q, self.k, self.v, self.kd, self.vd, self.mask)
            mark("tree_verify_topk")

    def backward(self):
        if self.kind == "prefill_bwd_whole":
            self.cp.backward(self.q, self.k, self.v, self.d_out, self.dq, self.dk, self.dv)
        else:
            self.plan.backward(self.q, self.k, self.v, self.d_out, self.dq, self.dk, self.dv)

    # the dominant call alone (the attention call of the step)
    def dominant_call(self):
        pl = self.plan
        if self.kind == "prefill_whole":
            raise NotImplementedError("timed by graph difference only")
        if self.kind in ("prefill_bwd", "prefill_bwd_whole"):
            self.backward()
            return
        if self.kind == "prefill":
            pl.attend(self.q, self.k, self.v)
        elif self.kind == "decode":
            pl.attend(self.q, self.k, self.v, self.seqlens)
        else:
            pl.attend(self.q, self.k, self.v, self.kd, self.vd, self.mask)

    # ---- algorithmic work (what the method must touch / compute) ----------
    def work(self):
        c, p = self.case, self.p
        if self.kind == "prefill_whole":
            h_kv, n_k, d = c.k.shape
            h_q = c.q.shape[1]
            keys = sum(_kept_keys(x, p) for x in range(n_k))
            nvis = sum(_n_windows(x + 1, p.kernel_size, p.kernel_stride) for x in range(n_k))
            return {"dominant": "sparse_attn_prefill", "bound": "mfma",
                    "flop": 4.0 * d * h_q * keys, "score_flop": 2.0 * d * h_kv * float(nvis),
                    "src": "attn_bf16.hip", "launches": len(self.cp.plans)}
        if self.kind == "prefill_bwd_whole":
            h_kv, n_k, d = c.k.shape
            h_q = c.q.shape[1]
            keys = sum(_kept_keys(x, p) for x in range(n_k))
            return {"dominant": "sparse_attn_prefill_backward", "bound": "mfma",
                    "flop": 10.0 * d * h_q * keys, "score_flop": 0.0,
                    "src": "attn_bwd.hip", "launches": len(self.cp.plans),
                    "launches_in_call": 7}
        if self.kind == "prefill_bwd":
            # five products over the kept keys (S, dP, dV, dK, dQ), 2 d flop
            # per (row, head, key) each: 2.5 times the forward's two
            h_kv, n_k, d = c.k.shape
            h_q = c.q.shape[1]
            pos = np.arange(n_k - c.n_q, n_k)
            keys = sum(_visible_selected_keys(int(x), p, p.topk) for x in pos)
            return {"dominant": "sparse_attn_prefill_backward", "bound": "mfma",
                    "flop": 10.0 * d * h_q * keys, "score_flop": 0.0,
                    "src": "attn_bwd.hip", "launches_in_call": 7}
        if self.kind == "prefill":
            h_kv, n_k, d = c.k.shape
            h_q = c.q.shape[1]
            pos = np.arange(n_k - c.n_q, n_k)
            keys = sum(_visible_selected_keys(int(x), p, p.topk) for x in pos)
            attn_flop = 4.0 * d * h_q * keys
            nvis = np.array([_n_windows(int(x) + 1, p.kernel_size, p.kernel_stride)
                             for x in pos])
            score_flop = 2.0 * d * h_kv * float(nvis.sum())
            return {"dominant": "sparse_attn_prefill", "bound": "mfma",
                    "flop": attn_flop, "score_flop": score_flop,
                    "src": "attn_bf16.hip"}
        d = c.q.shape[2]
        h_q = c.q.shape[1]
        if self.kind == "decode":
            # the selecting attention call's own bytes: the block scores of
            # each sparse row's eligible blocks and its selection written, K
            # and V of the kept keys, Q and O (the compressed keys are read by
            # the scoring stage, not here)
            total = 0.0
            for L in np.tile(np.asarray(c.seqlens), self.rep):
                L = int(L)
                h_kv = c.k[0].shape[0]
                if L < p.dense_len:
                    kv = h_kv * L * d * 2 * 2
                else:
                    kv = h_kv * _visible_selected_keys(L - 1, p, p.topk) * d * 2 * 2
                    kv += h_kv * ((L - 1) // p.block_size + 1 + p.topk) * 4
                total += kv + h_q * d * 2 * 2
            return {"dominant": "sparse_attn_decode_topk", "bound": "hbm", "bytes": total,
                    "src": "attn_bf16.hip"}
        # tree: union of kept blocks per KV head + drafts + Q/O + masks
        h_kv, n_ctx, _ = c.k.shape
        sel = self.plan.block_idx.cpu().numpy()
        union = sum(len(np.unique(sel[:, g][sel[:, g] >= 0])) for g in range(h_kv))
        T = c.q.shape[0]
        total = (union * p.block_size * d * 2 * 2 + T * h_q * d * 2 * 2 +
                 2 * h_kv * T * d * 2 + T * 8)
        if not self.plan.dense:
            # block scores read and selection written by the selecting call
            total += T * h_kv * ((n_ctx - 1) // p.block_size + 1 + p.topk) * 4
        return {"dominant": "tree_verify_topk", "bound": "hbm", "bytes": float(total),
                "union_blocks": int(union), "src": "attn_bf16.hip"}


# ---- CPU baseline: the oracle as it stands, over the host's cores ----------
# Worker processes are forked before the GPU is touched; they inherit the
# host inputs through this module-level dict and compute oracle rows only.
_CPU = {}


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)            # one BLAS thread per worker process


def _cpu_row(i):
    import oracle as O
    c, p, kind = _CPU["case"], _CPU["case"].params, _CPU["kind"]
    if kind == "prefill":
        O.prefill(c.q, c.k, c.v, p, "bf16", rows=[i], ck=_CPU["ck"])
    elif kind == "prefill_whole":
        nw = O.num_windows(i + 1, p.kernel_size, p.kernel_stride)
        O.prefill(c.q[i:i + 1], c.k[:, :i + 1], c.v[:, :i + 1], p, "bf16", rows=[0],
                  ck=_CPU["ck"][:, :nw])
    elif kind == "decode":
        O.decode(c.q[i:i + 1], [c.k[i]], [c.v[i]], [c.seqlens[i]], p, "bf16")
    elif kind == "tree":
        O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, c.mask, p, "bf16",
                      ck=_CPU["ck"], drafts=[i])
    return i


def _cpu_bwd_row(arg):
    import oracle as O
    i, sel_row = arg
    c = _CPU["case"]
    sel_rows = [None] * c.q.shape[0]
    sel_rows[i] = sel_row
    O.prefill_backward(c.q, c.k, c.v, sel_rows, c.params, _CPU["d_out"], rows=[i])
    return i


def _one_thread():
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=1)


def cpu_workers():
    """Worker count: the host cores this process may run on, at most 16 (a
    one-GPU share of the host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


class CpuBaseline:
    """Times the CPU oracle on a bounded sample of a workload, rows spread
    over a pool of forked worker processes (one BLAS thread each)."""

    def __init__(self, case, kind, workers):
        import multiprocessing

        import copy

        import oracle as O
        # the oracle works in float64: upcast the inputs once here (exact),
        # not in every row's call
        case = copy.copy(case)
        for name in ("q", "k", "v", "k_draft", "v_draft"):
            x = getattr(case, name, None)
            if isinstance(x, list):
                setattr(case, name, [np.asarray(a, np.float64) for a in x])
            elif isinstance(x, np.ndarray):
                setattr(case, name, np.asarray(x, np.float64))
        _CPU.clear()
        _CPU.update(case=case, kind=kind)
        self.case, self.kind, self.workers = case, kind, workers
        # compressed keys of the whole context, once, in this process (timed
        # and counted with the rows); the workers inherit them
        self.ck_s = 0.0
        if kind in ("prefill", "prefill_whole", "tree"):
            t0 = time.perf_counter()
            with_one_thread = _one_thread()
            with with_one_thread:
                _CPU["ck"] = O.compress_keys(case.k, case.params, "bf16")
            self.ck_s = time.perf_counter() - t0
        self.pool = multiprocessing.get_context("fork").Pool(workers, _cpu_worker_init)

    def close(self):
        self.pool.terminate()
        self.pool.join()

    def _run(self, fn, items, budget_s, t0):
        done = 0
        while time.perf_counter() - t0 < budget_s and done < len(items):
            batch = items[done:done + self.workers]
            self.pool.map(fn, batch, chunksize=1)
            done += len(batch)
        return done, time.perf_counter() - t0

    def measure(self, budget_s, wl=None):
        import oracle as O
        c, p, kind, W = self.case, self.case.params, self.kind, self.workers
        tail = f"float64 numpy oracle, {W} worker processes x 1 thread"
        t0 = time.perf_counter() - self.ck_s
        if kind in ("prefill", "prefill_whole"):
            n = c.q.shape[0]
            step = max(1, n // 4096)
            rows = list(range(0, n, step))
            done, dt = self._run(_cpu_row, rows, budget_s, t0)
            what = "prompt positions" if kind == "prefill_whole" else "chunk queries"
            return {"value": done / dt, "unit": "tokens/s", "cores": W, "kind": "oracle",
                    "sample": f"{done} of {n} {what} (every {step}th) incl. compressing "
                              f"all {_CPU['ck'].shape[1]} windows once; {tail}"}
        if kind in ("prefill_bwd", "prefill_bwd_whole"):
            sel = (wl.cp.idx_buf.view(c.q.shape[0], c.k.shape[0], p.topk)
                   if kind == "prefill_bwd_whole" else wl.plan.block_idx).cpu().numpy()
            dense_row = [False] * c.q.shape[0]
            if kind == "prefill_bwd_whole":
                for (q0, q1, _, _, _), pc in zip(wl.cp.sched, wl.cp.plans):
                    for r in range(q0, q1):
                        dense_row[r] = pc.dense
            n = c.q.shape[0]
            step = max(1, n // 1024)
            items = [(i, None if dense_row[i] else [s_[s_ >= 0] for s_ in sel[i]])
                     for i in range(0, n, step)]
            t0 = time.perf_counter()
            done, dt = self._run(_cpu_bwd_row, items, budget_s, t0)
            return {"value": done / dt, "unit": "tokens/s", "cores": W, "kind": "oracle",
                    "sample": f"{done} of {n} queries (every {step}th): dq of the row and "
                              f"its dk/dv contributions; {tail}"}
        if kind == "tree":
            T = c.q.shape[0]
            done, dt = self._run(_cpu_row, list(range(T)), budget_s, t0)
            return {"value": done / dt, "unit": "tokens/s", "cores": W, "kind": "oracle",
                    "sample": f"{done} of {T} drafts incl. compressing the context; {tail}"}
        n = len(c.seqlens)
        done, dt = self._run(_cpu_row, list(range(n)), budget_s, t0)
        return {"value": done / dt, "unit": "tokens/s", "cores": W, "kind": "oracle",
                "sample": f"{done} of {n} sequences, each from its compressed keys; {tail}"}


def _keep_busy(fn, seconds, torch):
    """Call fn (one step or one graph replay) at least once and until
    `seconds` of wall time have passed; synchronises at the end."""
    t0 = time.perf_counter()
    while True:
        fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break


def _capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _stats(xs):
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean()), "n": int(a.size)}


class Flush:
    """Evicts the caches between timed iterations, on the current stream,
    outside the timed brackets, with a 1 GiB buffer (4x the 256 MB Infinity
    Cache, far beyond the L2s).
      write_read (default): write the buffer, then read it back (a sum), so
        the caches hold clean lines of unrelated data, as after the weight
        reads of a model's other layers;
      rmw: one read-modify-write pass, which leaves the caches full of dirty
        lines that the timed step must write back as it evicts them;
      none: no flush (warm caches)."""
    BYTES = 1 << 30

    def __init__(self, torch, mode="write_read"):
        self.mode = mode
        self.buf = torch.zeros(self.BYTES // 4, dtype=torch.float32, device="cuda:0")
        self.acc = torch.zeros((), dtype=torch.float32, device="cuda:0")
        self.torch = torch

    def __call__(self):
        if self.mode == "none":
            return
        if self.mode == "rmw":
            self.buf.add_(1.0)
            return
        self.buf.fill_(1.0)
        self.torch.sum(self.buf, dim=0, out=self.acc)


def _timed_loop(torch, iters, flush, before, timed):
    """iters x (flush; before(); event; timed(); event): per-iteration
    milliseconds of timed() on the current stream, caches cold each time.
    Returns (list of ms, wall seconds of the whole loop incl. flushes)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        flush()
        if before is not None:
            before()
        e0.record()
        timed()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [e0.elapsed_time(e1) for e0, e1 in evs], wall


def time_workload(wl, torch, steps, warmup, warm_seconds, flush):
    """Cold-cache timing of one workload.

    * step: the whole step (every stage) captured as one HIP graph; each of
      `steps` iterations flushes the caches, then replays the graph between
      two HIP events.  ms_per_step = median; p10 / p90 / mean reported.
    * dominant call: the step's stages before it replayed untimed after the
      flush (so its inputs are as cold as in a real step: the selections
      were just written, K/V were not touched), then the call itself,
      launched eagerly between two events.  For the whole-prompt workload, whose attention
      calls interleave with the other stages, it is the median step minus
      the median step without those calls.
    * warm: the step graph replayed `steps` times back to back, no flush.
    * stages: eager steps with events between the library calls, flushed."""
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    _keep_busy(wl.step, warm_seconds, torch)

    # per-stage times of eager steps (flush before each step)
    stage_ev = []
    for _ in range(steps):
        flush()
        ev = []
        wl.step(ev)
        stage_ev.append(ev)
    torch.cuda.synchronize()
    stages = {}
    for ev in stage_ev:
        per = {}
        for (n0, e0), (n1, e1) in zip(ev[:-1], ev[1:]):
            per[n1] = per.get(n1, 0.0) + e0.elapsed_time(e1)
        for k, v in per.items():
            stages.setdefault(k, []).append(v)
    stage_ms = {k: float(np.median(v)) for k, v in stages.items()}

    g_step = _capture(torch, wl.step)
    separable = wl.kind != "prefill_whole"
    has_pre = wl.kind not in ("prefill_bwd", "prefill_bwd_whole")
    g_pre = _capture(torch, lambda: wl.step(skip_dominant=True)) if has_pre else None
    torch.cuda.synchronize()
    # capturing left the GPU idle: untimed flushed replays until it is warm again
    _keep_busy(lambda: (flush(), g_step.replay()), warm_seconds, torch)

    step_ms, wall = _timed_loop(torch, steps, flush, None, g_step.replay)
    if separable:
        # the call itself is launched eagerly (queued behind the flush, so no
        # host gap): events then bracket its kernels without a graph launch
        dom_ms, _ = _timed_loop(torch, steps, flush,
                                g_pre.replay if g_pre is not None else None, wl.dominant_call)
        dom = _stats(dom_ms)
    else:
        pre_ms, _ = _timed_loop(torch, steps, flush, None, g_pre.replay)
        d = float(np.median(step_ms) - np.median(pre_ms))
        dom = {"median": d, "p10": None, "p90": None, "mean": d, "n": steps,
               "method": "median step - median step without the attention calls"}
    # warm: back-to-back replays of the step graph, no flush
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        g_step.replay()
    e1.record()
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / steps
    return {"step": _stats(step_ms), "dominant": dom, "warm_ms_per_step": warm_ms,
            "stages_ms": stage_ms, "timed_loop_wall_s": wall}


def _roofline(wl, w, dom):
    """Roofline object for the dominant call: algorithmic work per launch
    over its mean cold-cache duration."""
    src = os.path.join(ROOT, "block_sparse_long_infllmv2_amd", "csrc", w["src"])
    t_ms = dom["mean"]
    if w["bound"] == "mfma":
        achieved = w["flop"] / (t_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": _traffic(w["dominant"], src, wl.name)
                if w.get("launches", 1) == 1 else None,
                "kernel": w["dominant"],
                ("algorithmic_gflop_per_step" if w.get("launches", 1) > 1
                 else "algorithmic_gflop_per_launch"): round(w["flop"] / 1e9, 2)}
        if w.get("launches", 1) > 1:
            roof["launches_per_step"] = w["launches"]
        if "launches_in_call" in w:
            # a call of several kernels: no single-launch counter figure
            roof["traffic"] = None
            roof["kernels_in_call"] = w["launches_in_call"]
            if "algorithmic_gflop_per_launch" in roof:
                roof["algorithmic_gflop_per_call"] = roof.pop("algorithmic_gflop_per_launch")
    else:
        achieved = w["bytes"] / (t_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": _traffic(w["dominant"], src, wl.name), "kernel": w["dominant"],
                "algorithmic_mb_per_launch": round(w["bytes"] / 1e6, 3)}
        if "union_blocks" in w:
            roof["union_blocks"] = w["union_blocks"]
    roof["kernel_ms"] = round(t_ms, 4)
    roof["kernel_ms_median"] = round(dom["median"], 4)
    if dom.get("p10") is not None:
        roof["kernel_ms_p10"] = round(dom["p10"], 4)
        roof["kernel_ms_p90"] = round(dom["p90"], 4)
    roof["timing"] = "HIP events on the launch stream, caches flushed before each launch"
    return roof


def _config(wl):
    cfg = {"workload": wl.name}
    c = wl.case
    if wl.kind == "prefill_whole":
        cfg.update({"context": int(c.k.shape[1]), "chunk_queries": 8192,
                    "chunks": len(wl.cp.plans)})
    elif wl.kind == "prefill_bwd_whole":
        cfg.update({"context": int(c.k.shape[1]), "chunk_queries": 8192,
                    "chunks": len(wl.cp.plans), "pass": "backward (dq, dk, dv)"})
    elif wl.kind in ("prefill", "prefill_bwd"):
        cfg.update({"context": int(c.k.shape[1]), "chunk_queries": int(c.n_q)})
        if wl.kind == "prefill_bwd":
            cfg["pass"] = "backward (dq, dk, dv)"
    elif wl.kind == "decode":
        lens = [int(x) for x in np.tile(np.asarray(c.seqlens), wl.rep)]
        cfg.update({"batch": len(lens), "seqlens": lens})
    else:
        cfg.update({"context": int(c.k.shape[1]), "drafts": int(c.q.shape[0])})
    cfg.update({"h_q": int(c.q.shape[1]), "h_kv": 2, "head_dim": int(c.q.shape[2]),
                "block_size": wl.p.block_size, "kernel_size": wl.p.kernel_size,
                "kernel_stride": wl.p.kernel_stride, "topk": wl.p.topk,
                "init_blocks": wl.p.init_blocks, "local_blocks": wl.p.local_blocks,
                "dense_len": wl.p.dense_len})
    return cfg


def _record(wl, t):
    """Throughput and roofline of one timed workload."""
    w = wl.work()
    st = t["step"]
    ms = st["median"]
    rec = {"value": round(wl.tokens / (ms * 1e-3), 2), "unit": "tokens/s",
           "ms_per_step": round(ms, 4), "ms_per_step_p10": round(st["p10"], 4),
           "ms_per_step_p90": round(st["p90"], 4), "ms_per_step_mean": round(st["mean"], 4),
           "warm_ms_per_step": round(t["warm_ms_per_step"], 4),
           "config": _config(wl), "roofline": _roofline(wl, w, t["dominant"]),
           "stages_ms": {k: round(v, 4) for k, v in t["stages_ms"].items()}}
    if w["bound"] == "mfma":
        rec["scoring_gflop"] = round(w["score_flop"] / 1e9, 2)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100,
                    help="timed iterations (each: cache flush, then one step)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--also", default="4,5,3",
                    help="comma-separated workloads timed in the same run and reported "
                         "in the same line (4 = ragged decode, 5 = 128K decode at batch 1, "
                         "3 = tree verification); empty for none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--score-mode", type=int, default=None, choices=[0, 1],
                    help="group score reading: 0 summed query (default), 1 sum of "
                         "per-head softmaxes over the visible windows")
    ap.add_argument("--warm-seconds", type=float, default=0.3,
                    help="untimed work after the warm-up steps and after graph capture, "
                         "so that timing starts at steady clocks")
    ap.add_argument("--flush", default="write_read", choices=["write_read", "rmw", "none"],
                    help="cache flush before each timed iteration (see Flush)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (3 times): the reference "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the path is "
              "built and measured on one GPU; a multi-GPU run is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": a.numel() * 4,
                          "bytes_written": b.numel() * 4, "launches": 3}))
        return

    # host inputs first; the CPU oracle's worker processes are forked now,
    # before this process touches the GPU
    case = build_case(args.workload, score_mode=args.score_mode)
    kind_of = {7: "prefill_whole", 9: "prefill_bwd", 10: "prefill_bwd_whole", 3: "tree",
               1: "decode", 4: "decode", 5: "decode", 6: "decode"}
    kind = kind_of.get(args.workload, "prefill")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = CpuBaseline(case[0], kind, cpu_workers())
    print(f"[bench] workload {case[1]}: host inputs ready", file=sys.stderr, flush=True)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    flush = Flush(torch, args.flush)
    wl = Workload(args.workload, torch, case=case)
    print(f"[bench] workload {wl.name}: setup done", file=sys.stderr, flush=True)
    t = time_workload(wl, torch, args.steps, args.warmup, args.warm_seconds, flush)
    rec = _record(wl, t)
    print(f"[bench] {wl.name}: median step {rec['ms_per_step']} ms "
          f"(p10 {rec['ms_per_step_p10']}, p90 {rec['ms_per_step_p90']}), "
          f"roofline {rec['roofline']['frac']}", file=sys.stderr, flush=True)

    out = {"metric": METRIC, "value": rec["value"], "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": rec["ms_per_step"],
           "ms_per_step_p10": rec["ms_per_step_p10"], "ms_per_step_p90": rec["ms_per_step_p90"],
           "ms_per_step_mean": rec["ms_per_step_mean"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": rec["config"], "roofline": rec["roofline"],
           "timing": f"per step: 1 GiB cache flush ({args.flush}), then the step's HIP graph "
                     "between HIP events; median over the timed steps",
           "timed_loop_wall_s": round(t["timed_loop_wall_s"], 4),
           "warm_ms_per_step": rec["warm_ms_per_step"], "launch": "hip_graph",
           "score_mode": wl.p.score_mode, "stages_ms": rec["stages_ms"]}
    if "scoring_gflop" in rec:
        out["scoring_gflop"] = rec["scoring_gflop"]

    # the other workloads of the metric, timed the same way in this run
    names = {4: "decode", 5: "decode_batch1_128k", 3: "tree", 1: "decode_batch1_32k",
             6: "decode_batch32_128k", 8: "prefill_block128_top6", 2: "prefill"}
    also = [int(x) for x in args.also.split(",") if x.strip()]
    keep = wl
    for wid in also:
        if wid == args.workload:
            continue
        w2 = Workload(wid, torch)
        t2 = time_workload(w2, torch, args.steps, args.warmup, args.warm_seconds, flush)
        r2 = _record(w2, t2)
        out[names.get(wid, f"workload_{wid}")] = r2
        print(f"[bench] {w2.name}: median step {r2['ms_per_step']} ms, roofline "
              f"{r2['roofline']['frac']}", file=sys.stderr, flush=True)
        del w2
        torch.cuda.empty_cache()

    if cpu is not None:
        print(f"[bench] timing the CPU oracle on a sample ({cpu.workers} workers)",
              file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu.measure(args.cpu_budget, keep)
        cpu.close()
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
