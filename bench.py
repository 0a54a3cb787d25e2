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

Prints one JSON line: tokens/s over K timed steps (the K steps captured as one
HIP graph and replayed once; --eager times individual launches), per-stage
times from HIP events recorded between the library calls of eager steps, the
dominant call's roofline fraction (its time = HIP-event time of the K-step
graph minus that of the same K steps without the call, median of 5 such pairs,
events on the graph's stream), and the CPU oracle timed on a bounded sample of the same workload.
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


# ----------------------------------------------------------------------------
class Workload:
    """Builds inputs on the GPU and exposes step() plus algorithmic work."""

    def __init__(self, wid, torch, seed=0, score_mode=None):
        from block_sparse_long_infllmv2_amd import binding as B
        from block_sparse_long_infllmv2_amd import pipeline as PL
        from block_sparse_long_infllmv2_amd.workloads import CONFIG_NAMES, Params, config
        self.torch, self.B, self.PL = torch, B, PL
        self.wid = wid
        dev = torch.device("cuda:0")
        self.dev = dev
        # batched decode at 128K: `rep` copies of one 131072-token sequence, each
        # in its own HBM (same values, separate addresses, so every sequence's
        # K/V is really read); shows the decode kernel where HBM bandwidth,
        # not launch latency, is the limit
        self.rep = 1
        if wid == 7:
            # the whole 128K prompt: queries at every position, 16 chunks of 8192
            self.case = config(2, seed=seed, n_q=131072)
            self.name = "sparse_prefill_bf16_128k_whole_16x8192"
        elif wid == 8:
            # the final chunk again with the other variant the pages describe:
            # 128-token blocks, top-6
            self.case = config(2, seed=seed, params=Params(block_size=128, topk=6))
            self.name = "sparse_prefill_bf16_128k_chunk8192_block128_top6"
        elif wid == 9:
            self.case = config(2, seed=seed)
            self.name = "sparse_prefill_backward_bf16_128k_chunk8192"
        elif wid == 10:
            self.case = config(2, seed=seed, n_q=131072)
            self.name = "sparse_prefill_backward_bf16_128k_whole_16x8192"
        elif wid == 5:
            self.case = config(1, seed=seed, seqlen=131072, n_planted=64)
            self.name = "decode_bf16_128k"
        elif wid == 6:
            self.case = config(1, seed=seed, seqlen=131072, n_planted=64)
            self.rep = 32
            self.name = "decode_bf16_128k_batch32"
        else:
            self.case = config(wid, seed=seed)
            self.name = CONFIG_NAMES[wid]
        c = self.case
        if score_mode is not None:
            c.params = c.params.replace(score_mode=score_mode)
        p = c.params
        self.p = p
        bf = torch.bfloat16
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev, bf)
        if wid == 7:
            self.q, self.k, self.v = up(c.q), up(c.k), up(c.v)
            h_kv, n_k, d = c.k.shape
            self.cp = PL.ChunkedPrefill(n_k, 8192, c.q.shape[1], h_kv, d, bf, p, device=dev)
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
        else:
            raise SystemExit(f"workload {wid} is a parity case, not a bench workload")

    # one step, with optional per-stage event recording; skip_dominant leaves
    # out the attention call (to time that call inside real steps by difference)
    def step(self, ev=None, skip_dominant=False):
        def mark(name):
            if ev is not None:
                e = self.torch.cuda.Event(enable_timing=True)
                e.record()
                ev.append((name, e))
        pl = self.plan
        if self.kind == "prefill_whole":
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
            mark("scores_topk")
            if not skip_dominant:
                pl.attend(self.q, self.k, self.v, self.seqlens)
            mark("sparse_attn_decode")
        else:
            mark("start")
            pl.select(self.q, self.ck)
            mark("scores_topk")
            if not skip_dominant:
                pl.attend(self.q, self.k, self.v, self.kd, self.vd, self.mask)
            mark("tree_verify")

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
            # the attention call's own bytes: K and V of the kept keys, Q and O
            # (the compressed keys are read by the scoring stage, not here)
            total = 0.0
            for L in np.tile(np.asarray(c.seqlens), self.rep):
                L = int(L)
                h_kv = c.k[0].shape[0]
                if L < p.dense_len:
                    kv = h_kv * L * d * 2 * 2
                else:
                    kv = h_kv * _visible_selected_keys(L - 1, p, p.topk) * d * 2 * 2
                total += kv + h_q * d * 2 * 2
            return {"dominant": "sparse_attn_decode", "bound": "hbm", "bytes": total,
                    "src": "attn_bf16.hip"}
        # tree: union of kept blocks per KV head + drafts + Q/O + masks
        h_kv, n_ctx, _ = c.k.shape
        sel = self.plan.block_idx.cpu().numpy()
        union = sum(len(np.unique(sel[:, g][sel[:, g] >= 0])) for g in range(h_kv))
        T = c.q.shape[0]
        total = (union * p.block_size * d * 2 * 2 + T * h_q * d * 2 * 2 +
                 2 * h_kv * T * d * 2 + T * 8)
        return {"dominant": "tree_verify", "bound": "hbm", "bytes": float(total),
                "union_blocks": int(union), "src": "attn_bf16.hip"}


def cpu_baseline(wl, budget_s=20.0):
    """The CPU oracle as it stands, single-threaded, on a bounded sample."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    c, p = wl.case, wl.p
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if wl.kind == "prefill_whole":
            # query i sees keys [0, i]: the oracle's prefill of that prefix with
            # one query, its compressed keys cut from the whole prompt's
            ck = O.compress_keys(c.k, p, "bf16")
            n = c.k.shape[1]
            rows, i = [], 0
            step = max(1, n // 256)
            while time.perf_counter() - t0 < budget_s and i < n:
                nw = O.num_windows(i + 1, p.kernel_size, p.kernel_stride)
                O.prefill(c.q[i:i + 1], c.k[:, :i + 1], c.v[:, :i + 1], p, "bf16", rows=[0],
                          ck=ck[:, :nw])
                rows.append(i)
                i += step
            dt = time.perf_counter() - t0
            return {"value": len(rows) / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                    "sample": f"{len(rows)} of {n} prompt positions (every {step}th) incl. "
                              f"compressing all {ck.shape[1]} windows, float64 numpy, 1 thread"}
        if wl.kind in ("prefill_bwd", "prefill_bwd_whole"):
            # gradients of single rows, selections taken from the GPU forward
            sel = (wl.cp.idx_buf.view(c.q.shape[0], c.k.shape[0], p.topk) if
                   wl.kind == "prefill_bwd_whole" else wl.plan.block_idx).cpu().numpy()
            dense_row = [False] * c.n_q
            if wl.kind == "prefill_bwd_whole":
                for (q0, q1, _, _, _), pc in zip(wl.cp.sched, wl.cp.plans):
                    for r in range(q0, q1):
                        dense_row[r] = pc.dense
            d_out = wl.d_out.float().cpu().numpy()
            sel_rows = [None] * c.n_q
            rows, i = [], 0
            step = max(1, c.n_q // 256)
            while time.perf_counter() - t0 < budget_s and i < c.n_q:
                sel_rows[i] = None if dense_row[i] else [s[s >= 0] for s in sel[i]]
                O.prefill_backward(c.q, c.k, c.v, sel_rows, p, d_out, rows=[i])
                rows.append(i)
                i += step
            dt = time.perf_counter() - t0
            return {"value": len(rows) / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                    "sample": f"{len(rows)} of {c.n_q} queries (every {step}th): dq of "
                              f"the row and its dk/dv contributions, float64 numpy, 1 thread"}
        if wl.kind == "prefill":
            ck = O.compress_keys(c.k, p, "bf16")
            rows, i = [], 0
            step = max(1, c.n_q // 256)
            while time.perf_counter() - t0 < budget_s and i < c.n_q:
                O.prefill(c.q, c.k, c.v, p, "bf16", rows=[i], ck=ck)
                rows.append(i)
                i += step
            dt = time.perf_counter() - t0
            return {"value": len(rows) / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                    "sample": f"{len(rows)} of {c.n_q} chunk queries (every {step}th) incl. "
                              f"compressing all {ck.shape[1]} windows, float64 numpy, 1 thread"}
        if wl.kind == "decode":
            n = 0
            while time.perf_counter() - t0 < budget_s and n < len(c.seqlens):
                O.decode(c.q[n:n + 1], [c.k[n]], [c.v[n]], [c.seqlens[n]], p, "bf16")
                n += 1
            dt = time.perf_counter() - t0
            return {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                    "sample": f"{n} of {len(c.seqlens)} sequences, float64 numpy, 1 thread"}
        T = c.q.shape[0]
        n = 0
        ck = O.compress_keys(c.k, p, "bf16")
        while time.perf_counter() - t0 < budget_s and n < T:
            O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, c.mask, p, "bf16", ck=ck,
                          drafts=[n])
            n += 1
        dt = time.perf_counter() - t0
        return {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                "sample": f"{n} of {T} drafts, float64 numpy, 1 thread"}


def _keep_busy(fn, seconds, torch):
    """Call fn (one step or one graph replay) at least once and until
    `seconds` of wall time have passed; synchronises at the end."""
    t0 = time.perf_counter()
    while True:
        fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--eager", action="store_true",
                    help="time steps as individual launches instead of HIP graph replays")
    ap.add_argument("--score-mode", type=int, default=None, choices=[0, 1],
                    help="group score reading: 0 summed query (default), 1 sum of "
                         "per-head softmaxes over the visible windows")
    ap.add_argument("--warm-seconds", type=float, default=0.3,
                    help="untimed work after the warm-up steps and after graph capture, "
                         "so that timing starts at steady clocks")
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
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": a.numel() * 4,
                          "bytes_written": b.numel() * 4, "launches": 3}))
        return
    wl = Workload(args.workload, torch, score_mode=args.score_mode)
    print(f"[bench] workload {wl.name}: setup done", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    # The clocks ramp up under sustained load and fall back while the GPU idles
    # (a kernel's duration drifts down by ~20% over the first ~100 ms of work):
    # keep stepping, untimed, for at least --warm-seconds before any timing.
    _keep_busy(wl.step, args.warm_seconds, torch)

    # per-stage times: eager steps with HIP events between the library calls
    evs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ev = []
        wl.step(ev)
        evs.append(ev)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    stages = {}
    for ev in evs:
        per_step = {}
        for (n0, e0), (n1, e1) in zip(ev[:-1], ev[1:]):
            per_step[n1] = per_step.get(n1, 0.0) + e0.elapsed_time(e1)
        for k, v in per_step.items():
            stages.setdefault(k, []).append(v)
    stage_ms = {k: float(np.mean(v)) for k, v in stages.items()}

    w = wl.work()
    dom = w["dominant"]
    if args.eager:
        wall = wall_eager
        dom_ms = stage_ms[dom]
        mode = "eager"
    else:
        # The K timed steps as one HIP graph (the library only launches kernels
        # on the caller's stream and allocates nothing, so steps capture whole):
        # the GPU runs them back to back with no host launch gaps, which
        # otherwise dominate the small decode steps.  One untimed replay first.
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(args.steps):
                wl.step()
        # the same K steps without the dominant call: the difference is that
        # call's cost inside real steps (same neighbours, same cache state)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for _ in range(args.steps):
                wl.step(skip_dominant=True)
        # capturing left the GPU idle: untimed replays until it is warm again
        _keep_busy(g.replay, args.warm_seconds, torch)
        gr.replay()
        torch.cuda.synchronize()
        # the timed K steps: one replay, wall clock and events
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        t0 = time.perf_counter()
        ev[0].record()
        g.replay()
        ev[1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # dominant call: median over 5 (full, without-the-call) replay pairs
        diffs = []
        for i in range(5):
            if i:
                ev[0].record()
                g.replay()
                ev[1].record()
            ev[2].record()
            gr.replay()
            ev[3].record()
            torch.cuda.synchronize()
            diffs.append(ev[0].elapsed_time(ev[1]) - ev[2].elapsed_time(ev[3]))
        dom_ms = float(np.median(diffs)) / args.steps
        mode = "hip_graph"
    print(f"[bench] {args.steps} steps in {wall:.4f} s ({mode}); eager {wall_eager:.4f} s",
          file=sys.stderr, flush=True)
    ms_per_step = wall * 1e3 / args.steps
    value = wl.tokens / (ms_per_step / 1e3)
    src = os.path.join(ROOT, "block_sparse_long_infllmv2_amd", "csrc", w["src"])
    if w["bound"] == "mfma":
        achieved = w["flop"] / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                # the counter figure is per launch of the final-chunk workload
                "traffic": _traffic(dom, src, wl.name) if w.get("launches", 1) == 1 else None,
                "kernel": dom,
                ("algorithmic_gflop_per_step" if w.get("launches", 1) > 1
                 else "algorithmic_gflop_per_launch"): round(w["flop"] / 1e9, 2),
                "kernel_ms": round(dom_ms, 4)}
        if w.get("launches", 1) > 1:
            roof["launches_per_step"] = w["launches"]
        if "launches_in_call" in w:
            # a call of several kernels: no single-launch counter figure
            roof["traffic"] = None
            roof["kernels_in_call"] = w["launches_in_call"]
            if "algorithmic_gflop_per_launch" in roof:
                roof["algorithmic_gflop_per_call"] = roof.pop("algorithmic_gflop_per_launch")
    else:
        achieved = w["bytes"] / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": _traffic(dom, src, wl.name), "kernel": dom,
                "algorithmic_mb_per_launch": round(w["bytes"] / 1e6, 3),
                "kernel_ms": round(dom_ms, 4)}

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

    out = {"metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": cfg, "roofline": roof, "launch": mode,
           "score_mode": wl.p.score_mode,
           "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
           "eager_ms_per_step": round(wall_eager * 1e3 / args.steps, 4)}
    if w["bound"] == "mfma":
        out["scoring_gflop"] = round(w["score_flop"] / 1e9, 2)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
