"""Oracle rows computed in forked worker processes (test infrastructure).

The full-size parity tests compare hundreds of rows of the 128K workloads
with the CPU oracle; each row is independent, so they are spread over a pool
of worker processes (one BLAS thread each).  The workers only run the
oracle on host arrays; they never touch the GPU.  Inputs are upcast to
float64 once, before the fork, and inherited by the workers.
"""
from __future__ import annotations

import multiprocessing
import os

import numpy as np

import oracle as O

_STATE = {}


def workers():
    """Host cores this process may run on, at most 16 (one GPU's share)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _prefill_row(i):
    s = _STATE
    r = O.prefill(s["q"], s["k"], s["v"], s["p"], s["dtype"], rows=[i], ck=s["ck"])
    return i, r["o"][i], r["lse"][i], r["S"].get(i), r["sel"].get(i)


def prefill_rows(q, k, v, p, dtype, ck, rows):
    """O.prefill for each of `rows` (query indices of the chunk): dict
    row -> (o, lse, S, sel)."""
    _STATE.clear()
    _STATE.update(q=np.asarray(q, np.float64), k=np.asarray(k, np.float64),
                  v=np.asarray(v, np.float64), p=p, dtype=dtype, ck=ck)
    try:
        with multiprocessing.get_context("fork").Pool(workers(), _init) as pool:
            out = pool.map(_prefill_row, list(rows), chunksize=4)
    finally:
        _STATE.clear()
    return {i: (o, lse, S, sel) for i, o, lse, S, sel in out}
