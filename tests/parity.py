"""Comparison helpers for the GPU parity tests (no GPU needed to import).

Selections: the GPU's kept set P must equal the oracle's set O, except when
the oracle's k'-th and (k'+1)-th best non-forced block scores are within a
relative 1e-3 of each other (k' = |O| - |forced|); then P may swap blocks
inside that band (same size, forced blocks kept).  Outputs are compared with
the oracle's attention evaluated on the GPU's own selection, so an allowed
swap cannot fail the output check.

Tolerances: bf16 inputs (float32 accumulation): max-abs 2e-2, mean-abs 2e-3;
float32 inputs: max-abs 1e-4.  Gradients (bf16 inputs) are sums of many
bf16-rounded products whose size grows with the number of rows that attend a
key, so they are held to the same bars relative to the reference's largest
magnitude: max-abs <= 2e-2 max|ref|, mean-abs <= 2e-3 max|ref| (max|ref|
floored at 1e-3).
"""
from __future__ import annotations

import numpy as np

TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, 1e-4)}
GRAD_SCALE_FLOOR = 1e-3
TIE_REL = 1e-3


def forced_set(pos, p):
    b_own = pos // p.block_size
    f = set(range(min(p.init_blocks, b_own + 1)))
    f |= set(range(max(0, b_own - p.local_blocks + 1), b_own + 1))
    return f


def check_selection(gpu_row, S_g, oracle_sel, pos, p, where=""):
    """gpu_row: int array [topk] (ascending, -1 pad); S_g: oracle block scores
    (float64, eligible blocks); oracle_sel: oracle kept blocks.  Returns the
    GPU set as a sorted int array."""
    g = np.asarray(gpu_row)
    P = g[g >= 0]
    assert np.all(np.diff(P) > 0), f"{where}: GPU selection not ascending/unique: {P}"
    assert np.all(g[len(P):] == -1), f"{where}: padding not at the end: {g}"
    O = set(int(b) for b in oracle_sel)
    Ps = set(int(b) for b in P)
    if Ps == O:
        return P
    F = forced_set(pos, p)
    rest = sorted((b for b in range(len(S_g)) if b not in F), key=lambda b: (-S_g[b], b))
    kprime = len(O) - len(F & O)
    assert len(Ps) == len(O), f"{where}: size {len(Ps)} != {len(O)}"
    assert F <= Ps, f"{where}: forced blocks missing: {F - Ps}"
    assert 0 < kprime < len(rest), f"{where}: sets differ with no tie band: {Ps ^ O}"
    sk, sk1 = S_g[rest[kprime - 1]], S_g[rest[kprime]]
    band = TIE_REL * max(abs(sk), abs(sk1), 1e-30)
    assert np.isfinite(sk) and abs(sk - sk1) < band, (
        f"{where}: sets differ outside the tie band: diff {sorted(Ps ^ O)}, "
        f"s_k={sk!r} s_k+1={sk1!r}")
    for b in Ps ^ O:
        assert abs(S_g[b] - sk) <= band, f"{where}: block {b} (score {S_g[b]}) outside band"
    return P


def check_close(got, ref, dtype, where=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{where}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = TOL[dtype]
    assert err.max() <= mx, f"{where}: max-abs {err.max():.3g} > {mx}"
    assert err.mean() <= mean, f"{where}: mean-abs {err.mean():.3g} > {mean}"
    return err.max(), err.mean()


def check_grad(got, ref, where="", dtype="bf16"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{where}: non-finite gradient"
    mx, mean = TOL[dtype]
    # floor: a gradient that vanishes in exact arithmetic (one key: dq = 0)
    # is held to 2e-5 absolute instead of a bar relative to its rounding noise
    scale = max(float(np.abs(ref).max()), GRAD_SCALE_FLOOR)
    err = np.abs(got - ref)
    print(f"  {where}: max|ref| {scale:.3g} max-abs {err.max():.3g} mean-abs {err.mean():.3g}",
          flush=True)
    assert err.max() <= mx * scale, f"{where}: max-abs {err.max():.3g} > {mx} x {scale:.3g}"
    assert err.mean() <= mean * scale, f"{where}: mean-abs {err.mean():.3g} > {mean} x {scale:.3g}"
    return err.max() / scale, err.mean() / scale
