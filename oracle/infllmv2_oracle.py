"""CPU oracle for InfLLM v2 block-sparse attention (TEST INFRASTRUCTURE ONLY).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module.  The product (the HIP library and its Python
binding) never calls it and shares no code with it.

It computes, slowly and literally, in float64, what the method defines:

  * the context is cut into fixed-size token blocks (64 tokens on the page
    "MiniCPM 4.0 ..." (shadowrocket9.top), section on native sparsity /
    InfLLM v2; 128 on the page "MiniCPM4: running LLMs on phones and PCs"
    (xugj520.cn), section 1.1 -- so the size is a parameter);
  * "semantic kernels" are overlapping 32-token units with stride 16 that add
    no parameters (xugj520.cn, section 1.1; shadowrocket9.top, InfLLM v2
    section).  Pooling is the arithmetic mean;
  * every query scores the kernels of its GQA group, the kernel scores are
    max-pooled to block scores, and the query keeps the top-k blocks
    (top-64 on shadowrocket9.top; top-6 on xugj520.cn) -- the initial block
    and a sliding local window are always kept (xugj520.cn, section 1.1);
  * attention then runs over only the kept blocks, causally;
  * contexts shorter than dense_len (8192) use plain dense attention instead
    (shadowrocket9.top, InfLLM v2 section, on the dual-frequency switch; the
    lianzai.com post, section 2 (2));
  * tree speculative decoding passes a uint64-packed ancestor mask
    (xugj520.cn, section 1.1 technical notes; the pomoai.com CPM.cu article,
    section 2 on the tree verification structure).

Readings where the pages leave a step open:
  R3  dense iff the sequence's total KV length n_k < dense_len.
  R5  only full kernel windows exist (no padded tail window).
  R6  a window is visible to a query at position p iff it ends at or before p.
  R7  group score = sum over the group's heads of scale * q_h . ck
      -- parity unpinned by the pages (no worked example exists).  With
      score_mode = 1 the other plain reading: the sum over the group's
      heads of each head's softmax over the windows visible to the query
      (pinned by invariants: each head's share sums to 1; one head per
      group selects what mode 0 selects; identical kernels give a uniform
      share).
  R8  block score = max over every visible window that overlaps the block
      -- parity unpinned by the pages.
  R9  forced blocks count toward top-k.
  R10 the local window is the query's own block and the local-1 before it.
  R11 equal scores: the lower block index wins.
  R12 scale = 1/sqrt(d) unless given.
  R13 prefill queries are the last n_q positions of the KV; decode's query
      sits at seqlen-1 with its own K/V already stored.
  R14 mask bit j of mask[i] (LSB first) means draft i may attend draft j;
      a draft always attends itself, whether or not its own bit is set, and
      bits at or above the draft count are ignored; drafts are not part of
      block selection, which runs over the context as seen from its last
      position.
  R15 head h belongs to KV group floor(h * h_kv / h_q).
  R16 compressed keys are stored in K's dtype (round-to-nearest-even).
  R18 if a query has no more eligible blocks than k, it keeps all of them.
  R21 training: gradients of the attention over each query's kept keys with
      the selection held fixed (top-k passes no gradient; compressed keys and
      block scores receive none); a key's dk / dv sum the contributions of
      every row that attends it.

Everything is float64; inputs are upcast exactly.  No blocking, no online
softmax, no fusion: each function is one step of the definition.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_round", "store_round", "num_windows", "compress_keys",
    "windows_of_block", "kernel_scores", "block_scores", "select_blocks",
    "attend", "attend_selected", "dense_attend", "forced_blocks", "prefill",
    "decode", "tree_verify", "attend_backward", "prefill_backward",
]


# --------------------------------------------------------------------------
# Storage rounding
# --------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value of each float64 (ties to even), as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range.  For a
    value in [2^(e-1), 2^e) the spacing is 2^(e-8); below the normal range
    the spacing is fixed at 2^-133.  Rounding x/spacing to the nearest
    integer with ties to even (np.rint) is exactly round-to-nearest-even.
    Values beyond the largest finite bfloat16 become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    m, e = np.frexp(x[nz])                      # x = m * 2^e, 0.5 <= |m| < 1
    spacing = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(x[nz] / spacing) * spacing
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > max_bf16, np.copysign(np.inf, r), r)
    out[nz] = r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def store_round(x, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype ("f32" or "bf16")."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_round(x)
    raise ValueError(dtype)


def _scale(params, d: int) -> float:
    return float(params.scale) if params.scale else 1.0 / math.sqrt(d)


def _group_of_head(h: int, h_q: int, h_kv: int) -> int:
    return (h * h_kv) // h_q                                       # R15


# --------------------------------------------------------------------------
# Step 2: semantic kernels (compressed keys)
# --------------------------------------------------------------------------
def num_windows(n_k: int, kernel_size: int, kernel_stride: int) -> int:
    """Number of full windows [m*s, m*s+ks) inside n_k tokens (R5)."""
    if n_k < kernel_size:
        return 0
    return (n_k - kernel_size) // kernel_stride + 1


def compress_keys(k: np.ndarray, params, dtype: str) -> np.ndarray:
    """ck[g, m] = mean of k[g, m*s : m*s+ks], rounded to the storage dtype.

    k: [h_kv][n_k][d].  Returns float64 [h_kv][n_c][d] holding values that
    are exactly representable in `dtype` (R16).
    """
    k = np.asarray(k, dtype=np.float64)
    h_kv, n_k, d = k.shape
    ks, s = params.kernel_size, params.kernel_stride
    n_c = num_windows(n_k, ks, s)
    ck = np.zeros((h_kv, n_c, d), dtype=np.float64)
    for m in range(n_c):
        ck[:, m, :] = k[:, m * s:m * s + ks, :].mean(axis=1)
    return store_round(ck, dtype)


# --------------------------------------------------------------------------
# Steps 3-4: kernel scores and block scores
# --------------------------------------------------------------------------
def windows_of_block(b: int, params, n_c: int) -> range:
    """Windows whose token span [m*s, m*s+ks) meets block b's span
    [b*B, (b+1)*B): m*s <= (b+1)*B - 1 and m*s + ks - 1 >= b*B."""
    B, ks, s = params.block_size, params.kernel_size, params.kernel_stride
    lo = max(0, -(-(b * B - ks + 1) // s))
    hi = min(n_c - 1, ((b + 1) * B - 1) // s)
    return range(lo, hi + 1)


def kernel_scores(q_row: np.ndarray, ck: np.ndarray, pos: int, params,
                  h_kv: int) -> np.ndarray:
    """sigma[g, m] = scale * sum_{h in g} q_h . ck[g, m] for windows that end
    at or before pos (R6, R7); -inf for the others.  score_mode 1 (the other
    reading of R7): sigma[g, m] = sum_{h in g} of head h's softmax over the
    visible windows of scale * q_h . ck[g, m'], taken at m.

    q_row: [h_q][d] (one query token), ck: [h_kv][n_c][d].
    """
    q_row = np.asarray(q_row, dtype=np.float64)
    h_q, d = q_row.shape
    n_c = ck.shape[1]
    scale = _scale(params, d)
    ks, s = params.kernel_size, params.kernel_stride
    mode = getattr(params, "score_mode", 0)
    sigma = np.full((h_kv, n_c), -np.inf)
    visible = np.array([m * s + ks - 1 <= pos for m in range(n_c)], dtype=bool)
    for g in range(h_kv):
        heads = [h for h in range(h_q) if _group_of_head(h, h_q, h_kv) == g]
        if mode == 0:
            qsum = q_row[heads].sum(axis=0)
            vals = scale * (ck[g] @ qsum)
            sigma[g, visible] = vals[visible]
        elif visible.any():
            total = np.zeros(int(visible.sum()))
            for h in heads:
                logits = scale * (ck[g][visible] @ q_row[h])
                w = np.exp(logits - logits.max())
                total += w / w.sum()
            sigma[g, visible] = total
    return sigma


def block_scores(sigma: np.ndarray, pos: int, params) -> np.ndarray:
    """S[g, b] = max of sigma[g, m] over windows m overlapping block b (R8),
    for the eligible blocks b = 0 .. floor(pos / B); -inf if none visible."""
    h_kv, n_c = sigma.shape
    n_elig = pos // params.block_size + 1
    S = np.full((h_kv, n_elig), -np.inf)
    for b in range(n_elig):
        ms = list(windows_of_block(b, params, n_c))
        if ms:
            S[:, b] = sigma[:, ms].max(axis=1)
    return S


# --------------------------------------------------------------------------
# Step 5: block selection
# --------------------------------------------------------------------------
def forced_blocks(pos: int, params) -> set:
    """Initial blocks and the local window (own block + local-1 before it),
    restricted to eligible blocks (R9, R10)."""
    b_own = pos // params.block_size
    init = set(range(min(params.init_blocks, b_own + 1)))
    local = set(range(max(0, b_own - params.local_blocks + 1), b_own + 1))
    return init | local


def select_blocks(S_g: np.ndarray, pos: int, params) -> np.ndarray:
    """Kept blocks for one (query, group): forced blocks, then the best
    remaining eligible blocks by (score descending, index ascending) until
    min(topk, #eligible) are kept (R9, R11, R18).  Ascending block ids."""
    n_elig = pos // params.block_size + 1
    assert S_g.shape[0] == n_elig
    F = forced_blocks(pos, params)
    budget = min(params.topk, n_elig)
    rest = [b for b in range(n_elig) if b not in F]
    rest.sort(key=lambda b: (-S_g[b], b))
    chosen = sorted(F) + rest[:max(0, budget - len(F))]
    return np.array(sorted(chosen), dtype=np.int64)


# --------------------------------------------------------------------------
# Step 6: attention over a key set
# --------------------------------------------------------------------------
def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """softmax(scale * keys @ q) @ values and its natural-log normaliser.

    q: [d], keys/values: [n][d] (n >= 1).  Returns (o [d], lse)."""
    logits = scale * (np.asarray(keys, np.float64) @ np.asarray(q, np.float64))
    mx = logits.max()
    w = np.exp(logits - mx)
    z = w.sum()
    o = (w / z) @ np.asarray(values, np.float64)
    return o, mx + math.log(z)


def _block_tokens(blocks, pos: int, B: int) -> np.ndarray:
    toks = [t for b in blocks for t in range(b * B, (b + 1) * B) if t <= pos]
    return np.array(toks, dtype=np.int64)


def dense_attend(q_row, k, v, pos: int, params):
    """Causal dense attention of one query token (all heads) over keys
    0..pos.  Returns (o [h_q][d], lse [h_q])."""
    q_row = np.asarray(q_row, np.float64)
    h_q, d = q_row.shape
    h_kv = k.shape[0]
    scale = _scale(params, d)
    o = np.zeros((h_q, d))
    lse = np.zeros(h_q)
    for h in range(h_q):
        g = _group_of_head(h, h_q, h_kv)
        o[h], lse[h] = attend(q_row[h], k[g, :pos + 1], v[g, :pos + 1], scale)
    return o, lse


# --------------------------------------------------------------------------
# Whole-path drivers
# --------------------------------------------------------------------------
def attend_selected(q_row, k, v, sel, pos, params, extra=None):
    """Step 6 for one query token given its kept blocks per KV head:
    attention over the keys j <= pos of those blocks, plus `extra` =
    (k_x, v_x) [h_kv][n][d] keys attended in the same softmax (tree drafts).
    Returns (o [h_q][d], lse [h_q])."""
    q_row = np.asarray(q_row, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    h_q, d = q_row.shape
    h_kv = k.shape[0]
    scale = _scale(params, d)
    o = np.zeros((h_q, d))
    lse = np.zeros(h_q)
    for h in range(h_q):
        g = _group_of_head(h, h_q, h_kv)
        toks = _block_tokens(sel[g], pos, params.block_size)
        keys, vals = k[g, toks], v[g, toks]
        if extra is not None:
            keys = np.concatenate([keys, np.asarray(extra[0][g], np.float64)], axis=0)
            vals = np.concatenate([vals, np.asarray(extra[1][g], np.float64)], axis=0)
        o[h], lse[h] = attend(q_row[h], keys, vals, scale)
    return o, lse


# --------------------------------------------------------------------------
# Step 7 (training): gradients through the kept keys, the selection fixed
# (top-k is not differentiable; "trainable" sparse attention trains the
# attention over the blocks it keeps)
# --------------------------------------------------------------------------
def attend_backward(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
                    d_o: np.ndarray):
    """Gradients of o = softmax(scale * keys @ q) @ values with respect to
    q, keys and values, given d_o = dL/do.  q, d_o: [d]; keys/values: [n][d].
    Returns (dq [d], dkeys [n][d], dvalues [n][d])."""
    q = np.asarray(q, np.float64)
    keys = np.asarray(keys, np.float64)
    values = np.asarray(values, np.float64)
    d_o = np.asarray(d_o, np.float64)
    logits = scale * (keys @ q)
    p = np.exp(logits - logits.max())
    p /= p.sum()                                   # attention weights
    o = p @ values
    dvalues = np.outer(p, d_o)                     # o = sum_j p_j v_j
    dp = values @ d_o                              # dL/dp_j = v_j . d_o
    ds = p * (dp - d_o @ o)                        # through the softmax
    dq = scale * (ds @ keys)
    dkeys = scale * np.outer(ds, q)
    return dq, dkeys, dvalues


def prefill_backward(q, k, v, sel_rows, params, d_out, rows=None):
    """Gradients of the prefill attention (queries = the last n_q positions
    of n_k keys) with each row's kept blocks fixed: sel_rows[i][g] are row
    i's kept blocks for KV head g, or sel_rows[i] is None for a dense row
    (every key up to its position).  q, d_out: [n_q][h_q][d]; k, v:
    [h_kv][n_k][d].  Returns (dq [n_q][h_q][d], dk, dv [h_kv][n_k][d]);
    dk / dv sum the contributions of every row that attends a key.  `rows`
    restricts the work to those query rows (dq of the others stays 0, and
    dk / dv hold only the listed rows' contributions)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    d_out = np.asarray(d_out, np.float64)
    n_q, h_q, d = q.shape
    h_kv, n_k, _ = k.shape
    scale = _scale(params, d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for i in (range(n_q) if rows is None else rows):
        pos = n_k - n_q + i
        for h in range(h_q):
            g = _group_of_head(h, h_q, h_kv)
            if sel_rows[i] is None:
                toks = np.arange(pos + 1)
            else:
                toks = _block_tokens(sel_rows[i][g], pos, params.block_size)
            gq, gk, gv = attend_backward(q[i, h], k[g, toks], v[g, toks], scale, d_out[i, h])
            dq[i, h] = gq
            dk[g, toks] += gk
            dv[g, toks] += gv
    return dq, dk, dv


def _sparse_row(q_row, k, v, ck, pos, params, extra=None):
    """Steps 3-6 for one query token.  `extra` = (k_x, v_x) [h_kv][n][d]
    additional keys attended densely (tree drafts)."""
    q_row = np.asarray(q_row, np.float64)
    h_kv = k.shape[0]
    sigma = kernel_scores(q_row, ck, pos, params, h_kv)
    S = block_scores(sigma, pos, params)
    sel = [select_blocks(S[g], pos, params) for g in range(h_kv)]
    o, lse = attend_selected(q_row, k, v, sel, pos, params, extra)
    return o, lse, S, sel


def prefill(q, k, v, params, dtype: str, rows=None, ck=None):
    """Chunked prefill: queries are the last n_q positions of n_k keys (R13).

    q: [n_q][h_q][d], k/v: [h_kv][n_k][d].  `rows` restricts the work to a
    subset of query indices.  Returns a dict with per-row outputs and, when
    the sparse path runs, the compressed keys, block scores and selections.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n_q, h_q, d = q.shape
    h_kv, n_k, _ = k.shape
    rows = range(n_q) if rows is None else list(rows)
    res = {"rows": list(rows), "o": {}, "lse": {}, "S": {}, "sel": {},
           "dense": n_k < params.dense_len}
    if res["dense"]:                                               # R3
        for i in rows:
            pos = n_k - n_q + i
            res["o"][i], res["lse"][i] = dense_attend(q[i], k, v, pos, params)
        return res
    if ck is None:
        ck = compress_keys(k, params, dtype)
    res["ck"] = ck
    for i in rows:
        pos = n_k - n_q + i
        o, lse, S, sel = _sparse_row(q[i], k, v, ck, pos, params)
        res["o"][i], res["lse"][i], res["S"][i], res["sel"][i] = o, lse, S, sel
    return res


def decode(q, ks, vs, seqlens, params, dtype: str, cks=None):
    """One query per sequence at position seqlen-1 (R13), each sequence
    dense or sparse on its own length (R3).

    q: [batch][h_q][d]; ks/vs: per-sequence [h_kv][L_i][d]."""
    out = {"o": [], "lse": [], "S": [], "sel": [], "dense": [], "ck": []}
    for i, L in enumerate(seqlens):
        L = int(L)
        k = np.asarray(ks[i], np.float64)[:, :L]
        v = np.asarray(vs[i], np.float64)[:, :L]
        pos = L - 1
        if L < params.dense_len:
            o, lse = dense_attend(q[i], k, v, pos, params)
            out["o"].append(o); out["lse"].append(lse)
            out["S"].append(None); out["sel"].append(None)
            out["dense"].append(True); out["ck"].append(None)
            continue
        ck = compress_keys(k, params, dtype) if cks is None else cks[i]
        o, lse, S, sel = _sparse_row(q[i], k, v, ck, pos, params)
        out["o"].append(o); out["lse"].append(lse)
        out["S"].append(S); out["sel"].append(sel)
        out["dense"].append(False); out["ck"].append(ck)
    return out


def tree_verify(q, k, v, k_draft, v_draft, mask, params, dtype: str,
                ck=None, drafts=None):
    """Tree speculative verification (R14).

    q: [T][h_q][d] drafts' queries; k/v: [h_kv][n_ctx][d] context;
    k_draft/v_draft: [h_kv][T][d]; mask: uint64 [T].  Every draft selects
    blocks over the context as seen from position n_ctx-1 and attends, in
    one softmax, its selected context keys and the drafts set in its mask.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    kd = np.asarray(k_draft, np.float64)
    vd = np.asarray(v_draft, np.float64)
    T = q.shape[0]
    n_ctx = k.shape[1]
    pos = n_ctx - 1
    drafts = range(T) if drafts is None else list(drafts)
    dense = n_ctx < params.dense_len
    if not dense and ck is None:
        ck = compress_keys(k, params, dtype)
    res = {"o": {}, "lse": {}, "S": {}, "sel": {}, "ck": ck, "dense": dense}
    n_b = -(-n_ctx // params.block_size)
    for i in drafts:
        bits = int(mask[i])
        # bit j (LSB first) of mask[i]: draft i attends draft j; the draft
        # always attends itself, and bits at or above T name no draft (R14)
        anc = sorted({i} | {j for j in range(T) if (bits >> j) & 1})
        extra = (kd[:, anc], vd[:, anc])
        if dense:
            # dense context (R3): every context block, i.e. every key
            # 0 .. n_ctx-1, in the same softmax as the drafts
            every = [np.arange(n_b)] * k.shape[0]
            o, lse = attend_selected(q[i], k, v, every, pos, params, extra=extra)
            res["o"][i], res["lse"][i] = o, lse
            continue
        o, lse, S, sel = _sparse_row(q[i], k, v, ck, pos, params, extra=extra)
        res["o"][i], res["lse"][i], res["S"][i], res["sel"][i] = o, lse, S, sel
    return res
