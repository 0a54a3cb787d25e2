"""Pre-planned call sequences over the C ABI: chunked prefill, ragged decode
and tree verification.

A plan allocates (through torch, once) every buffer a step needs -- positions,
block scores, selections, workspaces, outputs -- and `run` issues the library
calls on the current stream.  The plans perform no arithmetic of their own.
"""
from __future__ import annotations

import torch

from . import binding as B


def _windows(n: int, ks: int, s: int) -> int:
    return 0 if n < ks else (n - ks) // s + 1


class PrefillPlan:
    """The final n_q queries of an n_k-token sequence (chunked prefill).

    Calls: compress_keys (windows completed by this chunk) -> block_scores ->
    select_topk -> sparse_attn_prefill.  Dense (n_k < dense_len): attention only.
    """

    def __init__(self, n_q, n_k, h_q, h_kv, d, dtype, params, device="cuda",
                 out=None, lse=None, score_buf=None, idx_buf=None):
        """`out` [n_q][h_q][d] and `lse` [n_q][h_q] may be views into a larger
        output; `score_buf` / `idx_buf` are flat float32 / int32 scratch
        buffers, large enough, that plans run one after another on a stream
        may share."""
        self.p = B.to_params(params)
        self.n_q, self.n_k, self.h_q, self.h_kv, self.d = n_q, n_k, h_q, h_kv, d
        self.dtype = dtype
        self.dense = n_k < self.p.dense_len
        self.nb = (n_k + self.p.block_size - 1) // self.p.block_size
        dev = torch.device(device)
        self.seqlens = torch.tensor([n_k], dtype=torch.int32, device=dev)
        self.row_pos = torch.arange(n_k - n_q, n_k, dtype=torch.int32, device=dev)

        def scratch(buf, shape, dt):
            if buf is None:
                return torch.empty(shape, dtype=dt, device=dev)
            n = shape[0] * shape[1] * shape[2]
            assert buf.dtype == dt and buf.numel() >= n
            return buf[:n].view(shape)

        self.scores = None if self.dense else scratch(score_buf, (n_q, h_kv, self.nb),
                                                      torch.float32)
        self.block_idx = None if self.dense else scratch(idx_buf, (n_q, h_kv, self.p.topk),
                                                         torch.int32)
        self.out = out if out is not None else torch.empty((n_q, h_q, d), dtype=dtype,
                                                           device=dev)
        self.lse = lse if lse is not None else torch.empty((n_q, h_q), dtype=torch.float32,
                                                           device=dev)
        # windows completed by this chunk: all windows not complete before it
        self.m_begin = _windows(n_k - n_q, self.p.kernel_size, self.p.kernel_stride)
        self.m_end = _windows(n_k, self.p.kernel_size, self.p.kernel_stride)

    def compress(self, k_cache, ck_cache, m_begin=None):
        """k_cache [h_kv][cap][d] -> ck_cache [h_kv][nc_cap][d], windows
        [m_begin, m_end)."""
        mb = self.m_begin if m_begin is None else m_begin
        B.infllmv2_compress_keys(k_cache.unsqueeze(0), self.seqlens, mb, self.m_end,
                                 ck_cache.unsqueeze(0), self.p)

    def score(self, q, ck_cache):
        B.infllmv2_block_scores(q, None, self.row_pos, ck_cache.unsqueeze(0), self.seqlens,
                                self.scores, self.n_k - 1, self.p)

    def topk(self):
        B.infllmv2_select_topk(self.scores, None, self.row_pos, self.seqlens, self.block_idx,
                               self.p)

    def select(self, q, ck_cache):
        self.score(q, ck_cache)
        self.topk()

    def attend(self, q, k_cache, v_cache):
        B.infllmv2_sparse_attn_prefill(q, k_cache, v_cache, self.n_k, self.block_idx, self.out,
                                       self.lse, self.p)

    def backward_workspace_bytes(self):
        return B.infllmv2_workspace_size(B.OP_PREFILL_BWD, self.n_q, self.h_q, self.h_kv,
                                         self.d, self.n_k, self.p)

    def backward(self, q, k_cache, v_cache, d_out, dq, dk, dv, ws=None):
        """Gradients of the last attend() with its selection fixed: dq
        [n_q][h_q][d] written, float32 dk / dv [h_kv][cap][d] added into.
        Without `ws` the plan allocates its workspace on the first call."""
        if ws is None:
            if getattr(self, "bwd_ws", None) is None:
                self.bwd_ws = torch.empty(self.backward_workspace_bytes(), dtype=torch.uint8,
                                          device=self.out.device)
            ws = self.bwd_ws
        B.infllmv2_sparse_attn_prefill_backward(q, k_cache, v_cache, self.n_k, self.block_idx,
                                                self.out, self.lse, d_out, dq, dk, dv, ws,
                                                self.p)

    def run(self, q, k_cache, v_cache, ck_cache, m_begin=None):
        if not self.dense:
            self.compress(k_cache, ck_cache, m_begin)
            self.select(q, ck_cache)
        self.attend(q, k_cache, v_cache)
        return self.out


def chunk_schedule(n: int, chunk: int, params) -> list:
    """Chunks of a whole-prompt prefill: (q_begin, q_end, n_k, m_begin, m_end)
    per chunk, queries [q_begin, q_end) over keys [0, n_k = q_end), and the
    compressed-key windows [m_begin, m_end) that complete inside it."""
    p = B.to_params(params)
    out = []
    for q0 in range(0, n, chunk):
        q1 = min(n, q0 + chunk)
        out.append((q0, q1, q1, _windows(q0, p.kernel_size, p.kernel_stride),
                    _windows(q1, p.kernel_size, p.kernel_stride)))
    return out


class ChunkedPrefill:
    """A whole prompt of n tokens prefilled chunk by chunk (chunk c: queries
    [c*chunk, (c+1)*chunk) over the keys up to its end), as an engine runs a
    long prompt.  Each chunk: compress the windows it completes, block
    scores, top-k, sparse attention (a chunk whose keys number fewer than
    dense_len: its windows, then dense attention only).  Plans and buffers
    are made once; all chunks share one score scratch buffer and write into
    one output.  The chunks share one selection buffer too, unless
    keep_selections is set (training): then every chunk keeps its own rows'
    selections, which backward() needs.

    overlap: each chunk's compress, scores and top-k run on a second stream
    (default priority) while the previous chunk's attention runs on the
    caller's stream; chunk i's attention waits for chunk i's selection only.
    Selections then alternate between two buffers (unless kept), and the
    selection of chunk i waits for the attention of chunk i - 2, the last
    reader of the buffer it overwrites.  The results are the same."""

    def __init__(self, n, chunk, h_q, h_kv, d, dtype, params, device="cuda",
                 keep_selections=False, overlap=False):
        self.p = B.to_params(params)
        self.n, self.chunk = n, chunk
        dev = torch.device(device)
        self.sched = chunk_schedule(n, chunk, params)
        self.out = torch.empty((n, h_q, d), dtype=dtype, device=dev)
        self.lse = torch.empty((n, h_q), dtype=torch.float32, device=dev)
        nb_max = (n + self.p.block_size - 1) // self.p.block_size
        self.score_buf = torch.empty(chunk * h_kv * nb_max, dtype=torch.float32, device=dev)
        per_row = h_kv * self.p.topk
        self.keep_selections = keep_selections
        self.overlap = overlap
        n_sel = n if keep_selections else (2 if overlap else 1) * chunk
        self.idx_buf = torch.empty(n_sel * per_row, dtype=torch.int32, device=dev)

        def idx_view(i, q0):
            if keep_selections:
                return self.idx_buf[q0 * per_row:]
            return self.idx_buf[(i % 2 if overlap else 0) * chunk * per_row:]
        self.plans = [PrefillPlan(q1 - q0, n_k, h_q, h_kv, d, dtype, params, device=dev,
                                  out=self.out[q0:q1], lse=self.lse[q0:q1],
                                  score_buf=self.score_buf, idx_buf=idx_view(i, q0))
                      for i, (q0, q1, n_k, _, _) in enumerate(self.sched)]
        self.side = torch.cuda.Stream(device=dev) if overlap else None
        self.bwd_ws = None

    def _select(self, pl, qc, k_cache, ck_cache, m0, m1):
        # every chunk appends the windows it completes (a dense chunk too:
        # later sparse chunks score against all of them)
        if m1 > m0:
            pl.compress(k_cache, ck_cache, m_begin=m0)
        if not pl.dense:
            pl.select(qc, ck_cache)

    def run(self, q, k_cache, v_cache, ck_cache, skip_attention=False):
        """q [n][h_q][d]; K/V caches [h_kv][cap >= n][d]; ck_cache
        [h_kv][>= windows(n)][d] (filled here, window by window)."""
        if not self.overlap:
            for (q0, q1, _, m0, m1), pl in zip(self.sched, self.plans):
                qc = q[q0:q1]
                self._select(pl, qc, k_cache, ck_cache, m0, m1)
                if not skip_attention:
                    pl.attend(qc, k_cache, v_cache)
            return self.out
        main, side = torch.cuda.current_stream(), self.side
        side.wait_stream(main)                      # the inputs are ready
        attended = []
        for i, ((q0, q1, _, m0, m1), pl) in enumerate(zip(self.sched, self.plans)):
            qc = q[q0:q1]
            with torch.cuda.stream(side):
                if i >= 2 and not self.keep_selections:
                    side.wait_event(attended[i - 2])
                self._select(pl, qc, k_cache, ck_cache, m0, m1)
                selected = torch.cuda.Event()
                selected.record(side)
            main.wait_event(selected)
            if not skip_attention:
                pl.attend(qc, k_cache, v_cache)
            done = torch.cuda.Event()
            done.record(main)
            attended.append(done)
        main.wait_stream(side)
        return self.out

    def attend_all(self, q, k_cache, v_cache):
        """The attention calls of every chunk (selections from the last run)."""
        for (q0, q1, _, _, _), pl in zip(self.sched, self.plans):
            pl.attend(q[q0:q1], k_cache, v_cache)

    def backward(self, q, k_cache, v_cache, d_out, dq, dk, dv):
        """Gradients of the whole prompt's attention (the last run, its
        selections fixed): dq [n][h_q][d] written, float32 dk / dv
        [h_kv][cap][d] added into by every chunk (zero them first).  Needs
        keep_selections."""
        if not self.keep_selections:
            raise ValueError("backward() needs ChunkedPrefill(..., keep_selections=True)")
        if self.bwd_ws is None:
            n = max(pl.backward_workspace_bytes() for pl in self.plans)
            self.bwd_ws = torch.empty(n, dtype=torch.uint8, device=self.out.device)
        for (q0, q1, _, _, _), pl in zip(self.sched, self.plans):
            pl.backward(q[q0:q1], k_cache, v_cache, d_out[q0:q1], dq[q0:q1], dk, dv,
                        ws=self.bwd_ws)


class DecodePlan:
    """One new query per sequence of a ragged batch (its K/V already cached).

    Calls: block_scores -> sparse_attn_decode_topk (the top-k selection,
    split-KV attention and combine; the selection runs inside the attention
    kernel where it fits).  select_in_attend=False: block_scores ->
    select_topk -> sparse_attn_decode instead (the same results).  Compressed
    keys are assumed current (append windows with compress_keys as the caches
    grow).
    """

    def __init__(self, batch, max_seqlen, h_q, h_kv, d, dtype, params, device="cuda",
                 select_in_attend=True):
        self.p = B.to_params(params)
        self.batch, self.max_seqlen = batch, max_seqlen
        self.h_q, self.h_kv, self.d, self.dtype = h_q, h_kv, d, dtype
        self.select_in_attend = select_in_attend
        self.dense = max_seqlen < self.p.dense_len
        dev = torch.device(device)
        self.nb = (max_seqlen + self.p.block_size - 1) // self.p.block_size
        self.row_seq = torch.arange(batch, dtype=torch.int32, device=dev)
        self.scores = torch.empty((batch, h_kv, self.nb), dtype=torch.float32, device=dev)
        self.block_idx = torch.empty((batch, h_kv, self.p.topk), dtype=torch.int32, device=dev)
        ws = B.infllmv2_workspace_size(B.OP_DECODE, batch, h_q, h_kv, d, max_seqlen, self.p)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.out = torch.empty((batch, h_q, d), dtype=dtype, device=dev)
        self.lse = torch.empty((batch, h_q), dtype=torch.float32, device=dev)

    def select(self, q, ck_cache, seqlens):
        """Block scores (and, unless the attention call selects, the top-k)."""
        if self.dense:
            return
        B.infllmv2_block_scores(q, self.row_seq, None, ck_cache, seqlens, self.scores,
                                self.max_seqlen - 1, self.p)
        if not self.select_in_attend:
            B.infllmv2_select_topk(self.scores, self.row_seq, None, seqlens, self.block_idx,
                                   self.p)

    def attend(self, q, k_cache, v_cache, seqlens):
        if self.select_in_attend and not self.dense:
            B.infllmv2_sparse_attn_decode_topk(q, k_cache, v_cache, seqlens, self.max_seqlen,
                                               self.scores, self.block_idx, self.out, self.lse,
                                               self.ws, self.p)
        else:
            B.infllmv2_sparse_attn_decode(q, k_cache, v_cache, seqlens, self.max_seqlen,
                                          self.block_idx, self.out, self.lse, self.ws, self.p)

    def run(self, q, k_cache, v_cache, ck_cache, seqlens):
        self.select(q, ck_cache, seqlens)
        self.attend(q, k_cache, v_cache, seqlens)
        return self.out


class TreePlan:
    """n_draft tree-shaped draft tokens after an n_ctx-token context.

    Calls: block_scores (every draft at the context's last position) ->
    tree_verify_topk (top-k selection, union planner where used, split-KV,
    combine).  select_in_attend=False: block_scores -> select_topk ->
    tree_verify instead (the same results).
    """

    def __init__(self, n_draft, n_ctx, h_q, h_kv, d, dtype, params, device="cuda",
                 select_in_attend=True):
        self.p = B.to_params(params)
        self.n_draft, self.n_ctx = n_draft, n_ctx
        self.h_q, self.h_kv, self.d, self.dtype = h_q, h_kv, d, dtype
        self.select_in_attend = select_in_attend
        self.dense = n_ctx < self.p.dense_len
        dev = torch.device(device)
        self.nb = (n_ctx + self.p.block_size - 1) // self.p.block_size
        self.seqlens = torch.tensor([n_ctx], dtype=torch.int32, device=dev)
        self.row_pos = torch.full((n_draft,), n_ctx - 1, dtype=torch.int32, device=dev)
        self.scores = None if self.dense else torch.empty(
            (n_draft, h_kv, self.nb), dtype=torch.float32, device=dev)
        self.block_idx = None if self.dense else torch.empty(
            (n_draft, h_kv, self.p.topk), dtype=torch.int32, device=dev)
        ws = B.infllmv2_workspace_size(B.OP_TREE, n_draft, h_q, h_kv, d, n_ctx, self.p)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.out = torch.empty((n_draft, h_q, d), dtype=dtype, device=dev)
        self.lse = torch.empty((n_draft, h_q), dtype=torch.float32, device=dev)

    def select(self, q, ck_cache):
        """Block scores (and, unless the verification call selects, the top-k)."""
        if self.dense:
            return
        B.infllmv2_block_scores(q, None, self.row_pos, ck_cache.unsqueeze(0), self.seqlens,
                                self.scores, self.n_ctx - 1, self.p)
        if not self.select_in_attend:
            B.infllmv2_select_topk(self.scores, None, self.row_pos, self.seqlens,
                                   self.block_idx, self.p)

    def attend(self, q, k_cache, v_cache, k_draft, v_draft, tree_mask):
        if self.select_in_attend and not self.dense:
            B.infllmv2_tree_verify_topk(q, k_cache, v_cache, self.n_ctx, k_draft, v_draft,
                                        tree_mask, self.scores, self.block_idx, self.out,
                                        self.lse, self.ws, self.p)
        else:
            B.infllmv2_tree_verify(q, k_cache, v_cache, self.n_ctx, k_draft, v_draft, tree_mask,
                                   self.block_idx, self.out, self.lse, self.ws, self.p)

    def run(self, q, k_cache, v_cache, ck_cache, k_draft, v_draft, tree_mask):
        self.select(q, ck_cache)
        self.attend(q, k_cache, v_cache, k_draft, v_draft, tree_mask)
        return self.out
