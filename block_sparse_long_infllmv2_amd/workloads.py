"""Seeded synthetic workloads for InfLLM v2 block-sparse attention.

This module only draws random inputs: Gaussian queries, keys and values, a
shared unit direction planted into a few key blocks and into every query (so
that block selection has a non-trivial answer), ragged sequence lengths and
random draft trees.  It holds none of the method's arithmetic (no pooling,
scoring, selection or attention), so both the CPU oracle's tests and the GPU
path can consume the very same arrays.

Every array is float32 holding values exactly representable in the workload's
storage dtype ("bf16" inputs are rounded to bfloat16, round-to-nearest-even,
before they are handed out), so the GPU path and the oracle read identical
numbers.

Shapes follow the library's layouts:
  queries      [rows][h_q][d]
  keys/values  [h_kv][n][d]      (one array per sequence)
  draft K/V    [h_kv][n_draft][d]

The five workloads are the ones the pages' headline numbers are about
(long-context MiniCPM4 inference: a 128K context, a 64-token block, top-64
selection, dense below 8192 tokens; page "MiniCPM 4.0" (shadowrocket9.top),
section on native sparsity / InfLLM v2), made concrete with a 32-query-head /
2-KV-head / d=128 layout.  The pages publish no inputs; these stand in.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Params", "PrefillCase", "DecodeCase", "TreeCase",
    "round_to_bf16", "make_prefill", "make_decode", "make_tree", "make_upstream_grad",
    "config", "CONFIG_NAMES",
]


@dataclass
class Params:
    """Sparse-attention parameters (names follow the pages' sparse_config)."""
    block_size: int = 64
    kernel_size: int = 32
    kernel_stride: int = 16
    topk: int = 64
    init_blocks: int = 1
    local_blocks: int = 2
    dense_len: int = 8192
    scale: float = 0.0          # 0 -> 1/sqrt(head_dim)
    score_mode: int = 0         # 0: summed-query group score; 1: sum of per-head softmaxes

    def replace(self, **kw) -> "Params":
        return dataclasses.replace(self, **kw)


@dataclass
class PrefillCase:
    """One sequence: the final n_q queries of an n_k-token context."""
    name: str
    dtype: str                  # "f32" | "bf16"
    q: np.ndarray               # [n_q][h_q][d]
    k: np.ndarray               # [h_kv][n_k][d]
    v: np.ndarray               # [h_kv][n_k][d]
    params: Params
    planted: np.ndarray         # planted block ids (for reporting only)

    @property
    def n_q(self) -> int:
        return self.q.shape[0]

    @property
    def n_k(self) -> int:
        return self.k.shape[1]


@dataclass
class DecodeCase:
    """A batch of sequences, one new query each, at position seqlen-1."""
    name: str
    dtype: str
    q: np.ndarray               # [batch][h_q][d]
    k: list                     # per sequence [h_kv][L_i][d]
    v: list
    seqlens: np.ndarray         # int32 [batch]
    params: Params
    planted: list = field(default_factory=list)


@dataclass
class TreeCase:
    """n_draft draft tokens after an n_ctx-token context, tree-shaped."""
    name: str
    dtype: str
    q: np.ndarray               # [n_draft][h_q][d]
    k: np.ndarray               # [h_kv][n_ctx][d]
    v: np.ndarray
    k_draft: np.ndarray         # [h_kv][n_draft][d]
    v_draft: np.ndarray
    parents: np.ndarray         # int32 [n_draft], -1 for the root
    mask: np.ndarray            # uint64 [n_draft]; bit j of mask[i]: i sees draft j
    params: Params
    planted: np.ndarray = None

    @property
    def n_ctx(self) -> int:
        return self.k.shape[1]


def round_to_bf16(x: np.ndarray, inplace: bool = False) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to even), returned as float32.
    Inputs are finite, so the 32-bit sum below cannot wrap."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not inplace:
        x = x.copy()
    bits = x.view(np.uint32)
    tmp = bits >> np.uint32(16)
    tmp &= np.uint32(1)
    tmp += np.uint32(0x7FFF)
    bits += tmp
    bits &= np.uint32(0xFFFF0000)
    return x


def _to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round a freshly drawn float32 array (owned here) to the dtype in place."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return round_to_bf16(x, inplace=True) if dtype == "bf16" else x


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def _unit(rng: np.random.Generator, d: int) -> np.ndarray:
    u = rng.standard_normal(d)
    return (u / np.linalg.norm(u)).astype(np.float32)


def _pick_planted(rng, n_k: int, p: Params, count: int) -> np.ndarray:
    """Distinct full blocks, never block 0..init-1 nor the last local blocks."""
    n_b = -(-n_k // p.block_size)
    lo = p.init_blocks
    hi = n_b - p.local_blocks          # exclusive
    pool = np.arange(lo, max(lo, hi))
    count = min(count, pool.size)
    return np.sort(rng.choice(pool, size=count, replace=False)).astype(np.int64)


def _plant(k: np.ndarray, blocks: np.ndarray, u: np.ndarray, beta: float, bs: int):
    for b in blocks:
        k[:, b * bs:(b + 1) * bs, :] += beta * u


def make_prefill(seed: int, n_k: int, n_q: int, h_q: int, h_kv: int, d: int,
                 params: Params, dtype: str, n_planted: int, alpha: float,
                 beta: float, name: str = "prefill") -> PrefillCase:
    """Queries = the last n_q positions of an n_k-token context."""
    assert 0 < n_q <= n_k
    u = _unit(_rng(seed, 3), d)
    planted = _pick_planted(_rng(seed, 4), n_k, params, n_planted)
    k = _rng(seed, 1).standard_normal((h_kv, n_k, d), dtype=np.float32)
    v = _rng(seed, 2).standard_normal((h_kv, n_k, d), dtype=np.float32)
    q = _rng(seed, 0).standard_normal((n_q, h_q, d), dtype=np.float32)
    _plant(k, planted, u, beta, params.block_size)
    q += alpha * u
    return PrefillCase(name, dtype, _to_dtype(q, dtype), _to_dtype(k, dtype),
                       _to_dtype(v, dtype), params, planted)


def make_upstream_grad(seed: int, n_q: int, h_q: int, d: int, dtype: str) -> np.ndarray:
    """Gradient arriving at the attention output, [n_q][h_q][d]: N(0, 1)."""
    g = _rng(seed, 9).standard_normal((n_q, h_q, d), dtype=np.float32)
    return _to_dtype(g, dtype)


def make_decode(seed: int, seqlens, h_q: int, h_kv: int, d: int, params: Params,
                dtype: str, planted_per_token: float = None, n_planted: int = None,
                alpha: float = 1.5, beta: float = 1.5,
                name: str = "decode") -> DecodeCase:
    """One query per sequence.  Planted count is n_planted, or L // (1/ratio)."""
    seqlens = np.asarray(seqlens, dtype=np.int32)
    u = _unit(_rng(seed, 3), d)
    qs = _rng(seed, 0).standard_normal((len(seqlens), h_q, d), dtype=np.float32)
    qs += alpha * u
    ks, vs, planted = [], [], []
    for i, L in enumerate(seqlens):
        L = int(L)
        cnt = n_planted if n_planted is not None else int(L * planted_per_token)
        pl = _pick_planted(_rng(seed, 100 + 4 * i), L, params, cnt)
        k = _rng(seed, 101 + 4 * i).standard_normal((h_kv, L, d), dtype=np.float32)
        v = _rng(seed, 102 + 4 * i).standard_normal((h_kv, L, d), dtype=np.float32)
        _plant(k, pl, u, beta, params.block_size)
        ks.append(_to_dtype(k, dtype))
        vs.append(_to_dtype(v, dtype))
        planted.append(pl)
    return DecodeCase(name, dtype, _to_dtype(qs, dtype), ks, vs, seqlens, params,
                      planted)


def random_tree(rng, n_draft: int, max_depth: int):
    """Parent array (parent[0] = -1; parent[i] < i, depth <= max_depth) and
    the LSB-first uint64 ancestor mask (self bit included)."""
    assert 1 <= n_draft <= 64
    parents = np.full(n_draft, -1, dtype=np.int32)
    depth = np.zeros(n_draft, dtype=np.int64)
    depth[0] = 1
    for i in range(1, n_draft):
        cand = np.nonzero(depth[:i] < max_depth)[0]
        parents[i] = int(rng.choice(cand))
        depth[i] = depth[parents[i]] + 1
    mask = np.zeros(n_draft, dtype=np.uint64)
    for i in range(n_draft):
        m = np.uint64(1) << np.uint64(i)
        if parents[i] >= 0:
            m |= mask[parents[i]]
        mask[i] = m
    return parents, mask


def make_tree(seed: int, n_ctx: int, n_draft: int, h_q: int, h_kv: int, d: int,
              params: Params, dtype: str, n_planted: int, alpha: float = 1.5,
              beta: float = 1.5, max_depth: int = 6, parents=None,
              name: str = "tree") -> TreeCase:
    u = _unit(_rng(seed, 3), d)
    planted = _pick_planted(_rng(seed, 4), n_ctx, params, n_planted)
    k = _rng(seed, 1).standard_normal((h_kv, n_ctx, d), dtype=np.float32)
    v = _rng(seed, 2).standard_normal((h_kv, n_ctx, d), dtype=np.float32)
    _plant(k, planted, u, beta, params.block_size)
    q = _rng(seed, 0).standard_normal((n_draft, h_q, d), dtype=np.float32)
    q += alpha * u
    kd = _rng(seed, 5).standard_normal((h_kv, n_draft, d), dtype=np.float32)
    vd = _rng(seed, 6).standard_normal((h_kv, n_draft, d), dtype=np.float32)
    if parents is None:
        parents, mask = random_tree(_rng(seed, 7), n_draft, max_depth)
    else:
        parents = np.asarray(parents, dtype=np.int32)
        mask = np.zeros(n_draft, dtype=np.uint64)
        for i in range(n_draft):
            m = np.uint64(1) << np.uint64(i)
            if parents[i] >= 0:
                m |= mask[parents[i]]
            mask[i] = m
    return TreeCase(name, dtype, _to_dtype(q, dtype), _to_dtype(k, dtype),
                    _to_dtype(v, dtype), _to_dtype(kd, dtype), _to_dtype(vd, dtype),
                    parents, mask, params, planted)


CONFIG_NAMES = {
    0: "tiny_prefill_f32_n2048",
    1: "decode_bf16_32k",
    2: "sparse_prefill_bf16_128k_chunk8192",
    3: "tree_verify_bf16_128k_16drafts",
    4: "ragged_decode_bf16_8seq",
}


def config(cfg: int, seed: int = 0, **over):
    """The five standard workloads.  Keyword overrides shrink them for tests
    (e.g. n_k, n_q, seqlens, n_ctx)."""
    if cfg == 0:
        p = Params(block_size=64, kernel_size=32, kernel_stride=16, topk=8,
                   init_blocks=1, local_blocks=2, dense_len=0)
        n = over.get("n_k", 2048)
        return make_prefill(seed, n_k=n, n_q=over.get("n_q", n), h_q=2, h_kv=1,
                            d=64, params=p, dtype="f32", n_planted=4, alpha=2.0,
                            beta=2.0, name=CONFIG_NAMES[0])
    if cfg == 1:
        p = Params()
        L = over.get("seqlen", 32768)
        return make_decode(seed + 1, [L], h_q=32, h_kv=2, d=128, params=p,
                           dtype="bf16", n_planted=over.get("n_planted", 16),
                           name=CONFIG_NAMES[1])
    if cfg == 2:
        p = over.get("params", Params())
        n_k = over.get("n_k", 131072)
        n_q = over.get("n_q", 8192)
        return make_prefill(seed + 2, n_k=n_k, n_q=n_q, h_q=32, h_kv=2, d=128,
                            params=p, dtype="bf16",
                            n_planted=over.get("n_planted", 64), alpha=1.5,
                            beta=1.5, name=CONFIG_NAMES[2])
    if cfg == 3:
        p = Params()
        n_ctx = over.get("n_ctx", 131072)
        return make_tree(seed + 3, n_ctx=n_ctx, n_draft=over.get("n_draft", 16),
                         h_q=32, h_kv=2, d=128, params=p, dtype="bf16",
                         n_planted=over.get("n_planted", max(1, n_ctx // 2048)),
                         name=CONFIG_NAMES[3])
    if cfg == 4:
        p = Params()
        if "seqlens" in over:
            lens = np.asarray(over["seqlens"], dtype=np.int32)
        else:
            lo, hi = over.get("len_range", (4096, 131072))
            lens = _rng(seed + 4, 9).integers(lo, hi, size=over.get("batch", 8),
                                              endpoint=True).astype(np.int32)
        return make_decode(seed + 4, lens, h_q=32, h_kv=2, d=128, params=p,
                           dtype="bf16", planted_per_token=1.0 / 2048,
                           name=CONFIG_NAMES[4])
    raise ValueError(f"unknown workload {cfg}")
