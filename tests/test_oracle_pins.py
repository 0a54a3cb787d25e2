"""Pins for the CPU oracle against facts fixed outside the oracle itself:
closed forms, hand-worked values, brute-force enumeration on tiny inputs and
library routines (torch's bfloat16 conversion, torch's scaled-dot-product
attention in float64).  All CPU."""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_long_infllmv2_amd.workloads import Params, make_prefill, \
    make_decode, make_tree

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- bf16 ----
def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) *
         np.exp2(rng.integers(-140, 120, 200000))).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1.0, 65504.0, 3.0e38, 1e-40])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_round(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_round_ties_and_no_double_rounding():
    # halfway between 1 and 1+2^-7: ties to the even mantissa (1.0)
    assert O.bf16_round(1.0 + 2.0 ** -8) == 1.0
    # halfway between 1+2^-7 (odd) and 1+2^-6 (even): goes up
    assert O.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    # just above halfway (by less than a float32 ulp): must round up; a
    # float64 -> float32 -> bfloat16 path would wrongly give 1.0
    assert O.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert O.bf16_round(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == -(1.0 + 2.0 ** -7)


# ------------------------------------------------------------- windows ----
def test_num_windows_counts():
    assert O.num_windows(31, 32, 16) == 0
    assert O.num_windows(32, 32, 16) == 1
    assert O.num_windows(47, 32, 16) == 1
    assert O.num_windows(48, 32, 16) == 2
    assert O.num_windows(256, 32, 16) == 15
    assert O.num_windows(131072, 32, 16) == 8191


def test_compress_constant_and_ramp_closed_forms():
    p = Params()
    k = np.full((2, 200, 8), 0.375)
    ck = O.compress_keys(k, p, "f32")
    assert ck.shape == (2, 11, 8)
    assert np.all(ck == 0.375)
    # ramp: K[t] = t * e  ->  mean over [16m, 16m+32) = (16m + 15.5) * e
    t = np.arange(200, dtype=np.float64)
    e = np.array([1.0, -2.0, 0.5, 4.0])
    k = (t[:, None] * e[None, :])[None]
    ck = O.compress_keys(k, p, "f32")
    for m in range(ck.shape[1]):
        np.testing.assert_array_equal(ck[0, m], (16 * m + 15.5) * e)


def test_compress_one_hot_token_lands_in_its_windows():
    p = Params()
    for tok in [0, 15, 16, 31, 32, 100, 127]:
        k = np.zeros((1, 128, 2))
        k[0, tok, 0] = 32.0
        ck = O.compress_keys(k, p, "f32")
        for m in range(ck.shape[1]):
            inside = 16 * m <= tok < 16 * m + 32
            assert ck[0, m, 0] == (1.0 if inside else 0.0), (tok, m)
            assert ck[0, m, 1] == 0.0


def test_compress_rounds_to_bf16_storage():
    # mean = 1 + 2^-8 + 2^-10: above the tie -> rounds up to 1 + 2^-7
    k = np.ones((1, 32, 1))
    k[0, 0, 0] += 32 * (2.0 ** -8 + 2.0 ** -10)
    assert O.compress_keys(k, Params(), "bf16")[0, 0, 0] == 1.0 + 2.0 ** -7
    assert O.compress_keys(k, Params(), "f32")[0, 0, 0] == np.float32(
        1.0 + 2.0 ** -8 + 2.0 ** -10)


def test_windows_of_block_golden():
    rows = [list(map(int, ln.split())) for ln in open(
        os.path.join(GOLDEN, "window_block_overlap.txt")) if ln.strip()
        and not ln.startswith("#")]
    p = Params()
    n_c = O.num_windows(256, 32, 16)
    assert n_c == 15
    for b, lo, hi, first_pos in rows:
        r = O.windows_of_block(b, p, n_c)
        assert (r.start, r.stop - 1) == (lo, hi)
        # first position from which a window of this block is visible
        k = np.zeros((1, 256, 1))
        sig = lambda pos: O.kernel_scores(np.ones((1, 1)), np.ones((1, n_c, 1)),
                                          pos, p, 1)
        S = O.block_scores(sig(first_pos), first_pos, p)
        assert np.isfinite(S[0, b])
        if first_pos - 1 >= b * 64:
            S = O.block_scores(sig(first_pos - 1), first_pos - 1, p)
            assert S[0, b] == -np.inf


@pytest.mark.parametrize("B,ks,s", [(64, 32, 16), (128, 32, 16), (64, 48, 16),
                                    (64, 16, 16), (32, 32, 8), (16, 32, 16)])
def test_windows_of_block_brute_force(B, ks, s):
    p = Params(block_size=B, kernel_size=ks, kernel_stride=s)
    n_k = 700
    n_c = O.num_windows(n_k, ks, s)
    for b in range(-(-n_k // B)):
        blk = set(range(b * B, min((b + 1) * B, n_k)))
        want = [m for m in range(n_c) if blk & set(range(m * s, m * s + ks))]
        assert list(O.windows_of_block(b, p, n_c)) == want


# -------------------------------------------------------------- scores ----
def test_kernel_scores_group_sum_and_scale_by_hand():
    # h_q=4, h_kv=2: heads 0,1 -> group 0; heads 2,3 -> group 1.
    p = Params(scale=0.5)
    q = np.array([[1.0, 0.0], [2.0, 1.0], [0.0, 3.0], [1.0, -1.0]])
    ck = np.array([[[1.0, 2.0], [3.0, -1.0]],        # group 0, windows 0,1
                   [[2.0, 2.0], [-1.0, 4.0]]])       # group 1
    sig = O.kernel_scores(q, ck, pos=100, params=p, h_kv=2)
    # group 0: qsum = (3, 1); group 1: qsum = (1, 2)
    np.testing.assert_array_equal(sig, [[0.5 * 5, 0.5 * 8], [0.5 * 6, 0.5 * 7]])
    # position 40: window 1 = tokens [16, 48) ends at 47 > 40 -> invisible
    sig = O.kernel_scores(q, ck, pos=40, params=p, h_kv=2)
    assert sig[0, 1] == -np.inf and sig[1, 1] == -np.inf
    assert sig[0, 0] == 2.5


def test_score_mode1_by_hand():
    # the same two groups as above, each head's softmax over the two windows
    p = Params(scale=0.5, score_mode=1)
    q = np.array([[1.0, 0.0], [2.0, 1.0], [0.0, 3.0], [1.0, -1.0]])
    ck = np.array([[[1.0, 2.0], [3.0, -1.0]],
                   [[2.0, 2.0], [-1.0, 4.0]]])
    sig = O.kernel_scores(q, ck, pos=100, params=p, h_kv=2)
    # group 0: head 0 logits (0.5, 1.5), head 1 logits (2.0, 2.5)
    e1, eh = math.e, math.exp(0.5)
    g0 = [1 / (1 + e1) + 1 / (1 + eh), e1 / (1 + e1) + eh / (1 + eh)]
    # group 1: head 2 logits (3.0, 6.0), head 3 logits (0.0, -2.5)
    e3, e25 = math.exp(3.0), math.exp(2.5)
    g1 = [1 / (1 + e3) + e25 / (1 + e25), e3 / (1 + e3) + 1 / (1 + e25)]
    np.testing.assert_allclose(sig, [g0, g1], rtol=1e-14)
    # only window 0 visible at position 40: each head gives it all of its share
    sig = O.kernel_scores(q, ck, pos=40, params=p, h_kv=2)
    np.testing.assert_allclose(sig[:, 0], [2.0, 2.0], rtol=1e-15)
    assert sig[0, 1] == -np.inf and sig[1, 1] == -np.inf


@pytest.mark.parametrize("h_q,h_kv", [(2, 1), (32, 2), (8, 8)])
def test_score_mode1_shares_sum_to_group_size(h_q, h_kv):
    rng = np.random.default_rng(7)
    d, n_c = 16, 50
    q = rng.standard_normal((h_q, d)) * 3
    ck = rng.standard_normal((h_kv, n_c, d))
    p = Params(score_mode=1)
    for pos in (31, 300, 815):
        sig = O.kernel_scores(q, ck, pos, p, h_kv)
        vis = np.isfinite(sig[0])
        assert vis.sum() == O.num_windows(pos + 1, 32, 16)
        np.testing.assert_allclose(sig[:, vis].sum(axis=1), h_q // h_kv, rtol=1e-12)
        assert np.all(sig[:, vis] > 0)


def test_score_mode1_uniform_when_kernels_are_identical():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((32, 16))
    ck = np.broadcast_to(rng.standard_normal((2, 1, 16)), (2, 40, 16)).copy()
    sig = O.kernel_scores(q, ck, 500, Params(score_mode=1), 2)
    n_vis = O.num_windows(501, 32, 16)
    np.testing.assert_allclose(sig[:, :n_vis], 16.0 / n_vis, rtol=1e-13)


def test_score_mode1_single_head_per_group_selects_as_mode0():
    # one query head per group: each group's mode-1 score is an increasing
    # function of its mode-0 score, so block maxima and selections agree
    rng = np.random.default_rng(9)
    h, d, n_k = 4, 16, 3000
    p0, p1 = Params(topk=8), Params(topk=8, score_mode=1)
    ck = rng.standard_normal((h, O.num_windows(n_k, 32, 16), d))
    for pos in (700, 1500, 2999):
        q = rng.standard_normal((h, d)) * 2
        s0 = O.block_scores(O.kernel_scores(q, ck, pos, p0, h), pos, p0)
        s1 = O.block_scores(O.kernel_scores(q, ck, pos, p1, h), pos, p1)
        for g in range(h):
            assert np.array_equal(O.select_blocks(s0[g], pos, p0),
                                  O.select_blocks(s1[g], pos, p1))


def test_block_scores_are_overlap_max_brute_force():
    rng = np.random.default_rng(3)
    p = Params()
    n_k = 600
    n_c = O.num_windows(n_k, 32, 16)
    sigma = rng.standard_normal((2, n_c))
    for pos in [0, 30, 31, 100, 255, 256, 599]:
        sig = sigma.copy()
        for m in range(n_c):
            if m * 16 + 31 > pos:
                sig[:, m] = -np.inf
        S = O.block_scores(sig, pos, p)
        assert S.shape == (2, pos // 64 + 1)
        for b in range(pos // 64 + 1):
            toks = set(range(64 * b, 64 * b + 64))
            ms = [m for m in range(n_c) if toks & set(range(16 * m, 16 * m + 32))
                  and 16 * m + 31 <= pos]
            for g in range(2):
                want = max(sigma[g, ms]) if ms else -np.inf
                assert S[g, b] == want


# ----------------------------------------------------------- selection ----
def _brute_select(S_g, pos, p):
    """Exhaustive: keep init + local blocks, then the subset of the rest of
    the right size with the largest total score (exact integer scores);
    among equal totals the lexicographically smallest sorted tuple."""
    n_elig = pos // p.block_size + 1
    b_own = pos // p.block_size
    forced = {b for b in range(n_elig) if b < p.init_blocks or
              b_own - p.local_blocks < b <= b_own}
    rest = [b for b in range(n_elig) if b not in forced]
    need = max(0, min(p.topk, n_elig) - len(forced))
    best = None
    for combo in itertools.combinations(rest, need):
        total = sum(int(S_g[b]) for b in combo)
        key = (-total, tuple(sorted(set(combo) | forced)))
        if best is None or key < best:
            best = key
    return list(best[1])


def test_select_matches_brute_force_with_ties():
    rng = np.random.default_rng(7)
    for trial in range(300):
        B = 16
        n_b = int(rng.integers(1, 13))
        pos = int(rng.integers((n_b - 1) * B, n_b * B))
        p = Params(block_size=B, topk=int(rng.integers(2, 9)),
                   init_blocks=int(rng.integers(0, 2)),
                   local_blocks=int(rng.integers(0, 3)))
        if p.topk < p.init_blocks + p.local_blocks:
            continue
        S = rng.integers(-3, 4, size=n_b).astype(np.float64)   # many ties
        S[rng.random(n_b) < 0.15] = -1e6                       # "no window"
        got = list(O.select_blocks(S, pos, p))
        assert got == _brute_select(S, pos, p), (trial, S, pos, p)


def test_select_invariants_forced_and_count():
    rng = np.random.default_rng(8)
    p = Params(topk=8)
    for pos in [0, 5, 63, 64, 200, 511, 512, 4000]:
        S = rng.standard_normal(pos // 64 + 1)
        S[0] = -np.inf
        sel = O.select_blocks(S, pos, p)
        n_elig = pos // 64 + 1
        assert len(sel) == min(8, n_elig)
        assert list(sel) == sorted(set(sel))
        b_own = pos // 64
        assert 0 in sel and b_own in sel
        if b_own >= 1:
            assert b_own - 1 in sel


# ----------------------------------------------------------- attention ----
def _sdpa(q, keys, vals, mask, scale):
    """torch scaled-dot-product attention in float64 on the CPU."""
    q = torch.from_numpy(np.asarray(q, np.float64))[None, None]
    k = torch.from_numpy(np.asarray(keys, np.float64))[None, None]
    v = torch.from_numpy(np.asarray(vals, np.float64))[None, None]
    m = torch.from_numpy(np.asarray(mask, bool))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=m, scale=scale)[0, 0].numpy()


def _dense_ref(q, k, v, p):
    n_q, h_q, d = q.shape
    h_kv, n_k, _ = k.shape
    out = np.zeros((n_q, h_q, d))
    pos = n_k - n_q + np.arange(n_q)
    mask = np.arange(n_k)[None, :] <= pos[:, None]
    for h in range(h_q):
        g = h * h_kv // h_q
        out[:, h] = _sdpa(q[:, h], k[g], v[g], mask, 1 / math.sqrt(d))
    return out


def test_sparse_equals_dense_when_topk_covers_every_block():
    p = Params(topk=16, dense_len=0)
    c = make_prefill(11, n_k=640, n_q=200, h_q=4, h_kv=2, d=16, params=p,
                     dtype="f32", n_planted=2, alpha=1.0, beta=1.0)
    r = O.prefill(c.q, c.k, c.v, p, "f32")
    assert not r["dense"]
    ref = _dense_ref(c.q.astype(np.float64), c.k.astype(np.float64),
                     c.v.astype(np.float64), p)
    got = np.stack([r["o"][i] for i in range(c.n_q)])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_dense_len_threshold():
    p = Params(topk=3, dense_len=640)
    for n_k, dense in [(639, True), (640, False)]:
        c = make_prefill(12, n_k=n_k, n_q=64, h_q=2, h_kv=1, d=8, params=p,
                         dtype="f32", n_planted=1, alpha=0.0, beta=0.0)
        r = O.prefill(c.q, c.k, c.v, p, "f32")
        assert r["dense"] == dense
        ref = _dense_ref(c.q.astype(np.float64), c.k.astype(np.float64),
                         c.v.astype(np.float64), p)
        got = np.stack([r["o"][i] for i in range(c.n_q)])
        err = np.abs(got - ref).max()
        if dense:
            assert err < 1e-12
        else:
            assert err > 1e-3      # 3 of 10 blocks kept: must differ


def test_softmax_rows_sum_to_one_and_key_count_by_hand():
    # q = 0: every logit is 0, so lse = ln(#keys attended) exactly.
    # pos 300, B 64, topk 3, init 1, local 2: blocks {0, 3, 4}; block 4 holds
    # tokens 256..300 -> 64 + 64 + 45 = 173 keys.
    p = Params(topk=3, dense_len=0)
    n_k = 301
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, n_k, 8))
    v = np.ones((1, n_k, 8))
    q = np.zeros((1, 2, 8))
    r = O.prefill(q, k, v, p, "f32")
    assert list(r["sel"][0][0]) == [0, 3, 4]
    np.testing.assert_allclose(r["lse"][0], [math.log(173)] * 2, atol=1e-13)
    np.testing.assert_allclose(r["o"][0], 1.0, atol=1e-12)
    # random q, v = ones: rows still sum to one
    q = rng.standard_normal((5, 2, 8))
    r = O.prefill(q, k, v, p, "f32")
    for i in range(5):
        np.testing.assert_allclose(r["o"][i], 1.0, atol=1e-12)


def test_sparse_attention_matches_sdpa_on_selected_keys():
    p = Params(topk=4, dense_len=0)
    c = make_prefill(13, n_k=1000, n_q=40, h_q=4, h_kv=2, d=16, params=p,
                     dtype="f32", n_planted=3, alpha=2.0, beta=2.0)
    r = O.prefill(c.q, c.k, c.v, p, "f32")
    q = c.q.astype(np.float64); k = c.k.astype(np.float64)
    v = c.v.astype(np.float64)
    for i in range(c.n_q):
        pos = c.n_k - c.n_q + i
        for h in range(4):
            g = h // 2
            sel = r["sel"][i][g]
            mask = np.zeros((1, c.n_k), bool)
            for b in sel:
                mask[0, b * 64:(b + 1) * 64] = True
            mask[0, pos + 1:] = False
            ref = _sdpa(q[i, h][None], k[g], v[g], mask, 0.25)[0]
            np.testing.assert_allclose(r["o"][i][h], ref, atol=1e-12)


def test_planted_blocks_are_selected():
    c = make_prefill(0, n_k=2048, n_q=64, h_q=2, h_kv=1, d=64,
                     params=Params(topk=8, dense_len=0), dtype="f32",
                     n_planted=4, alpha=4.0, beta=4.0)
    r = O.prefill(c.q, c.k, c.v, c.params, "f32", rows=[63])
    assert set(c.planted) <= set(r["sel"][63][0])


def test_decode_equals_last_prefill_row():
    p = Params(topk=4, dense_len=512)
    c = make_prefill(14, n_k=777, n_q=3, h_q=4, h_kv=2, d=16, params=p,
                     dtype="bf16", n_planted=2, alpha=1.5, beta=1.5)
    r = O.prefill(c.q, c.k, c.v, p, "bf16")
    d = O.decode(c.q[-1:], [c.k], [c.v], [777], p, "bf16")
    np.testing.assert_array_equal(d["o"][0], r["o"][2])
    np.testing.assert_array_equal(d["sel"][0][0], r["sel"][2][0])


def test_ragged_decode_each_sequence_independent():
    p = Params(topk=4, dense_len=600)
    c = make_decode(15, [300, 700, 1025], h_q=4, h_kv=2, d=16, params=p,
                    dtype="bf16", n_planted=2)
    r = O.decode(c.q, c.k, c.v, c.seqlens, p, "bf16")
    assert r["dense"] == [True, False, False]
    for i in range(3):
        one = O.decode(c.q[i:i + 1], [c.k[i]], [c.v[i]], [c.seqlens[i]], p, "bf16")
        np.testing.assert_array_equal(one["o"][0], r["o"][i])


# ---------------------------------------------------------------- tree ----
def test_tree_chain_equals_causal_over_selected_context_and_prefix():
    p = Params(topk=4, dense_len=0)
    T = 5
    c = make_tree(16, n_ctx=900, n_draft=T, h_q=4, h_kv=2, d=16, params=p,
                  dtype="f32", n_planted=3, parents=[-1, 0, 1, 2, 3])
    r = O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, c.mask, p, "f32")
    q = c.q.astype(np.float64)
    keys = np.concatenate([c.k, c.k_draft], axis=1).astype(np.float64)
    vals = np.concatenate([c.v, c.v_draft], axis=1).astype(np.float64)
    for i in range(T):
        for h in range(4):
            g = h // 2
            mask = np.zeros((1, 900 + T), bool)
            for b in r["sel"][i][g]:
                mask[0, b * 64:min((b + 1) * 64, 900)] = True
            mask[0, 900:900 + i + 1] = True             # drafts 0..i
            ref = _sdpa(q[i, h][None], keys[g], vals[g], mask, 0.25)[0]
            np.testing.assert_allclose(r["o"][i][h], ref, atol=1e-12)


def test_tree_non_ancestor_drafts_do_not_matter_and_self_only():
    p = Params(topk=4, dense_len=0)
    T = 6
    c = make_tree(17, n_ctx=700, n_draft=T, h_q=4, h_kv=2, d=16, params=p,
                  dtype="f32", n_planted=2, parents=[-1, 0, 0, 1, 1, 2])
    r = O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, c.mask, p, "f32")
    rng = np.random.default_rng(0)
    for i in range(T):
        anc = [j for j in range(T) if (int(c.mask[i]) >> j) & 1]
        other = [j for j in range(T) if j not in anc]
        kd = c.k_draft.copy(); vd = c.v_draft.copy()
        kd[:, other] = rng.standard_normal(kd[:, other].shape)
        vd[:, other] = rng.standard_normal(vd[:, other].shape)
        r2 = O.tree_verify(c.q, c.k, c.v, kd, vd, c.mask, p, "f32", drafts=[i])
        np.testing.assert_array_equal(r2["o"][i], r["o"][i])
    # self-only mask: context keys plus the draft itself
    selfmask = np.array([1 << i for i in range(T)], dtype=np.uint64)
    r3 = O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, selfmask, p, "f32")
    assert int(c.mask[3]) == 0b1011
    for i in range(T):
        assert list(r3["sel"][i][0]) == list(r["sel"][i][0])
    np.testing.assert_array_equal(r3["o"][0], r["o"][0])  # root: same keys
    assert np.abs(r3["o"][3] - r["o"][3]).max() > 1e-6


def test_tree_dense_chain_equals_causal_prefill_of_context_plus_drafts():
    # context shorter than dense_len: with chain parents (draft i's ancestors
    # are drafts 0..i) the drafts are just the next T tokens of one sequence,
    # so draft i's output is row n_ctx+i of dense causal attention over the
    # n_ctx+T tokens (torch SDPA with is_causal, float64)
    p = Params(topk=4, dense_len=4096)
    T, n_ctx, h_q, h_kv, d = 5, 700, 4, 2, 16
    c = make_tree(18, n_ctx=n_ctx, n_draft=T, h_q=h_q, h_kv=h_kv, d=d, params=p,
                  dtype="f32", n_planted=2, parents=[-1, 0, 1, 2, 3])
    r = O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, c.mask, p, "f32")
    assert r["dense"] and not r["sel"]
    keys = torch.from_numpy(np.concatenate([c.k, c.k_draft], axis=1).astype(np.float64))
    vals = torch.from_numpy(np.concatenate([c.v, c.v_draft], axis=1).astype(np.float64))
    n = n_ctx + T
    for h in range(h_q):
        g = h * h_kv // h_q
        # queries of the whole sequence: the drafts' own at the last T rows
        qq = torch.zeros((n, d), dtype=torch.float64)
        qq[n_ctx:] = torch.from_numpy(c.q[:, h].astype(np.float64))
        o = torch.nn.functional.scaled_dot_product_attention(
            qq[None, None], keys[g][None, None], vals[g][None, None],
            is_causal=True, scale=0.25)[0, 0].numpy()
        logits = 0.25 * (qq[n_ctx:] @ keys[g].T)
        causal = torch.arange(n)[None, :] <= (n_ctx + torch.arange(T))[:, None]
        lse = torch.logsumexp(logits.masked_fill(~causal, -math.inf), dim=1).numpy()
        for i in range(T):
            np.testing.assert_allclose(r["o"][i][h], o[n_ctx + i], atol=1e-12)
            np.testing.assert_allclose(r["lse"][i][h], lse[i], atol=1e-12)


def test_tree_dense_self_only_equals_sdpa_over_context_and_self():
    p = Params(topk=4, dense_len=4096)
    T, n_ctx = 4, 300
    c = make_tree(19, n_ctx=n_ctx, n_draft=T, h_q=2, h_kv=1, d=8, params=p,
                  dtype="f32", n_planted=1)
    selfmask = np.array([1 << i for i in range(T)], dtype=np.uint64)
    r = O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, selfmask, p, "f32")
    keys = np.concatenate([c.k, c.k_draft], axis=1)
    vals = np.concatenate([c.v, c.v_draft], axis=1)
    for i in range(T):
        mask = np.zeros((1, n_ctx + T), bool)
        mask[0, :n_ctx] = True
        mask[0, n_ctx + i] = True
        for h in range(2):
            ref = _sdpa(c.q[i, h][None], keys[0], vals[0], mask, 1 / math.sqrt(8))[0]
            np.testing.assert_allclose(r["o"][i][h], ref, atol=1e-12)


@pytest.mark.parametrize("dense_len", [0, 4096])
def test_tree_self_bit_always_honoured_and_high_bits_ignored(dense_len):
    # a draft attends itself whether or not its own bit is set, and mask bits
    # at or above the draft count name no draft
    p = Params(topk=4, dense_len=dense_len)
    T = 6
    c = make_tree(20, n_ctx=800, n_draft=T, h_q=4, h_kv=2, d=16, params=p,
                  dtype="f32", n_planted=2, parents=[-1, 0, 0, 1, 3, 2])
    r = O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, c.mask, p, "f32")
    odd = c.mask.copy()
    for i in range(T):
        odd[i] = np.uint64(int(odd[i]) & ~(1 << i)) | (np.uint64(1) << np.uint64(63 - i))
    assert all(not (int(odd[i]) >> i) & 1 for i in range(T))
    r2 = O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, odd, p, "f32")
    for i in range(T):
        np.testing.assert_array_equal(r2["o"][i], r["o"][i])
        np.testing.assert_array_equal(r2["lse"][i], r["lse"][i])
    # an all-zero mask is the self-only mask
    zero = np.zeros(T, dtype=np.uint64)
    selfmask = np.array([1 << i for i in range(T)], dtype=np.uint64)
    r3 = O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, zero, p, "f32")
    r4 = O.tree_verify(c.q, c.k, c.v, c.k_draft, c.v_draft, selfmask, p, "f32")
    for i in range(T):
        np.testing.assert_array_equal(r3["o"][i], r4["o"][i])
    # dropping a real ancestor changes the output (the pin can see a draft)
    assert np.abs(r4["o"][4] - r["o"][4]).max() > 1e-6


# ----------------------------------------------------- backward (training) ----
def _torch_selected_grads(q, k, v, sel_rows, p, d_out):
    """torch autograd (float64) of the same attention, row by row."""
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    n_q, h_q, d = q.shape
    h_kv, n_k, _ = k.shape
    scale = 1.0 / math.sqrt(d)
    loss = 0.0
    for i in range(n_q):
        pos = n_k - n_q + i
        for h in range(h_q):
            g = h * h_kv // h_q
            if sel_rows[i] is None:
                toks = list(range(pos + 1))
            else:
                toks = [t for b in sel_rows[i][g] for t in range(b * p.block_size,
                                                                 (b + 1) * p.block_size)
                        if t <= pos]
            idx = torch.tensor(toks)
            w = torch.softmax(scale * (kt[g, idx] @ qt[i, h]), dim=0)
            o = w @ vt[g, idx]
            loss = loss + (o * torch.tensor(d_out[i, h])).sum()
    loss.backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def test_prefill_backward_matches_torch_autograd():
    rng = np.random.default_rng(21)
    p = Params(block_size=16, topk=3, init_blocks=1, local_blocks=1)
    n_k, n_q, h_q, h_kv, d = 90, 40, 4, 2, 8
    q = rng.standard_normal((n_q, h_q, d))
    k = rng.standard_normal((h_kv, n_k, d))
    v = rng.standard_normal((h_kv, n_k, d))
    d_out = rng.standard_normal((n_q, h_q, d))
    sel_rows = []
    for i in range(n_q):
        pos = n_k - n_q + i
        own = pos // p.block_size
        if i % 7 == 0:
            sel_rows.append(None)                 # a dense row
        else:
            cand = [b for b in range(1, own)]
            pick = sorted(rng.choice(cand, size=min(1, len(cand)), replace=False).tolist())
            sel_rows.append([sorted({0, own} | set(pick)) for _ in range(h_kv)])
    dq, dk, dv = O.prefill_backward(q, k, v, sel_rows, p, d_out)
    tq, tk, tv = _torch_selected_grads(q, k, v, sel_rows, p, d_out)
    np.testing.assert_allclose(dq, tq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv, rtol=1e-10, atol=1e-12)


def test_attend_backward_finite_differences():
    rng = np.random.default_rng(22)
    n, d, scale = 7, 5, 0.6
    q, keys, vals, d_o = (rng.standard_normal(d), rng.standard_normal((n, d)),
                          rng.standard_normal((n, d)), rng.standard_normal(d))
    dq, dk, dv = O.attend_backward(q, keys, vals, scale, d_o)

    def loss(q_, k_, v_):
        return float(O.attend(q_, k_, v_, scale)[0] @ d_o)

    eps = 1e-6
    for arr, grad, which in ((q, dq, 0), (keys, dk, 1), (vals, dv, 2)):
        num = np.zeros_like(arr)
        for ix in np.ndindex(arr.shape):
            plus, minus = arr.copy(), arr.copy()
            plus[ix] += eps
            minus[ix] -= eps
            args_p = [q, keys, vals]
            args_m = [q, keys, vals]
            args_p[which], args_m[which] = plus, minus
            num[ix] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def test_prefill_backward_dense_equals_sdpa_backward():
    # every row dense: the gradients of causal scaled-dot-product attention
    rng = np.random.default_rng(23)
    n, h, d = 24, 2, 8
    q, k, v, d_out = (rng.standard_normal((n, h, d)), rng.standard_normal((h, n, d)),
                      rng.standard_normal((h, n, d)), rng.standard_normal((n, h, d)))
    dq, dk, dv = O.prefill_backward(q, k, v, [None] * n, Params(), d_out)
    qt = torch.tensor(q.transpose(1, 0, 2), requires_grad=True)     # [h][n][d]
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    (o * torch.tensor(d_out.transpose(1, 0, 2))).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-10, atol=1e-12)
