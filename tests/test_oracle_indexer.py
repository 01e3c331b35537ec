"""Pins for the oracle's token-level indexer (index scores, token selection,
token-gather attention).

Checked against: a different order of the same arithmetic where the ReLU is
inactive (sum the weighted heads first, one library matmul after), a closed
form where it is active (a head pair x, -x gives |x . k|), an invariant
(future tokens never change a row), the dense special case (every token
kept equals causal SDPA from torch), closed forms for one and two kept tokens
and for a repeated kept position, and brute-force subsets for the selection.
Runs on the CPU.
"""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from dynamic_block_sparse_dsa_amd.inputs import INDEX_WORKLOADS, make_index

BOTH = O.FORCE_SINK | O.FORCE_DIAG


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_scores_without_active_relu_are_one_matmul():
    """Non-negative index queries and keys make every dot product >= 0, so
    I[t, s] = (sum_h w[t, h] qi[t, h]) . ki[s]: the weighted heads summed
    first, then a single matmul."""
    B, N, HI, dI = 2, 40, 5, 12
    rng = np.random.default_rng(1)
    qi, ki, wi = np.abs(rng.standard_normal((B, N, HI, dI))), np.abs(rng.standard_normal((B, N, dI))), rng.random((B, N, HI))
    got = O.index_scores(qi, ki, wi)
    comb = torch.from_numpy(np.einsum("bth,bthd->btd", wi, qi))
    want = torch.matmul(comb, torch.from_numpy(ki).transpose(1, 2)).numpy()
    tri = np.tril(np.ones((N, N), dtype=bool))
    np.testing.assert_allclose(got[:, tri], want[:, tri], rtol=1e-12)
    assert np.isneginf(got[:, ~tri]).all()


def test_relu_closed_form_absolute_value():
    """Two heads with queries x and -x and unit weights: max(0, a) + max(0, -a)
    = |a|, so I[t, s] = |x . k_s|; a third head with zero weight adds nothing."""
    N, dI = 30, 8
    rng = np.random.default_rng(2)
    x = rng.standard_normal((N, dI))
    qi = np.stack([x, -x, rng.standard_normal((N, dI))], axis=1)[None]
    ki = rng.standard_normal((1, N, dI))
    wi = np.tile([1.0, 1.0, 0.0], (1, N, 1))
    got = O.index_scores(qi, ki, wi)
    for t in range(N):
        np.testing.assert_allclose(got[0, t, : t + 1], np.abs(ki[0, : t + 1] @ x[t]), rtol=1e-12, atol=1e-14)


def test_scores_do_not_see_future_tokens():
    B, N, HI, dI = 1, 24, 4, 6
    qi, ki, wi = rnd((B, N, HI, dI), 3), rnd((B, N, dI), 4), np.random.default_rng(5).random((B, N, HI))
    base = O.index_scores(qi, ki, wi)
    for t in (0, 5, 23):
        k2 = ki.copy()
        k2[:, t + 1 :] = 1e6
        np.testing.assert_array_equal(O.index_scores(qi, k2, wi)[:, t], base[:, t])


def test_positive_weight_scaling_keeps_the_selection():
    B, N, HI, dI = 1, 50, 4, 8
    qi, ki, wi = rnd((B, N, HI, dI), 6), rnd((B, N, dI), 7), np.random.default_rng(8).random((B, N, HI))
    a = O.select_tokens(O.index_scores(qi, ki, wi), 6)[0]
    b = O.select_tokens(O.index_scores(qi, ki, 4.0 * wi), 6)[0]
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("Hq,Hkv,N,d", [(2, 2, 37, 16), (4, 1, 64, 8), (6, 2, 20, 32)])
def test_every_token_kept_is_dense_causal_attention(Hq, Hkv, N, d):
    q, k, v = rnd((1, Hq, N, d), 9), rnd((1, Hkv, N, d), 10), rnd((1, Hkv, N, d), 11)
    qi, ki, wi = rnd((1, N, 3, 4), 12), rnd((1, N, 4), 13), np.random.default_rng(14).random((1, N, 3))
    r = O.index_prefill(qi, ki, wi, q, k, v, topk=N)
    assert (r["cnt"][0] == np.arange(1, N + 1)).all()
    G = Hq // Hkv
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k).repeat_interleave(G, 1), torch.from_numpy(v).repeat_interleave(G, 1),
        is_causal=True).numpy()
    np.testing.assert_allclose(r["o"], ref, rtol=1e-11, atol=1e-12)


def test_one_and_two_kept_tokens_closed_forms():
    """Self only: O = v_t, LSE = q . k_t / sqrt(d).  Sink + self: the
    two-way softmax written out."""
    N, d = 12, 8
    q, k, v = rnd((1, 2, N, d), 15), rnd((1, 1, N, d), 16), rnd((1, 1, N, d), 17)
    qi, ki, wi = rnd((1, N, 2, 4), 18), rnd((1, N, 4), 19), np.random.default_rng(20).random((1, N, 2))
    r = O.index_prefill(qi, ki, wi, q, k, v, topk=1, flags=O.FORCE_DIAG)
    s = 1.0 / math.sqrt(d)
    for h in range(2):
        for t in range(N):
            np.testing.assert_allclose(r["o"][0, h, t], v[0, 0, t], rtol=1e-13)
            assert r["lse"][0, h, t] == pytest.approx(s * q[0, h, t] @ k[0, 0, t], rel=1e-12)
    r = O.index_prefill(qi, ki, wi, q, k, v, topk=2, flags=BOTH)
    for t in range(1, N):
        a, b = s * q[0, 1, t] @ k[0, 0, 0], s * q[0, 1, t] @ k[0, 0, t]
        w0 = 1.0 / (1.0 + math.exp(b - a))
        np.testing.assert_allclose(r["o"][0, 1, t], w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, t], rtol=1e-11)


def test_token_selection_is_the_best_subset():
    """Brute force over all subsets of the earlier tokens on a tiny problem."""
    N = 9
    qi, ki, wi = rnd((1, N, 3, 4), 21), rnd((1, N, 4), 22), np.random.default_rng(23).random((1, N, 3))
    sc = O.index_scores(qi, ki, wi)
    idx, cnt, _ = O.select_tokens(sc, 4, BOTH)
    for t in range(N):
        forced = sorted({0, t})
        cand = [s for s in range(t + 1) if s not in forced]
        m = min(max(4, len(forced)), t + 1) - len(forced)
        best = max(itertools.combinations(cand, m), key=lambda sub: (sum(Fraction(sc[0, t, s]) for s in sub),
                                                                      [-s for s in sub]))
        assert list(idx[0, t, : cnt[0, t]]) == sorted(set(forced) | set(best))


def test_planted_clusters_are_found():
    """On the tiny workload the tokens of a query token's target cluster rank
    high: most of the kept tokens of late rows share one cluster direction
    with the query (checked through the index keys' alignment)."""
    w = INDEX_WORKLOADS["index_tiny_n512"]
    qi, ki, wi, q, k, v = make_index(w)
    f = lambda x: x.float().numpy().astype(np.float64)
    qi, ki = f(qi), f(ki)
    sc = O.index_scores(qi, ki, wi.numpy().astype(np.float64))
    idx, cnt, _ = O.select_tokens(sc, w.topk)
    t = w.seq_len - 1
    kept = idx[0, t, : cnt[0, t]]
    qdir = qi[0, t].mean(axis=0)
    align = ki[0, kept] @ qdir / np.linalg.norm(qdir)
    everyone = ki[0, : t + 1] @ qdir / np.linalg.norm(qdir)
    assert np.median(align) > np.percentile(everyone, 90)


def test_a_repeated_position_counts_once_per_occurrence():
    """idx rows may repeat a position: token a listed twice with token b
    weighs like a with ln 2 added to its logit, written out here:
    w_a = 2 e^A / (2 e^A + e^B), LSE = ln(2 e^A + e^B)."""
    N, d = 9, 8
    q, k, v = rnd((1, 1, N, d), 21), rnd((1, 1, N, d), 22), rnd((1, 1, N, d), 23)
    s = 1.0 / math.sqrt(d)
    t, a, b = 7, 2, 5
    idx = np.full((1, N, 3), -1, dtype=np.int32)
    cnt = np.zeros((1, N), dtype=np.int32)
    idx[0, t] = [a, b, a]
    cnt[0, t] = 3
    o, lse = O.token_attend(q, k, v, idx, cnt, units=[(0, 0, t)])
    A, B = s * q[0, 0, t] @ k[0, 0, a], s * q[0, 0, t] @ k[0, 0, b]
    Z = 2 * math.exp(A) + math.exp(B)
    np.testing.assert_allclose(o[0, 0, t], (2 * math.exp(A) * v[0, 0, a] + math.exp(B) * v[0, 0, b]) / Z, rtol=1e-12)
    assert lse[0, 0, t] == pytest.approx(math.log(Z), rel=1e-13)


def test_token_near_ties_have_an_absolute_floor():
    """Token rows flag two scores within 1e-6 of each other (a ReLU'd dot
    product within fp32 rounding of zero may be clipped on one side only):
    at the budget boundary, 5e-7 against 0 is a near tie, 5e-6 against 0 is
    not.  The block path (``select_topk`` without the floor) keeps the
    relative rule alone."""
    # query token 4 sees tokens 0..4; forced {0, 4}; topk 3 keeps one of {1, 2, 3}
    sc = np.full((1, 5, 5), -np.inf)
    sc[0, 4, :5] = [9.0, 5e-7, 0.0, 0.0, 9.0]
    for t in range(4):
        sc[0, t, : t + 1] = np.arange(t + 1, dtype=np.float64)
    _, _, rows = O.select_tokens(sc, 3)
    assert rows[4].flagged and rows[4].band == {1, 2, 3}
    _, _, rows = O.select_topk(sc[:, None], 3)
    assert not rows[4].flagged and rows[4].idx == [0, 1, 4]
    sc[0, 4, 1] = 5e-6
    _, _, rows = O.select_tokens(sc, 3)
    assert not rows[4].flagged and rows[4].idx == [0, 1, 4]
