"""Pins that tie the fp64 oracle to facts other than its own code.

Each test checks the oracle against a library routine, a brute-force
enumeration, scalar loops, a closed form, a mathematical identity or an
invariant, chosen so that a plausible slip (a dropped term, a wrong sign or
index, a transposed operand, an off-by-one in the causal rule) fails one of
them.  Runs on the CPU.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle as O
from dynamic_block_sparse_dsa_amd import work
from dynamic_block_sparse_dsa_amd.inputs import WORKLOADS, Workload, make_decode, make_prefill

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BOTH = O.FORCE_SINK | O.FORCE_DIAG


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def sdpa_causal(q, k, v):
    """Dense causal attention from torch's library routine, in fp64 on the CPU
    (K/V heads repeated for grouped-query attention)."""
    G = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True).numpy()


# ---------------------------------------------------------------- P1 dense
@pytest.mark.parametrize("B,Hq,Hkv,N,d,b", [(1, 2, 2, 256, 16, 32), (2, 4, 2, 200, 8, 64), (1, 4, 1, 130, 32, 64),
                                           (1, 1, 1, 64, 8, 64), (1, 2, 2, 1, 8, 64)])
def test_dense_when_every_block_is_kept(B, Hq, Hkv, N, d, b):
    """k >= number of blocks keeps every causal block, so the method must equal
    dense causal softmax attention (ragged N and GQA included)."""
    q, k, v = rnd((B, Hq, N, d), 1), rnd((B, Hkv, N, d), 2), rnd((B, Hkv, N, d), 3)
    nb = O.n_blocks(N, b)
    r = O.prefill(q, k, v, b, topk=nb + 3)
    assert all((r["cnt"][..., i] == i + 1).all() for i in range(nb))
    ref = sdpa_causal(q, k, v)
    np.testing.assert_allclose(r["o"], ref, rtol=1e-11, atol=1e-12)
    # LSE: log of the causal normaliser, written out with logsumexp per row
    G = Hq // Hkv
    s = 1.0 / math.sqrt(d)
    for (bi, h, p) in [(0, 0, 0), (B - 1, Hq - 1, N - 1), (0, Hq // 2, N // 2)]:
        logits = s * (k[bi, h // G, : p + 1] @ q[bi, h, p])
        m = logits.max()
        assert r["lse"][bi, h, p] == pytest.approx(m + math.log(np.exp(logits - m).sum()), rel=1e-12)


def test_dense_fraction_budget():
    """num/den = 1 keeps every visible block: dense again."""
    q, k, v = rnd((1, 2, 192, 8), 4), rnd((1, 2, 192, 8), 5), rnd((1, 2, 192, 8), 6)
    r = O.prefill(q, k, v, 32, topk=0, num=1, den=1)
    np.testing.assert_allclose(r["o"], sdpa_causal(q, k, v), rtol=1e-11, atol=1e-12)


def test_decode_dense_when_every_block_is_kept():
    S, Hq, Hkv, L, d, b = 3, 4, 2, 300, 16, 64
    q, kc, vc = rnd((S, Hq, d), 7), rnd((S, Hkv, L, d), 8), rnd((S, Hkv, L, d), 9)
    r = O.decode(q, kc, vc, b, topk=O.n_blocks(L, b))
    G = Hq // Hkv
    qt = torch.from_numpy(q)[:, :, None, :]
    kt = torch.from_numpy(kc).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(vc).repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, :, 0].numpy()
    np.testing.assert_allclose(r["o"], ref, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- P2 brute-force selection
def brute_select(scores, n_vis, k, forced):
    cand = [j for j in range(n_vis) if j not in forced]
    m = min(max(k, len(forced)), n_vis) - len(forced)
    best, best_key = None, None
    for sub in itertools.combinations(cand, m):  # combinations come out lexicographically sorted
        key = sum(Fraction(scores[j]) for j in sub)  # exact sum: no rounding can reorder subsets
        if best is None or key > best_key:
            best, best_key = sub, key
    return sorted(set(forced) | set(best))


@settings(max_examples=150, deadline=None)
@given(nb=st.integers(1, 10), k=st.integers(1, 11), flags=st.sampled_from([0, 1, 2, 3]), seed=st.integers(0, 10**6),
       ties=st.booleans())
def test_selection_is_the_best_subset(nb, k, flags, seed, ties):
    """For every row the kept set maximises the summed score among all sets of
    its size (ties: the lexicographically smallest set, i.e. lower indices)."""
    rng = np.random.default_rng(seed)
    s = rng.integers(-3, 3, size=(nb, nb)).astype(float) if ties else rng.standard_normal((nb, nb))
    sc = np.where(np.tril(np.ones((nb, nb))) > 0, s, -np.inf)[None, None]
    idx, cnt, _ = O.select_topk(sc, topk=k, flags=flags)
    for i in range(nb):
        f = O.forced_set(i + 1, flags)
        assert list(idx[0, 0, i, : cnt[0, 0, i]]) == brute_select(s[i], i + 1, k, f)
        assert (idx[0, 0, i, cnt[0, 0, i]:] == -1).all()


@settings(max_examples=60, deadline=None)
@given(nb=st.integers(2, 9), num=st.integers(1, 100), den=st.integers(1, 100), seed=st.integers(0, 10**6))
def test_fraction_budget_is_exact_ceiling(nb, num, den, seed):
    """Budget ceil(num*n/den) against exact rational arithmetic."""
    sc = np.where(np.tril(np.ones((nb, nb))) > 0, np.random.default_rng(seed).standard_normal((nb, nb)), -np.inf)
    _, cnt, _ = O.select_topk(sc[None, None], topk=0, num=num, den=den)
    for i in range(nb):
        want = math.ceil(Fraction(num * (i + 1), den))
        assert cnt[0, 0, i] == min(max(want, len(O.forced_set(i + 1, BOTH))), i + 1)


def test_fraction_budget_at_gqa_workload():
    """k_i = ceil(0.15 * (i+1)) for the 512-block GQA workload, checked against
    Fraction(15, 100); floating 0.15*n would be off at some rows."""
    for i in range(512):
        want = math.ceil(Fraction(15, 100) * (i + 1))
        assert O.row_budget(i + 1, 0, 15, 100, len(O.forced_set(i + 1, BOTH))) == min(max(want, min(2, i + 1)), i + 1)


# ---------------------------------------------------------------- P3 scalar brute-force attention
def scalar_attention_row(q, k, v, sel_blocks, b, p):
    d = len(q)
    s = 1.0 / math.sqrt(d)
    logits = []
    for c in range(k.shape[0]):
        if c // b in sel_blocks and c <= p:
            logits.append((c, s * sum(float(q[t]) * float(k[c, t]) for t in range(d))))
    mx = max(l for _, l in logits)
    z = sum(math.exp(l - mx) for _, l in logits)
    out = [0.0] * d
    for c, l in logits:
        w = math.exp(l - mx) / z
        for t in range(d):
            out[t] += w * float(v[c, t])
    return out, mx + math.log(z)


def test_attention_against_scalar_loops():
    w = WORKLOADS["prefill_tiny_n1024"]
    q, k, v = (x.double().numpy() for x in make_prefill(w))
    # a short prefix keeps the scalar loops fast: 5 blocks of 64
    q, k, v = q[:, :, :320], k[:, :, :320], v[:, :, :320]
    r = O.prefill(q, k, v, 64, topk=3)
    rows = [0, 1, 63, 64, 127, 190, 256, 319]
    for h in range(2):
        for p in rows:
            i = p // 64
            sel = set(int(j) for j in r["idx"][0, h, i, : r["cnt"][0, h, i]])
            want, lse = scalar_attention_row(q[0, h, p], k[0, h], v[0, h], sel, 64, p)
            np.testing.assert_allclose(r["o"][0, h, p], want, rtol=1e-11, atol=1e-13)
            assert r["lse"][0, h, p] == pytest.approx(lse, rel=1e-12)


# ---------------------------------------------------------------- P4 tile-mean identity
@pytest.mark.parametrize("N,b,G", [(256, 64, 1), (200, 64, 2), (96, 32, 4)])
def test_block_score_is_mean_of_tile_logits(N, b, G):
    """mean(Q tile) . mean(K tile) / sqrt(d) equals the mean of the dense
    scaled logits over the tile (bilinearity); the group score is the max over
    the group's heads; blocks after the query block are -inf."""
    d, Hkv = 16, 2
    q, k = rnd((1, Hkv * G, N, d), 10), rnd((1, Hkv, N, d), 11)
    s = 1.0 / math.sqrt(d)
    sc = O.block_scores(O.block_means(q, b), O.block_means(k, b), s)
    nb = O.n_blocks(N, b)
    for g in range(Hkv):
        for i in range(nb):
            for j in range(nb):
                if j > i:
                    assert sc[0, g, i, j] == -np.inf
                    continue
                per_head = []
                for h in range(g * G, (g + 1) * G):
                    tile = s * (q[0, h, i * b : (i + 1) * b] @ k[0, g, j * b : (j + 1) * b].T)
                    per_head.append(tile.mean())
                assert sc[0, g, i, j] == pytest.approx(max(per_head), rel=1e-12, abs=1e-14)


def test_decode_score_is_mean_of_block_logits():
    S, Hq, Hkv, L, d, b = 2, 4, 2, 200, 8, 64
    q, kc, vc = rnd((S, Hq, d), 12), rnd((S, Hkv, L, d), 13), rnd((S, Hkv, L, d), 14)
    r = O.decode(q, kc, vc, b, topk=2)
    s = 1.0 / math.sqrt(d)
    for si in range(S):
        for g in range(Hkv):
            for j in range(O.n_blocks(L, b)):
                want = max((s * (kc[si, g, j * b : (j + 1) * b] @ q[si, h])).mean() for h in (2 * g, 2 * g + 1))
                assert r["scores"][si, g, j] == pytest.approx(want, rel=1e-12, abs=1e-14)


# ---------------------------------------------------------------- P5 invariants
def test_rows_sum_to_one_and_constant_values():
    """With one-hot values the output row is the weight vector (sums to 1);
    constant values give that constant back."""
    N, d, b = 192, 8, 32
    q, k = rnd((1, 2, N, d), 15), rnd((1, 2, N, d), 16)
    sel = O.prefill(q, k, np.zeros((1, 2, N, d)), b, topk=3)
    v1 = np.zeros((1, 2, N, N))
    v1[0, :, np.arange(N), np.arange(N)] = 1.0
    q1 = np.concatenate([q, np.zeros((1, 2, N, N - d))], axis=-1)  # same logits, d padded with zeros
    k1 = np.concatenate([k, np.zeros((1, 2, N, N - d))], axis=-1)
    o, _ = O.attend(q1 * math.sqrt(N / d), k1, v1, sel["idx"], sel["cnt"], b)  # rescale: s = 1/sqrt(N) now
    np.testing.assert_allclose(o.sum(-1), 1.0, rtol=0, atol=1e-13)
    assert (o >= 0).all()
    # zero weight exactly on every key that is not kept or not causal
    for h in range(2):
        for p in range(N):
            i = p // b
            allowed = np.zeros(N, bool)
            for j in sel["idx"][0, h, i, : sel["cnt"][0, h, i]]:
                allowed[j * b : (j + 1) * b] = True
            allowed[p + 1 :] = False
            assert (o[0, h, p, ~allowed] == 0).all()
    o2, _ = O.attend(q, k, np.full((1, 2, N, d), 3.25), sel["idx"], sel["cnt"], b)
    np.testing.assert_allclose(o2, 3.25, rtol=1e-14)


def test_unselected_values_never_leak():
    """Poisoning the values of every block a row does not keep (NaN / 1e30)
    leaves that row bitwise unchanged; V does not enter the scores."""
    w = WORKLOADS["prefill_tiny_n1024"]
    q, k, v = (x.double().numpy() for x in make_prefill(w))
    q, k, v = q[:, :, :512], k[:, :, :512], v[:, :, :512]
    base = O.prefill(q, k, v, 64, topk=4)
    for h in range(2):
        i = 7
        keep = set(int(j) for j in base["idx"][0, h, i, : base["cnt"][0, h, i]])
        vp = v.copy()
        for j in range(8):
            if j not in keep:
                vp[0, h, j * 64 : (j + 1) * 64] = np.nan if j % 2 else 1e30
        r = O.prefill(q, k, vp, 64, topk=4)
        assert np.array_equal(r["o"][0, h, 7 * 64 :], base["o"][0, h, 7 * 64 :])


def test_causality_inside_the_diagonal_block():
    """Poisoning K and V at every position >= t leaves rows < t bitwise
    unchanged when the index set is held fixed."""
    N, d, b = 256, 8, 64
    q, k, v = rnd((1, 1, N, d), 17), rnd((1, 1, N, d), 18), rnd((1, 1, N, d), 19)
    base = O.prefill(q, k, v, b, topk=2)
    for t in (1, 70, 100, 191, 255):
        kp, vp = k.copy(), v.copy()
        kp[0, 0, t:] = np.nan
        vp[0, 0, t:] = np.inf
        o, _ = O.attend(q, kp, vp, base["idx"], base["cnt"], b)
        assert np.array_equal(o[0, 0, :t], base["o"][0, 0, :t])


# ---------------------------------------------------------------- P6 closed forms
def test_zero_queries_keep_lowest_candidates_and_average_values():
    """Q = 0 makes every score 0: each row keeps its forced blocks plus the
    lowest-index candidates, and each output row is the plain mean of the
    values it can see."""
    N, d, b, k_keep = 448, 8, 64, 4
    q = np.zeros((1, 2, N, d))
    k, v = rnd((1, 2, N, d), 20), rnd((1, 2, N, d), 21)
    r = O.prefill(q, k, v, b, topk=k_keep)
    for i in range(7):
        f = O.forced_set(i + 1, BOTH)
        m = min(k_keep, i + 1) - len(f)
        want = sorted(set(f) | set(range(1, 1 + max(m, 0))))
        assert list(r["idx"][0, 0, i, : r["cnt"][0, 0, i]]) == want
        for p in range(i * b, (i + 1) * b, 13):
            vis = [c for c in range(p + 1) if c // b in want]
            np.testing.assert_allclose(r["o"][0, 0, p], v[0, 0, vis].mean(0), rtol=1e-12, atol=1e-14)


def test_k2_keeps_sink_and_diagonal_only_and_row0_copies_v0():
    N, d, b = 320, 8, 64
    q, k, v = rnd((1, 1, N, d), 22), rnd((1, 1, N, d), 23), rnd((1, 1, N, d), 24)
    r = O.prefill(q, k, v, b, topk=2)
    for i in range(5):
        assert list(r["idx"][0, 0, i, : r["cnt"][0, 0, i]]) == sorted({0, i})
    assert np.array_equal(r["o"][0, 0, 0], v[0, 0, 0])
    assert r["lse"][0, 0, 0] == pytest.approx(float(q[0, 0, 0] @ k[0, 0, 0]) / math.sqrt(d), rel=1e-14)


def test_k1_without_forcing_and_flags_off():
    """flags = 0 forces nothing: k = 1 keeps the single best visible block."""
    N, d, b = 320, 8, 64
    q, k = rnd((1, 1, N, d), 25), rnd((1, 1, N, d), 26)
    r = O.prefill(q, k, np.zeros_like(k), b, topk=1, flags=0)
    for i in range(5):
        assert list(r["idx"][0, 0, i, : r["cnt"][0, 0, i]]) == [int(np.argmax(r["scores"][0, 0, i, : i + 1]))]


# ---------------------------------------------------------------- P7 GQA reduction
def test_gqa_with_identical_heads_equals_single_head():
    """A group whose query heads are identical selects exactly what one head
    alone selects, and every head's output equals the single-head output."""
    N, d, b = 384, 8, 64
    q1, k, v = rnd((1, 1, N, d), 27), rnd((1, 1, N, d), 28), rnd((1, 1, N, d), 29)
    r1 = O.prefill(q1, k, v, b, topk=3)
    r4 = O.prefill(np.repeat(q1, 4, axis=1), k, v, b, topk=3)
    assert np.array_equal(r1["idx"], r4["idx"])
    assert np.array_equal(r1["scores"], r4["scores"])
    for h in range(4):
        assert np.array_equal(r4["o"][0, h], r1["o"][0, 0])


def test_gqa_score_is_max_over_heads():
    N, d, b = 256, 8, 64
    q, k = rnd((1, 4, N, d), 30), rnd((1, 1, N, d), 31)
    s = 1.0 / math.sqrt(d)
    qb, kb = O.block_means(q, b), O.block_means(k, b)
    sc = O.block_scores(qb, kb, s)
    per = [O.block_scores(qb[:, h : h + 1], kb, s) for h in range(4)]
    assert np.array_equal(sc, np.maximum.reduce(per))


# ---------------------------------------------------------------- P8 scale invariance
def test_scaling_queries_keeps_selection():
    w = WORKLOADS["prefill_tiny_n1024"]
    q, k, v = (x.double().numpy() for x in make_prefill(w))
    a = O.prefill(q, k, v, 64, topk=4, attend_blocks=[])
    b_ = O.prefill(q * 4.0, k, v, 64, topk=4, attend_blocks=[])  # power of two: exact
    assert np.array_equal(a["idx"], b_["idx"])
    assert [r.flagged for r in a["rows"]] == [r.flagged for r in b_["rows"]]


# ---------------------------------------------------------------- P9 planted recovery
def test_planted_blocks_are_recovered():
    """The planted targets of the synthetic workload are found in nearly every
    unflagged row (a statistical check of the generator and the selection)."""
    w = Workload("planted_small", "prefill", 1, 4, 4, 4096, 128, 64, 16, structure="planted", amplitude=2.0, seed=11)
    q, k, v = make_prefill(w)
    r = O.prefill(q.double().numpy(), k.double().numpy(), v.double().numpy(), 64, topk=16, attend_blocks=[])
    # rebuild the planted targets from the generator's own CPU stream
    from dynamic_block_sparse_dsa_amd.inputs import _gen, _target_matrix
    hits = total = 0
    for h in range(4):
        m = _target_matrix(w.n_blocks, 1, lambda i: i - 1, 4, _gen("cpu", w.seed, h, 2), w.n_blocks)
        for i in range(2, w.n_blocks):
            rs = r["rows"][h * w.n_blocks + i]
            if rs.flagged:
                continue
            tg = set(int(j) for j in torch.nonzero(m[i]).flatten())
            total += 1
            hits += tg <= set(rs.idx)
    assert total > 200 and hits / total >= 0.97, (hits, total)


# ---------------------------------------------------------------- P10 count facts printed by the pages
def test_dense_count_facts():
    facts = json.load(open(os.path.join(GOLDEN, "count_facts.json")))["facts"]
    a, b_, c = facts
    assert work.dense_pairs(a["tokens"]) == pytest.approx(a["value"], rel=a["rel_tol"])
    assert work.dense_growth(b_["from_tokens"], b_["to_tokens"]) == b_["value"]
    assert work.dense_pairs(c["tokens"]) == c["value"]


def test_flop_count_of_a_tiny_pattern():
    """4 b^2 d per executed tile per query head: 2 heads share each group tile."""
    cnt = np.array([[[1, 2, 2]]])  # one group, three rows
    assert work.prefill_flops(cnt, group=2, block=64, head_dim=128) == 5 * 2 * 4 * 64 * 64 * 128


# ---------------------------------------------------------------- tie bands
def test_near_tie_band_and_acceptance():
    sc = np.array([0.0, 5.0, 3.0, 3.0000001, 1.0, -np.inf])  # row 4 sees blocks 0..4
    rs = O.select_row(sc, 5, 4, O.forced_set(5, BOTH))  # forced {0, 4}; two of {1, 2, 3}
    assert rs.flagged and rs.idx == [0, 1, 3, 4] and rs.need == 1 and rs.band == {2, 3} and rs.must == {1}
    # either of the two near-tied blocks is accepted ...
    assert O.accepts(rs, [0, 1, 3, 4])[0] and O.accepts(rs, [0, 1, 2, 4])[0]
    # ... not both, not the must-keep block dropped, not the sink dropped, not unsorted
    assert not O.accepts(rs, [0, 2, 3, 4])[0]
    assert not O.accepts(rs, [1, 2, 3, 4])[0]
    assert not O.accepts(rs, [0, 2, 1, 4])[0]
    clear = O.select_row(np.array([0.0, 5.0, 3.0, 1.0, 2.0]), 5, 4, O.forced_set(5, BOTH))
    assert not clear.flagged and clear.idx == [0, 1, 2, 4]
    assert not O.accepts(clear, [0, 1, 3, 4])[0]


def test_block_near_ties_are_relative_only():
    """Block selection flags a row only on the acceptance rule's relative gap
    (< 1e-3): two scores on either side of zero, 4e-7 apart, are distinct
    (relative gap 2), while 1.0 and 1.0009 are a near tie and 1.0 and 1.0011
    are not."""
    forced = O.forced_set(5, BOTH)  # {0, 4}; one of {1, 2, 3} is kept (k = 3)
    rs = O.select_row(np.array([0.0, 2e-7, -2e-7, -5.0, 0.0]), 5, 3, forced)
    assert not rs.flagged and rs.idx == [0, 1, 4]
    assert O.select_row(np.array([0.0, 1.0, 1.0009, -5.0, 0.0]), 5, 3, forced).flagged
    rs = O.select_row(np.array([0.0, 1.0, 1.0011, -5.0, 0.0]), 5, 3, forced)
    assert not rs.flagged and rs.idx == [0, 2, 4]
    # exact ties are always flagged (rel = 0), whatever their value
    assert O.select_row(np.array([0.0, 0.0, 0.0, -5.0, 0.0]), 5, 3, forced).flagged
    assert O.near(0.0, 0.0) and not O.near(1e-9, -1e-9) and O.near(1e-9, -1e-9, abs_floor=1e-6)


def test_generator_is_reproducible_per_unit():
    w = WORKLOADS["decode_s32_l65536"]
    small = Workload("dec_small", "decode", 2, 8, 2, 640, 32, 64, 4, structure="planted", amplitude=2.0, seed=5)
    q, kc, vc = make_decode(small)
    q1, k1, v1 = make_decode(small, units=[(1, 1)])
    assert torch.equal(q1[0], q[1, 4:8]) and torch.equal(k1[0], kc[1, 1]) and torch.equal(v1[0], vc[1, 1])
    assert w.n_blocks == 1024
