"""Pins for the oracle's selection variants (global anchors + local window
as the forced set, threshold selection, entropy budget, bitmap output).

Each test ties the oracle to something other than its own formulas: an
independently written rule checked by brute-force subset enumeration, a
library routine (scipy's softmax and entropy), a closed form, or an
invariant -- chosen so that a plausible slip (a window off by one, a softmax
over the candidates only instead of every visible block, a natural/binary log
mix-up, a bit order reversed) fails one of them.  Runs on the CPU.
"""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import scipy.stats
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle as O

BOTH = O.FORCE_SINK | O.FORCE_DIAG


def tril_scores(s):
    nb = s.shape[-1]
    return np.where(np.tril(np.ones((nb, nb))) > 0, s, -np.inf)


# ---------------------------------------------------------------- forced set
def forced_by_distance(i, flags, anchors, window):
    """Row i (blocks 0..i visible): block j is a global anchor when j <
    anchors, in the local window when its distance to the row's own block,
    i - j, is below the window length."""
    out = []
    for j in range(i + 1):
        if (flags & O.FORCE_SINK and j < anchors) or (flags & O.FORCE_DIAG and i - j < window):
            out.append(j)
    return out


def brute_select(scores, n_vis, k, forced):
    cand = [j for j in range(n_vis) if j not in forced]
    m = min(max(k, len(forced)), n_vis) - len(forced)
    best, best_key = None, None
    for sub in itertools.combinations(cand, m):
        key = sum(Fraction(scores[j]) for j in sub)
        if best is None or key > best_key:
            best, best_key = sub, key
    return sorted(set(forced) | set(best))


@settings(max_examples=150, deadline=None)
@given(nb=st.integers(1, 10), k=st.integers(1, 11), flags=st.sampled_from([0, 1, 2, 3]), anchors=st.integers(1, 4),
       window=st.integers(1, 4), seed=st.integers(0, 10**6))
def test_anchor_window_selection_is_the_best_subset(nb, k, flags, anchors, window, seed):
    """With anchors and a window the kept set still maximises the summed score
    among sets of its size that hold the forced blocks, and the forced blocks
    are exactly those the distance rule names."""
    s = np.random.default_rng(seed).standard_normal((nb, nb))
    spec = O.SelectSpec(anchors=anchors, window=window)
    idx, cnt, _ = O.select_topk(tril_scores(s)[None, None], topk=k, flags=flags, spec=spec)
    for i in range(nb):
        f = forced_by_distance(i, flags, anchors, window)
        assert O.forced_set(i + 1, flags, anchors, window) == f
        assert list(idx[0, 0, i, : cnt[0, 0, i]]) == brute_select(s[i], i + 1, k, f)


def test_default_forced_set_is_sink_and_diagonal():
    """anchors = window = 1 is the plain sink + diagonal rule."""
    for nv in range(1, 9):
        assert O.forced_set(nv, BOTH, 1, 1) == sorted({0, nv - 1})
        assert O.forced_set(nv, BOTH) == O.forced_set(nv, BOTH, 1, 1)


def test_decode_window_forces_the_last_blocks():
    """Decode sees every block: a window of 3 forces the last three, 2
    anchors the first two."""
    assert O.forced_set(10, BOTH, 2, 3) == [0, 1, 7, 8, 9]
    assert O.forced_set(4, BOTH, 2, 3) == [0, 1, 2, 3]


# ---------------------------------------------------------------- block distribution
@pytest.mark.parametrize("seed", range(5))
def test_block_shares_and_entropy_match_scipy(seed):
    row = np.random.default_rng(seed).standard_normal(37) * 3
    p = O.block_shares(row)
    np.testing.assert_allclose(p, scipy.special.softmax(row), rtol=1e-13, atol=0)
    assert O.block_entropy(row) == pytest.approx(scipy.stats.entropy(scipy.special.softmax(row)), rel=1e-12)


def test_entropy_closed_forms():
    """Uniform over n blocks: H = ln n.  p = (1/2, 1/4, 1/4): H = 1.5 ln 2.
    A block with all the mass: H = 0."""
    for n in (1, 2, 7, 64):
        assert O.block_entropy(np.full(n, 0.3)) == pytest.approx(math.log(n), abs=1e-12)
    assert O.block_entropy(np.log([0.5, 0.25, 0.25]) + 1.7) == pytest.approx(1.5 * math.log(2), rel=1e-12)
    assert O.block_entropy(np.array([0.0, -2000.0, -3000.0])) == 0.0


def test_entropy_budget_closed_forms():
    """exp(H) is the effective number of blocks: 2^1.5 = 2.83 -> 3; uniform
    over n -> n; clamped to [k_min, k_max]; raised to the forced count."""
    row = np.log([0.5, 0.25, 0.25])
    assert O.entropy_budgets(row, 3, 1, 10, 0) == [3]
    assert O.entropy_budgets(np.zeros(12), 12, 1, 64, 2) == [12]
    assert O.entropy_budgets(np.zeros(12), 12, 1, 5, 2) == [5]
    assert O.entropy_budgets(np.array([0.0, -2000.0, -3000.0, -4000.0]), 4, 2, 8, 1) == [2]
    assert O.entropy_budgets(np.array([0.0, -2000.0, -3000.0, -4000.0]), 4, 1, 8, 3) == [3]
    # a share vector with exp(H) = 5.0000...: either side of the integer is accepted
    both = O.entropy_budgets(np.zeros(5), 8, 1, 8, 0)
    assert both == [5, 6]


def test_entropy_counts_every_visible_block():
    """The forced blocks are part of the row's distribution: two forced blocks
    with most of the mass make exp(H) small; over the candidates alone (all
    equal) it would be their count."""
    row = np.array([8.0, 0, 0, 0, 0, 0, 0, 0, 0, 8.0])
    sc = tril_scores(np.tile(row, (10, 1)))[None, None]
    spec = O.SelectSpec(mode=O.SELECT_ENTROPY, k_min=1, k_max=10)
    _, cnt, rows = O.select_topk(sc, topk=0, flags=BOTH, spec=spec)
    p = scipy.special.softmax(row)
    want = math.ceil(math.exp(scipy.stats.entropy(p)))
    assert want == 3
    assert cnt[0, 0, 9] == want


# ---------------------------------------------------------------- threshold
def test_threshold_two_levels_closed_form():
    """Row of 10 visible blocks: the forced sink and diagonal score 2, three
    candidates score 1, the other five 0.  Shares: e^2/Z, e/Z, 1/Z with
    Z = 2e^2 + 3e + 5.  A threshold just under e/Z keeps the three; just over
    it keeps none.  (A softmax over the candidates alone would give the three
    e/(3e + 5) and keep them at both thresholds.)"""
    row = np.array([2.0, 0, 1, 0, 1, 0, 1, 0, 0, 2.0])
    z = 2 * math.e ** 2 + 3 * math.e + 5
    mid = math.e / z
    for tau, want in [(mid * 0.99, [0, 2, 4, 6, 9]), (mid * 1.01, [0, 9])]:
        rs = O.threshold_row(row, 10, tau, [0, 9])
        assert rs.idx == want and not rs.flagged


def test_threshold_invariants():
    rng = np.random.default_rng(3)
    for _ in range(20):
        nv = int(rng.integers(2, 60))
        row = rng.standard_normal(nv) * 2
        tau = float(rng.uniform(0.005, 0.3))
        f = O.forced_set(nv, BOTH)
        rs = O.threshold_row(row, nv, tau, f)
        # shift invariance: the distribution ignores a common offset
        assert O.threshold_row(row + 5.0, nv, tau, f).idx == rs.idx
        kept = [j for j in rs.idx if j not in f]
        assert len(kept) <= math.floor(1 / tau)
        # the kept candidates are the best-scoring ones: a top-k with that budget
        assert O.select_row(row, nv, len(f) + len(kept), f).idx == rs.idx
    # tiny threshold keeps everything, one above every share keeps the forced only
    row = rng.standard_normal(20)
    assert O.threshold_row(row, 20, 1e-12, [0, 19]).idx == list(range(20))
    assert O.threshold_row(row, 20, 0.999, [0, 19]).idx == [0, 19]


def test_threshold_uses_the_fp32_value():
    """The boundary carries the threshold as fp32: 0.1 becomes
    0.100000001490116..., so ten equal shares of exactly 0.1 all fall below it
    and the index width is the forced count + floor(1 / tau) = 2 + 9."""
    spec = O.SelectSpec(mode=O.SELECT_THRESHOLD, threshold=0.1)
    tau = O.spec_tau(spec)
    assert tau == float(np.float32(0.1)) and tau > 0.1
    rs = O.threshold_row(np.zeros(10), 10, tau, [])
    assert rs.idx == [] and rs.flagged  # every share is within the band of tau
    assert O.kmax(64, 0, 0, 1, BOTH, True, 64, spec) == 11


def test_threshold_band_accepts_either_choice():
    """A candidate whose share sits on the threshold may be kept or dropped."""
    row = np.zeros(4)  # shares 1/4
    rs = O.threshold_row(row, 4, 0.25, [0])
    assert rs.flagged and rs.band == {1, 2, 3} and rs.need == -1
    for got in ([0], [0, 2], [0, 1, 2, 3]):
        assert O.accepts(rs, got)[0]
    assert not O.accepts(rs, [1, 2])[0]  # forced block missing


def test_entropy_alternative_budget_is_accepted():
    """Row 7 sees four equal blocks and four with no mass: exp(H) = 4 to
    rounding, so budgets 4 and 5 are both accepted (and not 3 or 6)."""
    row = np.array([0.0, -2000, 0, -2000, 0, -2000, 0, -2000])
    sc = tril_scores(np.tile(row, (8, 1)))[None, None]
    spec = O.SelectSpec(mode=O.SELECT_ENTROPY, k_min=1, k_max=8)
    _, _, rows = O.select_topk(sc, topk=0, flags=0, spec=spec)
    rs = rows[7]
    assert rs.flagged and len(rs.alts) == 1
    assert O.accepts(rs, [0, 2, 4, 6])[0]
    assert O.accepts(rs, [0, 1, 2, 4, 6])[0]
    assert not O.accepts(rs, [0, 2, 4])[0]
    assert not O.accepts(rs, [0, 1, 2, 3, 4, 6])[0]


# ---------------------------------------------------------------- bitmap
def test_bitmap_written_out():
    """Blocks 0, 1, 33, 63 of a 64-block row: words 0x00000003, 0x80000002."""
    idx = np.array([[0, 1, 33, 63, -1]], dtype=np.int32)
    bm = O.bitmap(idx, np.array([4], dtype=np.int32), 64)
    assert bm.tolist() == [[0x00000003, 0x80000002]]
    bm = O.bitmap(idx, np.array([4], dtype=np.int32), 65)  # ragged: a third word
    assert bm.tolist() == [[0x00000003, 0x80000002, 0]]


@settings(max_examples=50, deadline=None)
@given(nb=st.integers(1, 100), seed=st.integers(0, 10**6))
def test_bitmap_round_trip(nb, seed):
    """Unpacking the words (numpy's little-endian bit order) gives the kept
    blocks back; the popcount is the count."""
    sc = tril_scores(np.random.default_rng(seed).standard_normal((nb, nb)))[None]
    idx, cnt, _ = O.select_topk(sc, topk=5, flags=BOTH)
    bm = O.bitmap(idx, cnt, nb)
    bits = np.unpackbits(bm.view(np.uint8), axis=-1, bitorder="little")
    for i in range(nb):
        assert list(np.nonzero(bits[0, i])[0]) == list(idx[0, i, : cnt[0, i]])
        assert int(bits[0, i].sum()) == cnt[0, i]
