"""The plain-Python selection rules (selection_rules.py) that the validator's
GPU test compares the validator with, pinned against the oracle: every
selection the oracle makes -- prefill under each rule (top-k, fraction, no
forcing, anchors and windows, threshold, entropy), decode rows that see every
block, token selection -- breaks none of them, and single planted faults
raise exactly the slot they break, by exactly the count the fault implies."""

import numpy as np
import pytest
import torch
from selection_rules import (FORCE_DIAG, FORCE_SINK, SELECT_ENTROPY, SELECT_THRESHOLD, SELECT_TOPK, clean,
                             corrupt, count_rule, forcing, ref_report)

from oracle import dsa_oracle as O

NB = 37

CASES = [
    # (id, topk, num, den, flags, spec kwargs)
    ("topk6", 6, 0, 1, 3, {}),
    ("frac15", 0, 15, 100, 3, {}),
    ("noforce_k5", 5, 0, 1, 0, {}),
    ("sink_only", 4, 0, 1, FORCE_SINK, {}),
    ("diag_only", 4, 0, 1, FORCE_DIAG, {}),
    ("anchor2_window3", 8, 0, 1, 3, {"anchors": 2, "window": 3}),
    ("threshold", 0, 0, 1, 3, {"mode": SELECT_THRESHOLD, "threshold": 0.05}),
    ("entropy", 0, 0, 1, 3, {"mode": SELECT_ENTROPY, "k_min": 2, "k_max": 9}),
]


def oracle_selection(topk, num, den, flags, spec, causal=True, seed=5):
    g = np.random.default_rng(seed)
    scores = g.standard_normal((3, NB, NB)) * 2.0
    sp = O.SelectSpec(**spec)
    idx, cnt, _ = O.select_topk(scores, topk, num, den, flags, causal=causal, spec=sp)
    return idx, cnt


def rule_of(topk, num, den, spec):
    return count_rule(spec.get("mode", SELECT_TOPK), topk, num, den, spec.get("threshold", 0.0),
                      spec.get("k_min", 0), spec.get("k_max", 0))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_oracle_prefill_selection_obeys_the_rules(case):
    _, topk, num, den, flags, spec = case
    idx, cnt = oracle_selection(topk, num, den, flags, spec)
    anchors, window = forcing(flags, spec.get("anchors", 0), spec.get("window", 0))
    rep = ref_report(idx, cnt, lambda r: r % NB + 1, rule_of(topk, num, den, spec), anchors, window)
    assert rep == clean(3 * NB)
    # the count taken from the -1 padding (no cnt) gives the same verdict
    rep = ref_report(idx, None, lambda r: r % NB + 1, rule_of(topk, num, den, spec), anchors, window)
    assert rep == clean(3 * NB)


@pytest.mark.parametrize("case", CASES[:6], ids=[c[0] for c in CASES[:6]])
def test_oracle_decode_selection_obeys_the_rules(case):
    _, topk, num, den, flags, spec = case
    idx, cnt = oracle_selection(topk, num, den, flags, spec, causal=False)
    anchors, window = forcing(flags, spec.get("anchors", 0), spec.get("window", 0))
    assert ref_report(idx, cnt, lambda r: NB, rule_of(topk, num, den, spec), anchors, window) == clean(3 * NB)


@pytest.mark.parametrize("flags", [3, 1, 2, 0])
def test_oracle_token_selection_obeys_the_rules(flags):
    g = np.random.default_rng(6)
    N = 90
    scores = np.maximum(g.standard_normal((2, N, N)), 0.0)
    idx, cnt, _ = O.select_tokens(scores, 7, flags)
    anchors, window = (1 if flags & FORCE_SINK else 0), (1 if flags & FORCE_DIAG else 0)
    assert ref_report(idx, cnt, lambda r: r % N + 1, count_rule(SELECT_TOPK, 7), anchors, window) == clean(2 * N)


def test_planted_faults_raise_their_slot_by_their_count():
    idx, cnt = oracle_selection(6, 0, 1, 3, {})
    vis = lambda r: r % NB + 1
    rule = count_rule(SELECT_TOPK, 6)
    base = clean(3 * NB)

    def report(ix, ct=cnt):
        return ref_report(ix, ct, vis, rule, 1, 1)

    r = 20  # row 20 sees 21 blocks and keeps 6: [0, a, b, c, d, 20]
    row = idx.reshape(-1, idx.shape[-1])[r]
    assert row[0] == 0 and row[5] == 20 and cnt.reshape(-1)[r] == 6
    cases = []
    ix = idx.copy(); f = ix.reshape(-1, ix.shape[-1]); f[r, 1], f[r, 2] = f[r, 2], f[r, 1]
    cases.append((ix, cnt, {"order": 1}))  # one adjacent pair out of order
    ix = idx.copy(); f = ix.reshape(-1, ix.shape[-1]); f[r, 2] = f[r, 1]
    cases.append((ix, cnt, {"order": 1}))  # a repeat
    ix = idx.copy(); f = ix.reshape(-1, ix.shape[-1]); f[r, 5] = 21
    cases.append((ix, cnt, {"range": 1, "forced": 1}))  # the diagonal replaced by a future block
    ix = idx.copy(); f = ix.reshape(-1, ix.shape[-1]); f[r, 0] = -1
    cases.append((ix, cnt, {"range": 1, "forced": 1}))  # the sink replaced by the padding value
    ct = cnt.copy(); ct.reshape(-1)[r] = 5
    cases.append((idx, ct, {"count": 1, "forced": 1, "padding": 1}))  # the diagonal falls into the padding
    ct = cnt.copy(); ct.reshape(-1)[r] = -4
    cases.append((idx, ct, {"count": 1, "forced": 2, "padding": 6}))
    r3 = 3  # row 3 sees 4 blocks, keeps all 4: [0, 1, 2, 3, -1, -1]
    assert idx.reshape(-1, idx.shape[-1])[r3].tolist() == [0, 1, 2, 3, -1, -1]
    ix = idx.copy(); f = ix.reshape(-1, ix.shape[-1]); f[r3, 5] = 2
    cases.append((ix, cnt, {"padding": 1}))
    ct = cnt.copy(); ct.reshape(-1)[r3] = 1000
    cases.append((idx, ct, {"count": 1, "range": 2, "order": 2}))  # the -1 padding read as ids
    for ix, ct, want in cases:
        assert report(ix, ct) == {**base, **want}


def test_corrupt_helper_raises_every_slot():
    idx, cnt = oracle_selection(6, 0, 1, 3, {})
    vis = lambda r: r % NB + 1
    bix, bct, hit = corrupt(torch.from_numpy(idx), torch.from_numpy(cnt), vis, 3)
    rep = ref_report(bix.numpy(), bct.numpy(), vis, count_rule(SELECT_TOPK, 6), 1, 1)
    assert rep["order"] >= 2 and rep["range"] >= 2 and rep["forced"] >= 1 and rep["padding"] >= 1
    assert rep["count"] >= hit["count"] >= 2
