"""The rules a selection's index array obeys, written out in plain Python for
the selection validator's tests: for each row, the kept count allowed by the
selection rule, ids inside the row's visible range, strictly ascending lists,
the forced ids present, and -1 padding past the count.  The rules are the
block selection of "dynamic sparse attention explainer", section
"基于Top-k选择的局部-全局混合" (anchors, local window, best others up to the
budget), with the threshold rule of DeepSeek NSA article section 2.2 and the
entropy budget of the explainer's "工程实践建议", and the token selection of
the DeepSeek-V3.2 lightning indexer.  Shared by the CPU test that checks them
against the oracle's selections and by the GPU test of the validator."""

import math

import numpy as np
import torch

SLOTS = ("rows", "count", "range", "order", "forced", "padding")
SELECT_TOPK, SELECT_THRESHOLD, SELECT_ENTROPY = 0, 1, 2
FORCE_SINK, FORCE_DIAG = 1, 2
MAX_BLOCKS = 4096


def count_rule(mode, topk=0, num=0, den=1, threshold=0.0, k_min=0, k_max=0):
    """(lo, hi) of the kept count of a row with `v` visible ids, `nf` forced."""
    def rng(v, nf):
        if mode == SELECT_THRESHOLD:
            cap = min(math.floor(1.0 / float(np.float32(threshold))), MAX_BLOCKS)
            return nf, min(nf + cap, v)
        if mode == SELECT_ENTROPY:
            return min(max(k_min, nf), v), min(max(k_max, nf), v)
        k = topk if topk > 0 else -(-num * v // den)
        k = min(max(k, nf), v)
        return k, k
    return rng


def ref_report(idx, cnt, visible, rng, anchors, window):
    idx = idx.reshape(-1, idx.shape[-1]).tolist()
    cnt = None if cnt is None else cnt.reshape(-1).tolist()
    km = len(idx[0]) if idx else 0
    rep = dict.fromkeys(SLOTS, 0)
    for r, row in enumerate(idx):
        v = visible(r)
        if cnt is None:
            n = row.index(-1) if -1 in row else km
        else:
            n = cnt[r]
        na = min(anchors, v)
        ws = max(v - window, na)
        nf = na + (v - ws)
        lo, hi = rng(v, nf)
        rep["rows"] += 1
        rep["count"] += int(n < lo or n > hi or n > km)
        n = min(max(n, 0), km)
        lst = row[:n]
        rep["range"] += sum(1 for e in lst if e < 0 or e >= v)
        rep["order"] += sum(1 for t in range(1, n) if lst[t] <= lst[t - 1])
        hits = sum(1 for e in lst if 0 <= e < v and (e < na or e >= ws))
        rep["forced"] += max(nf - hits, 0)
        rep["padding"] += sum(1 for e in row[n:] if e != -1)
    return rep


def clean(rows):
    return {s: (rows if s == "rows" else 0) for s in SLOTS}


def forcing(flags, n_anchor=0, window=0):
    return (max(1, n_anchor) if flags & FORCE_SINK else 0), (max(1, window) if flags & FORCE_DIAG else 0)


def corrupt(idx, cnt, visible, seed):
    """Corrupted CPU copies: one row per kind of fault."""
    g = np.random.default_rng(seed)
    ix = idx.cpu().numpy().copy()
    flat = ix.reshape(-1, ix.shape[-1])
    ct = None if cnt is None else cnt.cpu().numpy().copy()
    cflat = None if ct is None else ct.reshape(-1)
    R, km = flat.shape

    def n_of(r):
        if cflat is not None:
            return int(cflat[r])
        row = flat[r].tolist()
        return row.index(-1) if -1 in row else km

    rows = [r for r in g.permutation(R).tolist() if n_of(r) >= 2]
    assert len(rows) >= 7, "too few rows with two kept ids to corrupt"
    hit = {}
    r = rows[0]  # swap the first two ids
    flat[r, 0], flat[r, 1] = flat[r, 1], flat[r, 0]
    hit["order"] = r
    r = rows[1]  # repeat an id
    flat[r, 1] = flat[r, 0]
    hit["order2"] = r
    r = rows[2]  # an id past the row's visible range, at the end of its list
    flat[r, n_of(r) - 1] = visible(r) + 3
    hit["range"] = r
    r = rows[3]  # a negative id at the front
    flat[r, 0] = -5
    hit["range2"] = r
    r = rows[4]  # drop the first id (a forced anchor when the sink is forced)
    n = n_of(r)
    flat[r, : n - 1] = flat[r, 1:n].copy()
    flat[r, n - 1] = visible(r) - 1 if flat[r, n - 2] < visible(r) - 1 else flat[r, n - 2] + 1
    hit["forced"] = r
    count_rows = rows[5:9] if cflat is not None else []
    pad_rows = [q for q in range(R) if q not in rows[:5] and q not in count_rows and n_of(q) < km]
    if pad_rows:  # garbage in the padding
        flat[pad_rows[0], km - 1] = 2
        hit["padding"] = pad_rows[0]
    if count_rows:  # counts: one too many, one too few, negative, above kmax
        for q, f in zip(count_rows, (lambda c: c + 1, lambda c: c - 1, lambda c: -2, lambda c: km + 3)):
            cflat[q] = f(int(cflat[q]))
        hit["count"] = 2 if len(count_rows) == 4 else 0  # the last two break every rule
    return torch.from_numpy(ix), (None if ct is None else torch.from_numpy(ct)), hit
