"""The streaming rule behind the fused token selection, checked on the host
against the plain definition (best m by score, ties to the lower position).

The kernel sees a row's keys in ascending position order, 64 at a time.  A
key joins the row's candidate list when it exceeds the row's threshold T
(0 at first); a list that may overflow its 256 slots is cut back (keep every
entry >= T' for a T' that at least m entries reach, found bit by bit from
the common leading bits of the largest and smallest entry and stopping once
at most 128 remain; if the bits run out first, T' is the m-th largest and
the entries equal to it are cut to the lowest positions), and T becomes
max(T, T').  Rows longer than one chunk of 2048 keys keep a list per chunk,
each cut to its best m; the concatenated lists are cut once more.  This
model follows those steps on integer keys (order-preserving images of the
fp32 scores) and must return exactly the definition's set, on random keys,
heavily tied keys, ascending keys (every key a new record) and a narrow
range."""

import numpy as np
import pytest

CAP, CHUNK = 256, 2048


def cut(keys, pos, m, limit, thr):
    k = np.asarray(keys, dtype=np.int64)
    mx, mn = int(k.max()), int(k.min())
    x = mx ^ mn
    bit = x.bit_length() - 1 if x else -1
    T = (mx & ~((2 << bit) - 1)) if x else mx
    nT = len(k)
    while bit >= 0 and nT > limit:
        trial = T | (1 << bit)
        c = int((k >= trial).sum())
        if c >= m:
            T, nT = trial, c
        bit -= 1
    tie_cut = nT > limit
    n_gt = int((k > T).sum()) if tie_cut else 0
    out_k, out_p, r = [], [], 0
    for kk, pp in zip(keys, pos):
        if kk > T or (kk == T and (not tie_cut or r < m - n_gt)):
            out_k.append(kk)
            out_p.append(pp)
        r += kk == T
    return out_k, out_p, max(thr, T)


def stream_chunk(keys, lo, hi, m):
    lk, lp, thr = [], [], 0
    for base in range(lo, hi, 64):
        for p in range(base, min(base + 64, hi)):
            if keys[p] > thr:
                lk.append(keys[p])
                lp.append(p)
        assert len(lk) <= CAP
        if len(lk) > CAP - 64:
            lk, lp, thr = cut(lk, lp, m, max(CAP // 2, m), thr)
    if len(lk) > m:
        lk, lp, _ = cut(lk, lp, m, m, 0)
    return lk, lp


def streamed_selection(keys, m):
    lk, lp = [], []
    for c0 in range(0, len(keys), CHUNK):
        k, p = stream_chunk(keys, c0, min(c0 + CHUNK, len(keys)), m)
        lk += k
        lp += p
    if len(lk) > m:
        lk, lp, _ = cut(lk, lp, m, m, 0)
    return lp


def definition(keys, m):
    order = sorted(range(len(keys)), key=lambda p: (-keys[p], p))
    return sorted(order[:m])


@pytest.mark.parametrize("kind", ["random", "ties", "ascending", "narrow"])
def test_stream_rule_equals_the_definition(kind):
    rng = np.random.default_rng({"random": 1, "ties": 2, "ascending": 3, "narrow": 4}[kind])
    for _ in range(25):
        n = int(rng.integers(1, 7000))
        m = int(rng.integers(1, 129))
        if kind == "random":
            keys = rng.integers(1, 2**32 - 1, n)
        elif kind == "ties":
            keys = rng.integers(1, 12, n)
        elif kind == "ascending":
            keys = np.sort(rng.integers(1, 2**32 - 1, n))
        else:
            keys = 0x80000000 + 7 * rng.integers(0, 4096, n)
        keys = [int(x) for x in keys]
        assert streamed_selection(keys, m) == definition(keys, m), (kind, n, m)
