"""Pins for the oracle's FP8 (E4M3) cache rows.

The E4M3 value set is written out from the format's definition (sign, 4-bit
exponent with bias 7, 3-bit mantissa, subnormals below exponent 1, 448 the
largest finite value), and every quantized element is checked to be the
nearest member of that set to fp32(x / scale), ties to the even mantissa:
this pins the library cast the oracle uses.  Also: round-trip error bounds,
exact round trips of representable rows, the row scale's definition, and the
fp8 paged decode equalling the paged decode of the dequantized pools.
"""

import math

import numpy as np
import pytest

import oracle as O


def e4m3_table():
    """All finite E4M3 values by code (NaN codes 0x7F, 0xFF excluded)."""
    vals = {}
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals[code] = -mag if s else mag
    return vals


def test_value_set():
    t = e4m3_table()
    assert max(t.values()) == 448.0 and min(t.values()) == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6
    codes = np.array(sorted(t), dtype=np.uint8)
    np.testing.assert_array_equal(O.fp8_values(codes), np.array([t[c] for c in codes]))


@pytest.mark.parametrize("seed", range(4))
def test_codes_are_the_nearest_values_ties_to_even(seed):
    t = e4m3_table()
    codes_pos = np.array(sorted(c for c in t if c < 128), dtype=np.int64)  # ascending value with the code
    vals = np.array([t[c] for c in codes_pos])
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((64, 128)) * rng.choice([1e-3, 1.0, 50.0], size=(64, 1))
    x[0, :4] = [0.0, 0.0, 0.0, 0.0]
    codes, scale = O.quantize_fp8(x)
    y = (x.astype(np.float32) / scale[:, None]).astype(np.float32).astype(np.float64)
    got = O.fp8_values(codes)
    a = np.abs(y).ravel()
    hi = np.clip(np.searchsorted(vals, a), 1, len(vals) - 1)
    lo = hi - 1
    dlo, dhi = a - vals[lo], vals[hi] - a
    # nearest magnitude; on a tie the neighbour whose code is even
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(codes_pos[lo] % 2 == 0, lo, hi)))
    best = vals[pick].reshape(y.shape)
    assert (np.abs(got) == best).all()
    nz = got != 0
    assert (np.sign(got[nz]) == np.sign(y[nz])).all()


def test_scale_definition_and_round_trip_bounds():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((100, 64)) * 3
    x[5] = 0.0
    codes, scale = O.quantize_fp8(x)
    amax = np.abs(x.astype(np.float32)).max(axis=1)
    np.testing.assert_array_equal(scale[amax > 0], (amax / np.float32(448))[amax > 0])
    assert scale[5] == 1.0 and (codes[5] == 0).all()
    deq = O.dequantize_fp8(codes, scale)
    # half a unit in the last place: 2^-4 relative in the normal range, 2^-10 scale below it
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scale[:, None] * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(deq - x) <= bound).all()
    # the row maximum lands on 448 * scale
    i = np.abs(x[0]).argmax()
    assert abs(O.fp8_values(codes[0, i])) == 448.0


def test_representable_rows_round_trip_exactly():
    t = e4m3_table()
    vals = np.array([t[c] for c in (0x7E, 0x3C, 0x01, 0xB5, 0x10)])  # 448 is in the row
    x = vals * 0.25  # scale 0.25 exactly
    codes, scale = O.quantize_fp8(x[None])
    assert scale[0] == np.float32(0.25)
    np.testing.assert_array_equal(O.dequantize_fp8(codes, scale)[0], x)


def test_fp8_paged_decode_is_the_decode_of_the_dequantized_pools():
    rng = np.random.default_rng(8)
    S, Hq, Hkv, d, block, n_pages = 2, 4, 2, 16, 8, 9
    q = rng.standard_normal((S, Hq, d))
    kp, vp = rng.standard_normal((n_pages, Hkv, block, d)), rng.standard_normal((n_pages, Hkv, block, d))
    k8, ks = O.quantize_fp8(kp)
    v8, vs = O.quantize_fp8(vp)
    table = rng.permutation(n_pages)[:8].reshape(S, 4).astype(np.int32)
    lengths = np.array([32, 13], dtype=np.int32)
    kd, vd = O.dequantize_fp8(k8, ks), O.dequantize_fp8(v8, vs)
    r = O.paged_decode(q, kd, vd, table, lengths, block, 2)
    # every block kept: single-query attention over the dequantized rows
    full = O.paged_decode(q, kd, vd, table, lengths, block, 10)
    for s in range(S):
        L = int(lengths[s])
        ks_ = O.paged_gather(kd, table, s, L, block)
        vs_ = O.paged_gather(vd, table, s, L, block)
        for h in range(Hq):
            lg = ks_[h // 2] @ q[s, h] / math.sqrt(d)
            w = np.exp(lg - lg.max())
            np.testing.assert_allclose(full["o"][s, h], (w / w.sum()) @ vs_[h // 2], rtol=1e-12)
    assert r["cnt"].max() == 2


def test_fp8_appends_quantize_each_row_and_average_the_dequantized_page():
    rng = np.random.default_rng(9)
    S, Hkv, d, block = 2, 2, 8, 4
    n_pages = 6
    table = np.array([[3, 0, 5], [1, 4, 2]], dtype=np.int32)
    k8 = np.zeros((n_pages, Hkv, block, d), np.uint8)
    v8 = np.zeros_like(k8)
    ks = np.zeros((n_pages, Hkv, block), np.float32)
    vs = np.zeros_like(ks)
    kbar = np.zeros((n_pages, Hkv, d))
    lengths = np.zeros(S, np.int32)
    rows = rng.standard_normal((7, S, Hkv, d))
    for t in range(7):
        O.kv_append_fp8(k8, v8, ks, vs, kbar, table, lengths, rows[t], rows[t] * 2, block)
    assert (lengths == 7).all()
    for s in range(S):
        c, sc = O.quantize_fp8(rows[:, s])  # [7, Hkv, d], [7, Hkv]
        for t in range(7):
            page, slot = table[s, t // block], t % block
            np.testing.assert_array_equal(k8[page, :, slot], c[t])
            np.testing.assert_array_equal(ks[page, :, slot], sc[t])
        page = table[s, 1]  # rows 4..6
        np.testing.assert_allclose(kbar[page], O.dequantize_fp8(c[4:7], sc[4:7]).mean(axis=0), rtol=1e-13)
