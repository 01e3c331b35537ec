"""Pins for the oracle's paged KV cache (gather, decode with per-sequence
lengths, appends, per-page block means).

Against: single-query SDPA from torch over each sequence's first L tokens
when every block is kept (pages shuffled, the slots past a length poisoned),
the contiguous decode of the truncated cache, and a token-by-token rebuild of
the pools whose page means are compared with plain means of the rows
written so far.  Runs on the CPU.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O

BOTH = O.FORCE_SINK | O.FORCE_DIAG


def build_paged(kc, vc, lengths, block, rng, poison=1e6):
    """Scatter contiguous caches [S, Hkv, Lmax, d] into shuffled pages; slots
    past each length hold ``poison``."""
    S, Hkv, Lmax, d = kc.shape
    mb = -(-Lmax // block)
    n_pages = S * mb + 3
    perm = rng.permutation(n_pages)
    table = perm[: S * mb].reshape(S, mb).astype(np.int32)
    kp = np.full((n_pages, Hkv, block, d), poison)
    vp = np.full((n_pages, Hkv, block, d), poison)
    for s in range(S):
        for j in range(-(-int(lengths[s]) // block)):
            rows = min(block, int(lengths[s]) - j * block)
            kp[table[s, j], :, :rows] = kc[s, :, j * block : j * block + rows]
            vp[table[s, j], :, :rows] = vc[s, :, j * block : j * block + rows]
    return kp, vp, table


@pytest.mark.parametrize("block", [16, 32])
def test_every_block_kept_is_single_query_attention(block):
    rng = np.random.default_rng(1)
    S, Hq, Hkv, Lmax, d = 3, 4, 2, 150, 8
    q, kc, vc = rng.standard_normal((S, Hq, d)), rng.standard_normal((S, Hkv, Lmax, d)), rng.standard_normal((S, Hkv, Lmax, d))
    lengths = np.array([150, 37, 1], dtype=np.int32)
    kp, vp, table = build_paged(kc, vc, lengths, block, rng)
    r = O.paged_decode(q, kp, vp, table, lengths, block, topk=10**6)
    G = Hq // Hkv
    for s in range(S):
        L = int(lengths[s])
        qt = torch.from_numpy(q[s : s + 1, :, None, :])
        kt = torch.from_numpy(kc[s : s + 1, :, :L]).repeat_interleave(G, 1)
        vt = torch.from_numpy(vc[s : s + 1, :, :L]).repeat_interleave(G, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0].numpy()
        np.testing.assert_allclose(r["o"][s], ref, rtol=1e-11, atol=1e-12)
        assert (r["cnt"][s] == -(-L // block)).all()


def test_paged_equals_contiguous_decode_of_the_truncated_cache():
    rng = np.random.default_rng(2)
    S, Hq, Hkv, Lmax, d, block = 4, 4, 2, 200, 16, 16
    q, kc, vc = rng.standard_normal((S, Hq, d)), rng.standard_normal((S, Hkv, Lmax, d)), rng.standard_normal((S, Hkv, Lmax, d))
    lengths = np.array([200, 131, 16, 77], dtype=np.int32)
    kp, vp, table = build_paged(kc, vc, lengths, block, rng)
    spec = O.SelectSpec(anchors=2, window=2)
    r = O.paged_decode(q, kp, vp, table, lengths, block, 4, flags=BOTH, spec=spec)
    for s in range(S):
        L = int(lengths[s])
        ref = O.decode(q[s : s + 1], kc[s : s + 1, :, :L], vc[s : s + 1, :, :L], block, 4, flags=BOTH, spec=spec)
        np.testing.assert_allclose(r["o"][s], ref["o"][0], rtol=1e-12, atol=1e-13)
        for g in range(Hkv):
            c = r["cnt"][s, g]
            assert list(r["idx"][s, g, :c]) == list(ref["idx"][0, g, : ref["cnt"][0, g]])
            assert (r["idx"][s, g, c:] == -1).all()


def test_appends_rebuild_the_cache_and_the_page_means():
    rng = np.random.default_rng(3)
    S, Hkv, d, block, T = 2, 2, 4, 8, 21
    mb = -(-T // block)
    n_pages = S * mb + 2
    table = rng.permutation(n_pages)[: S * mb].reshape(S, mb).astype(np.int32)
    kp, vp = np.zeros((n_pages, Hkv, block, d)), np.zeros((n_pages, Hkv, block, d))
    kbar = np.zeros((n_pages, Hkv, d))
    lengths = np.zeros(S, dtype=np.int32)
    ks, vs = rng.standard_normal((T, S, Hkv, d)), rng.standard_normal((T, S, Hkv, d))
    for t in range(T):
        O.kv_append(kp, vp, kbar, table, lengths, ks[t], vs[t], block)
        for s in range(S):
            page, slot = table[s, t // block], t % block
            written = ks[t - slot : t + 1, s]  # the rows of this page so far, [slot + 1, Hkv, d]
            np.testing.assert_allclose(kbar[page], written.mean(axis=0), rtol=1e-13)
    assert (lengths == T).all()
    for s in range(S):
        np.testing.assert_array_equal(O.paged_gather(kp, table, s, T, block), ks[:, s].transpose(1, 0, 2))
        np.testing.assert_array_equal(O.paged_gather(vp, table, s, T, block), vs[:, s].transpose(1, 0, 2))
    np.testing.assert_allclose(O.paged_block_means(kp, table, lengths, block, n_pages), kbar, rtol=1e-13)


def test_page_means_equal_the_contiguous_block_means():
    rng = np.random.default_rng(4)
    S, Hkv, Lmax, d, block = 3, 2, 100, 8, 32
    kc = rng.standard_normal((S, Hkv, Lmax, d))
    lengths = np.array([100, 33, 64], dtype=np.int32)
    kp, _, table = build_paged(kc, kc, lengths, block, rng)
    kb = O.paged_block_means(kp, table, lengths, block, kp.shape[0])
    for s in range(S):
        ref = O.block_means(kc[s : s + 1, :, : lengths[s]], block)[0]  # [Hkv, nB, d]
        for j in range(ref.shape[1]):
            np.testing.assert_allclose(kb[table[s, j]], ref[:, j], rtol=1e-13)
