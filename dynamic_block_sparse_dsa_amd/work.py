"""Work accounting: the algorithmic FLOPs and bytes a call must do.

These counts price only what the method has to do (the executed tiles of the
sparse attention, the bytes a decode step must read), never the dense work it
skips; they are the numerators of the roofline fractions.
"""

from __future__ import annotations

import numpy as np


def dense_pairs(n_tokens: int) -> int:
    """Query-key pairs of dense attention over one sequence (every pair)."""
    return n_tokens * n_tokens


def dense_growth(n_from: int, n_to: int) -> float:
    """Factor by which dense attention work grows from n_from to n_to tokens."""
    return (n_to / n_from) ** 2


def prefill_tiles(cnt: np.ndarray, group: int) -> int:
    """Executed (query block, key block) tiles summed over the query heads.

    cnt: [B, Hkv, nB] kept blocks per row of each selection unit; every query
    head of a group runs the group's tiles."""
    return int(np.asarray(cnt, dtype=np.int64).sum()) * group


def prefill_flops(cnt: np.ndarray, group: int, block: int, head_dim: int) -> int:
    """MFMA work of the sparse attention: 2*b*b*d for Q K^T plus 2*b*b*d for
    P V per executed tile, the diagonal tile counted whole."""
    return prefill_tiles(cnt, group) * 4 * block * block * head_dim


def prefill_unique_bytes(batch: int, hq: int, hkv: int, n: int, d: int) -> int:
    """Q, K, V read once and O written once, bf16."""
    return 2 * n * d * batch * (2 * hq + 2 * hkv)


def decode_bytes(n_seq: int, hq: int, hkv: int, cache_len: int, d: int, block: int, kept: int) -> int:
    """Bytes one decode step must move: the kept K and V blocks (bf16), the
    fp32 block means of the whole key cache, q and o (bf16) and the indices."""
    n_blocks = -(-cache_len // block)
    kv = n_seq * hkv * kept * block * d * 2 * 2
    kbar = n_seq * hkv * n_blocks * d * 4
    qo = n_seq * hq * d * 2 * 2
    idx = n_seq * hkv * kept * 4
    return kv + kbar + qo + idx


def decode_flops(n_seq: int, hq: int, kept: int, block: int, d: int, n_blocks: int) -> int:
    """Score scan (2*d per block per head) plus attention (4*d per key per head)."""
    return n_seq * hq * (2 * d * n_blocks + 4 * d * kept * block)


def paged_decode_bytes(lengths, idx, cnt, hq: int, d: int, block: int, kv_bytes: int = 2, row_scales: bool = False) -> int:
    """Bytes one paged decode step must move with a length per sequence: per
    (sequence, KV head) the fp32 means of its ceil(L / block) pages and the
    valid rows of its kept pages (K and V: kv_bytes per element, bf16 = 2,
    E4M3 = 1, plus a 4-byte scale per K and V row with row_scales), plus q, o
    and the indices.
    lengths [S]; idx [S, Hkv, kmax]; cnt [S, Hkv] (numpy)."""
    S, hkv = cnt.shape
    total = 0
    for s in range(S):
        L = int(lengths[s])
        nb = -(-L // block)
        for g in range(hkv):
            rows = sum(min(block, L - int(j) * block) for j in idx[s, g, : cnt[s, g]])
            total += nb * d * 4 + rows * d * kv_bytes * 2 + int(cnt[s, g]) * 4
            if row_scales:
                total += rows * 4 * 2
    return total + S * hq * d * 2 * 2

