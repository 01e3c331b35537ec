"""Pins of the oracle's backward (O5) against things other than its own
formulas: central finite differences of the forward, torch autograd of a
dense causal attention (the special case where every block is kept), and
closed forms.  CPU only."""

import numpy as np
import pytest
import torch

import oracle as O


def _random_selection(rng, B, Hkv, nB, k, flags=3):
    """A valid ascending selection per (b, g, i) with the forced blocks."""
    km = O.kmax(nB, k, 0, 1, flags, True, nB)
    idx = np.full((B, Hkv, nB, km), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv, nB), dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            for i in range(nB):
                f = O.forced_set(i + 1, flags)
                kb = O.row_budget(i + 1, k, 0, 1, len(f))
                rest = [j for j in range(i + 1) if j not in f]
                pick = sorted(set(f) | set(rng.choice(rest, size=kb - len(f), replace=False).tolist())) if kb > len(f) \
                    else sorted(f)
                idx[b, g, i, : len(pick)] = pick
                cnt[b, g, i] = len(pick)
    return idx, cnt


def _case(seed, B=1, Hq=2, Hkv=1, N=37, d=8, block=8, k=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d))
    kk = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    do = rng.standard_normal((B, Hq, N, d))
    idx, cnt = _random_selection(rng, B, Hkv, O.n_blocks(N, block), k)
    return q, kk, v, do, idx, cnt, block


@pytest.mark.parametrize("seed,Hq,Hkv,N,d,block,k", [(0, 2, 1, 37, 8, 8, 2), (1, 3, 3, 20, 4, 4, 3),
                                                      (2, 4, 2, 33, 8, 16, 1)])
def test_backward_matches_central_differences(seed, Hq, Hkv, N, d, block, k):
    q, kk, v, do, idx, cnt, block = _case(seed, 1, Hq, Hkv, N, d, block, k)
    dq, dk, dv = O.attend_backward(q, kk, v, do, idx, cnt, block)

    def loss(q_, k_, v_):
        o, _ = O.attend(q_, k_, v_, idx, cnt, block)
        return float((o * do).sum())

    rng = np.random.default_rng(100 + seed)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", kk, dk), ("v", v, dv)):
        for _ in range(12):
            pos = tuple(int(rng.integers(s)) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[pos] += eps
            xm[pos] -= eps
            args_p = [q, kk, v]
            args_m = [q, kk, v]
            j = "qkv".index(name)
            args_p[j], args_m[j] = xp, xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])


@pytest.mark.parametrize("Hq,Hkv,N,d,block", [(2, 2, 50, 8, 16), (4, 2, 64, 16, 16), (3, 1, 21, 4, 8)])
def test_backward_dense_equals_autograd_of_causal_sdpa(Hq, Hkv, N, d, block):
    """k >= number of blocks keeps every causal key: the gradients are those
    of dense causal attention (torch autograd, float64, heads repeated for
    GQA so the KV gradients sum over the group)."""
    rng = np.random.default_rng(N + d)
    q = rng.standard_normal((1, Hq, N, d))
    kk = rng.standard_normal((1, Hkv, N, d))
    v = rng.standard_normal((1, Hkv, N, d))
    do = rng.standard_normal((1, Hq, N, d))
    nB = O.n_blocks(N, block)
    sc = O.block_scores(O.block_means(q, block), O.block_means(kk, block), 1.0 / np.sqrt(d))
    idx, cnt, _ = O.select_topk(sc, nB)
    dq, dk, dv = O.attend_backward(q, kk, v, do, idx, cnt, block)

    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(kk, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    G = Hq // Hkv
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1),
                                                         is_causal=True)
    o.backward(torch.tensor(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_backward_closed_forms():
    q, kk, v, do, idx, cnt, block = _case(5, 1, 4, 2, 40, 8, 8, 2)
    dq, dk, dv = O.attend_backward(q, kk, v, do, idx, cnt, block)
    # every row's weights sum to one: the value gradients of a KV head add up
    # to the sum of its query heads' output gradients
    G = 2
    for g in range(2):
        np.testing.assert_allclose(dv[0, g].sum(axis=0), do[0, g * G:(g + 1) * G].sum(axis=(0, 1)), rtol=1e-12,
                                   atol=1e-12)
    # keys that no row keeps get exactly zero gradient
    seen = np.zeros((1, 2, 40), dtype=bool)
    for g in range(2):
        for i in range(idx.shape[2]):
            for j in idx[0, g, i, : cnt[0, g, i]]:
                seen[0, g, j * block: min(40, (j + 1) * block)] = True
    assert (dk[~seen] == 0).all() and (dv[~seen] == 0).all()
    # all keys of a head equal: every row's logits are equal, so dQ = 0
    k_same = np.broadcast_to(kk[:, :, :1], kk.shape).copy()
    dq2, _, _ = O.attend_backward(q, k_same, v, do, idx, cnt, block)
    assert np.abs(dq2).max() < 1e-12


def test_backward_with_given_output_reproduces_exact_path():
    """Handing the exact forward output as ``o`` gives the same gradients as
    the default (the identity sum_c w_c dw_c = do . o)."""
    q, kk, v, do, idx, cnt, block = _case(7, 1, 4, 2, 45, 8, 8, 3)
    o, _ = O.attend(q, kk, v, idx, cnt, block)
    a = O.attend_backward(q, kk, v, do, idx, cnt, block)
    b = O.attend_backward(q, kk, v, do, idx, cnt, block, o=o)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-10, atol=1e-12)
