"""GPU parity of the paged decode (per-sequence lengths, block table, token
appends, per-page block means) through the C ABI against the fp64 oracle.

Caches come from the decode input generator, poisoned past each sequence's
length and scattered into shuffled pages.  Bars as for the contiguous decode:
selections bit-exact except in flagged near-tie rows (accepted sets there),
O within max-abs 2e-2 / mean-abs 2e-3, LSE 1e-3, page means to fp32
rounding (rel 1e-5); appended pools bit-exact, and the means written by an
append bit-identical to dsa_paged_kv_block_means (same summation order).
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import dynamic_block_sparse_dsa_amd as dsa
from dynamic_block_sparse_dsa_amd.inputs import WORKLOADS, Workload, make_decode
from test_gpu_parity import check_out, check_rows, np64, say

pytestmark = pytest.mark.gpu
POISON = 30000.0


def to_paged(kc, vc, lengths, block, seed, extra=5):
    """Contiguous caches [S, Hkv, L, d] -> shuffled page pools, the table and
    the lengths tensor; rows past each length are poisoned first."""
    S, Hkv, L, d = kc.shape
    mb = -(-L // block)
    kc, vc = kc.clone(), vc.clone()
    for s in range(S):
        kc[s, :, lengths[s]:] = POISON
        vc[s, :, lengths[s]:] = POISON
    pad = mb * block - L
    if pad:
        kc = torch.nn.functional.pad(kc, (0, 0, 0, pad), value=POISON)
        vc = torch.nn.functional.pad(vc, (0, 0, 0, pad), value=POISON)
    n_pages = S * mb + extra
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    perm = torch.randperm(n_pages, generator=g)
    table = perm[: S * mb].view(S, mb).to(torch.int32).to(kc.device)
    kp = torch.full((n_pages, Hkv, block, d), POISON, dtype=torch.bfloat16, device=kc.device)
    vp = torch.full_like(kp, POISON)
    flat = table.reshape(-1).long()
    kp[flat] = kc.view(S, Hkv, mb, block, d).permute(0, 2, 1, 3, 4).reshape(S * mb, Hkv, block, d)
    vp[flat] = vc.view(S, Hkv, mb, block, d).permute(0, 2, 1, 3, 4).reshape(S * mb, Hkv, block, d)
    lens = torch.tensor(lengths, dtype=torch.int32, device=kc.device)
    return kp, vp, table, lens


def paged_case(dev, w, lengths, flags=3, n_anchor=0, window=0, units=None, seed=0):
    q, kc, vc = make_decode(w, device=dev)
    kp, vp, table, lens = to_paged(kc, vc, lengths, w.block, seed)
    shape = dsa.paged_shape(kp, table, w.n_q_heads)
    kbar = torch.zeros((kp.shape[0], w.n_kv_heads, w.head_dim), dtype=torch.float32, device=dev)
    dsa.dsa_paged_kv_block_means(shape, kp, table, lens, kbar)
    o, lse, idx, cnt = dsa.paged_decode(q, kp, vp, kbar, table, lens, w.block, w.topk, w.topk_num, w.topk_den, flags,
                                        n_anchor=n_anchor, window=window)
    torch.cuda.synchronize()
    return q, kp, vp, kbar, table, lens, o, lse, idx, cnt


def check_against_oracle(name, w, q, kp, vp, kbar, table, lens, o, lse, idx, cnt, flags, spec, units):
    tb, ln = table.cpu().numpy(), lens.cpu().numpy()
    as64 = lambda t: t.numpy() if t.dtype == torch.float64 else np64(t)
    kp64, vp64 = as64(kp), as64(vp)
    # page means of the used pages
    ref_kb = O.paged_block_means(kp64, tb, ln, w.block, kp.shape[0])
    used = sorted({int(tb[s, j]) for s in range(w.batch) for j in range(-(-int(ln[s]) // w.block))})
    np.testing.assert_allclose(np64(kbar)[used], ref_kb[used], rtol=1e-5, atol=1e-6)
    ref = O.paged_decode(np64(q), kp64, vp64, tb, ln, w.block, w.topk, w.topk_num, w.topk_den, flags, spec,
                         units=units)
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for s in range(w.batch):
        for g in range(w.n_kv_heads):
            rs = ref["rows"][s * w.n_kv_heads + g]
            if rs is None:  # empty sequence
                assert gcnt[s, g] == 0 and (gidx[s, g] == -1).all()
                G = w.group
                assert (o[s, g * G : (g + 1) * G].float() == 0).all()
                assert torch.isneginf(lse[s, g * G : (g + 1) * G]).all()
                continue
            check_rows([rs], gidx[s : s + 1, g : g + 1, None], gcnt[s : s + 1, g : g + 1, None])
    todo = units if units is not None else [(s, g) for s in range(w.batch) for g in range(w.n_kv_heads)]
    G = w.group
    for (s, g) in todo:
        if ln[s] == 0:
            continue
        # the oracle evaluated on the GPU's own kept blocks (accepted sets)
        keys = np.concatenate([np.arange(j * w.block, min(int(ln[s]), (j + 1) * w.block))
                               for j in gidx[s, g, : gcnt[s, g]]])
        kseq = O.paged_gather(kp64, tb, s, int(ln[s]), w.block)[g]
        vseq = O.paged_gather(vp64, tb, s, int(ln[s]), w.block)[g]
        for hh in range(G):
            logits = (kseq[keys] @ np64(q[s, g * G + hh])) / math.sqrt(w.head_dim)
            wts = np.exp(logits - logits.max())
            check_out(np64(o[s, g * G + hh])[None], ((wts / wts.sum()) @ vseq[keys])[None],
                      np.array([float(lse[s, g * G + hh])]), np.array([logits.max() + math.log(wts.sum())]),
                      f"{name} s{s} g{g} h{hh}")


CASES = [
    # name, workload, lengths, flags, n_anchor, window
    ("d128_b64_g4_varlen", Workload("p", "decode", 6, 8, 2, 64 * 40, 128, 64, 8, structure="planted", amplitude=8.0,
                                    seed=71), [2560, 1000, 1, 64, 65, 0], 3, 0, 0),
    ("d64_b128_g1_anchors_window", Workload("q", "decode", 4, 4, 4, 128 * 20 + 50, 64, 128, 6, seed=72),
     [2610, 2560, 129, 777], 3, 2, 3),
    ("d128_b128_g8_sink_only", Workload("r", "decode", 3, 8, 1, 128 * 12, 128, 128, 4, seed=73), [1536, 300, 1], 1, 3,
     0),
    ("d64_b64_g2_fraction", Workload("t", "decode", 3, 4, 2, 64 * 64, 64, 64, 0, 1, 4, seed=74), [4096, 2049, 640], 3,
     0, 0),
]


@pytest.mark.parametrize("name,w,lengths,flags,n_anchor,window", CASES, ids=[c[0] for c in CASES])
def test_paged_decode_small(cuda_device, name, w, lengths, flags, n_anchor, window):
    say(f"paged {name}: S{w.batch} Hq{w.n_q_heads} Hkv{w.n_kv_heads} cap{w.seq_len} d{w.head_dim} b{w.block} "
        f"lengths {lengths}")
    r = paged_case(cuda_device, w, lengths, flags, n_anchor, window, seed=1)
    spec = O.SelectSpec(anchors=max(1, n_anchor), window=max(1, window))
    check_against_oracle(name, w, *r, flags, spec, None)


def test_paged_matches_contiguous_decode(cuda_device):
    """Every sequence at full length with shuffled pages: the same selection
    as the contiguous decode and the same outputs to rounding."""
    w = Workload("u", "decode", 8, 16, 4, 64 * 300, 128, 64, 16, structure="planted", amplitude=8.0, seed=75)
    q, kc, vc = make_decode(w, device=cuda_device)
    kbar_c = dsa.kv_block_means(kc, w.block)
    o_c, lse_c, idx_c = dsa.decode(q, kc, vc, kbar_c, w.block, w.topk)
    kp, vp, table, lens = to_paged(kc, vc, [w.seq_len] * w.batch, w.block, 2)
    kbar = torch.zeros((kp.shape[0], w.n_kv_heads, w.head_dim), dtype=torch.float32, device=cuda_device)
    dsa.dsa_paged_kv_block_means(dsa.paged_shape(kp, table, w.n_q_heads), kp, table, lens, kbar)
    o, lse, idx, cnt = dsa.paged_decode(q, kp, vp, kbar, table, lens, w.block, w.topk)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_c)
    assert (cnt == w.topk).all()
    assert (o.float() - o_c.float()).abs().max() <= 1e-2
    assert (lse - lse_c).abs().max() <= 1e-4


def test_appends_match_the_oracle_and_the_page_means(cuda_device):
    w = Workload("v", "decode", 4, 4, 2, 64 * 6, 128, 64, 4, seed=76)
    start = [10, 63, 64, 384]  # the last one is full: appends leave it alone
    q, kc, vc = make_decode(w, device=cuda_device)
    kp, vp, table, lens = to_paged(kc, vc, start, w.block, 3)
    shape = dsa.paged_shape(kp, table, w.n_q_heads)
    kbar = torch.zeros((kp.shape[0], w.n_kv_heads, w.head_dim), dtype=torch.float32, device=cuda_device)
    dsa.dsa_paged_kv_block_means(shape, kp, table, lens, kbar)
    kp_o, vp_o, kb_o = np64(kp), np64(vp), np64(kbar)
    ln_o = lens.cpu().numpy().copy()
    tb = table.cpu().numpy()
    g = torch.Generator(device=cuda_device)
    g.manual_seed(77)
    for step in range(70):
        kn = torch.randn((w.batch, w.n_kv_heads, w.head_dim), generator=g, device=cuda_device).to(torch.bfloat16)
        vn = torch.randn((w.batch, w.n_kv_heads, w.head_dim), generator=g, device=cuda_device).to(torch.bfloat16)
        dsa.dsa_paged_kv_append(shape, kn, vn, table, lens, kp, vp, kbar)
        for s in range(w.batch):  # the oracle's append, skipping full sequences
            if ln_o[s] >= w.seq_len:
                continue
            one = np.array([ln_o[s]], dtype=np.int32)
            O.kv_append(kp_o, vp_o, kb_o, tb[s : s + 1], one, np64(kn)[s : s + 1], np64(vn)[s : s + 1], w.block)
            ln_o[s] = one[0]
    torch.cuda.synchronize()
    assert (lens.cpu().numpy() == ln_o).all(), (lens, ln_o)
    assert ln_o[3] == w.seq_len
    np.testing.assert_array_equal(np64(kp), kp_o)
    np.testing.assert_array_equal(np64(vp), vp_o)
    np.testing.assert_allclose(np64(kbar), kb_o, rtol=1e-5, atol=1e-6)
    # recomputing every page's mean gives the same bits as the appends left
    kbar2 = kbar.clone()
    dsa.dsa_paged_kv_block_means(shape, kp, table, lens, kbar2)
    torch.cuda.synchronize()
    assert torch.equal(kbar2, kbar)


def test_paged_decode_full_size_sampled(cuda_device):
    """The 32-sequence, 65 536-token decode workload in shuffled pages, with
    varied lengths; selection and attention checked on sampled units."""
    w = WORKLOADS["decode_s32_l65536"]
    lengths = [65536 - 2001 * s for s in range(w.batch)]  # 65 536 down to 3 505, most ragged
    say("paged full: building the paged cache")
    r = paged_case(cuda_device, w, lengths, seed=4)
    units = [(0, 0), (5, 3), (17, 7), (31, 2)]
    # the oracle needs the sampled sequences only: restrict to them
    q, kp, vp, kbar, table, lens, o, lse, idx, cnt = r
    say("paged full: oracle on sampled units")
    tb, ln = table.cpu().numpy(), lens.cpu().numpy()
    for (s, g) in units:
        L = int(ln[s])
        pages = [int(tb[s, j]) for j in range(-(-L // w.block))]
        kseq = np64(kp[pages, g]).reshape(-1, w.head_dim)[:L]
        vseq = np64(vp[pages, g]).reshape(-1, w.head_dim)[:L]
        G = w.group
        ref = O.decode(np64(q[s : s + 1, g * G : (g + 1) * G]), kseq[None, None], vseq[None, None], w.block, w.topk,
                       units=[(0, 0)])
        check_rows(ref["rows"], idx.cpu().numpy()[s : s + 1, g : g + 1, None],
                   cnt.cpu().numpy()[s : s + 1, g : g + 1, None])
        np.testing.assert_allclose(np64(kbar[pages, g]), ref["kbar"][0, 0], rtol=1e-5, atol=1e-6)
        keys = np.concatenate([np.arange(j * w.block, min(L, (j + 1) * w.block))
                               for j in idx.cpu().numpy()[s, g, : int(cnt[s, g])]])
        for hh in range(G):
            logits = (kseq[keys] @ np64(q[s, g * G + hh])) / math.sqrt(w.head_dim)
            wts = np.exp(logits - logits.max())
            check_out(np64(o[s, g * G + hh])[None], ((wts / wts.sum()) @ vseq[keys])[None],
                      np.array([float(lse[s, g * G + hh])]), np.array([logits.max() + math.log(wts.sum())]),
                      f"paged full s{s} g{g} h{hh}")


# ------------------------------------------------------------------ FP8 cache
def quantize_pools(kp, vp, shape):
    n_pages, Hkv, b, d = kp.shape
    k8 = torch.empty((n_pages, Hkv, b, d), dtype=torch.uint8, device=kp.device)
    v8 = torch.empty_like(k8)
    ks = torch.empty((n_pages, Hkv, b), dtype=torch.float32, device=kp.device)
    vs = torch.empty_like(ks)
    dsa.dsa_paged_quantize_fp8(shape, kp, vp, k8, v8, ks, vs)
    return k8, v8, ks, vs


def test_fp8_quantization_is_bit_exact(cuda_device):
    g = torch.Generator(device=cuda_device)
    g.manual_seed(81)
    for d, b in ((128, 64), (64, 128)):
        kp = (torch.randn((5, 2, b, d), generator=g, device=cuda_device) * 3).to(torch.bfloat16)
        vp = (torch.randn((5, 2, b, d), generator=g, device=cuda_device) * 1e-3).to(torch.bfloat16)
        kp[1, 0, 3] = 0  # an all-zero row
        kp[2, 1, 7] *= 1e4
        shape = dsa.paged_shape(kp, torch.zeros((1, 4), dtype=torch.int32), 2)
        k8, v8, ks, vs = quantize_pools(kp, vp, shape)
        torch.cuda.synchronize()
        for pool, codes, scales in ((kp, k8, ks), (vp, v8, vs)):
            rc, rs = O.quantize_fp8(np64(pool))
            np.testing.assert_array_equal(codes.cpu().numpy(), rc)
            np.testing.assert_array_equal(scales.cpu().numpy(), rs)


FP8_CASES = [CASES[0], CASES[1]]


@pytest.mark.parametrize("name,w,lengths,flags,n_anchor,window", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_fp8_paged_decode_small(cuda_device, name, w, lengths, flags, n_anchor, window):
    say(f"fp8 paged {name}: lengths {lengths}")
    q, kc, vc = make_decode(w, device=cuda_device)
    kp, vp, table, lens = to_paged(kc, vc, lengths, w.block, 5)
    shape = dsa.paged_shape(kp, table, w.n_q_heads)
    k8, v8, ks, vs = quantize_pools(kp, vp, shape)
    kbar = torch.zeros((kp.shape[0], w.n_kv_heads, w.head_dim), dtype=torch.float32, device=cuda_device)
    dsa.dsa_paged_kv_block_means_fp8(shape, k8, ks, table, lens, kbar)
    dshape = dsa.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, shape.seq_len, w.head_dim, w.block, w.topk,
                            w.topk_num, w.topk_den, flags, n_anchor=n_anchor, window=window)
    km = dsa.dsa_decode_kmax(dshape)
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.n_q_heads), dtype=torch.float32, device=cuda_device)
    idx = torch.empty((w.batch, w.n_kv_heads, km), dtype=torch.int32, device=cuda_device)
    cnt = torch.empty((w.batch, w.n_kv_heads), dtype=torch.int32, device=cuda_device)
    dsa.dsa_paged_decode_fp8(dshape, q, k8, v8, ks, vs, kbar, table, lens, o, lse, idx, cnt)
    torch.cuda.synchronize()
    # the oracle sees the dequantized pools (as bf16-free float64 tensors)
    kd = O.dequantize_fp8(k8.cpu().numpy(), ks.cpu().numpy())
    vd = O.dequantize_fp8(v8.cpu().numpy(), vs.cpu().numpy())
    spec = O.SelectSpec(anchors=max(1, n_anchor), window=max(1, window))
    check_against_oracle(name + "_fp8", w, q, torch.from_numpy(kd), torch.from_numpy(vd), kbar, table, lens, o, lse,
                         idx, cnt, flags, spec, None)


def test_fp8_appends(cuda_device):
    w = Workload("f8", "decode", 3, 4, 2, 64 * 4, 128, 64, 4, seed=82)
    start = [0, 63, 256]
    q, kc, vc = make_decode(w, device=cuda_device)
    kp, vp, table, lens = to_paged(kc, vc, start, w.block, 6)
    shape = dsa.paged_shape(kp, table, w.n_q_heads)
    k8, v8, ks, vs = quantize_pools(kp, vp, shape)
    kbar = torch.zeros((kp.shape[0], w.n_kv_heads, w.head_dim), dtype=torch.float32, device=cuda_device)
    dsa.dsa_paged_kv_block_means_fp8(shape, k8, ks, table, lens, kbar)
    o8, ov8, oks, ovs, okb = (x.cpu().numpy().copy() for x in (k8, v8, ks, vs, kbar))
    okb = okb.astype(np.float64)
    ln_o = lens.cpu().numpy().copy()
    tb = table.cpu().numpy()
    g = torch.Generator(device=cuda_device)
    g.manual_seed(83)
    for step in range(70):
        kn = (torch.randn((w.batch, w.n_kv_heads, w.head_dim), generator=g, device=cuda_device) * 2).to(torch.bfloat16)
        vn = torch.randn((w.batch, w.n_kv_heads, w.head_dim), generator=g, device=cuda_device).to(torch.bfloat16)
        dsa.dsa_paged_kv_append_fp8(shape, kn, vn, table, lens, k8, v8, ks, vs, kbar)
        for s in range(w.batch):
            if ln_o[s] >= w.seq_len:
                continue
            one = np.array([ln_o[s]], dtype=np.int32)
            O.kv_append_fp8(o8, ov8, oks, ovs, okb, tb[s : s + 1], one, np64(kn)[s : s + 1], np64(vn)[s : s + 1],
                            w.block)
            ln_o[s] = one[0]
    torch.cuda.synchronize()
    assert (lens.cpu().numpy() == ln_o).all()
    np.testing.assert_array_equal(k8.cpu().numpy(), o8)
    np.testing.assert_array_equal(v8.cpu().numpy(), ov8)
    np.testing.assert_array_equal(ks.cpu().numpy(), oks)
    np.testing.assert_array_equal(vs.cpu().numpy(), ovs)
    np.testing.assert_allclose(np64(kbar), okb, rtol=1e-5, atol=1e-6)
    kbar2 = kbar.clone()
    dsa.dsa_paged_kv_block_means_fp8(shape, k8, ks, table, lens, kbar2)
    torch.cuda.synchronize()
    assert torch.equal(kbar2, kbar)


@pytest.mark.parametrize("lengths,topk,flags", [([64 * 300 - 5, 64 * 120 + 1, 64, 0], 17, 3),
                                                ([64 * 1100, 64 * 700, 64 * 5], 40, 1)])
def test_paged_decode_exact_ties(cuda_device, lengths, topk, flags):
    """Integer-valued block scores (many exact ties) through the page table:
    each sequence's selection equals the oracle's exactly on its own
    ceil(L_s / 64) blocks (ties go to the lower block)."""
    from test_gpu_parity import tied_decode_inputs
    S, Hkv, G, d = len(lengths), 2, 2, 128
    nblk = -(-max(lengths) // 64)
    say(f"paged exact ties lengths {lengths} k{topk} flags{flags}")
    q, kc, vc, v = tied_decode_inputs(cuda_device, S, Hkv, G, nblk, d, seed=topk, tail=0)
    kp, vp, table, lens = to_paged(kc, vc, lengths, 64, seed=topk)
    shape = dsa.paged_shape(kp, table, Hkv * G)
    kbar = torch.zeros((kp.shape[0], Hkv, d), dtype=torch.float32, device=cuda_device)
    dsa.dsa_paged_kv_block_means(shape, kp, table, lens, kbar)
    o, lse, idx, cnt = dsa.paged_decode(q, kp, vp, kbar, table, lens, 64, topk, 0, 1, flags)
    torch.cuda.synchronize()
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for s, L in enumerate(lengths):
        nb = -(-L // 64)
        if nb == 0:
            assert (gcnt[s] == 0).all() and (gidx[s] == -1).all()
            continue
        scores = (v[s : s + 1, :, :nb].astype(np.float64) / math.sqrt(d))[:, :, None, :]
        ref_idx, ref_cnt, _ = O.select_topk(scores, topk, 0, 1, flags, causal=False)
        km = ref_idx.shape[-1]
        assert np.array_equal(gcnt[s], ref_cnt[0, :, 0]), s
        assert np.array_equal(gidx[s, :, :km], ref_idx[0, :, 0]), s
        assert (gidx[s, :, km:] == -1).all(), s
