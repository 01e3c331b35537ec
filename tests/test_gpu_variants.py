"""GPU parity of the selection variants (through the C ABI) against the fp64
oracle on the same seeded inputs: global anchors + a local window as the
forced set, threshold selection, the entropy budget, and the bitmap form of
a selection.

Bars as for the plain path: every row's selection is the oracle's, except
in flagged rows (a near-tie at the m-th candidate, a share within 1e-3 of the
threshold, or an exp(entropy) within 1e-4 of an integer), where it must be
one of the accepted sets; attention over the GPU's sets within max-abs 2e-2,
mean-abs 2e-3 and LSE 1e-3; bitmaps bit-exact.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import dynamic_block_sparse_dsa_amd as dsa
from dynamic_block_sparse_dsa_amd.inputs import WORKLOADS, Workload, make_decode, make_prefill
from test_gpu_parity import check_out, check_rows, np64, say
from test_gpu_backward import check_grad

pytestmark = pytest.mark.gpu


def spec_of(sel):
    return O.SelectSpec(mode=sel.get("select_mode", 0), anchors=max(1, sel.get("n_anchor", 0)),
                        window=max(1, sel.get("window", 0)), threshold=sel.get("threshold", 0.0),
                        k_min=sel.get("k_min", 0), k_max=sel.get("k_max", 0))


def check_bitmap(idx, cnt, n_cols):
    bm = dsa.bitmap(idx, cnt, n_cols)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    gc = cnt.cpu().numpy() if cnt is not None else np.full(gi.shape[:-1], gi.shape[-1], dtype=np.int32)
    want = O.bitmap(gi, gc, n_cols).view(np.int32)
    assert np.array_equal(bm.cpu().numpy(), want)


def planted(name, B, Hq, Hkv, N, d, b, topk, amp, seed):
    return Workload(name, "prefill", B, Hq, Hkv, N, d, b, topk, structure="planted", amplitude=amp, seed=seed)


CASES = [
    # name, workload, flags, selection arguments
    ("anchors3_window2_k8", planted("a", 1, 4, 2, 2048, 128, 64, 8, 2.0, 41), 3, dict(n_anchor=3, window=2)),
    ("anchors2_sink_only_k5", planted("b", 1, 2, 2, 1500, 64, 64, 5, 2.0, 42), 1, dict(n_anchor=2)),
    ("window4_diag_only_b128", planted("c", 1, 2, 1, 3000, 128, 128, 6, 2.0, 43), 2, dict(window=4)),
    ("anchors4_window4_long_rows", Workload("d", "prefill", 1, 1, 1, 64 * 1300, 64, 64, 40, seed=44), 3,
     dict(n_anchor=4, window=4)),
    ("threshold_0.05_amp8", planted("e", 1, 8, 2, 4096, 128, 64, 0, 8.0, 45), 3,
     dict(select_mode=1, threshold=0.05)),
    ("threshold_0.1_anchors2_window2", planted("f", 1, 4, 4, 2048, 128, 64, 0, 6.0, 46), 3,
     dict(select_mode=1, threshold=0.1, n_anchor=2, window=2)),
    ("threshold_0.01_sink_only_b128", planted("g", 2, 2, 2, 5000, 64, 128, 0, 8.0, 47), 1,
     dict(select_mode=1, threshold=0.01)),
    ("threshold_0.002_long_rows", planted("h", 1, 1, 1, 64 * 1100, 64, 64, 0, 8.0, 48), 3,
     dict(select_mode=1, threshold=0.002)),
    ("entropy_2_32_amp8", planted("i", 1, 8, 2, 4096, 128, 64, 0, 8.0, 49), 3, dict(select_mode=2, k_min=2, k_max=32)),
    ("entropy_1_8_plain", Workload("j", "prefill", 1, 2, 2, 1024, 64, 64, 0, seed=50), 3,
     dict(select_mode=2, k_min=1, k_max=8)),
    ("entropy_3_200_long_rows", planted("k", 1, 1, 1, 64 * 1100, 64, 64, 0, 8.0, 51), 3,
     dict(select_mode=2, k_min=3, k_max=200, n_anchor=2, window=2)),
]


@pytest.mark.parametrize("name,w,flags,sel", CASES, ids=[c[0] for c in CASES])
def test_prefill_selection_variant(cuda_device, name, w, flags, sel):
    say(f"variant {name}: B{w.batch} Hq{w.n_q_heads} Hkv{w.n_kv_heads} N{w.seq_len} d{w.head_dim} b{w.block} {sel}")
    q, k, v = make_prefill(w, device=cuda_device)
    o, lse, idx, cnt = dsa.prefill(q, k, v, w.block, w.topk, w.topk_num, w.topk_den, flags, **sel)
    torch.cuda.synchronize()
    qn, kn, vn = np64(q), np64(k), np64(v)
    ref = O.prefill(qn, kn, vn, w.block, w.topk, w.topk_num, w.topk_den, flags, attend_blocks=[], spec=spec_of(sel))
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    assert gidx.shape[-1] == ref["idx"].shape[-1]
    check_rows(ref["rows"], gidx, gcnt)
    say(f"variant {name}: kept per row min {gcnt.min()} mean {gcnt.mean():.2f} max {gcnt.max()} (width {gidx.shape[-1]})")
    nB = w.n_blocks
    # attention over the GPU's sets: every row for short sequences, a sample otherwise
    units = None if w.seq_len <= 5000 else [(b, h, i) for b in range(w.batch) for h in range(w.n_q_heads)
                                             for i in (0, 1, nB // 2, nB - 1)]
    o_ref, lse_ref = O.attend(qn, kn, vn, gidx, gcnt, w.block, units=units)
    if units is None:
        check_out(np64(o), o_ref, np64(lse), lse_ref, name)
    else:
        for (b, h, i) in units:
            lo, hi = i * w.block, min(w.seq_len, (i + 1) * w.block)
            check_out(np64(o[b, h, lo:hi]), o_ref[b, h, lo:hi], np64(lse[b, h, lo:hi]), lse_ref[b, h, lo:hi],
                      f"{name} b{b} h{h} i{i}")
    check_bitmap(idx, cnt, nB)


def test_threshold_selection_actually_varies(cuda_device):
    """With planted targets and a threshold the kept count differs between
    rows (not just the forced blocks, not a constant)."""
    w = planted("v", 1, 4, 4, 4096, 128, 64, 0, 8.0, 52)
    q, k, v = make_prefill(w, device=cuda_device)
    _, _, _, cnt = dsa.prefill(q, k, v, w.block, 0, 0, 1, 3, select_mode=1, threshold=0.05)
    c = cnt.cpu().numpy()[:, :, 2:]
    assert c.max() > 2 and len(np.unique(c)) >= 3, np.unique(c)


def test_full_prefill_n8192_variants(cuda_device):
    """The 8 192-token workload with threshold and entropy selection: every
    row's selection checked, attention on sampled query blocks."""
    w = WORKLOADS["prefill_n8192_h32"]
    q, k, v = make_prefill(w, device=cuda_device)
    s = 1.0 / math.sqrt(w.head_dim)
    for sel in (dict(select_mode=1, threshold=0.02), dict(select_mode=2, k_min=2, k_max=24, n_anchor=2, window=2)):
        say(f"full prefill_n8192_h32 {sel}")
        o, lse, idx, cnt = dsa.prefill(q, k, v, w.block, 0, 0, 1, 3, **sel)
        torch.cuda.synchronize()
        gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
        flagged = 0
        for h in range(w.n_kv_heads):
            qn, kn = np64(q[:, h : h + 1]), np64(k[:, h : h + 1])
            sc = O.block_scores(O.block_means(qn, w.block), O.block_means(kn, w.block), s)
            _, _, rows = O.select_topk(sc, 0, 0, 1, 3, spec=spec_of(sel))
            flagged += check_rows(rows, gidx[:, h : h + 1], gcnt[:, h : h + 1])[0]
        say(f"full {sel}: {flagged} flagged rows; kept per row mean {gcnt.mean():.2f} max {gcnt.max()}")
        for (h, i) in [(0, 127), (13, 64), (31, 5)]:
            qn, kn, vn = np64(q[:, h : h + 1]), np64(k[:, h : h + 1]), np64(v[:, h : h + 1])
            o_ref, lse_ref = O.attend(qn, kn, vn, gidx[:, h : h + 1], gcnt[:, h : h + 1], w.block, units=[(0, 0, i)])
            lo, hi = i * w.block, (i + 1) * w.block
            check_out(np64(o[:, h, lo:hi]), o_ref[:, 0, lo:hi], np64(lse[:, h, lo:hi]), lse_ref[:, 0, lo:hi],
                      f"n8192 {sel} h{h} i{i}")
        check_bitmap(idx, cnt, w.n_blocks)


def test_backward_over_a_threshold_selection(cuda_device):
    """The backward takes the variant's index width and per-row counts."""
    w = planted("w", 1, 4, 2, 1500, 128, 64, 0, 6.0, 53)
    sel = dict(select_mode=1, threshold=0.05, n_anchor=2, window=2)
    q, k, v = make_prefill(w, device=cuda_device)
    o, lse, idx, cnt = dsa.prefill(q, k, v, w.block, 0, 0, 1, 3, **sel)
    g = torch.Generator(device=cuda_device)
    g.manual_seed(54)
    dout = torch.randn(q.shape, generator=g, device=cuda_device, dtype=torch.float32).to(torch.bfloat16)
    dq, dk, dv = dsa.attn_backward(q, k, v, o, lse, dout, idx, cnt, w.block, 0, 0, 1, 3, **sel)
    torch.cuda.synchronize()
    ref = O.attend_backward(np64(q), np64(k), np64(v), np64(dout), idx.cpu().numpy(), cnt.cpu().numpy(), w.block,
                            o=np64(o))
    for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        check_grad("threshold", np64(got), want, name)


DECODE_CASES = [
    ("anchors2_window3", Workload("x", "decode", 4, 8, 2, 64 * 300, 128, 64, 12, structure="planted", amplitude=8.0,
                                  seed=55), dict(n_anchor=2, window=3)),
    ("window6_b128_ragged", Workload("y", "decode", 3, 4, 4, 128 * 70 + 17, 64, 128, 9, seed=56), dict(window=6)),
]


@pytest.mark.parametrize("name,w,sel", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_anchors_and_window(cuda_device, name, w, sel):
    say(f"decode variant {name}: S{w.batch} Hq{w.n_q_heads} Hkv{w.n_kv_heads} L{w.seq_len} {sel}")
    q, kc, vc = make_decode(w, device=cuda_device)
    kbar = dsa.kv_block_means(kc, w.block)
    o, lse, idx = dsa.decode(q, kc, vc, kbar, w.block, w.topk, 0, 1, 3, **sel)
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()
    G = w.group
    for s in range(w.batch):
        for g in range(w.n_kv_heads):
            qn = np64(q[s : s + 1, g * G : (g + 1) * G])
            kn, vn = np64(kc[s : s + 1, g : g + 1]), np64(vc[s : s + 1, g : g + 1])
            ref = O.decode(qn, kn, vn, w.block, w.topk, 0, 1, 3, units=[], spec=spec_of(sel))
            check_rows(ref["rows"], gidx[s : s + 1, g : g + 1, None, :],
                       np.full((1, 1, 1), gidx.shape[-1], dtype=np.int32))
            keys = np.concatenate([np.arange(j * w.block, min(w.seq_len, (j + 1) * w.block)) for j in gidx[s, g]])
            for hh in range(G):
                logits = (kn[0, 0, keys] @ qn[0, hh]) / math.sqrt(w.head_dim)
                wts = np.exp(logits - logits.max())
                check_out(np64(o[s, g * G + hh])[None], ((wts / wts.sum()) @ vn[0, 0, keys])[None],
                          np.array([float(lse[s, g * G + hh])]), np.array([logits.max() + math.log(wts.sum())]),
                          f"decode {name} s{s} g{g} h{hh}")
    check_bitmap(idx, None, w.n_blocks)
