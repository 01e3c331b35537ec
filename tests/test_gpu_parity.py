"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Bars: block indices bit-exact except in oracle-flagged near-tie rows, where
the GPU's set must be one of the accepted sets; outputs within max-abs 2e-2
and mean-abs 2e-3 (bf16 inputs), compared with the oracle evaluated on the
GPU's own (accepted) index sets; block means and scores to fp32 rounding;
LSE within 1e-3.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
import dynamic_block_sparse_dsa_amd as dsa
from dynamic_block_sparse_dsa_amd.inputs import WORKLOADS, Workload, make_decode, make_prefill

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_ABS = 2e-2, 2e-3, 1e-3


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def shape_of(w: Workload, flags: int = 3):
    return dsa.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block, w.topk, w.topk_num,
                          w.topk_den, flags)


def check_rows(rows, gidx, gcnt):
    """Every row's GPU set is accepted; returns (#flagged, #rows).  A flagged
    row's count may differ from the oracle's own pick (a threshold band, an
    alternative entropy budget): ``accepts`` checks it."""
    flat_idx = gidx.reshape(-1, gidx.shape[-1])
    flat_cnt = gcnt.reshape(-1)
    assert len(rows) == flat_idx.shape[0]
    flagged = 0
    for r, rs in enumerate(rows):
        c = int(flat_cnt[r])
        got = [int(x) for x in flat_idx[r, :c]]
        assert (flat_idx[r, c:] == -1).all(), r
        if not rs.flagged:
            assert c == len(rs.idx), (r, c, rs.idx)
            assert got == rs.idx, (r, got, rs.idx)
        else:
            flagged += 1
            ok, why = O.accepts(rs, got)
            assert ok, (r, why)
    say(f"selection: {len(rows)} rows, {flagged} near-tie flagged (accepted set), 0 unflagged mismatches")
    return flagged, len(rows)


def check_out(o_gpu, o_ref, lse_gpu=None, lse_ref=None, what=""):
    err = np.abs(o_gpu - o_ref)
    assert np.isfinite(o_gpu).all(), what
    lerr = np.abs(lse_gpu - lse_ref).max() if lse_gpu is not None else float("nan")
    say(f"error {what}: O max-abs {err.max():.3g} mean-abs {err.mean():.3g}, LSE max-abs {lerr:.3g}")
    assert err.max() <= O_MAX, (what, err.max())
    assert err.mean() <= O_MEAN, (what, err.mean())
    if lse_gpu is not None:
        assert lerr <= LSE_ABS, (what, lerr)
    return err.max(), err.mean()


def run_steps(shape, q, k, v):
    """The four steps through their own entry points; the block scores both
    from Q and K (dsa_block_scores, whose result the selection uses) and from
    the block means (dsa_block_scores_from_means): the same bits."""
    B, Hq, N, d = q.shape
    Hkv, nB = k.shape[1], shape.n_blocks
    km = dsa.dsa_kmax(shape)
    dev = q.device
    qbar = torch.empty((B, Hq, nB, d), dtype=torch.float32, device=dev)
    kbar = torch.empty((B, Hkv, nB, d), dtype=torch.float32, device=dev)
    sc = torch.empty((B, Hkv, nB, nB), dtype=torch.float32, device=dev)
    sc_means = torch.full((B, Hkv, nB, nB), float("nan"), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Hkv, nB, km), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hkv, nB), dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    sc.fill_(float("nan"))  # every element must be written
    dsa.dsa_block_means(shape, Hq, q, qbar)
    dsa.dsa_block_means(shape, Hkv, k, kbar)
    dsa.dsa_block_scores_from_means(shape, qbar, kbar, sc_means)
    dsa.dsa_block_scores(shape, q, k, sc)
    dsa.dsa_select_topk(shape, sc, idx, cnt)
    dsa.dsa_sparse_attn_fwd(shape, q, k, v, idx, cnt, o, lse)
    torch.cuda.synchronize()
    assert torch.equal(sc, sc_means)
    return dict(qbar=qbar, kbar=kbar, scores=sc, idx=idx, cnt=cnt, o=o, lse=lse)


SMALL = [
    # name, workload, flags
    ("tiny_n1024_d64_k4", WORKLOADS["prefill_tiny_n1024"], 3),
    ("ragged_n1000", Workload("r", "prefill", 1, 2, 2, 1000, 64, 64, 4, seed=21), 3),
    ("gqa_frac_n2048", Workload("g", "prefill", 1, 8, 2, 2048, 128, 64, 0, 15, 100, structure="planted",
                                amplitude=2.0, seed=22), 3),
    ("b128_n1500", Workload("b", "prefill", 1, 2, 2, 1500, 128, 128, 4, seed=23), 3),
    ("d64_b128_gqa2_n777", Workload("c", "prefill", 2, 2, 1, 777, 64, 128, 3, seed=24), 3),
    ("gqa8_b128_n1024", Workload("e", "prefill", 1, 16, 2, 1024, 128, 128, 3, seed=25), 3),
    ("gqa3_n640", Workload("f", "prefill", 1, 6, 2, 640, 128, 64, 3, seed=26), 3),
    ("k1_no_forcing", Workload("h", "prefill", 1, 2, 2, 640, 128, 64, 1, seed=27), 0),
    ("sink_only_k3", Workload("i", "prefill", 1, 2, 2, 640, 128, 64, 3, seed=28), 1),
    ("diag_only_k3", Workload("j", "prefill", 1, 2, 2, 640, 128, 64, 3, seed=29), 2),
    ("dense_k_all", Workload("k", "prefill", 2, 4, 2, 512, 128, 64, 8, seed=30), 3),
    ("short_n37", Workload("l", "prefill", 1, 2, 2, 37, 64, 64, 4, seed=31), 3),
    ("single_row_n1", Workload("m", "prefill", 1, 1, 1, 1, 128, 64, 4, seed=32), 3),
    ("heavy_b128_n2048", Workload("n", "prefill", 1, 2, 2, 2048, 128, 128, 6, structure="heavy", amplitude=3.0,
                                  heavy_frac=0.05, seed=33), 3),
    ("gqa16_d64_n1100", Workload("o", "prefill", 1, 16, 1, 1100, 64, 64, 5, seed=34), 3),
    ("strips_n20000_b64", Workload("s", "prefill", 1, 2, 2, 20000, 64, 64, 6, seed=35), 3),
]


@pytest.mark.parametrize("name,w,flags", SMALL, ids=[c[0] for c in SMALL])
def test_prefill_small(cuda_device, name, w, flags):
    say(f"prefill {name}: B{w.batch} Hq{w.n_q_heads} Hkv{w.n_kv_heads} N{w.seq_len} d{w.head_dim} b{w.block}")
    q, k, v = make_prefill(w, device=cuda_device)
    shape = dsa.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block, w.topk, w.topk_num,
                           w.topk_den, flags)
    g = run_steps(shape, q, k, v)
    o2, lse2, idx2, cnt2 = dsa.prefill(q, k, v, w.block, w.topk, w.topk_num, w.topk_den, flags)
    torch.cuda.synchronize()
    # the fused call runs the same kernels: identical results
    assert torch.equal(idx2, g["idx"]) and torch.equal(cnt2, g["cnt"])
    assert torch.equal(o2, g["o"]) and torch.equal(lse2, g["lse"])
    qn, kn, vn = np64(q), np64(k), np64(v)
    ref = O.prefill(qn, kn, vn, w.block, w.topk, w.topk_num, w.topk_den, flags, attend_blocks=[])
    np.testing.assert_allclose(np64(g["qbar"]), ref["qbar"], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(np64(g["kbar"]), ref["kbar"], rtol=1e-5, atol=1e-6)
    gs = np64(g["scores"])
    fin = np.isfinite(ref["scores"])
    assert (np.isfinite(gs) == fin).all()
    np.testing.assert_allclose(gs[fin], ref["scores"][fin], rtol=1e-4, atol=1e-5)
    gidx, gcnt = g["idx"].cpu().numpy(), g["cnt"].cpu().numpy()
    check_rows(ref["rows"], gidx, gcnt)
    o_ref, lse_ref = O.attend(qn, kn, vn, gidx, gcnt, w.block)
    check_out(np64(g["o"]), o_ref, np64(g["lse"]), lse_ref, name)


def test_unselected_values_do_not_leak(cuda_device):
    """NaN in every V block a query block does not keep leaves that query
    block's output bitwise unchanged (index set held fixed)."""
    w = Workload("p", "prefill", 1, 2, 2, 1024, 128, 64, 4, seed=40)
    say("poison unselected V")
    q, k, v = make_prefill(w, device=cuda_device)
    shape = shape_of(w)
    g = run_steps(shape, q, k, v)
    idx = g["idx"].cpu().numpy()
    for i in (5, 11, 15):
        vp = v.clone()
        for h in range(2):
            keep = set(int(j) for j in idx[0, h, i] if j >= 0)
            for j in range(16):
                if j not in keep:
                    vp[0, h, j * 64 : (j + 1) * 64] = float("nan")
        o = torch.empty_like(q)
        dsa.dsa_sparse_attn_fwd(shape, q, k, vp, g["idx"], g["cnt"], o, None)
        torch.cuda.synchronize()
        assert torch.equal(o[0, :, i * 64 : (i + 1) * 64], g["o"][0, :, i * 64 : (i + 1) * 64]), i


@pytest.mark.parametrize("block", [64, 128])
def test_causal_mask_is_a_select(cuda_device, block):
    """NaN in K and 1e30 in V at every position >= t leave rows < t bitwise
    unchanged: the diagonal mask selects (a NaN logit cannot pass) and the
    masked weights are exactly zero (a huge value cannot leak).  V stays
    finite because the diagonal tile's P V product multiplies the zero
    weights by the tile's later rows, which are real tokens."""
    w = Workload("c", "prefill", 1, 2, 2, 4 * block, 128, block, 2, seed=41)
    say(f"causal select b{block}")
    q, k, v = make_prefill(w, device=cuda_device)
    shape = shape_of(w)
    g = run_steps(shape, q, k, v)
    for t in (1, block // 2 + 3, 2 * block + 17, 4 * block - 1):
        kp, vp = k.clone(), v.clone()
        kp[:, :, t:] = float("nan")
        vp[:, :, t:] = 1e30
        o = torch.empty_like(q)
        dsa.dsa_sparse_attn_fwd(shape, q, kp, vp, g["idx"], g["cnt"], o, None)
        torch.cuda.synchronize()
        assert torch.equal(o[:, :, :t], g["o"][:, :, :t]), t


def test_zero_queries_take_lowest_blocks(cuda_device):
    """Q = 0 ties every score at 0: the lowest-index candidates are kept (the
    tie rule), and O is the plain mean of the visible values."""
    w = Workload("z", "prefill", 1, 2, 2, 640, 128, 64, 4, seed=42)
    say("zero queries")
    _, k, v = make_prefill(w, device=cuda_device)
    q = torch.zeros((1, 2, 640, 128), dtype=torch.bfloat16, device=cuda_device)
    o, lse, idx, cnt = dsa.prefill(q, k, v, 64, 4)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    for i in range(10):
        want = sorted({0, i} | set(range(1, 1 + max(0, min(4, i + 1) - len({0, i})))))
        assert [int(j) for j in idx[0, 0, i] if j >= 0] == want
    ref, _ = O.attend(np64(q), np64(k), np64(v), idx, cnt.cpu().numpy(), 64)
    check_out(np64(o), ref, what="zero-q")


@pytest.mark.parametrize("nb,topk,num,den,flags", [(100, 7, 0, 1, 3), (700, 20, 0, 1, 3), (2000, 33, 0, 1, 3),
                                                  (300, 0, 3, 10, 1), (1500, 0, 1, 7, 2), (64, 5, 0, 1, 0)])
def test_select_topk_exact_with_ties(cuda_device, nb, topk, num, den, flags):
    """dsa_select_topk on integer-valued scores (many exact ties) equals the
    oracle's selection exactly: the tie rule (lower block first) and the
    budget are the same on both sides.  Covers rows up to 256, 1024 and
    4096 blocks (4, 16 and 64 keys per lane)."""
    say(f"select exact nb{nb} k{topk} {num}/{den} flags{flags}")
    rng = np.random.default_rng(nb + topk)
    raw = rng.integers(-6, 6, size=(1, 2, nb, nb)).astype(np.float32)
    causal = np.tril(np.ones((nb, nb), dtype=bool))
    sc = np.where(causal, raw, -np.inf).astype(np.float32)
    shape = dsa.make_shape(1, 2, 2, nb * 64, 128, 64, topk, num, den, flags)
    km = dsa.dsa_kmax(shape)
    scores = torch.from_numpy(sc).to(cuda_device)
    idx = torch.empty((1, 2, nb, km), dtype=torch.int32, device=cuda_device)
    cnt = torch.empty((1, 2, nb), dtype=torch.int32, device=cuda_device)
    dsa.dsa_select_topk(shape, scores, idx, cnt)
    torch.cuda.synchronize()
    ref_idx, ref_cnt, _ = O.select_topk(sc.astype(np.float64), topk, num, den, flags)
    assert np.array_equal(cnt.cpu().numpy(), ref_cnt)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)


@pytest.mark.parametrize("nb,topk,flags", [(1024, 66, 3), (1024, 67, 3), (300, 16, 3), (3000, 40, 1), (200, 64, 0),
                                           (200, 65, 0), (1024, 2, 2)])
def test_select_topk_distinct_scores(cuda_device, nb, topk, flags):
    """dsa_select_topk on continuous random scores equals the oracle exactly,
    with the number of free picks on both sides of 64 (the one-key-per-lane
    path and the full search), short and long rows."""
    say(f"select distinct nb{nb} k{topk} flags{flags}")
    rng = np.random.default_rng(7 * nb + topk)
    raw = rng.standard_normal(size=(1, 2, nb, nb)).astype(np.float32)
    causal = np.tril(np.ones((nb, nb), dtype=bool))
    sc = np.where(causal, raw, -np.inf).astype(np.float32)
    shape = dsa.make_shape(1, 2, 2, nb * 64, 128, 64, topk, 0, 1, flags)
    km = dsa.dsa_kmax(shape)
    scores = torch.from_numpy(sc).to(cuda_device)
    idx = torch.empty((1, 2, nb, km), dtype=torch.int32, device=cuda_device)
    cnt = torch.empty((1, 2, nb), dtype=torch.int32, device=cuda_device)
    dsa.dsa_select_topk(shape, scores, idx, cnt)
    torch.cuda.synchronize()
    ref_idx, ref_cnt, _ = O.select_topk(sc.astype(np.float64), topk, 0, 1, flags)
    assert np.array_equal(cnt.cpu().numpy(), ref_cnt)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)


def test_prefill_rows_longer_than_1024_blocks(cuda_device):
    """N = 64 * 1300: selection rows longer than 1024 blocks (64 keys per
    lane), checked on every row; attention on sampled query blocks."""
    w = Workload("long", "prefill", 1, 2, 1, 64 * 1300, 64, 64, 8, seed=60)
    say("prefill nB=1300")
    q, k, v = make_prefill(w, device=cuda_device)
    o, lse, idx, cnt = dsa.prefill(q, k, v, w.block, w.topk)
    torch.cuda.synchronize()
    qn, kn, vn = np64(q), np64(k), np64(v)
    ref = O.prefill(qn, kn, vn, w.block, w.topk, attend_blocks=[])
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    check_rows(ref["rows"], gidx, gcnt)
    for (h, i) in [(0, 1299), (1, 1025), (0, 3)]:
        o_ref, lse_ref = O.attend(qn[:, h : h + 1], kn, vn, gidx, gcnt, w.block, units=[(0, 0, i)])
        lo, hi = i * 64, (i + 1) * 64
        check_out(np64(o[:, h, lo:hi]), o_ref[:, 0, lo:hi], np64(lse[:, h, lo:hi]), lse_ref[:, 0, lo:hi], f"h{h} i{i}")


# ------------------------------------------------------------------ full sizes
def sample_query_blocks(w, n_random=56, n_heavy=8, seed=0):
    """(head, query block) units for the full-size output checks: the n_heavy
    heaviest query blocks (the last ones, which keep the most keys) spread
    over different heads, block 0 of one head, and n_random more drawn
    uniformly (seeded)."""
    rng = np.random.default_rng(seed)
    heads = rng.permutation(w.n_q_heads)
    units = {(int(heads[t % w.n_q_heads]), w.n_blocks - 1 - t // max(1, w.n_q_heads)) for t in range(n_heavy)}
    units.add((int(heads[-1]), 0))
    while len(units) < n_heavy + 1 + n_random:
        units.add((int(rng.integers(w.n_q_heads)), int(rng.integers(w.n_blocks))))
    return sorted(units)


def full_prefill_check(cuda_device, wname):
    w = WORKLOADS[wname]
    say(f"full {wname}: generating")
    q, k, v = make_prefill(w, device=cuda_device)
    say(f"full {wname}: prefill")
    o, lse, idx, cnt = dsa.prefill(q, k, v, w.block, w.topk, w.topk_num, w.topk_den)
    torch.cuda.synchronize()
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    # the workspace-free score call gives the bits of the means path
    shape = shape_of(w)
    nB = w.n_blocks
    sc_a = torch.empty((w.batch, w.n_kv_heads, nB, nB), dtype=torch.float32, device=cuda_device)
    sc_b = torch.empty_like(sc_a)
    qbar = torch.empty((w.batch, w.n_q_heads, nB, w.head_dim), dtype=torch.float32, device=cuda_device)
    kbar = torch.empty((w.batch, w.n_kv_heads, nB, w.head_dim), dtype=torch.float32, device=cuda_device)
    dsa.dsa_block_means(shape, w.n_q_heads, q, qbar)
    dsa.dsa_block_means(shape, w.n_kv_heads, k, kbar)
    dsa.dsa_block_scores_from_means(shape, qbar, kbar, sc_a)
    dsa.dsa_block_scores(shape, q, k, sc_b)
    torch.cuda.synchronize()
    assert torch.equal(sc_a, sc_b)
    del sc_a, sc_b, qbar, kbar
    say(f"full {wname}: oracle selection")
    G = w.group
    s = 1.0 / math.sqrt(w.head_dim)
    flagged = total = 0
    for g in range(w.n_kv_heads):
        qn = np64(q[:, g * G : (g + 1) * G])
        kn = np64(k[:, g : g + 1])
        sc = O.block_scores(O.block_means(qn, w.block), O.block_means(kn, w.block), s)
        _, _, rows = O.select_topk(sc, w.topk, w.topk_num, w.topk_den)
        f, t = check_rows(rows, gidx[:, g : g + 1], gcnt[:, g : g + 1])
        flagged += f
        total += t
    units = sample_query_blocks(w)
    say(f"full {wname}: {flagged}/{total} rows flagged; attention on {len(units)} sampled query blocks")
    worst = (0.0, 0.0)
    by_group = {}
    for (h, i) in units:
        by_group.setdefault(h // G, []).append((h, i))
    for g, us in sorted(by_group.items()):
        kn, vn = np64(k[:, g : g + 1]), np64(v[:, g : g + 1])
        for (h, i) in us:
            qn = np64(q[:, h : h + 1])
            o_ref, lse_ref = O.attend(qn, kn, vn, gidx[:, g : g + 1], gcnt[:, g : g + 1], w.block, units=[(0, 0, i)])
            lo, hi = i * w.block, min(w.seq_len, (i + 1) * w.block)
            e = check_out(np64(o[:, h, lo:hi]), o_ref[:, 0, lo:hi], np64(lse[:, h, lo:hi]), lse_ref[:, 0, lo:hi],
                          f"{wname} h{h} i{i}")
            worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    say(f"full {wname}: worst over {len(units)} query blocks: O max-abs {worst[0]:.3g}, mean-abs {worst[1]:.3g}")
    assert torch.isfinite(o.float()).all()


def test_full_prefill_n8192(cuda_device):
    full_prefill_check(cuda_device, "prefill_n8192_h32")


def test_full_prefill_gqa_n32768(cuda_device):
    full_prefill_check(cuda_device, "prefill_gqa_n32768")


def test_full_prefill_n131072(cuda_device):
    full_prefill_check(cuda_device, "prefill_n131072_b128")


# ------------------------------------------------------------------ decode
def decode_check(cuda_device, w, flags=3, sample=None, o_units=None):
    say(f"decode S{w.batch} Hq{w.n_q_heads} Hkv{w.n_kv_heads} L{w.seq_len} d{w.head_dim} b{w.block} k{w.topk}")
    q, kc, vc = make_decode(w, device=cuda_device)
    kbar = dsa.kv_block_means(kc, w.block)
    o, lse, idx = dsa.decode(q, kc, vc, kbar, w.block, w.topk, w.topk_num, w.topk_den, flags)
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()
    units = sample if sample is not None else [(s, g) for s in range(w.batch) for g in range(w.n_kv_heads)]
    o_units = units if o_units is None else o_units
    G = w.group
    for (s, g) in units:
        qn = np64(q[s : s + 1, g * G : (g + 1) * G])
        kn = np64(kc[s : s + 1, g : g + 1])
        # the oracle's selection only (units=[]: its attention is not needed);
        # V is read where outputs are checked
        vn = np64(vc[s : s + 1, g : g + 1]) if (s, g) in o_units else None
        ref = O.decode(qn, kn, kn if vn is None else vn, w.block, w.topk, w.topk_num, w.topk_den, flags, units=[])
        np.testing.assert_allclose(np64(kbar[s, g]), ref["kbar"][0, 0], rtol=1e-5, atol=1e-6)
        check_rows(ref["rows"], gidx[s : s + 1, g : g + 1, None, :],
                   np.full((1, 1, 1), gidx.shape[-1], dtype=np.int32))
        if (s, g) in o_units:
            # evaluate the oracle on the GPU's accepted set
            sel = gidx[s, g]
            keys = np.concatenate([np.arange(j * w.block, min(w.seq_len, (j + 1) * w.block)) for j in sel])
            for hh in range(G):
                logits = (kn[0, 0, keys] @ qn[0, hh]) / math.sqrt(w.head_dim)
                wts = np.exp(logits - logits.max())
                o_ref = (wts / wts.sum()) @ vn[0, 0, keys]
                lse_ref = logits.max() + math.log(wts.sum())
                check_out(np64(o[s, g * G + hh])[None], o_ref[None], np.array([float(lse[s, g * G + hh])]),
                          np.array([lse_ref]), f"decode s{s} g{g} h{hh}")
    return o, lse, idx


DECODE_SMALL = [
    ("planted_ragged", Workload("d1", "decode", 3, 8, 2, 1000, 128, 64, 4, structure="planted", amplitude=2.0,
                                seed=50), 3),
    ("mha_d64_b128", Workload("d2", "decode", 2, 2, 2, 1300, 64, 128, 3, seed=51), 3),
    ("gqa8", Workload("d3", "decode", 2, 8, 1, 4096, 128, 64, 6, seed=52), 3),
    ("dense_all_blocks", Workload("d4", "decode", 2, 4, 2, 640, 128, 64, 10, seed=53), 3),
    ("single_key", Workload("d5", "decode", 2, 4, 2, 1, 128, 64, 4, seed=54), 3),
    ("no_forcing_k2", Workload("d6", "decode", 2, 4, 2, 2048, 128, 64, 2, seed=55), 0),
    ("fraction", Workload("d7", "decode", 1, 4, 1, 4096, 128, 64, 0, 1, 8, seed=56), 3),
    ("rows_over_1024_blocks", Workload("d8", "decode", 2, 4, 2, 64 * 1100 + 5, 128, 64, 12, seed=58), 3),
]


@pytest.mark.parametrize("name,w,flags", DECODE_SMALL, ids=[c[0] for c in DECODE_SMALL])
def test_decode_small(cuda_device, name, w, flags):
    decode_check(cuda_device, w, flags)


# >= 256 (sequence, KV head) units: one workgroup per unit does the whole step
DECODE_FUSED = [
    ("ragged_gqa4", Workload("f1", "decode", 256, 4, 1, 1000, 128, 64, 4, structure="planted", amplitude=2.0,
                             seed=70), 3),
    ("d64_b128_ragged_tail", Workload("f2", "decode", 64, 8, 4, 1300, 64, 128, 3, seed=71), 3),
    ("mha_single_key", Workload("f3", "decode", 128, 2, 2, 1, 128, 64, 4, seed=72), 3),
    ("gqa8_no_forcing", Workload("f4", "decode", 32, 64, 8, 2048, 128, 64, 5, seed=73), 0),
    ("fraction_sink_only", Workload("f5", "decode", 64, 16, 4, 3000, 128, 64, 0, 1, 6, seed=74), 1),
    ("over_1024_blocks", Workload("f6", "decode", 64, 16, 4, 64 * 1100 + 5, 128, 64, 12, seed=75), 3),
]


@pytest.mark.parametrize("name,w,flags", DECODE_FUSED, ids=[c[0] for c in DECODE_FUSED])
def test_decode_fused_path(cuda_device, name, w, flags):
    units = w.batch * w.n_kv_heads
    assert units >= 256
    rng = np.random.default_rng(units)
    sample = sorted({(0, 0), (w.batch - 1, w.n_kv_heads - 1)} |
                    {(int(rng.integers(w.batch)), int(rng.integers(w.n_kv_heads))) for _ in range(6)})
    decode_check(cuda_device, w, flags, sample=sample, o_units=sample[:4])


def test_decode_full(cuda_device):
    """The 32-sequence, 65 536-token decode: the selection of every one of the
    256 (sequence, KV head) units, the outputs of 32 of them (seeded) on the
    GPU's accepted sets."""
    w = WORKLOADS["decode_s32_l65536"]
    rng = np.random.default_rng(0)
    units = [(s, g) for s in range(w.batch) for g in range(w.n_kv_heads)]
    o_units = {units[int(t)] for t in rng.permutation(len(units))[:32]}
    decode_check(cuda_device, w, 3, sample=units, o_units=o_units)


def tied_decode_inputs(dev, S, Hkv, G, nblk, d, seed, tail=5):
    """Caches whose block b of unit (s, g) has every key equal to v e0 with v an
    integer in [-6, 6) (many exact ties), q = e0 for every head: block means
    and scores are exact, score = v / sqrt(d).  Returns q, kc, vc, v."""
    rng = np.random.default_rng(seed)
    L = nblk * 64 - tail
    v = rng.integers(-6, 6, size=(S, Hkv, nblk)).astype(np.float32)
    kc = torch.zeros((S, Hkv, nblk * 64, d), dtype=torch.bfloat16, device=dev)
    kc[..., 0] = torch.from_numpy(v).to(dev).repeat_interleave(64, dim=2).to(torch.bfloat16)
    kc = kc[:, :, :L].contiguous()
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    vc = torch.randn((S, Hkv, L, d), generator=g, device=dev).to(torch.bfloat16)
    q = torch.zeros((S, Hkv * G, d), dtype=torch.bfloat16, device=dev)
    q[..., 0] = 1.0
    return q, kc, vc, v


@pytest.mark.parametrize("S,Hkv,G,nblk,topk,flags", [(2, 2, 2, 300, 17, 3), (64, 4, 2, 300, 17, 3),
                                                     (32, 8, 1, 1100, 40, 1), (32, 8, 2, 200, 150, 0),
                                                     (3, 2, 4, 50, 49, 3)])
def test_decode_exact_ties(cuda_device, S, Hkv, G, nblk, topk, flags):
    """Integer-valued block scores (many exact ties): the decode selection
    equals the oracle's exactly (ties go to the lower block), on the split
    path (few units) and the fused path (>= 256 units), rows of up to 1 100
    blocks, with and without forcing."""
    say(f"decode exact ties S{S} Hkv{Hkv} G{G} nB{nblk} k{topk} flags{flags}")
    d = 128
    # a ragged last block only where it is forced (its mean is a division by
    # the row count, exact in the oracle but not necessarily on the GPU)
    tail = 5 if flags & O.FORCE_DIAG else 0
    q, kc, vc, v = tied_decode_inputs(cuda_device, S, Hkv, G, nblk, d, seed=nblk + topk, tail=tail)
    kbar = dsa.kv_block_means(kc, 64)
    o, lse, idx = dsa.decode(q, kc, vc, kbar, 64, topk, flags=flags)
    torch.cuda.synchronize()
    scores = (v.astype(np.float64) / math.sqrt(d))[:, :, None, :]
    ref_idx, ref_cnt, _ = O.select_topk(scores, topk, 0, 1, flags, causal=False)
    gidx = idx.cpu().numpy()
    km = ref_idx.shape[-1]
    assert np.array_equal(gidx[..., :km], ref_idx[:, :, 0]) and (gidx[..., km:] == -1).all()
    assert torch.isfinite(o.float()).all()


def test_decode_split_count_does_not_change_results(cuda_device):
    """One sequence alone (8 units: the split path, many splits per unit) and
    inside a batch of 32 (256 units: the fused one-workgroup-per-unit path)
    selects the same blocks and agrees to fp32 rounding."""
    w = Workload("ds", "decode", 32, 32, 8, 4096, 128, 64, 16, seed=57)
    say("decode split invariance")
    q, kc, vc = make_decode(w, device=cuda_device)
    kbar = dsa.kv_block_means(kc, 64)
    o_all, _, idx_all = dsa.decode(q, kc, vc, kbar, 64, 16)
    o_one, _, idx_one = dsa.decode(q[5:6].contiguous(), kc[5:6].contiguous(), vc[5:6].contiguous(),
                                   kbar[5:6].contiguous(), 64, 16)
    torch.cuda.synchronize()
    assert torch.equal(idx_all[5:6], idx_one)
    assert (o_all[5:6].float() - o_one.float()).abs().max().item() <= 1e-2
