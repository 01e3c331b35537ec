"""The selection validator (dsa_check_block_selection, dsa_check_token_selection)
through the C ABI.

1. Every index array a selection call writes -- prefill under each selection
   rule (top-k, fraction, no forcing, anchors and windows, threshold,
   entropy), dense decode on both of its paths, paged decode with empty,
   partial and full sequences, token selection -- passes: every slot of the
   report but ROWS is 0 and ROWS is the number of rows.
2. Corrupted copies (swapped, repeated, out-of-range and negative ids, a
   dropped forced id, bad padding, wrong counts) give exactly the counts of
   the rules written out below in plain Python, and each corruption raises
   the slot it breaks.  The rules in plain Python are in selection_rules.py
   (pinned on the CPU against the oracle's selections).
"""

import sys

import pytest
import torch
from selection_rules import SLOTS, clean, corrupt, count_rule, forcing, ref_report

import dynamic_block_sparse_dsa_amd as dsa
from dynamic_block_sparse_dsa_amd.inputs import INDEX_WORKLOADS, WORKLOADS, Workload, make_decode, make_index, \
    make_prefill

pytestmark = pytest.mark.gpu
assert tuple(SLOTS) == dsa.CHECK_SLOTS


def say(msg):
    print(f"[gpu-check] {msg}", flush=True)
    sys.stdout.flush()


def run_checks(name, check, idx, cnt, visible, rng, anchors, window, dev, seed):
    rows = idx.numel() // idx.shape[-1]
    got = check(idx, cnt)
    assert got == clean(rows), f"{name}: selection output flagged: {got}"
    ref = ref_report(idx.cpu().numpy(), None if cnt is None else cnt.cpu().numpy(), visible, rng, anchors, window)
    assert ref == clean(rows), f"{name}: the plain rules flag the selection output: {ref}"
    bix, bct, hit = corrupt(idx, cnt, visible, seed)
    got = check(bix.to(dev), None if bct is None else bct.to(dev))
    ref = ref_report(bix.numpy(), None if bct is None else bct.numpy(), visible, rng, anchors, window)
    assert got == ref, f"{name}: corrupted arrays: validator {got} != rules {ref}"
    assert got["order"] >= 2 and got["range"] >= 2, got
    if anchors:
        assert got["forced"] >= 1, got
    if "padding" in hit:
        assert got["padding"] >= 1, got
    if "count" in hit:
        assert got["count"] >= hit["count"], got
    say(f"{name}: {rows} rows clean; corrupted copy -> {got}")


# ---------------------------------------------------------------- prefill
PREFILL_CASES = [
    # (id, block, topk, num, den, flags, select)
    ("topk6", 64, 6, 0, 1, 3, {}),
    ("frac15", 64, 0, 15, 100, 3, {}),
    ("noforce_k5", 64, 5, 0, 1, 0, {}),
    ("anchor2_window3", 64, 8, 0, 1, 3, {"n_anchor": 2, "window": 3}),
    ("threshold", 64, 0, 0, 1, 3, {"select_mode": dsa.SELECT_THRESHOLD, "threshold": 0.05}),
    ("entropy", 64, 0, 0, 1, 3, {"select_mode": dsa.SELECT_ENTROPY, "k_min": 2, "k_max": 9}),
    ("sink_only_b128", 128, 4, 0, 1, 1, {}),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_selection(cuda_device, case):
    name, block, topk, num, den, flags, sel = case
    w = Workload("chk", "prefill", 2, 8, 2, block * 40 + 17, 128, block, topk, num, den, structure="planted",
                 amplitude=3.0, seed=71)
    q, k, v = make_prefill(w, device=cuda_device)
    _, _, idx, cnt = dsa.prefill(q, k, v, block, topk, num, den, flags, **sel)
    shape = dsa.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, block, topk, num, den, flags,
                           **sel)
    nB = shape.n_blocks
    anchors, window = forcing(flags, sel.get("n_anchor", 0), sel.get("window", 0))
    rng = count_rule(sel.get("select_mode", dsa.SELECT_TOPK), topk, num, den, sel.get("threshold", 0.0),
                     sel.get("k_min", 0), sel.get("k_max", 0))
    say(f"prefill {name}: B{w.batch} Hkv{w.n_kv_heads} N{w.seq_len} b{block} nB{nB} kmax{idx.shape[-1]}")
    run_checks(f"prefill {name}", lambda ix, ct: dsa.check_selection(shape, ix, ct), idx, cnt,
               lambda r: r % nB + 1, rng, anchors, window, cuda_device, 72)


def test_prefill_selection_full_size(cuda_device):
    """The 8192-token, 32-head workload's selection through the fused step."""
    w = WORKLOADS["prefill_n8192_h32"]
    q, k, v = make_prefill(w, device=cuda_device)
    _, _, idx, cnt = dsa.prefill(q, k, v, w.block, w.topk, w.topk_num, w.topk_den)
    shape = dsa.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block, w.topk, w.topk_num,
                           w.topk_den)
    got = dsa.check_selection(shape, idx, cnt)
    assert got == clean(w.batch * w.n_kv_heads * w.n_blocks), got
    say(f"prefill {w.name}: {got['rows']} rows clean")


# ---------------------------------------------------------------- decode
DECODE_CASES = [
    Workload("chk_split", "decode", 4, 16, 4, 64 * 90 + 13, 128, 64, 8, structure="planted", amplitude=2.0, seed=73),
    Workload("chk_fused", "decode", 64, 16, 4, 4096, 128, 64, 16, structure="planted", amplitude=2.0, seed=74),
]


@pytest.mark.parametrize("w", DECODE_CASES, ids=[w.name for w in DECODE_CASES])
@pytest.mark.parametrize("force", [(3, 0, 0), (3, 2, 3), (2, 0, 0)], ids=["sink_diag", "anchor2_window3", "diag"])
def test_decode_selection(cuda_device, w, force):
    flags, n_anchor, window = force
    q, kc, vc = make_decode(w, device=cuda_device)
    kbar = dsa.kv_block_means(kc, w.block)
    _, _, idx = dsa.decode(q, kc, vc, kbar, w.block, w.topk, flags=flags, n_anchor=n_anchor, window=window)
    shape = dsa.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block, w.topk, flags=flags,
                           n_anchor=n_anchor, window=window)
    nB = shape.n_blocks
    anchors, win = forcing(flags, n_anchor, window)
    say(f"decode {w.name} flags{flags} anchors{anchors} window{win}: S{w.batch} Hkv{w.n_kv_heads} nB{nB}")
    run_checks(f"decode {w.name}", lambda ix, ct: dsa.check_selection(shape, ix, None, layout=dsa.LAYOUT_DECODE),
               idx, None, lambda r: nB, count_rule(dsa.SELECT_TOPK, w.topk), anchors, win, cuda_device, 75)


def test_paged_selection(cuda_device):
    w = Workload("chk_paged", "decode", 7, 8, 2, 64 * 20, 128, 64, 6, structure="planted", amplitude=3.0, seed=76)
    S, Hkv, L, d, b = w.batch, w.n_kv_heads, w.seq_len, w.head_dim, w.block
    mb = L // b
    q, kc, vc = make_decode(w, device=cuda_device)
    n_pages = S * mb + 2
    perm = torch.randperm(n_pages, generator=torch.Generator(device="cpu").manual_seed(77))
    table = perm[: S * mb].view(S, mb).to(torch.int32).to(cuda_device)
    kp = torch.zeros((n_pages, Hkv, b, d), dtype=torch.bfloat16, device=cuda_device)
    vp = torch.zeros_like(kp)
    flat = table.reshape(-1).long()
    kp[flat] = kc.view(S, Hkv, mb, b, d).permute(0, 2, 1, 3, 4).reshape(S * mb, Hkv, b, d)
    vp[flat] = vc.view(S, Hkv, mb, b, d).permute(0, 2, 1, 3, 4).reshape(S * mb, Hkv, b, d)
    lengths = [0, 1, 64, 65, 700, 1279, 1280]  # empty, one token, one full block, ..., full
    lens = torch.tensor(lengths, dtype=torch.int32, device=cuda_device)
    shape = dsa.make_shape(S, w.n_q_heads, Hkv, L, d, b, w.topk)
    kbar = torch.zeros((n_pages, Hkv, d), dtype=torch.float32, device=cuda_device)
    dsa.dsa_paged_kv_block_means(shape, kp, table, lens, kbar)
    _, _, idx, cnt = dsa.paged_decode(q, kp, vp, kbar, table, lens, b, w.topk)
    torch.cuda.synchronize()
    vis = lambda r: -(-lengths[r // Hkv] // b)
    rng = count_rule(dsa.SELECT_TOPK, w.topk)
    say(f"paged: S{S} Hkv{Hkv} capacity {L} lengths {lengths}")
    for use_cnt in (True, False):
        run_checks(f"paged cnt={'given' if use_cnt else 'NULL'}",
                   lambda ix, ct: dsa.check_selection(shape, ix, ct, lens, layout=dsa.LAYOUT_PAGED), idx,
                   cnt if use_cnt else None, vis, rng, 1, 1, cuda_device, 78)


# ---------------------------------------------------------------- token selection
@pytest.mark.parametrize("flags", [3, 1, 0], ids=["sink_diag", "sink", "none"])
def test_token_selection(cuda_device, flags):
    w = INDEX_WORKLOADS["index_tiny_n512"]
    x = make_index(w, device=cuda_device)
    _, _, idx, cnt = dsa.index_prefill(*x, w.topk, flags)
    shape = dsa.make_index_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.n_index_heads,
                                 w.index_dim, w.topk, flags)
    N = w.seq_len
    anchors, window = (1 if flags & 1 else 0), (1 if flags & 2 else 0)
    say(f"token flags{flags}: B{w.batch} N{N} topk{w.topk}")
    run_checks(f"token flags{flags}", lambda ix, ct: dsa.check_selection(shape, ix, ct), idx, cnt,
               lambda r: r % N + 1, count_rule(dsa.SELECT_TOPK, w.topk), anchors, window, cuda_device, 79)


def test_empty_shapes_clear_the_report(cuda_device):
    """No rows: the report is still written (all zero) over whatever it held."""
    rep = torch.full((len(SLOTS),), 99, dtype=torch.int64, device=cuda_device)
    shape = dsa.make_shape(0, 4, 2, 1024, 128, 64, 4)
    idx = torch.empty((0, 2, 16, dsa.dsa_prefill_kmax(shape)), dtype=torch.int32, device=cuda_device)
    cnt = torch.empty((0, 2, 16), dtype=torch.int32, device=cuda_device)
    dsa.dsa_check_block_selection(shape, dsa.LAYOUT_PREFILL, idx, cnt, None, rep)
    torch.cuda.synchronize()
    assert rep.tolist() == [0] * len(SLOTS)
