"""GPU parity of the attention backward (dsa_sparse_attn_bwd through the C
ABI) against the oracle's backward (fp64) evaluated on the GPU's own
selection, same seeded inputs and output gradient.

The reference is the exact chain rule through the attention definition
(``O.attend_backward`` with ``o=None``: the term sum_c w_c dO.v_c from the
exact weights).  Bar: per element |got - ref| <= REL_MAX_EXACT * (|ref| + rms)
and mean |got - ref| <= REL_MEAN * rms, rms being the reference tensor's root
mean square.  Elementwise relative because gradient magnitudes are
heavy-tailed (a row that sees two keys, or a key kept by many rows, is tens
of times the rms); the rms term covers elements near zero.

REL_MAX_EXACT = 1e-1 is the sum of two parts:
  * 5e-2 for the kernel's own rounding: P and dS are rounded to bf16 as MFMA
    operands and the gradients are stored in bf16 (relative 2^-9 each).  An
    element's error is a few 2^-9 of the sum of its terms' magnitudes, and the
    terms cancel (each row of dS sums to zero over its keys), so an element
    can be ~10x smaller than that sum;
  * 5e-2 for D = rowsum(dO * O): the call is handed the forward's bf16 O (as
    FlashAttention-2 is), so D carries O's bf16 rounding, |dD| <= 2^-9
    sum_e |dO_e O_e|.  That error enters every dS of the row as P_c dD and
    does not cancel in dQ = dS K / sqrt(d).  Evaluating the oracle once with
    the exact O and once with O rounded to bf16 (on the CPU, the shapes
    below) moves dQ by at most 0.041 and dK by at most 0.024 in this metric
    (means <= 3e-4 rms); dV does not depend on D.
The mean bar (4e-3; observed 1.2e-3 .. 1.8e-3) is the check against
systematic error.  The oracle evaluated with the GPU's bf16 O (``o=``) is
also printed as a diagnostic of the kernel's own rounding (same 5e-2 bar).
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
import dynamic_block_sparse_dsa_amd as dsa
from dynamic_block_sparse_dsa_amd.inputs import WORKLOADS, Workload, make_prefill

pytestmark = pytest.mark.gpu

REL_MAX_EXACT, REL_MAX_GIVEN_O, REL_MEAN = 1e-1, 5e-2, 4e-3


def say(msg):
    print(f"[gpu-backward] {msg}", flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_grad(name, got, ref, what, bar=REL_MAX_EXACT, label="exact"):
    assert np.isfinite(got).all(), (what, name)
    rms = math.sqrt(float((ref ** 2).mean())) or 1.0
    diff = np.abs(got - ref)
    rel = diff / (np.abs(ref) + rms)
    say(f"{what} {name} vs {label}: rms {rms:.3g}, max |d|/(|ref|+rms) {rel.max():.3g}, "
        f"mean |d|/rms {diff.mean() / rms:.3g}")
    assert rel.max() <= bar, (what, name, label, rel.max())
    assert diff.mean() / rms <= REL_MEAN, (what, name, label, diff.mean() / rms)


def run(cuda_device, w, flags=3, seed=0):
    q, k, v = make_prefill(w, device=cuda_device)
    o, lse, idx, cnt = dsa.prefill(q, k, v, w.block, w.topk, w.topk_num, w.topk_den, flags)
    g = torch.Generator(device=cuda_device)
    g.manual_seed(1000 + seed)
    dout = torch.randn(q.shape, generator=g, device=cuda_device, dtype=torch.float32).to(torch.bfloat16)
    dq, dk, dv = dsa.attn_backward(q, k, v, o, lse, dout, idx, cnt, w.block, w.topk, w.topk_num, w.topk_den, flags)
    torch.cuda.synchronize()
    return q, k, v, o, lse, idx, cnt, dout, dq, dk, dv


SMALL = [
    ("tiny_n1024_d64_k4", WORKLOADS["prefill_tiny_n1024"], 3),
    ("ragged_n1000", Workload("r", "prefill", 1, 2, 2, 1000, 64, 64, 4, seed=21), 3),
    ("gqa4_frac_n2048", Workload("g", "prefill", 1, 8, 2, 2048, 128, 64, 0, 15, 100, structure="planted",
                                 amplitude=2.0, seed=22), 3),
    ("b128_n1500", Workload("b", "prefill", 1, 2, 2, 1500, 128, 128, 4, seed=23), 3),
    ("d64_b128_gqa2_n777", Workload("c", "prefill", 2, 2, 1, 777, 64, 128, 3, seed=24), 3),
    ("gqa3_n640", Workload("f", "prefill", 1, 6, 2, 640, 128, 64, 3, seed=26), 3),
    ("k1_no_forcing", Workload("h", "prefill", 1, 2, 2, 640, 128, 64, 1, seed=27), 0),
    ("dense_k_all", Workload("k", "prefill", 2, 4, 2, 512, 128, 64, 8, seed=30), 3),
    ("short_n37", Workload("l", "prefill", 1, 2, 2, 37, 64, 64, 4, seed=31), 3),
    ("single_row_n1", Workload("m", "prefill", 1, 1, 1, 1, 128, 64, 4, seed=32), 3),
]


@pytest.mark.parametrize("name,w,flags", SMALL, ids=[c[0] for c in SMALL])
def test_backward_small(cuda_device, name, w, flags):
    say(f"backward {name}: B{w.batch} Hq{w.n_q_heads} Hkv{w.n_kv_heads} N{w.seq_len} d{w.head_dim} b{w.block}")
    q, k, v, o, lse, idx, cnt, dout, dq, dk, dv = run(cuda_device, w, flags)
    args = (np64(q), np64(k), np64(v), np64(dout), idx.cpu().numpy(), cnt.cpu().numpy(), w.block)
    rq, rk, rv = O.attend_backward(*args)
    check_grad("dq", np64(dq), rq, name)
    check_grad("dk", np64(dk), rk, name)
    check_grad("dv", np64(dv), rv, name)
    # diagnostic: the oracle handed the GPU's own bf16 O isolates the kernel's rounding
    gq, gk, gv = O.attend_backward(*args, o=np64(o))
    for nm, got, ref in (("dq", dq, gq), ("dk", dk, gk), ("dv", dv, gv)):
        check_grad(nm, np64(got), ref, name, REL_MAX_GIVEN_O, "given-O")
    # keys no row kept: exactly zero on both sides
    unkept = (rk == 0).all(axis=-1) & (rv == 0).all(axis=-1)
    assert (np64(dk)[unkept] == 0).all() and (np64(dv)[unkept] == 0).all()


def test_backward_diagonal_only(cuda_device):
    """Every block kept only by its own query block (causal within it)."""
    # diagonal forcing only and k = 1: block j is kept by query block j alone,
    # and within it only by the rows at or after each key
    w1 = Workload("z1", "prefill", 1, 2, 2, 2048, 128, 64, 1, seed=41)
    q, k, v, o, lse, idx, cnt, dout, dq, dk, dv = run(cuda_device, w1, flags=2)
    rq, rk, rv = O.attend_backward(np64(q), np64(k), np64(v), np64(dout), idx.cpu().numpy(), cnt.cpu().numpy(), 64)
    check_grad("dq", np64(dq), rq, "diag-only")
    check_grad("dk", np64(dk), rk, "diag-only")
    check_grad("dv", np64(dv), rv, "diag-only")


def test_backward_full_prefill_n8192_sampled(cuda_device):
    """The full 32-head, 8192-token workload: dQ on sampled query blocks; dK,
    dV on sampled KV blocks (all rows that kept them)."""
    w = WORKLOADS["prefill_n8192_h32"]
    say("backward full prefill_n8192_h32")
    q, k, v, o, lse, idx, cnt, dout, dq, dk, dv = run(cuda_device, w)
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    G = w.group
    for (h, i) in [(0, 0), (0, 127), (7, 64), (31, 100)]:
        gh = h // G
        qn, kn, vn, don = np64(q[:, h:h + 1]), np64(k[:, gh:gh + 1]), np64(v[:, gh:gh + 1]), np64(dout[:, h:h + 1])
        rq, _, _ = O.attend_backward(qn, kn, vn, don, gi[:, gh:gh + 1], gc[:, gh:gh + 1], w.block, units=[(0, 0, i)])
        lo, hi = i * w.block, (i + 1) * w.block
        check_grad("dq", np64(dq[:, h, lo:hi]), rq[:, 0, lo:hi], f"n8192 h{h} i{i}")
    for (g, j) in [(0, 0), (3, 5), (31, 127), (17, 60)]:
        rows = [i for i in range(w.n_blocks) if j in gi[0, g, i, : gc[0, g, i]]]
        qn, kn, vn, don = np64(q[:, g:g + 1]), np64(k[:, g:g + 1]), np64(v[:, g:g + 1]), np64(dout[:, g:g + 1])
        _, rk, rv = O.attend_backward(qn, kn, vn, don, gi[:, g:g + 1], gc[:, g:g + 1], w.block,
                                      units=[(0, 0, i) for i in rows])
        lo, hi = j * w.block, (j + 1) * w.block
        check_grad("dk", np64(dk[:, g, lo:hi]), rk[:, 0, lo:hi], f"n8192 g{g} j{j} ({len(rows)} rows)")
        check_grad("dv", np64(dv[:, g, lo:hi]), rv[:, 0, lo:hi], f"n8192 g{g} j{j} ({len(rows)} rows)")
