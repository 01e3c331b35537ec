"""Index arrays that did not come from a selection call: the attention
kernels clamp each row's count into [0, kmax] and every block id into
[0, nB) where they read them, so out-of-range entries act exactly like their
clamped values (the results are then not the method's, but no access leaves
the tensors).  Checked through the C ABI by comparing a call on a corrupted
idx/cnt with the same call on its clamped copy, bit for bit, for the forward
and for the backward (whose inverted lists are built from the same arrays)."""

import sys

import pytest
import torch

import dynamic_block_sparse_dsa_amd as dsa
from dynamic_block_sparse_dsa_amd.inputs import Workload, make_prefill

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-clamp] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("block", [64, 128])
def test_out_of_range_indices_act_as_clamped(cuda_device, block):
    w = Workload("clamp", "prefill", 1, 4, 2, block * 12 + 5, 128, block, 4, structure="planted", amplitude=3.0,
                 seed=61)
    B, Hq, Hkv, N, d, nB = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.n_blocks
    q, k, v = make_prefill(w, device=cuda_device)
    o, lse, idx, cnt = dsa.prefill(q, k, v, w.block, w.topk)
    shape = dsa.make_shape(B, Hq, Hkv, N, d, w.block, w.topk)
    km = idx.shape[-1]
    torch.cuda.synchronize()
    # corrupt: negative and too-large block ids, counts above kmax and below 0
    bad_idx, bad_cnt = idx.clone(), cnt.clone()
    bad_idx[0, 0, 3, 0] = -9
    bad_idx[0, 1, 5, 1] = nB + 7
    bad_idx[0, 0, nB - 1, :] = 1 << 30
    bad_cnt[0, 0, 2] = km + 5
    bad_cnt[0, 1, 4] = -3
    bad_cnt[0, 1, nB - 1] = 1 << 30
    ok_idx = bad_idx.clamp(0, nB - 1)
    ok_cnt = bad_cnt.clamp(0, km)
    say(f"block {block}: N{N} nB{nB} kmax{km}: forward and backward on corrupted vs clamped indices")

    def fwd(ix, ct):
        oo = torch.full_like(q, float("nan"))
        ll = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=cuda_device)
        dsa.dsa_sparse_attn_fwd(shape, q, k, v, ix, ct, oo, ll)
        return oo, ll

    fb, fc = fwd(bad_idx, bad_cnt), fwd(ok_idx, ok_cnt)
    torch.cuda.synchronize()
    for a_, b_ in zip(fb, fc):  # a row whose count clamps to 0 divides 0 by 0 in both
        torch.testing.assert_close(a_, b_, rtol=0, atol=0, equal_nan=True)

    g = torch.Generator(device=cuda_device)
    g.manual_seed(62)
    dout = torch.randn(q.shape, generator=g, device=cuda_device).to(torch.bfloat16)
    ws = torch.empty(max(1, dsa.dsa_attn_bwd_workspace_bytes(shape)), dtype=torch.uint8, device=cuda_device)

    def bwd(ix, ct):
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        dsa.dsa_sparse_attn_bwd(shape, q, k, v, o, lse, dout, ix, ct, *grads, ws)
        torch.cuda.synchronize()
        return grads

    gb, gc = bwd(bad_idx, bad_cnt), bwd(ok_idx, ok_cnt)
    for a_, b_ in zip(gb, gc):
        torch.testing.assert_close(a_, b_, rtol=0, atol=0, equal_nan=True)
    say(f"block {block}: corrupted indices give the clamped indices' results")
