"""dsa_decode_noalloc (the decode entry point that allocates nothing: its
split partials live in a library-owned device array) against dsa_decode with
a caller workspace, through the C ABI: two calls in a row, the second on a
smaller input, each bit-identical to dsa_decode (same kernels, same order)."""

import sys

import pytest
import torch

import dynamic_block_sparse_dsa_amd as dsa
from dynamic_block_sparse_dsa_amd.inputs import Workload, make_decode

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-noalloc] {msg}", flush=True)
    sys.stdout.flush()


def decode_both(dev, w, flags=3):
    q, kc, vc = make_decode(w, device=dev)
    kbar = dsa.kv_block_means(kc, w.block)
    shape = dsa.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block, w.topk, w.topk_num,
                           w.topk_den, flags)
    km = dsa.dsa_kmax(shape)
    S, Hq, Hkv = w.batch, w.n_q_heads, w.n_kv_heads
    outs = []
    for noalloc in (False, True):
        o = torch.full((S, Hq, w.head_dim), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((S, Hq), float("nan"), dtype=torch.float32, device=dev)
        idx = torch.full((S, Hkv, km), -7, dtype=torch.int32, device=dev)
        if noalloc:
            dsa.dsa_decode_noalloc(shape, q, kc, vc, kbar, o, lse, idx)
        else:
            ws = torch.empty(max(1, dsa.dsa_decode_workspace_bytes(shape)), dtype=torch.uint8, device=dev)
            dsa.dsa_decode(shape, q, kc, vc, kbar, o, lse, idx, ws)
        torch.cuda.synchronize()
        outs.append((o, lse, idx))
    return outs, dsa.dsa_decode_workspace_bytes(shape)


def test_noalloc_decode_matches_decode_twice(cuda_device):
    cases = [
        Workload("na1", "decode", 4, 32, 8, 16384, 128, 64, 16, structure="planted", amplitude=2.0, seed=81),
        Workload("na2", "decode", 1, 8, 2, 3000, 64, 128, 5, seed=82),
    ]
    for w in cases:
        (ref, got), need = decode_both(cuda_device, w)
        say(f"{w.name}: S{w.batch} Hq{w.n_q_heads} Hkv{w.n_kv_heads} L{w.seq_len} d{w.head_dim} b{w.block} "
            f"k{w.topk}: split partials {need} bytes")
        assert need > 0  # the split path, which uses the scratch
        assert torch.equal(got[2], ref[2])
        assert torch.equal(got[0], ref[0])
        assert torch.equal(got[1], ref[1])


def test_noalloc_decode_rejects_bad_shapes(cuda_device):
    s = dsa.make_shape(2, 12, 2, 4096, 128, 64, 8)  # group of 6: not built for decode
    with pytest.raises(dsa.DsaError):
        q = torch.zeros((2, 12, 128), dtype=torch.bfloat16, device=cuda_device)
        dsa.dsa_decode_noalloc(s, q, None, None, None, None, None, None)
