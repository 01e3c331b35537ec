"""HIP graph capture of the library's steps, through the C ABI.

torch.cuda.CUDAGraph records the kernels the library launches on the capturing
stream.  The library makes no allocation, memset or synchronisation inside a
call, so a captured step replays the same kernels on whatever its buffers hold
at replay time.  Each test replays a captured step several times, with eager
work (new inputs written into the captured buffers, outputs poisoned, other
kernels, device synchronisations) between the replays, and checks every replay
bit for bit against the same call made eagerly on the same inputs into other
buffers: the same kernels in the same order give identical bits.
"""

import sys

import pytest
import torch

import dynamic_block_sparse_dsa_amd as dsa
from dynamic_block_sparse_dsa_amd.inputs import Workload, make_decode, make_prefill

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-graph] {msg}", flush=True)
    sys.stdout.flush()


def poison(*ts):
    for t in ts:
        if t.is_floating_point():
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


def capture(fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        fn()
    torch.cuda.synchronize()
    return g


def replay(g):
    g.replay()
    torch.cuda.synchronize()


def assert_same(got, ref, what):
    for n, (a, b) in enumerate(zip(got, ref)):
        assert torch.equal(a, b), f"{what}: output {n} differs"


def test_prefill_step_replays(cuda_device):
    """dsa_prefill (block means, block scores, top-k, attention: four
    launches) captured once; three replays on three different Q/K/V."""
    w = Workload("g_prefill", "prefill", 1, 8, 2, 64 * 37 + 21, 128, 64, 6, structure="planted", amplitude=3.0,
                 seed=91)
    shape = dsa.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block, w.topk)
    km = dsa.dsa_prefill_kmax(shape)
    q, k, v = make_prefill(w, device=cuda_device)
    B, Hq, Hkv, N, nB = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.n_blocks

    def outputs():
        return (torch.empty_like(q), torch.empty((B, Hq, N), dtype=torch.float32, device=cuda_device),
                torch.empty((B, Hkv, nB, km), dtype=torch.int32, device=cuda_device),
                torch.empty((B, Hkv, nB), dtype=torch.int32, device=cuda_device))

    outs = outputs()
    ws = torch.empty(max(1, dsa.dsa_prefill_workspace_bytes(shape)), dtype=torch.uint8, device=cuda_device)
    g = capture(lambda: dsa.dsa_prefill(shape, q, k, v, *outs, ws))
    say(f"prefill B{B} Hq{Hq} Hkv{Hkv} N{N} d{w.head_dim} b{w.block} k{w.topk}: captured")
    for rep in range(3):
        if rep:
            q2, k2, v2 = make_prefill(w, device=cuda_device, seed=91 + 17 * rep)
            q.copy_(q2), k.copy_(k2), v.copy_(v2)
        ref = outputs()
        ws2 = torch.empty_like(ws)
        dsa.dsa_prefill(shape, q, k, v, *ref, ws2)
        poison(*outs)
        torch.cuda.synchronize()
        replay(g)
        assert_same(outs, ref, f"prefill replay {rep}")
        assert int(ref[3].min()) >= 1  # every row kept something: the comparison covers the attention
    say("prefill: 3 replays identical to the eager calls")


DECODES = [
    # split path (fewer than 256 (sequence, KV head) units): select, split attention, combine
    Workload("g_split", "decode", 4, 16, 4, 64 * 90 + 13, 128, 64, 8, structure="planted", amplitude=2.0, seed=92),
    # fused path (256 units: one launch)
    Workload("g_fused", "decode", 64, 16, 4, 4096, 128, 64, 16, structure="planted", amplitude=2.0, seed=93),
]


@pytest.mark.parametrize("w", DECODES, ids=[w.name for w in DECODES])
@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_decode_step_replays(cuda_device, w, noalloc):
    """dsa_decode (caller workspace) or dsa_decode_noalloc (library-owned
    scratch) captured once; three replays with a new query each.  With
    DSA_DETERMINISTIC, so that the one-launch path's merge order is fixed."""
    S, Hq, Hkv, L, d, nB = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.n_blocks
    shape = dsa.make_shape(S, Hq, Hkv, L, d, w.block, w.topk,
                           flags=dsa.FORCE_SINK | dsa.FORCE_DIAG | dsa.DETERMINISTIC)
    km = dsa.dsa_kmax(shape)
    q, kc, vc = make_decode(w, device=cuda_device)
    kbar = dsa.kv_block_means(kc, w.block)

    def outputs():
        return (torch.empty_like(q), torch.empty((S, Hq), dtype=torch.float32, device=cuda_device),
                torch.empty((S, Hkv, km), dtype=torch.int32, device=cuda_device))

    ws = torch.empty(max(1, dsa.dsa_decode_workspace_bytes(shape)), dtype=torch.uint8, device=cuda_device)

    def call(outs):
        if noalloc:
            dsa.dsa_decode_noalloc(shape, q, kc, vc, kbar, *outs)
        else:
            dsa.dsa_decode(shape, q, kc, vc, kbar, *outs, ws)

    outs = outputs()
    call(outputs())  # first call on the device outside the capture (the no-alloc scratch's address is looked up)
    torch.cuda.synchronize()
    g = capture(lambda: call(outs))
    say(f"decode {w.name} {'noalloc' if noalloc else 'workspace'}: S{S} Hq{Hq} Hkv{Hkv} L{L} k{w.topk}: captured")
    gen = torch.Generator(device=cuda_device)
    gen.manual_seed(94)
    for rep in range(3):
        if rep:
            q.add_(torch.randn(q.shape, generator=gen, device=cuda_device).to(torch.bfloat16))
        ref = outputs()
        call(ref)
        poison(*outs)
        torch.cuda.synchronize()
        replay(g)
        assert_same(outs, ref, f"decode {w.name} replay {rep}")
    say(f"decode {w.name}: 3 replays identical to the eager calls")


def test_paged_serving_step_replays(cuda_device):
    """One serving step -- dsa_paged_kv_append of a token per sequence, then
    dsa_paged_decode (with DSA_DETERMINISTIC) -- captured once and replayed
    for five steps: the lengths advance on the device, so each replay appends
    at the next slot.
    The same five steps run eagerly on a copy of the initial pools."""
    w = Workload("g_paged", "decode", 6, 8, 2, 64 * 12, 128, 64, 5, structure="planted", amplitude=4.0, seed=95)
    S, Hq, Hkv, L, d, b = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block
    mb = -(-L // b)
    q, kc, vc = make_decode(w, device=cuda_device)
    n_pages = S * mb + 3
    perm = torch.randperm(n_pages, generator=torch.Generator(device="cpu").manual_seed(96))
    table = perm[: S * mb].view(S, mb).to(torch.int32).to(cuda_device)
    kp = torch.zeros((n_pages, Hkv, b, d), dtype=torch.bfloat16, device=cuda_device)
    vp = torch.zeros_like(kp)
    flat = table.reshape(-1).long()
    kp[flat] = kc.view(S, Hkv, mb, b, d).permute(0, 2, 1, 3, 4).reshape(S * mb, Hkv, b, d)
    vp[flat] = vc.view(S, Hkv, mb, b, d).permute(0, 2, 1, 3, 4).reshape(S * mb, Hkv, b, d)
    lens = torch.tensor([700, 63, 64, 1, 765, 768], dtype=torch.int32, device=cuda_device)  # the last one is full
    # DSA_DETERMINISTIC: the attention walk's merge order is fixed
    shape = dsa.make_shape(S, Hq, Hkv, mb * b, d, b, w.topk,
                           flags=dsa.FORCE_SINK | dsa.FORCE_DIAG | dsa.DETERMINISTIC)
    km = dsa.dsa_kmax(shape)
    kbar = torch.zeros((n_pages, Hkv, d), dtype=torch.float32, device=cuda_device)
    dsa.dsa_paged_kv_block_means(shape, kp, table, lens, kbar)
    kn = torch.empty((S, Hkv, d), dtype=torch.bfloat16, device=cuda_device)
    vn = torch.empty_like(kn)

    def state():
        return [kp.clone(), vp.clone(), kbar.clone(), lens.clone()]

    def outputs():
        return (torch.empty_like(q), torch.empty((S, Hq), dtype=torch.float32, device=cuda_device),
                torch.empty((S, Hkv, km), dtype=torch.int32, device=cuda_device),
                torch.empty((S, Hkv), dtype=torch.int32, device=cuda_device))

    def step(st, outs):
        k_, v_, kb_, ln_ = st
        dsa.dsa_paged_kv_append(shape, kn, vn, table, ln_, k_, v_, kb_)
        dsa.dsa_paged_decode(shape, q, k_, v_, kb_, table, ln_, *outs)

    eager, graphed = state(), state()
    outs = outputs()
    g = capture(lambda: step(graphed, outs))
    # capturing runs nothing: the graphed state is still the initial one
    assert torch.equal(graphed[3], lens) and torch.equal(graphed[0], kp)
    gen = torch.Generator(device=cuda_device)
    gen.manual_seed(97)
    for rep in range(5):
        kn.copy_(torch.randn(kn.shape, generator=gen, device=cuda_device).to(torch.bfloat16))
        vn.copy_(torch.randn(vn.shape, generator=gen, device=cuda_device).to(torch.bfloat16))
        q.copy_(torch.randn(q.shape, generator=gen, device=cuda_device).to(torch.bfloat16))
        ref = outputs()
        step(eager, ref)
        poison(*outs)
        torch.cuda.synchronize()
        replay(g)
        assert_same(outs, ref, f"paged step {rep}")
        assert_same(graphed, eager, f"paged state after step {rep}")
    assert graphed[3].tolist() == [705, 68, 69, 6, 768, 768]
    say("paged serving step: 5 replays identical to the eager steps (appends included)")


def test_decode_deterministic_flag(cuda_device):
    """The one-launch decode path (256 units) gives the same bits on every call
    under DSA_DETERMINISTIC; without it the chunks are taken first come first
    served, the selection is the same and the outputs agree to the rounding of
    the merge order."""
    w = DECODES[1]
    S, Hq, Hkv, L, d = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim
    q, kc, vc = make_decode(w, device=cuda_device)
    kbar = dsa.kv_block_means(kc, w.block)
    runs = {}
    for name, fl in (("fixed", dsa.DETERMINISTIC), ("free", 0)):
        shape = dsa.make_shape(S, Hq, Hkv, L, d, w.block, w.topk, flags=dsa.FORCE_SINK | dsa.FORCE_DIAG | fl)
        km = dsa.dsa_kmax(shape)
        assert dsa.dsa_decode_workspace_bytes(shape) == 0  # the one-launch path
        outs = []
        for _ in range(4):
            o = torch.empty_like(q)
            lse = torch.empty((S, Hq), dtype=torch.float32, device=cuda_device)
            idx = torch.empty((S, Hkv, km), dtype=torch.int32, device=cuda_device)
            dsa.dsa_decode(shape, q, kc, vc, kbar, o, lse, idx, torch.empty(1, dtype=torch.uint8, device=cuda_device))
            outs.append((o, lse, idx))
        torch.cuda.synchronize()
        runs[name] = outs
    for o, lse, idx in runs["fixed"][1:]:
        assert_same((o, lse, idx), runs["fixed"][0], "deterministic decode")
    ref = runs["fixed"][0]
    for o, lse, idx in runs["free"]:
        assert torch.equal(idx, ref[2])
        assert (o.float() - ref[0].float()).abs().max() <= 2 ** -7 * ref[0].float().abs().max()
        assert torch.allclose(lse, ref[1], rtol=1e-5, atol=1e-5)
    say("decode: DSA_DETERMINISTIC gives identical bits; first come first served agrees to rounding")


def test_paged_deterministic_flag(cuda_device):
    """dsa_paged_decode under DSA_DETERMINISTIC gives the same bits on every
    call; without it the chunks are taken first come first served: the same
    selection and outputs that agree to the rounding of the merge order."""
    w = Workload("g_paged_det", "decode", 64, 16, 4, 64 * 40, 128, 64, 12, structure="planted", amplitude=3.0, seed=98)
    S, Hq, Hkv, L, d, b = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block
    mb = L // b
    q, kc, vc = make_decode(w, device=cuda_device)
    n_pages = S * mb
    perm = torch.randperm(n_pages, generator=torch.Generator(device="cpu").manual_seed(99))
    table = perm.view(S, mb).to(torch.int32).to(cuda_device)
    kp = torch.empty((n_pages, Hkv, b, d), dtype=torch.bfloat16, device=cuda_device)
    vp = torch.empty_like(kp)
    flat = table.reshape(-1).long()
    kp[flat] = kc.view(S, Hkv, mb, b, d).permute(0, 2, 1, 3, 4).reshape(S * mb, Hkv, b, d)
    vp[flat] = vc.view(S, Hkv, mb, b, d).permute(0, 2, 1, 3, 4).reshape(S * mb, Hkv, b, d)
    lens = torch.randint(1, L + 1, (S,), generator=torch.Generator(device="cpu").manual_seed(100))
    lens = lens.to(torch.int32).to(cuda_device)
    kbar = torch.zeros((n_pages, Hkv, d), dtype=torch.float32, device=cuda_device)
    dsa.dsa_paged_kv_block_means(dsa.make_shape(S, Hq, Hkv, L, d, b, w.topk), kp, table, lens, kbar)
    runs = {}
    for name, fl in (("fixed", dsa.DETERMINISTIC), ("free", 0)):
        runs[name] = [dsa.paged_decode(q, kp, vp, kbar, table, lens, b, w.topk, flags=3 | fl) for _ in range(3)]
    torch.cuda.synchronize()
    ref = runs["fixed"][0]
    for r in runs["fixed"][1:]:
        assert_same(r, ref, "deterministic paged decode")
    for o, lse, idx, cnt in runs["free"]:
        assert torch.equal(idx, ref[2]) and torch.equal(cnt, ref[3])
        assert (o.float() - ref[0].float()).abs().max() <= 2 ** -7 * ref[0].float().abs().max()
        assert torch.allclose(lse, ref[1], rtol=1e-5, atol=1e-5)
    say("paged decode: DSA_DETERMINISTIC gives identical bits; first come first served agrees to rounding")
