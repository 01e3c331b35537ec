"""One workload, nothing else, for a profiler to watch.

    python3 -m dynamic_block_sparse_dsa_amd.profile_run attn   --workload prefill_n8192_h32 --reps 3
    python3 -m dynamic_block_sparse_dsa_amd.profile_run decode --workload decode_s32_l65536 --reps 3
    python3 -m dynamic_block_sparse_dsa_amd.profile_run paged  --workload decode_s32_l65536 --reps 3 [--fp8]
    python3 -m dynamic_block_sparse_dsa_amd.profile_run bwd    --workload prefill_n8192_h32 --reps 3
    python3 -m dynamic_block_sparse_dsa_amd.profile_run index  --workload index_n8192 --reps 3
    python3 -m dynamic_block_sparse_dsa_amd.profile_run copy   --mib 256 --reps 3
    python3 -m dynamic_block_sparse_dsa_amd.profile_run gemm   --n 8192 --reps 3

``attn`` selects once (dsa_prefill) and then launches dsa_sparse_attn_fwd
``reps`` times on the same indices; ``bwd`` selects and attends once and then
launches dsa_sparse_attn_bwd ``reps`` times (seeded output gradient);
``decode`` runs ``reps`` decode steps; ``paged`` runs ``reps`` paged decode steps
on the same caches scattered into shuffled pages, every sequence at full
length (``--fp8``: the pools quantized to E4M3 first); ``index`` runs ``reps`` token-indexer
steps (dsa_index_prefill);
``copy`` copies a ``mib`` MiB device buffer into another ``reps`` times (a plain
copy kernel of known size: it reads and writes exactly ``mib`` MiB), which
calibrates the HBM byte counters; ``gemm`` multiplies two n x n bf16 matrices
``reps`` times with torch.matmul (the vendor library's dense GEMM: context for
the MFMA counters of the attention kernels, not part of the library).  Each
launch is followed by a device synchronisation so that counter samples are
per dispatch.
"""

import argparse
import sys

import torch

import dynamic_block_sparse_dsa_amd as dsa
from dynamic_block_sparse_dsa_amd.inputs import INDEX_WORKLOADS, WORKLOADS, make_decode, make_index, make_prefill


def run_attn(w, reps, stream):
    q, k, v = make_prefill(w, device="cuda")
    o, lse, idx, cnt = dsa.prefill(q, k, v, w.block, w.topk, w.topk_num, w.topk_den)
    shape = dsa.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block, w.topk, w.topk_num,
                           w.topk_den)
    torch.cuda.synchronize()
    for _ in range(reps):
        dsa.dsa_sparse_attn_fwd(shape, q, k, v, idx, cnt, o, lse, stream=stream)
        stream.synchronize()


def run_bwd(w, reps, stream):
    q, k, v = make_prefill(w, device="cuda")
    o, lse, idx, cnt = dsa.prefill(q, k, v, w.block, w.topk, w.topk_num, w.topk_den)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    dout = torch.randn(q.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    shape = dsa.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block, w.topk, w.topk_num,
                           w.topk_den)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(dsa.dsa_attn_bwd_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(reps):
        dsa.dsa_sparse_attn_bwd(shape, q, k, v, o, lse, dout, idx, cnt, dq, dk, dv, ws, stream=stream)
        stream.synchronize()


def run_index(w, reps, stream):
    qi, ki, wi, q, k, v = make_index(w, device="cuda")
    for _ in range(reps):
        dsa.index_prefill(qi, ki, wi, q, k, v, w.topk, stream=stream)
        stream.synchronize()


def run_decode(w, reps, stream):
    q, kc, vc = make_decode(w, device="cuda")
    S, Hq, Hkv, d, nB = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks
    shape = dsa.make_shape(S, Hq, Hkv, w.seq_len, d, w.block, w.topk, w.topk_num, w.topk_den)
    km = dsa.dsa_decode_kmax(shape)
    kbar = torch.empty((S, Hkv, nB, d), dtype=torch.float32, device="cuda")
    dsa.dsa_kv_block_means(shape, kc, kbar, stream=stream)
    o = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device="cuda")
    idx = torch.empty((S, Hkv, km), dtype=torch.int32, device="cuda")
    ws = torch.empty(dsa.dsa_decode_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(reps):
        dsa.dsa_decode(shape, q, kc, vc, kbar, o, lse, idx, ws, stream=stream)
        stream.synchronize()


def run_paged(w, reps, stream, fp8):
    q, kc, vc = make_decode(w, device="cuda")
    S, Hq, Hkv, L, d, b = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block
    mb = -(-L // b)
    n_pages = S * mb + 64
    g = torch.Generator(device="cpu")
    g.manual_seed(9)
    table = torch.randperm(n_pages, generator=g)[: S * mb].view(S, mb).to(torch.int32).to("cuda")
    kp = torch.empty((n_pages, Hkv, b, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    flat = table.reshape(-1).long()
    kp[flat] = kc.view(S, Hkv, mb, b, d).permute(0, 2, 1, 3, 4).reshape(S * mb, Hkv, b, d)
    vp[flat] = vc.view(S, Hkv, mb, b, d).permute(0, 2, 1, 3, 4).reshape(S * mb, Hkv, b, d)
    del kc, vc
    shape = dsa.make_shape(S, Hq, Hkv, mb * b, d, b, w.topk, w.topk_num, w.topk_den)
    km = dsa.dsa_kmax(shape)
    kbar = torch.zeros((n_pages, Hkv, d), dtype=torch.float32, device="cuda")
    lens = torch.full((S,), L, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device="cuda")
    idx = torch.empty((S, Hkv, km), dtype=torch.int32, device="cuda")
    cnt = torch.empty((S, Hkv), dtype=torch.int32, device="cuda")
    if fp8:
        k8 = torch.empty((n_pages, Hkv, b, d), dtype=torch.uint8, device="cuda")
        v8 = torch.empty_like(k8)
        ks = torch.empty((n_pages, Hkv, b), dtype=torch.float32, device="cuda")
        vs = torch.empty_like(ks)
        dsa.dsa_paged_quantize_fp8(shape, kp, vp, k8, v8, ks, vs, stream=stream)
        dsa.dsa_paged_kv_block_means_fp8(shape, k8, ks, table, lens, kbar, stream=stream)
    else:
        dsa.dsa_paged_kv_block_means(shape, kp, table, lens, kbar, stream=stream)
    torch.cuda.synchronize()
    for _ in range(reps):
        if fp8:
            dsa.dsa_paged_decode_fp8(shape, q, k8, v8, ks, vs, kbar, table, lens, o, lse, idx, cnt, stream=stream)
        else:
            dsa.dsa_paged_decode(shape, q, kp, vp, kbar, table, lens, o, lse, idx, cnt, stream=stream)
        stream.synchronize()


def run_copy(mib, reps, stream):
    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(reps):
            dst.copy_(src)
            stream.synchronize()


def run_gemm(n, reps, stream):
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    a = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(reps):
            torch.matmul(a, b)
            stream.synchronize()


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("what", choices=["attn", "bwd", "decode", "paged", "index", "copy", "gemm"])
    ap.add_argument("--workload", default=None)
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--mib", type=int, default=256)
    ap.add_argument("--n", type=int, default=8192)
    ap.add_argument("--fp8", action="store_true")
    a = ap.parse_args(argv)
    dsa.load()
    stream = torch.cuda.Stream()
    if a.what == "copy":
        run_copy(a.mib, a.reps, stream)
    elif a.what == "gemm":
        run_gemm(a.n, a.reps, stream)
    elif a.what == "paged":
        run_paged(WORKLOADS[a.workload or "decode_s32_l65536"], a.reps, stream, a.fp8)
    elif a.what == "index":
        run_index(INDEX_WORKLOADS[a.workload or "index_n8192"], a.reps, stream)
    else:
        name = a.workload or ("decode_s32_l65536" if a.what == "decode" else "prefill_n8192_h32")
        w = WORKLOADS[name]
        dict(attn=run_attn, bwd=run_bwd, decode=run_decode)[a.what](w, a.reps, stream)
    torch.cuda.synchronize()
    print(f"profile_run {a.what} done", flush=True)


if __name__ == "__main__":
    sys.exit(main())
