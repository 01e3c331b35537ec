"""One workload, nothing else, for a profiler to watch.

    python3 -m dynamic_block_sparse_dsa_amd.profile_run attn   --workload prefill_n8192_h32 --reps 3
    python3 -m dynamic_block_sparse_dsa_amd.profile_run decode --workload decode_s32_l65536 --reps 3
    python3 -m dynamic_block_sparse_dsa_amd.profile_run bwd    --workload prefill_n8192_h32 --reps 3
    python3 -m dynamic_block_sparse_dsa_amd.profile_run index  --workload index_n8192 --reps 3
    python3 -m dynamic_block_sparse_dsa_amd.profile_run copy   --mib 256 --reps 3
    python3 -m dynamic_block_sparse_dsa_amd.profile_run gemm   --n 8192 --reps 3

``attn`` selects once (dsa_prefill) and then launches dsa_sparse_attn_fwd
``reps`` times on the same indices; ``bwd`` selects and attends once and then
launches dsa_sparse_attn_bwd ``reps`` times (seeded output gradient);
``decode`` runs ``reps`` decode steps; ``index`` runs ``reps`` token-indexer
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
    ap.add_argument("what", choices=["attn", "bwd", "decode", "index", "copy", "gemm"])
    ap.add_argument("--workload", default=None)
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--mib", type=int, default=256)
    ap.add_argument("--n", type=int, default=8192)
    a = ap.parse_args(argv)
    dsa.load()
    stream = torch.cuda.Stream()
    if a.what == "copy":
        run_copy(a.mib, a.reps, stream)
    elif a.what == "gemm":
        run_gemm(a.n, a.reps, stream)
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
