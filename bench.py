#!/usr/bin/env python3
"""Throughput of block-sparse attention on one MI355X.

Prints one JSON line.  The step is one fused prefill (block means of Q and
K, block scores, top-k selection, sparse attention) over inputs already
resident in device memory; `value` is prefill tokens/s.  `roofline` prices
the sparse-attention kernel (where nearly all the time goes) against the
bf16 MFMA peak using its algorithmic FLOPs (4*b*b*d per executed tile) over
its average launch time from HIP events on the stream it runs on.  `decode`
reports a single-token decode step of 32 sequences against the HBM peak.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same
prefill workload.  The headline workload is the 131 072-token prefill (the
largest configuration); the 8 192-token and the grouped-query 32 768-token
prefills are reported beside it under `prefill_workloads`.  Every timed
prefill launch follows a 512 MiB read that evicts the last-level cache.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn prefill tokens/s + % MFMA peak; decode tokens/s + % HBM BW"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
# L2 -> CU fill path: 64 bytes per clock per CU (measured 62.7 with LDS DMA
# from an L2-resident source) x 256 CUs x 2.4 GHz
PEAK_FILL_GBS = 64 * 256 * 2.4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
ATTN_SRC = os.path.join(ROOT, "dynamic_block_sparse_dsa_amd", "csrc", "attn_fwd.hip")
DECODE_SRC = os.path.join(ROOT, "dynamic_block_sparse_dsa_amd", "csrc", "decode.hip")
BWD_SRC = os.path.join(ROOT, "dynamic_block_sparse_dsa_amd", "csrc", "attn_bwd.hip")
INDEX_SRC = os.path.join(ROOT, "dynamic_block_sparse_dsa_amd", "csrc", "indexer.hip")
PAGED_SRC = os.path.join(ROOT, "dynamic_block_sparse_dsa_amd", "csrc", "decode_paged.hip")


def log(msg):
    """Progress on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def src_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(workload, kernel_src):
    """HBM bytes per launch from the committed counter summary, or None when
    it is missing or was taken on a different kernel source."""
    try:
        t = json.load(open(TRAFFIC_FILE))[workload]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("src_sha256_16") != src_hash(kernel_src):
        return None
    return t.get("bytes_per_launch")


def time_events(fn, n, stream):
    import torch

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) / n  # ms per launch


def read_flush(flush, stream):
    """Evict the last-level cache by reading a buffer twice its size (a
    write-based flush would leave dirty lines whose write-back is charged to
    the next timed launch)."""
    import torch

    with torch.cuda.stream(stream):
        flush.sum()


def stats_us(t):
    """median, min and 90th percentile of a list of times in us."""
    import statistics

    t = sorted(t)
    return dict(median=round(statistics.median(t), 2), min=round(t[0], 2),
                p90=round(t[min(len(t) - 1, int(0.9 * len(t)))], 2), n=len(t))


def bench_prefill(args, dev, stream, flush, wname, n_steps):
    """One prefill workload: the fused step (dsa_prefill: block means, block
    scores, top-k, attention) timed alone n_steps times with HIP events after
    a read-based cache flush each, then the attention kernel alone, also
    flushed before each launch."""
    import torch

    import dynamic_block_sparse_dsa_amd as dsa
    from dynamic_block_sparse_dsa_amd import work
    from dynamic_block_sparse_dsa_amd.inputs import WORKLOADS, make_prefill

    w = WORKLOADS[wname]
    log(f"prefill {wname}: inputs")
    q, k, v = make_prefill(w, device=dev)
    B, Hq, Hkv, N, d, nB = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.n_blocks
    shape = dsa.make_shape(B, Hq, Hkv, N, d, w.block, w.topk, w.topk_num, w.topk_den)
    km = dsa.dsa_kmax(shape)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Hkv, nB, km), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hkv, nB), dtype=torch.int32, device=dev)
    ws = torch.empty(dsa.dsa_prefill_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        dsa.dsa_prefill(shape, q, k, v, o, lse, idx, cnt, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    steps_us = []
    for _ in range(n_steps):
        read_flush(flush, stream)
        steps_us.append(time_events(step, 1, stream) * 1e3)
    ms_step = sum(steps_us) / len(steps_us) * 1e-3

    # the dominant kernel alone, same inputs and indices, HIP events on its stream
    def attn():
        dsa.dsa_sparse_attn_fwd(shape, q, k, v, idx, cnt, o, lse, stream=stream)

    for _ in range(args.warmup):
        attn()
    attn_us = []
    for _ in range(max(n_steps, 20)):
        read_flush(flush, stream)
        attn_us.append(time_events(attn, 1, stream) * 1e3)
    ms_attn = sum(attn_us) / len(attn_us) * 1e-3
    log(f"prefill {wname}: step {ms_step:.3f} ms, attention {ms_attn:.3f} ms")
    cnt_h = cnt.cpu().numpy()
    flops = work.prefill_flops(cnt_h, w.group, w.block, d)
    tflops = flops / (ms_attn * 1e-3) / 1e12
    tiles = work.prefill_tiles(cnt_h, w.group)
    traffic = measured_traffic(w.name, ATTN_SRC)
    res = dict(
        ms_per_step=ms_step,
        step_us=stats_us(steps_us),
        value=B * N / (ms_step * 1e-3),
        config=dict(workload=w.name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, seq_len=N, head_dim=d, block=w.block,
                    topk=w.topk, topk_num=w.topk_num, topk_den=w.topk_den, structure=w.structure),
        roofline=dict(bound="mfma", achieved=round(tflops, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                      frac=round(tflops / PEAK_BF16_TFLOPS, 4), traffic=traffic, kernel="sparse_attn_fwd_kernel",
                      avg_launch_us=round(ms_attn * 1e3, 2), launch_us=stats_us(attn_us), flops_per_launch=flops,
                      executed_tiles=tiles,
                      step_frac=round(flops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)),
    )
    return res, (q, k, v, w)


def bench_decode(args, dev, stream, flush):
    import torch

    import dynamic_block_sparse_dsa_amd as dsa
    from dynamic_block_sparse_dsa_amd import work
    from dynamic_block_sparse_dsa_amd.inputs import WORKLOADS, make_decode

    w = WORKLOADS[args.decode_workload]
    q, kc, vc = make_decode(w, device=dev)
    S, Hq, Hkv, L, d, nB = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.n_blocks
    shape = dsa.make_shape(S, Hq, Hkv, L, d, w.block, w.topk, w.topk_num, w.topk_den)
    km = dsa.dsa_kmax(shape)
    kbar = torch.empty((S, Hkv, nB, d), dtype=torch.float32, device=dev)
    dsa.dsa_kv_block_means(shape, kc, kbar, stream=stream)  # cache-time work, outside the step
    o = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device=dev)
    idx = torch.empty((S, Hkv, km), dtype=torch.int32, device=dev)
    ws = torch.empty(dsa.dsa_decode_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        dsa.dsa_decode(shape, q, kc, vc, kbar, o, lse, idx, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    # each step timed alone with events, the cache flushed in between
    steps_us = []
    for _ in range(args.steps):
        read_flush(flush, stream)
        steps_us.append(time_events(step, 1, stream) * 1e3)
    ms = sum(steps_us) / len(steps_us) * 1e-3
    step_stats = stats_us(steps_us)
    nbytes = work.decode_bytes(S, Hq, Hkv, L, d, w.block, km)
    gbs = nbytes / (ms * 1e-3) / 1e9
    args._decode_inputs = (q, kc, vc, w, flush)  # reused by the paged bench

    # the same step captured in a HIP graph and replayed (the library records
    # no allocation or memset), timed the same way; its selection must equal
    # the eager step's and its outputs agree to the rounding of the merge order
    # (the one-launch path takes chunks first come first served unless the
    # shape asks for DSA_DETERMINISTIC)
    o_eager, lse_eager, idx_eager = o.clone(), lse.clone(), idx.clone()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        dsa.dsa_decode(shape, q, kc, vc, kbar, o, lse, idx, ws)

    def replay():
        with torch.cuda.stream(stream):
            graph.replay()

    for _ in range(args.warmup):
        replay()
    graph_us = []
    for _ in range(args.steps):
        read_flush(flush, stream)
        graph_us.append(time_events(replay, 1, stream) * 1e3)
    torch.cuda.synchronize()
    graph_check = dict(idx_equal=bool(torch.equal(idx, idx_eager)),
                       o_max_abs_diff=float((o.float() - o_eager.float()).abs().max()),
                       lse_max_abs_diff=float((lse - lse_eager).abs().max()))
    del graph
    return dict(
        value=S / (ms * 1e-3), unit="tokens/s", ms_per_step=ms, step_us=step_stats,
        graph_step_us=dict(stats_us(graph_us), **graph_check),
        config=dict(workload=w.name, sequences=S, n_q_heads=Hq, n_kv_heads=Hkv, cache_len=L, head_dim=d,
                    block=w.block, topk=w.topk),
        roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=round(gbs / PEAK_HBM_GBS, 4), traffic=measured_traffic(w.name, DECODE_SRC),
                      kernel=("decode step: decode_fused_kernel, one launch" if S * Hkv >= 256 else
                              "decode step: select, split attention, combine"), bytes_per_step=nbytes),
    )


def bench_paged(args, dev, stream):
    """dsa_paged_decode on the decode workload's caches scattered into
    shuffled pages: every sequence at full length, then lengths drawn in
    [L/4, L]; each step timed alone with events after a read-based cache
    flush, priced in algorithmic bytes (work.paged_decode_bytes).  Also one
    dsa_paged_kv_append of a token per sequence."""
    import torch

    import dynamic_block_sparse_dsa_amd as dsa
    from dynamic_block_sparse_dsa_amd import work

    q, kc, vc, w, flush = args._decode_inputs
    S, Hq, Hkv, L, d, b = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block
    mb = -(-L // b)
    n_pages = S * mb + 64  # room for appends
    g = torch.Generator(device="cpu")
    g.manual_seed(9)
    table = torch.randperm(n_pages, generator=g)[: S * mb].view(S, mb).to(torch.int32).to(dev)
    kp = torch.empty((n_pages, Hkv, b, d), dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    flat = table.reshape(-1).long()
    kp[flat] = kc.view(S, Hkv, mb, b, d).permute(0, 2, 1, 3, 4).reshape(S * mb, Hkv, b, d)
    vp[flat] = vc.view(S, Hkv, mb, b, d).permute(0, 2, 1, 3, 4).reshape(S * mb, Hkv, b, d)
    kbar = torch.zeros((n_pages, Hkv, d), dtype=torch.float32, device=dev)
    shape = dsa.make_shape(S, Hq, Hkv, mb * b, d, b, w.topk, w.topk_num, w.topk_den)
    km = dsa.dsa_kmax(shape)
    o = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device=dev)
    idx = torch.empty((S, Hkv, km), dtype=torch.int32, device=dev)
    cnt = torch.empty((S, Hkv), dtype=torch.int32, device=dev)
    out = {}
    gl = torch.Generator(device="cpu")
    gl.manual_seed(10)
    cases = [("full_length", [L] * S),
             ("mixed_lengths", torch.randint(L // 4, L + 1, (S,), generator=gl).tolist())]
    for name, lens_list in cases:
        lens = torch.tensor(lens_list, dtype=torch.int32, device=dev)
        dsa.dsa_paged_kv_block_means(shape, kp, table, lens, kbar, stream=stream)

        def step():
            dsa.dsa_paged_decode(shape, q, kp, vp, kbar, table, lens, o, lse, idx, cnt, stream=stream)

        for _ in range(args.warmup):
            step()
        tot = 0.0
        for _ in range(args.steps):
            with torch.cuda.stream(stream):
                flush.sum()
            tot += time_events(step, 1, stream)
        ms = tot / args.steps
        nbytes = work.paged_decode_bytes(lens.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), Hq, d, b)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = dict(value=S / (ms * 1e-3), unit="tokens/s", ms_per_step=ms, tokens_in_caches=int(sum(lens_list)),
                         roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                                       frac=round(gbs / PEAK_HBM_GBS, 4), bytes_per_step=nbytes,
                                       traffic=(measured_traffic("paged_" + w.name, PAGED_SRC)
                                                if name == "full_length" else None),
                                       kernel="decode_paged_kernel"))
    # the same caches in FP8 (E4M3 codes, a scale per row), full length
    k8 = torch.empty((n_pages, Hkv, b, d), dtype=torch.uint8, device=dev)
    v8 = torch.empty_like(k8)
    ks = torch.empty((n_pages, Hkv, b), dtype=torch.float32, device=dev)
    vs = torch.empty_like(ks)
    dsa.dsa_paged_quantize_fp8(shape, kp, vp, k8, v8, ks, vs, stream=stream)
    lens = torch.full((S,), L, dtype=torch.int32, device=dev)
    dsa.dsa_paged_kv_block_means_fp8(shape, k8, ks, table, lens, kbar, stream=stream)

    def step8():
        dsa.dsa_paged_decode_fp8(shape, q, k8, v8, ks, vs, kbar, table, lens, o, lse, idx, cnt, stream=stream)

    for _ in range(args.warmup):
        step8()
    tot = 0.0
    for _ in range(args.steps):
        with torch.cuda.stream(stream):
            flush.sum()
        tot += time_events(step8, 1, stream)
    ms = tot / args.steps
    nbytes = work.paged_decode_bytes(lens.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), Hq, d, b, kv_bytes=1,
                                     row_scales=True)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out["fp8_full_length"] = dict(value=S / (ms * 1e-3), unit="tokens/s", ms_per_step=ms,
                                  roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                                                frac=round(gbs / PEAK_HBM_GBS, 4), bytes_per_step=nbytes,
                                                traffic=measured_traffic("paged8_" + w.name, PAGED_SRC),
                                                kernel="decode_paged_kernel (fp8)"))
    # one append of a token per sequence (the mixed lengths leave room)
    kn = torch.randn((S, Hkv, d), device=dev).to(torch.bfloat16)
    vn = torch.randn((S, Hkv, d), device=dev).to(torch.bfloat16)
    lens = torch.tensor(cases[1][1], dtype=torch.int32, device=dev).clamp(max=L - args.steps - args.warmup - 1)

    def app():
        dsa.dsa_paged_kv_append(shape, kn, vn, table, lens, kp, vp, kbar, stream=stream)

    for _ in range(args.warmup):
        app()
    out["append_us"] = round(time_events(app, args.steps, stream) * 1e3, 2)

    def app8():
        dsa.dsa_paged_kv_append_fp8(shape, kn, vn, table, lens, k8, v8, ks, vs, kbar, stream=stream)

    lens = torch.tensor(cases[1][1], dtype=torch.int32, device=dev).clamp(max=L - 2 * (args.steps + args.warmup) - 1)
    for _ in range(args.warmup):
        app8()
    out["append_fp8_us"] = round(time_events(app8, args.steps, stream) * 1e3, 2)
    out["config"] = dict(workload=w.name + "_paged", sequences=S, n_q_heads=Hq, n_kv_heads=Hkv, capacity=L, head_dim=d,
                         block=b, topk=w.topk, pages=n_pages)
    return out


def bench_backward(args, dev, stream, inputs):
    """dsa_sparse_attn_bwd on the prefill workload (selection and forward from
    dsa_prefill, a seeded output gradient): event-timed over its four
    launches.  Algorithmic FLOPs: the five products a backward needs per kept
    tile (S recomputed, dP, dV, dQ, dK), 2.5x the forward's."""
    import torch

    import dynamic_block_sparse_dsa_amd as dsa
    from dynamic_block_sparse_dsa_amd import work

    q, k, v, w = inputs
    B, Hq, Hkv, N, d, nB = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.n_blocks
    o, lse, idx, cnt = dsa.prefill(q, k, v, w.block, w.topk, w.topk_num, w.topk_den, stream=stream)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    dout = torch.randn(q.shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    shape = dsa.make_shape(B, Hq, Hkv, N, d, w.block, w.topk, w.topk_num, w.topk_den)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(dsa.dsa_attn_bwd_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        dsa.dsa_sparse_attn_bwd(shape, q, k, v, o, lse, dout, idx, cnt, dq, dk, dv, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    ms = time_events(step, args.steps, stream)
    flops = 2.5 * work.prefill_flops(cnt.cpu().numpy(), w.group, w.block, d)
    tflops = flops / (ms * 1e-3) / 1e12
    return dict(value=B * N / (ms * 1e-3), unit="tokens/s", ms_per_step=ms,
                config=dict(workload=w.name),
                roofline=dict(bound="mfma", achieved=round(tflops, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                              frac=round(tflops / PEAK_BF16_TFLOPS, 4),
                              traffic=measured_traffic("backward_" + w.name, BWD_SRC),
                              kernel="backward step: prep, invert, dq, dkdv", flops_per_step=flops))


SELECT_VARIANTS = [
    ("topk", {}),
    ("anchors4_window4", dict(n_anchor=4, window=4)),
    ("threshold_0.02", dict(select_mode=1, threshold=0.02)),
    ("entropy_2_24", dict(select_mode=2, k_min=2, k_max=24)),
]


def bench_selection(args, dev, stream, inputs):
    """dsa_select_topk for each selection variant on the prefill workload's
    block scores, and dsa_indices_to_bitmap on the top-k selection; each
    event-timed alone.  Bytes per launch: the visible (causal) scores read
    plus the index rows and counts written; priced against HBM."""
    import torch

    import dynamic_block_sparse_dsa_amd as dsa

    q, k, v, w = inputs
    B, Hq, Hkv, N, d, nB = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.n_blocks
    base = dsa.make_shape(B, Hq, Hkv, N, d, w.block, w.topk, w.topk_num, w.topk_den)
    qbar = torch.empty((B, Hq, nB, d), dtype=torch.float32, device=dev)
    kbar = torch.empty((B, Hkv, nB, d), dtype=torch.float32, device=dev)
    sc = torch.empty((B, Hkv, nB, nB), dtype=torch.float32, device=dev)
    dsa.dsa_block_means(base, Hq, q, qbar, stream=stream)
    dsa.dsa_block_means(base, Hkv, k, kbar, stream=stream)
    dsa.dsa_block_scores_from_means(base, qbar, kbar, sc, stream=stream)
    rows = B * Hkv * nB
    out = {}
    for name, sel in SELECT_VARIANTS:
        topk = w.topk if not sel.get("select_mode") else 0
        shape = dsa.make_shape(B, Hq, Hkv, N, d, w.block, topk, w.topk_num, w.topk_den, **sel)
        km = dsa.dsa_kmax(shape)
        idx = torch.empty((B, Hkv, nB, km), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, Hkv, nB), dtype=torch.int32, device=dev)

        def step():
            dsa.dsa_select_topk(shape, sc, idx, cnt, stream=stream)

        for _ in range(args.warmup):
            step()
        ms = time_events(step, args.steps, stream)
        nbytes = B * Hkv * (nB * (nB + 1) // 2) * 4 + rows * (km + 1) * 4
        gbs = nbytes / (ms * 1e-3) / 1e9
        c = cnt.float()
        out[name] = dict(us=round(ms * 1e3, 2), kept_mean=round(float(c.mean()), 2), kept_max=int(c.max()),
                         index_width=km, bytes_per_launch=nbytes, achieved_GBs=round(gbs, 1),
                         frac_hbm=round(gbs / PEAK_HBM_GBS, 5))
        if name == "topk":
            bm = torch.empty((B, Hkv, nB, (nB + 31) // 32), dtype=torch.int32, device=dev)

            def pack():
                dsa.dsa_indices_to_bitmap(idx, cnt, nB, bm, stream=stream)

            for _ in range(args.warmup):
                pack()
            ms_b = time_events(pack, args.steps, stream)
            out["bitmap_us"] = round(ms_b * 1e3, 2)
    out["config"] = dict(workload=w.name, rows=rows, kernel="select_topk_wave_kernel", bound="hbm (launch-bound at "
                         "this size)")
    return out


def bench_index(args, dev, stream, wname=None):
    """Token-level indexer workload: the chained step (wall clock) and its
    launches alone (HIP events): the fused index scores + token selection
    (index_topk_kernel, plus index_merge_kernel for rows longer than one chunk
    of keys) and the token attention.  Algorithmic work: index scores 2 HI dI
    FLOP per causal (query token, token) pair (MFMA); token attention reads Q
    and every KV head's K and V rows once and writes O (unique bytes, priced
    against HBM), and gathers the kept tokens' K and V rows of every KV head
    (d * 2 bytes each, mostly L2 hits)."""
    import torch

    import dynamic_block_sparse_dsa_amd as dsa
    from dynamic_block_sparse_dsa_amd.inputs import INDEX_WORKLOADS, make_index

    w = INDEX_WORKLOADS[wname or args.index_workload]
    qi, ki, wi, q, k, v = make_index(w, device=dev)
    B, Hq, Hkv, N, d, HI, dI = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.n_index_heads, w.index_dim
    shape = dsa.make_index_shape(B, Hq, Hkv, N, d, HI, dI, w.topk)
    km = dsa.dsa_index_kmax(shape)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    idx = torch.empty((B, N, km), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, N), dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, dsa.dsa_index_workspace_bytes(shape)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        dsa.dsa_index_prefill(shape, qi, ki, wi, q, k, v, o, lse, idx, cnt, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    parts = dict(
        topk=lambda: dsa.dsa_index_topk(shape, qi, ki, wi, idx, cnt, ws, stream=stream),
        attention=lambda: dsa.dsa_token_attn_fwd(shape, q, k, v, idx, cnt, o, lse, stream=stream),
    )
    us = {}
    for name, fn in parts.items():
        for _ in range(args.warmup):
            fn()
        us[name] = time_events(fn, args.steps, stream) * 1e3
    pairs = B * N * (N + 1) // 2
    flops = 2 * HI * dI * pairs
    kept = int(cnt.sum())
    gather_bytes = kept * Hkv * d * 2 * 2 + 2 * B * Hq * N * d * 2
    unique_bytes = 2 * B * Hq * N * d * 2 + 2 * B * Hkv * N * d * 2
    tf = flops / (us["topk"] * 1e-6) / 1e12
    att_gbs = unique_bytes / (us["attention"] * 1e-6) / 1e9
    fill_gbs = gather_bytes / (us["attention"] * 1e-6) / 1e9
    return dict(
        value=B * N / (ms_step * 1e-3), unit="tokens/s", ms_per_step=ms_step,
        config=dict(workload=w.name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, seq_len=N, head_dim=d, index_heads=HI,
                    index_dim=dI, topk=w.topk),
        kernels_us={kk: round(vv, 2) for kk, vv in us.items()},
        roofline=dict(bound="mfma", achieved=round(tf, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                      frac=round(tf / PEAK_BF16_TFLOPS, 4), traffic=measured_traffic("index_" + w.name, INDEX_SRC),
                      kernel="index_topk_kernel + index_merge_kernel", flops_per_launch=flops),
        attention_roofline=dict(bound="hbm", achieved=round(att_gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                                frac=round(att_gbs / PEAK_HBM_GBS, 4), bytes_per_launch=unique_bytes,
                                mfma_frac=round(4 * Hq * kept * d / (us["attention"] * 1e-6) / 1e12
                                                / PEAK_BF16_TFLOPS, 4),
                                # the gathered rows come mostly from the L2s (the K and V of
                                # one KV head fit one XCD's L2): the L2 -> CU fill rate
                                gather_bytes=gather_bytes, gather_gbs=round(fill_gbs, 1),
                                gather_frac_of_l2_fill=round(fill_gbs / PEAK_FILL_GBS, 4)),
    )


def ceilings(dev, stream):
    """Measured ceilings for context (library and torch code, not this
    library's path): a bf16 GEMM through torch.matmul (hipBLASLt) and a plain
    device-to-device copy, each timed with HIP events."""
    import torch

    n = 8192
    with torch.cuda.stream(stream):
        a = torch.randn((n, n), device=dev, dtype=torch.float32).to(torch.bfloat16)
        b = torch.randn((n, n), device=dev, dtype=torch.float32).to(torch.bfloat16)
        c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
        src = torch.ones(1 << 28, device=dev, dtype=torch.float32)  # 1 GiB
        dst = torch.empty_like(src)

    def gemm():
        with torch.cuda.stream(stream):
            torch.matmul(a, b, out=c)

    def copy():
        with torch.cuda.stream(stream):
            dst.copy_(src)

    for _ in range(3):
        gemm()
        copy()
    ms_g = time_events(gemm, 10, stream)
    ms_c = time_events(copy, 5, stream)
    return dict(gemm_bf16=dict(shape=[n, n, n], tflops=round(2 * n**3 / (ms_g * 1e-3) / 1e12, 1),
                               frac_of_peak=round(2 * n**3 / (ms_g * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                               source="torch.matmul (hipBLASLt)"),
                copy=dict(bytes=2 * src.numel() * 4, gbs=round(2 * src.numel() * 4 / (ms_c * 1e-3) / 1e9, 1),
                          frac_of_peak=round(2 * src.numel() * 4 / (ms_c * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                          source="torch copy_, 1 GiB read + 1 GiB written"))


def cpu_baseline(args, inputs):
    """The oracle, as it stands, on a seeded sample of the prefill workload,
    with as many BLAS threads as the process has host cores.  For sampled KV
    groups it runs the whole selection (block means, block scores, top-k) and
    for sampled query blocks (drawn uniformly over heads and blocks) the
    attention, each timed; the time of the full problem is extrapolated as
    groups x selection time per group + query blocks x attention time per
    block.  Host copies and the fp64 upcast of the inputs are not timed."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O

    q, k, v, w = inputs
    G, nB = w.group, w.n_blocks
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(12345)
    groups = [int(x) for x in rng.permutation(w.n_kv_heads)][:2]
    t_sel, t_att, n_att = 0.0, 0.0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=cores):
        for n, g in enumerate(groups):
            qn = q[:, g * G : (g + 1) * G].float().cpu().numpy().astype(np.float64)
            kn = k[:, g : g + 1].float().cpu().numpy().astype(np.float64)
            vn = v[:, g : g + 1].float().cpu().numpy().astype(np.float64)
            s0 = time.perf_counter()
            qbar, kbar = O.block_means(qn, w.block), O.block_means(kn, w.block)
            sc = O.block_scores(qbar, kbar, 1.0 / (w.head_dim ** 0.5))
            idx, cnt, _ = O.select_topk(sc, w.topk, w.topk_num, w.topk_den)
            t_sel += time.perf_counter() - s0
            # attention of query blocks of this group until its share of the budget is spent
            deadline = t0 + args.cpu_seconds * (n + 1) / len(groups)
            while True:
                hh, i = int(rng.integers(G)), int(rng.integers(nB))
                s0 = time.perf_counter()
                O.attend(qn[:, hh : hh + 1], kn, vn, idx, cnt, w.block, units=[(0, 0, i)])
                t_att += time.perf_counter() - s0
                n_att += 1
                if time.perf_counter() >= deadline:
                    break
    n_sel = len(groups)
    blocks_total = w.batch * w.n_q_heads * nB
    t_full = w.batch * w.n_kv_heads * (t_sel / n_sel) + blocks_total * (t_att / max(n_att, 1))
    return dict(value=round(w.batch * w.seq_len / t_full, 2), unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{w.name}: selection (block means, scores, top-k) of {n_sel} of {w.batch * w.n_kv_heads} KV "
                       f"groups ({t_sel:.1f} s), attention of {n_att} of {blocks_total} query blocks drawn uniformly, "
                       f"seed 12345 ({t_att:.1f} s); extrapolated full-problem time {t_full:.0f} s; "
                       f"{cores} BLAS threads")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_n131072_b128")
    ap.add_argument("--extra-workloads", default="prefill_n8192_h32,prefill_gqa_n32768",
                    help="comma-separated prefill workloads reported beside the headline ('' for none)")
    ap.add_argument("--decode-workload", default="decode_s32_l65536")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-selection", action="store_true")
    ap.add_argument("--no-index", action="store_true")
    ap.add_argument("--no-paged", action="store_true")
    ap.add_argument("--index-workload", default="index_n8192")
    ap.add_argument("--extra-index-workloads", default="index_n32768",
                    help="comma-separated token-indexer workloads reported beside it ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}); the library has no multi-GPU path",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    import dynamic_block_sparse_dsa_amd as dsa

    dsa.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    # 512 MiB, twice the last-level cache, read between timed launches
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    pre, inputs = bench_prefill(args, dev, stream, flush, args.workload, args.steps)
    out = {
        "metric": METRIC,
        "value": round(pre["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "step_us": pre["step_us"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": pre["config"],
        "roofline": pre["roofline"],
    }
    extra = [x for x in args.extra_workloads.split(",") if x and x != args.workload]
    if extra:
        out["prefill_workloads"] = {}
        for name in extra:
            r, _ = bench_prefill(args, dev, stream, flush, name, args.steps)
            out["prefill_workloads"][name] = dict(value=round(r["value"], 1), unit="tokens/s",
                                                  ms_per_step=round(r["ms_per_step"], 4), step_us=r["step_us"],
                                                  config=r["config"], roofline=r["roofline"])
            torch.cuda.empty_cache()
    if not args.no_decode:
        log("decode")
        out["decode"] = bench_decode(args, dev, stream, flush)
        if not args.no_paged:
            log("paged decode")
            out["paged_decode"] = bench_paged(args, dev, stream)
        del args._decode_inputs
    if not args.no_backward:
        log("backward")
        out["backward"] = bench_backward(args, dev, stream, inputs)
    if not args.no_selection:
        log("selection variants")
        out["selection"] = bench_selection(args, dev, stream, inputs)
    if not args.no_index:
        log("token indexer")
        out["indexer"] = bench_index(args, dev, stream)
        extra = [x for x in args.extra_index_workloads.split(",") if x and x != args.index_workload]
        if extra:
            out["indexer_workloads"] = {x: bench_index(args, dev, stream, x) for x in extra}
    if not args.no_ceilings:
        log("ceilings")
        out["ceilings"] = ceilings(dev, stream)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(args, inputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
