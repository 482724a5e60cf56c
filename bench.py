#!/usr/bin/env python3
"""Benchmark of the compressed-attention decode hot path on one MI355X.

Default workload (csa_decode_128k): CSA decode at 128K context, batch 32,
64 query heads over one shared 512-d KV entry (448 FP8 + 64 BF16), 4x
compression (32768 entries per row), indexer 16 heads x 64 dims FP4,
top-k 512, window 128, 16 planted needle blocks per row.  One step = one
decode token per row through the whole CSA path: decode_append_topk (the
ring append, the pooling and quantisation of the block every 4th token
completes, and the top-k selection, in one launch) and csa_attend (with its
split-K combine).  Steps rotate over --layers copies of
the cache (distinct HBM addresses) so that every step reads its cache cold
from HBM rather than from the 256 MB Infinity Cache, as a multi-layer decode
does.  hca_decode_1m (HCA at 1M context, batch 16: compress_append +
hca_attend) is the other workload.

The timed region replays a HIP graph of the steps (captured through
torch.cuda.graph on the library's stream); the dominant kernel's average
duration is measured with HIP events around each of its launches (eager
loop, same launch configuration).  The oracle (plain C, CPU) is timed on the
host cores on a bounded sample of the same step as the CPU baseline.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode queries/s and HBM GB/s for CSA/HCA at 128K-1M ctx; % of roofline"

WORKLOADS = {
    # name: (csa?, batch, context, ratio, heads, indexer heads, k, needles, window)
    "csa_decode_128k": (True, 32, 131072, 4, 64, 16, 512, 16, 128),
    "hca_decode_1m": (False, 16, 1048576, 128, 64, 0, 0, 0, 128),
}


# Interleaved streaming decode: `pairs` x (CSA layer, HCA layer) at `ctx`,
# each step appends one token per row to every layer and runs every layer.
# name: (batch, context, pairs, CSA heads, CSA indexer heads, CSA k, HCA heads,
#        window, needles per row, outlier channels)
INTERLEAVED = {
    # the tiny CPU-scale decode: one row at 4K, one CSA + one HCA layer of 16 heads
    "tiny_decode_4k": (1, 4096, 1, 16, 4, 64, 16, 128, 4, 0),
    "interleaved_1m": (8, 1 << 20, 8, 16, 4, 64, 64, 128, 0, 26),          # CSA layers shaped as the tiny decode
    "interleaved_1m_wide": (8, 1 << 20, 8, 64, 16, 512, 64, 128, 0, 26),   # CSA layers shaped as the 128K decode
}


# Prefill chunk: one row with a prior context given as a cache image, then a
# chunk of new tokens through compress_append, indexer_topk for every chunk
# query (causal) and csa_attend -- or, for HCA (no indexer), hca_attend over
# every block visible to each query.
# name: (prior tokens, chunk, ratio, heads, indexer heads, k, window, ring)
PREFILL = {
    "csa_prefill_chunk": (262144, 4096, 4, 64, 16, 512, 128, 8192),
    "hca_prefill_chunk": (262144, 4096, 128, 64, 0, 0, 128, 8192),
}
FP16_MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 / fp16 matrix cores
FP8_MFMA_PEAK_TFLOPS = 5000.0      # dense FP8-rate matrix peak (the scoring's FP8-rate reference)
FP4_MFMA_PEAK_TFLOPS = 10100.0     # dense MXFP4 matrix peak


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def measure_peaks():
    """The chip's ceilings measured here (libpeak.so): matrix-instruction
    issue rates with register operands (fp16 32x32x16, fp8 and fp4
    32x32x64), and HBM copy and read rates over 2 GiB buffers (far above the
    256 MB Infinity Cache).  Best of 3 timed launches each, HIP events on the
    launching stream."""
    import ctypes as C
    import torch
    lib = C.CDLL(os.path.join(ROOT, "long_context_compressed_append_amd", "libpeak.so"))
    P = C.c_void_p
    lib.peak_mfma.argtypes = [C.c_int, C.c_int, C.c_int, P, P]
    lib.peak_copy.argtypes = [P, P, C.c_int64, C.c_int, P]
    lib.peak_read.argtypes = [P, C.c_int64, C.c_int, P, P]
    stream = torch.cuda.current_stream()
    sp = P(stream.cuda_stream)

    def best_ms(launch):
        launch()                                          # warm
        ts = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return min(ts)

    out = {}
    blocks, iters = 2048, 2000                      # 8 wavefronts per SIMD
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    for kind, name, flops in ((0, "mfma_fp16_tflops", 32768), (1, "mfma_fp8_tflops", 131072),
                              (2, "mfma_fp4_tflops", 131072)):
        def go(kind=kind):
            if lib.peak_mfma(kind, blocks, iters, P(sink.data_ptr()), sp) != 0:
                raise RuntimeError("peak_mfma launch failed")
        ms = best_ms(go)
        out[name] = round(blocks * 4 * iters * 4 * flops / (ms * 1e-3) / 1e12, 1)
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(3)
    words = torch.empty(16384 * 256, dtype=torch.int32, device="cuda")

    def cp():
        if lib.peak_copy(P(src.data_ptr()), P(dst.data_ptr()), nbytes, 16384, sp) != 0:
            raise RuntimeError("peak_copy launch failed")

    def rd():
        if lib.peak_read(P(src.data_ptr()), nbytes, 16384, P(words.data_ptr()), sp) != 0:
            raise RuntimeError("peak_read launch failed")
    out["hbm_copy_gbs"] = round(2 * nbytes / (best_ms(cp) * 1e-3) / 1e9, 1)
    out["hbm_read_gbs"] = round(nbytes / (best_ms(rd) * 1e-3) / 1e9, 1)
    del src, dst, words, sink
    torch.cuda.empty_cache()
    return out


def emit(res, args):
    """Print the JSON line, with the ceilings measured in this run beside the
    published peak the roofline uses."""
    peaks = getattr(args, "peaks", None)
    if peaks:
        roof = res["roofline"]
        if roof["bound"] == "hbm":
            roof["measured_peak"] = peaks["hbm_read_gbs"]
        elif roof["kernel"] == "indexer_score":
            roof["measured_peak"] = peaks["mfma_fp8_tflops"]
        else:
            roof["measured_peak"] = peaks["mfma_fp16_tflops"]
        roof["frac_of_measured"] = round(roof["achieved"] / roof["measured_peak"], 4)
        res["config"]["measured_peaks"] = peaks
    print(json.dumps(res), flush=True)


def spread_us(durations_ms):
    """mean / p10 / p50 / p90 of per-launch durations, in microseconds."""
    d = np.asarray(durations_ms, np.float64) * 1e3
    if d.size == 0:
        return None
    return {"mean": round(float(d.mean()), 3), "p10": round(float(np.percentile(d, 10)), 3),
            "p50": round(float(np.percentile(d, 50)), 3), "p90": round(float(np.percentile(d, 90)), 3),
            "launches": int(d.size)}


def algorithmic_bytes(wl):
    """Bytes the method must move per step (entries 604 B, idx keys 34 B,
    window token 1024 B, q H*1024, out H*2048, iq+iw H_I*260, top-k 2*k*4)."""
    csa, B, ctx, m, H, HI, k, _, W = wl
    nv = ctx // m
    per_row = W * 1024 + H * 1024 + H * 2048
    if csa:
        per_row += nv * 34 + HI * 260 + 2 * k * 4 + min(k, nv) * 604
    else:
        per_row += nv * 604
    return per_row * B


def dominant_bytes(wl):
    """Algorithmic bytes of one launch of the dominant kernel."""
    csa, B, ctx, m, H, HI, k, _, W = wl
    nv = ctx // m
    if csa:   # indexer_score: every visible key (34 B) plus the query and weights
        return B * (nv * 34 + HI * 260)
    # attend (HCA): every entry, the window, q in, partial/final out
    return B * (nv * 604 + W * 1024 + H * 1024 + H * 2048)


def build_host_layer(wl, seed):
    from synth import layers as SL
    csa, B, ctx, m, H, HI, k, needles, W = wl
    L0 = ctx - 1                      # the step appends the query token -> ctx
    tag = "csa" if csa else "hca"
    t = time.time()
    ref = SL.make_layer(seed, tag, B, m, W, 256, int(csa), ctx // m + 64, [L0] * B)
    Q = SL.queries(seed, tag, B, 1, H, HI)
    if needles:
        for b in range(B):
            SL.plant_needles(ref, seed, tag, b, needles, Q["iq"][b, 0], Q["iw"][b, 0], Q["q"][b, 0])
    log(f"host image built in {time.time() - t:.1f}s")
    return ref, Q


def cpu_baseline(wl, ref, Q, tokens):
    """The oracle, as it stands, on one step of the workload for a sample of rows."""
    import oracle
    csa, B, ctx, m, H, HI, k, _, W = wl
    nthreads = oracle.nthreads_default()
    rows = B                          # the oracle's work unit is one (row, query): one row per thread
    sub = dict(ref)
    sub["batch"] = rows
    paged = bool(ref.get("page_blocks"))
    for f in ("seq_len", "nope", "rope", "kv_scale", "idx_code", "idx_scale", "ring_kv",
              "ring_gate", "ring_ikey", "ring_igate", "page_table"):
        if f not in ref:
            continue
        if paged and f in ("nope", "rope", "kv_scale", "idx_code", "idx_scale"):
            sub[f] = ref[f].copy()                                  # the page pool, whole
        else:
            sub[f] = np.ascontiguousarray(ref[f][:rows]).copy()      # the oracle appends in place
    scale = np.float32(1.0 / np.sqrt(512.0))
    t0 = time.perf_counter()
    oracle.compress_append(sub, tokens["kv"][:rows], tokens["gate"][:rows],
                           tokens["ikey"][:rows] if csa else None,
                           tokens["igate"][:rows] if csa else None)
    if csa:
        topk = oracle.indexer_topk(sub, Q["iq"][:rows], Q["iw"][:rows], k, nthreads=nthreads)
        oracle.csa_attend(sub, Q["q"][:rows], topk, scale, nthreads=nthreads)
    else:
        oracle.hca_attend(sub, Q["q"][:rows], scale, nthreads=nthreads)
    dt = time.perf_counter() - t0
    return dict(value=rows / dt, unit="queries/s", cores=min(nthreads, rows), kind="oracle",
                sample=f"one decode step (compress_append + "
                       f"{'indexer_topk + csa_attend' if csa else 'hca_attend'}) for all {rows} rows "
                       f"at full context, {dt:.2f}s wall, {min(nthreads, rows)} threads (the job's "
                       f"CPU share: affinity capped by OMP_NUM_THREADS)")


def counter_traffic(dominant, workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE / WRITE_SIZE scaled by a plain copy), or None when the
    summary is missing or the kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_counters_{dominant}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        nbytes = int(fields["traffic_bytes_per_launch"])
        src_name, src_hash = fields["traffic_source"].split()
    except (KeyError, ValueError):
        return None
    src = os.path.join(ROOT, "long_context_compressed_append_amd", "csrc", src_name)
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != src_hash:
        return None
    return nbytes


def valu_bound_us(workload):
    """The scoring kernel's VALU issue bound (us) from the committed SQ
    counter summary, or None when it is missing or the kernel source changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"sq_counters_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        bound = float(fields["valu_bound_us"])
        src_name, src_hash = fields["valu_source"].split()
    except (KeyError, ValueError):
        return None
    src = os.path.join(ROOT, "long_context_compressed_append_amd", "csrc", src_name)
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != src_hash:
        return None
    return bound


def interleaved_bytes(B, ctx, H_c, HI, k, H_h, W):
    """Algorithmic bytes of one layer pair (per the per-row figures above)."""
    nc, nh = ctx // 4, ctx // 128
    csa = B * (nc * 34 + HI * 260 + 2 * k * 4 + min(k, nc) * 604 + W * 1024 + H_c * 1024 + H_c * 2048)
    hca = B * (nh * 604 + W * 1024 + H_h * 1024 + H_h * 2048)
    return csa, hca


def prefill_score_flops(prior, n, m, HI):
    """Scoring work of a chunk: every visible (query, block) pair, H_I heads x
    64-d dot products (2 flops per multiply-add)."""
    pairs = sum((prior + i + 1) // m for i in range(n))
    return pairs * HI * 64 * 2, pairs


def prefill_attend_flops(prior, n, m, H, k, W):
    """Attention work of a chunk: per query, every attended key (the listed
    blocks that are visible, then the window) costs H heads x (512-d q.k +
    512-d p.v), 2 flops per multiply-add."""
    keys = sum(min(k, (prior + i + 1) // m) + min(W, prior + i + 1) for i in range(n))
    return keys * H * 2 * 512 * 2


def run_prefill(args):
    import torch
    import long_context_compressed_append_amd as lca
    from synth import layers as SL

    prior, n, m, H, HI, k, W, R = PREFILL[args.workload]
    csa = HI > 0
    seed, tag = 1004, "prefill"
    t = time.time()
    ref = SL.make_layer(seed, tag, 1, m, W, R, int(csa), (prior + n) // m + 64, [prior])
    tok = SL.tokens(seed, "chunk", 1, n, int(csa))
    Q = SL.queries(seed, tag, 1, n, H, HI)
    log(f"host image built in {time.time() - t:.1f}s")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    lay = lca.Layer.from_host(ref, device=dev)
    d_tok = {kk: up(v) for kk, v in tok.items()}
    q = up(Q["q"])
    iq, iw = (up(Q["iq"]), up(Q["iw"])) if csa else (None, None)
    topk = torch.empty((1, n, max(k, 1)), dtype=torch.int32, device=dev)
    out = torch.empty((1, n, H, 512), dtype=torch.float32, device=dev)
    scale = float(1.0 / np.sqrt(512.0))

    def reset():                      # back to the prior context (outside the timed kernels)
        lay.seq_len.fill_(prior)
        lay.len_min = lay.len_max = prior

    def step():
        if csa:
            lca.compress_append(lay, d_tok["kv"], d_tok["gate"], d_tok["ikey"], d_tok["igate"])
            lca.indexer_topk(lay, iq, iw, k, out=topk)
            lca.csa_attend(lay, q, topk, scale, out=out)
        else:
            lca.compress_append(lay, d_tok["kv"], d_tok["gate"])
            lca.hca_attend(lay, q, scale, out=out)

    for _ in range(args.warmup):
        reset()
        step()
    torch.cuda.synchronize()
    # whole steps between HIP events on the stream the library launches on
    # (torch's current stream), then each kernel alone (every launch
    # bracketed by events) over further steps
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(args.steps):
        reset()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    ms_per_step = float(np.median(times))
    kernels, spreads = {}, {}
    for name in ("compress", "indexer_score", "topk_select", "attend", "attend_combine"):
        with lca.KernelTimer(name) as kt:
            for _ in range(max(1, args.steps // 2)):
                reset()
                step()
            torch.cuda.synchronize()
        if kt.launches:
            kernels[name] = round(kt.total_ms * 1e3 / kt.launches, 1)
            spreads[name] = spread_us(kt.durations_ms)
    flops, pairs = prefill_score_flops(prior, n, m, HI)
    score_us = kernels.get("indexer_score", 0.0)
    tflops = flops / (score_us * 1e-6) / 1e12 if score_us else 0.0
    # HCA attends to every visible block: a list longer than any row
    att_flops = prefill_attend_flops(prior, n, m, H, k if csa else (prior + n) // m + 1, W)
    att_us = kernels.get("attend", 0.0)
    att_tflops = att_flops / (att_us * 1e-6) / 1e12 if att_us else 0.0
    if csa:
        # the roofline object covers the scoring, the prefill target (FP4
        # operands, priced at the FP8 rate); the attention, the longer kernel
        # here, is reported beside it against the fp16 peak
        roof = {"kernel": "indexer_score", "bound": "mfma", "achieved": round(tflops, 1),
                "peak": FP8_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / FP8_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                "kernel_avg_us": score_us, "kernel_us": spreads.get("indexer_score"),
                "flops_per_launch": flops}
        vb = valu_bound_us(args.workload)
        roof["valu_bound_us"] = vb          # the exact epilogue's VALU issue time (SQ counters)
        roof["frac_of_valu_bound"] = round(vb / score_us, 4) if vb and score_us else None
    else:
        roof = {"kernel": "attend", "bound": "mfma", "achieved": round(att_tflops, 1),
                "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(att_tflops / FP16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                "kernel_avg_us": att_us, "kernel_us": spreads.get("attend"),
                "flops_per_launch": att_flops}
    cpu = None
    if not args.no_cpu_baseline:
        try:
            cpu = prefill_cpu_baseline(ref, tok, Q, prior, n, m, k, csa)
        except Exception as e:  # report, never hide
            cpu = dict(error=repr(e))
    res = {
        "metric": METRIC,
        "value": round(n / (ms_per_step / 1e3), 1),
        "unit": ("queries/s (prefill chunk tokens through compress + indexer + top-k + attention)" if csa
                 else "queries/s (prefill chunk tokens through compress + dense attention)"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp4 scoring (exact fp32 scores); fp8/bf16 storage; bf16/fp16 MFMA attention" if csa
                  else "fp8/bf16 storage; bf16/fp16 MFMA attention"),
        "data": "synthetic (seeded cache image of the prior context, N(0,1) chunk)",
        "config": {
            "workload": args.workload, "batch": 1, "prior_tokens": prior, "chunk": n, "ratio": m,
            "heads": H, "indexer_heads": HI, "topk": k, "window": W, "ring": R,
            "kernel_us": kernels,
            **({"score_visible_pairs": pairs,
                "score_flops": flops,
                "score_fp4_peak_frac": round(tflops / FP4_MFMA_PEAK_TFLOPS, 4),
                "score_fp8_rate_frac": round(tflops / FP8_MFMA_PEAK_TFLOPS, 4)} if csa else {}),
            "attend_flops": att_flops,
            "attend_tflops": round(att_tflops, 1),
            "attend_fp16_peak_frac": round(att_tflops / FP16_MFMA_PEAK_TFLOPS, 4),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    emit(res, args)


def prefill_cpu_baseline(ref, tok, Q, prior, n, m, k, csa=True):
    """The oracle on a sample of the chunk: the whole compress_append, then
    indexer_topk and csa_attend (HCA: hca_attend) for 4 of the chunk's queries
    (each on a view whose length ends at that query)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    nthreads = oracle.nthreads_default()
    scale = np.float32(1.0 / np.sqrt(512.0))
    V = oracle.row_view(ref, 0)
    t0 = time.perf_counter()
    if csa:
        oracle.compress_append(V, tok["kv"], tok["gate"], tok["ikey"], tok["igate"])
    else:
        oracle.compress_append(V, tok["kv"], tok["gate"])
    t_comp = time.perf_counter() - t0
    # one query per oracle call (each on a view whose length ends at that
    # query), the calls spread over the job's threads
    n_s = max(16, nthreads)
    sample = [int(i * (n - 1) / (n_s - 1)) for i in range(n_s)]

    def one(qi):
        Vq = dict(V)
        Vq["seq_len"] = np.array([prior + qi + 1], np.int32)
        if csa:
            tk = oracle.indexer_topk(Vq, Q["iq"][:, qi:qi + 1], Q["iw"][:, qi:qi + 1], k, nthreads=1)
            oracle.csa_attend(Vq, Q["q"][:, qi:qi + 1], tk, scale, nthreads=1)
        else:
            oracle.hca_attend(Vq, Q["q"][:, qi:qi + 1], scale, nthreads=1)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=nthreads) as pool:
        list(pool.map(one, sample))
    t_q = (time.perf_counter() - t0) / len(sample)      # per query, all threads busy
    per_chunk = t_comp + t_q * n
    return dict(value=n / per_chunk, unit="queries/s", cores=nthreads, kind="oracle",
                sample=f"compress_append of the {n}-token chunk ({t_comp:.2f}s) plus "
                       f"{'indexer_topk + csa_attend' if csa else 'hca_attend'} for {len(sample)} of its "
                       f"queries spread over {nthreads} threads ({t_q:.3f}s per query), scaled to the "
                       f"chunk")


def run_interleaved(args):
    import torch
    import long_context_compressed_append_amd as lca
    from synth import layers as SL

    B, ctx, P, H_c, HI, k, H_h, W, needles, n_out = INTERLEAVED[args.workload]
    seed = 1005
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t = time.time()
    n_set = 1 if needles else 4       # needles target one query set
    # one host image per layer kind (with its outlier channels), copied to
    # every layer of that kind; from then on the layers diverge by their tokens
    images, chans = {}, {}
    qc_host = [SL.queries(seed, "csaq", B, 1, H_c, HI, step=s) for s in range(n_set)]
    # tokens appended after the image: warm-up, eager and graph timing, kernel timing
    extra = args.warmup + 2 * min(args.steps, 128) + 64
    for kind, m, has_idx in (("csa", 4, 1), ("hca", 128, 0)):
        ref = SL.make_layer(seed, kind, B, m, W, 256, has_idx, (ctx + extra) // m + 64, [ctx - 1] * B)
        chans[kind] = SL.outlier_channels(seed, kind, 0, n_out) if n_out else None
        if n_out:
            SL.apply_outliers(ref, chans[kind])
        if needles and kind == "csa":
            for b in range(B):
                SL.plant_needles(ref, seed, kind, b, needles, qc_host[0]["iq"][b, 0], qc_host[0]["iw"][b, 0],
                                 qc_host[0]["q"][b, 0])
        images[kind] = ref
    log(f"host images built in {time.time() - t:.1f}s")

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    layers = {"csa": [], "hca": []}
    for kind in ("csa", "hca"):
        base = lca.Layer.from_host(images[kind], device=dev)
        layers[kind].append(base)
        for _ in range(P - 1):
            lay = lca.Layer(base.batch, base.ratio, base.window, base.ring, base.has_indexer,
                            base.max_blocks, device=dev, pos_bias=images[kind]["pos_bias"],
                            ipos_bias=images[kind].get("ipos_bias"))
            for f in lca.Layer.PLANES:
                src = getattr(base, f)
                if src is not None:
                    getattr(lay, f).copy_(src)
            lay.len_min, lay.len_max = base.len_min, base.len_max
            layers[kind].append(lay)
    all_layers = layers["csa"] + layers["hca"]
    torch.cuda.synchronize()
    log(f"{2 * P} device layers ready in {time.time() - t:.1f}s")

    def host_tokens(kind, l, s):
        tk = SL.tokens(seed, f"{kind}{l}", B, 1, kind == "csa", step=s)
        return SL.outlier_tokens(tk, chans[kind]) if n_out else tk

    toks = {kind: [[{kk: up(v) for kk, v in host_tokens(kind, l, s).items()} for s in range(n_set)]
                   for l in range(P)] for kind in ("csa", "hca")}
    qs = {"csa": [up(x["q"]) for x in qc_host],
          "hca": [up(SL.queries(seed, "hcaq", B, 1, H_h, step=s)["q"]) for s in range(n_set)]}
    iq = [(up(x["iq"]), up(x["iw"])) for x in qc_host]
    topk = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    out_c = torch.empty((B, 1, H_c, 512), dtype=torch.float32, device=dev)
    out_h = torch.empty((B, 1, H_h, 512), dtype=torch.float32, device=dev)
    # the graph's inputs: fixed buffers, filled from the rotating sets
    g_tok = {kind: [{kk: v.clone() for kk, v in toks[kind][l][0].items()} for l in range(P)]
             for kind in ("csa", "hca")}
    g_q = {"csa": qs["csa"][0].clone(), "hca": qs["hca"][0].clone()}
    g_iq = (iq[0][0].clone(), iq[0][1].clone())

    def step_with(tc_of, th_of, qc, qh, iqw, plan_len=None):
        for l in range(P):
            c, h = layers["csa"][l], layers["hca"][l]
            tc, th = tc_of(l), th_of(l)
            if plan_len is not None:          # the selection plans for the length after the token
                c.len_max = plan_len - 1
            lca.decode_append_topk(c, tc["kv"], tc["gate"], tc["ikey"], tc["igate"], iqw[0], iqw[1], k, out=topk)
            lca.csa_attend(c, qc, topk, out=out_c)
            lca.compress_append(h, th["kv"], th["gate"])
            if plan_len is not None:
                h.len_max = plan_len
            lca.hca_attend(h, qh, out=out_h)

    def step(s):
        j = s % n_set
        step_with(lambda l: toks["csa"][l][j], lambda l: toks["hca"][l][j], qs["csa"][j], qs["hca"][j], iq[j])

    def fill_graph_inputs(s):
        j = s % n_set
        for kind in ("csa", "hca"):
            for l in range(P):
                for kk, v in toks[kind][l][j].items():
                    g_tok[kind][l][kk].copy_(v)
        g_q["csa"].copy_(qs["csa"][j])
        g_q["hca"].copy_(qs["hca"][j])
        g_iq[0].copy_(iq[j][0])
        g_iq[1].copy_(iq[j][1])

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    done = args.warmup
    stream = torch.cuda.current_stream()
    # eager: one step at a time between HIP events (per-step latency); the HCA
    # layers finalise a block on the first step after every 128th token
    nsteps = min(args.steps, 128)

    def timed(run_one, first, prep=None):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nsteps)]
        t0 = time.perf_counter()
        for i in range(nsteps):
            if prep is not None:          # outside the events: input copies of a graph replay
                prep(first + i)
            ev[i][0].record(stream)
            run_one(first + i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return np.array([a.elapsed_time(b) for a, b in ev]), wall

    eager_times, eager_wall = timed(step, done)
    done += nsteps
    graph_times = None
    if not args.eager:
        final_len = max(x.len_max for x in all_layers) + nsteps + 2
        saved = [(x.len_min, x.len_max) for x in all_layers]
        for x in all_layers:                  # workspaces sized for the planned lengths before capture
            x.len_max = final_len
        for c in layers["csa"]:
            c.indexer_workspace(1, lca.indexer_workspace_bytes(c, 1, HI, k))
            c.workspace(lca.attend_workspace_bytes(c, 1, H_c, k), "attend")
        for h in layers["hca"]:
            h.workspace(lca.attend_workspace_bytes(h, 1, H_h, 0), "attend")
        for x, (a, b) in zip(all_layers, saved):
            x.len_min, x.len_max = a, b
        fill_graph_inputs(done)
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step_with(lambda l: g_tok["csa"][l], lambda l: g_tok["hca"][l], g_q["csa"], g_q["hca"], g_iq,
                      plan_len=final_len)
        torch.cuda.synchronize()
        for x, (a, b) in zip(all_layers, saved):      # capture ran nothing on the device
            x.len_min, x.len_max = a, b

        graph_times, graph_wall = timed(lambda s: g.replay(), done, prep=fill_graph_inputs)
        for x in all_layers:
            x.len_min += nsteps
            x.len_max += nsteps
        done += nsteps
        del g
    # the dominant kernel (CSA indexer score) alone, HIP events around its launches
    with lca.KernelTimer("indexer_score") as kt:
        for i in range(max(1, 32 // P)):
            step(done + i)
        torch.cuda.synchronize()
    kernel_ms = kt.total_ms / max(1, kt.launches)
    csa_b, hca_b = interleaved_bytes(B, ctx, H_c, HI, k, H_h, W)
    times = graph_times if graph_times is not None else eager_times
    step_ms = float(times.mean())
    dom_bytes = B * ((ctx // 4) * 34 + HI * 260)
    achieved = dom_bytes / (kernel_ms / 1e3) / 1e9 if kernel_ms > 0 else 0.0

    def lat(ts):
        if ts is None:
            return None
        return {"step_ms_mean": round(float(ts.mean()), 4), "step_ms_p50": round(float(np.median(ts)), 4),
                "step_ms_p90": round(float(np.percentile(ts, 90)), 4), "step_ms_max": round(float(ts.max()), 4),
                "pair_us_mean": round(float(ts.mean()) * 1e3 / P, 2)}

    cpu = None
    if not args.no_cpu_baseline:
        try:
            cpu = interleaved_cpu_baseline(images, qc_host[0], SL.queries(seed, "hcaq", B, 1, H_h, step=0),
                                           {kind: host_tokens(kind, 0, 0) for kind in ("csa", "hca")}, k, P)
        except Exception as e:  # report, never hide
            cpu = dict(error=repr(e))
    res = {
        "metric": METRIC,
        "value": round(B / (step_ms / 1e3), 1),
        "unit": "tokens/s (one token per row through every layer)",
        "n_gpus": 1, "steps": nsteps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4/fp8 storage; fp32 scores; bf16/fp16 MFMA with fp32 accumulate",
        "data": ("synthetic (seeded cache images"
                 + (f", {n_out} outlier channels x20 per layer kind" if n_out else "")
                 + (f", {needles} needle blocks per row" if needles else "") + ")"),
        "config": {
            "workload": args.workload, "batch": B, "context": ctx, "layer_pairs": P,
            "csa": {"heads": H_c, "indexer_heads": HI, "topk": k, "ratio": 4},
            "hca": {"heads": H_h, "ratio": 128}, "window": W,
            "launch": "hip_graph" if graph_times is not None else "eager",
            "eager": lat(eager_times), "graph": lat(graph_times),
            "step_algorithmic_bytes": P * (csa_b + hca_b),
            "step_hbm_gbs": round(P * (csa_b + hca_b) / (step_ms / 1e3) / 1e9, 1),
            "eager_wall_ms_per_step": round(eager_wall * 1e3 / nsteps, 4),
        },
        "roofline": {
            "kernel": "indexer_score", "bound": "hbm", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None, "kernel_avg_us": round(kernel_ms * 1e3, 3),
            "kernel_us": spread_us(kt.durations_ms), "bytes_per_launch": dom_bytes,
        },
        "cpu_baseline": cpu,
    }
    emit(res, args)


def interleaved_cpu_baseline(images, qc, qh, tok, k, P):
    """The oracle on one layer pair of one step for every row (a CSA layer:
    compress_append, indexer_topk, csa_attend; an HCA layer: compress_append,
    hca_attend), scaled to the P pairs a token goes through."""
    import oracle
    nthreads = oracle.nthreads_default()
    scale = np.float32(1.0 / np.sqrt(512.0))
    views = {}
    for kind, ref in images.items():
        v = dict(ref)
        for f in ("seq_len", "nope", "rope", "kv_scale", "idx_code", "idx_scale", "ring_kv", "ring_gate",
                  "ring_ikey", "ring_igate"):
            v[f] = ref[f].copy()                       # the oracle appends in place
        views[kind] = v
    B = int(views["csa"]["batch"])
    tc, th = tok["csa"], tok["hca"]
    reps = 0
    t0 = time.perf_counter()
    # repeated steps (one more token each) until about 2 s of work, for short ones
    while reps < 64 and (reps == 0 or time.perf_counter() - t0 < 2.0):
        oracle.compress_append(views["csa"], tc["kv"], tc["gate"], tc["ikey"], tc["igate"])
        tk = oracle.indexer_topk(views["csa"], qc["iq"], qc["iw"], k, nthreads=nthreads)
        oracle.csa_attend(views["csa"], qc["q"], tk, scale, nthreads=nthreads)
        oracle.compress_append(views["hca"], th["kv"], th["gate"])
        oracle.hca_attend(views["hca"], qh["q"], scale, nthreads=nthreads)
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    return dict(value=B / (dt * P), unit="tokens/s", cores=min(nthreads, B), kind="oracle",
                sample=f"one layer pair of one step for all {B} rows ({dt:.4f}s wall per step over "
                       f"{reps} steps, {min(nthreads, B)} threads), scaled to {P} pairs per token")


def calibrate_copy(mib):
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give the
    factor between the counters and the bytes a kernel really moves."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="csa_decode_128k",
                    choices=sorted(WORKLOADS) + sorted(INTERLEAVED) + sorted(PREFILL))
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-ceiling microbenchmarks")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--paged", type=int, default=0, metavar="PB",
                    help="decode workloads: keep the compressed entries in a shared pool of pages of PB "
                         "blocks (rows map their pages in a seeded random order)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (the "
                         "reference kernel for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: there is no multi-GPU path (decode rows would shard "
              "across GPUs with no exchange).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    args.peaks = None
    if not args.no_peaks:
        import torch
        torch.cuda.set_device(0)
        args.peaks = measure_peaks()
        log("measured ceilings", args.peaks)

    if args.workload in INTERLEAVED:
        return run_interleaved(args)
    if args.workload in PREFILL:
        if args.steps == 200 and args.warmup == 16:     # defaults sized for decode steps
            args.steps, args.warmup = 12, 2
        return run_prefill(args)

    import torch
    import long_context_compressed_append_amd as lca
    from synth import layers as SL

    wl = WORKLOADS[args.workload]
    csa, B, ctx, m, H, HI, k, needles, W = wl
    seed = 1001 if csa else 1002
    NL = args.layers
    n_eager = 4 * NL                                     # eager pass timing the dominant kernel
    total_steps = args.warmup + args.steps + n_eager
    ref, Q = build_host_layer(wl, seed)
    if args.paged:                        # the same entries in a page pool; pages for every append to come
        grow_blocks = (total_steps + NL - 1) // NL // m + 2
        mb = (ref["max_blocks"] + args.paged - 1) // args.paged * args.paged
        if mb != ref["max_blocks"]:
            for f in ("nope", "rope", "kv_scale", "idx_code", "idx_scale"):
                pad = np.zeros((B, mb - ref["max_blocks"]) + ref[f].shape[2:], ref[f].dtype)
                ref[f] = np.concatenate([ref[f], pad], axis=1) if ref[f].shape[1] else ref[f][:, :0]
            ref["max_blocks"] = mb
        ref = SL.paginate(ref, seed, args.paged, reserve_blocks=grow_blocks)
    # tokens: a few distinct sets, rotated
    n_tok = 8
    toks = [SL.tokens(seed, "step", B, 1, int(csa), step=s) for s in range(n_tok)]
    qs = [SL.queries(seed, "stepq", B, 1, H, HI, step=s) for s in range(n_tok)]

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    t = time.time()
    layers = []
    base = lca.Layer.from_host(ref, device=dev)
    for i in range(NL):
        if i == 0:
            lay = base
        else:
            lay = lca.Layer(B, m, W, ref["ring"], csa, ref["max_blocks"], device=dev,
                            pos_bias=ref["pos_bias"], ipos_bias=ref.get("ipos_bias"),
                            page_blocks=base.page_blocks, pool_pages=base.pool_pages)
            for f in base.planes:
                src = getattr(base, f)
                if src is not None:
                    getattr(lay, f).copy_(src)
            lay.len_min, lay.len_max = base.len_min, base.len_max
        layers.append(lay)
    # every layer gets at most ceil(total_steps / NL) appends: size the plans for that
    grow = (total_steps + NL - 1) // NL + 1
    for lay in layers:
        assert (lay.len_max + grow) // m <= lay.max_blocks
    torch.cuda.synchronize()
    log(f"{NL} device layers ready in {time.time() - t:.1f}s "
        f"({sum(x.nope.numel() for x in layers) / 1e9:.2f} GB of FP8 codes)")

    d_tok = [{kk: up(v) for kk, v in tk.items()} for tk in toks]
    d_q = [{kk: up(v) for kk, v in qq.items()} for qq in qs]
    topk_buf = torch.empty((B, 1, max(k, 1)), dtype=torch.int32, device=dev)
    out_buf = torch.empty((B, 1, H, 512), dtype=torch.float32, device=dev)

    def step(i, plan_len=None):
        lay = layers[i % NL]
        tk, qq = d_tok[i % n_tok], d_q[i % n_tok]
        if csa:
            # the append and the selection in one launch; under graph capture
            # the selection plans for the largest length reached
            if plan_len is not None:
                lay.len_max = plan_len - 1
            lca.decode_append_topk(lay, tk["kv"], tk["gate"], tk["ikey"], tk["igate"], qq["iq"], qq["iw"], k,
                                   out=topk_buf)
            lca.csa_attend(lay, qq["q"], topk_buf, out=out_buf)
        else:
            lca.compress_append(lay, tk["kv"], tk["gate"])
            if plan_len is not None:          # graph capture: plan for the largest length reached
                lay.len_max = plan_len
            lca.hca_attend(lay, qq["q"], out=out_buf)

    # warm-up (eager): allocates workspaces, loads code objects
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    done = args.warmup

    dominant = "indexer_score" if csa else "attend"
    # eager pass with the dominant kernel bracketed by HIP events
    t0 = time.perf_counter()
    with lca.KernelTimer(dominant) as kt:
        for i in range(done, done + n_eager):
            step(i)
        torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / n_eager
    done += n_eager
    kernel_ms = kt.total_ms / max(1, kt.launches)
    kernel_spread = spread_us(kt.durations_ms)

    # graph of NL steps (one per layer), replayed; plans sized for the final lengths
    graph_ms = None
    if not args.eager:
        reps = (args.steps + NL - 1) // NL
        final_len = max(x.len_max for x in layers) + reps + 2
        for lay in layers:
            assert (final_len + 1) // m <= lay.max_blocks
        lens_before = [(x.len_min, x.len_max) for x in layers]
        for lay in layers:       # size the workspaces for the planned lengths before capture
            lay.len_max = final_len
            if csa:
                lay.indexer_workspace(1, lca.indexer_workspace_bytes(lay, 1, HI, k))
            lay.workspace(lca.attend_workspace_bytes(lay, 1, H, k), "attend")
        for lay, (a, b) in zip(layers, lens_before):
            lay.len_min, lay.len_max = a, b
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(done, done + NL):
                step(i, plan_len=final_len)
        torch.cuda.synchronize()
        # capture does not execute: restore the host mirrors, then replay
        for lay, (a, b) in zip(layers, lens_before):
            lay.len_min, lay.len_max = a, b
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        steps_timed = reps * NL
        for lay in layers:
            lay.len_min += reps
            lay.len_max += reps
        graph_ms = elapsed * 1e3 / steps_timed
        ms_per_step = graph_ms
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(done, done + args.steps):
            step(i)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        steps_timed = args.steps
        ms_per_step = elapsed * 1e3 / steps_timed

    # final sanity: lengths on the device advanced as many steps as were run
    dev_len = int(layers[0].seq_len[0].item())
    log(f"layer 0 length {dev_len}, host mirror {layers[0].len_max}")

    value = B / (ms_per_step / 1e3)
    dom_bytes = dominant_bytes(wl)
    achieved = dom_bytes / (kernel_ms / 1e3) / 1e9 if kernel_ms > 0 else 0.0
    step_bytes = algorithmic_bytes(wl)
    cpu = None
    if not args.no_cpu_baseline:
        try:
            cpu = cpu_baseline(wl, ref, Q, toks[0])
        except Exception as e:  # report, never hide
            cpu = dict(error=repr(e))
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4/fp8 storage; fp32 scores; bf16/fp16 MFMA with fp32 accumulate",
        "data": "synthetic (seeded cache images, needle blocks)",
        "config": {
            "workload": args.workload,
            "batch": B, "context": ctx, "ratio": m, "heads": H, "indexer_heads": HI, "topk": k,
            "window": W, "layers_rotated": NL, "launch": "eager" if args.eager else "hip_graph",
            "page_blocks": args.paged or None,
            "eager_ms_per_step": round(eager_ms, 4),
            "graph_ms_per_step": round(graph_ms, 5) if graph_ms else None,
            "step_algorithmic_bytes": step_bytes,
            "step_hbm_gbs": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
            "step_hbm_frac": round(step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "kernel": dominant,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": counter_traffic(dominant, args.workload),
            "kernel_avg_us": round(kernel_ms * 1e3, 3),
            "kernel_us": kernel_spread,
            "bytes_per_launch": dom_bytes,
        },
        "cpu_baseline": cpu,
    }
    emit(res, args)


if __name__ == "__main__":
    main()
