"""Benchmark of causal block-sparse prefill attention on one MI355X.

One step = one call of the C-ABI entry point ``bsp_attn_fwd`` over the whole
workload (all query heads, all causal (tile, block) pairs): the Llama-3.1-8B
shaped attention layer at 32768 tokens (32 query heads, 8 KV heads,
head_dim 128, bf16, block_q = block_k = 128) by default. The timed step runs
at lambda = +inf (dense mode, where every visited block is kept); the same
workload is then timed at its finite lambdas to report the skip fraction and
the speed-up over the kernel's own dense mode.

Prints one JSON line. Inputs are synthetic (seeded AR(1) latents with sink
and vertical keys) and resident in HBM before timing starts.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}  # MI355X dense MFMA (fp32: matrix/vector)
HBM_GBS = 8000.0


def pair_counts(seqlens, bq, bk):
    """Visited (tile, block) pairs of one head under the causal mask."""
    n = 0
    for L in seqlens:
        for t in range((L + bq - 1) // bq):
            r1 = min(L, (t + 1) * bq)
            n += (r1 - 1) // bk + 1
    return n


def dense_causal_flops(seqlens, H, D):
    return sum(4.0 * D * H * L * (L + 1) / 2 for L in seqlens)


def measured_traffic(workload, dtype, dense):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary of this workload, if it was measured on the current kernel source
    (else None). The figure is replayed from that summary, not measured by
    this run (rocprofv3 counters need a run of their own)."""
    import hashlib

    import re

    short = re.sub(r"_(bf16|fp8|fp32)$", "", workload)
    path = os.path.join(ROOT, "profiles", "fwd_mfma_%s_%s_dense_hbm_bytes.json" % (dtype, short))
    if not dense or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "block_sparse_long_bsp_amd", "csrc", "bsp_attn.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("workload") != workload or rec.get("dtype") != dtype or rec.get("kernel_source_sha256") != sha:
        return None
    return float(rec["traffic_bytes_per_launch"])


def time_calls(fn, steps, warmup):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per call


def time_interleaved(fns, rounds, segment_ms=10.0, warmup_s=0.25):
    """Mean call time of each callable in ``fns`` (a dict), taken in turns.

    After a warm-up of at least ``warmup_s`` seconds of calls of all of them,
    each round times one segment of back-to-back calls of every callable
    (about ``segment_ms`` long; the order alternates between rounds), so that
    clock and temperature drift reach all of them alike. Returns the median
    over the rounds of each callable's per-call time (ms), and the calls per
    segment."""
    import statistics

    import torch

    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    while True:
        for fn in fns.values():
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= warmup_s:
            break

    def segment(fn, n):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / n

    est = min(segment(fn, 1) for fn in fns.values())
    calls = max(1, int(round(segment_ms / max(est, 1e-3))))
    times = {key: [] for key in fns}
    keys = list(fns)
    for r in range(max(1, rounds)):
        for key in (keys if r % 2 == 0 else keys[::-1]):
            times[key].append(segment(fns[key], calls))
    return {key: statistics.median(v) for key, v in times.items()}, calls


def time_each(fn, steps, flush=None):
    """Median of per-call event timings; with ``flush`` (a callable writing a
    buffer larger than the last-level cache) run between calls, outside the
    timed events."""
    import torch

    stream = torch.cuda.current_stream()
    out = []
    for _ in range(steps):
        if flush is not None:
            flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        out.append(a.elapsed_time(b))
    return float(np.median(out))


def decode_rows(bsp, w, q, k, v, scales, dense_lam, finite, steps):
    """Decoding steps (bsp_attn_decode) after the workload's single sequence: one
    context at the workload's lambdas (its own keys), and a batch of 16 contexts
    of the same length on distinct pages of random data at lambda = +inf."""
    import torch

    H, D = w.n_heads_q, w.head_dim
    L = int(q.shape[0])
    # ---- decoding steps (bsp_attn_decode): one new query row per sequence.
    # Algorithmic HBM bytes: K of every key, V of the blocks some query head of
    # the KV group keeps (here: of every block for lambda = +inf).
    dec = []
    es = k.element_size()
    kv_row_bytes = w.n_heads_kv * D * es
    cu1 = torch.tensor([0, L], dtype=torch.int32, device="cuda")
    q1 = q[L - 1:].contiguous()
    ws1 = torch.empty(bsp.decode_workspace_bytes(H, w.n_heads_kv, 1, L, L, D, w.block_k), dtype=torch.uint8,
                      device="cuda")
    sc1 = torch.empty(H, dtype=torch.int64, device="cuda")
    vc1 = torch.empty(H, dtype=torch.int64, device="cuda")
    for lam in [dense_lam] + [x for x in (5.3,) if finite] + finite[-1:]:
        def fn(lam=lam):
            return bsp.decode(q1, k, v, cu1, L, block_k=w.block_k, lam=lam, q_scale=scales[0],
                              k_scale=scales[1], v_scale=scales[2], want_bitmap=False, skip_count=sc1,
                              visited_count=vc1, workspace=ws1)
        ms_d = time_calls(fn, steps * 5, 5)
        f = int(sc1.sum().item()) / max(1, int(vc1.sum().item()))
        byts = L * kv_row_bytes * (2.0 - f)  # V skipped only where every head of a group skips: an upper bound
        dec.append({"batch": 1, "lk": L, "lambda": lam, "ms": ms_d, "tokens_per_s": 1.0 / (ms_d * 1e-3),
                    "skip_fraction": f, "kv_gbs_upper": byts / (ms_d * 1e-3) / 1e9})
    # a batch of 16 contexts of the same length, distinct pages of random data (lambda = +inf)
    B, page = 16, 64
    n_pages = B * L // page
    kp = torch.randn((n_pages, page, w.n_heads_kv, D), device="cuda").to(k.dtype)
    vp = torch.randn((n_pages, page, w.n_heads_kv, D), device="cuda").to(k.dtype)
    table = torch.randperm(n_pages, device="cuda", dtype=torch.int64).to(torch.int32).view(B, L // page).contiguous()
    cuB = torch.arange(0, (B + 1) * L, L, dtype=torch.int32, device="cuda")
    qB = torch.randn((B, H, D), device="cuda").to(q.dtype)
    wsB = torch.empty(bsp.decode_workspace_bytes(H, w.n_heads_kv, B, B * L, L, D, w.block_k), dtype=torch.uint8,
                      device="cuda")

    def fnB():
        return bsp.decode(qB, kp, vp, cuB, L, total_k=B * L, block_table=table, block_k=w.block_k, lam=dense_lam,
                          q_scale=scales[0], k_scale=scales[1], v_scale=scales[2], want_bitmap=False,
                          workspace=wsB)
    ms_b = time_calls(fnB, steps * 2, 3)
    byts = B * L * kv_row_bytes * 2.0
    dec.append({"batch": B, "lk": L, "lambda": dense_lam, "paged": page, "ms": ms_b, "tokens_per_s": B / (ms_b * 1e-3),
                "skip_fraction": 0.0, "kv_gbs": byts / (ms_b * 1e-3) / 1e9,
                "hbm_frac": byts / (ms_b * 1e-3) / 1e9 / HBM_GBS, "data": "random normal (timing only)"})
    del kp, vp, wsB
    return dec


def cpu_baseline(inp, w, lam, target_s=15.0):
    """Time the CPU oracle on a bounded, deterministic sample of the workload
    and scale its rate to the whole job by visited (tile, block) pairs. The
    sample is every n-th query tile (plus the first and last) of query head 0
    or, when all tiles of one head take less than target_s, every tile of the
    first few heads (spread over the KV heads). Its size comes from a
    calibration run of the same oracle, on the same threads, over a smaller
    sample, so that the timed sample takes about target_s seconds."""
    import oracle
    import synth

    nproc = os.cpu_count() or 1
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else nproc
    # on a shared multi-GPU host one GPU's job gets a share of 16 host cores, whatever nproc shows
    threads = int(os.environ.get("BSP_ORACLE_THREADS", "0")) or min(16, avail)
    L = inp.seqlens
    H, G = w.n_heads_q, w.n_heads_q // w.n_heads_kv
    head_order = [g + G * i for g in range(G) for i in range(H // G)]  # one head per KV head first

    def sample(heads, stride):
        work = synth.work_items(L, H, w.block_q, heads=heads, tile_stride=stride)
        pairs = sum(((min(L[s], (t + 1) * w.block_q) - 1) // w.block_k + 1) for s, _, t in work)
        return work, pairs

    n_tiles = sum((x + w.block_q - 1) // w.block_q for x in L)
    _, pairs_h0 = sample([0], 1)
    # calibration: about 2 tiles per thread, spread over the sequence
    cal_work, cal_pairs = sample([0], max(1, n_tiles // (2 * threads)))
    oracle.run_inputs(inp, w.block_q, w.block_k, lam, work=cal_work[:1], n_threads=1)  # first touch of the inputs
    t0 = time.perf_counter()
    oracle.run_inputs(inp, w.block_q, w.block_k, lam, work=cal_work, n_threads=threads)
    t_cal = time.perf_counter() - t0
    want = cal_pairs / max(t_cal, 1e-6) * target_s  # pairs that take about target_s
    if want >= pairs_h0:
        heads, stride = head_order[:max(1, min(H, int(round(want / pairs_h0))))], 1
    else:
        heads, stride = [0], max(1, int(round(pairs_h0 / want)))
    work, pairs = sample(heads, stride)
    t0 = time.perf_counter()
    oracle.run_inputs(inp, w.block_q, w.block_k, lam, work=work, n_threads=threads)
    t_sample = time.perf_counter() - t0
    total_pairs = pair_counts(L, w.block_q, w.block_k) * H
    t_full = t_sample * total_pairs / pairs
    what = (f"query heads {heads}, every query tile" if stride == 1 else
            f"query head 0, every {stride}th query tile (+first/last)")
    return {
        "value": sum(L) / t_full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "sample": f"{what}: {work.shape[0]} (head, tile) items, {pairs} of {total_pairs} visited (tile, block) "
                  f"pairs, lambda={lam}; {t_sample:.1f} s wall, scaled to the whole job by pairs",
        "sample_seconds": round(t_sample, 2), "cpu_model": cpu_model(), "nproc": nproc, "affinity": avail,
        "threads": threads,
        "threads_note": ("BSP_ORACLE_THREADS" if os.environ.get("BSP_ORACLE_THREADS") else
                         "min(16, CPUs this process may run on): the host-core share of one GPU on a shared host"),
    }


def cpu_model():
    """Model name of the host CPU (from /proc/cpuinfo)."""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def mfma_probe(steps=3):
    """Measured matrix-core rate (TFLOP/s) of this GPU: the best of `steps`
    runs of the probe kernels in libbsp_mfma_peak.so (chains of independent
    bf16 / fp8 MFMAs on register operands, several waves per SIMD on every
    compute unit), timed with HIP events on the launch stream."""
    import ctypes

    import torch

    import block_sparse_long_bsp_amd.build as bld

    lib = ctypes.CDLL(bld.PROBE_LIB)
    lib.bsp_probe_mfma.restype = ctypes.c_int
    lib.bsp_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.bsp_probe_mfma_flops.restype = ctypes.c_double
    lib.bsp_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 8 * n_cu, 64
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for name, fp8 in (("bf16", 0), ("fp8", 1)):
        best = 0.0
        for i in range(steps + 1):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = lib.bsp_probe_mfma(fp8, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                                    ctypes.c_void_p(stream.cuda_stream))
            b.record(stream)
            b.synchronize()
            if rc != 0:
                raise RuntimeError(f"probe launch failed ({rc})")
            if i > 0:  # the first run warms up the clocks
                best = max(best, lib.bsp_probe_mfma_flops(fp8, blocks, iters) / (a.elapsed_time(b) * 1e-3) / 1e12)
        res[name] = best
    return {"bf16_tflops": res["bf16"], "fp8_tflops": res["fp8"], "datasheet_bf16_tflops": PEAK_TFLOPS["bf16"],
            "datasheet_fp8_tflops": PEAK_TFLOPS["fp8"], "compute_units": n_cu,
            "what": "chains of independent v_mfma_f32_32x32x16_bf16 / v_mfma_scale_f32_32x32x64_f8f6f4 on register "
                    "operands, 8 workgroups of 4 waves per compute unit; best of %d runs" % steps}


def workload_row(bsp, name, dtype, rounds):
    """Dense-mode and finite-lambda timings of another named workload (one
    call of the C ABI over the whole workload per step, the lambdas timed in
    turns over ``rounds`` rounds), with its skip fractions, executed TFLOP/s
    and roofline fraction."""
    import torch

    import synth

    w = synth.WORKLOADS[name]
    t0 = time.perf_counter()
    inp = synth.make_workload(name, dtype)
    gen_s = time.perf_counter() - t0

    def up(a):
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        if dtype == "fp8":
            return torch.from_numpy(a).cuda().view(torch.float8_e4m3fn)
        return torch.from_numpy(a).cuda()

    q = up(inp.q)
    k, v = (up(inp.k_pages), up(inp.v_pages)) if w.paged else (up(inp.k), up(inp.v))
    table = torch.from_numpy(inp.block_table).cuda() if w.paged else None
    cu = torch.from_numpy(inp.cu_seqlens).cuda()
    scales = [None if x is None else torch.from_numpy(x).cuda() for x in (inp.q_scale, inp.k_scale, inp.v_scale)]
    H, D = w.n_heads_q, w.head_dim
    T = inp.total_tokens
    o = torch.empty((T, H, D), dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    sc = torch.empty((H,), dtype=torch.int64, device="cuda")
    vc = torch.empty((H,), dtype=torch.int64, device="cuda")
    visited = pair_counts(inp.seqlens, w.block_q, w.block_k) * H
    unit = 2.0 * w.block_q * w.block_k * D
    max_len = inp.max_seqlen
    del inp

    def call(lam):
        return lambda: bsp.fwd(q, k, v, cu, max_len, block_table=table, block_q=w.block_q,
                               block_k=w.block_k, lam=lam, q_scale=scales[0], k_scale=scales[1], v_scale=scales[2],
                               out=o, lse=lse, want_bitmap=False, skip_count=sc, visited_count=vc)

    lams = [math.inf] + [x for x in w.lambdas if not math.isinf(x)]
    skipped = {}
    for lam in lams:  # one call each for the skip counts
        call(lam)()
        torch.cuda.synchronize()
        skipped[lam] = int(sc.sum().item())
    times, seg_calls = time_interleaved({lam: call(lam) for lam in lams}, rounds=rounds)
    rows = []
    dense_ms = None
    for lam in lams:
        ms = times[lam]
        kept = visited - skipped[lam]
        f = 1.0 - kept / visited
        ex = unit * (visited + kept)
        if dtype == "fp8":  # QK^T at the fp8 rate, PV at the bf16 rate
            peak = ex / (unit * visited / PEAK_TFLOPS["fp8"] + unit * kept / PEAK_TFLOPS["bf16"])
        else:
            peak = PEAK_TFLOPS[dtype]
        row = {"lambda": lam, "ms": ms, "tokens_per_s": T / (ms * 1e-3), "skip_fraction": f,
               "executed_tflops": ex / (ms * 1e-3) / 1e12, "roofline_frac": ex / (ms * 1e-3) / 1e12 / peak}
        if math.isinf(lam):
            dense_ms = ms
        else:
            row["speedup_vs_dense"] = dense_ms / ms
            row["flop_model_speedup"] = 1.0 / (1.0 - f / 2.0)
        rows.append(row)
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return {"workload": name, "dtype": dtype, "block_q": w.block_q, "block_k": w.block_k, "total_tokens": T,
            "paged": w.paged, "generation_s": round(gen_s, 1), "rows": rows,
            "timing": f"every lambda (dense included) timed in turns: median over {max(1, rounds)} rounds of "
                      f"{seg_calls}-call segments, after a 0.25 s warm-up of all of them"}


EXTRA_WORKLOADS = (("llama8b_8k_bf16", "bf16"), ("varlen16_paged_bf16", "bf16"), ("llama8b_128k", "bf16"),
                   ("llama8b_128k", "fp8"))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_32k_bf16")
    ap.add_argument("--dtype", default=None)
    ap.add_argument("--lambdas", default=None,
                    help="comma-separated finite lambdas to time instead of the workload's own (e.g. 8)")
    ap.add_argument("--sparse-steps", type=int, default=10,
                    help="rounds of the timing in turns of dense mode and the finite lambdas; 0 skips them")
    ap.add_argument("--extra-steps", type=int, default=10,
                    help="calls per extra measurement (median/flushed timing, chunk, decode), and rounds of the timing in "
                         "turns of the ablation switches and of the other workloads; 0 skips")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decoding steps (single-sequence workloads); for kernel traces")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="skip the rows of the other workloads (8K, varlen, 128K bf16 and fp8)")
    ap.add_argument("--no-mfma-probe", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size first (scales HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the block-sparse prefill path has no "
                                   "multi-GPU mode (--gpus must be 1)"}))
        sys.exit(2)

    import torch

    import block_sparse_long_bsp_amd as bsp
    import synth

    bsp.load_library()
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    dtype = args.dtype or w.dtypes[0]
    t0 = time.perf_counter()
    inp = synth.make_workload(w.name, dtype)
    gen_s = time.perf_counter() - t0
    print(f"# generated {w.name} ({dtype}) in {gen_s:.1f} s", file=sys.stderr, flush=True)

    def up(a):
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        if dtype == "fp8":
            return torch.from_numpy(a).cuda().view(torch.float8_e4m3fn)
        return torch.from_numpy(a).cuda()

    q = up(inp.q)
    if w.paged:
        k, v = up(inp.k_pages), up(inp.v_pages)
        table = torch.from_numpy(inp.block_table).cuda()
    else:
        k, v = up(inp.k), up(inp.v)
        table = None
    cu = torch.from_numpy(inp.cu_seqlens).cuda()
    scales = [None if s is None else torch.from_numpy(s).cuda() for s in (inp.q_scale, inp.k_scale, inp.v_scale)]
    H, D = w.n_heads_q, w.head_dim
    T_tok = inp.total_tokens
    o = torch.empty((T_tok, H, D), dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")
    lse = torch.empty((H, T_tok), dtype=torch.float32, device="cuda")
    words = bsp.skip_bitmap_words(H, len(inp.seqlens), inp.max_seqlen, w.block_q, w.block_k)
    bm = torch.empty((words,), dtype=torch.int32, device="cuda")
    sc = torch.empty((H,), dtype=torch.int64, device="cuda")
    vc = torch.empty((H,), dtype=torch.int64, device="cuda")

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def call(lam):
        return lambda: bsp.fwd(q, k, v, cu, inp.max_seqlen, block_table=table, block_q=w.block_q,
                               block_k=w.block_k, lam=lam, q_scale=scales[0], k_scale=scales[1],
                               v_scale=scales[2], out=o, lse=lse, bitmap=bm, skip_count=sc, visited_count=vc)

    lambdas = list(w.lambdas) if args.lambdas is None else [float(x) for x in args.lambdas.split(",")]
    dense_lam = math.inf
    visited = pair_counts(inp.seqlens, w.block_q, w.block_k) * H
    unit_flops = 2.0 * w.block_q * w.block_k * D
    dense_flops = dense_causal_flops(inp.seqlens, H, D)

    if args.decode_only:
        finite = [x for x in lambdas if not math.isinf(x)]
        print(json.dumps({"workload": w.name, "dtype": dtype,
                          "decode": decode_rows(bsp, w, q, k, v, scales, dense_lam, finite, max(1, args.extra_steps))}),
              flush=True)
        return

    # ---- timed step: dense mode (lambda = +inf)
    ms = time_calls(call(dense_lam), args.steps, args.warmup)
    kept = visited - int(sc.sum().item())
    assert int(vc.sum().item()) == visited, "visited count mismatch"
    exec_flops = unit_flops * (visited + kept)
    tokens_s = T_tok / (ms * 1e-3)
    exec_tflops = exec_flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic(w.name, dtype, True)
    traffic_src = (None if traffic is None else
                   "replayed from profiles/fwd_mfma_%s_%s_dense_hbm_bytes.json: rocprofv3 FETCH_SIZE and WRITE_SIZE "
                   "passes on the same kernel source (SHA-256 matches), each scaled by a plain-copy calibration; "
                   "not measured in this run" % (dtype, w.name.replace("_bf16", "").replace("_fp8", "")))
    # The fp8 kernel runs QK^T on the fp8 MFMA and PV on the bf16 MFMA: its
    # peak is the rate at which that mix of work can retire.
    if dtype == "fp8":
        qk, pv = unit_flops * visited, unit_flops * kept
        peak = (qk + pv) / (qk / PEAK_TFLOPS["fp8"] + pv / PEAK_TFLOPS["bf16"])
    else:
        peak = PEAK_TFLOPS[dtype]
    result = {
        "metric": "prefill tokens/s (+ executed TFLOP/s vs MFMA peak; skip fraction)",
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded AR(1) latents + sink/vertical keys)",
        "config": {"workload": w.name, "seq_lens": list(inp.seqlens) if len(inp.seqlens) <= 16 else len(inp.seqlens),
                   "total_tokens": T_tok, "n_heads_q": H, "n_heads_kv": w.n_heads_kv, "head_dim": D,
                   "block_q": w.block_q, "block_k": w.block_k, "lambda": "inf", "paged": w.paged},
        "executed_tflops": exec_tflops,
        "effective_tflops": dense_flops / (ms * 1e-3) / 1e12,
        "skip_fraction": 1.0 - kept / visited,
        "roofline": {
            "bound": "mfma",
            "achieved": exec_tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": exec_tflops / peak,
            "traffic": traffic,  # HBM bytes per launch (rocprofv3), or None
            "traffic_source": traffic_src,
            "per_launch": f"{visited} visited + {kept} kept (tile, block) pairs x 2*{w.block_q}*{w.block_k}*{D} "
                          f"FLOP = {exec_flops:.4g} FLOP",
        },
        "generation_s": round(gen_s, 1),
    }

    # ---- the workload's finite lambdas: skip fraction and speed-up over dense mode
    # Dense mode and every finite lambda are timed in turns, so that the speed-ups
    # compare calls made under the same clocks.
    sparse = []
    finite_l = [x for x in lambdas if not math.isinf(x)]
    if finite_l and args.sparse_steps > 0:
        skipped_l = {}
        for lam in finite_l:  # one call each for the skip counts
            call(lam)()
            torch.cuda.synchronize()
            skipped_l[lam] = int(sc.sum().item())
        fns = {dense_lam: call(dense_lam)}
        fns.update({lam: call(lam) for lam in finite_l})
        times, seg_calls = time_interleaved(fns, rounds=args.sparse_steps)
        for lam in finite_l:
            ms_l = times[lam]
            kept_l = visited - skipped_l[lam]
            f = skipped_l[lam] / visited
            sparse.append({
                "lambda": lam, "ms": ms_l, "tokens_per_s": T_tok / (ms_l * 1e-3), "skip_fraction": f,
                "executed_tflops": unit_flops * (visited + kept_l) / (ms_l * 1e-3) / 1e12,
                "effective_tflops": dense_flops / (ms_l * 1e-3) / 1e12,
                "speedup_vs_dense": times[dense_lam] / ms_l, "flop_model_speedup": 1.0 / (1.0 - f / 2.0),
            })
        result["sparse_timing"] = {
            "dense_ms": times[dense_lam],
            "how": f"dense mode and each finite lambda timed in turns: median over {args.sparse_steps} rounds of "
                   f"{seg_calls}-call segments after a 0.25 s warm-up; speed-ups are against this dense time",
        }
    result["sparse"] = sparse

    # ---- per-call median, warm and with the last-level cache flushed between calls
    if args.extra_steps > 0:
        flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        result["timing"] = {
            "mean_ms": ms,
            "median_ms_warm": time_each(call(dense_lam), args.extra_steps),
            "median_ms_flushed": time_each(call(dense_lam), args.extra_steps, flush=lambda: flush_buf.fill_(7)),
            "flush": "512 MiB device fill between calls (MI355X last-level cache is 256 MiB)",
        }
        del flush_buf

    # ---- ablation switches at the smallest finite lambda: what each saving is worth
    finite = [x for x in lambdas if not math.isinf(x)]
    if args.extra_steps > 0 and finite:
        lam_a = min(finite)

        def call_flags(fl):
            return lambda: bsp.fwd(q, k, v, cu, inp.max_seqlen, block_table=table, block_q=w.block_q,
                                   block_k=w.block_k, lam=lam_a, q_scale=scales[0], k_scale=scales[1],
                                   v_scale=scales[2], out=o, lse=lse, bitmap=bm, skip_count=sc,
                                   visited_count=vc, flags=fl)

        variants = (("skip_all", 0), ("load_skipped_v", bsp.FLAG_LOAD_SKIPPED_V),
                    ("exp_skipped", bsp.FLAG_EXP_SKIPPED),
                    ("load_v_and_exp_skipped", bsp.FLAG_LOAD_SKIPPED_V | bsp.FLAG_EXP_SKIPPED))
        ab, seg_calls = time_interleaved({name: call_flags(fl) for name, fl in variants}, rounds=args.extra_steps)
        ab["skip_fraction"] = int(sc.sum().item()) / visited
        result["ablation"] = {"lambda": lam_a, "ms": ab, "dense_ms": ms,
                              "note": "flags keep the decisions and outputs; they only add back the V load "
                                      "and/or the exps of skipped blocks",
                              "timing": f"the four variants timed in turns: median over {args.extra_steps} rounds "
                                        f"of {seg_calls}-call segments after a 0.25 s warm-up"}

    # ---- chunked prefill against a cached prefix and one decoding step (single-sequence workloads)
    if args.extra_steps > 0 and len(inp.seqlens) == 1 and not w.paged and inp.seqlens[0] >= 16384:
        L = inp.seqlens[0]
        cu_k = torch.tensor([0, L], dtype=torch.int32, device="cuda")
        rows = []
        for lq in (8192, 1):
            q_c = q[L - lq:].contiguous()
            o_c = torch.empty((lq, H, D), dtype=o.dtype, device="cuda")
            lse_c = torch.empty((H, lq), dtype=torch.float32, device="cuda")
            cu_q = torch.tensor([0, lq], dtype=torch.int32, device="cuda")
            for lam in [dense_lam] + finite[-1:]:
                def fn(lam=lam):
                    return bsp.fwd(q_c, k, v, cu_q, lq, block_q=w.block_q, block_k=w.block_k, lam=lam,
                                   q_scale=scales[0], k_scale=scales[1], v_scale=scales[2], out=o_c,
                                   lse=lse_c, want_bitmap=False, skip_count=sc, visited_count=vc,
                                   cu_seqlens_k=cu_k, max_seqlen_k=L)
                ms_c = time_calls(fn, args.extra_steps, 2)
                vis, skp = int(vc.sum().item()), int(sc.sum().item())
                kept_c = vis - skp
                kv_bytes = (vis + kept_c) * w.block_k * D * k.element_size() * (w.n_heads_kv / H)
                rows.append({"lq": lq, "lk": L, "lambda": lam, "ms": ms_c, "query_tokens_per_s": lq / (ms_c * 1e-3),
                             "skip_fraction": skp / vis,
                             "executed_tflops": unit_flops * (vis + kept_c) / (ms_c * 1e-3) / 1e12,
                             "kv_gbs": kv_bytes / (ms_c * 1e-3) / 1e9 if lq == 1 else None})
        result["chunked"] = rows

        result["decode"] = decode_rows(bsp, w, q, k, v, scales, dense_lam, finite, args.extra_steps)

    if not args.no_mfma_probe:
        result["roofline"]["measured_peak"] = mfma_probe()

    if not args.no_extra_workloads and args.extra_steps > 0:
        rows = []
        for name, dt in EXTRA_WORKLOADS:
            if (name, dt) == (w.name, dtype):
                continue
            print(f"# extra workload {name} ({dt})", file=sys.stderr, flush=True)
            rows.append(workload_row(bsp, name, dt, args.extra_steps))
        result["workloads"] = rows

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, w, dense_lam, target_s=args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
