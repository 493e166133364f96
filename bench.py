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


def cpu_baseline(inp, w, lam, target_s=15.0):
    """Time the CPU oracle on a bounded, deterministic sample of the workload
    and scale its rate to the whole job (by visited pairs)."""
    import oracle
    import synth

    threads = int(os.environ.get("BSP_ORACLE_THREADS", "0")) or min(16, os.cpu_count() or 1)
    L = inp.seqlens
    T = [(x + w.block_q - 1) // w.block_q for x in L]
    # calibration: one heavy tile of head 0 of the longest sequence
    s_long = int(np.argmax(L))
    cal = np.array([[s_long, 0, T[s_long] - 1]], np.int32)
    t0 = time.perf_counter()
    oracle.run_inputs(inp, w.block_q, w.block_k, lam, work=cal, n_threads=1)
    t_cal = time.perf_counter() - t0
    pairs_cal = (min(L[s_long], T[s_long] * w.block_q) - 1) // w.block_k + 1
    per_pair = t_cal / pairs_cal  # single-thread seconds per visited pair
    budget_pairs = max(1, int(target_s * threads / per_pair))
    # sample: head 0 of every sequence, every n-th tile (first and last included)
    stride = 1
    while True:
        work = synth.work_items(L, w.n_heads_q, w.block_q, heads=[0], tile_stride=stride)
        pairs = sum(((min(L[s], (t + 1) * w.block_q) - 1) // w.block_k + 1) for s, _, t in work)
        if pairs <= budget_pairs or stride > 4096:
            break
        stride *= 2
    t0 = time.perf_counter()
    oracle.run_inputs(inp, w.block_q, w.block_k, lam, work=work, n_threads=threads)
    t_sample = time.perf_counter() - t0
    total_pairs = pair_counts(L, w.block_q, w.block_k) * w.n_heads_q
    t_full = t_sample * total_pairs / pairs
    return {
        "value": sum(L) / t_full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "sample": f"head 0, every {stride}th query tile (+first/last): {work.shape[0]} tiles, {pairs} of "
                  f"{total_pairs} visited (tile, block) pairs, lambda={lam}; {t_sample:.1f} s wall, scaled by pairs",
        "sample_seconds": round(t_sample, 2), "cpu": platform.processor() or platform.machine(),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_32k_bf16")
    ap.add_argument("--dtype", default=None)
    ap.add_argument("--sparse-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    lambdas = list(w.lambdas)
    dense_lam = math.inf
    visited = pair_counts(inp.seqlens, w.block_q, w.block_k) * H
    unit_flops = 2.0 * w.block_q * w.block_k * D
    dense_flops = dense_causal_flops(inp.seqlens, H, D)

    # ---- timed step: dense mode (lambda = +inf)
    ms = time_calls(call(dense_lam), args.steps, args.warmup)
    kept = visited - int(sc.sum().item())
    assert int(vc.sum().item()) == visited, "visited count mismatch"
    exec_flops = unit_flops * (visited + kept)
    tokens_s = T_tok / (ms * 1e-3)
    exec_tflops = exec_flops / (ms * 1e-3) / 1e12
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
            "peak": PEAK_TFLOPS[dtype],
            "unit": "TFLOP/s",
            "frac": exec_tflops / PEAK_TFLOPS[dtype],
            "traffic": None,
            "per_launch": f"{visited} visited + {kept} kept (tile, block) pairs x 2*{w.block_q}*{w.block_k}*{D} "
                          f"FLOP = {exec_flops:.4g} FLOP",
        },
        "generation_s": round(gen_s, 1),
    }

    # ---- the workload's finite lambdas: skip fraction and speed-up over dense mode
    sparse = []
    for lam in lambdas:
        if math.isinf(lam) or args.sparse_steps <= 0:
            continue
        ms_l = time_calls(call(lam), args.sparse_steps, 2)
        skipped = int(sc.sum().item())
        kept_l = visited - skipped
        f = skipped / visited
        sparse.append({
            "lambda": lam, "ms": ms_l, "tokens_per_s": T_tok / (ms_l * 1e-3), "skip_fraction": f,
            "executed_tflops": unit_flops * (visited + kept_l) / (ms_l * 1e-3) / 1e12,
            "effective_tflops": dense_flops / (ms_l * 1e-3) / 1e12,
            "speedup_vs_dense": ms / ms_l, "flop_model_speedup": 1.0 / (1.0 - f / 2.0),
        })
    result["sparse"] = sparse

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, w, dense_lam, target_s=args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
