"""Parity protocol between the HIP path and the CPU oracle (test infrastructure).

For one (inputs, block sizes, lambda) case:
  1. run the HIP library through its C ABI (``block_sparse_long_bsp_amd.fwd``);
  2. run the oracle on the same inputs for a set of work items (all, or a
     deterministic sample for large workloads);
  3. the skip bitmaps must be identical on every visited pair whose decision
     margin |min gap - lambda| exceeds the band of 1e-3 (scores are fp32 on
     the GPU and fp64 in the oracle, so pairs inside that band may
     legitimately flip). The same band holds for fp8 inputs: their MFMA dot
     product does not round once (tests/test_gpu_exact.py pins its error
     within 2^-11 of the scaled sum_i |q_i k_i|), but on the 128K fp8
     workload every flip seen lies within 1e-3; the flip counts by margin
     are reported (Report.n_flips_tight / n_flips_wide, FLIP_TALLY);
  4. where they differ inside the band, the oracle is re-run with the GPU's
     decisions forced, and outputs are compared against that run;
  5. O must satisfy the dtype's tolerance (bf16: max-abs <= 2e-2 and
     mean-abs <= 2e-3; fp32: max-abs <= 1e-4; fp8: max-abs <= 6e-2) and LSE
     |delta| <= 1e-2 (1e-4 for fp32);
  6. per-head skip counts equal the bitmap's popcount and the visited counts
     equal the causal pair count.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

import oracle
import synth

MARGIN_BAND = {"f32": 1e-3, "bf16": 1e-3, "fp8": 1e-3}
TOL = {
    "f32": dict(max_abs=1e-4, mean_abs=1e-4, lse=1e-4),
    "bf16": dict(max_abs=2e-2, mean_abs=2e-3, lse=1e-2),
    "fp8": dict(max_abs=6e-2, mean_abs=6e-3, lse=1e-2),
}


def to_device(inp: synth.Inputs, device="cuda"):
    """Upload storage arrays as torch tensors; returns a dict of tensors."""
    import torch

    def conv(a, dtype):
        if dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
        if dtype == "fp8":
            return torch.from_numpy(np.ascontiguousarray(a)).to(device).view(torch.float8_e4m3fn)
        raise ValueError(dtype)

    d = dict(q=conv(inp.q, inp.dtype), k=conv(inp.k, inp.dtype), v=conv(inp.v, inp.dtype),
             cu=torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device))
    if inp.k_pages is not None:
        d["k_pages"] = conv(inp.k_pages, inp.dtype)
        d["v_pages"] = conv(inp.v_pages, inp.dtype)
        d["table"] = torch.from_numpy(inp.block_table.astype(np.int32)).to(device)
    for nm in ("q_scale", "k_scale", "v_scale"):
        a = getattr(inp, nm)
        d[nm] = None if a is None else torch.from_numpy(a.astype(np.float32)).to(device)
    return d


@dataclass
class Chunk:
    """Chunked prefill: sequence s's queries are its last lq[s] positions."""
    lq: Sequence[int]

    def rows(self, inp: synth.Inputs) -> np.ndarray:
        cu = inp.cu_seqlens
        return np.concatenate([np.arange(int(cu[s + 1]) - n, int(cu[s + 1])) for s, n in enumerate(self.lq)]
                              + [np.zeros(0, int)]).astype(np.int64)

    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lq)]).astype(np.int32)


def run_gpu(inp: synth.Inputs, dev: Dict, block_q: int, block_k: int, lam: float, paged: bool = False,
            chunk: Optional[Chunk] = None, lam_seq: Optional[Sequence[float]] = None, flags: int = 0,
            decode: bool = False):
    import torch

    import block_sparse_long_bsp_amd as bsp

    k = dev["k_pages"] if paged else dev["k"]
    v = dev["v_pages"] if paged else dev["v"]
    n_seqs = len(inp.seqlens)
    if decode:
        # bsp_attn_decode: the last row of every sequence against all of its keys
        # (the chunk-of-one case of the oracle)
        assert chunk is not None and all(n == 1 for n in chunk.lq)
        q = dev["q"][torch.from_numpy(chunk.rows(inp)).to(dev["q"].device)].contiguous()
        seq_sc = torch.empty(n_seqs, dtype=torch.int64, device=q.device)
        seq_vc = torch.empty(n_seqs, dtype=torch.int64, device=q.device)
        lps = None if lam_seq is None else torch.tensor(list(lam_seq), dtype=torch.float32, device=q.device)
        o, lse, bitmap, sc, vc = bsp.decode(q, k, v, dev["cu"], inp.max_seqlen, total_k=inp.total_tokens,
                                            block_table=dev.get("table") if paged else None, block_k=block_k,
                                            lam=lam, q_scale=dev["q_scale"], k_scale=dev["k_scale"],
                                            v_scale=dev["v_scale"], lam_per_seq=lps, seq_skip_count=seq_sc,
                                            seq_visited_count=seq_vc, flags=flags)
        torch.cuda.synchronize()
        return dict(o=o.float().cpu().numpy(), lse=lse.cpu().numpy(),
                    bits=bsp.unpack_bitmap(bitmap, inp.q.shape[1], n_seqs, 1, 1, block_k, inp.max_seqlen),
                    skip_count=sc.cpu().numpy(), visited_count=vc.cpu().numpy(),
                    seq_skip_count=seq_sc.cpu().numpy(), seq_visited_count=seq_vc.cpu().numpy())
    kw = {}
    q, cu, max_q = dev["q"], dev["cu"], inp.max_seqlen
    if chunk is not None:
        q = dev["q"][torch.from_numpy(chunk.rows(inp)).to(q.device)].contiguous()
        cu = torch.from_numpy(chunk.cu_q()).to(q.device)
        max_q = max(list(chunk.lq) + [0])
        kw.update(cu_seqlens_k=dev["cu"], max_seqlen_k=inp.max_seqlen)
    if lam_seq is not None:
        kw["lam_per_seq"] = torch.tensor(list(lam_seq), dtype=torch.float32, device=q.device)
    seq_sc = torch.empty(n_seqs, dtype=torch.int64, device=q.device)
    seq_vc = torch.empty(n_seqs, dtype=torch.int64, device=q.device)
    out = bsp.fwd(q, k, v, cu, max_q, block_table=dev.get("table") if paged else None,
                  block_q=block_q, block_k=block_k, lam=lam, q_scale=dev["q_scale"], k_scale=dev["k_scale"],
                  v_scale=dev["v_scale"], seq_skip_count=seq_sc, seq_visited_count=seq_vc, flags=flags, **kw)
    torch.cuda.synchronize()
    o, lse, bitmap, sc, vc = out
    return dict(o=o.float().cpu().numpy(), lse=lse.cpu().numpy(),
                bits=bsp.unpack_bitmap(bitmap, inp.q.shape[1], n_seqs, max_q, block_q, block_k, inp.max_seqlen),
                skip_count=sc.cpu().numpy(), visited_count=vc.cpu().numpy(),
                seq_skip_count=seq_sc.cpu().numpy(), seq_visited_count=seq_vc.cpu().numpy())


@dataclass
class Report:
    n_items: int = 0
    n_pairs: int = 0
    n_skipped: int = 0
    n_band_flips: int = 0    # decisions that differ from the oracle's (all inside the band, else a problem)
    n_flips_tight: int = 0   # ... of which with |margin| <= 1e-3
    n_flips_wide: int = 0    # ... of which with 1e-3 < |margin| <= the dtype's band
    max_flip_margin: float = 0.0
    max_abs: float = 0.0
    mean_abs: float = 0.0
    lse_max: float = 0.0
    problems: List[str] = field(default_factory=list)

    def ok(self):
        return not self.problems


def compare(inp: synth.Inputs, gpu: Dict, block_q: int, block_k: int, lam: float,
            work: Optional[np.ndarray] = None, n_threads: int = 0, check_counts: bool = True,
            chunk: Optional[Chunk] = None, lam_seq: Optional[Sequence[float]] = None,
            band: Optional[float] = None) -> Report:
    """Steps 2-6 of the protocol for the given work items (default: all).

    ``band`` overrides the dtype's decision band (0: the bitmaps must be
    identical, for inputs whose scores every side computes exactly)."""
    band = MARGIN_BAND[inp.dtype] if band is None else band
    Hq = inp.q.shape[1]
    n_seqs = len(inp.seqlens)
    J = max(1, (inp.max_seqlen + block_k - 1) // block_k)
    if chunk is None:
        cu = inp.cu_seqlens
        lq = list(inp.seqlens)

        def run_ref(**kw):
            return oracle.run_inputs(inp, block_q, block_k, lam, n_threads=n_threads, j_max=J, lam_seq=lam_seq, **kw)
    else:
        cu = chunk.cu_q()
        lq = list(chunk.lq)
        qrows = inp.q[chunk.rows(inp)]

        def run_ref(**kw):
            return oracle.run(qrows, inp.k, inp.v, cu, Hq, inp.k.shape[1], block_q, block_k, lam,
                              q_scale=inp.q_scale, k_scale=inp.k_scale, v_scale=inp.v_scale, n_threads=n_threads,
                              j_max=J, cu_seqlens_k=inp.cu_seqlens, lam_seq=lam_seq, **kw)
    if work is None and chunk is not None:
        work = synth.work_items(lq, Hq, block_q)
    ref = run_ref(work=work)
    lam_of = (lambda s_: lam) if lam_seq is None else (lambda s_: lam_seq[s_])
    rep = Report(n_items=ref.work.shape[0])
    gbits = np.zeros_like(ref.skip)
    for w, (s, h, t) in enumerate(ref.work):
        gbits[w] = gpu["bits"][h, s, t, :J]
    vis = ref.visited.astype(bool)
    rep.n_pairs = int(vis.sum())
    # bits outside the visited range must be zero
    if np.any(gbits.astype(bool) & ~vis):
        rep.problems.append("GPU bitmap has bits on unvisited pairs")
    diff = (gbits != ref.skip) & vis
    if diff.any():
        lam_item = np.array([lam_of(int(s_)) for s_ in ref.work[:, 0]])[:, None]
        with np.errstate(invalid="ignore"):
            margin = np.abs(ref.mingap - lam_item)
        hard = diff & ~(margin <= band)
        if hard.any():
            idx = np.argwhere(hard)[:5]
            rep.problems.append(f"{int(hard.sum())} skip decisions differ outside the margin band, e.g. "
                                + ", ".join(f"item{tuple(ref.work[i])} block {j} gap {ref.mingap[i, j]:.6g}"
                                            for i, j in idx))
        rep.n_band_flips = int(diff.sum())
        soft = diff & ~hard
        rep.n_flips_tight = int((soft & (margin <= 1e-3)).sum())
        rep.n_flips_wide = int((soft & (margin > 1e-3)).sum())
        rep.max_flip_margin = float(margin[soft].max()) if soft.any() else 0.0
        forced = np.where(vis, gbits, 0).astype(np.uint8)
        ref = run_ref(work=ref.work, forced=forced)
    rep.n_skipped = int((ref.skip.astype(bool) & vis).sum())
    tol = TOL[inp.dtype]
    errs = []
    lse_err = 0.0
    for w, (s, h, t) in enumerate(ref.work):
        L = int(cu[s + 1] - cu[s])
        r0, r1 = t * block_q, min(L, (t + 1) * block_q)
        if r1 <= r0:
            continue
        a, b = int(cu[s]) + r0, int(cu[s]) + r1
        e = np.abs(gpu["o"][a:b, h, :].astype(np.float64) - ref.o[w, : r1 - r0])
        errs.append(e.ravel())
        le = np.abs(gpu["lse"][h, a:b].astype(np.float64) - ref.lse[w, : r1 - r0])
        lse_err = max(lse_err, float(np.nanmax(le)) if le.size else 0.0)
        if not np.all(np.isfinite(gpu["o"][a:b, h, :])):
            rep.problems.append(f"non-finite output in item {(s, h, t)}")
    if errs:
        allerr = np.concatenate(errs)
        rep.max_abs = float(allerr.max())
        rep.mean_abs = float(allerr.mean())
    rep.lse_max = lse_err
    if rep.max_abs > tol["max_abs"]:
        rep.problems.append(f"max-abs {rep.max_abs:.3g} > {tol['max_abs']}")
    if rep.mean_abs > tol["mean_abs"]:
        rep.problems.append(f"mean-abs {rep.mean_abs:.3g} > {tol['mean_abs']}")
    if rep.lse_max > tol["lse"]:
        rep.problems.append(f"LSE max error {rep.lse_max:.3g} > {tol['lse']}")
    if check_counts:
        bits = gpu["bits"]
        pop = bits.reshape(Hq, -1).sum(axis=1)
        if not np.array_equal(pop, gpu["skip_count"].astype(np.int64)):
            rep.problems.append(f"skip_count {gpu['skip_count'][:4]}... != bitmap popcount {pop[:4]}...")
        vis_expect = 0
        vis_seq = np.zeros(n_seqs, dtype=np.int64)
        for s, L in enumerate(lq):
            off = int(inp.seqlens[s]) - L
            for t in range((L + block_q - 1) // block_q):
                r1 = min(L, (t + 1) * block_q)
                vis_seq[s] += ((off + r1 - 1) // block_k + 1) * Hq
        vis_expect = np.full(Hq, vis_seq.sum() // max(Hq, 1), dtype=np.int64)
        if not np.array_equal(vis_expect, gpu["visited_count"].astype(np.int64)):
            rep.problems.append(f"visited_count {gpu['visited_count'][:4]} != {vis_expect[:4]}")
        if "seq_skip_count" in gpu:
            pop_seq = bits.transpose(1, 0, 2, 3).reshape(n_seqs, -1).sum(axis=1)
            if not np.array_equal(pop_seq, gpu["seq_skip_count"].astype(np.int64)):
                rep.problems.append(f"per-sequence skip counts {gpu['seq_skip_count'][:4]} != {pop_seq[:4]}")
            if not np.array_equal(vis_seq, gpu["seq_visited_count"].astype(np.int64)):
                rep.problems.append(f"per-sequence visited counts {gpu['seq_visited_count'][:4]} != {vis_seq[:4]}")
    return rep


def check_case(inp: synth.Inputs, block_q: int, block_k: int, lams: Sequence[float], paged: bool = False,
               work: Optional[np.ndarray] = None, dev=None, chunk: Optional[Chunk] = None,
               lam_seq: Optional[Sequence[float]] = None, flags: int = 0, decode: bool = False,
               band: Optional[float] = None) -> List[Report]:
    """Run the GPU for each lambda and compare; raise AssertionError on any problem.

    Every report's flip counts are also added to ``FLIP_TALLY`` (per dtype)."""
    dev = dev or to_device(inp)
    reps = []
    for lam in lams:
        gpu = run_gpu(inp, dev, block_q, block_k, lam, paged=paged, chunk=chunk, lam_seq=lam_seq, flags=flags,
                      decode=decode)
        rep = compare(inp, gpu, block_q, block_k, lam, work=work, chunk=chunk, lam_seq=lam_seq, band=band)
        reps.append(rep)
        t = FLIP_TALLY.setdefault(inp.dtype, dict(pairs=0, tight=0, wide=0, max_margin=0.0))
        t["pairs"] += rep.n_pairs
        t["tight"] += rep.n_flips_tight
        t["wide"] += rep.n_flips_wide
        t["max_margin"] = max(t["max_margin"], rep.max_flip_margin)
        assert rep.ok(), (f"lambda={lam}: " + "; ".join(rep.problems)
                          + f" [flips: {rep.n_flips_tight} with |margin| <= 1e-3, {rep.n_flips_wide} wider]")
    return reps


# Decision flips (GPU vs oracle) seen by check_case in this process, per input dtype:
# visited pairs compared, flips with |margin| <= 1e-3, flips with a wider margin.
FLIP_TALLY: Dict[str, Dict[str, float]] = {}
