"""CPU oracle for causal block-sparse prefill attention (test infrastructure).

Only the tests, the smoke check in ``__graft_entry__`` and the benchmark's
CPU-baseline leg may import this package. It shares nothing with the HIP
library in ``block_sparse_long_bsp_amd`` and never imports it.

The arithmetic lives in ``bsp_oracle.c`` (plain C, double precision, OpenMP
over work items); this module only compiles it with gcc, loads it with ctypes
and reshapes its outputs. The method follows the page "长上下文推理加速方案部署实战：
基于动态稀疏注意力机制的推理服务优化指南" (a deployment guide for a dynamic sparse
attention kernel), sections 3.2 and 6.1: per key block, in ascending order,
compare the running maximum of the scores with the block's local maximum and
skip the block (exp, V load, PV) when the gap exceeds lambda.

Every function here has its pins in ``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bsp_oracle.c")
_LIB = os.path.join(_HERE, "libbsp_oracle.so")
RULE = 255  # forced-decision value meaning "apply the rule"

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """Load a compiled oracle library and declare its entry point."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.bsp_oracle_fwd.restype = ctypes.c_int
    lib.bsp_oracle_fwd.argtypes = [P, P, P, ctypes.c_int, P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, P, P,
                                   ctypes.c_int64, P, ctypes.c_int, P, P, P, P, P, P, ctypes.c_int,
                                   ctypes.c_int]
    return lib


def compile_source(src: str, out: str) -> str:
    """Compile oracle C source text to a shared library at ``out``."""
    c_path = out + ".c"
    with open(c_path, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
                    "-ffp-contract=off", c_path, "-o", out, "-lm"], check=True)
    return out


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = load_library(_LIB)
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


@dataclass
class OracleResult:
    """Per-work-item outputs; row r of item w is query row tile*block_q + r of
    the sequence's query rows (its chunk, with a cached prefix)."""
    work: np.ndarray        # int32 [n, 3] (seq, head, tile)
    o: np.ndarray           # float64 [n, block_q, D]
    lse: np.ndarray         # float64 [n, block_q]  (NaN past the sequence end)
    skip: np.ndarray        # uint8  [n, j_max]     1 = visited and skipped
    visited: np.ndarray     # uint8  [n, j_max]
    mingap: np.ndarray      # float64 [n, j_max]    NaN where not visited
    p: Optional[np.ndarray]  # float64 [n, block_q, p_cols] or None
    block_q: int
    block_k: int


_IN_DTYPES = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.uint8): 2}


def run(q32: np.ndarray, k32: np.ndarray, v32: np.ndarray, cu_seqlens: np.ndarray,
        n_heads_q: int, n_heads_kv: int, block_q: int, block_k: int, lam: float,
        work: Optional[np.ndarray] = None, q_scale=None, k_scale=None, v_scale=None,
        forced: Optional[np.ndarray] = None, export_p: bool = False, n_threads: int = 0,
        j_max: Optional[int] = None, cu_seqlens_k: Optional[np.ndarray] = None,
        lam_seq: Optional[Sequence[float]] = None) -> OracleResult:
    """Run the oracle on packed varlen inputs.

    ``q32`` [Tq, Hq, D], ``k32``/``v32`` [Tk, Hkv, D] hold storage values: float32,
    bf16 bit patterns (uint16) or fp8 e4m3 codes (uint8), all three of one
    type; the optional per-head scales multiply them (fp8).
    ``cu_seqlens`` delimits the query rows of each sequence and ``cu_seqlens_k``
    (default: the same) its keys/values; with Lk > Lq the queries are the last
    Lq positions of the sequence (chunked prefill against a cached prefix).
    ``lam_seq`` gives one lambda per sequence (default: ``lam`` for all).
    ``work`` lists (seq, head, tile) triples; default: every tile of every head.
    ``forced`` [n, j_max] uint8 overrides decisions (0 keep, 1 skip, RULE).
    """
    lib = _load()
    q32 = np.ascontiguousarray(q32)
    k32 = np.ascontiguousarray(k32)
    v32 = np.ascontiguousarray(v32)
    if not (q32.dtype == k32.dtype == v32.dtype) or q32.dtype not in _IN_DTYPES:
        raise ValueError("q, k, v must share one storage dtype (float32, uint16 bf16 bits, uint8 fp8 codes)")
    in_dtype = _IN_DTYPES[q32.dtype]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    n_seqs = len(cu) - 1
    cuk = None if cu_seqlens_k is None else np.ascontiguousarray(cu_seqlens_k, dtype=np.int32)
    if cuk is not None and len(cuk) != n_seqs + 1:
        raise ValueError("cu_seqlens_k must have n_seqs + 1 entries")
    lam_arr = None if lam_seq is None else np.ascontiguousarray(lam_seq, dtype=np.float64)
    if lam_arr is not None and len(lam_arr) != n_seqs:
        raise ValueError("lam_seq must have one entry per sequence")
    D = q32.shape[2]
    seqlens = np.diff(cu)
    seqlens_k = seqlens if cuk is None else np.diff(cuk)
    max_len = int(seqlens_k.max()) if n_seqs > 0 else 0
    if j_max is None:
        j_max = max(1, (max_len + block_k - 1) // block_k)
    if work is None:
        tri = []
        for s in range(n_seqs):
            T = (int(seqlens[s]) + block_q - 1) // block_q
            for h in range(n_heads_q):
                for t in range(T):
                    tri.append((s, h, t))
        work = np.asarray(tri, dtype=np.int32).reshape(-1, 3)
    work = np.ascontiguousarray(work, dtype=np.int32).reshape(-1, 3)
    n = work.shape[0]
    o = np.zeros((n, block_q, D))
    lse = np.zeros((n, block_q))
    skip = np.zeros((n, j_max), dtype=np.uint8)
    visited = np.zeros((n, j_max), dtype=np.uint8)
    mingap = np.zeros((n, j_max))
    p_cols = max_len if export_p else 0
    p = np.zeros((n, block_q, p_cols)) if export_p else None
    sc = [None if x is None else np.ascontiguousarray(x, dtype=np.float64) for x in (q_scale, k_scale, v_scale)]
    if forced is not None:
        forced = np.ascontiguousarray(forced, dtype=np.uint8)
        assert forced.shape == (n, j_max)
    rc = lib.bsp_oracle_fwd(_ptr(q32), _ptr(k32), _ptr(v32), in_dtype, _ptr(sc[0]), _ptr(sc[1]), _ptr(sc[2]),
                            _ptr(cu), _ptr(cuk), n_seqs, n_heads_q, n_heads_kv, D, block_q, block_k, float(lam),
                            _ptr(lam_arr), _ptr(work), n, _ptr(forced), j_max, _ptr(o), _ptr(lse), _ptr(skip),
                            _ptr(visited), _ptr(mingap), _ptr(p), p_cols, int(n_threads))
    if rc != 0:
        raise ValueError(f"bsp_oracle_fwd failed with code {rc}")
    return OracleResult(work=work, o=o, lse=lse, skip=skip, visited=visited, mingap=mingap, p=p,
                        block_q=block_q, block_k=block_k)


def run_inputs(inp, block_q: int, block_k: int, lam: float, **kw) -> OracleResult:
    """``run`` on a ``synth.Inputs`` object (fp8 scales applied)."""
    return run(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.q.shape[1], inp.k.shape[1], block_q, block_k,
               lam, q_scale=inp.q_scale, k_scale=inp.k_scale, v_scale=inp.v_scale, **kw)


def scatter(res: OracleResult, cu_seqlens: np.ndarray, n_heads_q: int):
    """Place per-item outputs into full arrays: O [T, Hq, D] and LSE [Hq, T]
    (NaN where no work item covered a row)."""
    cu = np.asarray(cu_seqlens)
    T = int(cu[-1])
    D = res.o.shape[2]
    O = np.full((T, n_heads_q, D), np.nan)
    LSE = np.full((n_heads_q, T), np.nan)
    for w, (s, h, t) in enumerate(res.work):
        L = int(cu[s + 1] - cu[s])
        r0 = t * res.block_q
        r1 = min(r0 + res.block_q, L)
        if r1 <= r0:
            continue
        O[cu[s] + r0: cu[s] + r1, h] = res.o[w, : r1 - r0]
        LSE[h, cu[s] + r0: cu[s] + r1] = res.lse[w, : r1 - r0]
    return O, LSE
