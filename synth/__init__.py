"""Seeded synthetic inputs for causal block-sparse prefill attention.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds none of the attention arithmetic: it only draws a latent
AR(1) process per KV head, derives noisy queries and keys from it, adds
"sink" and "vertical" keys, rounds the values to their storage type
(fp32, bf16, fp8 e4m3) and lays K/V out either contiguously or in
randomly-permuted fixed-size pages.

Workloads (all causal, scale = 1/sqrt(head_dim)):

* ``single_1k_fp32``   one sequence of 1024 tokens, 1 head, D=64, fp32,
  64/64 tiles, lambda in {8, +inf}; AR(1) rho=0.99, 4 sink keys.
* ``llama8b_8k_bf16``  one 8192-token sequence with the attention shape of a
  Llama-3.1-8B layer (32 query heads, 8 KV heads, D=128), bf16,
  128/64 tiles, lambda in {+inf, 8, 4}.
* ``llama8b_32k_bf16`` same shape at 32768 tokens, 128/128 tiles,
  lambda in {+inf, 6, 3}; rho=0.995 and 64 "vertical" keys per KV head.
* ``llama8b_128k``     same shape at 131072 tokens, bf16 and fp8 e4m3 with
  per-head scales, 128/128 tiles, lambda in {+inf, 6, 3}; rho=0.998 and 128
  vertical keys.
* ``varlen16_paged_bf16`` 16 sequences with log-uniform lengths in
  [512, 32768], packed by cu_seqlens, K/V in 64-token pages scattered by a
  random permutation, bf16, 64/64 tiles, lambda in {6, +inf}.

Generation recipe, per sequence and per KV head g (independent RNG stream):
  x_0 ~ N(0, I_D);  x_t = rho x_{t-1} + sqrt(1-rho^2) eps_t
  q_t^{(h)} = 2 x_t + N(0, I)  for each of the group's query heads h
  k_t = 2 x_t + N(0, I);  v_t ~ N(0, I)
  mu = mean over positions and over the group's query heads of q
  k_0..k_3 += 3 mu (attention sinks)
  k_p += 2 mu for n_vert positions p drawn without replacement from [4, L)
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
from scipy.signal import lfilter

BASE_SEED = 20261202

# Purpose codes mixed into the seed sequence so that independent draws never
# share a stream.
_P_HEAD = 1
_P_LENS = 2
_P_PAGES = 3


# --------------------------------------------------------------------------
# Storage-type rounding (bit-level definitions, no attention arithmetic)
# --------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); returns the
    16-bit patterns as uint16. Inputs must be finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


FP8_E4M3_MAX = 448.0


def fp8_e4m3_decode_table() -> np.ndarray:
    """Values of the 256 OCP fp8 e4m3 (e4m3fn) codes as float64.

    Layout s.eeee.mmm, exponent bias 7; exponent field 0 encodes subnormals
    m/8 * 2^-6; codes 0x7F and 0xFF are NaN; there is no infinity.
    """
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if (c >> 7) & 1 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            t[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_FP8_TABLE = fp8_e4m3_decode_table()
# The 127 non-negative finite codes 0x00..0x7E are monotonically increasing.
_FP8_POS = _FP8_TABLE[:0x7F].copy()


def fp8_e4m3_quantize(y: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest fp8 e4m3 code (ties to the even
    code, i.e. even mantissa), saturating to +-448. Returns uint8 codes."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), FP8_E4M3_MAX)
    hi = np.searchsorted(_FP8_POS, a, side="left")  # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    vhi = _FP8_POS[hi]
    vlo = _FP8_POS[lo]
    dhi = vhi - a
    dlo = a - vlo
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = (y < 0) & (code != 0)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def fp8_e4m3_to_f32(c: np.ndarray) -> np.ndarray:
    """Decode fp8 e4m3 codes to float32 (exact)."""
    return _FP8_TABLE[np.asarray(c, dtype=np.uint8)].astype(np.float32)


# --------------------------------------------------------------------------
# Workload specifications
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    seqlens: Tuple[int, ...]          # filled in by ``seqlens_for`` for varlen
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    dtypes: Tuple[str, ...]           # "f32", "bf16", "fp8"
    block_q: int
    block_k: int
    lambdas: Tuple[float, ...]
    rho: float
    n_vert: int
    paged: bool = False
    page_size: int = 64
    n_varlen: int = 0                 # >0: draw this many log-uniform lengths
    varlen_range: Tuple[int, int] = (512, 32768)
    sink_tokens: int = 4
    sink_gain: float = 3.0
    vert_gain: float = 2.0
    code: int = 0                     # mixed into the seed

    @property
    def group(self) -> int:
        return self.n_heads_q // self.n_heads_kv


INF = math.inf

WORKLOADS: Dict[str, Workload] = {
    "single_1k_fp32": Workload(
        name="single_1k_fp32", seqlens=(1024,), n_heads_q=1, n_heads_kv=1, head_dim=64,
        dtypes=("f32",), block_q=64, block_k=64, lambdas=(8.0, INF), rho=0.99, n_vert=0, code=1),
    "llama8b_8k_bf16": Workload(
        name="llama8b_8k_bf16", seqlens=(8192,), n_heads_q=32, n_heads_kv=8, head_dim=128,
        dtypes=("bf16",), block_q=128, block_k=64, lambdas=(INF, 8.0, 4.0), rho=0.99, n_vert=0, code=2),
    "llama8b_32k_bf16": Workload(
        name="llama8b_32k_bf16", seqlens=(32768,), n_heads_q=32, n_heads_kv=8, head_dim=128,
        dtypes=("bf16",), block_q=128, block_k=128, lambdas=(INF, 6.0, 3.0), rho=0.995, n_vert=64, code=3),
    "llama8b_128k": Workload(
        name="llama8b_128k", seqlens=(131072,), n_heads_q=32, n_heads_kv=8, head_dim=128,
        dtypes=("bf16", "fp8"), block_q=128, block_k=128, lambdas=(INF, 6.0, 3.0), rho=0.998, n_vert=128,
        code=4),
    "varlen16_paged_bf16": Workload(
        name="varlen16_paged_bf16", seqlens=(), n_heads_q=32, n_heads_kv=8, head_dim=128,
        dtypes=("bf16",), block_q=64, block_k=64, lambdas=(6.0, INF), rho=0.99, n_vert=0,
        paged=True, page_size=64, n_varlen=16, code=5),
}


def seqlens_for(w: Workload) -> Tuple[int, ...]:
    """Sequence lengths of a workload (drawn log-uniformly for varlen)."""
    if w.n_varlen <= 0:
        return tuple(w.seqlens)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, w.code, _P_LENS])))
    lo, hi = w.varlen_range
    u = rng.uniform(math.log(lo), math.log(hi), size=w.n_varlen)
    return tuple(int(round(math.exp(x))) for x in u)


def _head_rng(code: int, seq: int, kv_head: int, salt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, code, _P_HEAD, seq, kv_head, salt])))


def gen_group(L: int, G: int, D: int, rho: float, n_vert: int, code: int, seq: int, g: int, salt: int = 0,
              sink_tokens: int = 4, sink_gain: float = 3.0, vert_gain: float = 2.0):
    """Draw one KV head's group for one sequence: a list of G float32 query
    arrays [L, D] and float32 k, v arrays [L, D]."""
    rng = _head_rng(code, seq, g, salt)
    c = math.sqrt(max(0.0, 1.0 - rho * rho))
    e = rng.standard_normal((L, D))
    if L > 1:
        e[1:] *= c
    x = lfilter([1.0], [1.0, -rho], e, axis=0) if L > 0 else e.copy()
    np.multiply(x, 2.0, out=x)                 # x now holds 2 x_t
    buf = e                                    # reuse the innovation buffer
    qs = []
    mu = np.zeros(D)
    for _ in range(G):
        rng.standard_normal(out=buf)
        buf += x
        if L > 0:
            mu += buf.sum(axis=0)
        qs.append(buf.astype(np.float32))
    mu /= max(1, L * G)
    rng.standard_normal(out=buf)
    buf += x
    k = buf
    v = rng.standard_normal((L, D), dtype=np.float64).astype(np.float32)
    ns = min(sink_tokens, L)
    k[:ns] += sink_gain * mu
    nv = min(n_vert, max(0, L - sink_tokens))
    if nv > 0:
        pos = rng.choice(np.arange(sink_tokens, L), size=nv, replace=False)
        k[pos] += vert_gain * mu
    return qs, k.astype(np.float32), v


def gen_sequence(L: int, n_heads_q: int, n_heads_kv: int, D: int, rho: float, n_vert: int,
                 code: int, seq: int, salt: int = 0, sink_tokens: int = 4,
                 sink_gain: float = 3.0, vert_gain: float = 2.0):
    """Draw float32 q [L, Hq, D], k/v [L, Hkv, D] for one sequence."""
    G = n_heads_q // n_heads_kv
    qh, kh, vh = [], [], []
    for g in range(n_heads_kv):
        qs, k, v = gen_group(L, G, D, rho, n_vert, code, seq, g, salt, sink_tokens, sink_gain, vert_gain)
        qh += qs
        kh.append(k)
        vh.append(v)
    return np.stack(qh, axis=1), np.stack(kh, axis=1), np.stack(vh, axis=1)


@dataclass
class Inputs:
    """Host-side arrays for one (workload, dtype) case.

    ``q``/``k``/``v`` hold the storage values (float32, bf16 bits as uint16 or
    fp8 e4m3 codes as uint8) in packed varlen layout [total_tokens, heads, D].
    ``q_scale``/``k_scale``/``v_scale`` are per-head float32 dequantisation
    scales (fp8 only, else None). ``k_pages``/``v_pages`` hold the paged layout
    [n_pages, page_size, Hkv, D] and ``block_table`` [n_seqs, max_pages] its
    page ids when the workload is paged. ``q32``/``k32``/``v32`` widen the
    storage values to float32 exactly (fp8 codes decoded, not scaled).
    """
    workload: Workload
    dtype: str
    seqlens: Tuple[int, ...]
    cu_seqlens: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_scale: Optional[np.ndarray] = None
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    k_pages: Optional[np.ndarray] = None
    v_pages: Optional[np.ndarray] = None
    block_table: Optional[np.ndarray] = None
    page_size: int = 0

    @property
    def max_seqlen(self) -> int:
        return max(self.seqlens) if self.seqlens else 0

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    def widen(self, a: np.ndarray) -> np.ndarray:
        if self.dtype == "f32":
            return a
        if self.dtype == "bf16":
            return bf16_to_f32(a)
        return fp8_e4m3_to_f32(a)

    @property
    def q32(self):
        return self.widen(self.q)

    @property
    def k32(self):
        return self.widen(self.k)

    @property
    def v32(self):
        return self.widen(self.v)


def _round_store(x32: np.ndarray, dtype: str, scale: Optional[float] = None) -> np.ndarray:
    """Round float32 values to their storage type."""
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return bf16_round(x32)
    if dtype == "fp8":
        return fp8_e4m3_quantize(x32.astype(np.float64) / float(scale))
    raise ValueError(dtype)


_STORE_DT = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}


def build_inputs(seqlens: Sequence[int], n_heads_q: int, n_heads_kv: int, head_dim: int, dtype: str,
                 rho: float = 0.99, n_vert: int = 0, code: int = 0, salt: int = 0,
                 paged: bool = False, page_size: int = 64, workload: Optional[Workload] = None,
                 sink_tokens: int = 4, sink_gain: float = 3.0, vert_gain: float = 2.0) -> Inputs:
    """Generate packed varlen inputs (any shape; the named workloads call this)."""
    seqlens = tuple(int(x) for x in seqlens)
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    T = int(cu[-1])
    G = n_heads_q // n_heads_kv
    D = head_dim
    # per sequence, per head float32 arrays (kept only until they are rounded)
    per_seq = []
    for s, L in enumerate(seqlens):
        qh, kh, vh = [], [], []
        for g in range(n_heads_kv):
            qs, k, v = gen_group(L, G, D, rho, n_vert, code, s, g, salt, sink_tokens, sink_gain, vert_gain)
            qh += qs
            kh.append(k)
            vh.append(v)
        per_seq.append((qh, kh, vh))
    scales = [None, None, None]
    if dtype == "fp8":
        for i, H in enumerate((n_heads_q, n_heads_kv, n_heads_kv)):
            amax = np.zeros(H)
            for parts in per_seq:
                for h, a in enumerate(parts[i]):
                    if a.size:
                        amax[h] = max(amax[h], float(np.abs(a).max()))
            scales[i] = np.maximum(amax / FP8_E4M3_MAX, np.finfo(np.float32).tiny).astype(np.float32)
    out = []
    for i, H in enumerate((n_heads_q, n_heads_kv, n_heads_kv)):
        dst = np.empty((T, H, D), dtype=_STORE_DT[dtype])
        for s, parts in enumerate(per_seq):
            heads = [_round_store(a, dtype, None if scales[i] is None else scales[i][h])
                     for h, a in enumerate(parts[i])]
            dst[cu[s]:cu[s + 1]] = np.stack(heads, axis=1) if heads and seqlens[s] > 0 else 0
            parts[i].clear()
        out.append(dst)
    w = workload
    if w is None:
        w = Workload(name="custom", seqlens=seqlens, n_heads_q=n_heads_q, n_heads_kv=n_heads_kv,
                     head_dim=head_dim, dtypes=(dtype,), block_q=0, block_k=0, lambdas=(), rho=rho,
                     n_vert=n_vert, paged=paged, page_size=page_size, code=code)
    inp = Inputs(workload=w, dtype=dtype, seqlens=seqlens, cu_seqlens=cu, q=out[0], k=out[1], v=out[2],
                 q_scale=scales[0], k_scale=scales[1], v_scale=scales[2])
    if paged:
        page_tensors(inp, page_size, code)
    return inp


def page_tensors(inp: Inputs, page_size: int, code: int = 0) -> None:
    """Scatter K/V into ``page_size``-token pages by a seeded random permutation.

    Logical page p of sequence s is stored at physical page
    ``block_table[s, p]``; slots past the end of a sequence and unused table
    entries hold zero.
    """
    n_pages_seq = [(L + page_size - 1) // page_size for L in inp.seqlens]
    P = int(sum(n_pages_seq))
    maxp = max(n_pages_seq) if n_pages_seq else 0
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, code, _P_PAGES, page_size])))
    perm = rng.permutation(P).astype(np.int32)
    table = np.zeros((len(inp.seqlens), max(1, maxp)), dtype=np.int32)
    Hkv, D = inp.k.shape[1], inp.k.shape[2]
    slots = np.empty(inp.total_tokens, dtype=np.int64)   # physical slot of every packed token
    off = 0
    for s, L in enumerate(inp.seqlens):
        table[s, : n_pages_seq[s]] = perm[off: off + n_pages_seq[s]]
        tok = np.arange(L)
        slots[inp.cu_seqlens[s]: inp.cu_seqlens[s + 1]] = table[s, tok // page_size].astype(np.int64) * page_size \
            + tok % page_size
        off += n_pages_seq[s]
    kp = np.zeros((max(1, P) * page_size, Hkv, D), dtype=inp.k.dtype)
    vp = np.zeros((max(1, P) * page_size, Hkv, D), dtype=inp.v.dtype)
    kp[slots] = inp.k
    vp[slots] = inp.v
    kp = kp.reshape(max(1, P), page_size, Hkv, D)
    vp = vp.reshape(max(1, P), page_size, Hkv, D)
    inp.k_pages, inp.v_pages, inp.block_table, inp.page_size = kp, vp, table, page_size


def make_workload(name: str, dtype: Optional[str] = None, salt: int = 0) -> Inputs:
    """Inputs of a named workload (``WORKLOADS``) for one of its dtypes."""
    w = WORKLOADS[name]
    dt = dtype or w.dtypes[0]
    if dt not in w.dtypes:
        raise ValueError(f"{name} is defined for dtypes {w.dtypes}, not {dt}")
    return build_inputs(seqlens_for(w), w.n_heads_q, w.n_heads_kv, w.head_dim, dt, rho=w.rho,
                        n_vert=w.n_vert, code=w.code, salt=salt, paged=w.paged, page_size=w.page_size,
                        workload=w, sink_tokens=w.sink_tokens, sink_gain=w.sink_gain, vert_gain=w.vert_gain)


def tile_count(L: int, block_q: int) -> int:
    return (L + block_q - 1) // block_q


def work_items(seqlens: Sequence[int], n_heads_q: int, block_q: int,
               heads: Optional[Sequence[int]] = None, tile_stride: int = 1,
               extra_tiles: Sequence[int] = ()) -> np.ndarray:
    """(seq, head, tile) triples as int32 [n, 3]. ``tile_stride`` > 1 keeps
    every n-th tile plus the first, last and any in ``extra_tiles`` (a
    deterministic sample for large workloads)."""
    hs = list(range(n_heads_q)) if heads is None else list(heads)
    out: List[Tuple[int, int, int]] = []
    for s, L in enumerate(seqlens):
        T = tile_count(L, block_q)
        if tile_stride <= 1:
            tiles = range(T)
        else:
            sel = set(range(0, T, tile_stride)) | {0, T - 1} | {t for t in extra_tiles if 0 <= t < T}
            tiles = sorted(x for x in sel if T > 0)
        for h in hs:
            for t in tiles:
                out.append((s, h, t))
    return np.asarray(out, dtype=np.int32).reshape(-1, 3)


def build_integer_inputs(seqlens: Sequence[int], n_heads_q: int, n_heads_kv: int, head_dim: int, dtype: str,
                         qk_range: int = 3, code: int = 0, paged: bool = False, page_size: int = 64,
                         sink_tokens: int = 4, sink_dims: int = 32) -> Inputs:
    """Inputs whose q and k are small integers, uniform in [-qk_range, qk_range]
    (v ~ N(0, 1)), stored as fp32 or bf16 (both exact for these values).
    Sink structure in integers: on the first ``sink_dims`` dims every query
    is positive (uniform in [1, qk_range]) and the first ``sink_tokens`` keys
    of each sequence hold +qk_range, so those keys score high for every
    query and many later blocks fall far below the running maximum.

    Every product q_i k_i is then an integer and every dot product is an
    integer well below 2^24, so fp32 accumulation (the GPU) and fp64 (the
    oracle) give the same exact scores. With head_dim 64 the score scale
    1/8 is a power of two, so a gap of g raw units is exactly g/8 in
    natural-log units: a threshold lambda = g/8 puts that gap exactly on it.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError("integer inputs are built for f32 and bf16 storage")
    seqlens = tuple(int(x) for x in seqlens)
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    T = int(cu[-1])
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, code, _P_HEAD, 0, 0, 77])))
    q = rng.integers(-qk_range, qk_range + 1, size=(T, n_heads_q, head_dim)).astype(np.float32)
    k = rng.integers(-qk_range, qk_range + 1, size=(T, n_heads_kv, head_dim)).astype(np.float32)
    v = rng.standard_normal((T, n_heads_kv, head_dim)).astype(np.float32)
    sd = min(sink_dims, head_dim)
    q[:, :, :sd] = rng.integers(1, qk_range + 1, size=(T, n_heads_q, sd))
    for s0, L in zip(cu[:-1], seqlens):
        k[s0: s0 + min(sink_tokens, L), :, :sd] = qk_range
    w = Workload(name="integer", seqlens=seqlens, n_heads_q=n_heads_q, n_heads_kv=n_heads_kv, head_dim=head_dim,
                 dtypes=(dtype,), block_q=0, block_k=0, lambdas=(), rho=0.0, n_vert=0, paged=paged,
                 page_size=page_size, code=code)
    inp = Inputs(workload=w, dtype=dtype, seqlens=seqlens, cu_seqlens=cu, q=_round_store(q, dtype),
                 k=_round_store(k, dtype), v=_round_store(v, dtype))
    if paged:
        page_tensors(inp, page_size, code)
    return inp
