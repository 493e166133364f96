"""Python binding of ``libbsp_attn.so`` (causal block-sparse prefill attention
with dynamic block skipping, MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/bsp_attn.h``. PyTorch supplies
device memory and the current stream. There is no fallback: when the library
is missing or the device is not gfx950 the calls raise.

Method: page "长上下文推理加速方案部署实战：基于动态稀疏注意力机制的推理服务优化指南"
(deployment guide for a dynamic sparse attention kernel), sections 3.2, 3.3,
3.5 and 5 (steps 3 and 4).
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch  # must be imported before the library so both share one HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
# BSP_ATTN_LIB may point at another build of the same library (A/B measurements).
LIB_PATH = os.environ.get("BSP_ATTN_LIB") or os.path.join(_PKG, "libbsp_attn.so")

BSP_OK, BSP_ERR_INVALID_ARG, BSP_ERR_UNSUPPORTED, BSP_ERR_HIP, BSP_ERR_DEVICE = range(5)
BSP_F32, BSP_BF16, BSP_FP8_E4M3 = 0, 1, 2

EXPORTED = ("bsp_attn_fwd", "bsp_attn_fwd_ex", "bsp_attn_decode", "bsp_decode_workspace_bytes",
            "bsp_skip_bitmap_words", "bsp_skip_bitmap_words_kv", "bsp_status_string", "bsp_last_error_detail",
            "bsp_version", "bsp_validate_host", "bsp_attn_decode_noalloc")

# size of the static scratch array behind bsp_attn_decode_noalloc (BSP_DECODE_SCRATCH_BYTES)
DECODE_SCRATCH_BYTES = 96 << 20

# ablation switches of bsp_attn_fwd_ex (results unchanged, only the work done changes)
FLAG_LOAD_SKIPPED_V = 1  # copy V also for blocks every query head of the workgroup skips
FLAG_EXP_SKIPPED = 2     # compute (and drop) the exponentials of skipped blocks


class BspError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"bsp_attn_fwd failed: {status_string(status)} ({detail})")
        self.status = status
        self.detail = detail


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("stride_token", ctypes.c_int64),
                ("stride_head", ctypes.c_int64), ("scale", ctypes.c_void_p)]


class Seqs(ctypes.Structure):
    _fields_ = [("cu_seqlens", ctypes.c_void_p), ("n_seqs", ctypes.c_int32), ("max_seqlen", ctypes.c_int32),
                ("total_tokens", ctypes.c_int64)]


class BlockTable(ctypes.Structure):
    _fields_ = [("table", ctypes.c_void_p), ("max_pages_per_seq", ctypes.c_int32), ("page_size", ctypes.c_int32)]


class SkipOut(ctypes.Structure):
    _fields_ = [("bitmap", ctypes.c_void_p), ("bitmap_words", ctypes.c_int64), ("skip_count", ctypes.c_void_p),
                ("visited_count", ctypes.c_void_p)]


class Options(ctypes.Structure):
    _fields_ = [("cu_seqlens_k", ctypes.c_void_p), ("max_seqlen_k", ctypes.c_int32), ("lambda_per_seq", ctypes.c_void_p),
                ("skip_count_per_seq", ctypes.c_void_p), ("visited_count_per_seq", ctypes.c_void_p),
                ("flags", ctypes.c_uint32)]


class DecodeOptions(ctypes.Structure):
    _fields_ = [("lambda_per_seq", ctypes.c_void_p), ("skip_count_per_seq", ctypes.c_void_p),
                ("visited_count_per_seq", ctypes.c_void_p), ("flags", ctypes.c_uint32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python __graft_entry__.py` or "
                           "`python block_sparse_long_bsp_amd/build.py`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.bsp_attn_fwd.restype = ctypes.c_int
    lib.bsp_attn_fwd.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_float, P, P]
    lib.bsp_attn_fwd_ex.restype = ctypes.c_int
    lib.bsp_attn_fwd_ex.argtypes = lib.bsp_attn_fwd.argtypes + [P]
    lib.bsp_attn_decode.restype = ctypes.c_int
    lib.bsp_attn_decode.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_float, P, P, P, P, ctypes.c_int64]
    lib.bsp_attn_decode_noalloc.restype = ctypes.c_int
    lib.bsp_attn_decode_noalloc.argtypes = lib.bsp_attn_decode.argtypes[:-2]
    lib.bsp_decode_workspace_bytes.restype = ctypes.c_int64
    lib.bsp_decode_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int]
    lib.bsp_skip_bitmap_words.restype = ctypes.c_int64
    lib.bsp_skip_bitmap_words.argtypes = [ctypes.c_int] * 5
    lib.bsp_skip_bitmap_words_kv.restype = ctypes.c_int64
    lib.bsp_skip_bitmap_words_kv.argtypes = [ctypes.c_int] * 6
    lib.bsp_status_string.restype = ctypes.c_char_p
    lib.bsp_status_string.argtypes = [ctypes.c_int]
    lib.bsp_last_error_detail.restype = ctypes.c_char_p
    lib.bsp_last_error_detail.argtypes = []
    lib.bsp_version.restype = ctypes.c_int
    lib.bsp_version.argtypes = []
    lib.bsp_validate_host.restype = ctypes.c_int
    lib.bsp_validate_host.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_int64, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().bsp_status_string(int(status)).decode()


def last_error_detail() -> str:
    return load_library().bsp_last_error_detail().decode()


def skip_bitmap_words(n_heads_q: int, n_seqs: int, max_seqlen: int, block_q: int, block_k: int) -> int:
    return int(load_library().bsp_skip_bitmap_words(n_heads_q, n_seqs, max_seqlen, block_q, block_k))


def skip_bitmap_words_kv(n_heads_q: int, n_seqs: int, max_seqlen_q: int, max_seqlen_k: int, block_q: int,
                         block_k: int) -> int:
    return int(load_library().bsp_skip_bitmap_words_kv(n_heads_q, n_seqs, max_seqlen_q, max_seqlen_k, block_q,
                                                       block_k))


def validate_host(cu_seqlens_q, cu_seqlens_k=None, *, max_seqlen_q: int, max_seqlen_k: int = 0,
                  total_q: int = -1, total_k: int = -1, block_table=None, page_size: int = 0,
                  n_pages: int = 0) -> Tuple[int, str]:
    """``bsp_validate_host`` on host arrays (numpy int32 or sequences):
    returns (status, detail)."""
    import numpy as np

    lib = load_library()
    cq = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    ck = None if cu_seqlens_k is None else np.ascontiguousarray(cu_seqlens_k, dtype=np.int32)
    bt = None if block_table is None else np.ascontiguousarray(block_table, dtype=np.int32)
    if bt is not None and bt.ndim != 2:
        raise ValueError("block_table must be [n_seqs, max_pages_per_seq]")
    st = int(lib.bsp_validate_host(cq.ctypes.data, None if ck is None else ck.ctypes.data, len(cq) - 1,
                                   int(max_seqlen_q), int(max_seqlen_k), int(total_q), int(total_k),
                                   None if bt is None else bt.ctypes.data, 0 if bt is None else bt.shape[1],
                                   int(page_size), int(n_pages)))
    return st, last_error_detail() if st != BSP_OK else ""


def _check_index_tensor(name: str, x: Optional[torch.Tensor], device, ndim: int) -> None:
    """Descriptor arrays go to the kernels as raw int32 pointers: anything else
    would be read as other values (e.g. int64 as pairs of int32)."""
    if x is None:
        return
    if x.dtype != torch.int32 or not x.is_contiguous() or x.device != device or x.dim() != ndim:
        raise ValueError(f"{name} must be a contiguous {ndim}-d torch.int32 tensor on {device}")


def fwd_raw(q: Tensor, k: Tensor, v: Tensor, o: Tensor, lse_ptr: int, seqs: Seqs, block_table: Optional[BlockTable],
            n_heads_q: int, n_heads_kv: int, head_dim: int, block_q: int, block_k: int, lam: float,
            skip_out: Optional[SkipOut], stream_ptr: int, options: Optional[Options] = None) -> int:
    """Direct call of the C entry point (``bsp_attn_fwd``, or ``bsp_attn_fwd_ex``
    when options are given) with prepared descriptors; returns the status."""
    lib = load_library()
    bt = ctypes.byref(block_table) if block_table is not None else None
    so = ctypes.byref(skip_out) if skip_out is not None else None
    args = (ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(o), ctypes.c_void_p(lse_ptr or None),
            ctypes.byref(seqs), bt, n_heads_q, n_heads_kv, head_dim, block_q, block_k, ctypes.c_float(lam), so,
            ctypes.c_void_p(stream_ptr or None))
    if options is None:
        return int(lib.bsp_attn_fwd(*args))
    return int(lib.bsp_attn_fwd_ex(*args, ctypes.byref(options)))


_DT = {torch.float32: BSP_F32, torch.bfloat16: BSP_BF16}
if hasattr(torch, "float8_e4m3fn"):
    _DT[torch.float8_e4m3fn] = BSP_FP8_E4M3


def _desc(x: torch.Tensor, scale: Optional[torch.Tensor] = None) -> Tensor:
    if x.dim() != 3:
        raise ValueError("expected a [tokens, heads, head_dim] tensor")
    if x.stride(2) != 1:
        raise ValueError("head_dim must be contiguous")
    if x.dtype not in _DT:
        raise ValueError(f"unsupported dtype {x.dtype}")
    # the stride of a dimension of size 1 is arbitrary (views from unsqueeze or
    # [:, None] carry 0): never used for addressing, so pass a dense one
    sh = x.stride(1) if x.shape[1] > 1 else x.shape[2]
    st = x.stride(0) if x.shape[0] > 1 else x.shape[1] * sh
    return Tensor(x.data_ptr(), _DT[x.dtype], st, sh, scale.data_ptr() if scale is not None else None)


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int, *,
        block_table: Optional[torch.Tensor] = None, page_size: int = 64, block_q: int = 128, block_k: int = 128,
        lam: float = math.inf, q_scale: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
        v_scale: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None, bitmap: Optional[torch.Tensor] = None,
        skip_count: Optional[torch.Tensor] = None, visited_count: Optional[torch.Tensor] = None,
        want_bitmap: bool = True, want_lse: bool = True, cu_seqlens_k: Optional[torch.Tensor] = None,
        max_seqlen_k: Optional[int] = None, lam_per_seq: Optional[torch.Tensor] = None,
        seq_skip_count: Optional[torch.Tensor] = None, seq_visited_count: Optional[torch.Tensor] = None,
        flags: int = 0) -> Tuple[torch.Tensor, ...]:
    """Block-sparse causal prefill attention on the current stream.

    q [Tq, Hq, D]; k, v [Tk, Hkv, D] packed, or paged [n_pages, page_size, Hkv, D]
    with ``block_table`` int32 [n_seqs, max_pages]. cu_seqlens int32 [n_seqs+1]
    on the device. Returns (o, lse, bitmap, skip_count, visited_count); the
    optional outputs are None when not requested. Output buffers may be passed
    in to avoid allocation.

    Options (``bsp_attn_fwd_ex``): ``cu_seqlens_k`` (device int32, with
    ``max_seqlen_k``) gives each sequence Lk >= Lq keys of which its queries
    are the last Lq (chunked prefill against a cached prefix; Lq = 1 is a
    decoding step); ``lam_per_seq`` (device float32 [n_seqs]) replaces ``lam``
    per sequence; ``seq_skip_count`` / ``seq_visited_count`` (device int64
    [n_seqs], filled in place) count skipped / visited pairs per sequence;
    ``flags`` holds the FLAG_* ablation switches.
    """
    load_library()
    if q.device.type != "cuda":
        raise ValueError("q must be a device tensor")
    T, Hq, D = q.shape
    _check_index_tensor("cu_seqlens", cu_seqlens, q.device, 1)
    _check_index_tensor("block_table", block_table, q.device, 2)
    paged = block_table is not None
    if paged:
        if k.dim() != 4:
            raise ValueError("paged k/v must be [n_pages, page_size, Hkv, D]")
        page_size = k.shape[1]
        k3 = k.view(k.shape[0] * k.shape[1], k.shape[2], k.shape[3])
        v3 = v.view(v.shape[0] * v.shape[1], v.shape[2], v.shape[3])
    else:
        k3, v3 = k, v
    Hkv = k3.shape[1]
    n_seqs = cu_seqlens.numel() - 1
    use_ex = (cu_seqlens_k is not None or lam_per_seq is not None or seq_skip_count is not None
              or seq_visited_count is not None or flags != 0)
    max_k = int(max_seqlen_k) if cu_seqlens_k is not None else int(max_seqlen)
    odt = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    if out is None:
        out = torch.empty((T, Hq, D), dtype=odt, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    words = skip_bitmap_words_kv(Hq, n_seqs, max_seqlen, max_k, block_q, block_k) if n_seqs > 0 else 0
    if want_bitmap and bitmap is None:
        bitmap = torch.empty((max(words, 1),), dtype=torch.int32, device=q.device)
    if skip_count is None:
        skip_count = torch.empty((Hq,), dtype=torch.int64, device=q.device)
    if visited_count is None:
        visited_count = torch.empty((Hq,), dtype=torch.int64, device=q.device)
    seqs = Seqs(cu_seqlens.data_ptr(), n_seqs, int(max_seqlen), T)
    bt = BlockTable(block_table.data_ptr(), block_table.shape[1], page_size) if paged else None
    so = SkipOut(bitmap.data_ptr() if bitmap is not None else None, bitmap.numel() if bitmap is not None else 0,
                 skip_count.data_ptr(), visited_count.data_ptr())
    stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = None
    if use_ex:
        for name, x, dt in (("cu_seqlens_k", cu_seqlens_k, torch.int32), ("lam_per_seq", lam_per_seq, torch.float32),
                            ("seq_skip_count", seq_skip_count, torch.int64),
                            ("seq_visited_count", seq_visited_count, torch.int64)):
            if x is not None and (x.dtype != dt or not x.is_contiguous() or x.device != q.device):
                raise ValueError(f"{name} must be a contiguous {dt} tensor on {q.device}")
        opts = Options(cu_seqlens_k.data_ptr() if cu_seqlens_k is not None else None, max_k,
                       lam_per_seq.data_ptr() if lam_per_seq is not None else None,
                       seq_skip_count.data_ptr() if seq_skip_count is not None else None,
                       seq_visited_count.data_ptr() if seq_visited_count is not None else None, int(flags))
    st = fwd_raw(_desc(q, q_scale), _desc(k3, k_scale), _desc(v3, v_scale), _desc(out), lse.data_ptr() if lse is not None else 0,
                 seqs, bt, Hq, Hkv, D, block_q, block_k, float(lam), so, stream, opts)
    if st != BSP_OK:
        raise BspError(st, last_error_detail())
    return out, lse, bitmap, skip_count, visited_count


def decode_workspace_bytes(n_heads_q: int, n_heads_kv: int, n_seqs: int, total_k: int, max_seqlen_k: int,
                           head_dim: int, block_k: int) -> int:
    return int(load_library().bsp_decode_workspace_bytes(n_heads_q, n_heads_kv, n_seqs, total_k, max_seqlen_k,
                                                         head_dim, block_k))


def _decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_k: int, *,
            total_k: Optional[int] = None, block_table: Optional[torch.Tensor] = None, block_k: int = 128,
            lam: float = math.inf, q_scale: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
            v_scale: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, bitmap: Optional[torch.Tensor] = None,
            skip_count: Optional[torch.Tensor] = None, visited_count: Optional[torch.Tensor] = None,
            want_bitmap: bool = True, want_lse: bool = True, lam_per_seq: Optional[torch.Tensor] = None,
            seq_skip_count: Optional[torch.Tensor] = None, seq_visited_count: Optional[torch.Tensor] = None,
            flags: int = 0, workspace: Optional[torch.Tensor] = None,
            noalloc: bool = False) -> Tuple[torch.Tensor, ...]:
    """One decoding step (``bsp_attn_decode``) on the current stream.

    q [n_seqs, Hq, D]: each sequence's new query row, which sees all of its
    keys; k, v packed [total_k, Hkv, D] or paged [n_pages, page_size, Hkv, D]
    with ``block_table``; cu_seqlens_k int32 [n_seqs+1] on the device (the
    key counts include the new token). ``total_k`` is cu_seqlens_k[-1]
    (rows of the score workspace; for packed K/V it defaults to k's rows).
    Returns (o, lse, bitmap, skip_count, visited_count); the bitmap rows are
    [Hq, n_seqs, 1, J] in the layout of ``unpack_bitmap``. ``workspace``
    (uint8, at least ``decode_workspace_bytes`` bytes) may be passed in to
    avoid an allocation.
    """
    load_library()
    if q.device.type != "cuda":
        raise ValueError("q must be a device tensor")
    n_seqs, Hq, D = q.shape
    _check_index_tensor("cu_seqlens_k", cu_seqlens_k, q.device, 1)
    _check_index_tensor("block_table", block_table, q.device, 2)
    paged = block_table is not None
    if paged:
        if k.dim() != 4:
            raise ValueError("paged k/v must be [n_pages, page_size, Hkv, D]")
        page_size = k.shape[1]
        k3 = k.view(k.shape[0] * k.shape[1], k.shape[2], k.shape[3])
        v3 = v.view(v.shape[0] * v.shape[1], v.shape[2], v.shape[3])
        if total_k is None:
            raise ValueError("paged decoding needs total_k (= cu_seqlens_k[-1])")
    else:
        k3, v3 = k, v
        if total_k is None:
            total_k = k.shape[0]
    Hkv = k3.shape[1]
    if out is None:
        out = torch.empty((n_seqs, Hq, D), dtype=torch.bfloat16, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((Hq, n_seqs), dtype=torch.float32, device=q.device)
    words = skip_bitmap_words_kv(Hq, n_seqs, 1, max_seqlen_k, 1, block_k) if n_seqs > 0 else 0
    if want_bitmap and bitmap is None:
        bitmap = torch.empty((max(words, 1),), dtype=torch.int32, device=q.device)
    if skip_count is None:
        skip_count = torch.empty((Hq,), dtype=torch.int64, device=q.device)
    if visited_count is None:
        visited_count = torch.empty((Hq,), dtype=torch.int64, device=q.device)
    need = decode_workspace_bytes(Hq, Hkv, n_seqs, int(total_k), int(max_seqlen_k), D, block_k)
    if need < 0:
        raise ValueError("invalid decode sizes")
    if workspace is None and not noalloc:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=q.device)
    for name, x, dt in (("cu_seqlens_k", cu_seqlens_k, torch.int32), ("lam_per_seq", lam_per_seq, torch.float32),
                        ("seq_skip_count", seq_skip_count, torch.int64),
                        ("seq_visited_count", seq_visited_count, torch.int64)):
        if x is not None and (x.dtype != dt or not x.is_contiguous() or x.device != q.device):
            raise ValueError(f"{name} must be a contiguous {dt} tensor on {q.device}")
    seqs = Seqs(cu_seqlens_k.data_ptr(), n_seqs, int(max_seqlen_k), int(total_k))
    bt = BlockTable(block_table.data_ptr(), block_table.shape[1], page_size) if paged else None
    so = SkipOut(bitmap.data_ptr() if bitmap is not None else None, bitmap.numel() if bitmap is not None else 0,
                 skip_count.data_ptr(), visited_count.data_ptr())
    opts = DecodeOptions(lam_per_seq.data_ptr() if lam_per_seq is not None else None,
                         seq_skip_count.data_ptr() if seq_skip_count is not None else None,
                         seq_visited_count.data_ptr() if seq_visited_count is not None else None, int(flags))
    stream = torch.cuda.current_stream(q.device).cuda_stream
    lib = load_library()
    args = (ctypes.byref(_desc(q, q_scale)), ctypes.byref(_desc(k3, k_scale)), ctypes.byref(_desc(v3, v_scale)),
            ctypes.byref(_desc(out)), ctypes.c_void_p(lse.data_ptr() if lse is not None else None), ctypes.byref(seqs),
            ctypes.byref(bt) if bt is not None else None, Hq, Hkv, D, block_k, ctypes.c_float(float(lam)),
            ctypes.byref(so), ctypes.c_void_p(stream or None), ctypes.byref(opts))
    if noalloc:
        st = int(lib.bsp_attn_decode_noalloc(*args))
    else:
        st = int(lib.bsp_attn_decode(*args, ctypes.c_void_p(workspace.data_ptr()),
                                     ctypes.c_int64(workspace.numel() * workspace.element_size())))
    if st != BSP_OK:
        raise BspError(st, last_error_detail())
    return out, lse, bitmap, skip_count, visited_count


def decode(q, k, v, cu_seqlens_k, max_seqlen_k, **kw) -> Tuple[torch.Tensor, ...]:
    """One decoding step through ``bsp_attn_decode`` (keyword arguments of
    ``_decode``; ``workspace`` may be passed in to avoid an allocation)."""
    return _decode(q, k, v, cu_seqlens_k, max_seqlen_k, **kw)


def decode_noalloc(q, k, v, cu_seqlens_k, max_seqlen_k, **kw) -> Tuple[torch.Tensor, ...]:
    """One decoding step through ``bsp_attn_decode_noalloc``: the library takes
    the step's workspace from its static per-GPU scratch array instead of a
    caller's buffer (at most ``DECODE_SCRATCH_BYTES``; calls that overlap in
    time on one GPU race). The C call allocates nothing; pass every output
    tensor (out, lse, bitmap, counts) to keep this function from allocating
    them."""
    if "workspace" in kw:
        raise ValueError("decode_noalloc takes no workspace")
    return _decode(q, k, v, cu_seqlens_k, max_seqlen_k, noalloc=True, **kw)


def unpack_bitmap(bitmap: torch.Tensor, n_heads_q: int, n_seqs: int, max_seqlen: int, block_q: int,
                  block_k: int, max_seqlen_k: Optional[int] = None):
    """Host-side view of the bitmap as a bool numpy array [Hq, n_seqs, T_max, J_max]."""
    import numpy as np

    T = (max_seqlen + block_q - 1) // block_q
    J = ((max_seqlen if max_seqlen_k is None else max_seqlen_k) + block_k - 1) // block_k
    W = (J + 31) // 32
    words = bitmap[: n_heads_q * n_seqs * T * W].cpu().numpy().view(np.uint32).reshape(n_heads_q, n_seqs, T, W)
    bits = ((words[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(bool)
    return bits.reshape(n_heads_q, n_seqs, T, W * 32)[..., :J]
