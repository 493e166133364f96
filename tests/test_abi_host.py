"""Host-only checks of the C ABI (no GPU needed).

The library must load, export every function declared in include/bsp_attn.h,
compute the bitmap size, and reject invalid arguments with the documented
status before touching the device (validation runs before any HIP call, so
fake device addresses are never dereferenced here).
"""

import ctypes
import math
import os
import re
import subprocess

import pytest

import block_sparse_long_bsp_amd as bsp
from block_sparse_long_bsp_amd import BlockTable, Seqs, SkipOut, Tensor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsp_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bsp.LIB_PATH):
        from block_sparse_long_bsp_amd import build

        build.build()
    return bsp.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsp_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert "bsp_attn_fwd" in names
    assert set(names) == set(bsp.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", bsp.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (bsp_[a-z_]+)\b", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_header_compiles_as_c():
    src = '#include "bsp_attn.h"\nint main(void){ return (int)sizeof(bsp_tensor_t) > 0 ? 0 : 1; }\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-x", "c", "-",
                        "-o", os.devnull], input=src, text=True, capture_output=True)
    assert r.returncode == 0, r.stderr


def test_struct_layouts_match_the_header():
    # offsets of the ctypes mirrors against the C compiler's view of the header
    prog = r'''
#include <stdio.h>
#include <stddef.h>
#include "bsp_attn.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu\n", sizeof(bsp_tensor_t), offsetof(bsp_tensor_t, dtype),
         offsetof(bsp_tensor_t, stride_token), offsetof(bsp_tensor_t, stride_head), offsetof(bsp_tensor_t, scale), (size_t)0);
  printf("%zu %zu %zu %zu %zu %zu\n", sizeof(bsp_seqs_t), offsetof(bsp_seqs_t, n_seqs), offsetof(bsp_seqs_t, max_seqlen),
         offsetof(bsp_seqs_t, total_tokens), sizeof(bsp_block_table_t), offsetof(bsp_block_table_t, page_size));
  printf("%zu %zu %zu %zu %zu %zu\n", sizeof(bsp_skip_out_t), offsetof(bsp_skip_out_t, bitmap_words),
         offsetof(bsp_skip_out_t, skip_count), offsetof(bsp_skip_out_t, visited_count), (size_t)0, (size_t)0);
  printf("%zu %zu %zu %zu %zu %zu\n", sizeof(bsp_fwd_options_t), offsetof(bsp_fwd_options_t, max_seqlen_k),
         offsetof(bsp_fwd_options_t, lambda_per_seq), offsetof(bsp_fwd_options_t, skip_count_per_seq),
         offsetof(bsp_fwd_options_t, visited_count_per_seq), offsetof(bsp_fwd_options_t, flags));
  printf("%zu %zu %zu %zu %zu %zu\n", sizeof(bsp_decode_options_t), offsetof(bsp_decode_options_t, lambda_per_seq),
         offsetof(bsp_decode_options_t, skip_count_per_seq), offsetof(bsp_decode_options_t, visited_count_per_seq),
         offsetof(bsp_decode_options_t, flags), (size_t)0);
  return 0;
}
'''
    exe = os.path.join("/tmp", "bsp_layout_%d" % os.getpid())
    r = subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), "-x", "c", "-", "-o", exe], input=prog,
                       text=True, capture_output=True)
    assert r.returncode == 0, r.stderr
    vals = [list(map(int, ln.split())) for ln in subprocess.run([exe], capture_output=True, text=True).stdout.split("\n") if ln]
    os.unlink(exe)
    assert vals[0][:5] == [ctypes.sizeof(Tensor), Tensor.dtype.offset, Tensor.stride_token.offset,
                           Tensor.stride_head.offset, Tensor.scale.offset]
    assert vals[1] == [ctypes.sizeof(Seqs), Seqs.n_seqs.offset, Seqs.max_seqlen.offset, Seqs.total_tokens.offset,
                       ctypes.sizeof(BlockTable), BlockTable.page_size.offset]
    assert vals[2][:4] == [ctypes.sizeof(SkipOut), SkipOut.bitmap_words.offset, SkipOut.skip_count.offset,
                           SkipOut.visited_count.offset]
    O = bsp.Options
    assert vals[3] == [ctypes.sizeof(O), O.max_seqlen_k.offset, O.lambda_per_seq.offset, O.skip_count_per_seq.offset,
                       O.visited_count_per_seq.offset, O.flags.offset]
    DO = bsp.DecodeOptions
    assert vals[4][:5] == [ctypes.sizeof(DO), DO.lambda_per_seq.offset, DO.skip_count_per_seq.offset,
                           DO.visited_count_per_seq.offset, DO.flags.offset]


def test_bitmap_words_formula(lib):
    # rows of ceil(ceil(L/bk)/32) words per (head, seq, tile)
    assert bsp.skip_bitmap_words(32, 1, 32768, 128, 128) == 32 * 256 * 8
    assert bsp.skip_bitmap_words(32, 1, 131072, 128, 128) == 32 * 1024 * 32
    assert bsp.skip_bitmap_words(1, 1, 1024, 64, 64) == 16
    assert bsp.skip_bitmap_words(4, 3, 100, 64, 64) == 4 * 3 * 2 * 1
    assert bsp.skip_bitmap_words(0, 1, 10, 64, 64) == 0
    assert bsp.skip_bitmap_words(1, 1, 0, 64, 64) == 0


def test_status_strings(lib):
    assert bsp.status_string(0) == "ok"
    assert "invalid" in bsp.status_string(1)
    assert "unsupported" in bsp.status_string(2)
    assert bsp.status_string(99) == "unknown status"
    assert lib.bsp_version() >= 100


FAKE = 0x10000  # 16-byte aligned address that is never dereferenced here


def _call(**over):
    """A valid-looking bf16 call with fake device addresses, with overrides."""
    D = over.pop("head_dim", 128)
    Hq = over.pop("n_heads_q", 32)
    Hkv = over.pop("n_heads_kv", 8)
    q = over.pop("q", Tensor(FAKE, bsp.BSP_BF16, Hq * D, D, None))
    k = over.pop("k", Tensor(FAKE, bsp.BSP_BF16, Hkv * D, D, None))
    v = over.pop("v", Tensor(FAKE, bsp.BSP_BF16, Hkv * D, D, None))
    o = over.pop("o", Tensor(FAKE, bsp.BSP_BF16, Hq * D, D, None))
    seqs = over.pop("seqs", Seqs(FAKE, 1, 256, 256))
    bt = over.pop("bt", None)
    bq = over.pop("block_q", 128)
    bk = over.pop("block_k", 128)
    lam = over.pop("lam", 4.0)
    so = over.pop("so", SkipOut(FAKE, bsp.skip_bitmap_words(Hq, 1, 256, bq, bk), FAKE, FAKE))
    assert not over
    return bsp.fwd_raw(q, k, v, o, FAKE, seqs, bt, Hq, Hkv, D, bq, bk, lam, so, 0)


@pytest.mark.parametrize("case,expect", [
    (dict(lam=float("nan")), bsp.BSP_ERR_INVALID_ARG),
    (dict(lam=-0.5), bsp.BSP_ERR_INVALID_ARG),
    (dict(n_heads_q=30), bsp.BSP_ERR_INVALID_ARG),
    (dict(n_heads_kv=0), bsp.BSP_ERR_INVALID_ARG),
    (dict(q=Tensor(0, bsp.BSP_BF16, 4096, 128, None)), bsp.BSP_ERR_INVALID_ARG),
    (dict(q=Tensor(FAKE + 2, bsp.BSP_BF16, 4096, 128, None)), bsp.BSP_ERR_INVALID_ARG),
    (dict(k=Tensor(FAKE, bsp.BSP_BF16, 1028, 128, None)), bsp.BSP_ERR_INVALID_ARG),
    (dict(k=Tensor(FAKE, bsp.BSP_F32, 1024, 128, None)), bsp.BSP_ERR_INVALID_ARG),
    (dict(o=Tensor(FAKE, bsp.BSP_F32, 4096, 128, None)), bsp.BSP_ERR_INVALID_ARG),
    (dict(q=Tensor(FAKE, 7, 4096, 128, None)), bsp.BSP_ERR_INVALID_ARG),
    (dict(seqs=Seqs(0, 1, 256, 256)), bsp.BSP_ERR_INVALID_ARG),
    (dict(seqs=Seqs(FAKE, -1, 256, 256)), bsp.BSP_ERR_INVALID_ARG),
    (dict(so=SkipOut(FAKE, 10, None, None)), bsp.BSP_ERR_INVALID_ARG),
    (dict(bt=BlockTable(FAKE, 4, 48)), bsp.BSP_ERR_INVALID_ARG),       # not a power of two
    (dict(bt=BlockTable(FAKE, 1, 64)), bsp.BSP_ERR_INVALID_ARG),       # too few pages for max_seqlen
    (dict(bt=BlockTable(0, 4, 64)), bsp.BSP_ERR_INVALID_ARG),
    (dict(head_dim=96, q=Tensor(FAKE, bsp.BSP_BF16, 32 * 96, 96, None), k=Tensor(FAKE, bsp.BSP_BF16, 8 * 96, 96, None),
          v=Tensor(FAKE, bsp.BSP_BF16, 8 * 96, 96, None), o=Tensor(FAKE, bsp.BSP_BF16, 32 * 96, 96, None)),
     bsp.BSP_ERR_UNSUPPORTED),
    (dict(block_q=64, block_k=128), bsp.BSP_ERR_UNSUPPORTED),
    (dict(block_q=32, block_k=32), bsp.BSP_ERR_UNSUPPORTED),
])
def test_invalid_arguments_rejected_before_the_device(lib, case, expect):
    st = _call(**case)
    assert st == expect, (st, bsp.last_error_detail())
    assert bsp.last_error_detail() != ""


def test_fp8_requires_scales(lib):
    t = lambda: Tensor(FAKE, bsp.BSP_FP8_E4M3, 4096, 128, None)
    kv = lambda: Tensor(FAKE, bsp.BSP_FP8_E4M3, 1024, 128, None)
    st = _call(q=t(), k=kv(), v=kv())
    assert st == bsp.BSP_ERR_INVALID_ARG


def test_bitmap_words_with_separate_key_lengths(lib):
    # rows per (head, seq, query tile); words per row from the key length
    assert bsp.skip_bitmap_words_kv(32, 2, 1, 4096, 64, 64) == 32 * 2 * 1 * 2
    assert bsp.skip_bitmap_words_kv(4, 1, 300, 300, 128, 64) == bsp.skip_bitmap_words(4, 1, 300, 128, 64)
    assert bsp.skip_bitmap_words_kv(4, 1, 10, -1, 64, 64) == 0


def _call_ex(opts, **over):
    D, Hq, Hkv = 128, 32, 8
    q = Tensor(FAKE, bsp.BSP_BF16, Hq * D, D, None)
    kv = Tensor(FAKE, bsp.BSP_BF16, Hkv * D, D, None)
    o = Tensor(FAKE, bsp.BSP_BF16, Hq * D, D, None)
    seqs = Seqs(FAKE, 1, 256, 256)
    so = over.pop("so", SkipOut(FAKE, bsp.skip_bitmap_words(Hq, 1, 256, 128, 128), FAKE, FAKE))
    return bsp.fwd_raw(q, kv, kv, o, FAKE, seqs, over.pop("bt", None), Hq, Hkv, D, 128, 128, 2.0, so, 0, opts)


@pytest.mark.parametrize("opts,expect", [
    (bsp.Options(None, 0, None, None, None, 4), bsp.BSP_ERR_INVALID_ARG),            # unknown flag bit
    (bsp.Options(FAKE, -1, None, None, None, 0), bsp.BSP_ERR_INVALID_ARG),           # negative max_seqlen_k
    (bsp.Options(FAKE + 2, 512, None, None, None, 0), bsp.BSP_ERR_INVALID_ARG),      # misaligned cu_seqlens_k
    (bsp.Options(None, 0, FAKE + 1, None, None, 0), bsp.BSP_ERR_INVALID_ARG),        # misaligned lambda array
    (bsp.Options(None, 0, None, FAKE + 4, None, 0), bsp.BSP_ERR_INVALID_ARG),        # misaligned counts
    (bsp.Options(FAKE, 8192, None, None, None, 0), bsp.BSP_ERR_INVALID_ARG),         # bitmap sized for 256 keys
])
def test_extended_options_rejected_before_the_device(lib, opts, expect):
    st = _call_ex(opts)
    assert st == expect, (st, bsp.last_error_detail())
    assert bsp.last_error_detail() != ""


def test_fp8_head_dim_64_is_unsupported(lib):
    D = 64
    t = lambda H: Tensor(FAKE, bsp.BSP_FP8_E4M3, H * D, D, FAKE)
    st = _call(head_dim=D, q=t(32), k=t(8), v=t(8), o=Tensor(FAKE, bsp.BSP_BF16, 32 * D, D, None))
    assert st == bsp.BSP_ERR_UNSUPPORTED, bsp.last_error_detail()


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib

    r = subprocess.run(["python", "-c", "import block_sparse_long_bsp_amd as b; b.load_library('/nonexistent/lib.so')"],
                       capture_output=True, text=True, cwd=ROOT)
    assert r.returncode != 0 and "missing" in r.stderr


# ------------------------------------------------------------------ decoding step

def test_decode_workspace_bytes(lib):
    # scores [Hkv][total_k][G padded to 1/2/4/8] + block maxima [Hq][n_seqs][J]
    # + partials [Hq][n_seqs][chunks][D+1], 256-byte aligned parts
    n = bsp.decode_workspace_bytes(32, 8, 1, 32768, 32768, 128, 128)
    J = 256
    chunks = 64  # groups of 4 blocks (one per wave): 1 x 8 x 64 work items
    assert n == 8 * 32768 * 4 * 4 + 32 * J * 4 + 32 * chunks * 129 * 4
    # three query heads per KV head store their scores padded to four
    assert bsp.decode_workspace_bytes(24, 8, 1, 4096, 4096, 128, 128) == (8 * 4096 * 4 * 4 + 24 * 32 * 4
                                                                           + 24 * 8 * 129 * 4)
    # many sequences: blocks are grouped so that about 2048 work items remain
    n16 = bsp.decode_workspace_bytes(32, 8, 16, 16 * 20000, 32768, 128, 128)
    assert n16 >= 32 * 16 * 20000 * 4 + 32 * 16 * 256 * 4
    assert bsp.decode_workspace_bytes(32, 8, 1, 100, 100, 128, 0) == -1
    assert bsp.decode_workspace_bytes(0, 8, 1, 100, 100, 128, 128) == -1


def _call_dec(**over):
    D, Hq, Hkv = over.pop("D", 128), over.pop("Hq", 32), over.pop("Hkv", 8)
    dt = over.pop("dtype", bsp.BSP_BF16)
    scale = over.pop("scale", None)
    q = Tensor(FAKE, dt, Hq * D, D, scale)
    kv = Tensor(FAKE, dt, Hkv * D, D, scale)
    o = over.pop("o", Tensor(FAKE, bsp.BSP_BF16, Hq * D, D, None))
    seqs = over.pop("seqs", Seqs(FAKE, 2, 4096, 5000))
    bt = over.pop("bt", None)
    bk = over.pop("block_k", 128)
    lam = over.pop("lam", 3.0)
    need = bsp.decode_workspace_bytes(Hq, Hkv, seqs.n_seqs, seqs.total_tokens, seqs.max_seqlen, D, bk)
    ws = over.pop("ws", FAKE)
    ws_bytes = over.pop("ws_bytes", need)
    so = over.pop("so", SkipOut(FAKE, bsp.skip_bitmap_words_kv(Hq, seqs.n_seqs, 1, seqs.max_seqlen, 1, bk), FAKE, FAKE))
    opts = over.pop("opts", None)
    assert not over
    return int(lib_handle().bsp_attn_decode(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(kv), ctypes.byref(o),
                                            ctypes.c_void_p(FAKE), ctypes.byref(seqs),
                                            ctypes.byref(bt) if bt is not None else None, Hq, Hkv, D, bk,
                                            ctypes.c_float(lam), ctypes.byref(so), None,
                                            ctypes.byref(opts) if opts is not None else None,
                                            ctypes.c_void_p(ws), ctypes.c_int64(ws_bytes)))


def lib_handle():
    return bsp.load_library()


@pytest.mark.parametrize("case,expect", [
    (dict(ws=0), bsp.BSP_ERR_INVALID_ARG),                               # no workspace
    (dict(ws_bytes=1024), bsp.BSP_ERR_INVALID_ARG),                      # too small
    (dict(ws=FAKE + 16), bsp.BSP_ERR_INVALID_ARG),                       # not 256-byte aligned
    (dict(lam=-1.0), bsp.BSP_ERR_INVALID_ARG),
    (dict(block_k=0), bsp.BSP_ERR_INVALID_ARG),
    (dict(Hq=30), bsp.BSP_ERR_INVALID_ARG),
    (dict(seqs=Seqs(0, 2, 4096, 5000)), bsp.BSP_ERR_INVALID_ARG),
    (dict(so=SkipOut(FAKE, 3, None, None)), bsp.BSP_ERR_INVALID_ARG),    # bitmap too small
    (dict(bt=BlockTable(FAKE, 2, 64)), bsp.BSP_ERR_INVALID_ARG),         # pages cannot hold max_seqlen
    (dict(bt=BlockTable(FAKE, 64, 48)), bsp.BSP_ERR_INVALID_ARG),        # page size not a power of two
    (dict(o=Tensor(FAKE, bsp.BSP_F32, 32 * 128, 128, None)), bsp.BSP_ERR_INVALID_ARG),
    (dict(dtype=bsp.BSP_F32, o=Tensor(FAKE, bsp.BSP_F32, 32 * 128, 128, None)), bsp.BSP_ERR_UNSUPPORTED),
    (dict(dtype=bsp.BSP_FP8_E4M3), bsp.BSP_ERR_INVALID_ARG),             # fp8 without scales
    (dict(dtype=bsp.BSP_FP8_E4M3, scale=FAKE, D=64, o=Tensor(FAKE, bsp.BSP_BF16, 32 * 64, 64, None)),
     bsp.BSP_ERR_UNSUPPORTED),
    (dict(Hq=80, Hkv=8, o=Tensor(FAKE, bsp.BSP_BF16, 80 * 128, 128, None)), bsp.BSP_ERR_UNSUPPORTED),  # 10 heads per KV head
    (dict(opts=bsp.DecodeOptions(None, None, None, 8)), bsp.BSP_ERR_INVALID_ARG),   # unknown flag
    (dict(opts=bsp.DecodeOptions(FAKE + 2, None, None, 0)), bsp.BSP_ERR_INVALID_ARG),
])
def test_decode_invalid_arguments_rejected_before_the_device(lib, case, expect):
    st = _call_dec(**case)
    assert st == expect, (st, bsp.last_error_detail())
    assert bsp.last_error_detail() != ""


# ---- bsp_validate_host: the checks BSP_DEBUG_VALIDATE applies to copies of a call's device descriptors

def test_validate_host_accepts_good_descriptors(lib):
    cu = [0, 300, 300, 429]
    assert bsp.validate_host(cu, max_seqlen_q=300, total_q=429) == (bsp.BSP_OK, "")
    # chunked: keys >= queries per sequence
    assert bsp.validate_host([0, 45, 45, 46], [0, 300, 300, 429], max_seqlen_q=45, max_seqlen_k=300, total_q=46,
                             total_k=429)[0] == bsp.BSP_OK
    table = [[3, 1, 0, 0, 0], [0, 0, 0, 0, 0], [2, 4, 0, 0, 0]]  # 64-token pages; unused entries are not read
    assert bsp.validate_host(cu, max_seqlen_q=300, block_table=table, page_size=128, n_pages=5)[0] == bsp.BSP_OK


@pytest.mark.parametrize("kw,needle", [
    (dict(cu_seqlens_q=[1, 300, 429], max_seqlen_q=300), "must be 0"),
    (dict(cu_seqlens_q=[0, 300, 200, 429], max_seqlen_q=300), "decreases at sequence 1"),
    (dict(cu_seqlens_q=[0, 300, 429], max_seqlen_q=200), "above the stated maximum"),
    (dict(cu_seqlens_q=[0, 300, 429], max_seqlen_q=300, total_q=500), "states 500 tokens"),
    (dict(cu_seqlens_q=[0, 45, 100], cu_seqlens_k=[0, 300, 350], max_seqlen_q=55, max_seqlen_k=300),
     "has 55 queries but only 50 keys"),
    (dict(cu_seqlens_q=[0, 45], cu_seqlens_k=[0, 300], max_seqlen_q=45, max_seqlen_k=200), "cu_seqlens_k"),
    (dict(cu_seqlens_q=[0, 300, 429], max_seqlen_q=300, block_table=[[0, 1], [2, 3]], page_size=128, n_pages=8),
     "needs 3 pages"),
    (dict(cu_seqlens_q=[0, 300, 429], max_seqlen_q=300, block_table=[[0, 1, 2], [3, -1, 0]], page_size=128,
          n_pages=8), "block_table[1][1] = -1"),
    (dict(cu_seqlens_q=[0, 300, 429], max_seqlen_q=300, block_table=[[0, 1, 2], [3, 8, 0]], page_size=128,
          n_pages=8), "block_table[1][1] = 8"),
])
def test_validate_host_rejects_bad_descriptors(lib, kw, needle):
    st, detail = bsp.validate_host(**kw)
    assert st == bsp.BSP_ERR_INVALID_ARG
    assert needle in detail, detail


def test_validate_host_reads_only_pages_in_use(lib):
    # entries past a sequence's ceil(len / page) pages are never read, whatever they hold
    table = [[0, 1, 2, 99999], [3, 4, -7, -7]]
    assert bsp.validate_host([0, 300, 429], max_seqlen_q=300, block_table=table, page_size=128,
                             n_pages=5)[0] == bsp.BSP_OK


def test_decode_noalloc_rejects_calls_beyond_its_scratch_before_the_device(lib):
    # 8 KV heads x 4 query heads x 4 bytes of scores per key: 10M keys need ~640 MB, above the static array
    Hq, Hkv, D, bk = 32, 8, 128, 128
    seqs = Seqs(FAKE, 2, 4096, 10_000_000)
    need = bsp.decode_workspace_bytes(Hq, Hkv, seqs.n_seqs, seqs.total_tokens, seqs.max_seqlen, D, bk)
    assert need > bsp.DECODE_SCRATCH_BYTES
    q = Tensor(FAKE, bsp.BSP_BF16, Hq * D, D, None)
    kv = Tensor(FAKE, bsp.BSP_BF16, Hkv * D, D, None)
    o = Tensor(FAKE, bsp.BSP_BF16, Hq * D, D, None)
    so = SkipOut(FAKE, bsp.skip_bitmap_words_kv(Hq, 2, 1, 4096, 1, bk), FAKE, FAKE)
    st = int(lib.bsp_attn_decode_noalloc(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(kv), ctypes.byref(o),
                                         ctypes.c_void_p(FAKE), ctypes.byref(seqs), None, Hq, Hkv, D, bk,
                                         ctypes.c_float(3.0), ctypes.byref(so), None, None))
    assert st == bsp.BSP_ERR_INVALID_ARG
    assert "static scratch" in bsp.last_error_detail()
    # the header's constant and the binding's agree
    text = open(HEADER).read()
    assert "#define BSP_DECODE_SCRATCH_BYTES (96LL << 20)" in text and bsp.DECODE_SCRATCH_BYTES == 96 << 20
