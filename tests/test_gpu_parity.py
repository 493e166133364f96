"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small cases run the full oracle over several tiles with ragged tails, empty
and single-token sequences, GQA, every compiled (head_dim, block_q, block_k)
instance, packed and paged K/V. The named workloads run at their full sizes
in the same launch configuration the benchmark uses, with the oracle on a
deterministic sample of (sequence, head, tile) work items. The exact
reductions (GQA == repeated-KV MHA, identity page table == packed, packed
varlen == separate sequences, bitwise repeatability) compare GPU outputs
bit for bit.
"""

import math
import os

import numpy as np
import pytest

import synth
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_bsp_amd as bsp

    bsp.load_library()
    yield


def _log(msg):
    print(msg, flush=True)


INSTANCES = [(64, 64, 64), (64, 128, 64), (64, 128, 128), (128, 64, 64), (128, 128, 64), (128, 128, 128)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("inst", INSTANCES, ids=lambda x: "d%d_q%d_k%d" % x)
@pytest.mark.parametrize("paged", [False, True], ids=["packed", "paged"])
def test_small_cases(dtype, inst, paged):
    D, bq, bk = inst
    seqlens = (300, 0, 129, 1, 64)
    page = 64 if bk >= 64 else bk
    # strong sink keys make many blocks skippable at small lambda for every tile shape
    inp = synth.build_inputs(seqlens, 4, 2, D, dtype, rho=0.95, n_vert=2, code=201, paged=paged, page_size=page,
                             sink_gain=6.0)
    _log(f"small case dtype={dtype} D={D} bq={bq} bk={bk} paged={paged}")
    reps = parity.check_case(inp, bq, bk, [math.inf, 2.0, 0.0], paged=paged)
    assert reps[0].n_skipped == 0
    assert reps[2].n_skipped > 0


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("block_q", [64, 128])
@pytest.mark.parametrize("paged", [False, True], ids=["packed", "paged"])
def test_key_halves_decided_apart(dtype, block_q, paged):
    """64-key blocks on 128-key blocks: the two halves of a block take their own decisions.

    The oracle's decisions on these inputs hold, among pairs of 64-key blocks
    (2i, 2i + 1) that a tile visits, both a kept block followed by a skipped one
    and a skipped block followed by a kept one, so the second half's vote is
    exercised both with and without the first half's maximum in the running
    max. The GPU bitmap must equal the oracle's (outside the decision band),
    with the counts. (fp8 with paged K/V runs the lockstep loop instead.)
    """
    import oracle

    inp = synth.build_inputs((700, 300, 129, 64), 4, 2, 128, dtype, rho=0.95, n_vert=2, code=215, sink_gain=6.0,
                             paged=paged, page_size=64)
    ref = oracle.run_inputs(inp, block_q, 64, 1.0, j_max=(inp.max_seqlen + 63) // 64)
    sk, vis = ref.skip.astype(bool), ref.visited.astype(bool)
    J = sk.shape[1] // 2 * 2
    both = vis[:, 0:J:2] & vis[:, 1:J:2]
    kept_then_skipped = int((both & ~sk[:, 0:J:2] & sk[:, 1:J:2]).sum())
    skipped_then_kept = int((both & sk[:, 0:J:2] & ~sk[:, 1:J:2]).sum())
    assert kept_then_skipped > 0 and skipped_then_kept > 0
    _log(f"key halves dtype={dtype} bq={block_q} paged={paged}: {kept_then_skipped} kept/skipped, "
         f"{skipped_then_kept} skipped/kept pairs")
    reps = parity.check_case(inp, block_q, 64, [2.0, 1.0], paged=paged)
    assert reps[1].n_skipped > 0


FP8_INSTANCES = [(128, 64, 64), (128, 128, 64), (128, 128, 128)]


@pytest.mark.parametrize("inst", FP8_INSTANCES, ids=lambda x: "d%d_q%d_k%d" % x)
@pytest.mark.parametrize("paged", [False, True], ids=["packed", "paged"])
@pytest.mark.parametrize("gqa", [(4, 2), (3, 1)], ids=["g2", "g3"])
def test_small_cases_fp8(inst, paged, gqa):
    D, bq, bk = inst
    Hq, Hkv = gqa
    seqlens = (300, 0, 129, 1, 64)
    inp = synth.build_inputs(seqlens, Hq, Hkv, D, "fp8", rho=0.95, n_vert=2, code=209, paged=paged, page_size=64,
                             sink_gain=6.0)
    _log(f"small case fp8 D={D} bq={bq} bk={bk} paged={paged} Hq={Hq} Hkv={Hkv}")
    reps = parity.check_case(inp, bq, bk, [math.inf, 2.0, 0.0], paged=paged)
    assert reps[0].n_skipped == 0
    assert reps[2].n_skipped > 0


@pytest.mark.parametrize("inst", [(64, 64, 64), (128, 64, 64), (128, 128, 64), (128, 128, 128)],
                         ids=lambda x: "d%d_q%d_k%d" % x)
@pytest.mark.parametrize("cache", [(False, 64), (True, 16), (True, 64)], ids=["packed", "paged16", "paged64"])
def test_small_cases_odd_group_bf16(inst, cache):
    """bf16 with three query heads per KV head: one query head per workgroup (the lockstep loop, in both modes),
    packed and paged; 16-token pages make the copies of 128-row tiles look their pages up per lane."""
    D, bq, bk = inst
    paged, page = cache
    seqlens = (300, 0, 129, 1, 64)
    inp = synth.build_inputs(seqlens, 3, 1, D, "bf16", rho=0.95, n_vert=2, code=216, paged=paged, page_size=page,
                             sink_gain=6.0)
    _log(f"small case bf16 odd group D={D} bq={bq} bk={bk} paged={paged} page={page}")
    reps = parity.check_case(inp, bq, bk, [math.inf, 2.0, 0.0], paged=paged)
    assert reps[0].n_skipped == 0
    assert reps[2].n_skipped > 0


@pytest.mark.parametrize("paged", [False, True], ids=["packed", "paged"])
def test_two_hundred_ragged_sequences(paged):
    """200 sequences of seeded random lengths in [0, 600] (zeros and single tokens among them) and 8 KV heads:
    the work-item decoding, heaviest tile first, over many sequences and the XCD-partitioned order, on every
    tile against the oracle."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([synth.BASE_SEED, 218])))
    seqlens = [int(x) for x in rng.integers(0, 601, 200)]
    seqlens[:4] = [0, 1, 600, 129]
    inp = synth.build_inputs(seqlens, 16, 8, 128, "bf16", rho=0.95, n_vert=2, code=218, paged=paged, page_size=64)
    _log(f"200 ragged sequences ({sum(seqlens)} tokens) paged={paged}")
    reps = parity.check_case(inp, 64, 64, [math.inf, 2.0], paged=paged)
    assert reps[1].n_skipped > 0


def test_xcd_mapping_with_eight_kv_heads():
    # 8 KV heads switch on the XCD-partitioned work order
    inp = synth.build_inputs((517, 130), 16, 8, 128, "bf16", rho=0.97, n_vert=4, code=202)
    _log("xcd mapping case")
    parity.check_case(inp, 128, 64, [math.inf, 3.0])


def test_paged_small_pages():
    inp = synth.build_inputs((200, 77), 4, 1, 128, "bf16", rho=0.97, code=203, paged=True, page_size=16)
    _log("paged page_size=16")
    parity.check_case(inp, 64, 64, [math.inf, 1.0], paged=True)


def test_single_1k_fp32_full():
    w = synth.WORKLOADS["single_1k_fp32"]
    inp = synth.make_workload(w.name)
    _log("single_1k_fp32")
    reps = parity.check_case(inp, w.block_q, w.block_k, list(w.lambdas))
    _log(f"  skipped {[r.n_skipped for r in reps]} of {reps[0].n_pairs}; max-abs {[r.max_abs for r in reps]}")


def _sampled(name, heads, tile_stride, dtype=None):
    w = synth.WORKLOADS[name]
    inp = synth.make_workload(name, dtype)
    work = synth.work_items(inp.seqlens, w.n_heads_q, w.block_q, heads=heads, tile_stride=tile_stride)
    _log(f"{name} {inp.dtype}: {work.shape[0]} sampled work items")
    reps = parity.check_case(inp, w.block_q, w.block_k, list(w.lambdas), paged=w.paged, work=work)
    for lam, r in zip(w.lambdas, reps):
        _log(f"  lambda={lam}: skipped {r.n_skipped}/{r.n_pairs} band flips {r.n_band_flips} "
             f"max-abs {r.max_abs:.3g} mean-abs {r.mean_abs:.3g} lse {r.lse_max:.3g}")
    return reps


def test_half_million_token_sequence_sampled():
    """One sequence of 2^19 tokens, four times the longest workload: the 64-bit row offsets of Q, O, K and V, the
    LSE and bitmap rows and the 4096-block tiles at sizes past those of the workloads. First, middle and last tile
    of both query heads, dense and at lambda 3."""
    L = 1 << 19
    inp = synth.build_inputs((L,), 2, 1, 128, "bf16", rho=0.998, n_vert=64, code=217)
    T = L // 128
    work = synth.work_items((L,), 2, 128, heads=[0, 1], tile_stride=T, extra_tiles=(T // 2,))
    _log(f"2^19-token sequence: {work.shape[0]} sampled work items")
    reps = parity.check_case(inp, 128, 128, [math.inf, 3.0], work=work)
    assert reps[1].n_skipped > 0
    _log(f"  lambda=3: skipped {reps[1].n_skipped}/{reps[1].n_pairs}, max-abs {reps[1].max_abs:.3g}")


def test_llama8b_8k_bf16_sampled():
    _sampled("llama8b_8k_bf16", heads=[0, 13, 31], tile_stride=7)


def test_llama8b_32k_bf16_sampled():
    # one query head of every KV head, every 8th tile (+ first and last)
    _sampled("llama8b_32k_bf16", heads=[0, 5, 10, 15, 16, 21, 26, 31], tile_stride=8)


def test_varlen16_paged_bf16_sampled():
    _sampled("varlen16_paged_bf16", heads=[5, 30], tile_stride=37)


# 128K: every 8th tile (+ first and last) of four query heads per dtype; between the
# two dtypes every KV head is covered
def test_llama8b_128k_bf16_sampled():
    _sampled("llama8b_128k", heads=[0, 9, 18, 27], tile_stride=8, dtype="bf16")


def test_llama8b_128k_fp8_sampled():
    reps = _sampled("llama8b_128k", heads=[5, 14, 23, 31], tile_stride=8, dtype="fp8")
    _log("fp8 decision flips vs the oracle: " + ", ".join(
        f"lambda={lam}: {r.n_flips_tight} within 1e-3, {r.n_flips_wide} in (1e-3, {parity.MARGIN_BAND['fp8']}]"
        for lam, r in zip(synth.WORKLOADS["llama8b_128k"].lambdas, reps)))


# ---- chunked prefill against a cached prefix (queries = the last Lq positions) --

CHUNK_SEQS = (300, 129, 77, 513, 40)


@pytest.mark.parametrize("dtype,inst", [("bf16", (128, 128, 128)), ("bf16", (128, 128, 64)), ("bf16", (64, 64, 64)),
                                        ("fp8", (128, 128, 128)), ("f32", (64, 64, 64))],
                         ids=lambda x: x if isinstance(x, str) else "d%d_q%d_k%d" % x)
@pytest.mark.parametrize("paged", [False, True], ids=["packed", "paged"])
def test_chunked_prefill(dtype, inst, paged):
    D, bq, bk = inst
    inp = synth.build_inputs(CHUNK_SEQS, 4, 2, D, dtype, rho=0.95, n_vert=2, code=210, paged=paged, page_size=64,
                             sink_gain=6.0)
    chunk = parity.Chunk(lq=(45, 129, 1, 200, 0))
    _log(f"chunked prefill dtype={dtype} D={D} bq={bq} bk={bk} paged={paged}")
    reps = parity.check_case(inp, bq, bk, [math.inf, 2.0, 0.0], paged=paged, chunk=chunk)
    assert reps[0].n_skipped == 0 and reps[2].n_skipped > 0


@pytest.mark.parametrize("paged", [False, True], ids=["packed", "paged"])
def test_decode_step_is_a_chunk_of_one(paged):
    # one new token per sequence against its whole context
    seqs = (1, 64, 65, 700, 2049, 333)
    inp = synth.build_inputs(seqs, 8, 2, 128, "bf16", rho=0.97, n_vert=4, code=211, paged=paged, page_size=64,
                             sink_gain=6.0)
    _log(f"decode step paged={paged}")
    reps = parity.check_case(inp, 64, 64, [math.inf, 3.0, 1.0], paged=paged, chunk=parity.Chunk(lq=(1,) * len(seqs)))
    assert reps[2].n_skipped > 0


def test_chunk_after_whole_tiles_equals_rows_of_full_prefill():
    # same tiles, same blocks, same decisions: the chunk's outputs equal the full
    # prefill's rows bit for bit
    import torch

    import block_sparse_long_bsp_amd as bsp

    L, P = 700, 256
    inp = synth.build_inputs((L,), 8, 2, 128, "bf16", rho=0.97, n_vert=3, code=212, sink_gain=6.0)
    dev = parity.to_device(inp)
    for lam in (math.inf, 2.0):
        o, lse, bm, sc, vc = bsp.fwd(dev["q"], dev["k"], dev["v"], dev["cu"], L, block_q=128, block_k=128, lam=lam)
        cuq = torch.tensor([0, L - P], dtype=torch.int32, device="cuda")
        o2, lse2, bm2, _, _ = bsp.fwd(dev["q"][P:].contiguous(), dev["k"], dev["v"], cuq, L - P, block_q=128,
                                      block_k=128, lam=lam, cu_seqlens_k=dev["cu"], max_seqlen_k=L)
        torch.cuda.synchronize()
        assert torch.equal(o[P:], o2)
        assert torch.equal(lse[:, P:], lse2)
        b1 = bsp.unpack_bitmap(bm, 8, 1, L, 128, 128)
        b2 = bsp.unpack_bitmap(bm2, 8, 1, L - P, 128, 128, L)
        assert np.array_equal(b1[:, :, P // 128:], b2)


def test_chunk8k_of_llama8b_32k_sampled():
    # the last 8K-token chunk of the 32K layer against its 24K-token cached prefix
    w = synth.WORKLOADS["llama8b_32k_bf16"]
    inp = synth.make_workload(w.name)
    chunk = parity.Chunk(lq=(8192,))
    work = synth.work_items([8192], w.n_heads_q, w.block_q, heads=[3, 28], tile_stride=13)
    _log(f"chunk 8K of 32K: {work.shape[0]} sampled work items")
    reps = parity.check_case(inp, w.block_q, w.block_k, list(w.lambdas), work=work, chunk=chunk)
    for lam, r in zip(w.lambdas, reps):
        _log(f"  lambda={lam}: skipped {r.n_skipped}/{r.n_pairs} max-abs {r.max_abs:.3g}")


# ---- lambda per sequence, counts per sequence, ablation switches --

@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("block", [64, 128])
def test_lambda_per_sequence(dtype, block):
    # bf16 and fp8 (group 2): the two-head ping-pong schedule in sparse mode, at block 64 on
    # 128-row tiles whose halves vote apart; the oracle skips 6 of 100 pairs at block 128
    D = 64 if dtype == "f32" else 128
    seqs = (300, 129, 77, 513)
    inp = synth.build_inputs(seqs, 4, 2, D, dtype, rho=0.95, n_vert=2, code=213, sink_gain=6.0)
    bq = bk = block
    _log(f"lambda per sequence dtype={dtype} block={bq}")
    reps = parity.check_case(inp, bq, bk, [7.0], lam_seq=[0.0, math.inf, 2.0, 0.5])
    assert reps[0].n_skipped > 0


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("paged", [False, True], ids=["packed", "paged"])
def test_ablation_flags_against_the_oracle(dtype, block, paged):
    """The guide's skip_value_load / skip_softmax_exp switches (section 5, step 3).

    Each switch puts back work for skipped blocks (their V load, their
    exponentials) and must leave the decisions and results unchanged: every
    flagged run is checked against the oracle with the parity protocol, and
    against the unflagged run bit for bit. bf16 and fp8 with a group of 2 run
    the two-head schedule (at block 64 as 64-key halves and 64-row half tiles
    of 128 x 128); fp32 runs its own kernel.
    """
    import torch

    import block_sparse_long_bsp_amd as bsp

    D = 64 if dtype == "f32" else 128
    inp = synth.build_inputs((700, 129), 4, 2, D, dtype, rho=0.97, n_vert=2, code=214, sink_gain=6.0, paged=paged,
                             page_size=64)
    dev = parity.to_device(inp)
    lam = 1.0
    outs = []
    for flags in (0, bsp.FLAG_LOAD_SKIPPED_V, bsp.FLAG_EXP_SKIPPED, bsp.FLAG_LOAD_SKIPPED_V | bsp.FLAG_EXP_SKIPPED):
        gpu = parity.run_gpu(inp, dev, block, block, lam, paged=paged, flags=flags)
        rep = parity.compare(inp, gpu, block, block, lam)
        assert rep.ok(), f"flags={flags}: " + "; ".join(rep.problems)
        _log(f"ablation dtype={dtype} block={block} paged={paged} flags={flags}: skipped {rep.n_skipped}/"
             f"{rep.n_pairs} max-abs {rep.max_abs:.3g}")
        assert rep.n_skipped > 0
        outs.append(gpu)
    for x in outs[1:]:
        for key in ("o", "lse", "bits", "skip_count", "visited_count"):
            assert np.array_equal(outs[0][key], x[key], equal_nan=True), key


def test_repeat_runs_are_bit_identical():
    import torch

    import block_sparse_long_bsp_amd as bsp

    inp = synth.build_inputs((700, 45), 8, 2, 128, "bf16", rho=0.97, code=204)
    dev = parity.to_device(inp)
    outs = []
    for _ in range(3):
        o, lse, bm, sc, vc = bsp.fwd(dev["q"], dev["k"], dev["v"], dev["cu"], inp.max_seqlen, block_q=128,
                                     block_k=64, lam=2.0)
        torch.cuda.synchronize()
        outs.append((o.clone(), lse.clone(), bm.clone(), sc.clone()))
    for x in outs[1:]:
        for a, b in zip(outs[0], x):
            assert torch.equal(a, b)


@pytest.mark.parametrize("block,hq,exact", [(64, 6, True), (64, 4, False), (64, 8, False), (128, 8, False)],
                         ids=["64_g3", "64_g2", "64_g4", "128_g4"])
def test_gqa_equals_repeated_kv_mha(block, hq, exact):
    """Sharing a KV head among the query heads of a group gives what copies of it give.

    With an odd group at 64 x 64 both calls run the one-head lockstep loop and
    must agree bit for bit. With an even group the GQA call runs the two-head
    schedule (at 64 x 64 on 128-row tiles whose 64-row halves vote apart) and
    the MHA call the one-head loop, which sums the row sums in another order:
    the decisions (exact maxima of the same scores) must still agree bit for
    bit, O and LSE to rounding.
    """
    import torch

    import block_sparse_long_bsp_amd as bsp

    # sink and vertical-line structure: the oracle skips blocks in every case at lambda 1.5
    # (group 2 at 64: 38 of 84; group 4 at 64: 73 of 168, at 128: 7 of 48), no gap within 0.02 of it
    inp = synth.build_inputs((333,), hq, 2, 128, "bf16", rho=0.97, n_vert=3, code=205, sink_gain=6.0)
    dev = parity.to_device(inp)
    a = bsp.fwd(dev["q"], dev["k"], dev["v"], dev["cu"], inp.max_seqlen, block_q=block, block_k=block, lam=1.5)
    kr = dev["k"].repeat_interleave(hq // 2, dim=1).contiguous()
    vr = dev["v"].repeat_interleave(hq // 2, dim=1).contiguous()
    b = bsp.fwd(dev["q"], kr, vr, dev["cu"], inp.max_seqlen, block_q=block, block_k=block, lam=1.5)
    torch.cuda.synchronize()
    assert int(a[3].sum()) > 0  # some blocks skipped
    if exact:
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        return
    for x, y in zip(a[2:], b[2:]):  # bitmap, skip and visited counts
        assert torch.equal(x, y)
    assert float((a[0].float() - b[0].float()).abs().max()) <= 2e-2
    assert float((a[1] - b[1]).abs().max()) <= 1e-4


def test_identity_block_table_equals_packed():
    import torch

    import block_sparse_long_bsp_amd as bsp

    L = 320
    inp = synth.build_inputs((L,), 4, 2, 128, "bf16", rho=0.97, code=206)
    dev = parity.to_device(inp)
    kp = dev["k"].view(L // 64, 64, 2, 128)
    vp = dev["v"].view(L // 64, 64, 2, 128)
    table = torch.arange(L // 64, dtype=torch.int32, device="cuda").view(1, -1)
    a = bsp.fwd(dev["q"], dev["k"], dev["v"], dev["cu"], L, block_q=64, block_k=64, lam=1.0)
    b = bsp.fwd(dev["q"], kp, vp, dev["cu"], L, block_table=table, block_q=64, block_k=64, lam=1.0)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_packed_varlen_equals_separate_calls():
    import torch

    import block_sparse_long_bsp_amd as bsp

    seqlens = (130, 0, 257, 64)
    inp = synth.build_inputs(seqlens, 4, 2, 128, "bf16", rho=0.97, code=207)
    dev = parity.to_device(inp)
    o, lse, bm, sc, vc = bsp.fwd(dev["q"], dev["k"], dev["v"], dev["cu"], max(seqlens), block_q=128, block_k=64,
                                 lam=2.0)
    cu = inp.cu_seqlens
    bits = bsp.unpack_bitmap(bm, 4, len(seqlens), max(seqlens), 128, 64)
    for s, L in enumerate(seqlens):
        if L == 0:
            assert not bits[:, s].any()
            continue
        a, b = int(cu[s]), int(cu[s + 1])
        one = torch.tensor([0, L], dtype=torch.int32, device="cuda")
        o1, l1, b1, _, _ = bsp.fwd(dev["q"][a:b], dev["k"][a:b], dev["v"][a:b], one, L, block_q=128, block_k=64,
                                   lam=2.0)
        torch.cuda.synchronize()
        assert torch.equal(o[a:b], o1)
        assert torch.equal(lse[:, a:b], l1)
        bits1 = bsp.unpack_bitmap(b1, 4, 1, L, 128, 64)
        T1, J1 = bits1.shape[2], bits1.shape[3]
        assert np.array_equal(bits[:, s, :T1, :J1], bits1[:, 0])


def test_repeated_calls_allocate_nothing_in_the_library():
    import torch

    import block_sparse_long_bsp_amd as bsp

    inp = synth.build_inputs((512,), 8, 2, 128, "bf16", rho=0.97, code=208)
    dev = parity.to_device(inp)
    o, lse, bm, sc, vc = bsp.fwd(dev["q"], dev["k"], dev["v"], dev["cu"], 512, block_q=128, block_k=128, lam=2.0)
    torch.cuda.synchronize()
    before = torch.cuda.mem_get_info()[0]
    for _ in range(200):
        bsp.fwd(dev["q"], dev["k"], dev["v"], dev["cu"], 512, block_q=128, block_k=128, lam=2.0, out=o, lse=lse,
                bitmap=bm, skip_count=sc, visited_count=vc)
    torch.cuda.synchronize()
    after = torch.cuda.mem_get_info()[0]
    assert before - after < (8 << 20)


def test_single_hip_runtime_in_process():
    import block_sparse_long_bsp_amd as bsp

    bsp.load_library()
    maps = open("/proc/self/maps").read()
    paths = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(paths) == 1, paths
