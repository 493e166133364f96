"""Parity of the decoding entry point ``bsp_attn_decode`` with the oracle.

A decoding step appends one query row per sequence, which sees all of that
sequence's keys: the oracle's chunked-prefill case with one query row per
sequence (its pins: tests/test_oracle_pins.py). The GPU side is the
three-kernel split path (scores and block maxima, per-chunk decisions and PV,
combine). Same protocol and tolerances as tests/test_gpu_parity.py.
"""

import math

import numpy as np
import pytest

import synth
from tests import parity

pytestmark = pytest.mark.gpu

DECODE_SEQS = (1, 64, 65, 700, 2049, 333, 4100)


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


def _one_row_each(inp):
    return parity.Chunk(lq=(1,) * len(inp.seqlens))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("fp8", 128)], ids=["bf16_d128", "bf16_d64", "fp8"])
@pytest.mark.parametrize("heads", [(8, 2), (6, 2), (4, 4), (4, 2), (16, 2)], ids=["g4", "g3", "g1", "g2", "g8"])
@pytest.mark.parametrize("paged", [False, True], ids=["packed", "paged"])
def test_decode_small_cases(dtype, D, heads, paged):
    hq, hkv = heads
    inp = synth.build_inputs(DECODE_SEQS, hq, hkv, D, dtype, rho=0.97, n_vert=4, code=301 + hq, paged=paged,
                             page_size=64, sink_gain=6.0)
    dev = parity.to_device(inp)
    for bk in (128, 64, 96):
        _log(f"decode {dtype} D={D} heads={heads} paged={paged} block_k={bk}")
        reps = parity.check_case(inp, 64, bk, [math.inf, 3.0, 1.0, 0.0], paged=paged, dev=dev,
                                 chunk=_one_row_each(inp), decode=True)
        assert reps[0].n_skipped == 0 and reps[3].n_skipped > 0


def test_decode_lambda_per_sequence_and_counts():
    inp = synth.build_inputs(DECODE_SEQS, 8, 2, 128, "bf16", rho=0.97, n_vert=4, code=311, sink_gain=6.0)
    lam_seq = [math.inf, 0.5, 3.0, 1.0, math.inf, 2.0, 0.0]
    reps = parity.check_case(inp, 64, 128, [4.0], chunk=_one_row_each(inp), lam_seq=lam_seq, decode=True)
    assert reps[0].n_skipped > 0


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("paged", [False, True], ids=["packed", "paged"])
def test_decode_ablation_flags_against_the_oracle(dtype, paged):
    """The V-load and exponential switches (the guide's section 5, step 3) leave
    the decoding step's decisions and results unchanged: each flagged run is
    checked against the oracle, and against the unflagged run bit for bit."""
    import block_sparse_long_bsp_amd as bsp

    inp = synth.build_inputs(DECODE_SEQS, 8, 2, 128, dtype, rho=0.97, n_vert=4, code=312, sink_gain=6.0,
                             paged=paged, page_size=64)
    dev = parity.to_device(inp)
    chunk = _one_row_each(inp)
    outs = []
    for flags in (0, bsp.FLAG_LOAD_SKIPPED_V, bsp.FLAG_EXP_SKIPPED, bsp.FLAG_LOAD_SKIPPED_V | bsp.FLAG_EXP_SKIPPED):
        gpu = parity.run_gpu(inp, dev, 64, 128, 1.0, paged=paged, chunk=chunk, flags=flags, decode=True)
        rep = parity.compare(inp, gpu, 64, 128, 1.0, chunk=chunk)
        assert rep.ok(), f"flags={flags}: " + "; ".join(rep.problems)
        assert rep.n_skipped > 0
        outs.append(gpu)
    for other in outs[1:]:
        for key in ("o", "lse", "bits", "skip_count", "visited_count"):
            assert np.array_equal(outs[0][key], other[key], equal_nan=True), key


def test_decode_repeat_runs_are_bit_identical_and_workspace_reused():
    import torch

    import block_sparse_long_bsp_amd as bsp

    big = synth.build_inputs((5000, 300, 77), 8, 2, 128, "bf16", rho=0.97, n_vert=3, code=313, sink_gain=6.0)
    small = synth.build_inputs((129, 40), 8, 2, 128, "bf16", rho=0.97, n_vert=2, code=314, sink_gain=6.0)
    ws = torch.empty(bsp.decode_workspace_bytes(8, 2, 3, big.total_tokens, big.max_seqlen, 128, 128),
                     dtype=torch.uint8, device="cuda")
    for inp in (big, small):
        dev = parity.to_device(inp)
        q = dev["q"][torch.from_numpy(_one_row_each(inp).rows(inp)).cuda()].contiguous()
        runs = []
        for _ in range(2):
            r = bsp.decode(q, dev["k"], dev["v"], dev["cu"], inp.max_seqlen, block_k=128, lam=2.0, workspace=ws)
            torch.cuda.synchronize()
            runs.append([x.clone() for x in r])
        for a, b in zip(*runs):
            assert torch.equal(a, b)
        # and the shared workspace gave the oracle's answer
        parity.check_case(inp, 64, 128, [2.0], dev=dev, chunk=_one_row_each(inp), decode=True)


def test_decode_sequence_without_keys_writes_nothing():
    import torch

    import block_sparse_long_bsp_amd as bsp

    inp = synth.build_inputs((300, 77), 4, 2, 128, "bf16", rho=0.97, code=315)
    dev = parity.to_device(inp)
    # three sequences: the middle one has no keys
    cu = torch.tensor([0, 300, 300, 377], dtype=torch.int32, device="cuda")
    rows = torch.tensor([299, 0, 376], dtype=torch.int64, device="cuda")
    q = dev["q"][rows].contiguous()
    out = torch.full((3, 4, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    o, lse, bm, sc, vc = bsp.decode(q, dev["k"], dev["v"], cu, 300, block_k=128, lam=1.0, out=out)
    torch.cuda.synchronize()
    assert torch.all(o[1] == 7.0)
    assert torch.all(torch.isfinite(o[0].float())) and torch.all(torch.isfinite(o[2].float()))
    bits = bsp.unpack_bitmap(bm, 4, 3, 1, 1, 128, 300)
    assert not bits[:, 1].any()
    assert int(vc[0]) == 3 + 1  # blocks of the two sequences with keys, per query head


def _decode_workload(name, dtype, lams):
    w = synth.WORKLOADS[name]
    inp = synth.make_workload(name, dtype)
    _log(f"decode {name} {inp.dtype}: {len(inp.seqlens)} sequences, max {inp.max_seqlen} keys")
    reps = parity.check_case(inp, 64, w.block_k, lams, paged=w.paged, chunk=_one_row_each(inp), decode=True)
    for lam, r in zip(lams, reps):
        _log(f"  lambda={lam}: skipped {r.n_skipped}/{r.n_pairs} band flips {r.n_band_flips} "
             f"max-abs {r.max_abs:.3g} mean-abs {r.mean_abs:.3g} lse {r.lse_max:.3g}")
    return reps


def test_decode_after_llama8b_32k():
    reps = _decode_workload("llama8b_32k_bf16", None, [math.inf, 5.3, 3.0])
    assert reps[2].n_skipped > 0


def test_decode_after_varlen16_paged():
    _decode_workload("varlen16_paged_bf16", None, [math.inf, 5.3, 3.0])


def test_decode_after_llama8b_128k_fp8():
    _decode_workload("llama8b_128k", "fp8", [math.inf, 5.3])
