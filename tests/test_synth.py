"""Checks of the seeded input generator (storage rounding, layout, determinism)."""

import math

import numpy as np
import pytest

import synth


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = 2.0 ** -7  # bf16 spacing at 1.0
    vals = np.array([1.0, 1.0 + ulp / 2, 1.0 + 1.5 * ulp, 1.0 + ulp / 4, -2.5, 3.0e38], np.float32)
    got = synth.bf16_to_f32(synth.bf16_round(vals))
    # halfway cases go to the even mantissa: 1+ulp/2 -> 1, 1+1.5ulp -> 1+2ulp
    assert got[0] == one
    assert got[1] == one
    assert got[2] == np.float32(1.0 + 2 * ulp)
    assert got[3] == one
    assert got[4] == np.float32(-2.5)
    # round trip of representable values is exact
    x = synth.bf16_to_f32(synth.bf16_round(np.random.default_rng(0).standard_normal(1000).astype(np.float32)))
    assert np.array_equal(synth.bf16_to_f32(synth.bf16_round(x)), x)


def test_fp8_e4m3_table_and_rounding():
    t = synth.fp8_e4m3_decode_table()
    assert np.nanmax(t) == 448.0 and np.nanmin(t) == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x01] == 2.0 ** -9  # smallest subnormal
    assert t[0x08] == 2.0 ** -6  # smallest normal
    assert t[0x38] == 1.0
    assert np.sum(np.isfinite(t)) == 254
    # ties: 1 + 1/16 lies halfway between 1 (mantissa 0) and 1.125 (mantissa 1) -> 1
    c = synth.fp8_e4m3_quantize(np.array([1.0625, 1.1875, 500.0, -1e9, 2.0 ** -10, 0.0, -0.0]))
    assert t[c[0]] == 1.0
    assert t[c[1]] == 1.25  # halfway between 1.125 (odd) and 1.25 (even)
    assert t[c[2]] == 448.0 and t[c[3]] == -448.0
    assert t[c[4]] == 0.0  # 2^-10 is half of the smallest subnormal -> even (0)
    # every finite code round-trips
    finite = np.nonzero(np.isfinite(t))[0]
    assert np.array_equal(t[synth.fp8_e4m3_quantize(t[finite])], t[finite])


def test_generator_is_deterministic_and_structured():
    a = synth.build_inputs((300, 50), 4, 2, 16, "bf16", rho=0.99, n_vert=3, code=7)
    b = synth.build_inputs((300, 50), 4, 2, 16, "bf16", rho=0.99, n_vert=3, code=7)
    c = synth.build_inputs((300, 50), 4, 2, 16, "bf16", rho=0.99, n_vert=3, code=8)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    assert not np.array_equal(a.q, c.q)
    assert a.q.dtype == np.uint16 and a.q.shape == (350, 4, 16) and a.k.shape == (350, 2, 16)
    assert list(a.cu_seqlens) == [0, 300, 350]
    # sink keys carry the group's mean query direction: strongly positive scores
    q = a.q32[:300].astype(np.float64)
    k = a.k32[:300].astype(np.float64)
    sink = (q[:, 0:2, :] @ k[0, 0, :]).mean()
    other = (q[:, 0:2, :] @ k[100:200, 0, :].T).mean()
    assert sink > other


def test_paged_layout_round_trips():
    inp = synth.build_inputs((130, 64, 5), 2, 1, 8, "f32", code=9, paged=True, page_size=64)
    cu = inp.cu_seqlens
    assert sorted(inp.block_table[inp.block_table >= 0].ravel().tolist())[:1] == [0]
    for s, L in enumerate(inp.seqlens):
        for tok in range(L):
            p, o = divmod(tok, 64)
            phys = inp.block_table[s, p]
            assert np.array_equal(inp.k_pages[phys, o], inp.k[cu[s] + tok])
            assert np.array_equal(inp.v_pages[phys, o], inp.v[cu[s] + tok])
    used = [inp.block_table[s, p] for s, L in enumerate(inp.seqlens) for p in range((L + 63) // 64)]
    assert sorted(used) == list(range(len(used)))


def test_named_workloads_have_expected_shapes():
    w = synth.WORKLOADS["varlen16_paged_bf16"]
    lens = synth.seqlens_for(w)
    assert len(lens) == 16 and min(lens) >= 512 and max(lens) <= 32768
    assert synth.seqlens_for(w) == lens
    assert synth.WORKLOADS["llama8b_32k_bf16"].seqlens == (32768,)
    small = synth.make_workload("single_1k_fp32")
    assert small.q.dtype == np.float32 and small.q.shape == (1024, 1, 64)
