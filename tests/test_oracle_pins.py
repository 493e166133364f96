"""Pins for the CPU oracle (``oracle/``) against things other than itself.

The method (page "长上下文推理加速方案部署实战：基于动态稀疏注意力机制的推理服务优化指南",
sections 3.2 and 6.1) prints no worked numbers, so the oracle is pinned by:

* a closed form: with lambda = +inf nothing is skipped and the result must be
  naive dense causal softmax attention (written here with numpy matmuls);
* an invariant: the exported probabilities of every row sum to 1 and are
  exactly 0 on skipped blocks and masked keys;
* brute force: for lambda >= 0 a skipped block can never raise the running
  maximum (its local maximum is below running max - lambda), so the running
  maximum before block j equals the dense prefix maximum of the block maxima
  and the skip set has the closed form
      skip(t, j)  <=>  min_{rows r of t} ( max_{j'<j} M[r, j'] - M[r, j] ) > lambda;
  enumerated here from a dense score matrix;
* the kept-key closed form: given the skip set, O and LSE equal softmax
  attention restricted to the kept keys;
* hand-derived worked examples (``tests/golden/worked_examples.json``),
  including ties at gap == lambda (strict rule) and the tile-wide minimum;
* reductions: GQA == MHA with repeated K/V heads; packed varlen == separate
  sequences; forced all-keep == dense; error bound vs dense; monotonicity.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


# ---------------------------------------------------------------- helpers --

def dense_scores(q, k, cu, hq, hkv):
    """Per (seq, head): fp64 scaled causal score matrix (-inf above diagonal)."""
    D = q.shape[2]
    G = hq // hkv
    out = {}
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        L = b - a
        mask = np.triu(np.ones((L, L), dtype=bool), 1)
        for h in range(hq):
            S = (q[a:b, h, :].astype(np.float64) @ k[a:b, h // G, :].astype(np.float64).T) / math.sqrt(D)
            S[mask] = -np.inf
            out[(s, h)] = S
    return out


def naive_dense(q, k, v, cu, hq, hkv, keep=None):
    """Naive softmax attention. ``keep[(s,h)]`` optionally masks out keys
    (boolean [L, L]); returns O [T, Hq, D], LSE [Hq, T]."""
    T, D = q.shape[0], q.shape[2]
    G = hq // hkv
    O = np.zeros((T, hq, D))
    LSE = np.zeros((hq, T))
    S_all = dense_scores(q, k, cu, hq, hkv)
    for (s, h), S in S_all.items():
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        if keep is not None:
            S = np.where(keep[(s, h)], S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        P = np.exp(S - m)
        l = P.sum(axis=1, keepdims=True)
        O[a:b, h] = (P @ v[a:b, h // G, :].astype(np.float64)) / l
        LSE[h, a:b] = (m + np.log(l))[:, 0]
    return O, LSE


def brute_force_skips(q, k, cu, hq, hkv, bq, bk, lam):
    """Closed-form skip set {(s, h, t, j)} and visited set, from dense scores."""
    skips, visited = set(), set()
    for (s, h), S in dense_scores(q, k, cu, hq, hkv).items():
        L = S.shape[0]
        if L == 0:
            continue
        J = (L + bk - 1) // bk
        M = np.full((L, J), -np.inf)
        for j in range(J):
            M[:, j] = S[:, j * bk: min(L, (j + 1) * bk)].max(axis=1)
        for t in range((L + bq - 1) // bq):
            r0, r1 = t * bq, min(L, (t + 1) * bq)
            diag = (r1 - 1) // bk
            for j in range(diag + 1):
                visited.add((s, h, t, j))
                prefix = M[r0:r1, :j].max(axis=1) if j > 0 else np.full(r1 - r0, -np.inf)
                loc = M[r0:r1, j]
                gaps = []
                for pm, lm in zip(prefix, loc):
                    if lm == -np.inf:
                        gaps.append(np.inf)
                    elif pm == -np.inf:
                        gaps.append(-np.inf)
                    else:
                        gaps.append(pm - lm)
                if min(gaps) > lam:
                    skips.add((s, h, t, j))
    return skips, visited


def oracle_sets(res):
    sk, vi = set(), set()
    for w, (s, h, t) in enumerate(res.work):
        for j in np.nonzero(res.skip[w])[0]:
            sk.add((int(s), int(h), int(t), int(j)))
        for j in np.nonzero(res.visited[w])[0]:
            vi.add((int(s), int(h), int(t), int(j)))
    return sk, vi


def keep_mask_from(skips, cu, hq, bq, bk):
    keep = {}
    for s in range(len(cu) - 1):
        L = int(cu[s + 1] - cu[s])
        for h in range(hq):
            keep[(s, h)] = np.ones((L, L), dtype=bool)
    for (s, h, t, j) in skips:
        L = int(cu[s + 1] - cu[s])
        keep[(s, h)][t * bq: min(L, (t + 1) * bq), j * bk: min(L, (j + 1) * bk)] = False
    return keep


def small_inputs(seqlens, hq, hkv, D, rho=0.95, n_vert=2, salt=0, code=101):
    return synth.build_inputs(seqlens, hq, hkv, D, "f32", rho=rho, n_vert=n_vert, code=code, salt=salt)


CASES = [
    # seqlens, Hq, Hkv, D, bq, bk
    ((70,), 1, 1, 8, 16, 16),
    ((129,), 2, 1, 16, 32, 16),
    ((100, 1, 33, 0, 64), 4, 2, 8, 16, 32),
    ((96,), 4, 4, 32, 32, 32),
    ((65, 17), 2, 2, 8, 8, 16),
]


# ----------------------------------------------------------------- tests --

@pytest.mark.parametrize("case", CASES)
def test_dense_limit_equals_naive_softmax(case):
    seqlens, hq, hkv, D, bq, bk = case
    inp = small_inputs(seqlens, hq, hkv, D)
    res = oracle.run_inputs(inp, bq, bk, math.inf)
    assert res.skip.sum() == 0
    O, LSE = oracle.scatter(res, inp.cu_seqlens, hq)
    O_ref, LSE_ref = naive_dense(inp.q32, inp.k32, inp.v32, inp.cu_seqlens, hq, hkv)
    np.testing.assert_allclose(O, O_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE, LSE_ref, rtol=1e-14, atol=1e-12)


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("lam", [0.0, 0.5, 2.0, 4.0])
def test_skip_set_matches_brute_force(case, lam):
    seqlens, hq, hkv, D, bq, bk = case
    inp = small_inputs(seqlens, hq, hkv, D, salt=1)
    res = oracle.run_inputs(inp, bq, bk, lam)
    got_skip, got_vis = oracle_sets(res)
    ref_skip, ref_vis = brute_force_skips(inp.q32, inp.k32, inp.cu_seqlens, hq, hkv, bq, bk, lam)
    assert got_vis == ref_vis
    assert got_skip == ref_skip
    # the brute force must be exercising skips somewhere in this suite
    if lam == 0.0:
        assert len(ref_skip) > 0


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("lam", [0.0, 1.0, 3.0])
def test_kept_key_closed_form(case, lam):
    seqlens, hq, hkv, D, bq, bk = case
    inp = small_inputs(seqlens, hq, hkv, D, salt=2)
    res = oracle.run_inputs(inp, bq, bk, lam)
    skips, _ = oracle_sets(res)
    keep = keep_mask_from(skips, inp.cu_seqlens, hq, bq, bk)
    O_ref, LSE_ref = naive_dense(inp.q32, inp.k32, inp.v32, inp.cu_seqlens, hq, hkv, keep=keep)
    O, LSE = oracle.scatter(res, inp.cu_seqlens, hq)
    np.testing.assert_allclose(O, O_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE, LSE_ref, rtol=1e-14, atol=1e-12)


@pytest.mark.parametrize("lam", [0.0, 1.5, math.inf])
def test_probabilities_sum_to_one_and_reproduce_output(lam):
    seqlens, hq, hkv, D, bq, bk = (90, 40), 2, 1, 16, 16, 16
    inp = small_inputs(seqlens, hq, hkv, D, salt=3)
    res = oracle.run_inputs(inp, bq, bk, lam, export_p=True)
    cu = inp.cu_seqlens
    n_skipped_entries = 0
    for w, (s, h, t) in enumerate(res.work):
        L = int(cu[s + 1] - cu[s])
        r0, r1 = t * bq, min(L, (t + 1) * bq)
        P = res.p[w, : r1 - r0, :L]
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        for r in range(r1 - r0):
            assert np.all(P[r, r0 + r + 1:] == 0.0)  # causal mask
        for j in np.nonzero(res.skip[w])[0]:
            blk = P[:, j * bk: min(L, (j + 1) * bk)]
            assert np.all(blk == 0.0)
            n_skipped_entries += blk.size
        # O = P V over the sequence's keys
        V = inp.v32[cu[s]: cu[s + 1], h // (hq // hkv), :].astype(np.float64)
        np.testing.assert_allclose(res.o[w, : r1 - r0], P @ V, rtol=0, atol=1e-12)
    if lam == 0.0:
        assert n_skipped_entries > 0


def test_block_zero_never_skipped_and_output_finite():
    inp = small_inputs((200,), 2, 1, 16, salt=4)
    res = oracle.run_inputs(inp, 32, 16, 0.0)
    assert np.all(res.skip[:, 0] == 0)
    assert np.all(res.visited[:, 0] == 1)
    O, LSE = oracle.scatter(res, inp.cu_seqlens, 2)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(LSE))
    assert res.skip.sum() > 0


def test_skip_sets_are_monotone_in_lambda():
    inp = small_inputs((160,), 2, 2, 16, salt=5)
    prev = None
    for lam in [0.0, 0.25, 1.0, 2.0, 4.0, 8.0, math.inf]:
        sk, _ = oracle_sets(oracle.run_inputs(inp, 16, 16, lam))
        if prev is not None:
            assert sk <= prev
        prev = sk


@pytest.mark.parametrize("lam", [0.5, 2.0, 5.0])
def test_error_bound_against_dense(lam):
    seqlens, hq, hkv, D, bq, bk = (150,), 2, 1, 16, 16, 16
    inp = small_inputs(seqlens, hq, hkv, D, salt=6)
    res = oracle.run_inputs(inp, bq, bk, lam)
    O, LSE = oracle.scatter(res, inp.cu_seqlens, hq)
    Od, LSEd = naive_dense(inp.q32, inp.k32, inp.v32, inp.cu_seqlens, hq, hkv)
    skips, _ = oracle_sets(res)
    vmax = np.abs(inp.v32).max()
    L = seqlens[0]
    for h in range(hq):
        nd = np.zeros(L)
        for (s, hh, t, j) in skips:
            if hh != h:
                continue
            for r in range(t * bq, min(L, (t + 1) * bq)):
                nd[r] += max(0, min(r + 1, (j + 1) * bk, L) - j * bk)
        x = nd * math.exp(-lam)
        d_lse = LSEd[h] - LSE[h]
        assert np.all(d_lse >= -1e-12)
        assert np.all(d_lse <= np.log1p(x) + 1e-12)
        d_o = np.abs(Od[:, h] - O[:, h]).max(axis=1)
        assert np.all(d_o <= 2 * vmax * x / (1 + x) + 1e-12)


def test_gqa_equals_repeated_mha():
    inp = small_inputs((120,), 4, 2, 16, salt=7)
    G = 2
    k_rep = np.repeat(inp.k32, G, axis=1)
    v_rep = np.repeat(inp.v32, G, axis=1)
    for lam in [1.0, math.inf]:
        a = oracle.run(inp.q32, inp.k32, inp.v32, inp.cu_seqlens, 4, 2, 16, 16, lam)
        b = oracle.run(inp.q32, k_rep, v_rep, inp.cu_seqlens, 4, 4, 16, 16, lam)
        assert np.array_equal(a.skip, b.skip)
        assert np.array_equal(a.o, b.o)
        assert np.array_equal(a.lse, b.lse, equal_nan=True)


def test_varlen_equals_separate_sequences():
    seqlens = (50, 0, 77, 3)
    inp = small_inputs(seqlens, 2, 1, 8, salt=8)
    lam = 1.0
    packed = oracle.run_inputs(inp, 16, 16, lam)
    Op, Lp = oracle.scatter(packed, inp.cu_seqlens, 2)
    cu = inp.cu_seqlens
    for s, L in enumerate(seqlens):
        if L == 0:
            continue
        a, b = int(cu[s]), int(cu[s + 1])
        one = oracle.run(inp.q32[a:b], inp.k32[a:b], inp.v32[a:b], np.array([0, L], np.int32), 2, 1, 16, 16, lam)
        O1, L1 = oracle.scatter(one, np.array([0, L]), 2)
        assert np.array_equal(Op[a:b], O1)
        assert np.array_equal(Lp[:, a:b], L1)


def test_forced_all_keep_equals_dense_and_forced_skips_apply():
    inp = small_inputs((100,), 2, 1, 16, salt=9)
    dense = oracle.run_inputs(inp, 16, 16, math.inf)
    n, J = dense.skip.shape
    forced_keep = np.zeros((n, J), np.uint8)
    r = oracle.run_inputs(inp, 16, 16, 0.0, forced=forced_keep, work=dense.work)
    assert r.skip.sum() == 0
    assert np.array_equal(r.o, dense.o)
    # force a pattern of skips (never block 0) and compare with the kept-key form
    rng = np.random.default_rng(0)
    forced = np.where(rng.random((n, J)) < 0.3, 1, 0).astype(np.uint8)
    forced[:, 0] = 0
    r2 = oracle.run_inputs(inp, 16, 16, math.inf, forced=forced, work=dense.work)
    skips, _ = oracle_sets(r2)
    keep = keep_mask_from(skips, inp.cu_seqlens, 2, 16, 16)
    O_ref, LSE_ref = naive_dense(inp.q32, inp.k32, inp.v32, inp.cu_seqlens, 2, 1, keep=keep)
    O, LSE = oracle.scatter(r2, inp.cu_seqlens, 2)
    np.testing.assert_allclose(O, O_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE, LSE_ref, rtol=1e-14, atol=1e-12)
    # RULE entries fall back to the rule
    rule = np.full((n, J), oracle.RULE, np.uint8)
    r3 = oracle.run_inputs(inp, 16, 16, 1.0, forced=rule, work=dense.work)
    r4 = oracle.run_inputs(inp, 16, 16, 1.0, work=dense.work)
    assert np.array_equal(r3.skip, r4.skip) and np.array_equal(r3.o, r4.o)


@pytest.mark.parametrize("bq,bk", [(16, 16), (32, 16), (16, 32), (8, 24)])
@pytest.mark.parametrize("L", [1, 15, 16, 17, 33])
def test_edge_shapes(bq, bk, L):
    inp = small_inputs((L,), 1, 1, 8, salt=10)
    for lam in [0.0, math.inf]:
        res = oracle.run_inputs(inp, bq, bk, lam)
        O, LSE = oracle.scatter(res, inp.cu_seqlens, 1)
        skips, vis = oracle_sets(res)
        ref_s, ref_v = brute_force_skips(inp.q32, inp.k32, inp.cu_seqlens, 1, 1, bq, bk, lam)
        assert skips == ref_s and vis == ref_v
        keep = keep_mask_from(skips, inp.cu_seqlens, 1, bq, bk)
        O_ref, LSE_ref = naive_dense(inp.q32, inp.k32, inp.v32, inp.cu_seqlens, 1, 1, keep=keep)
        np.testing.assert_allclose(O, O_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(LSE, LSE_ref, rtol=1e-14, atol=1e-12)


def test_zero_length_sequences_do_nothing():
    inp = small_inputs((0, 5, 0), 1, 1, 8, salt=11)
    res = oracle.run_inputs(inp, 4, 4, 0.0)
    assert all(int(s) == 1 for s, _, _ in res.work)
    empty = oracle.run(inp.q32, inp.k32, inp.v32, inp.cu_seqlens, 1, 1, 4, 4, 0.0,
                       work=np.array([[0, 0, 0], [2, 0, 0]], np.int32), j_max=2)
    assert empty.skip.sum() == 0 and empty.visited.sum() == 0 and np.all(empty.o == 0)


def _eval_expr(expr):
    return float(eval(expr, {"__builtins__": {}}, {"exp": math.exp, "log": math.log}))


def test_golden_worked_examples():
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        q = np.array(case["q"], np.float32)[:, None, :]
        k = np.array(case["k"], np.float32)[:, None, :]
        v = np.array(case["v"], np.float32)[:, None, :]
        L = q.shape[0]
        cu = np.array([0, L], np.int32)
        bq, bk = case["block_q"], case["block_k"]
        for run in case["runs"]:
            lam = math.inf if run["lambda"] == "inf" else float(run["lambda"])
            res = oracle.run(q, k, v, cu, 1, 1, bq, bk, lam)
            got = sorted((int(t), int(j)) for (_, _, t, j) in oracle_sets(res)[0])
            assert got == sorted(tuple(x) for x in run["skipped"]), (case["name"], lam)
            O, LSE = oracle.scatter(res, cu, 1)
            for r in range(L):
                assert O[r, 0, 0] == pytest.approx(_eval_expr(run["o"][r]), abs=1e-12, rel=1e-12)
                assert LSE[0, r] == pytest.approx(_eval_expr(run["lse"][r]), abs=1e-12, rel=1e-12)


def test_tie_at_lambda_is_kept_on_random_integer_scores():
    # D=1, integer q and k: every gap is an exact integer, so lambda = gap is an
    # exact tie that the strict rule must keep, while lambda - 0.5 skips.
    rng = np.random.default_rng(3)
    L = 48
    q = np.ones((L, 1, 1), np.float32)
    k = rng.integers(-6, 7, size=(L, 1, 1)).astype(np.float32)
    v = rng.standard_normal((L, 1, 1)).astype(np.float32)
    cu = np.array([0, L], np.int32)
    res = oracle.run(q, k, v, cu, 1, 1, 8, 8, math.inf)
    gaps = res.mingap[np.isfinite(res.mingap) & (res.mingap > 0)]
    assert gaps.size > 0
    g = float(np.max(gaps))
    assert g == round(g)
    at = oracle_sets(oracle.run(q, k, v, cu, 1, 1, 8, 8, g))[0]
    below = oracle_sets(oracle.run(q, k, v, cu, 1, 1, 8, 8, g - 0.5))[0]
    ref_at = brute_force_skips(q, k, cu, 1, 1, 8, 8, g)[0]
    ref_below = brute_force_skips(q, k, cu, 1, 1, 8, 8, g - 0.5)[0]
    assert at == ref_at and below == ref_below
    assert len(below) > len(at)


def test_fp8_scales_are_applied_per_head():
    inp = synth.build_inputs((64,), 4, 2, 16, "fp8", rho=0.9, code=102)
    res = oracle.run_inputs(inp, 16, 16, math.inf)
    G = 2
    qd = inp.q32.astype(np.float64) * inp.q_scale[None, :, None].astype(np.float64)
    kd = inp.k32.astype(np.float64) * inp.k_scale[None, :, None].astype(np.float64)
    vd = inp.v32.astype(np.float64) * inp.v_scale[None, :, None].astype(np.float64)
    O_ref, LSE_ref = naive_dense(qd, kd, vd, inp.cu_seqlens, 4, 2)
    O, LSE = oracle.scatter(res, inp.cu_seqlens, 4)
    np.testing.assert_allclose(O, O_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE, LSE_ref, rtol=1e-14, atol=1e-12)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_storage_types_widen_exactly(dtype):
    # the oracle widens bf16 bit patterns / fp8 codes itself; the result must be
    # bit-identical to a run on the same values widened by numpy to float32
    inp = synth.build_inputs((70, 33), 4, 2, 16, dtype, rho=0.9, code=103)
    a = oracle.run_inputs(inp, 16, 16, 1.0)
    b = oracle.run(inp.q32, inp.k32, inp.v32, inp.cu_seqlens, 4, 2, 16, 16, 1.0,
                   q_scale=inp.q_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
    assert np.array_equal(a.o, b.o) and np.array_equal(a.skip, b.skip)
    assert np.array_equal(a.lse, b.lse, equal_nan=True)
    # and the widened values are the storage type's exact values
    if dtype == "bf16":
        assert np.array_equal(inp.q32.view(np.uint32) & 0xFFFF, np.zeros_like(inp.q32.view(np.uint32)))


def test_deterministic_across_runs_and_thread_counts():
    inp = small_inputs((130, 60), 4, 2, 16, salt=12)
    a = oracle.run_inputs(inp, 32, 16, 1.0, n_threads=1)
    b = oracle.run_inputs(inp, 32, 16, 1.0, n_threads=4)
    c = oracle.run_inputs(inp, 32, 16, 1.0)
    for x in (b, c):
        assert np.array_equal(a.o, x.o) and np.array_equal(a.skip, x.skip)
        assert np.array_equal(a.lse, x.lse, equal_nan=True)


def test_invalid_arguments_rejected():
    inp = small_inputs((10,), 3, 1, 8)
    with pytest.raises(ValueError):
        oracle.run_inputs(inp, 4, 4, -1.0)
    with pytest.raises(ValueError):
        oracle.run_inputs(inp, 4, 4, float("nan"))
    with pytest.raises(ValueError):
        oracle.run(inp.q32, inp.k32, inp.v32, inp.cu_seqlens, 3, 2, 4, 4, 1.0)


# ------------------------------------------ chunked prefill, per-sequence lambda --
# The queries of a sequence may be the last Lq of its Lk positions (prefill in
# chunks against a cached prefix, the FlowPrefill page, sections 2.1 and 4.5.2): query row r of the
# chunk sits at key position (Lk - Lq) + r. Pinned against numpy and brute force
# written with that offset, and against the plain prefill of the whole sequence.

def chunk_inputs(lk, lq, hq=4, hkv=2, D=16, code=111):
    """Full-sequence inputs of lengths ``lk`` and their chunks: the last lq[s] rows."""
    inp = synth.build_inputs(lk, hq, hkv, D, "f32", rho=0.95, n_vert=2, code=code, sink_gain=4.0)
    cuk = inp.cu_seqlens
    rows = np.concatenate([np.arange(int(cuk[s + 1]) - lq[s], int(cuk[s + 1])) for s in range(len(lk))]).astype(int)
    cuq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    return inp, inp.q32[rows], cuq, cuk


def dense_scores_kv(q, k, cuq, cuk, hq, hkv):
    D = q.shape[2]
    G = hq // hkv
    out = {}
    for s in range(len(cuq) - 1):
        a, b, ka, kb = int(cuq[s]), int(cuq[s + 1]), int(cuk[s]), int(cuk[s + 1])
        off = (kb - ka) - (b - a)
        mask = np.arange(kb - ka)[None, :] > (off + np.arange(b - a))[:, None]
        for h in range(hq):
            S = (q[a:b, h].astype(np.float64) @ k[ka:kb, h // G].astype(np.float64).T) / math.sqrt(D)
            S[mask] = -np.inf
            out[(s, h)] = S
    return out


def naive_kv(q, k, v, cuq, cuk, hq, hkv, keep=None):
    T, D = q.shape[0], q.shape[2]
    G = hq // hkv
    O, LSE = np.zeros((T, hq, D)), np.zeros((hq, T))
    for (s, h), S in dense_scores_kv(q, k, cuq, cuk, hq, hkv).items():
        a, b, ka, kb = int(cuq[s]), int(cuq[s + 1]), int(cuk[s]), int(cuk[s + 1])
        if b == a:
            continue
        if keep is not None:
            S = np.where(keep[(s, h)], S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        P = np.exp(S - m)
        l = P.sum(axis=1, keepdims=True)
        O[a:b, h] = (P @ v[ka:kb, h // G].astype(np.float64)) / l
        LSE[h, a:b] = (m + np.log(l))[:, 0]
    return O, LSE


def brute_force_skips_kv(q, k, cuq, cuk, hq, hkv, bq, bk, lam_of):
    skips, visited, keep = set(), set(), {}
    for (s, h), S in dense_scores_kv(q, k, cuq, cuk, hq, hkv).items():
        Lq, Lk = S.shape
        keep[(s, h)] = np.ones((Lq, Lk), dtype=bool)
        if Lq == 0:
            continue
        off = Lk - Lq
        J = (Lk + bk - 1) // bk
        M = np.full((Lq, J), -np.inf)
        for j in range(J):
            M[:, j] = S[:, j * bk: min(Lk, (j + 1) * bk)].max(axis=1)
        for t in range((Lq + bq - 1) // bq):
            r0, r1 = t * bq, min(Lq, (t + 1) * bq)
            for j in range((off + r1 - 1) // bk + 1):
                visited.add((s, h, t, j))
                prefix = M[r0:r1, :j].max(axis=1) if j > 0 else np.full(r1 - r0, -np.inf)
                gaps = [np.inf if lm == -np.inf else (-np.inf if pm == -np.inf else pm - lm)
                        for pm, lm in zip(prefix, M[r0:r1, j])]
                if min(gaps) > lam_of(s):
                    skips.add((s, h, t, j))
                    keep[(s, h)][r0:r1, j * bk: min(Lk, (j + 1) * bk)] = False
    return skips, visited, keep


CHUNK_CASES = [
    # key lengths, query lengths (the chunk), bq, bk
    ((37, 130, 1, 64), (37, 50, 1, 1), 16, 16),
    ((300, 129), (300, 129), 32, 32),          # no cached prefix: plain prefill
    ((300, 257, 90), (45, 1, 90), 32, 16),
    ((200,), (0,), 16, 16),                    # empty chunk
]


def _scatter_kv(res, cuq, hq):
    return oracle.scatter(res, cuq, hq)


@pytest.mark.parametrize("case", CHUNK_CASES)
def test_chunked_dense_limit_equals_naive_softmax(case):
    lk, lq, bq, bk = case
    inp, qc, cuq, cuk = chunk_inputs(lk, lq)
    res = oracle.run(qc, inp.k32, inp.v32, cuq, 4, 2, bq, bk, math.inf, cu_seqlens_k=cuk)
    assert res.skip.sum() == 0
    O, LSE = _scatter_kv(res, cuq, 4)
    On, LSEn = naive_kv(qc, inp.k32, inp.v32, cuq, cuk, 4, 2)
    if O.size:
        assert np.abs(O - On).max() < 1e-12 and np.abs(LSE - LSEn).max() < 1e-12


@pytest.mark.parametrize("case", CHUNK_CASES)
@pytest.mark.parametrize("lam", [0.0, 1.5])
def test_chunked_skip_set_and_kept_keys_match_brute_force(case, lam):
    lk, lq, bq, bk = case
    inp, qc, cuq, cuk = chunk_inputs(lk, lq)
    res = oracle.run(qc, inp.k32, inp.v32, cuq, 4, 2, bq, bk, lam, cu_seqlens_k=cuk)
    skips, visited, keep = brute_force_skips_kv(qc, inp.k32, cuq, cuk, 4, 2, bq, bk, lambda s: lam)
    assert oracle_sets(res) == (skips, visited)
    O, LSE = _scatter_kv(res, cuq, 4)
    On, LSEn = naive_kv(qc, inp.k32, inp.v32, cuq, cuk, 4, 2, keep=keep)
    if O.size:
        assert np.abs(O - On).max() < 1e-12 and np.abs(LSE - LSEn).max() < 1e-12


@pytest.mark.parametrize("prefix_tiles", [0, 1, 3])
def test_chunk_after_whole_tiles_equals_rows_of_full_prefill(prefix_tiles):
    # With a cached prefix of whole query tiles, the chunk's tiles are the full
    # prefill's later tiles: same rows, same blocks, same decisions, same numbers.
    bq, bk, L = 32, 16, 150
    P = prefix_tiles * bq
    inp = synth.build_inputs((L,), 4, 2, 16, "f32", rho=0.95, n_vert=3, code=112, sink_gain=4.0)
    for lam in (0.5, 2.0, math.inf):
        full = oracle.run_inputs(inp, bq, bk, lam)
        cuq = np.array([0, L - P], np.int32)
        ch = oracle.run(inp.q32[P:], inp.k32, inp.v32, cuq, 4, 2, bq, bk, lam, cu_seqlens_k=inp.cu_seqlens)
        for w, (s, h, t) in enumerate(ch.work):
            wf = [i for i, x in enumerate(full.work) if tuple(x) == (s, h, t + prefix_tiles)][0]
            assert np.array_equal(ch.o[w], full.o[wf])
            assert np.array_equal(ch.lse[w], full.lse[wf], equal_nan=True)
            assert np.array_equal(ch.skip[w], full.skip[wf])


def test_lambda_per_sequence_equals_separate_runs():
    lk, lq = (120, 90, 64, 77), (120, 40, 64, 1)
    lams = [0.0, 1.0, math.inf, 3.0]
    inp, qc, cuq, cuk = chunk_inputs(lk, lq, code=113)
    res = oracle.run(qc, inp.k32, inp.v32, cuq, 4, 2, 16, 16, 99.0, cu_seqlens_k=cuk, lam_seq=lams)
    skips, visited, keep = brute_force_skips_kv(qc, inp.k32, cuq, cuk, 4, 2, 16, 16, lambda s: lams[s])
    assert oracle_sets(res) == (skips, visited)
    for s in range(len(lk)):
        one_q = qc[cuq[s]:cuq[s + 1]]
        one_kv = slice(int(cuk[s]), int(cuk[s + 1]))
        r1 = oracle.run(one_q, inp.k32[one_kv], inp.v32[one_kv], np.array([0, lq[s]], np.int32), 4, 2, 16, 16,
                        lams[s], cu_seqlens_k=np.array([0, lk[s]], np.int32))
        items = [w for w, x in enumerate(res.work) if x[0] == s]
        assert np.array_equal(res.o[items], r1.o)
        assert np.array_equal(res.skip[items][:, : r1.skip.shape[1]], r1.skip)


def test_chunked_and_per_sequence_arguments_rejected():
    inp, qc, cuq, cuk = chunk_inputs((40, 20), (10, 20))
    q35 = np.zeros((35,) + qc.shape[1:], np.float32)
    with pytest.raises(ValueError):   # a chunk longer than its sequence
        oracle.run(q35, inp.k32, inp.v32, np.array([0, 10, 35], np.int32), 4, 2, 8, 8, 1.0, cu_seqlens_k=cuk)
    with pytest.raises(ValueError):   # a negative per-sequence lambda
        oracle.run(qc, inp.k32, inp.v32, cuq, 4, 2, 8, 8, 1.0, cu_seqlens_k=cuk, lam_seq=[1.0, -1.0])
