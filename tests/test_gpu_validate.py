"""The BSP_DEBUG_VALIDATE mode on the GPU: bad device descriptors are caught
on the host before any launch (the guide's section 5, step 4: packed dynamic
batches and a paged KV cache are inputs a serving system builds at run time).

Order matters for safety: the first cases use descriptors that would be
harmless even if a kernel ran on them (a decreasing cu_seqlens only yields an
empty sequence and in-bounds rows); only once those have come back rejected,
which shows the mode is active, do page ids that would point outside the
cache go in (-1 and 2^30, rejected by the host checker whatever the cache
size, as the CPU tests of bsp_validate_host show).
"""

import math
import os

import numpy as np
import pytest
import torch

import synth
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture()
def validate_mode():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_bsp_amd as bsp

    bsp.load_library()
    old = os.environ.get("BSP_DEBUG_VALIDATE")
    os.environ["BSP_DEBUG_VALIDATE"] = "1"
    yield bsp
    if old is None:
        del os.environ["BSP_DEBUG_VALIDATE"]
    else:
        os.environ["BSP_DEBUG_VALIDATE"] = old


def _rejected(bsp, fn, needle):
    with pytest.raises(bsp.BspError) as ei:
        fn()
    assert ei.value.status == bsp.BSP_ERR_INVALID_ARG, ei.value
    assert needle in ei.value.detail, ei.value.detail
    print(f"rejected: {ei.value.detail}", flush=True)


def test_validate_mode_rejects_bad_descriptors_and_passes_good_ones(validate_mode):
    bsp = validate_mode
    inp = synth.build_inputs((300, 129), 4, 2, 128, "bf16", rho=0.97, n_vert=2, code=401, paged=True, page_size=64)
    dev = parity.to_device(inp)
    T = inp.total_tokens
    # a good call gives the same results with and without the mode
    a = bsp.fwd(dev["q"], dev["k"], dev["v"], dev["cu"], inp.max_seqlen, block_q=128, block_k=128, lam=2.0)
    del os.environ["BSP_DEBUG_VALIDATE"]
    b = bsp.fwd(dev["q"], dev["k"], dev["v"], dev["cu"], inp.max_seqlen, block_q=128, block_k=128, lam=2.0)
    os.environ["BSP_DEBUG_VALIDATE"] = "1"
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)

    # harmless-if-launched cases first
    bad_cu = torch.tensor([0, 300, 200, T], dtype=torch.int32, device="cuda")
    _rejected(bsp, lambda: bsp.fwd(dev["q"], dev["k"], dev["v"], bad_cu, 300, block_q=128, block_k=128, lam=2.0),
              "decreases at sequence 1")
    _rejected(bsp, lambda: bsp.fwd(dev["q"], dev["k"], dev["v"], dev["cu"], 200, block_q=128, block_k=128, lam=2.0),
              "above the stated maximum")
    short_cu = torch.tensor([0, 300, T - 29], dtype=torch.int32, device="cuda")
    _rejected(bsp, lambda: bsp.fwd(dev["q"], dev["k"], dev["v"], short_cu, 300, block_q=128, block_k=128, lam=2.0),
              f"states {T} tokens")
    # a chunk longer than its sequence (130 queries, 129 keys): the kernel would write nothing for it
    cu_q = torch.tensor([0, 45, 175], dtype=torch.int32, device="cuda")
    q_c = dev["q"][:175].contiguous()
    _rejected(bsp, lambda: bsp.fwd(q_c, dev["k"], dev["v"], cu_q, 130, block_q=128, block_k=128, lam=2.0,
                                   cu_seqlens_k=dev["cu"], max_seqlen_k=300), "has 130 queries but only 129 keys")
    lam_bad = torch.tensor([1.0, -2.0], dtype=torch.float32, device="cuda")
    _rejected(bsp, lambda: bsp.fwd(dev["q"], dev["k"], dev["v"], dev["cu"], 300, block_q=128, block_k=128, lam=2.0,
                                   lam_per_seq=lam_bad), "lambda_per_seq[1]")
    # the mode is active: now page ids that point outside the cache
    for bad_id in (-1, 1 << 30):
        table = dev["table"].clone()
        table[1, 1] = bad_id
        _rejected(bsp, lambda: bsp.fwd(dev["q"], dev["k_pages"], dev["v_pages"], dev["cu"], 300, block_table=table,
                                       block_q=128, block_k=128, lam=2.0), f"block_table[1][1] = {bad_id}")
    # paged, good table: runs
    bsp.fwd(dev["q"], dev["k_pages"], dev["v_pages"], dev["cu"], 300, block_table=dev["table"], block_q=128,
            block_k=128, lam=2.0)
    torch.cuda.synchronize()


def test_validate_mode_on_the_decoding_step(validate_mode):
    bsp = validate_mode
    inp = synth.build_inputs((300, 129), 4, 2, 128, "bf16", rho=0.97, n_vert=2, code=402, paged=True, page_size=64)
    dev = parity.to_device(inp)
    rows = torch.tensor([299, 428], dtype=torch.int64, device="cuda")
    q = dev["q"][rows].contiguous()
    bsp.decode(q, dev["k"], dev["v"], dev["cu"], 300, block_k=128, lam=2.0)
    bad_cu = torch.tensor([0, 300, 200], dtype=torch.int32, device="cuda")
    _rejected(bsp, lambda: bsp.decode(q, dev["k"], dev["v"], bad_cu, 300, block_k=128, lam=2.0),
              "decreases at sequence 1")
    table = dev["table"].clone()
    table[0, 2] = 1 << 30
    _rejected(bsp, lambda: bsp.decode(q, dev["k_pages"], dev["v_pages"], dev["cu"], 300, total_k=inp.total_tokens,
                                      block_table=table, block_k=128, lam=2.0), f"block_table[0][2] = {1 << 30}")
    torch.cuda.synchronize()
