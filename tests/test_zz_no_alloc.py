"""bsp_attn_decode_noalloc: the decoding step without a workspace argument.

The entry point takes the step's workspace from the library's static
per-GPU scratch array. It must give exactly what bsp_attn_decode gives with a
caller's workspace (same kernels, same inputs), and the oracle's answer within
the parity protocol, on two calls in a row, the second smaller than the first
(the array keeps the first call's contents, which the second must not see).
"""

import math

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


def _outputs(bsp, n_seqs, Hq, D, max_k, block_k, device="cuda"):
    import torch

    words = bsp.skip_bitmap_words_kv(Hq, n_seqs, 1, max_k, 1, block_k)
    return dict(out=torch.empty((n_seqs, Hq, D), dtype=torch.bfloat16, device=device),
                lse=torch.empty((Hq, n_seqs), dtype=torch.float32, device=device),
                bitmap=torch.empty((max(words, 1),), dtype=torch.int32, device=device),
                skip_count=torch.empty((Hq,), dtype=torch.int64, device=device),
                visited_count=torch.empty((Hq,), dtype=torch.int64, device=device))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("paged", [False, True], ids=["packed", "paged"])
def test_noalloc_decode_matches_the_workspace_entry_point(dtype, paged):
    import torch

    import block_sparse_long_bsp_amd as bsp

    big = synth.build_inputs((5000, 300, 77, 2049), 8, 2, 128, dtype, rho=0.97, n_vert=3, code=501, sink_gain=6.0,
                             paged=paged, page_size=64)
    small = synth.build_inputs((129, 40), 8, 2, 128, dtype, rho=0.97, n_vert=2, code=502, sink_gain=6.0,
                               paged=paged, page_size=64)
    for inp in (big, small):  # the second call is smaller than the first
        dev = parity.to_device(inp)
        chunk = parity.Chunk(lq=(1,) * len(inp.seqlens))
        q = dev["q"][torch.from_numpy(chunk.rows(inp)).cuda()].contiguous()
        k = dev["k_pages"] if paged else dev["k"]
        v = dev["v_pages"] if paged else dev["v"]
        kw = dict(total_k=inp.total_tokens, block_table=dev.get("table") if paged else None, block_k=128, lam=2.0,
                  q_scale=dev["q_scale"], k_scale=dev["k_scale"], v_scale=dev["v_scale"])
        n = len(inp.seqlens)
        need = bsp.decode_workspace_bytes(8, 2, n, inp.total_tokens, inp.max_seqlen, 128, 128)
        assert 0 < need <= bsp.DECODE_SCRATCH_BYTES
        ref_out = _outputs(bsp, n, 8, 128, inp.max_seqlen, 128)
        a = bsp.decode(q, k, v, dev["cu"], inp.max_seqlen, **kw, **ref_out)
        got = _outputs(bsp, n, 8, 128, inp.max_seqlen, 128)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        b = bsp.decode_noalloc(q, k, v, dev["cu"], inp.max_seqlen, **kw, **got)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] >= free0 - (2 << 20)  # nothing allocated by the call
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        assert int(b[3].sum()) > 0  # some blocks skipped
        # and the oracle's answer, with the parity protocol's tolerances
        gpu = dict(o=b[0].float().cpu().numpy(), lse=b[1].cpu().numpy(),
                   bits=bsp.unpack_bitmap(b[2], 8, n, 1, 1, 128, inp.max_seqlen),
                   skip_count=b[3].cpu().numpy(), visited_count=b[4].cpu().numpy())
        rep = parity.compare(inp, gpu, 64, 128, 2.0, chunk=chunk)
        assert rep.ok(), "; ".join(rep.problems)
        print(f"noalloc decode {dtype} paged={paged} seqs={inp.seqlens}: identical to bsp_attn_decode, "
              f"skipped {rep.n_skipped}/{rep.n_pairs}, max-abs {rep.max_abs:.3g}", flush=True)
