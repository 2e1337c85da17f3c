"""pisa_select_noalloc (the selection with the library's fixed per-GPU scratch instead of a caller
workspace) against pisa_select on the same inputs: two calls in a row, the second on a smaller shape
(the scratch then holds the first call's data), each bit-identical to pisa_select."""
import numpy as np
import pytest
import torch

from long_context_block_amd import inputs as I
from long_context_block_amd import pisa as P

from gpu_common import say, shape_of, to_device

pytestmark = pytest.mark.gpu


def _both(pf, q_tile):
    s = shape_of(pf, q_tile)
    q, k = to_device(pf.q), to_device(pf.k)
    pyr = torch.empty((P.pyramid_rows(s), pf.d), dtype=torch.float32, device="cuda")
    P.pisa_build_pyramid(s, k, pyr)
    out = []
    for noalloc in (True, False):
        sel = torch.full((pf.B, pf.Hkv, pf.N, pf.K), 7, dtype=torch.int32, device="cuda")
        lse = torch.full((pf.B, pf.Hq, pf.N, pf.K), 3.0, dtype=torch.float32, device="cuda")
        if noalloc:
            P.pisa_select_noalloc(s, q, k, pyr, sel, lse)
        else:
            P.pisa_select(s, q, k, pyr, sel, lse, P.alloc_workspace(s, P.PISA_OP_SELECT))
        torch.cuda.synchronize()
        out.append((sel.cpu().numpy(), lse.cpu().numpy()))
    (a_sel, a_lse), (b_sel, b_lse) = out
    assert np.array_equal(a_sel, b_sel)
    assert np.array_equal(a_lse.view(np.uint32), b_lse.view(np.uint32))
    return s


def test_noalloc_matches_workspace_call_twice():
    big = I.make_workload("prefill_16k")
    s = _both(big, 2)
    need = P.pisa_workspace_size(s, P.PISA_OP_SELECT)
    say(f"[noalloc] 16K: scratch used {need / 2**20:.1f} MiB of {P.pisa_select_noalloc_max_bytes() / 2**20:.0f} MiB")
    small = I.make_prefill(B=2, Hq=4, Hkv=1, N=3000, d=128, C=64, K=8, dtype="bf16", keys="ar1", seed=0,
                           workload_id=400)
    _both(small, 4)
    say("[noalloc] two calls in a row (16K, then 2 x 3000 tokens) bit-identical to pisa_select")


def test_noalloc_rejects_shapes_beyond_its_scratch():
    s = P.make_shape(batch=1, seq_len=65536, n_q_heads=32, n_kv_heads=8, head_dim=128, block=64, top_k=16, q_tile=4)
    assert P.pisa_workspace_size(s, P.PISA_OP_SELECT) > P.pisa_select_noalloc_max_bytes()
    g = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(P.PisaError) as e:
        P.pisa_select_noalloc(s, g, g, g, g)
    assert e.value.status == P.PISA_EUNSUPPORTED
    assert "scratch" in str(e.value)
