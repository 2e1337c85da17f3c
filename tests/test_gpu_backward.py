"""GPU parity of the block-sparse attention backward against the float64 oracle.

The forward (selection, then sparse attention with its LSE) runs on the GPU; a seeded dO is drawn; the
backward's dq, dk, dv are compared with the oracle's gradients of attention over the GPU's own selection
(the selection is not differentiated). Tolerance, per gradient tensor: max |gpu - oracle| <= 2e-2 times
max(1, the tensor's largest magnitude) -- the forward's bf16 bound for tensors of magnitude up to 1 --
and the relative Frobenius error <= 1e-2 where the tensor is not zero. The kernels round P and dS
(magnitudes <= 1) to bf16 for the matrix products and the outputs to bf16, each a relative error of at
most 2^-9; the bound leaves room for the sums of many such terms."""
import numpy as np
import pytest
import torch

import oracle as O
from long_context_block_amd import inputs as I
from long_context_block_amd import pisa as P

import gpu_common as GC
from gpu_common import shape_of, summary, to_device

pytestmark = pytest.mark.gpu


def run_backward(pf, q_tile, seed=7):
    s = shape_of(pf, q_tile)
    q, k, v = to_device(pf.q), to_device(pf.k), to_device(pf.v)
    pyr = torch.empty((P.pyramid_rows(s), pf.d), dtype=torch.float32, device="cuda")
    P.pisa_build_pyramid(s, k, pyr)
    sel = torch.empty((pf.B, pf.Hkv, pf.N, pf.K), dtype=torch.int32, device="cuda")
    P.pisa_select(s, q, k, pyr, sel, None, P.alloc_workspace(s, P.PISA_OP_SELECT))
    o = torch.empty_like(q)
    o_lse = torch.empty((pf.B, pf.Hq, pf.N), dtype=torch.float32, device="cuda")
    P.pisa_sparse_attn(s, q, k, v, sel, o, o_lse, P.alloc_workspace(s, P.PISA_OP_ATTN))
    rng = np.random.default_rng(seed)
    do_np = I.bf16_bits(rng.standard_normal(q.shape, dtype=np.float32))
    d_o = torch.from_numpy(do_np.view(np.int16)).cuda().view(torch.bfloat16)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = P.alloc_workspace(s, P.PISA_OP_ATTN_BWD)
    P.pisa_sparse_attn_backward(s, q, k, v, sel, o, o_lse, d_o, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return dict(sel=sel.cpu().numpy(), do=I.bf16_to_f32(do_np).astype(np.float64), dq=dq.float().cpu().numpy(),
                dk=dk.float().cpu().numpy(), dv=dv.float().cpu().numpy())


def _oracle_head(task):
    pf, g = GC._CTX["pf"], GC._CTX["g"]
    b, r = task
    G = pf.G
    qg = pf.q.f64((b, slice(r * G, (r + 1) * G)))
    dq, dk, dv = O.attention_backward_head(qg, pf.k.f64((b, r)), pf.v.f64((b, r)), g["sel"][b, r], pf.C, pf.scale,
                                           g["do"][b, r * G:(r + 1) * G])
    out = {}
    for name, ref, got in (("dq", dq, g["dq"][b, r * G:(r + 1) * G]), ("dk", dk, g["dk"][b, r]),
                           ("dv", dv, g["dv"][b, r])):
        out[name] = (float(np.abs(got - ref).max()), float(np.abs(ref).max()), float(np.sum((got - ref) ** 2)),
                     float(np.sum(ref ** 2)))
    return out


def check_backward(pf, q_tile, label):
    compare_backward(pf, run_backward(pf, q_tile), label)


def compare_backward(pf, g, label):
    heads = [(b, r) for b in range(pf.B) for r in range(pf.Hkv)]
    GC._CTX.update(pf=pf, g=g)
    try:
        parts = GC.pool_map(_oracle_head, heads)
    finally:
        GC._CTX.clear()
    msg = []
    for name in ("dq", "dk", "dv"):
        err = max(x[name][0] for x in parts)
        top = max(x[name][1] for x in parts)
        den = sum(x[name][3] for x in parts)
        rel = (sum(x[name][2] for x in parts) / den) ** 0.5 if den > 0 else float("nan")
        msg.append(f"{name}: max_err={err:.3g} max|ref|={top:.3g} rel_fro=" + (f"{rel:.3g}" if den > 0 else "n/a"))
        assert err <= 2e-2 * max(1.0, top), (name, err, top)
        assert top == 0.0 or rel <= 1e-2, (name, rel)
    summary(f"[backward {label}] " + "; ".join(msg))


SMALL = {
    "g4_c64": dict(B=1, Hq=8, Hkv=2, N=1500, d=128, C=64, K=4, dtype="bf16", keys="ar1"),
    "g2_c32_d64_b2": dict(B=2, Hq=4, Hkv=2, N=1100, d=64, C=32, K=6, dtype="bf16", keys="ar1"),
    "g8_ragged": dict(B=1, Hq=16, Hkv=2, N=777, d=128, C=64, K=5, dtype="bf16", keys="iid"),
    "g1_c32": dict(B=1, Hq=1, Hkv=1, N=2000, d=128, C=32, K=8, dtype="bf16", keys="ar1"),
    "one_token": dict(B=1, Hq=4, Hkv=1, N=1, d=128, C=64, K=4, dtype="bf16", keys="iid"),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_backward_small(name):
    pf = I.make_prefill(seed=0, workload_id=700, **SMALL[name])
    check_backward(pf, max(1, min(4, 16 // pf.G)), name)


@pytest.mark.timeout(900)
def test_backward_16k():
    pf = I.make_workload("prefill_16k")
    check_backward(pf, 2, "prefill_16k")


def test_chunked_attention_equals_one_chunk(monkeypatch):
    """The attention and its backward cut the batch into chunks of (sequence, KV head) slices. Forced to one
    slice per chunk (a 1 MiB budget), they give the same forward bits (O and its LSE) and the same dq bits
    as the single-chunk run; dk and dv sum a leaf's pairs in an order set by the regroup (pairs of one leaf
    are placed by atomic counters) and by where the task boundaries fall in the sorted pair list, which
    moves with the chunking, so they agree to the last bits of their bf16 outputs."""
    pf = I.make_prefill(B=2, Hq=8, Hkv=2, N=1500, d=128, C=64, K=6, dtype="bf16", keys="ar1", seed=0,
                        workload_id=710)
    s = shape_of(pf, 4)
    q, k, v = to_device(pf.q), to_device(pf.k), to_device(pf.v)
    pyr = torch.empty((P.pyramid_rows(s), pf.d), dtype=torch.float32, device="cuda")
    P.pisa_build_pyramid(s, k, pyr)
    sel = torch.empty((pf.B, pf.Hkv, pf.N, pf.K), dtype=torch.int32, device="cuda")
    P.pisa_select(s, q, k, pyr, sel, None, P.alloc_workspace(s, P.PISA_OP_SELECT))
    rng = np.random.default_rng(11)
    d_o = torch.from_numpy(I.bf16_bits(rng.standard_normal(q.shape, dtype=np.float32)).view(np.int16)).cuda()
    d_o = d_o.view(torch.bfloat16)

    def run():
        o = torch.empty_like(q)
        o_lse = torch.empty((pf.B, pf.Hq, pf.N), dtype=torch.float32, device="cuda")
        P.pisa_sparse_attn(s, q, k, v, sel, o, o_lse, P.alloc_workspace(s, P.PISA_OP_ATTN))
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        P.pisa_sparse_attn_backward(s, q, k, v, sel, o, o_lse, d_o, dq, dk, dv,
                                    P.alloc_workspace(s, P.PISA_OP_ATTN_BWD))
        torch.cuda.synchronize()
        return [x.float().cpu().numpy() for x in (o, o_lse, dq, dk, dv)]

    one = run()
    whole = P.pisa_workspace_size(s, P.PISA_OP_ATTN)
    monkeypatch.setenv("PISA_ATTN_CHUNK_MIB", "1")
    assert P.pisa_workspace_size(s, P.PISA_OP_ATTN) * 4 == pytest.approx(whole, rel=0.01)  # one of 4 slices
    chunked = run()
    for name, a, b in zip(("o", "o_lse", "dq"), one[:3], chunked[:3]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name
    for name, a, b in zip(("dk", "dv"), one[3:], chunked[3:]):
        assert np.abs(a - b).max() <= 2 ** -7 * max(1.0, float(np.abs(a).max())), name
    summary(f"[attention chunking] 4 one-slice chunks equal one chunk: O, LSE and dq bit for bit, dk/dv within bf16 "
            f"rounding (max diff {max(float(np.abs(a - b).max()) for a, b in zip(one[3:], chunked[3:])):.3g})")



def _boundary_selection(N, C, K, extra):
    """Left-packed, ascending selection [N, K]: every position keeps its own leaf, and leaf j gets extra[j]
    more positions (the first eligible ones with a free slot), so that leaf j's bucket of the attention
    regroup holds (tokens of leaf j) + extra[j] pairs."""
    sets = [[i // C] for i in range(N)]
    for j, n in sorted(extra.items()):
        i = C * (j + 1)
        while n:
            if len(sets[i]) < K and j not in sets[i]:
                sets[i].append(j)
                n -= 1
            i += 1
    sel = np.full((N, K), -1, dtype=np.int32)
    for i, lv in enumerate(sets):
        lv = sorted(lv)
        sel[i, :len(lv)] = lv
    return sel


@pytest.mark.parametrize("C", [64, 32])
def test_backward_task_boundaries(C):
    """dK / dV of leaves at every kind of edge of the dK/dV pass's 512-pair tasks, on a crafted selection
    (B = 1, one KV head, N = 4096, K = 4; C = 32 has two waves per token slice): leaf 0 fills task 0
    exactly; leaf 1 fills tasks 1 and 2 (it starts on a task boundary and continues); leaf 2 lies inside
    task 3; leaf 3 starts inside task 3 and ends inside task 5, across the whole of task 4; leaf 4 ends
    exactly on a task boundary; leaf 5 starts on one. Gradients against the oracle, as in the other
    backward tests."""
    pf = I.make_prefill(B=1, Hq=4, Hkv=1, N=4096, d=128, C=C, K=4, dtype="bf16", keys="ar1", seed=0,
                        workload_id=730)
    sizes = [512, 1024, 100, 1000, 436]
    sel_np = _boundary_selection(pf.N, pf.C, pf.K, {j: n - C for j, n in enumerate(sizes)})
    counts = np.bincount(sel_np[sel_np >= 0], minlength=pf.N // pf.C)
    starts = np.concatenate([[0], np.cumsum(counts)])
    assert list(counts[:6]) == sizes + [C]
    assert list(starts[:7]) == [0, 512, 1536, 1636, 2636, 3072, 3072 + C]
    s = shape_of(pf, 4)
    q, k, v = to_device(pf.q), to_device(pf.k), to_device(pf.v)
    sel = torch.from_numpy(sel_np.reshape(1, 1, pf.N, pf.K)).cuda()
    o = torch.empty_like(q)
    o_lse = torch.empty((pf.B, pf.Hq, pf.N), dtype=torch.float32, device="cuda")
    P.pisa_sparse_attn(s, q, k, v, sel, o, o_lse, P.alloc_workspace(s, P.PISA_OP_ATTN))
    rng = np.random.default_rng(5)
    do_np = I.bf16_bits(rng.standard_normal(q.shape, dtype=np.float32))
    d_o = torch.from_numpy(do_np.view(np.int16)).cuda().view(torch.bfloat16)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    P.pisa_sparse_attn_backward(s, q, k, v, sel, o, o_lse, d_o, dq, dk, dv, P.alloc_workspace(s, P.PISA_OP_ATTN_BWD))
    torch.cuda.synchronize()
    g = dict(sel=sel.cpu().numpy(), do=I.bf16_to_f32(do_np).astype(np.float64), dq=dq.float().cpu().numpy(),
             dk=dk.float().cpu().numpy(), dv=dv.float().cpu().numpy())
    compare_backward(pf, g, f"task boundaries C={C}")
