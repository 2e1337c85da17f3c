"""The GPU parity harness's host logic on the CPU: the vectorised selection invariants catch each kind of
malformed selection, and the forked oracle pool reports no mismatch when the "GPU" outputs are the
oracle's own (and does report a planted one)."""
import numpy as np

import oracle as O
from long_context_block_amd import inputs as I

import gpu_common as GC


def _oracle_outputs(pf):
    sel = np.empty((pf.B, pf.Hkv, pf.N, pf.K), dtype=np.int32)
    sel_lse = np.empty((pf.B, pf.Hq, pf.N, pf.K), dtype=np.float32)
    o = np.empty((pf.B, pf.Hq, pf.N, pf.d), dtype=np.float32)
    o_lse = np.empty((pf.B, pf.Hq, pf.N), dtype=np.float32)
    oc = GC.OracleCache(pf)
    G = pf.G
    for (b, r, i) in GC.units_all(pf):
        k, v, pyr = oc.head(b, r)
        qg = oc.q(b, r, i)
        us = O.select_unit(qg, k, pyr, i, pf.K, pf.scale)
        sel[b, r, i] = us.sel
        sel_lse[b, r * G:(r + 1) * G, i] = us.sel_lse
        oo, ll = O.attend_unit(qg, k, v, us.sel, i, pf.C, pf.scale, pf.N)
        o[b, r * G:(r + 1) * G, i] = oo
        o_lse[b, r * G:(r + 1) * G, i] = ll
    return GC.GpuOut(pyr=None, sel=sel, sel_lse=sel_lse, o=o, o_lse=o_lse, bsa=None), oc


def test_invariants_catch_each_malformation():
    pf = I.make_prefill(B=1, Hq=2, Hkv=1, N=300, d=16, C=32, K=3, dtype="fp32", keys="ar1", seed=0, workload_id=900)
    g, _ = _oracle_outputs(pf)
    assert GC.invariant_violations(g.sel, pf.C).size == 0
    cases = []
    s = g.sel.copy(); s[0, 0, 200, [0, 1]] = s[0, 0, 200, [1, 0]]; cases.append(s)  # not ascending
    s = g.sel.copy(); s[0, 0, 40, 1] = 5; cases.append(s)  # leaf 5 starts after position 40
    s = g.sel.copy(); s[0, 0, 250, 2] = -1; cases.append(s)  # one selection missing
    s = g.sel.copy(); s[0, 0, 0, 1] = -7; cases.append(s)  # padding other than -1
    s = g.sel.copy(); s[0, 0, 100, :] = [-1, 0, 1]; cases.append(s)  # not left-packed
    s = g.sel.copy(); s[0, 0, 120, 1] = s[0, 0, 120, 0]; cases.append(s)  # duplicate
    for x in cases:
        bad = GC.invariant_violations(x, pf.C)
        assert bad.size == 1, bad


def test_pool_compare_finds_planted_mismatch_only():
    pf = I.make_prefill(B=2, Hq=4, Hkv=2, N=200, d=16, C=32, K=3, dtype="fp32", keys="ar1", seed=0, workload_id=901)
    g, oc = _oracle_outputs(pf)
    rep = GC.compare(pf, g, GC.units_all(pf), oc, chunk=64)
    assert rep.n_units == pf.B * pf.Hkv * pf.N
    assert not rep.sel_mismatch and not rep.invariant_fail
    assert rep.attn_err < 1e-6 and rep.lse_err < 1e-5
    # plant a wrong (but well-formed) selection on a decided unit
    for i in range(199, 100, -1):
        us = O.select_unit(oc.q(1, 1, i), *oc.head(1, 1)[::2], i, pf.K, pf.scale)
        if us.margin >= GC.MARGIN:
            break
    cand = [j for j in range(i // pf.C + 1) if j not in us.sel.tolist()]
    wrong = sorted(us.sel.tolist()[1:] + [cand[0]])
    g.sel[1, 1, i] = wrong
    rep = GC.compare(pf, g, GC.units_all(pf), oc, chunk=64)
    assert len(rep.sel_mismatch) == 1 and rep.sel_mismatch[0][:3] == (1, 1, i)


def test_stratified_sample_covers_fraction_and_heads():
    pf = I.make_prefill(B=2, Hq=4, Hkv=2, N=1000, d=16, C=32, K=3, dtype="fp32", keys="iid", seed=0, workload_id=902)
    u = GC.units_stratified(pf, 0.05, seed=1)
    assert len(u) >= 0.05 * pf.B * pf.Hkv * pf.N
    assert {(b, r) for (b, r, _) in u} == {(b, r) for b in range(2) for r in range(2)}
    assert len(set(u)) == len(u)
