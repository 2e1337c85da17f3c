"""GPU parity of the selection-quality pass (the dense causal leaf scores and the measures built on them)
against the float64 oracle: every eligible leaf's per-head LSE and each row's LSE within 2e-4 (bf16) /
2e-5 (fp32); the flat exact Top-K equal to the oracle's brute force bit for bit on every unit whose flat
gap is at least 1e-3; Recall@K of the GPU's pyramid selection against it equal to the oracle's on those
units; the attention mass ratio of that selection within 1e-4 of the oracle's dense softmax."""
import numpy as np
import pytest
import torch

import oracle as O
from long_context_block_amd import inputs as I
from long_context_block_amd import pisa as P

import gpu_common as GC
from gpu_common import MARGIN, say, shape_of, summary, to_device

pytestmark = pytest.mark.gpu


def run_quality(pf, positions, q_tile, with_bsa=False):
    s = shape_of(pf, q_tile)
    q, k = to_device(pf.q), to_device(pf.k)
    pyr = torch.empty((P.pyramid_rows(s), pf.d), dtype=torch.float32, device="cuda")
    P.pisa_build_pyramid(s, k, pyr)
    sel = torch.empty((pf.B, pf.Hkv, pf.N, pf.K), dtype=torch.int32, device="cuda")
    P.pisa_select(s, q, k, pyr, sel, None, P.alloc_workspace(s, P.PISA_OP_SELECT))
    pos = torch.tensor(positions, dtype=torch.int32, device="cuda")
    n0 = -(-pf.N // pf.C)
    leaf = torch.empty((pf.B, pf.Hq, len(positions), n0), dtype=torch.float32, device="cuda")
    row = torch.empty((pf.B, pf.Hq, len(positions)), dtype=torch.float32, device="cuda")
    P.pisa_flat_leaf_lse(s, q, k, pos, leaf, row)
    out = {}
    sels = {"pisa": sel}
    if with_bsa:
        bsel = torch.empty_like(sel)
        P.bsa_select(s, q, k, bsel, P.alloc_workspace(s, P.PISA_OP_BSA))
        sels["bsa"] = bsel
    for name, sx in sels.items():
        flat = torch.empty((pf.B, pf.Hkv, len(positions), pf.K), dtype=torch.int32, device="cuda")
        rec = torch.empty((pf.B, pf.Hkv, len(positions)), dtype=torch.float32, device="cuda")
        mass = torch.empty((pf.B, pf.Hq, len(positions)), dtype=torch.float32, device="cuda")
        P.pisa_selection_quality(s, leaf, row, pos, sx, flat, rec, mass)
        torch.cuda.synchronize()
        out[name] = dict(sel=sx.cpu().numpy(), flat=flat.cpu().numpy(), recall=rec.cpu().numpy(),
                         mass=mass.cpu().numpy())
    out["leaf"] = leaf.cpu().numpy()
    out["row"] = row.cpu().numpy()
    return out


def _check_units(task):
    pf, g, positions, leaf_units = GC._CTX["pf"], GC._CTX["g"], GC._CTX["pos"], GC._CTX["leaf_units"]
    res = dict(n=0, decided=0, flat_mismatch=[], recall_mismatch=[], leaf_err=0.0, row_err=0.0, mass_err=0.0)
    heads = {}
    G = pf.G
    for (b, r, x) in task:
        if (b, r) not in heads:
            heads[(b, r)] = pf.k.f64((b, r))
        k = heads[(b, r)]
        i = positions[x]
        qg = pf.q.f64((b, slice(r * G, (r + 1) * G), i))
        res["n"] += 1
        L = O.row_lse_unit(qg, k, i, pf.scale)
        res["row_err"] = max(res["row_err"], float(np.abs(g["row"][b, r * G:(r + 1) * G, x] - L).max()))
        if (b, r, x) in leaf_units:
            ne = i // pf.C + 1
            want = np.stack([O.leaf_lse_per_head(qg, k, j, i, pf.C, pf.scale, pf.N) for j in range(ne)], axis=1)
            got = g["leaf"][b, r * G:(r + 1) * G, x]
            res["leaf_err"] = max(res["leaf_err"], float(np.abs(got[:, :ne] - want).max()))
            assert np.all(got[:, ne:] == -np.inf)
        fe, gap = O.flat_exact_select_unit(qg, k, i, pf.C, pf.K, pf.scale)
        p_ = g["pisa"]
        if gap >= MARGIN:
            res["decided"] += 1
            if p_["flat"][b, r, x].tolist() != fe.tolist():
                res["flat_mismatch"].append((b, r, i, p_["flat"][b, r, x].tolist(), fe.tolist()))
            want_rec = O.recall_at_k(p_["sel"][b, r, i], fe)
            if abs(p_["recall"][b, r, x] - want_rec) > 1e-6:
                res["recall_mismatch"].append((b, r, i, float(p_["recall"][b, r, x]), want_rec))
        m = O.attention_mass_unit(qg, k, p_["sel"][b, r, i], i, pf.C, pf.scale)
        res["mass_err"] = max(res["mass_err"], float(np.abs(p_["mass"][b, r * G:(r + 1) * G, x] - m).max()))
    return res


def check(pf, g, positions, label, leaf_frac=1.0):
    units = [(b, r, x) for b in range(pf.B) for r in range(pf.Hkv) for x in range(len(positions))]
    rng = np.random.default_rng(0)
    leaf_units = set(u for u in units if rng.random() < leaf_frac)
    tasks = [units[j:j + 256] for j in range(0, len(units), 256)]
    GC._CTX.update(pf=pf, g=g, pos=positions, leaf_units=leaf_units)
    try:
        parts = GC.pool_map(_check_units, tasks)
    finally:
        GC._CTX.clear()
    n = sum(x["n"] for x in parts)
    dec = sum(x["decided"] for x in parts)
    fm = [m for x in parts for m in x["flat_mismatch"]]
    rm = [m for x in parts for m in x["recall_mismatch"]]
    le = max(x["leaf_err"] for x in parts)
    re_ = max(x["row_err"] for x in parts)
    me = max(x["mass_err"] for x in parts)
    tol = 2e-4 if pf.dtype == "bf16" else 2e-5
    summary(f"[quality {label}] units={n} flat-decided={dec} ({dec / n:.4f}) flat_mismatch={len(fm)} "
            f"recall_mismatch={len(rm)} leaf_lse_err={le:.3g} ({len(leaf_units)} units) row_lse_err={re_:.3g} "
            f"mass_err={me:.3g}; mean recall@K={g['pisa']['recall'].mean():.4f} "
            f"mean mass={g['pisa']['mass'].mean():.4f}")
    assert not fm, fm[:5]
    assert not rm, rm[:5]
    assert le <= tol and re_ <= tol, (le, re_)
    assert me <= 1e-4, me
    assert dec >= 0.8 * n


@pytest.mark.parametrize("spec", [
    dict(B=1, Hq=1, Hkv=1, N=1024, d=64, C=32, K=4, dtype="fp32", keys="iid"),
    dict(B=2, Hq=8, Hkv=2, N=2100, d=128, C=64, K=6, dtype="bf16", keys="ar1"),
    dict(B=1, Hq=4, Hkv=2, N=1500, d=64, C=32, K=5, dtype="bf16", keys="ar1"),
], ids=["tiny_fp32", "bf16_g4_b2", "bf16_d64_c32"])
def test_quality_small_all_positions(spec):
    pf = I.make_prefill(seed=0, workload_id=500, **spec)
    positions = list(range(pf.N))
    g = run_quality(pf, positions, q_tile=max(1, min(4, 16 // pf.G)), with_bsa=True)
    check(pf, g, positions, f"small {spec['dtype']} N={pf.N}")
    # the BSA selection's measures come from the same pass
    assert np.all((g["bsa"]["recall"] >= 0) & (g["bsa"]["recall"] <= 1))
    assert np.array_equal(g["bsa"]["flat"], g["pisa"]["flat"])


def test_quality_ragged_positions_and_out_of_range():
    """Any subset of positions, in any order; a position outside [0, N) yields NaN rows only."""
    pf = I.make_prefill(B=1, Hq=4, Hkv=1, N=700, d=128, C=64, K=4, dtype="bf16", keys="ar1", seed=0,
                        workload_id=501)
    positions = [699, 0, 63, 64, 5000, 350, -3, 128]
    g = run_quality(pf, positions, q_tile=4)
    bad = [x for x, i in enumerate(positions) if not 0 <= i < pf.N]
    good = [x for x in range(len(positions)) if x not in bad]
    assert np.all(np.isnan(g["row"][:, :, bad])) and np.all(np.isnan(g["pisa"]["recall"][:, :, bad]))
    assert np.all(g["pisa"]["flat"][:, :, bad] == -1)
    gp = dict(g)
    gp["row"], gp["leaf"] = g["row"][:, :, good], g["leaf"][:, :, good]
    gp["pisa"] = {k_: (v[:, :, good] if k_ != "sel" else v) for k_, v in g["pisa"].items()}
    check(pf, gp, [positions[x] for x in good], "ragged positions")


@pytest.mark.timeout(900)
def test_quality_16k_all_positions():
    pf = I.make_workload("prefill_16k")
    positions = list(range(pf.N))
    g = run_quality(pf, positions, q_tile=2)
    check(pf, g, positions, "prefill_16k all positions", leaf_frac=0.02)


@pytest.mark.timeout(900)
def test_quality_64k_sampled_positions():
    pf = I.make_workload("prefill_64k")
    rng = np.random.default_rng(11)
    positions = sorted(set(rng.choice(pf.N, 512, replace=False).tolist()) | {0, 63, 64, pf.N - 1})
    g = run_quality(pf, positions, q_tile=4)
    check(pf, g, positions, f"prefill_64k {len(positions)} positions", leaf_frac=0.05)
