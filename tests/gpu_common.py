"""Shared plumbing for the GPU parity tests: upload seeded inputs, run the HIP path through the C ABI,
and compare with the float64 oracle unit by unit.

The oracle runs in a pool of forked worker processes (one per host core the test may use, at most 16).
The workers never touch the GPU: they read the inputs and the GPU's outputs, which the parent holds in
host memory before forking, and each returns a report for its share of the units."""
from __future__ import annotations

import dataclasses
import math
import multiprocessing as mp
import os
import sys
import time

import numpy as np
import torch

import oracle as O
from long_context_block_amd import inputs as I
from long_context_block_amd import pisa as P

DEV = "cuda"
TOL_ATTN = {"fp32": 1e-5, "bf16": 2e-2}
MARGIN = 1e-3
MAX_WORKERS = 16

# Lines collected for the end-of-run summary (printed by conftest's terminal-summary hook, so they
# appear in the output of a quiet run too).
SUMMARY: list[str] = []


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def summary(msg: str):
    say(msg)
    SUMMARY.append(msg)


def n_workers() -> int:
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, cores))


# Context read by the forked workers: set by the parent right before the pool forks.
_CTX: dict = {}


def _worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass


def progress(msg: str):
    """A progress line on the process's real stdout (not captured by pytest), so that a long oracle
    phase is visibly alive."""
    try:
        sys.__stdout__.write(msg + "\n")
        sys.__stdout__.flush()
    except Exception:  # pragma: no cover
        pass


def pool_map(fn, tasks, every_s=20.0):
    """fn over tasks in forked worker processes (results in task order). fn and the data it reads from
    _CTX are inherited by the fork; only the tasks and the results are pickled. Prints a progress line
    about every `every_s` seconds."""
    if len(tasks) <= 1 or n_workers() == 1:
        return [fn(t) for t in tasks]
    out = []
    t0 = last = time.time()
    with mp.get_context("fork").Pool(n_workers(), initializer=_worker_init) as pool:
        for res in pool.imap(fn, tasks, chunksize=1):
            out.append(res)
            if time.time() - last > every_s:
                last = time.time()
                progress(f"[oracle pool] {len(out)}/{len(tasks)} tasks done, {last - t0:.0f} s")
    return out


def to_device(t: I.Tensor) -> torch.Tensor:
    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t.data)).to(DEV)


def shape_of(pf: I.Prefill, q_tile: int) -> P.Shape:
    return P.make_shape(batch=pf.B, seq_len=pf.N, n_q_heads=pf.Hq, n_kv_heads=pf.Hkv, head_dim=pf.d, block=pf.C,
                        top_k=pf.K, q_tile=q_tile, dtype=pf.dtype)


@dataclasses.dataclass
class GpuOut:
    pyr: np.ndarray
    sel: np.ndarray
    sel_lse: np.ndarray | None
    o: np.ndarray | None
    o_lse: np.ndarray | None
    bsa: np.ndarray | None


def run_gpu(pf: I.Prefill, q_tile: int, *, lse=True, attn=True, bsa=False, dev=None) -> GpuOut:
    s = shape_of(pf, q_tile)
    q = to_device(pf.q) if dev is None else dev["q"]
    k = to_device(pf.k) if dev is None else dev["k"]
    v = (to_device(pf.v) if dev is None else dev["v"]) if attn else None
    rows = P.pyramid_rows(s)
    pyr = torch.empty((rows, pf.d), dtype=torch.float32, device=DEV)
    P.pisa_build_pyramid(s, k, pyr)
    sel = torch.empty((pf.B, pf.Hkv, pf.N, pf.K), dtype=torch.int32, device=DEV)
    sel_lse = torch.empty((pf.B, pf.Hq, pf.N, pf.K), dtype=torch.float32, device=DEV) if lse else None
    ws = P.alloc_workspace(s, P.PISA_OP_SELECT)
    P.pisa_select(s, q, k, pyr, sel, sel_lse, ws)
    del ws
    o = o_lse = None
    if attn:
        o = torch.empty_like(q)
        o_lse = torch.empty((pf.B, pf.Hq, pf.N), dtype=torch.float32, device=DEV)
        wsa = P.alloc_workspace(s, P.PISA_OP_ATTN)
        P.pisa_sparse_attn(s, q, k, v, sel, o, o_lse, wsa)
        del wsa
    bsel = None
    if bsa:
        bsel = torch.empty_like(sel)
        wsb = P.alloc_workspace(s, P.PISA_OP_BSA)
        P.bsa_select(s, q, k, bsel, wsb)
        del wsb
    torch.cuda.synchronize()
    out = GpuOut(pyr=pyr.cpu().numpy(), sel=sel.cpu().numpy(), sel_lse=sel_lse.cpu().numpy() if lse else None,
                 o=o.float().cpu().numpy() if attn else None, o_lse=o_lse.cpu().numpy() if attn else None,
                 bsa=bsel.cpu().numpy() if bsa else None)
    del q, k, v, pyr, sel, sel_lse, o, o_lse, bsel
    torch.cuda.empty_cache()
    return out


class OracleCache:
    """Per (b, r) float64 keys/values and pyramid, computed lazily."""

    def __init__(self, pf: I.Prefill):
        self.pf = pf
        self._heads = {}

    def head(self, b, r):
        if (b, r) not in self._heads:
            k = self.pf.k.f64((b, r))
            v = self.pf.v.f64((b, r))
            self._heads[(b, r)] = (k, v, O.build_pyramid(k, self.pf.C, 2))
        return self._heads[(b, r)]

    def q(self, b, r, i):
        G = self.pf.G
        return self.pf.q.f64((b, slice(r * G, (r + 1) * G), i))  # [G, d]


def units_all(pf):
    return [(b, r, i) for b in range(pf.B) for r in range(pf.Hkv) for i in range(pf.N)]


def units_sample(pf, n, seed=0, extra=()):
    rng = np.random.default_rng(seed)
    U = pf.B * pf.Hkv * pf.N
    picks = set(int(x) for x in rng.choice(U, size=min(n, U), replace=False))
    # always include the edges of each head: first, last, leaf boundaries near the end
    for b in range(pf.B):
        for r in range(pf.Hkv):
            base = (b * pf.Hkv + r) * pf.N
            for i in (0, 1, pf.C - 1, pf.C, pf.N - 1, pf.N - pf.C, pf.N - 2):
                if 0 <= i < pf.N:
                    picks.add(base + i)
    for u in extra:
        picks.add(int(u))
    out = []
    for u in sorted(picks):
        bh, i = divmod(u, pf.N)
        out.append((bh // pf.Hkv, bh % pf.Hkv, i))
    return out


def units_stratified(pf, frac, seed=0, extra=()):
    """A seeded sample of at least `frac` of the units, stratified by KV head and by position (one draw
    in every block of round(1 / frac) consecutive positions), plus the head edges and `extra`."""
    rng = np.random.default_rng(seed)
    step = max(1, int(round(1.0 / frac)))
    picks = set()
    for b in range(pf.B):
        for r in range(pf.Hkv):
            base = (b * pf.Hkv + r) * pf.N
            starts = np.arange(0, pf.N, step)
            offs = rng.integers(0, step, size=starts.size)
            for i in np.minimum(starts + offs, pf.N - 1):
                picks.add(base + int(i))
    return units_sample(pf, 0, seed=seed, extra=sorted(picks | set(int(u) for u in extra)))


@dataclasses.dataclass
class Report:
    n_units: int = 0
    n_decided: int = 0
    n_undecided_equal: int = 0  # undecided units whose GPU selection still equals the oracle's
    sel_mismatch: list = dataclasses.field(default_factory=list)
    invariant_fail: list = dataclasses.field(default_factory=list)
    lse_err: float = 0.0
    attn_err: float = 0.0
    olse_err: float = 0.0
    bsa_units: int = 0
    bsa_mismatch: list = dataclasses.field(default_factory=list)
    bsa_decided: int = 0

    def merge(self, o: "Report"):
        self.n_units += o.n_units
        self.n_decided += o.n_decided
        self.n_undecided_equal += o.n_undecided_equal
        self.sel_mismatch += o.sel_mismatch[:20]
        self.invariant_fail += o.invariant_fail[:20]
        self.lse_err = max(self.lse_err, o.lse_err)
        self.attn_err = max(self.attn_err, o.attn_err)
        self.olse_err = max(self.olse_err, o.olse_err)
        self.bsa_units += o.bsa_units
        self.bsa_mismatch += o.bsa_mismatch[:20]
        self.bsa_decided += o.bsa_decided

    @property
    def decided_frac(self) -> float:
        return self.n_decided / max(1, self.n_units)


def check_invariants(sel_row, i, C, K):
    got = [int(j) for j in sel_row if j >= 0]
    ok = len(got) == min(K, i // C + 1)
    ok &= got == sorted(set(got))
    ok &= all(j * C <= i for j in got)
    ok &= all(int(j) == -1 for j in sel_row[len(got):])
    return ok


def invariant_violations(sel: np.ndarray, C: int) -> np.ndarray:
    """Vectorised selection invariants over every unit of sel [..., N, K]: the selected leaves are a
    left-packed prefix of min(K, i // C + 1) entries, strictly ascending and eligible (j C <= i), and the
    rest is -1. Returns the flat indices (over the leading dims and N) of the units that violate any."""
    *lead, N, K = sel.shape
    s = sel.reshape(-1, N, K).astype(np.int64)
    i = np.arange(N, dtype=np.int64)[None, :, None]
    valid = s >= 0
    want = np.minimum(K, np.arange(N) // C + 1)[None, :]
    bad = valid.sum(-1) != want
    bad |= (valid[..., 1:] & ~valid[..., :-1]).any(-1)  # a selected entry after a padding entry
    bad |= (valid[..., 1:] & (np.diff(s, axis=-1) <= 0)).any(-1)  # not strictly ascending
    bad |= (valid & (s * C > i)).any(-1)  # not eligible
    bad |= (~valid & (s != -1)).any(-1)  # padding other than -1
    return np.flatnonzero(bad.reshape(-1))


def _compare_chunk(task) -> Report:
    """Worker: compare the units of one chunk. Reads the inputs and the GPU outputs from _CTX."""
    pf, g, check_attn, check_bsa = _CTX["pf"], _CTX["g"], _CTX["attn"], _CTX["bsa"]
    oc = _CTX["oc"]
    rep = Report()
    G, C, K = pf.G, pf.C, pf.K
    for (b, r, i) in task:
        k, v, pyr = oc.head(b, r)
        qg = oc.q(b, r, i)
        us = O.select_unit(qg, k, pyr, i, K, pf.scale)
        gsel = g.sel[b, r, i]
        rep.n_units += 1
        if not check_invariants(gsel, i, C, K):
            rep.invariant_fail.append((b, r, i, gsel.tolist()))
        if us.margin >= MARGIN:
            rep.n_decided += 1
            if gsel.tolist() != us.sel.tolist():
                rep.sel_mismatch.append((b, r, i, gsel.tolist(), us.sel.tolist(), us.margin))
            elif g.sel_lse is not None:
                nsel = int((us.sel >= 0).sum())
                e = np.abs(g.sel_lse[b, r * G:(r + 1) * G, i, :nsel] - us.sel_lse[:, :nsel]).max()
                rep.lse_err = max(rep.lse_err, float(e))
        elif gsel.tolist() == us.sel.tolist():
            rep.n_undecided_equal += 1
        if check_attn and g.o is not None:
            o_ref, lse_ref = O.attend_unit(qg, k, v, gsel, i, C, pf.scale, pf.N)
            e = np.abs(g.o[b, r * G:(r + 1) * G, i] - o_ref).max()
            rep.attn_err = max(rep.attn_err, float(e))
            el = np.abs(g.o_lse[b, r * G:(r + 1) * G, i] - lse_ref).max()
            rep.olse_err = max(rep.olse_err, float(el))
        if check_bsa and g.bsa is not None:
            bsel, bm = O.bsa_select_unit(qg, pyr.means[0], i, C, K, pf.scale)
            rep.bsa_units += 1
            if bm >= MARGIN:
                rep.bsa_decided += 1
                if g.bsa[b, r, i].tolist() != bsel.tolist():
                    rep.bsa_mismatch.append((b, r, i, g.bsa[b, r, i].tolist(), bsel.tolist(), bm))
            if not check_invariants(g.bsa[b, r, i], i, C, K):
                rep.invariant_fail.append(("bsa", b, r, i))
    return rep


def compare(pf: I.Prefill, g: GpuOut, units, oc: OracleCache | None = None, check_attn=True, check_bsa=False,
            chunk=512) -> Report:
    """The oracle on `units` (a list of (b, r, i)) in the worker pool, compared with the GPU outputs."""
    oc = oc or OracleCache(pf)
    # the pyramids of the touched heads are built once, before the fork, and shared by the workers
    for (b, r) in sorted({(b, r) for (b, r, _) in units}):
        oc.head(b, r)
    units = list(units)
    tasks = [units[x:x + chunk] for x in range(0, len(units), chunk)]
    _CTX.update(pf=pf, g=g, attn=check_attn, bsa=check_bsa, oc=oc)
    try:
        reps = pool_map(_compare_chunk, tasks)
    finally:
        _CTX.clear()
    rep = Report()
    for r_ in reps:
        rep.merge(r_)
    return rep


def check_path(pf: I.Prefill, oc: "OracleCache", b: int, r: int, i: int, rows: np.ndarray, tol: float = MARGIN,
               ref=None):
    """One unit's traced selection path (rows: int [n_levels, K], row l = the nodes kept at level l)
    checked level by level, from the top, against the oracle's float64 scores of the path's own
    candidates: the candidates of level l are the eligible children of the nodes kept at level l + 1
    (every eligible node at the top level); if there are at most K, all of them must be kept; else
    exactly K of them, such that every kept candidate scores at least as high as every dropped one up to
    tol. This validates an undecided unit's whole path, not just its final selection.
    Returns (problems, same, gap): problems lists the violated levels, same is True if every level equals
    the oracle's own walk (ref: its UnitSelection, computed if not given), gap is the smallest
    (lowest kept - highest dropped) over the scored levels."""
    k, _, pyr = oc.head(b, r)
    qg = oc.q(b, r, i)
    C, g, K, L = pf.C, 2, pf.K, pyr.root_level
    problems = []
    gap = math.inf
    if rows.shape[0] != L + 1:
        return [f"{rows.shape[0]} trace levels for a pyramid of {L + 1}"], False, gap
    got = {l: [int(x) for x in rows[l] if x >= 0] for l in range(L + 1)}
    for l in range(L + 1):
        pad = rows[l][len(got[l]):]
        if (pad != -1).any() or got[l] != sorted(set(got[l])):
            problems.append(f"level {l}: not an ascending, left-packed, -1 padded list: {rows[l].tolist()}")
    if problems:
        return problems, False, gap
    for l in range(L, -1, -1):
        if l == L:
            cand = [j for j in range(pyr.means[L].shape[0]) if O.eligible(L, j, i, C, g)]
        else:
            cand = sorted(c for p in got[l + 1] for c in O.children(l + 1, p, pyr) if O.eligible(l, c, i, C, g))
        if len(cand) <= K:
            if got[l] != cand:
                problems.append(f"level {l}: {len(cand)} candidates must all be kept, got {got[l]}")
            continue
        if len(got[l]) != K or not set(got[l]) <= set(cand):
            problems.append(f"level {l}: kept {got[l]} is not K of the candidates {cand}")
            continue
        if l == 0:
            score = {j: float(O.leaf_lse_per_head(qg, k, j, i, C, pf.scale, pf.N).sum()) for j in cand}
        else:
            score = {j: float(O.node_lse_per_head(qg, pyr, l, j, i, pf.scale).sum()) for j in cand}
        low_kept = min(score[j] for j in got[l])
        high_dropped = max(score[j] for j in cand if j not in set(got[l]))
        gap = min(gap, low_kept - high_dropped)
        if low_kept < high_dropped - tol:
            problems.append(f"level {l}: kept score {low_kept:.6g} below dropped {high_dropped:.6g} - {tol}")
    ref = ref if ref is not None else O.select_unit(qg, k, pyr, i, K, pf.scale)
    same = all(got[l] == list(ref.kept[l]) for l in range(L + 1) if l in ref.kept)
    return problems, same, gap


@dataclasses.dataclass
class PathReport:
    n_units: int = 0
    n_same: int = 0  # paths equal to the oracle's walk at every level
    n_decided: int = 0
    decided_differ: list = dataclasses.field(default_factory=list)  # decided units whose path differs
    invalid: list = dataclasses.field(default_factory=list)  # paths that fail check_path
    min_gap: float = math.inf

    def merge(self, o: "PathReport"):
        self.n_units += o.n_units
        self.n_same += o.n_same
        self.n_decided += o.n_decided
        self.decided_differ += o.decided_differ[:20]
        self.invalid += o.invalid[:20]
        self.min_gap = min(self.min_gap, o.min_gap)


def _path_chunk(task) -> PathReport:
    pf, oc, trace = _CTX["pf"], _CTX["oc"], _CTX["trace"]
    rep = PathReport()
    for t, (b, r, i) in task:
        k, _, pyr = oc.head(b, r)
        ref = O.select_unit(oc.q(b, r, i), k, pyr, i, pf.K, pf.scale)
        problems, same, gap = check_path(pf, oc, b, r, i, trace[t], ref=ref)
        margin = ref.margin
        rep.n_units += 1
        rep.n_same += int(same)
        rep.min_gap = min(rep.min_gap, gap)
        if problems:
            rep.invalid.append((b, r, i, problems))
        if margin >= MARGIN:
            rep.n_decided += 1
            if not same:
                rep.decided_differ.append((b, r, i, margin))
    return rep


def compare_paths(pf: I.Prefill, trace: np.ndarray, units, oc: "OracleCache | None" = None, chunk=64) -> PathReport:
    """check_path over every traced unit (trace[t] is the path of units[t] = (b, r, i)) in the worker pool."""
    oc = oc or OracleCache(pf)
    for (b, r) in sorted({(b, r) for (b, r, _) in units}):
        oc.head(b, r)
    items = list(enumerate(units))
    tasks = [items[x:x + chunk] for x in range(0, len(items), chunk)]
    _CTX.update(pf=pf, oc=oc, trace=trace)
    try:
        reps = pool_map(_path_chunk, tasks)
    finally:
        _CTX.clear()
    rep = PathReport()
    for r_ in reps:
        rep.merge(r_)
    return rep


def assert_report(rep: Report, dtype: str, check_attn=True, min_decided=0.9, label=""):
    msg = (f"{label} units={rep.n_units} decided={rep.n_decided} ({rep.decided_frac:.4f}, floor {min_decided}) "
           f"undecided_equal={rep.n_undecided_equal} sel_mismatch={len(rep.sel_mismatch)} "
           f"invariant_fail={len(rep.invariant_fail)} lse_err={rep.lse_err:.3g} attn_err={rep.attn_err:.3g} "
           f"olse_err={rep.olse_err:.3g}")
    if rep.bsa_units:
        msg += f" bsa_units={rep.bsa_units} bsa_decided={rep.bsa_decided} bsa_mismatch={len(rep.bsa_mismatch)}"
    summary(msg.strip())
    assert not rep.invariant_fail, rep.invariant_fail[:5]
    assert not rep.sel_mismatch, rep.sel_mismatch[:5]
    assert not rep.bsa_mismatch, rep.bsa_mismatch[:5]
    assert rep.n_units > 0
    assert rep.decided_frac >= min_decided, (rep.decided_frac, min_decided)
    assert rep.lse_err <= 2e-4 if dtype == "bf16" else rep.lse_err <= 2e-5
    if check_attn:
        assert rep.attn_err <= TOL_ATTN[dtype], rep.attn_err
        assert rep.olse_err <= (2e-4 if dtype == "bf16" else 2e-5), rep.olse_err


def pyramid_err(pf: I.Prefill, g: GpuOut, oc: OracleCache, heads=None) -> float:
    n, offs, nodes = P.pisa_pyramid_layout(shape_of(pf, 1))
    err = 0.0
    heads = heads or [(b, r) for b in range(pf.B) for r in range(pf.Hkv)]
    for (b, r) in heads:
        _, _, pyr = oc.head(b, r)
        base = (b * pf.Hkv + r) * nodes
        for l in range(n):
            got = g.pyr[base + offs[l]: base + offs[l] + pyr.means[l].shape[0]]
            err = max(err, float(np.abs(got - pyr.means[l]).max()))
    return err
