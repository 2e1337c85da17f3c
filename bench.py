"""Benchmark of PISA's hot path on one MI355X.

One step = the whole prefill hot path on one batch of seeded synthetic input: mean pyramid, pyramid
Top-K selection (routing, regroup, tiled leaf LSE, Top-K), block-sparse attention over the selection,
and the flat block selection used for comparison. The headline value is routed query heads per second
of the pyramid selection (B * Hq * N / (pyramid + selection seconds)). Per-stage times come from HIP
events recorded by the library around each kernel launch on the stream it uses.

Besides the timed step the line carries: the q_tile 1 selection time, the decode step latency, a
crossover sweep of the pyramid selection against the flat selection at 16K-256K tokens (prefixes of
the 256K planted-needle workload, same heads), the needle recall@K at 256K, and the float64 oracle's
selection rate on the host cores.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "PISA Top-K selection ms & routed q-heads/s at 64K-256K; sparse-attn TFLOP/s"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def scored_levels(i, C, K, n_levels):
    """Levels >= 1 at which unit position i has more than K eligible nodes (scored levels)."""
    return sum(1 for l in range(1, n_levels) if i // (C << l) + 1 > K)


def work_counts(pf, sel):
    """Algorithmic work of the step, from the shapes and the GPU's own selection."""
    B, Hq, Hkv, G, N, d, C, K = pf.B, pf.Hq, pf.Hkv, pf.G, pf.N, pf.d, pf.C, pf.K
    n_levels = int(math.ceil(math.log2(max(1, -(-N // C))))) + 1
    i = np.arange(N, dtype=np.int64)
    # routing: per scored intermediate level about 2K candidates x 2 children, one dot of length d per
    # head each (the exact count differs at the causal edge by at most one child per level)
    s_lv = np.zeros(N, dtype=np.int64)
    for l in range(1, n_levels):
        s_lv += (i // (C << l) + 1 > K).astype(np.int64)
    route_flops = B * Hkv * int(s_lv.sum()) * 4 * K * 2 * G * d
    # leaf stage: kept level-1 nodes per unit (min(K, eligible level-1 nodes)), 2C keys each
    e1 = i // (2 * C) + 1
    pairs = B * Hkv * int(np.minimum(K, e1).sum())
    leaf_flops = pairs * 2 * C * 2 * G * d
    # attention: attended keys per (b, h, i) from the selection
    A = 0
    for b in range(B):
        for r in range(Hkv):
            s = sel[b, r].astype(np.int64)
            valid = s >= 0
            cnt = np.where(valid, np.minimum(C, i[:, None] - s * C + 1), 0)
            A += int(cnt.sum()) * G
    attn_flops = 4 * d * A
    # flat selection: one dot of length d per (unit, eligible leaf) after summing the group's heads
    n_elig = i // C + 1
    bsa_flops = B * Hkv * int(n_elig.sum()) * 2 * d + B * Hq * N * d
    pyr_bytes = B * Hkv * N * d * (2 if pf.dtype == "bf16" else 4)
    return dict(route_flops=route_flops, leaf_flops=leaf_flops, leaf_pairs=pairs, attn_flops=attn_flops,
                attended_keys=A, bsa_flops=bsa_flops, pyramid_read_bytes=pyr_bytes)


def measured_traffic(workload):
    """HBM bytes per launch and stage from the committed counter summary for this workload (FETCH_SIZE and
    WRITE_SIZE, each scaled by a plain copy's reading), or None when there is none or the kernel sources
    have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    from long_context_block_amd.profile_summary import source_digest
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != source_digest():
        return None
    return {st: e["bytes"] for st, e in t["stages"].items()}


# ---------------------------------------------------------------- the oracle on the host cores
# Worker context, set in the parent before the pool forks (the workers never touch the GPU).
_CTX = {}


def _pool_workers():
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return max(1, min(16, cores))


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass


def _pool_map(fn, tasks):
    import multiprocessing as mp
    with mp.get_context("fork").Pool(_pool_workers(), initializer=_pool_init) as pool:
        return pool.map(fn, tasks, chunksize=1)


def _oracle_pyramid(bh):
    import oracle as O
    pf = _CTX["pf"]
    b, r = divmod(bh, pf.Hkv)
    t = time.perf_counter()
    O.build_pyramid(pf.k.f64((b, r)), pf.C, 2)
    return time.perf_counter() - t


def _oracle_select(units):
    """Selections of a list of units (b, r, i); returns (seconds in select_unit, undecided count)."""
    import oracle as O
    pf, heads = _CTX["pf"], _CTX["heads"]
    el = 0.0
    und = 0
    for (b, r, i) in units:
        k, pyr = heads[(b, r)]
        qg = pf.q.f64((b, slice(r * pf.G, (r + 1) * pf.G), i))
        t = time.perf_counter()
        us = O.select_unit(qg, k, pyr, i, pf.K, pf.scale)
        el += time.perf_counter() - t
        und += us.margin < 1e-3
    return el, und


def cpu_baseline(pf, cpu_seconds=20.0, seed=0):
    """The float64 oracle as it stands: the pyramids of every KV head, then the selection walk of a
    random sample of units sized to about cpu_seconds of CPU work, both spread over a pool of worker
    processes on the host cores. value = q-heads / (pyramid wall time + sample wall time scaled to all
    units), the same quantity as the GPU's routed q-heads/s."""
    workers = _pool_workers()
    U = pf.B * pf.Hkv * pf.N
    rng = np.random.default_rng(seed)
    _CTX["pf"] = pf
    try:
        t = time.perf_counter()
        pyr_cpu = _pool_map(_oracle_pyramid, list(range(pf.B * pf.Hkv)))
        t_pyr = time.perf_counter() - t
        # the walks below read the pyramids built here once (the timed builds ran in the workers)
        import oracle as O
        heads = {}
        for b in range(pf.B):
            for r in range(pf.Hkv):
                k = pf.k.f64((b, r))
                heads[(b, r)] = (k, O.build_pyramid(k, pf.C, 2))
        _CTX["heads"] = heads
        # per-unit cost from a short probe, then a sample of about cpu_seconds of CPU work
        probe = [divmod(int(u), pf.N) for u in rng.choice(U, size=64, replace=False)]
        probe = [(bh // pf.Hkv, bh % pf.Hkv, i) for bh, i in probe]
        per_unit = max(_oracle_select(probe)[0] / len(probe), 1e-4)
        n = int(min(U, max(256, cpu_seconds / per_unit)))
        picks = np.sort(rng.choice(U, size=n, replace=False))
        units = [((int(u) // pf.N) // pf.Hkv, (int(u) // pf.N) % pf.Hkv, int(u) % pf.N) for u in picks]
        chunks = [units[x::workers * 4] for x in range(workers * 4)]
        t = time.perf_counter()
        res = _pool_map(_oracle_select, chunks)
        t_sel = time.perf_counter() - t
    finally:
        _CTX.clear()
    cpu_sel = sum(x[0] for x in res)
    und = sum(x[1] for x in res)
    full_s = t_pyr + t_sel * U / n
    return {"value": round(pf.B * pf.Hq * pf.N / full_s, 1), "unit": "q-heads/s", "cores": workers, "kind": "oracle",
            "sample": f"float64 oracle in {workers} worker processes (one thread each): pyramids of all "
                      f"{pf.B * pf.Hkv} KV heads ({t_pyr:.2f} s wall, {sum(pyr_cpu):.2f} s CPU), then the "
                      f"selection walk of {n} random units of {U} ({t_sel:.2f} s wall, {cpu_sel:.1f} s CPU); "
                      f"full-problem time extrapolated as pyramid + sample x {U / n:.1f} = {full_s:.1f} s; "
                      f"{und / n:.3f} of the sampled units are undecided (margin < 1e-3)",
            "full_problem_s_extrapolated": round(full_s, 2), "undecided_frac_sample": round(float(und) / n, 4)}


def decode_latency(P, I, torch, steps_cap=None):
    """Per-step latency of the fused decode step on the 8 x 128K-token decode workload (256 steps)."""
    dec = I.make_workload("decode_128k")

    def dev(x):
        if x.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x.data).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x.data)).cuda()

    s = P.make_shape(batch=dec.B, seq_len=dec.Nmax, n_q_heads=dec.Hq, n_kv_heads=dec.Hkv, head_dim=dec.d,
                     block=dec.C, top_k=dec.K, q_tile=1, dtype=dec.dtype)
    kc, vc = dev(dec.k_cache), dev(dec.v_cache)
    qn, kn, vn = dev(dec.q_new), dev(dec.k_new), dev(dec.v_new)
    rows = P.pyramid_rows(s)
    psum = torch.zeros((rows, dec.d), dtype=torch.float32, device="cuda")
    pmean = torch.zeros_like(psum)
    o = torch.empty((dec.B, dec.Hq, dec.d), dtype=qn.dtype, device="cuda")
    sel = torch.empty((dec.B, dec.Hkv, dec.K), dtype=torch.int32, device="cuda")
    lens0 = [int(x) for x in dec.lens0]
    steps = dec.steps if steps_cap is None else min(steps_cap, dec.steps)
    ws = P.alloc_workspace(s, P.PISA_OP_DECODE)

    def run(record):
        P.pisa_build_pyramid(s, kc, pmean, psum, host_lens=lens0)
        lens = list(lens0)
        evs = []
        if record:
            # a device-side delay first, so that the host has queued every step before the GPU reaches
            # it: the events then bracket the kernel alone, not the host's launch cadence
            torch.cuda._sleep(100_000_000)
        for st in range(steps):
            if record:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
            P.pisa_decode_step(s, lens, qn[st], kn[st], vn[st], kc, vc, psum, pmean, o, sel, ws=ws)
            if record:
                b.record()
                evs.append((a, b))
            lens = [x + 1 for x in lens]
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    run(False)  # warm-up pass (the timed pass rebuilds the pyramid and rewrites the same cache rows)
    t = np.array(run(True))
    return {"workload": "decode_128k", "batch": dec.B, "cache_tokens": int(dec.lens0[0]), "steps": int(steps),
            "n_q_heads": dec.Hq, "n_kv_heads": dec.Hkv, "top_k": dec.K, "block": dec.C,
            "step_ms_median": round(float(np.median(t)), 4), "step_ms_p99": round(float(np.percentile(t, 99)), 4),
            "step_ms_mean": round(float(t.mean()), 4)}


def _needle_oracle(units):
    """Oracle selections of needle units: recall@K of each against its eligible needle leaves."""
    import oracle as O
    pf, heads = _CTX["pf"], _CTX["heads"]
    out = []
    for (b, r, i) in units:
        E = [int(j) for j in pf.needle_leaves[b, r] if j * pf.C <= i]
        k, pyr = heads[(b, r)]
        us = O.select_unit(pf.q.f64((b, slice(r * pf.G, (r + 1) * pf.G), i)), k, pyr, i, pf.K, pf.scale)
        out.append(len(set(us.sel.tolist()) & set(E)) / min(pf.K, len(E)))
    return out


def quality_measures(P, torch, pf, positions, q_tile):
    """Selection quality on one workload at the given query positions (digest 关键实验: Recall@K and the
    attention mass ratio): the dense causal pass scores every leaf at those positions; from it the flat
    exact Top-K, and for the pyramid selection, the flat selection (bsa_select) and the flat exact
    Top-K itself, the mean Recall@K against the flat exact Top-K and the mean share of full attention's
    softmax mass inside the selected blocks."""
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x.data).view(np.int16)).cuda().view(torch.bfloat16)
    q, k = dev(pf.q), dev(pf.k)
    s = P.make_shape(batch=pf.B, seq_len=pf.N, n_q_heads=pf.Hq, n_kv_heads=pf.Hkv, head_dim=pf.d, block=pf.C,
                     top_k=pf.K, q_tile=q_tile, dtype=pf.dtype)
    pyr = torch.empty((P.pyramid_rows(s), pf.d), dtype=torch.float32, device="cuda")
    P.pisa_build_pyramid(s, k, pyr)
    sels = {"pisa": torch.empty((pf.B, pf.Hkv, pf.N, pf.K), dtype=torch.int32, device="cuda")}
    P.pisa_select(s, q, k, pyr, sels["pisa"], None, P.alloc_workspace(s, P.PISA_OP_SELECT))
    sels["bsa"] = torch.empty_like(sels["pisa"])
    P.bsa_select(s, q, k, sels["bsa"], P.alloc_workspace(s, P.PISA_OP_BSA))
    pos = torch.tensor(positions, dtype=torch.int32, device="cuda")
    n0, npos = -(-pf.N // pf.C), len(positions)
    leaf = torch.empty((pf.B, pf.Hq, npos, n0), dtype=torch.float32, device="cuda")
    row = torch.empty((pf.B, pf.Hq, npos), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    P.pisa_stage_timing(True)
    P.pisa_flat_leaf_lse(s, q, k, pos, leaf, row)
    torch.cuda.synchronize()
    flat_ms = P.pisa_stage_times()["flat_leaf_lse"][0]
    P.pisa_stage_timing(False)
    flat = torch.empty((pf.B, pf.Hkv, npos, pf.K), dtype=torch.int32, device="cuda")
    rec = torch.empty((pf.B, pf.Hkv, npos), dtype=torch.float32, device="cuda")
    mass = torch.empty((pf.B, pf.Hq, npos), dtype=torch.float32, device="cuda")
    out = {"positions": npos, "position_sample": "all" if npos == pf.N else "seeded uniform sample"}
    for name in ("pisa", "bsa", "flat_exact"):
        if name == "flat_exact":
            # the flat exact Top-K placed at its positions of a full selection array
            sx = torch.full_like(sels["pisa"], -1)
            sx[:, :, pos.long()] = flat
        else:
            sx = sels[name]
        P.pisa_selection_quality(s, leaf, row, pos, sx, flat, rec, mass)
        torch.cuda.synchronize()
        out[f"{name}_recall_at_k"] = round(float(rec.mean()), 4)
        out[f"{name}_attention_mass"] = round(float(mass.mean()), 4)
    i = np.asarray(positions, dtype=np.int64)
    dense_flops = 2 * pf.B * pf.Hq * pf.d * int(((i // (2 * pf.C) + 1) * 2 * pf.C).sum())
    out["dense_pass_ms"] = round(flat_ms, 3)
    out["dense_pass_tflops"] = round(dense_flops / (flat_ms * 1e-3) / 1e12, 1)
    del q, k, pyr, sels, leaf, row, flat, rec, mass
    torch.cuda.empty_cache()
    return out


ABLATIONS = [  # name, pool, score, budget, max_level (None: from the root)
    ("method (LSE, mean pooling, fixed K)", "mean", "lse", "fixed", None),
    ("PISA-1 (mean scoring)", "mean", "mean", "fixed", None),
    ("PISA-2 (mean + variance scoring)", "mean", "mean_var", "fixed", None),
    ("sum pooling", "sum", "lse", "fixed", None),
    ("max pooling", "max", "lse", "fixed", None),
    ("halving budget", "mean", "lse", "halving", None),
    ("pool chain truncated at level 4", "mean", "lse", "fixed", 4),
]


def ablations(P, torch, pf, positions, reps=2):
    """The selection variants on one workload: time of the pooled pyramid + variant walk, and the Recall@K
    against the flat exact Top-K and the attention mass of each variant's selection at the positions."""
    pool_id = {"mean": P.PISA_POOL_MEAN, "sum": P.PISA_POOL_SUM, "max": P.PISA_POOL_MAX}
    score_id = {"lse": P.PISA_SCORE_LSE, "mean": P.PISA_SCORE_MEAN, "mean_var": P.PISA_SCORE_MEAN_VAR}
    budget_id = {"fixed": P.PISA_BUDGET_FIXED, "halving": P.PISA_BUDGET_HALVING}
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x.data).view(np.int16)).cuda().view(torch.bfloat16)
    q, k = dev(pf.q), dev(pf.k)
    s = P.make_shape(batch=pf.B, seq_len=pf.N, n_q_heads=pf.Hq, n_kv_heads=pf.Hkv, head_dim=pf.d, block=pf.C,
                     top_k=pf.K, q_tile=1, dtype=pf.dtype)
    rows = P.pyramid_rows(s)
    summ = torch.empty((rows, pf.d), dtype=torch.float32, device="cuda")
    var = torch.empty_like(summ)
    pos = torch.tensor(positions, dtype=torch.int32, device="cuda")
    n0, npos = -(-pf.N // pf.C), len(positions)
    leaf = torch.empty((pf.B, pf.Hq, npos, n0), dtype=torch.float32, device="cuda")
    row = torch.empty((pf.B, pf.Hq, npos), dtype=torch.float32, device="cuda")
    P.pisa_flat_leaf_lse(s, q, k, pos, leaf, row)
    flat = torch.empty((pf.B, pf.Hkv, npos, pf.K), dtype=torch.int32, device="cuda")
    rec = torch.empty((pf.B, pf.Hkv, npos), dtype=torch.float32, device="cuda")
    mass = torch.empty((pf.B, pf.Hq, npos), dtype=torch.float32, device="cuda")
    sel = torch.empty((pf.B, pf.Hkv, pf.N, pf.K), dtype=torch.int32, device="cuda")
    out = {"workload": "prefill_64k" if pf.N == 65536 else f"N={pf.N}", "positions": npos, "variants": {}}
    for name, pool, score, budget, cap in ABLATIONS:
        v = P.Variant(score_id[score], budget_id[budget], -1 if cap is None else cap)
        vv = var if score == "mean_var" else None

        def once():
            P.pisa_build_pyramid_pooled(s, k, pool_id[pool], summ, vv)
            P.pisa_select_variant(s, v, q, k, summ, sel, vv)

        once()
        torch.cuda.synchronize()
        P.pisa_stage_timing(True)
        for _ in range(reps):
            once()
        torch.cuda.synchronize()
        st = {n: t / reps for n, (t, c) in P.pisa_stage_times().items()}  # per call (a stage may launch per chunk)
        P.pisa_stage_timing(False)
        P.pisa_selection_quality(s, leaf, row, pos, sel, flat, rec, mass)
        torch.cuda.synchronize()
        out["variants"][name] = {"pool": pool, "score": score, "budget": budget, "max_level": cap,
                                 "ms": round(st.get("pyramid_pooled", 0.0) + st.get("select_variant", 0.0), 3),
                                 "recall_at_k": round(float(rec.mean()), 4),
                                 "attention_mass": round(float(mass.mean()), 4)}
        log(f"[bench] ablation {name}: {out['variants'][name]}")
    del q, k, summ, var, pos, leaf, row, flat, rec, mass, sel
    torch.cuda.empty_cache()
    return out


def crossover(P, I, torch, lengths=(16384, 32768, 65536, 131072, 262144), reps=4, oracle_needles=256):
    """Pyramid selection (pyramid + pisa_select, q_tile 4) against the flat selection (bsa_select, its
    own leaf pooling included) on prefixes of the 256K planted-needle workload (32 query / 8 KV heads,
    d 128, C 64, K 16, AR(1) keys), and the needle recall@K of the 256K selection."""
    import oracle as O
    log("[bench] crossover: generating prefill_256k_needles")
    t = time.time()
    pf = I.make_workload("prefill_256k_needles")
    log(f"[bench] generated in {time.time() - t:.1f}s")
    qa = torch.from_numpy(pf.q.data.view(np.int16)).cuda().view(torch.bfloat16)
    ka = torch.from_numpy(pf.k.data.view(np.int16)).cuda().view(torch.bfloat16)
    points = []
    sel_full = None
    for N in lengths:
        q = qa if N == pf.N else qa[:, :, :N].contiguous()
        k = ka if N == pf.N else ka[:, :, :N].contiguous()
        s = P.make_shape(batch=pf.B, seq_len=N, n_q_heads=pf.Hq, n_kv_heads=pf.Hkv, head_dim=pf.d, block=pf.C,
                         top_k=pf.K, q_tile=4, dtype=pf.dtype)
        pyr = torch.empty((P.pyramid_rows(s), pf.d), dtype=torch.float32, device="cuda")
        sel = torch.empty((pf.B, pf.Hkv, N, pf.K), dtype=torch.int32, device="cuda")
        bsel = torch.empty_like(sel)
        ws = P.alloc_workspace(s, P.PISA_OP_SELECT)
        wsb = P.alloc_workspace(s, P.PISA_OP_BSA)

        def once():
            P.pisa_build_pyramid(s, k, pyr)
            P.pisa_select(s, q, k, pyr, sel, None, ws)
            P.bsa_select(s, q, k, bsel, wsb)

        once()
        torch.cuda.synchronize()
        P.pisa_stage_timing(True)
        for _ in range(reps):
            once()
        torch.cuda.synchronize()
        st = {n: tot / reps for n, (tot, c) in P.pisa_stage_times().items()}  # per call
        P.pisa_stage_timing(False)
        pisa_ms = sum(st.get(n, 0.0) for n in ("pyramid", "route_planes", "route", "regroup_select", "leaf_lse",
                                                "finalize"))
        bsa_ms = st.get("bsa_pool", 0.0) + st.get("bsa_select", 0.0)
        i = np.arange(N, dtype=np.int64)
        n_levels = int(math.ceil(math.log2(max(1, -(-N // pf.C))))) + 1
        s_lv = sum((i // (pf.C << l) + 1 > pf.K).astype(np.int64) for l in range(1, n_levels))
        pisa_flops = pf.B * pf.Hkv * (int(s_lv.sum()) * 4 * pf.K * 2 * pf.G * pf.d +
                                      int(np.minimum(pf.K, i // (2 * pf.C) + 1).sum()) * 4 * pf.C * pf.G * pf.d)
        bsa_flops = pf.B * pf.Hkv * int((i // pf.C + 1).sum()) * 2 * pf.d
        points.append({"seq_len": N, "pisa_selection_ms": round(pisa_ms, 4), "bsa_selection_ms": round(bsa_ms, 4),
                       "bsa_over_pisa_time": round(bsa_ms / pisa_ms, 3), "pisa_flops": pisa_flops,
                       "bsa_flops": bsa_flops,
                       "pisa_stages_ms": {n: round(st[n], 4) for n in sorted(st) if not n.startswith("bsa")}})
        log(f"[bench] crossover N={N}: pisa {pisa_ms:.3f} ms, bsa {bsa_ms:.3f} ms")
        if N == pf.N:
            sel_full = sel.cpu().numpy()
        del q, k, pyr, sel, bsel, ws, wsb
        torch.cuda.empty_cache()
    del qa, ka
    torch.cuda.empty_cache()
    res = {"workload": "prefixes of prefill_256k_needles", "n_q_heads": pf.Hq, "n_kv_heads": pf.Hkv,
           "head_dim": pf.d, "block": pf.C, "top_k": pf.K, "q_tile": 4, "reps": reps, "points": points}
    if sel_full is not None:
        # needle recall@K = |sel(r, i) & E| / min(K, |E|), E = the eligible needle leaves, over every
        # needle query row (GPU) and, on a sample of needle units, for the oracle as well
        rec, units = [], []
        for b in range(pf.B):
            for h in range(pf.Hq):
                r = h // pf.G
                leaves = np.asarray(pf.needle_leaves[b, r])
                for i in pf.needle_queries[b, h]:
                    E = leaves[leaves * pf.C <= i]
                    if E.size:
                        row = sel_full[b, r, int(i)]
                        rec.append(np.isin(row[row >= 0], E).sum() / min(pf.K, E.size))
                        if h % pf.G == 0:
                            units.append((b, r, int(i)))
        rng = np.random.default_rng(3)
        pick = [units[x] for x in sorted(rng.choice(len(units), size=min(oracle_needles, len(units)), replace=False))]
        heads = {}
        for (b, r) in sorted({(b, r) for (b, r, _) in pick}):
            kk = pf.k.f64((b, r))
            heads[(b, r)] = (kk, O.build_pyramid(kk, pf.C, 2))
        _CTX.update(pf=pf, heads=heads)
        try:
            workers = _pool_workers()
            orc = [x for part in _pool_map(_needle_oracle, [pick[j::workers] for j in range(workers)]) for x in part]
        finally:
            _CTX.clear()
        gpu_s = []
        for (b, r, i) in pick:
            E = [int(j) for j in pf.needle_leaves[b, r] if j * pf.C <= i]
            gpu_s.append(len(set(sel_full[b, r, i].tolist()) & set(E)) / min(pf.K, len(E)))
        # the flat exact Top-K (every leaf scored exactly) at the sampled needle positions: how findable
        # the planted needles are for any selection of K leaves
        pos_l = sorted({i for (_, _, i) in pick})
        s = P.make_shape(batch=pf.B, seq_len=pf.N, n_q_heads=pf.Hq, n_kv_heads=pf.Hkv, head_dim=pf.d, block=pf.C,
                         top_k=pf.K, q_tile=4, dtype=pf.dtype)
        qa = torch.from_numpy(pf.q.data.view(np.int16)).cuda().view(torch.bfloat16)
        ka = torch.from_numpy(pf.k.data.view(np.int16)).cuda().view(torch.bfloat16)
        pos = torch.tensor(pos_l, dtype=torch.int32, device="cuda")
        n0 = -(-pf.N // pf.C)
        leaf = torch.empty((pf.B, pf.Hq, len(pos_l), n0), dtype=torch.float32, device="cuda")
        row = torch.empty((pf.B, pf.Hq, len(pos_l)), dtype=torch.float32, device="cuda")
        P.pisa_flat_leaf_lse(s, qa, ka, pos, leaf, row)
        dummy = torch.full((pf.B, pf.Hkv, pf.N, pf.K), -1, dtype=torch.int32, device="cuda")
        flat = torch.empty((pf.B, pf.Hkv, len(pos_l), pf.K), dtype=torch.int32, device="cuda")
        rr = torch.empty((pf.B, pf.Hkv, len(pos_l)), dtype=torch.float32, device="cuda")
        mm = torch.empty((pf.B, pf.Hq, len(pos_l)), dtype=torch.float32, device="cuda")
        P.pisa_selection_quality(s, leaf, row, pos, dummy, flat, rr, mm)
        flat_np = flat.cpu().numpy()
        del qa, ka, pos, leaf, row, dummy, flat, rr, mm
        torch.cuda.empty_cache()
        at = {i: x for x, i in enumerate(pos_l)}
        flat_rec = []
        for (b, r, i) in pick:
            E = [int(j) for j in pf.needle_leaves[b, r] if j * pf.C <= i]
            flat_rec.append(len(set(flat_np[b, r, at[i]].tolist()) & set(E)) / min(pf.K, len(E)))
        res["needle_recall_at_k"] = {"gpu_all_needle_queries": round(float(np.mean(rec)), 4),
                                     "needle_query_rows": len(rec),
                                     "sample_units": len(pick), "gpu_on_sample": round(float(np.mean(gpu_s)), 4),
                                     "oracle_on_sample": round(float(np.mean(orc)), 4),
                                     "flat_exact_topk_on_sample": round(float(np.mean(flat_rec)), 4)}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_64k")
    ap.add_argument("--q-tile", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="CPU seconds of oracle work in the host-core baseline sample")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-crossover", action="store_true")
    ap.add_argument("--no-quality", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes three times (the reference kernel that "
                         "scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py measures one GPU: every box in this setup has one GPU and the path is not sharded "
              "across GPUs here (see the design notes for how it would shard). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_block_amd import inputs as I
    from long_context_block_amd import pisa as P

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": args.copy_calibration, "launches": 3}))
        return
    log(f"[bench] generating {args.workload}")
    t = time.time()
    pf = I.make_workload(args.workload)
    log(f"[bench] generated in {time.time() - t:.1f}s: B={pf.B} Hq={pf.Hq} Hkv={pf.Hkv} N={pf.N} d={pf.d} "
        f"C={pf.C} K={pf.K} {pf.dtype}")
    qt = max(1, min(args.q_tile, 16 // pf.G))

    def dev(x):
        if x.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x.data).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x.data)).cuda()

    q, k, v = dev(pf.q), dev(pf.k), dev(pf.v)
    s = P.make_shape(batch=pf.B, seq_len=pf.N, n_q_heads=pf.Hq, n_kv_heads=pf.Hkv, head_dim=pf.d, block=pf.C,
                     top_k=pf.K, q_tile=qt, dtype=pf.dtype)
    pyr = torch.empty((P.pyramid_rows(s), pf.d), dtype=torch.float32, device="cuda")
    sel = torch.empty((pf.B, pf.Hkv, pf.N, pf.K), dtype=torch.int32, device="cuda")
    bsel = torch.empty_like(sel)
    o = torch.empty_like(q)
    ws_sel = P.alloc_workspace(s, P.PISA_OP_SELECT)
    ws_att = P.alloc_workspace(s, P.PISA_OP_ATTN)
    ws_bsa = P.alloc_workspace(s, P.PISA_OP_BSA)
    log(f"[bench] workspaces: select {ws_sel.numel() / 2**20:.0f} MiB, attention {ws_att.numel() / 2**20:.0f} MiB, "
        f"bsa {ws_bsa.numel() / 2**20:.0f} MiB")

    def step():
        P.pisa_build_pyramid(s, k, pyr)
        P.pisa_select(s, q, k, pyr, sel, None, ws_sel)
        P.pisa_sparse_attn(s, q, k, v, sel, o, None, ws_att)
        P.bsa_select(s, q, k, bsel, ws_bsa)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("[bench] warmup done")
    P.pisa_stage_timing(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / args.steps
    stages = P.pisa_stage_times()
    P.pisa_stage_timing(False)
    # per step: a stage's launches in one step add up (the attention launches once per chunk of slices)
    st_ms = {name: tot / args.steps for name, (tot, cnt) in stages.items()}
    launches = {name: cnt // args.steps for name, (tot, cnt) in stages.items()}
    log(f"[bench] step {step_ms:.3f} ms (wall {wall / args.steps * 1e3:.3f} ms); stages " +
        ", ".join(f"{n}={v:.3f}" for n, v in sorted(st_ms.items())))

    # the same selection with q_tile 1 (one unit per leaf-stage tile), for the q_tile comparison
    sel_q1_ms = None
    if qt > 1:
        s1 = P.make_shape(batch=pf.B, seq_len=pf.N, n_q_heads=pf.Hq, n_kv_heads=pf.Hkv, head_dim=pf.d, block=pf.C,
                          top_k=pf.K, q_tile=1, dtype=pf.dtype)
        ws1 = P.alloc_workspace(s1, P.PISA_OP_SELECT)
        sel1 = torch.empty_like(sel)
        for _ in range(2):
            P.pisa_select(s1, q, k, pyr, sel1, None, ws1)
        torch.cuda.synchronize()
        P.pisa_stage_timing(True)
        n1 = max(2, args.steps // 2)
        for _ in range(n1):
            P.pisa_build_pyramid(s1, k, pyr)
            P.pisa_select(s1, q, k, pyr, sel1, None, ws1)
        torch.cuda.synchronize()
        st1 = P.pisa_stage_times()
        P.pisa_stage_timing(False)
        sel_q1_ms = sum(tot / n1 for name, (tot, cnt) in st1.items())
        del ws1, sel1
    sel_np = sel.cpu().numpy()
    w = work_counts(pf, sel_np)
    sel_stage_names = ["pyramid", "route_planes", "route", "regroup_select", "leaf_lse", "finalize", "route_fused_leaf"]
    selection_ms = sum(st_ms.get(n, 0.0) for n in sel_stage_names)
    attn_ms = sum(st_ms.get(n, 0.0) for n in ("regroup_attn", "attn_leaf", "attn_merge"))
    bsa_ms = st_ms.get("bsa_pool", 0.0) + st_ms.get("bsa_select", 0.0)
    qheads = pf.B * pf.Hq * pf.N
    value = qheads / (selection_ms * 1e-3)
    peak_mma = PEAK_BF16_TFLOPS if pf.dtype == "bf16" else PEAK_FP32_TFLOPS

    # the dominant kernel and its roofline
    kern = {
        "route": ("mfma", w["route_flops"], st_ms.get("route", 0.0)),
        "leaf_lse": ("mfma", w["leaf_flops"], st_ms.get("leaf_lse", 0.0)),
        "attn_leaf": ("mfma", w["attn_flops"], st_ms.get("attn_leaf", 0.0)),
        "bsa_select": ("mfma", w["bsa_flops"], st_ms.get("bsa_select", 0.0)),
        "pyramid": ("hbm", w["pyramid_read_bytes"], st_ms.get("pyramid", 0.0)),
    }
    # the dominant kernel of the PISA path; the flat selection is the comparison baseline (listed below)
    dom = max((n for n in kern if n != "bsa_select"), key=lambda n: kern[n][2])
    bound, amount, ms = kern[dom]
    traffic = measured_traffic(args.workload)
    if bound == "hbm":
        achieved, peak, unit = amount / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = amount / (ms * 1e-3) / 1e12, peak_mma, "TFLOP/s"
    per_kernel = {}
    for n, (bd, amt, kms) in kern.items():
        if kms <= 0:
            continue
        if traffic and n in traffic:
            # the counter summary is per launch; a stage may launch once per chunk of slices in a step
            per_kernel.setdefault(n, {})["hbm_bytes_measured"] = round(traffic[n] * launches.get(n, 1))
            per_kernel[n]["hbm_GB/s_measured"] = round(traffic[n] * launches.get(n, 1) / (kms * 1e-3) / 1e9, 1)
        if bd == "hbm":
            per_kernel.setdefault(n, {}).update({"ms": round(kms, 4), "GB/s": round(amt / (kms * 1e-3) / 1e9, 1),
                                                 "frac_hbm": round(amt / (kms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})
        else:
            tf = amt / (kms * 1e-3) / 1e12
            per_kernel.setdefault(n, {}).update({"ms": round(kms, 4), "TFLOP/s": round(tf, 2),
                                                 "frac_mfma": round(tf / peak_mma, 4)})

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "q-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": pf.dtype,
        "data": "synthetic (seeded; AR(1) keys, i.i.d. queries and values)",
        "config": {"workload": args.workload, "batch": pf.B, "seq_len": pf.N, "n_q_heads": pf.Hq,
                   "n_kv_heads": pf.Hkv, "head_dim": pf.d, "block": pf.C, "top_k": pf.K, "branch": 2, "q_tile": qt},
        "selection_ms": round(selection_ms, 4),
        "selection_ms_q_tile_1": round(sel_q1_ms, 4) if sel_q1_ms else None,
        "sparse_attn_ms": round(attn_ms, 4),
        "sparse_attn_tflops": round(w["attn_flops"] / (attn_ms * 1e-3) / 1e12, 2) if attn_ms else None,
        "bsa_select_ms": round(bsa_ms, 4),
        "pisa_over_bsa_time": round(selection_ms / bsa_ms, 3) if bsa_ms else None,
        "stages_ms": {n: round(v_, 4) for n, v_ in sorted(st_ms.items())},
        "kernels": per_kernel,
        "work": w,
        "roofline": {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4),
                     "traffic": round(traffic[dom]) if traffic and dom in traffic else None,
                     "launches_per_step": launches.get(dom, 1)},
    }
    if not args.no_backward and pf.dtype == "bf16":
        # backward of the sparse attention on this step's selection: forward with its LSE once, then the
        # timed backward passes (seeded dO)
        o_lse = torch.empty((pf.B, pf.Hq, pf.N), dtype=torch.float32, device="cuda")
        P.pisa_sparse_attn(s, q, k, v, sel, o, o_lse, ws_att)
        del ws_att, ws_sel, ws_bsa
        torch.cuda.empty_cache()
        gen = torch.Generator(device="cuda").manual_seed(7)
        d_o = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_b = P.alloc_workspace(s, P.PISA_OP_ATTN_BWD)
        P.pisa_sparse_attn_backward(s, q, k, v, sel, o, o_lse, d_o, dq, dk, dv, ws_b)
        torch.cuda.synchronize()
        P.pisa_stage_timing(True)
        nb = max(2, args.steps // 2)
        for _ in range(nb):
            P.pisa_sparse_attn_backward(s, q, k, v, sel, o, o_lse, d_o, dq, dk, dv, ws_b)
        torch.cuda.synchronize()
        stb = {n_: t_ / nb for n_, (t_, c_) in P.pisa_stage_times().items()}  # per call
        P.pisa_stage_timing(False)
        b_ms = stb.get("regroup_attn_bwd", 0.0) + stb.get("attn_backward", 0.0)
        b_flops = 10 * pf.d * w["attended_keys"]  # S, dP, dV, dK and dQ: five products of 2 d per attended key
        out["backward"] = {"ms": round(b_ms, 4), "algorithmic_flops": b_flops,
                           "TFLOP/s": round(b_flops / (b_ms * 1e-3) / 1e12, 2),
                           "frac_mfma": round(b_flops / (b_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "stages_ms": {n_: round(t_, 4) for n_, t_ in sorted(stb.items())}}
        log(f"[bench] backward {out['backward']}")
        del o_lse, d_o, dq, dk, dv, ws_b
    else:
        del ws_att, ws_sel, ws_bsa
    del q, k, v, o, pyr, sel, bsel
    torch.cuda.empty_cache()
    if not args.no_decode:
        log("[bench] decode: generating the 8 x 128K cache and timing 256 steps")
        out["decode"] = decode_latency(P, I, torch)
        log(f"[bench] decode {out['decode']}")
    if not args.no_quality:
        log("[bench] selection quality (Recall@K, attention mass) at 16K and 64K")
        qual = {}
        pf16 = I.make_workload("prefill_16k")
        qual["prefill_16k"] = quality_measures(P, torch, pf16, list(range(pf16.N)), q_tile=2)
        del pf16
        rng = np.random.default_rng(12)
        pos64 = sorted(rng.choice(pf.N, 2048, replace=False).tolist()) if args.workload == "prefill_64k" else None
        if pos64 is not None:
            qual["prefill_64k"] = quality_measures(P, torch, pf, pos64, q_tile=4)
            log("[bench] selection variants at 64K")
            qual["ablations"] = ablations(P, torch, pf, pos64)
        out["quality"] = qual
        log(f"[bench] quality {json.dumps(qual)}")
    if not args.no_crossover:
        out["crossover"] = crossover(P, I, torch)
        log(f"[bench] crossover {json.dumps(out['crossover'])}")
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle's selection on the host cores")
        out["cpu_baseline"] = cpu_baseline(pf, args.cpu_seconds)
        log(f"[bench] cpu_baseline {out['cpu_baseline']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
