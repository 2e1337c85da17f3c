"""Benchmark of PISA's hot path on one MI355X.

One step = the whole prefill hot path on one batch of seeded synthetic input: mean pyramid, pyramid
Top-K selection (routing, regroup, tiled leaf LSE, Top-K), block-sparse attention over the selection,
and the flat block selection used for comparison. The headline value is routed query heads per second
of the pyramid selection (B * Hq * N / (pyramid + selection seconds)). Per-stage times come from HIP
events recorded by the library around each kernel launch on the stream it uses.

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


def cpu_baseline(pf, seconds_target=15.0, seed=0):
    """The float64 oracle (as it stands) on a bounded random sample of units, one thread."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    rng = np.random.default_rng(seed)
    U = pf.B * pf.Hkv * pf.N
    order = rng.permutation(U)
    heads = {}
    t0 = time.perf_counter()
    done = 0
    t_pyr = 0.0
    for u in order:
        bh, i = divmod(int(u), pf.N)
        b, r = divmod(bh, pf.Hkv)
        if (b, r) not in heads:
            tp = time.perf_counter()
            k = pf.k.f64((b, r))
            v = pf.v.f64((b, r))
            heads[(b, r)] = (k, v, O.build_pyramid(k, pf.C, 2))
            t_pyr += time.perf_counter() - tp
        k, v, pyr = heads[(b, r)]
        qg = pf.q.f64((b, slice(r * pf.G, (r + 1) * pf.G), i))
        us = O.select_unit(qg, k, pyr, i, pf.K, pf.scale)
        O.attend_unit(qg, k, v, us.sel, i, pf.C, pf.scale, pf.N)
        done += 1
        if time.perf_counter() - t0 > seconds_target:
            break
    el = time.perf_counter() - t0 - t_pyr
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    qheads_per_s = done * pf.G / el
    return {"value": qheads_per_s, "unit": "q-heads/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} random units (of {U}) of the same workload: float64 selection walk + sparse "
                      f"attention per unit, one thread, pyramid build of the touched heads excluded "
                      f"({t_pyr:.1f}s); value = units*G/s"}


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

    def run(record):
        P.pisa_build_pyramid(s, kc, pmean, psum, host_lens=lens0)
        lens = list(lens0)
        evs = []
        for st in range(steps):
            if record:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
            P.pisa_decode_step(s, lens, qn[st], kn[st], vn[st], kc, vc, psum, pmean, o, sel)
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_64k")
    ap.add_argument("--q-tile", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-decode", action="store_true")
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
    st_ms = {name: tot / cnt for name, (tot, cnt) in stages.items()}
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
        sel_q1_ms = sum(tot / cnt for name, (tot, cnt) in st1.items())
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
            per_kernel.setdefault(n, {})["hbm_bytes_measured"] = round(traffic[n])
            per_kernel[n]["hbm_GB/s_measured"] = round(traffic[n] / (kms * 1e-3) / 1e9, 1)
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
                     "traffic": round(traffic[dom]) if traffic and dom in traffic else None},
    }
    if not args.no_decode:
        log("[bench] decode: generating the 8 x 128K cache and timing 256 steps")
        del q, k, v, o, ws_sel, ws_att, ws_bsa, pyr, sel, bsel
        torch.cuda.empty_cache()
        out["decode"] = decode_latency(P, I, torch)
        log(f"[bench] decode {out['decode']}")
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a CPU sample")
        out["cpu_baseline"] = cpu_baseline(pf, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
