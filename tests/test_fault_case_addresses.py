"""Host emulation of the addresses that the GPU loads of one small case form, lane by lane.

The bf16 case B = 2, Hq = 8, Hkv = 2, N = 1000, d = 128, C = 64, K = 4 raised a GPU memory fault with a
variant (since removed) that read three families of rows quad-coalesced: lane 4 r + c loaded 16-byte
chunks 4 s + c of MFMA row r instead of lane r + 16 g loading chunks 4 s + g. This test forms, for every
unit of that case's seeded inputs and with the kept node sets the walk produces on them, the element
offsets of
  1. the q_tile 1 walk's leaf-pair key loads (tokens 2 p C .. 2 p C + 2C - 1 of each kept level-1 node
     p, rows past N clamped to N - 1),
  2. the routing-row gathers of every scored level (hi and lo planes of the candidates' child rows in
     the quad-interleaved fp16 layout, every M-tile loaded, invalid rows mapped to the level's first
     row) and their hi-plane bounds,
  3. the decode step's leaf-pair key loads (rows clamped to the cached length),
under both lane mappings, and checks that every offset lies inside its buffer (keys B Hkv N d, routing
planes B Hkv rnodes 2d, bounds B Hkv rnodes) and that the two mappings touch the same set of offsets."""
import numpy as np

import oracle as O
from long_context_block_amd import inputs as I

SPEC = dict(B=2, Hq=8, Hkv=2, N=1000, d=128, C=64, K=4, dtype="bf16", keys="ar1")
KM = 4  # M-tiles of 16 child rows per scored level (K <= 16)


def _routing_rows(n):
    """Routing-row offsets per level and the rows per KV head: a level of >= 4 nodes takes a multiple
    of 4 rows, and the total is rounded up to a multiple of 4."""
    roff, acc = [], 0
    for nl in n:
        roff.append(acc)
        acc += -(-nl // 4) * 4 if nl >= 4 else nl
    return roff, -(-acc // 4) * 4


def _plane_chunk(R, plane, c, D):
    """Element offset of 16-byte chunk c of routing row R in the quad-interleaved plane layout."""
    return ((R >> 2) * 2 + plane) * (4 * D) + 32 * c + 8 * (R & 3)


LANE = np.arange(64)
ROW_PER_LANE = (LANE & 15, LANE >> 4)  # lane r + 16 g: MFMA row r, chunks 4 s + g
QUAD = (LANE >> 2, LANE & 3)  # lane 4 r + c: MFMA row r, chunks 4 s + c


def _lane_offsets(row_elem, chunk_elem, D, lanes):
    """Sorted element offsets loaded by the 64 lanes of one mapping over the D / 32 k steps s:
    row_elem(r) is the offset of MFMA row r, chunk_elem(c) that of 16-byte chunk c within the row."""
    r, g = lanes
    s = np.arange(D // 32)[:, None]
    return np.unique(row_elem(r)[None, :] + chunk_elem(4 * s + g[None, :]))


def _key_chunks(t, D, lanes):
    """Key rows t[r] (r = 0..15) of one MFMA tile: offsets of the 16-byte chunks each lane loads."""
    return _lane_offsets(lambda r: t[r] * D, lambda c: 8 * c, D, lanes)


def test_fault_case_addresses_in_bounds_for_both_lane_mappings():
    pf = I.make_prefill(seed=0, workload_id=100, **SPEC)
    B, Hkv, N, D, C, K, G = pf.B, pf.Hkv, pf.N, pf.d, pf.C, pf.K, pf.G
    n = O.level_sizes(N, C, 2)
    assert n == [16, 8, 4, 2, 1]
    roff, rnodes = _routing_rows(n)
    k_elems, plane_elems, bound_elems = B * Hkv * N * D, B * Hkv * rnodes * 2 * D, B * Hkv * rnodes
    n_loads = {"leaf_pair": 0, "routing": 0, "decode": 0}
    for b in range(B):
        for r in range(Hkv):
            bh = b * Hkv + r
            k = pf.k.f64((b, r))
            pyr = O.build_pyramid(k, C)
            for i in range(N):
                us = O.select_unit(pf.q.f64((b, slice(r * G, (r + 1) * G), i)), k, pyr, i, K, pf.scale)
                # 1. q_tile 1 walk: key tiles of the kept level-1 nodes' leaf pairs
                for pn in us.kept.get(1, [0]):
                    for m in range(C // 8):
                        t = np.minimum(2 * pn * C + 16 * m + np.arange(16), N - 1)
                        a = _key_chunks(t, D, ROW_PER_LANE)
                        assert np.array_equal(a, _key_chunks(t, D, QUAD))
                        lo, hi = bh * N * D + a[0], bh * N * D + a[-1] + 8
                        assert 0 <= lo and hi <= k_elems, (b, r, i, pn, m)
                        n_loads["leaf_pair"] += 1
                # 2. routing rows of every scored level l >= 1: children (level l - 1) of the candidates
                for l in sorted(us.level_margins):
                    if l == 0:
                        continue
                    cand = sorted(c for p in us.kept[l + 1] for c in O.children(l + 1, p, pyr)
                                  if O.eligible(l, c, i, C, 2))
                    n_cand = len(cand)
                    assert K < n_cand <= 2 * K
                    e_child = i // (C << (l - 1)) + 1
                    n_full = n_cand if 2 * cand[-1] + 1 < e_child else n_cand - 1
                    rows = []
                    for m in range(KM):
                        for r16 in range(16):
                            row = 16 * m + r16
                            cidx = row >> 1
                            valid = cidx < n_cand and ((row & 1) == 0 or cidx < n_full)
                            rows.append(roff[l - 1] + (2 * cand[cidx] + (row & 1) if valid else 0))
                    base = bh * rnodes * 2 * D
                    rows = np.array(rows)
                    for m in range(KM):
                        R = rows[16 * m:16 * m + 16]
                        for plane in (0, 1):
                            sets = []
                            for rr_, g_ in (ROW_PER_LANE, QUAD):
                                sidx = np.arange(D // 32)[:, None]
                                Rl = R[rr_][None, :]
                                off = base + _plane_chunk(Rl, plane, 4 * sidx + g_[None, :], D)
                                sets.append(np.unique(off))
                            assert np.array_equal(sets[0], sets[1])
                            assert sets[0][0] >= 0 and sets[0][-1] + 8 <= plane_elems, (b, r, i, l, m)
                            n_loads["routing"] += 1
                    for c_, cn in enumerate(cand):
                        for bit in (0, 1) if c_ < n_full else (0,):
                            x = bh * rnodes + roff[l - 1] + 2 * cn + bit
                            assert 0 <= x < bound_elems
            # 3. decode: the kept level-1 nodes' leaf pairs, rows clamped to the cached length p + 1
            for p_ in range(0, N, 7):
                for pn in range(p_ // (2 * C) + 1):
                    for m in range(C // 8):
                        t = np.minimum(2 * pn * C + 16 * m + np.arange(16), p_)
                        a = _key_chunks(t, D, ROW_PER_LANE)
                        assert np.array_equal(a, _key_chunks(t, D, QUAD))
                        assert 0 <= bh * N * D + a[0] and bh * N * D + a[-1] + 8 <= k_elems
                        n_loads["decode"] += 1
    assert all(v > 0 for v in n_loads.values()), n_loads
