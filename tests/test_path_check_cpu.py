"""The traced-path validator (check_path in gpu_common) pinned on the CPU: it accepts the oracle's own
walk at every unit of a small workload and rejects planted mistakes (a kept node swapped for a dropped
candidate, a missing node, a list out of order, a level that must keep every candidate but drops one,
a wrong number of levels). Without these, a validator that never complains would pass every traced GPU
path."""
import numpy as np
import pytest

import oracle as O
from long_context_block_amd import inputs as I
from gpu_common import OracleCache, check_path

SPEC = dict(B=1, Hq=4, Hkv=2, N=700, d=64, C=32, K=5, dtype="fp32", keys="ar1")


def _rows(ref, n_levels, K):
    rows = np.full((n_levels, K), -1, dtype=np.int64)
    for l, kept in ref.kept.items():
        rows[l, :len(kept)] = kept
    rows[0, :] = ref.sel
    return rows


@pytest.fixture(scope="module")
def case():
    pf = I.make_prefill(seed=0, workload_id=100, **SPEC)
    return pf, OracleCache(pf)


def _ref(pf, oc, b, r, i):
    k, _, pyr = oc.head(b, r)
    return O.select_unit(oc.q(b, r, i), k, pyr, i, pf.K, pf.scale), pyr


def test_oracle_paths_pass(case):
    pf, oc = case
    n_same = 0
    for r in range(pf.Hkv):
        for i in range(0, pf.N, 7):
            ref, pyr = _ref(pf, oc, 0, r, i)
            problems, same, _ = check_path(pf, oc, 0, r, i, _rows(ref, pyr.root_level + 1, pf.K), ref=ref)
            assert not problems, (r, i, problems)
            n_same += same
            assert same
    assert n_same > 0


def _scored_unit(pf, oc, min_gap=0.05):
    """A unit with a scored level whose best dropped candidate trails the worst kept one by >= min_gap."""
    for i in range(pf.N - 1, 0, -1):
        ref, pyr = _ref(pf, oc, 0, 0, i)
        for l, m in sorted(ref.level_margins.items()):
            if l >= 1 and m >= min_gap:
                return i, l, ref, pyr
    raise AssertionError("no unit with a well separated scored level")


def test_planted_mistakes_fail(case):
    pf, oc = case
    i, l, ref, pyr = _scored_unit(pf, oc)
    good = _rows(ref, pyr.root_level + 1, pf.K)
    assert not check_path(pf, oc, 0, 0, i, good, ref=ref)[0]
    # the level's candidates and their scores, to pick the best dropped one
    k = oc.head(0, 0)[0]
    qg = oc.q(0, 0, i)
    cand = sorted(c for p in ref.kept[l + 1] for c in O.children(l + 1, p, pyr) if O.eligible(l, c, i, pf.C, 2))
    dropped = [c for c in cand if c not in ref.kept[l]]
    sc = {c: O.node_lse_per_head(qg, pyr, l, c, i, pf.scale).sum() for c in cand}
    worst_kept = min(ref.kept[l], key=lambda c: sc[c])
    best_dropped = max(dropped, key=lambda c: sc[c])
    swapped = good.copy()
    row = sorted([c for c in ref.kept[l] if c != worst_kept] + [best_dropped])
    swapped[l, :len(row)] = row
    probs, same, _ = check_path(pf, oc, 0, 0, i, swapped, ref=ref)
    assert probs and not same
    assert any(p.startswith(f"level {l}:") for p in probs), probs
    missing = good.copy()
    missing[l, len(ref.kept[l]) - 1] = -1
    assert check_path(pf, oc, 0, 0, i, missing, ref=ref)[0]
    unsorted = good.copy()
    unsorted[l, :2] = unsorted[l, 1::-1]
    assert check_path(pf, oc, 0, 0, i, unsorted, ref=ref)[0]
    assert check_path(pf, oc, 0, 0, i, good[:-1], ref=ref)[0]
    # the top level keeps every eligible node: dropping one fails
    top = pyr.root_level
    if len(ref.kept[top]) > 1:
        short = good.copy()
        short[top, len(ref.kept[top]) - 1] = -1
        assert check_path(pf, oc, 0, 0, i, short, ref=ref)[0]
    # a leaf-level swap is caught by the exact leaf scores
    leaf_cand = sorted(c for p in ref.kept[1] for c in O.children(1, p, pyr) if O.eligible(0, c, i, pf.C, 2))
    leaf_drop = [c for c in leaf_cand if c not in ref.sel]
    if leaf_drop and ref.level_margins.get(0, 0) >= 0.05:
        lsc = {c: O.leaf_lse_per_head(qg, k, c, i, pf.C, pf.scale, pf.N).sum() for c in leaf_cand}
        kept0 = [int(x) for x in ref.sel if x >= 0]
        w = min(kept0, key=lambda c: lsc[c])
        bd = max(leaf_drop, key=lambda c: lsc[c])
        leaf_swap = good.copy()
        leaf_swap[0, :len(kept0)] = sorted([c for c in kept0 if c != w] + [bd])
        assert check_path(pf, oc, 0, 0, i, leaf_swap, ref=ref)[0]
