"""Pins for the float64 oracle: each check ties it to something other than itself (a library routine,
a closed form, an invariant, a dense brute force, or a value printed on the pages)."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
from long_context_block_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _same_margin(a, b, tol=1e-9):
    """Both +inf (no scored level), or equal up to float64 rounding of the scores."""
    if math.isinf(a) or math.isinf(b):
        return a == b
    return abs(a - b) <= tol * (1.0 + abs(b))


# ---------------------------------------------------------------- C1: LogSumExp
def test_lse_matches_direct_and_library():
    x = _rng(1).uniform(-50, 50, size=(37, 19))
    direct = np.log(np.sum(np.exp(x), axis=-1))
    np.testing.assert_allclose(O.logsumexp(x), direct, rtol=1e-12, atol=0)
    np.testing.assert_allclose(O.logsumexp(x), scipy.special.logsumexp(x, axis=-1), rtol=1e-13, atol=0)


def test_lse_closed_forms():
    for n in (1, 2, 7, 64):
        for x0 in (-3.5, 0.0, 17.25, 900.0):  # 900 overflows a naive exp
            assert O.logsumexp(np.full(n, x0)) == pytest.approx(x0 + math.log(n), rel=1e-14, abs=1e-13)
    assert O.logsumexp(np.array([-np.inf, -np.inf])) == -np.inf
    assert O.logsumexp(np.array([-np.inf, 2.0])) == 2.0


# ---------------------------------------------------------------- C2: pyramid means
@pytest.mark.parametrize("N,C", [(1024, 32), (1000, 32), (777, 64), (64, 64), (1, 32), (129, 32)])
def test_pyramid_recursive_equals_direct_span_mean(N, C):
    k = _rng(2).standard_normal((N, 16))
    pyr = O.build_pyramid(k, C, 2)
    for l, m in enumerate(pyr.means):
        w = C * 2 ** l
        for j in range(m.shape[0]):
            t0, t1 = j * w, min(N, (j + 1) * w)
            np.testing.assert_allclose(m[j], k[t0:t1].mean(axis=0), rtol=1e-12, atol=1e-13)
            assert pyr.counts[l][j] == t1 - t0


@pytest.mark.parametrize("N,C", [(1024, 32), (1000, 32), (200, 64)])
def test_pyramid_closed_form_linear_keys(N, C):
    e = _rng(3).standard_normal(8)
    k = np.arange(N, dtype=np.float64)[:, None] * e[None, :]
    pyr = O.build_pyramid(k, C, 2)
    for l, m in enumerate(pyr.means):
        w = C * 2 ** l
        for j in range(m.shape[0]):
            first, last = j * w, min(N, (j + 1) * w) - 1
            np.testing.assert_allclose(m[j], 0.5 * (first + last) * e, rtol=1e-12, atol=1e-10)


def test_level_counts_match_pages():
    with open(os.path.join(GOLDEN, "pool_chain_levels.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        sizes = O.level_sizes(case["N"], case["C"], 2)
        assert len(sizes) - 1 == case["pool_levels"]
        assert sizes[-1] == 1
    # the tiny fp32 workload: 32 leaves, 6 levels including the root
    assert O.level_sizes(1024, 32) == [32, 16, 8, 4, 2, 1]


# ---------------------------------------------------------------- helpers
def _tiny(N=1024, d=64, C=32, G=1, seed=5, keys="iid"):
    p = I.make_prefill(B=1, Hq=G, Hkv=1, N=N, d=d, C=C, K=4, dtype="fp32", keys=keys, seed=seed)
    q = p.q.f64()[0]  # [G, N, d]
    k = p.k.f64()[0, 0]
    v = p.v.f64()[0, 0]
    return q, k, v, p.scale


def _brute_exact_topk(q, k, C, K, scale):
    """Independent brute force: dense masked score matrix, per-leaf LSE by scipy, lexsort Top-K."""
    G, N, _ = q.shape
    n0 = -(-N // C)
    S = scale * np.einsum("gnd,td->gnt", q, k)  # [G, N, N]
    mask = np.tril(np.ones((N, N), dtype=bool))
    S = np.where(mask[None], S, -np.inf)
    Sp = np.full((G, N, n0 * C), -np.inf)
    Sp[:, :, :N] = S
    F = scipy.special.logsumexp(Sp.reshape(G, N, n0, C), axis=-1).sum(axis=0)  # [N, n0]
    out = []
    for i in range(N):
        e = i // C + 1
        f = F[i, :e]
        order = np.lexsort((np.arange(e), -f))
        sel = sorted(order[:K].tolist())
        gap = (f[order[K - 1]] - f[order[K]]) if e > K else np.inf
        out.append((sel, gap))
    return out


# ---------------------------------------------------------------- C3: attention
def test_attention_all_blocks_equals_dense_sdpa():
    q, k, v, scale = _tiny(N=300, d=32, C=32, G=3)
    N = k.shape[0]
    n0 = -(-N // 32)
    pyr = O.build_pyramid(k, 32)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None, None].expand(1, 3, N, 32),
        torch.from_numpy(v)[None, None].expand(1, 3, N, 32), is_causal=True, scale=scale)[0].numpy()
    for i in range(N):
        us = O.select_unit(q[:, i], k, pyr, i, n0, scale)
        o, o_lse = O.attend_unit(q[:, i], k, v, us.sel, i, 32, scale, N)
        np.testing.assert_allclose(o, ref[:, i], rtol=0, atol=1e-12)
        full = scipy.special.logsumexp(scale * q[:, i] @ k[: i + 1].T, axis=-1)
        np.testing.assert_allclose(o_lse, full, rtol=1e-13)


def test_attention_closed_forms():
    q, k, v, scale = _tiny(N=200, d=16, C=32, G=2)
    const_v = np.tile(_rng(7).standard_normal(16), (200, 1))
    const_k = np.tile(_rng(8).standard_normal(16), (200, 1))
    for i in (0, 5, 31, 32, 199):
        sel = np.array([0, 2, 5, -1])
        sel = np.array([j for j in sel if j < 0 or j * 32 <= i] + [-1] * 4)[:4]
        o, _ = O.attend_unit(q[:, i], k, const_v, sel, i, 32, scale, 200)
        np.testing.assert_allclose(o, np.tile(const_v[0], (2, 1)), rtol=0, atol=1e-12)
        o2, lse2 = O.attend_unit(q[:, i], const_k, v, sel, i, 32, scale, 200)
        toks = [t for j in sel if j >= 0 for t in range(j * 32, min(200, (j + 1) * 32, i + 1))]
        np.testing.assert_allclose(o2, np.tile(v[toks].mean(axis=0), (2, 1)), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse2, scale * q[:, i] @ const_k[0] + math.log(len(toks)), rtol=1e-13)
    # query 0 attends only to itself
    us = O.select_unit(q[:, 0], k, O.build_pyramid(k, 32), 0, 4, scale)
    assert us.sel.tolist() == [0, -1, -1, -1]
    o, _ = O.attend_unit(q[:, 0], k, v, us.sel, 0, 32, scale, 200)
    np.testing.assert_allclose(o, np.tile(v[0], (2, 1)), rtol=0, atol=1e-15)


# ---------------------------------------------------------------- C4: selection vs brute force
@pytest.mark.parametrize("K", [16, 32])
def test_walk_equals_flat_exact_when_k_covers_level1(K):
    q, k, v, scale = _tiny(N=1024, d=64, C=32, G=1)
    pyr = O.build_pyramid(k, 32)
    assert pyr.means[1].shape[0] == 16 and pyr.means[0].shape[0] == 32
    brute = _brute_exact_topk(q, k, 32, K, scale)
    n_checked = 0
    for i in range(1024):
        us = O.select_unit(q[:, i], k, pyr, i, K, scale)
        sel_b, gap = brute[i]
        # with K >= n_1 only the leaf level can be scored, so the unit's margin is the leaf gap
        assert _same_margin(us.margin, gap), (i, us.margin, gap)
        if gap < 1e-9:
            continue
        got = [j for j in us.sel.tolist() if j >= 0]
        assert got == sel_b, (i, got, sel_b)
        fe, fgap = O.flat_exact_select_unit(q[:, i], k, i, 32, K, scale)
        assert [j for j in fe.tolist() if j >= 0] == sel_b
        assert _same_margin(fgap, gap)
        if K == 32:
            assert got == list(range(i // 32 + 1))
        n_checked += 1
    assert n_checked > 1000


def test_walk_gqa_equals_flat_exact_when_k_covers_level1():
    q, k, v, scale = _tiny(N=640, d=32, C=32, G=4, keys="ar1")
    pyr = O.build_pyramid(k, 32)
    K = pyr.means[1].shape[0]
    brute = _brute_exact_topk(q, k, 32, K, scale)
    for i in range(0, 640, 3):
        us = O.select_unit(q[:, i], k, pyr, i, K, scale)
        sel_b, gap = brute[i]
        assert _same_margin(us.margin, gap), (i, us.margin, gap)
        if gap >= 1e-9:
            assert [j for j in us.sel.tolist() if j >= 0] == sel_b


def _dense_two_level(q, k, C, K, scale):
    """Independent dense brute force for n_2 <= K < n_1: levels >= 2 keep everything, level 1 is
    scored by the LSE over its children's leaf means, the leaves by exact LSE."""
    G, N, d = q.shape
    n0 = -(-N // C)
    n1 = -(-n0 // 2)
    leaf_mean = np.stack([k[j * C:min(N, (j + 1) * C)].mean(axis=0) for j in range(n0)])
    lm = np.full((2 * n1, d), np.nan)
    lm[:n0] = leaf_mean
    Sm = scale * np.einsum("gnd,jd->gnj", q, np.nan_to_num(lm))  # [G, N, 2*n1]
    first_tok = np.arange(2 * n1) * C
    elig = (first_tok[None, :] <= np.arange(N)[:, None]) & (np.arange(2 * n1)[None, :] < n0)
    Sm = np.where(elig[None], Sm, -np.inf)
    L1 = scipy.special.logsumexp(Sm.reshape(G, N, n1, 2), axis=-1).sum(axis=0)  # [N, n1]
    S = scale * np.einsum("gnd,td->gnt", q, k)
    S = np.where(np.tril(np.ones((N, N), dtype=bool))[None], S, -np.inf)
    Sp = np.full((G, N, n0 * C), -np.inf)
    Sp[:, :, :N] = S
    F = scipy.special.logsumexp(Sp.reshape(G, N, n0, C), axis=-1).sum(axis=0)
    res = []
    for i in range(N):
        e1 = (i // (2 * C)) + 1
        s1 = L1[i, :e1]
        if e1 > K:
            o1 = np.lexsort((np.arange(e1), -s1))
            kept1 = sorted(o1[:K].tolist())
            gap1 = s1[o1[K - 1]] - s1[o1[K]]
        else:
            kept1, gap1 = list(range(e1)), np.inf
        cand = [c for p in kept1 for c in (2 * p, 2 * p + 1) if c < n0 and c * C <= i]
        f = F[i, cand]
        if len(cand) > K:
            o0 = np.lexsort((np.array(cand), -f))
            sel = sorted(cand[t] for t in o0[:K])
            gap0 = f[o0[K - 1]] - f[o0[K]]
        else:
            sel, gap0 = sorted(cand), np.inf
        res.append((sel, min(gap1, gap0)))
    return res


@pytest.mark.parametrize("K,G", [(7, 1), (5, 2), (4, 3)])
def test_walk_equals_dense_two_level_bruteforce(K, G):
    # N=512, C=32: 16 leaves, 8 level-1 nodes, 4 level-2 nodes; with n_2 <= K < n_1 only level 1 and the
    # leaves are scored.
    q, k, v, scale = _tiny(N=512 - 7, d=32, C=32, G=G, keys="ar1", seed=11)
    pyr = O.build_pyramid(k, 32)
    assert pyr.means[2].shape[0] <= K < pyr.means[1].shape[0]
    brute = _dense_two_level(q, k, 32, K, scale)
    n_ok = 0
    for i in range(q.shape[1]):
        us = O.select_unit(q[:, i], k, pyr, i, K, scale)
        sel_b, gap = brute[i]
        if gap < 1e-9:
            continue
        assert [j for j in us.sel.tolist() if j >= 0] == sel_b, i
        # the margin is the smaller of the level-1 and leaf gaps (each +inf when unscored)
        assert _same_margin(us.margin, gap), (i, us.margin, gap)
        n_ok += 1
    assert n_ok > 400


# ---------------------------------------------------------------- closed-form walks with K < n_1
@pytest.mark.parametrize("sign", [+1, -1])
@pytest.mark.parametrize("N", [1024, 1000])
def test_walk_monotone_keys_closed_form(sign, N):
    """Keys k_t = sign * a * t * e and a query along e: every level's scores are monotone in position,
    so the walk keeps the last (sign=+1) or first (sign=-1) K eligible nodes at every level and the
    selection is the last / first K eligible leaves."""
    d, C, K = 8, 32, 4
    e = np.zeros(d)
    e[0] = 1.0
    k = sign * 0.5 * np.arange(N, dtype=np.float64)[:, None] * e[None, :]
    q = np.stack([e * 2.0, e * 1.0])  # G=2, both aligned
    pyr = O.build_pyramid(k, C)
    for i in range(N):
        us = O.select_unit(q, k, pyr, i, K, 1.0 / math.sqrt(d))
        n_el = i // C + 1
        want = list(range(max(0, n_el - K), n_el)) if sign > 0 else list(range(min(K, n_el)))
        assert [j for j in us.sel.tolist() if j >= 0] == want, (i, us.sel)
        assert us.margin > 0


# ---------------------------------------------------------------- C5: invariants
def test_selection_invariants():
    q, k, v, scale = _tiny(N=1000, d=32, C=32, G=2, keys="ar1", seed=9)
    pyr = O.build_pyramid(k, 32)
    K = 4
    for i in range(0, 1000, 7):
        us = O.select_unit(q[:, i], k, pyr, i, K, scale)
        got = [j for j in us.sel.tolist() if j >= 0]
        assert len(got) == min(K, i // 32 + 1)
        assert got == sorted(set(got))
        assert all(j * 32 <= i for j in got)
        assert all(j == -1 for j in us.sel.tolist()[len(got):])
        for l in range(1, pyr.root_level + 1):
            anc = sorted({j >> l for j in got})
            assert set(anc) <= set(us.kept[l]), (i, l)
            assert len(us.kept[l]) <= K
        # bounded candidates: at most g*K per level
        for l in range(pyr.root_level):
            cand = [c for p in us.kept[l + 1] for c in O.children(l + 1, p, pyr) if c * 32 * 2 ** l <= i]
            assert len(cand) <= 2 * K
        assert np.all(np.isfinite(us.sel_lse[:, :len(got)]))


# ---------------------------------------------------------------- C6 / C7: symmetries
def test_translation_and_head_permutation_invariance():
    q, k, v, scale = _tiny(N=700, d=32, C=32, G=3, keys="ar1", seed=13)
    c = _rng(14).standard_normal(32) * 3.0
    pyr = O.build_pyramid(k, 32)
    pyr_t = O.build_pyramid(k + c, 32)
    perm = [2, 0, 1]
    for i in range(0, 700, 11):
        a = O.select_unit(q[:, i], k, pyr, i, 4, scale)
        if a.margin < 1e-6:
            continue
        b = O.select_unit(q[:, i], k + c, pyr_t, i, 4, scale)
        assert a.sel.tolist() == b.sel.tolist()
        oa, _ = O.attend_unit(q[:, i], k, v, a.sel, i, 32, scale, 700)
        ob, _ = O.attend_unit(q[:, i], k + c, v, b.sel, i, 32, scale, 700)
        np.testing.assert_allclose(oa, ob, rtol=0, atol=1e-10)
        p = O.select_unit(q[perm, i], k, pyr, i, 4, scale)
        assert p.sel.tolist() == a.sel.tolist()
        np.testing.assert_allclose(p.sel_lse, a.sel_lse[perm], rtol=1e-13)


# ---------------------------------------------------------------- C8: planted needle
def test_planted_needle_selected_with_ancestors():
    q, k, v, scale = _tiny(N=2048, d=32, C=32, G=2, keys="ar1", seed=15)
    u = _rng(16).standard_normal(32)
    u /= np.linalg.norm(u)
    needle = 21
    k = k.copy()
    k[needle * 32:(needle + 1) * 32] = 6.0 * u + 0.3 * _rng(17).standard_normal((32, 32))
    pyr = O.build_pyramid(k, 32)
    for i in (needle * 32 + 40, 1500, 2047):
        qq = np.stack([4.0 * u, 3.0 * u]) + 0.2 * _rng(i).standard_normal((2, 32))
        us = O.select_unit(qq, k, pyr, i, 4, scale)
        assert needle in us.sel.tolist()
        for l in range(1, pyr.root_level + 1):
            assert (needle >> l) in us.kept[l]


# ---------------------------------------------------------------- C9: decode
def test_decode_incremental_pyramid_and_step_equal_rebuild():
    C, d, K, G = 32, 16, 3, 2
    n0, steps = 130, 100  # crosses leaf boundaries and a new root level (5 -> 8 leaves)
    rng = _rng(21)
    k_all = rng.standard_normal((n0 + steps, d))
    v_all = rng.standard_normal((n0 + steps, d))
    q_all = rng.standard_normal((steps, G, d))
    sp = O.empty_sum_pyramid(n0 + steps, d, C)
    for p in range(n0):
        O.sum_pyramid_append(sp, p, k_all[p])
    kh = np.zeros_like(k_all)
    vh = np.zeros_like(v_all)
    kh[:n0] = k_all[:n0]
    vh[:n0] = v_all[:n0]
    scale = 1 / math.sqrt(d)
    for s in range(steps):
        p = n0 + s
        us, o, o_lse = O.decode_step_unit(q_all[s], kh, vh, sp, p, k_all[p], v_all[p], K, scale)
        reb = O.build_pyramid(k_all[: p + 1], C)
        inc = O.sum_pyramid_means(sp, p + 1)
        assert len(inc.means) == len(reb.means)
        for a, b in zip(inc.means, reb.means):
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
        ref = O.select_unit(q_all[s], k_all, reb, p, K, scale)
        assert us.sel.tolist() == ref.sel.tolist()
        o_ref, _ = O.attend_unit(q_all[s], k_all, v_all, ref.sel, p, C, scale, p + 1)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        # the new token is attended: query p sees its own key
        assert (p // C) in us.sel.tolist() or len([j for j in us.sel if j >= 0]) == K


# ---------------------------------------------------------------- flat BSA
def test_bsa_matches_dense_mean_key_scores():
    q, k, v, scale = _tiny(N=900, d=32, C=32, G=3, keys="ar1", seed=23)
    n0 = -(-900 // 32)
    leaf_mean = np.stack([k[j * 32:min(900, (j + 1) * 32)].mean(axis=0) for j in range(n0)])
    dense = scale * np.einsum("gnd,jd->nj", q, leaf_mean)  # heads summed by the contraction
    for i in range(0, 900, 5):
        e = i // 32 + 1
        f = dense[i, :e]
        o = np.lexsort((np.arange(e), -f))
        want = sorted(o[:6].tolist())
        sel, gap = O.bsa_select_unit(q[:, i], leaf_mean, i, 32, 6, scale)
        dense_gap = f[o[5]] - f[o[6]] if e > 6 else math.inf
        assert _same_margin(gap, dense_gap), (i, gap, dense_gap)
        if e > 6 and gap < 1e-9:
            continue
        assert [j for j in sel.tolist() if j >= 0] == want


# ---------------------------------------------------------------- exact ties break to the lowest index
@pytest.mark.parametrize("K", [3, 4, 6])
def test_exact_ties_break_to_lowest_index(K):
    """All keys equal: every full node at a level has the same score bit for bit, so the walk keeps the
    lowest-indexed candidates at each level and the selection is leaves 0..K-1 once i >= 2*K*C."""
    C, d, N = 32, 16, 1024
    k = np.tile(_rng(31).standard_normal(d), (N, 1))
    q = _rng(32).standard_normal((2, d))
    pyr = O.build_pyramid(k, C)
    for i in range(2 * K * C, N, 13):
        us = O.select_unit(q, k, pyr, i, K, 0.25)
        assert us.sel.tolist() == list(range(K)), (i, us.sel)
        assert us.margin == 0.0


# ---------------------------------------------------------------- per-head leaf LSEs of the selection
@pytest.mark.parametrize("G,keys", [(1, "iid"), (3, "ar1")])
def test_sel_lse_equals_library_lse_over_selected_tokens(G, keys):
    """Column s of sel_lse is, for each head, scipy's LSE of s * q_h . k_t over the tokens t <= i of the
    s-th selected leaf (ascending), and -inf past the selection."""
    q, k, v, scale = _tiny(N=777, d=32, C=32, G=G, keys=keys, seed=41)
    pyr = O.build_pyramid(k, 32)
    K = 5
    for i in range(0, 777, 5):
        us = O.select_unit(q[:, i], k, pyr, i, K, scale)
        row = scale * np.einsum("gd,td->gt", q[:, i], k[: i + 1])  # the causal score row, [G, i+1]
        for s_, j in enumerate(us.sel.tolist()):
            if j < 0:
                assert np.all(us.sel_lse[:, s_] == -np.inf)
                continue
            want = scipy.special.logsumexp(row[:, j * 32:min(i + 1, (j + 1) * 32)], axis=-1)
            np.testing.assert_allclose(us.sel_lse[:, s_], want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- dense brute force of the whole walk
def _dense_walk(q, k, C, K, scale, budgets=None, start=None):
    """Independent dense brute force of the walk at every level. Node means come straight from the raw
    keys of each node's span; every node's score for every query is one dense masked matrix (scipy
    LSE over eligible children, or over the leaf's tokens t <= i); the walk is boolean masks over whole
    levels, children by np.repeat, Top-K by lexsort. Returns per query (sel, per-head leaf LSEs of
    sel, margin = smallest gap over the scored levels)."""
    G, N, d = q.shape
    n = [-(-N // C)]
    while n[-1] > 1:
        n.append(-(-n[-1] // 2))
    L = len(n) - 1
    means = []
    for l in range(L + 1):
        w = C * 2 ** l
        means.append(np.stack([k[j * w:min(N, (j + 1) * w)].mean(axis=0) for j in range(n[l])]))
    pos = np.arange(N)
    elig = [(np.arange(n[l])[None, :] * (C * 2 ** l)) <= pos[:, None] for l in range(L + 1)]  # [N, n_l]
    S = {}
    for l in range(1, L + 1):
        X = scale * np.einsum("gnd,jd->gnj", q, means[l - 1])
        X = np.where(elig[l - 1][None], X, -np.inf)
        Xp = np.full((G, N, 2 * n[l]), -np.inf)
        Xp[:, :, :n[l - 1]] = X
        S[l] = scipy.special.logsumexp(Xp.reshape(G, N, n[l], 2), axis=-1).sum(axis=0)  # [N, n_l]
    T = scale * np.einsum("gnd,td->gnt", q, k)
    T = np.where(np.tril(np.ones((N, N), dtype=bool))[None], T, -np.inf)
    Tp = np.full((G, N, n[0] * C), -np.inf)
    Tp[:, :, :N] = T
    LH = scipy.special.logsumexp(Tp.reshape(G, N, n[0], C), axis=-1)  # [G, N, n_0], -inf when no token
    S[0] = LH.sum(axis=0)
    Kl = [K] * (L + 1) if budgets is None else list(budgets)
    top = L if start is None else start
    out = []
    for i in range(N):
        kept = np.ones(1, dtype=bool)  # the root
        gaps = []
        for l in range(top, -1, -1):
            cand = elig[l][i].copy() if l == top else np.repeat(kept, 2)[:n[l]] & elig[l][i]
            idx = np.flatnonzero(cand)
            if idx.size > Kl[l]:
                sc = S[l][i, idx]
                order = np.lexsort((idx, -sc))
                gaps.append(sc[order[Kl[l] - 1]] - sc[order[Kl[l]]])
                kept = np.zeros(n[l], dtype=bool)
                kept[idx[order[:Kl[l]]]] = True
            else:
                kept = cand
        sel = np.flatnonzero(kept)
        out.append((sel.tolist(), LH[:, i, sel], min(gaps) if gaps else math.inf))
    return out


@pytest.mark.parametrize("K,G", [(3, 1), (4, 2), (6, 4)])
def test_walk_equals_dense_all_levels_bruteforce(K, G):
    """N = 2000, C = 32: 63 leaves (the last one ragged) and 7 levels, so K = 3, 4, 6 score 5, 4 and 4
    levels. Selection, per-head leaf LSEs and margin all equal the dense brute force."""
    N, C = 2000, 32
    q, k, v, scale = _tiny(N=N, d=32, C=C, G=G, keys="ar1", seed=51 + K)
    pyr = O.build_pyramid(k, C)
    brute = _dense_walk(q, k, C, K, scale)
    n_ok = n_deep = 0
    for i in range(N):
        sel_b, lse_b, gap = brute[i]
        us = O.select_unit(q[:, i], k, pyr, i, K, scale)
        if gap < 1e-9:
            continue
        got = [j for j in us.sel.tolist() if j >= 0]
        assert got == sel_b, (i, got, sel_b)
        assert _same_margin(us.margin, gap), (i, us.margin, gap, us.level_margins)
        np.testing.assert_allclose(us.sel_lse[:, :len(got)], lse_b, rtol=1e-12, atol=1e-12)
        n_ok += 1
        n_deep += len(us.level_margins) >= 3
    assert n_ok > 0.9 * N
    assert n_deep > 0.5 * N  # most units are scored at three or more levels


# ---------------------------------------------------------------- selection quality (Recall@K, mass)
def test_row_lse_and_mass_closed_forms():
    """Identical keys: every score of a row is s q . k0, so the row LSE is s q . k0 + ln(i + 1) and a
    selection holds exactly |T| / (i + 1) of the softmax mass."""
    d, C, N = 16, 32, 300
    k = np.tile(_rng(61).standard_normal(d), (N, 1))
    q = _rng(62).standard_normal((3, d))
    scale = 0.25
    for i in (0, 31, 32, 100, 299):
        want = scale * q @ k[0] + math.log(i + 1)
        np.testing.assert_allclose(O.row_lse_unit(q, k, i, scale), want, rtol=1e-13)
        sel = np.array([j for j in (0, 2, 3) if j * C <= i] + [-1] * 3)[:3]
        T = sum(min(i + 1, (j + 1) * C) - j * C for j in sel if j >= 0)
        np.testing.assert_allclose(O.attention_mass_unit(q, k, sel, i, C, scale), T / (i + 1), rtol=1e-12)
        everything = np.arange(i // C + 1)
        np.testing.assert_allclose(O.attention_mass_unit(q, k, everything, i, C, scale), 1.0, rtol=1e-13)
        np.testing.assert_allclose(O.attention_mass_unit(q, k, np.array([-1, -1]), i, C, scale), 0.0, atol=0)


def test_mass_equals_leaf_lse_weights():
    """The mass of a selection is sum over its leaves of exp(leaf LSE - row LSE) per head: the leaf LSEs
    partition the row's LSE, checked against scipy on the raw causal row."""
    q, k, v, scale = _tiny(N=500, d=32, C=32, G=3, keys="ar1", seed=63)
    for i in (40, 255, 499):
        row = scale * q[:, i] @ k[: i + 1].T
        L = scipy.special.logsumexp(row, axis=-1)
        np.testing.assert_allclose(O.row_lse_unit(q[:, i], k, i, scale), L, rtol=1e-13)
        sel = np.array([0, 3, i // 32])
        leaf = np.stack([scipy.special.logsumexp(row[:, j * 32:min(i + 1, (j + 1) * 32)], axis=-1) for j in sel])
        np.testing.assert_allclose(O.attention_mass_unit(q[:, i], k, sel, i, 32, scale),
                                   np.exp(leaf - L[None]).sum(axis=0), rtol=1e-11)


def test_recall_of_walk_is_one_when_k_covers_level1():
    """With K >= n_1 the walk is the flat exact Top-K, so its Recall@K against it is 1 on every unit
    whose flat gap is clear; with K < n_1 it is a fraction in [0, 1]."""
    q, k, v, scale = _tiny(N=1024, d=64, C=32, G=1)
    pyr = O.build_pyramid(k, 32)
    for i in range(0, 1024, 9):
        us = O.select_unit(q[:, i], k, pyr, i, 16, scale)
        fe, gap = O.flat_exact_select_unit(q[:, i], k, i, 32, 16, scale)
        if gap >= 1e-9:
            assert O.recall_at_k(us.sel, fe) == 1.0
        us4 = O.select_unit(q[:, i], k, pyr, i, 4, scale)
        fe4, _ = O.flat_exact_select_unit(q[:, i], k, i, 32, 4, scale)
        r = O.recall_at_k(us4.sel, fe4)
        assert 0.0 <= r <= 1.0
    assert O.recall_at_k(np.array([1, 2, -1]), np.array([2, 5, 7])) == pytest.approx(1 / 3)


# ---------------------------------------------------------------- selection variants (ablations)
def test_variant_defaults_equal_the_walk():
    """LSE scoring, mean pooling, fixed budget and no cap: the variant walk is the walk itself."""
    q, k, v, scale = _tiny(N=1500, d=32, C=32, G=2, keys="ar1", seed=71)
    pyr = O.build_pyramid(k, 32)
    pooled = O.build_pyramid_pooled(k, 32, pool="mean")
    for a, b in zip(pyr.means, pooled.means):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    for i in range(0, 1500, 7):
        a = O.select_unit(q[:, i], k, pyr, i, 4, scale)
        b = O.select_unit_variant(q[:, i], k, pyr, i, 4, scale)
        assert a.sel.tolist() == b.sel.tolist() and a.margin == b.margin


@pytest.mark.parametrize("N", [1000, 777])
def test_pooled_summaries_closed_forms(N):
    """Sum pooling is the mean times the tokens held; max pooling of increasing keys k_t = t e (e > 0)
    is the key of the span's last token."""
    C = 32
    k = _rng(72).standard_normal((N, 8))
    mean = O.build_pyramid_pooled(k, C, pool="mean")
    summ = O.build_pyramid_pooled(k, C, pool="sum")
    for m, s_, c in zip(mean.means, summ.means, mean.counts):
        np.testing.assert_allclose(s_, m * c[:, None], rtol=1e-12, atol=1e-10)
    e = np.abs(_rng(73).standard_normal(8)) + 0.1
    kl = np.arange(N, dtype=np.float64)[:, None] * e[None, :]
    mx = O.build_pyramid_pooled(kl, C, pool="max")
    for l, m in enumerate(mx.means):
        for j in range(m.shape[0]):
            last = min(N, (j + 1) * C * 2 ** l) - 1
            np.testing.assert_allclose(m[j], last * e, rtol=1e-14)
    var = O.pyramid_variances(k, C)
    for l, vv in enumerate(var):
        w = C * 2 ** l
        for j in (0, vv.shape[0] - 1):
            np.testing.assert_allclose(vv[j], np.var(k[j * w:min(N, (j + 1) * w)], axis=0), rtol=1e-12)


def test_mean_scoring_with_k_covering_level1_is_flat_bsa():
    """PISA-1 (each node scored by s q . its mean) with K >= n_1 keeps every node above the leaves, so
    it ranks every eligible leaf by s q . mean(leaf): the flat BSA selection."""
    q, k, v, scale = _tiny(N=900, d=32, C=32, G=3, keys="ar1", seed=74)
    pyr = O.build_pyramid(k, 32)
    K = pyr.means[1].shape[0]
    for i in range(0, 900, 4):
        a = O.select_unit_variant(q[:, i], k, pyr, i, K, scale, score="mean")
        b, gap = O.bsa_select_unit(q[:, i], pyr.means[0], i, 32, K, scale)
        assert _same_margin(a.margin, gap)
        if gap >= 1e-9:
            assert a.sel.tolist() == b.tolist(), i


def test_mean_var_scoring_equals_dense_formula():
    """PISA-2 with K >= n_1: every eligible leaf ranked by sum_h [s q_h . mu + (s^2 / 2) sum_d q_hd^2
    var_d], computed here from reshaped leaf blocks; leaves holding one constant key reduce it to PISA-1."""
    N, C, G = 1024, 32, 2
    q, k, v, scale = _tiny(N=N, d=32, C=C, G=G, keys="ar1", seed=75)
    pyr = O.build_pyramid(k, C)
    var = O.pyramid_variances(k, C)
    K = pyr.means[1].shape[0]
    blocks = k.reshape(N // C, C, -1)
    mu, vr = blocks.mean(axis=1), blocks.var(axis=1)  # [n_0, d]
    F = scale * np.einsum("gnd,jd->nj", q, mu) + 0.5 * scale ** 2 * np.einsum("gnd,jd->nj", q * q, vr)
    for i in range(0, N, 5):
        e = i // C + 1
        f = F[i, :e]
        o = np.lexsort((np.arange(e), -f))
        want = sorted(o[:K].tolist()) if e > K else list(range(e))
        gap = f[o[K - 1]] - f[o[K]] if e > K else math.inf
        a = O.select_unit_variant(q[:, i], k, pyr, i, K, scale, score="mean_var", variances=var)
        assert _same_margin(a.margin, gap)
        if gap >= 1e-9:
            assert [j for j in a.sel.tolist() if j >= 0] == want
    kc = np.repeat(_rng(76).standard_normal((N // C, 32)), C, axis=0)  # one key per leaf
    pyr_c, var_c = O.build_pyramid(kc, C), O.pyramid_variances(kc, C)
    for i in range(0, N, 11):
        a = O.select_unit_variant(q[:, i], kc, pyr_c, i, K, scale, score="mean_var", variances=var_c)
        b = O.select_unit_variant(q[:, i], kc, pyr_c, i, K, scale, score="mean")
        assert a.sel.tolist() == b.sel.tolist()


@pytest.mark.parametrize("K,G", [(3, 1), (4, 2)])
def test_halving_budget_and_truncation_equal_dense_bruteforce(K, G):
    """The halving budget K_l = min(n_l, K 2^l) and a capped starting level, against the dense brute
    force of the whole walk run with the same per-level budgets and starting level."""
    N, C = 2000, 32
    q, k, v, scale = _tiny(N=N, d=32, C=C, G=G, keys="ar1", seed=77 + K)
    pyr = O.build_pyramid(k, C)
    n = [m.shape[0] for m in pyr.means]
    budgets = [min(n[l], K * 2 ** l) for l in range(len(n))]  # K at the leaves, doubling per coarser level
    cases = [("halving", None, budgets, None), ("fixed", 3, None, 3), ("halving", 4, budgets, 4)]
    for budget, cap, bl, st in cases:
        brute = _dense_walk(q, k, C, K, scale, budgets=bl, start=st)
        n_ok = 0
        for i in range(0, N, 3):
            sel_b, _, gap = brute[i]
            a = O.select_unit_variant(q[:, i], k, pyr, i, K, scale, budget=budget, max_level=cap)
            if gap < 1e-9:
                continue
            assert [j for j in a.sel.tolist() if j >= 0] == sel_b, (budget, cap, i)
            assert _same_margin(a.margin, gap)
            n_ok += 1
        assert n_ok > 0.9 * len(range(0, N, 3))


def test_truncation_that_keeps_every_start_node_changes_nothing():
    """A cap whose starting level holds at most K nodes keeps all of them, as the full walk does at and
    above that level: the selection is the full walk's."""
    q, k, v, scale = _tiny(N=2000, d=32, C=32, G=2, keys="ar1", seed=79)
    pyr = O.build_pyramid(k, 32)  # 63 leaves, 7 levels; level 4 has 4 nodes
    for i in range(0, 2000, 9):
        a = O.select_unit(q[:, i], k, pyr, i, 4, scale)
        b = O.select_unit_variant(q[:, i], k, pyr, i, 4, scale, max_level=4)
        assert a.sel.tolist() == b.sel.tolist()


# ---------------------------------------------------------------- backward of block-sparse attention
def _dense_masked_attention(qg, k, v, sel, C, scale):
    """Block-sparse attention written densely in torch (float64): scores masked to each query's selected
    tokens t <= i, so that autograd gives the gradients of the definition."""
    G, N, d = qg.shape
    mask = np.zeros((N, N), dtype=bool)
    for i in range(N):
        for j in sel[i]:
            if j >= 0:
                mask[i, j * C:min(N, (j + 1) * C, i + 1)] = True
    m = torch.from_numpy(mask)

    def f(q_, k_, v_):
        z = scale * torch.einsum("gnd,td->gnt", q_, k_)
        z = z.masked_fill(~m[None], float("-inf"))
        return torch.einsum("gnt,td->gnd", torch.softmax(z, dim=-1), v_)

    return f


def test_backward_equals_autograd_of_dense_masked_attention():
    q, k, v, scale = _tiny(N=300, d=16, C=32, G=3, keys="ar1", seed=81)
    pyr = O.build_pyramid(k, 32)
    sel = np.stack([O.select_unit(q[:, i], k, pyr, i, 3, scale).sel for i in range(300)])
    do = _rng(82).standard_normal(q.shape)
    dq, dk, dv = O.attention_backward_head(q, k, v, sel, 32, scale, do)
    f = _dense_masked_attention(q, k, v, sel, 32, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = f(tq, tk, tv)
    # the forward itself is the oracle's attention
    o_ref = np.stack([O.attend_unit(q[:, i], k, v, sel[i], i, 32, scale, 300)[0] for i in range(300)], axis=1)
    np.testing.assert_allclose(out.detach().numpy(), o_ref, rtol=0, atol=1e-12)
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


def test_backward_with_every_block_is_dense_causal_sdpa_backward():
    q, k, v, scale = _tiny(N=200, d=16, C=32, G=2, keys="iid", seed=83)
    n0 = -(-200 // 32)
    sel = np.tile(np.arange(n0), (200, 1))
    sel = np.where(sel * 32 <= np.arange(200)[:, None], sel, -1)
    do = _rng(84).standard_normal(q.shape)
    dq, dk, dv = O.attention_backward_head(q, k, v, sel, 32, scale, do)
    tq = torch.tensor(q[None], requires_grad=True)
    tk = torch.tensor(k[None, None], requires_grad=True)
    tv = torch.tensor(v[None, None], requires_grad=True)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk.expand(1, 2, 200, 16), tv.expand(1, 2, 200, 16),
                                                           is_causal=True, scale=scale)
    out.backward(torch.from_numpy(do[None]))
    np.testing.assert_allclose(dq, tq.grad.numpy()[0], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy()[0, 0], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy()[0, 0], rtol=0, atol=1e-11)


def test_backward_finite_differences():
    """Central differences of L = sum(dO * O) with the selection held fixed."""
    q, k, v, scale = _tiny(N=80, d=8, C=16, G=2, keys="ar1", seed=85)
    pyr = O.build_pyramid(k, 16)
    sel = np.stack([O.select_unit(q[:, i], k, pyr, i, 2, scale).sel for i in range(80)])
    do = _rng(86).standard_normal(q.shape)

    def loss(q_, k_, v_):
        o = np.stack([O.attend_unit(q_[:, i], k_, v_, sel[i], i, 16, scale, 80)[0] for i in range(80)], axis=1)
        return float(np.sum(do * o))

    dq, dk, dv = O.attention_backward_head(q, k, v, sel, 16, scale, do)
    rng = _rng(87)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(rng.integers(0, s_) for s_ in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert fd == pytest.approx(g[idx], rel=1e-6, abs=1e-7), (name, idx)
