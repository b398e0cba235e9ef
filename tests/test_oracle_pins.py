"""Pins of the fp64 oracle against what the source pages and mathematics fix.

None of these re-types the oracle's formulas: each checks the oracle against a
library routine, a closed form, an invariant the pages state, exact
enumeration of the output law, a Monte-Carlo law test, brute force on tiny
trees, or the expected-tokens values printed on the speculative-decoding page.
"""
import itertools
import json
import math
import multiprocessing as mp
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import (InvalidRow, chain_verify_one, inverse_cdf, pack_mask_rows, softmax_T,
                    tree_attention_mask_one, tree_greedy_one, tree_multi_one, tree_path_one)

GRID = 2 ** 24          # the library's uniforms are fp32 multiples of 2^-24


def f32(x):
    return float(np.float32(x))


def sm(z, T):
    """Library softmax of z / T (scipy), the independent route to a distribution."""
    return scipy.special.softmax(np.asarray(z, dtype=np.float64) / f32(T))


# ---------------------------------------------------------------------------
# softmax and inverse CDF against library routines
# ---------------------------------------------------------------------------


def test_softmax_matches_scipy():
    rng = np.random.default_rng(1)
    for V in (1, 2, 7, 1000, 4099):
        for T in (1.0, 0.7, 1.9):
            z = rng.normal(0.0, 3.0, V)
            if V > 3:
                z[rng.integers(0, V, 2)] = -np.inf
            got = softmax_T(z, f32(T))
            np.testing.assert_allclose(got, sm(z, T), rtol=1e-13, atol=0)
            lse = scipy.special.logsumexp(z / f32(T))
            fin = np.isfinite(z)
            np.testing.assert_allclose(np.log(got[fin]), z[fin] / f32(T) - lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("row", [[np.nan, 0.0], [np.inf, 0.0], [-np.inf, -np.inf]])
def test_softmax_rejects_undefined_rows(row):
    with pytest.raises(InvalidRow):
        softmax_T(np.array(row), 1.0)


def test_inverse_cdf_matches_searchsorted():
    rng = np.random.default_rng(2)
    for _ in range(300):
        V = int(rng.integers(1, 60))
        w = rng.random(V)
        w[rng.random(V) < 0.3] = 0.0
        if w.sum() == 0.0:
            w[-1] = 0.5
        c = np.cumsum(w)
        us = np.concatenate([[0.0], rng.random(20, dtype=np.float32).astype(np.float64),
                             [1.0 - 2.0 ** -24]])
        for u in us:
            tok, lo, hi = inverse_cdf(w, u)
            ref = int(np.searchsorted(c, u * c[-1], side="right"))
            if abs(u * c[-1] - c[min(ref, V - 1)]) > 1e-12 * c[-1]:
                assert tok == ref
            assert w[tok] > 0.0                 # zero-weight tokens are never drawn
            assert lo <= u < hi or (tok == np.nonzero(w)[0][-1] and u >= lo)


def test_inverse_cdf_zero_uniform_takes_first_positive():
    w = np.array([0.0, 0.0, 0.2, 0.0, 0.8])
    assert inverse_cdf(w, 0.0)[0] == 2
    assert inverse_cdf(w, 0.2 - 1e-12)[0] == 2
    assert inverse_cdf(w, 0.2)[0] == 4


# ---------------------------------------------------------------------------
# invariants stated for the method
# ---------------------------------------------------------------------------


def _rows(rng, k, V, sig_q=1.0):
    zt = rng.normal(0.0, 2.0, (k + 1, V))
    zq = zt[:k] + rng.normal(0.0, sig_q, (k, V))
    return zt, zq


def test_lambda_one_accepts_every_draft():
    rng = np.random.default_rng(3)
    for _ in range(50):
        k, V = int(rng.integers(1, 6)), int(rng.integers(2, 40))
        zt, zq = _rows(rng, k, V)
        x = rng.integers(0, V, k)
        r = chain_verify_one(zt, zq, x, rng.random(k), rng.random(), 1.0, 1.0)
        assert r.accepted == k and r.bonus
        assert np.all(r.a == 1.0)
        assert r.tokens[:k] == [int(v) for v in x]


@pytest.mark.parametrize("lam", [0.0, 0.3, 0.7, 1.0])
def test_identical_target_and_draft_accept_every_draft(lam):
    rng = np.random.default_rng(4)
    for _ in range(50):
        k, V = int(rng.integers(1, 6)), int(rng.integers(2, 40))
        z = rng.normal(0.0, 2.0, (k + 1, V))
        x = rng.integers(0, V, k)
        u = rng.random(k, dtype=np.float32)
        r = chain_verify_one(z, z[:k], x, u, rng.random(), lam, 0.8)
        assert r.accepted == k


def test_acceptance_rate_closed_form():
    """E_{x~q}[a(x)] = sum_v min(p~, q) = 1 - (1 - lam) * TV(p_t, q)."""
    rng = np.random.default_rng(5)
    for _ in range(40):
        V = int(rng.integers(2, 30))
        lam, T = float(rng.choice([0.0, 0.1, 0.3, 0.9])), float(rng.choice([1.0, 0.7, 1.5]))
        zt, zq = _rows(rng, 1, V)
        p, q = sm(zt[0], T), sm(zq[0], T)
        ea = sum(q[x] * chain_verify_one(zt, zq, [x], [0.5], 0.5, lam, T).a[0] for x in range(V))
        tv = 0.5 * np.abs(p - q).sum()
        lam32 = f32(lam)
        assert ea == pytest.approx(1.0 - (1.0 - lam32) * tv, abs=1e-12)
        alpha = chain_verify_one(zt, zq, [0], [0.5], 0.5, lam, T).alpha[0]
        assert alpha == pytest.approx(1.0 - (1.0 - lam32) * tv, abs=1e-12)


def test_acceptance_probability_at_least_lambda():
    rng = np.random.default_rng(6)
    for _ in range(100):
        V = int(rng.integers(2, 30))
        lam = float(rng.random())
        zt, zq = _rows(rng, 3, V, 3.0)
        r = chain_verify_one(zt, zq, rng.integers(0, V, 3), [0.0] * 3, 0.5, lam, 1.0)
        assert np.all(r.a >= f32(lam) - 1e-15) and np.all(r.a <= 1.0)


def test_residual_law_independent_of_lambda():
    """max(0, p~ - q) = (1 - lam) max(0, p_t - q): one law for every lam < 1."""
    rng = np.random.default_rng(7)
    done = 0
    while done < 40:
        V = int(rng.integers(3, 30))
        zt, zq = _rows(rng, 1, V, 2.0)
        p, q = sm(zt[0], 1.0), sm(zq[0], 1.0)
        x = int(np.argmax(q / p))                      # p_t(x) < q(x): rejectable
        us = rng.random()
        out = []
        for lam in (0.0, 0.25, 0.6):
            a = chain_verify_one(zt, zq, [x], [0.0], us, lam, 1.0).a[0]
            r = chain_verify_one(zt, zq, [x], [min(a + 1e-9, 1 - 2 ** -24)], us, lam, 1.0)
            if r.accepted == 0:
                out.append((r.tokens[0], r.F_lo, r.F_hi))
        if len(out) == 3:
            assert out[0][0] == out[1][0] == out[2][0]
            assert out[0][1] == pytest.approx(out[2][1], abs=1e-12)
            done += 1


def test_bad_token_and_parent_raise():
    zt, zq = np.zeros((2, 4)), np.zeros((1, 4))
    with pytest.raises(ValueError):
        chain_verify_one(zt, zq, [4], [0.1], 0.1, 0.0, 1.0)
    with pytest.raises(ValueError):
        tree_greedy_one(np.zeros((3, 4)), [0, 2], [0, 0])


# ---------------------------------------------------------------------------
# exact enumeration of the output law over the fp32 uniform grid
# ---------------------------------------------------------------------------


def _count_true(pred):
    """#grid points m in [0, GRID) with pred(m / GRID), pred True then False."""
    lo, hi = 0, GRID
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid / GRID):
            lo = mid + 1
        else:
            hi = mid
    return lo


def _enumerate(zt, zq, lam, T, space="prob"):
    """Exact law of every emitted position, the oracle used as a black box.

    Returns (emit[j, v] = P(position j emits v), stop[j] = P(n = j)).
    """
    k, V = zq.shape
    q = [sm(zq[i], T) for i in range(k)]
    emit = np.zeros((k + 1, V))
    stop = np.zeros(k + 1)
    for xs in itertools.product(range(V), repeat=k):
        px = math.prod(q[i][xs[i]] for i in range(k))
        if px == 0.0:
            continue

        def run(ua, us):
            return chain_verify_one(zt, zq, list(xs), ua, us, lam, T, space)

        reach = 1.0
        theta_m = []
        for i in range(k):
            def acc(u, i=i):
                return run([0.0] * i + [u] + [0.0] * (k - i - 1), 0.5).accepted > i
            theta_m.append(_count_true(acc) if reach > 0.0 else 0)
            reach *= theta_m[-1] / GRID
        reach = 1.0
        for j in range(k + 1):
            pj = reach * ((GRID - theta_m[j]) / GRID if j < k else 1.0)
            if pj > 0.0:
                ua = [0.0] * j + ([theta_m[j] / GRID] if j < k else []) + [0.0] * max(0, k - j - 1)
                cnt_prev = 0
                for v in range(V):
                    cnt = _count_true(lambda u, v=v: run(ua, u).tokens[-1] <= v)
                    emit[j, v] += px * pj * (cnt - cnt_prev) / GRID
                    cnt_prev = cnt
                for i in range(j):
                    emit[i, xs[i]] += px * pj
                stop[j] += px * pj
            if j < k:
                reach *= theta_m[j] / GRID
    return emit, stop


@pytest.mark.parametrize("V,k,lam,T,seed,space", [
    (3, 2, 0.0, 1.0, 11, "prob"), (4, 2, 0.3, 0.7, 12, "prob"), (2, 3, 0.5, 1.5, 13, "prob"),
    (3, 3, 0.0, 1.0, 14, "prob"), (4, 2, 0.3, 0.7, 15, "logit"), (3, 3, 0.6, 1.2, 16, "logit"),
])
def test_exact_enumeration_is_lossless(V, k, lam, T, seed, space):
    """Each emitted position follows p~ given that it is reached; the bonus follows p_t.

    [SD] "修改的拒绝采样" and [EAGLE] section 1: the output law equals the target
    law whatever the draft; with RAPID's mixture the target law is p~ (the
    mixture equation of section 2, or the pseudocode's softmax of mixed logits).
    """
    rng = np.random.default_rng(seed)
    zt, zq = _rows(rng, k, V, 1.5)
    zt[1, 0] = -np.inf                          # a token the target rules out
    emit, stop = _enumerate(zt, zq, lam, T, space)
    lam32 = f32(lam)
    reach = 1.0
    tol = 1e-6                                  # uniforms live on a 2^-24 grid
    for j in range(k):
        p, q = sm(zt[j], T), sm(zq[j], T)
        if space == "prob":
            pm = (1.0 - lam32) * p + lam32 * q  # the mixture equation of the RAPID page
        else:                                   # the pseudocode's mixed logits, via scipy
            pm = scipy.special.softmax(((1.0 - lam32) * zt[j] + lam32 * zq[j]) / f32(T))
        assert emit[j].sum() == pytest.approx(reach, abs=tol)
        np.testing.assert_allclose(emit[j], reach * pm, atol=tol)
        alpha = np.minimum(pm, q).sum()
        assert stop[j] == pytest.approx(reach * (1.0 - alpha), abs=tol)
        reach *= alpha
    np.testing.assert_allclose(emit[k], reach * sm(zt[k], T), atol=tol)
    assert stop.sum() == pytest.approx(1.0, abs=tol)


# ---------------------------------------------------------------------------
# Monte-Carlo law test, 10^6 seeded requests at V <= 8
# ---------------------------------------------------------------------------

_MC = dict(V=6, k=2, lam=0.3, T=0.8, n=1_000_000, workers=8)


def _mc_rows():
    rng = np.random.default_rng(2024)
    zt = rng.normal(0.0, 1.5, (_MC["k"] + 1, _MC["V"]))
    zq = zt[:_MC["k"]] + rng.normal(0.0, 1.0, (_MC["k"], _MC["V"]))
    zt[1, 2] = -np.inf
    return zt, zq


def _mc_worker(args):
    seed, n = args
    V, k, lam, T = _MC["V"], _MC["k"], _MC["lam"], _MC["T"]
    zt, zq = _mc_rows()
    rng = np.random.default_rng(seed)
    q = [sm(zq[i], T) for i in range(k)]
    xs = np.stack([rng.choice(V, size=n, p=q[i]) for i in range(k)], axis=1)
    ua = rng.random((n, k), dtype=np.float32)
    us = rng.random(n, dtype=np.float32)
    first = np.zeros(V, dtype=np.int64)
    second = np.zeros(V, dtype=np.int64)
    bonus = np.zeros(V, dtype=np.int64)
    nh = np.zeros(k + 1, dtype=np.int64)
    for i in range(n):
        r = chain_verify_one(zt, zq, xs[i], ua[i], us[i], lam, T)
        nh[r.accepted] += 1
        first[r.tokens[0]] += 1
        if r.accepted >= 1:
            second[r.tokens[1]] += 1
        if r.accepted == k:
            bonus[r.tokens[-1]] += 1
    return first, second, bonus, nh


def _chisq(obs, prob):
    obs = np.asarray(obs, dtype=np.float64)
    exp = prob * obs.sum()
    zero = exp == 0.0
    assert np.all(obs[zero] == 0)
    return scipy.stats.chisquare(obs[~zero], exp[~zero] * obs[~zero].sum() / exp[~zero].sum()).pvalue


@pytest.mark.slow
def test_monte_carlo_output_law():
    """10^6 seeded requests: emitted tokens follow p~ (bonus: p_t), chi-square p > 0.01."""
    V, k, lam, T, n, W = (_MC[s] for s in ("V", "k", "lam", "T", "n", "workers"))
    ctx = mp.get_context("fork")
    with ctx.Pool(W) as pool:
        parts = pool.map(_mc_worker, [(9000 + w, n // W) for w in range(W)])
    first, second, bonus, nh = (sum(p[i] for p in parts) for i in range(4))
    zt, zq = _mc_rows()
    lam32 = f32(lam)
    pm = [(1 - lam32) * sm(zt[j], T) + lam32 * sm(zq[j], T) for j in range(k)]
    alpha = [np.minimum(pm[j], sm(zq[j], T)).sum() for j in range(k)]
    law_n = np.array([1 - alpha[0], alpha[0] * (1 - alpha[1]), alpha[0] * alpha[1]])
    assert _chisq(first, pm[0]) > 0.01
    assert _chisq(second, pm[1]) > 0.01
    assert _chisq(bonus, sm(zt[2], T)) > 0.01
    assert _chisq(nh, law_n) > 0.01


# ---------------------------------------------------------------------------
# expected tokens per step: the values printed on the speculative-decoding page
# ---------------------------------------------------------------------------


def test_expected_tokens_match_printed_speedups(golden_dir):
    """Draft q = (1, 0), target p = (r, 1 - r): every position accepts with prob r.

    The expected number of emitted tokens, 1 + r + ... + r^k, must reproduce
    the printed 2 / 3.3 / 5 at r = 0.5 / 0.7 / 0.8 (k = 64).
    """
    with open(os.path.join(golden_dir, "sd_expected_tokens.json")) as f:
        gold = json.load(f)
    k = 64
    for case in gold["cases"]:
        r = case["r"]
        zq = np.tile([0.0, -np.inf], (k, 1))
        zt = np.tile([math.log(r), math.log(1.0 - r)], (k + 1, 1))
        theta = _count_true(lambda u: chain_verify_one(zt, zq, [0] * k, [u] + [0.99] * (k - 1),
                                                       0.5, 0.0, 1.0).accepted > 0) / GRID
        assert theta == pytest.approx(r, abs=2.0 ** -23)
        expected = sum(theta ** j for j in range(k + 1))
        assert abs(expected - case["printed"]) <= case["printed_precision"]
        # every accepted position emits its draft; the stop emits one more token
        for j in (0, 3, 17):
            res = chain_verify_one(zt, zq, [0] * k, [0.0] * j + [0.999] * (k - j), 0.5, 0.0, 1.0)
            assert res.accepted == j and len(res.tokens) == j + 1


# ---------------------------------------------------------------------------
# greedy tree verification against brute force
# ---------------------------------------------------------------------------


def _brute_greedy(zt, parent, tok):
    N = len(parent)
    am = [int(np.argmax(zt[r])) for r in range(N + 1)]
    best = []
    for v in range(1, N + 1):
        path, u = [], v
        while u != 0:
            path.append(u)
            u = int(parent[u - 1])
        path.reverse()
        prev, ok = 0, True
        for u in path:
            if int(tok[u - 1]) != am[prev]:
                ok = False
                break
            prev = u
        if ok and len(path) > len(best):
            best = path
    last = best[-1] if best else 0
    return len(best), [int(tok[u - 1]) for u in best] + [am[last]], best


def test_greedy_tree_matches_brute_force():
    rng = np.random.default_rng(21)
    for _ in range(600):
        N = int(rng.integers(1, 12))
        V = int(rng.integers(1, 5))
        parent = np.array([int(rng.integers(0, i)) for i in range(1, N + 1)])
        zt = rng.integers(-2, 3, (N + 1, V)).astype(np.float64)     # many ties
        tok = rng.integers(0, V, N)
        r = tree_greedy_one(zt, parent, tok)
        acc, toks, nodes = _brute_greedy(zt, parent, tok)
        assert (r.accepted, r.tokens, r.nodes) == (acc, toks, nodes)


def test_greedy_ties_take_lowest_token():
    zt = np.array([[1.0, 3.0, 3.0, 0.0], [0.0, 0.0, 5.0, 0.0], [9.0, 0.0, 0.0, 0.0]])
    r = tree_greedy_one(zt, [0, 0], [2, 1])
    assert r.accepted == 1 and r.nodes == [2] and r.tokens == [1, 0]


def test_greedy_chain_shaped_tree_is_prefix_match():
    rng = np.random.default_rng(22)
    for _ in range(100):
        N, V = int(rng.integers(1, 9)), int(rng.integers(2, 6))
        zt = rng.normal(size=(N + 1, V))
        am = np.argmax(zt, axis=1)
        tok = np.where(rng.random(N) < 0.7, am[:N], rng.integers(0, V, N))
        j = 0
        while j < N and tok[j] == am[j]:
            j += 1
        r = tree_greedy_one(zt, np.arange(N), tok)
        assert r.accepted == j and r.tokens[-1] == am[j]


def test_greedy_no_match_returns_root_argmax():
    zt = np.array([[0.0, 2.0, 1.0], [5.0, 0.0, 0.0], [0.0, 0.0, 5.0]])
    r = tree_greedy_one(zt, [0, 0], [0, 2])
    assert r.accepted == 0 and r.tokens == [1] and r.nodes == []


# ---------------------------------------------------------------------------
# path mode is the chain on the gathered rows
# ---------------------------------------------------------------------------


def test_path_mode_is_chain_on_gathered_rows():
    rng = np.random.default_rng(23)
    parent = np.array([0, 0, 1, 1, 2, 3, 5])          # nodes 1..7
    N, V = len(parent), 9
    zt = rng.normal(0, 2, (N + 1, V))
    zq = zt + rng.normal(0, 1, (N + 1, V))
    tok = rng.integers(0, V, N)
    path = np.array([2, 5, 7, -1, 9])                  # root -> 2 -> 5 -> 7 (entry after -1 ignored)
    for _ in range(30):
        ua, us = rng.random(5, dtype=np.float32), float(rng.random(dtype=np.float32))
        r = tree_path_one(zt, zq, tok, path, ua, us, 0.2, 0.9)
        c = chain_verify_one(zt[[0, 2, 5, 7]], zq[[0, 2, 5]], tok[[1, 4, 6]], ua[:3], us, 0.2, 0.9)
        assert (r.accepted, r.tokens) == (c.accepted, c.tokens)
        np.testing.assert_array_equal(r.a, c.a)


# ---------------------------------------------------------------------------
# tree-attention mask: each node sees its ancestor path (and itself)
# ---------------------------------------------------------------------------


def _closure(parent):
    """Ancestor-or-self relation by boolean matrix powers of the parent map
    (an independent route: no walk, no depth recursion)."""
    N = len(parent)
    A = np.zeros((N + 1, N + 1), dtype=np.int64)
    for i, p in enumerate(parent, start=1):
        A[i, p] = 1
    R = np.eye(N + 1, dtype=np.int64)
    while True:
        nxt = np.minimum(R + R @ A, 1)
        if np.array_equal(nxt, R):
            return R.astype(bool)
        R = nxt


def test_mask_of_chain_is_causal():
    for N in (0, 1, 5, 40):
        r = tree_attention_mask_one(np.arange(N))
        np.testing.assert_array_equal(r.mask, np.tril(np.ones((N + 1, N + 1), dtype=bool)))
        np.testing.assert_array_equal(r.depth, np.arange(N + 1))


def test_mask_of_star_is_root_plus_self():
    N = 9
    r = tree_attention_mask_one(np.zeros(N, dtype=int))
    want = np.eye(N + 1, dtype=bool)
    want[:, 0] = True
    np.testing.assert_array_equal(r.mask, want)
    np.testing.assert_array_equal(r.depth, [0] + [1] * N)


def test_mask_matches_matrix_closure():
    rng = np.random.default_rng(31)
    for _ in range(200):
        N = int(rng.integers(1, 40))
        parent = np.array([int(rng.integers(0, i)) for i in range(1, N + 1)])
        r = tree_attention_mask_one(parent)
        np.testing.assert_array_equal(r.mask, _closure(parent))
        # depth by the recursion depth[i] = depth[parent] + 1 in node order
        d = [0] * (N + 1)
        for i in range(1, N + 1):
            d[i] = d[parent[i - 1]] + 1
        np.testing.assert_array_equal(r.depth, d)
        assert not r.bad


def test_mask_bad_parent_reads_as_root_child():
    r = tree_attention_mask_one([0, 5, 1, -1])          # nodes 2 and 4 have bad parents
    assert r.bad
    good = tree_attention_mask_one([0, 0, 1, 0])
    np.testing.assert_array_equal(r.mask, good.mask)


def test_mask_packing_matches_packbits():
    rng = np.random.default_rng(32)
    m = rng.random((7, 70)) < 0.5
    words = 3
    packed = pack_mask_rows(m, words)
    pad = np.zeros((7, words * 32), dtype=bool)
    pad[:, :70] = m
    ref = np.packbits(pad, axis=1, bitorder="little").view("<u4")
    np.testing.assert_array_equal(packed, ref)


# ---------------------------------------------------------------------------
# logit-space mixture (the RAPID pseudocode's form)
# ---------------------------------------------------------------------------


def test_logit_mixture_at_lambda_zero_is_the_plain_chain():
    rng = np.random.default_rng(41)
    for _ in range(50):
        k, V = int(rng.integers(1, 5)), int(rng.integers(2, 30))
        zt, zq = _rows(rng, k, V, 2.0)
        x = rng.integers(0, V, k)
        ua, us = rng.random(k, dtype=np.float32), float(rng.random(dtype=np.float32))
        a = chain_verify_one(zt, zq, x, ua, us, 0.0, 0.9, "logit")
        b = chain_verify_one(zt, zq, x, ua, us, 0.0, 0.9, "prob")
        assert (a.accepted, a.tokens) == (b.accepted, b.tokens)
        np.testing.assert_array_equal(a.a, b.a)


def test_logit_mixture_at_lambda_one_accepts_every_draft():
    rng = np.random.default_rng(42)
    zt, zq = _rows(rng, 4, 12, 2.0)
    zt[0, :] = -np.inf                          # the target's own row no longer matters
    zt[0, 3] = 0.0
    for _ in range(20):
        x = rng.integers(0, 12, 4)
        r = chain_verify_one(zt, zq, x, rng.random(4, dtype=np.float32), 0.5, 1.0, 1.0, "logit")
        assert r.accepted == 4 and np.all(r.a == 1.0)


def test_logit_mixture_is_the_normalised_geometric_mixture():
    """softmax((1-l) z_t + l z_q) = p_t^(1-l) q^l / sum: an independent route
    through scipy's log_softmax, checked on the acceptance probabilities and
    the expected acceptance sum_v min(p~, q)."""
    rng = np.random.default_rng(43)
    for _ in range(60):
        k, V = int(rng.integers(1, 4)), int(rng.integers(2, 40))
        lam, T = float(rng.uniform(0.05, 0.95)), float(rng.uniform(0.5, 2.0))
        zt, zq = _rows(rng, k, V, 2.5)
        x = rng.integers(0, V, k)
        r = chain_verify_one(zt, zq, x, np.zeros(k, dtype=np.float32), 0.5, lam, T, "logit")
        l32, T32 = f32(lam), f32(T)
        for i in range(k):
            lp = scipy.special.log_softmax(zt[i] / T32)
            lq = scipy.special.log_softmax(zq[i] / T32)
            pe = scipy.special.softmax((1.0 - l32) * lp + l32 * lq)
            q = np.exp(lq)
            assert r.a[i] == pytest.approx(min(1.0, pe[x[i]] / q[x[i]]), rel=1e-12, abs=1e-15)
            assert r.alpha[i] == pytest.approx(np.minimum(pe, q).sum(), rel=1e-12)


def test_logit_mixture_identical_rows_accept_every_draft():
    rng = np.random.default_rng(44)
    zt, _ = _rows(rng, 3, 20, 2.0)
    zq = zt[:3].copy()
    for lam in (0.2, 0.5, 0.9):
        r = chain_verify_one(zt, zq, rng.integers(0, 20, 3), rng.random(3, dtype=np.float32),
                             0.3, lam, 1.1, "logit")
        assert r.accepted == 3


# ---------------------------------------------------------------------------
# multi-branch stochastic tree verification (sibling retries)
# ---------------------------------------------------------------------------


def test_multi_on_a_chain_shaped_tree_is_the_chain():
    rng = np.random.default_rng(51)
    for _ in range(80):
        N, V = int(rng.integers(1, 6)), int(rng.integers(2, 9))
        lam, T = float(rng.choice([0.0, 0.3])), float(rng.uniform(0.7, 1.3))
        space = str(rng.choice(["prob", "logit"]))
        zt = rng.normal(0, 2, (N + 1, V))
        zq = zt + rng.normal(0, 1, (N + 1, V))
        tok = rng.integers(0, V, N)
        ua, us = rng.random(N, dtype=np.float32), float(rng.random(dtype=np.float32))
        m = tree_multi_one(zt, zq, np.arange(N), tok, ua, us, lam, T, space)
        c = chain_verify_one(zt, zq[:N], tok, ua, us, lam, T, space)
        assert (m.accepted, m.tokens) == (c.accepted, c.tokens)
        k = len(m.tested)
        np.testing.assert_array_equal(m.a[:k], c.a[:k])


def test_multi_at_lambda_one_accepts_the_first_child():
    rng = np.random.default_rng(52)
    parent = [0, 0, 0, 1, 1, 2]
    zt = rng.normal(0, 2, (7, 5))
    zq = zt + rng.normal(0, 1, (7, 5))
    for _ in range(20):
        tok = rng.integers(0, 5, 6)
        m = tree_multi_one(zt, zq, parent, tok, rng.random(6, dtype=np.float32), 0.5, 1.0, 1.0)
        assert m.nodes[0] == 1 and m.tested[0] == 1 and m.a[0] == 1.0


def _tree_rows(rng, parent, tok, V, table):
    """Rows of a tree whose logits depend only on the token prefix of each node
    (as a language model's would): table maps a prefix tuple to (z_t, z_q)."""
    N = len(parent)
    prefix = [()] + [None] * N
    for i in range(1, N + 1):
        prefix[i] = prefix[parent[i - 1]] + (int(tok[i - 1]),)
    zt = np.stack([table(prefix[i])[0] for i in range(N + 1)])
    zq = np.stack([table(prefix[i])[1] for i in range(N + 1)])
    return zt, zq, prefix


def _enumerate_tree(parent, V, table, lam, T, space):
    """Exact law of the emitted token sequence, the oracle as a black box:
    every assignment of node tokens (each child an independent draw from its
    parent's q), every acceptance outcome (thresholds found by bisection over
    the fp32 grid, the next tested node read from the oracle's trace) and the
    final draw's CDF over the sampling uniform."""
    N = len(parent)
    law = {}

    def q_of(prefix):
        return sm(table(prefix)[1], T)

    for toks in itertools.product(range(V), repeat=N):
        zt, zq, prefix = _tree_rows(None, parent, toks, V, table)
        w0 = 1.0
        for i in range(1, N + 1):
            w0 *= q_of(prefix[parent[i - 1]])[toks[i - 1]]
        if w0 == 0.0:
            continue

        def run(fixed, us):
            ua = np.zeros(N, dtype=np.float64)
            for n, u in fixed.items():
                ua[n - 1] = u
            return tree_multi_one(zt, zq, parent, toks, ua, us, lam, T, space)

        def explore(fixed, w):
            r = run(fixed, 0.5)
            nxt = [n for n in r.tested if n not in fixed]
            if nxt:
                n = nxt[0]
                theta = _count_true(lambda u: n in run({**fixed, n: u}, 0.5).nodes)
                if theta > 0:
                    explore({**fixed, n: 0.0}, w * theta / GRID)
                if theta < GRID:
                    explore({**fixed, n: theta / GRID}, w * (GRID - theta) / GRID)
                return
            head = tuple(r.tokens[:-1])
            prev = 0
            for v in range(V):
                cnt = _count_true(lambda u: run(fixed, u).tokens[-1] <= v)
                if cnt > prev:
                    key = head + (v,)
                    law[key] = law.get(key, 0.0) + w * (cnt - prev) / GRID
                prev = cnt

        explore({}, w0)
    return law


def _check_conditional_laws(law, parent, table, lam, T, space, V):
    depth = [0] * (len(parent) + 1)
    for i in range(1, len(parent) + 1):
        depth[i] = depth[parent[i - 1]] + 1
    leaf_depth = max(depth)
    lam32 = f32(lam)
    assert sum(law.values()) == pytest.approx(1.0, abs=1e-6)
    prefixes = {k[:j] for k in law for j in range(len(k))}
    for s_ in prefixes:
        mass = np.array([sum(p for k, p in law.items() if len(k) > len(s_) and k[:len(s_) + 1] == s_ + (v,))
                         for v in range(V)])
        tot = mass.sum()
        if tot < 1e-9:
            continue
        zt_, zq_ = table(s_)
        if len(s_) < leaf_depth:
            if space == "prob":
                want = (1 - lam32) * sm(zt_, T) + lam32 * sm(zq_, T)
            else:
                want = scipy.special.softmax(((1 - lam32) * zt_ + lam32 * zq_) / f32(T))
        else:
            want = sm(zt_, T)                      # the bonus at a leaf: the target alone
        np.testing.assert_allclose(mass / tot, want, atol=2e-6 / tot)


def _prefix_table(seed, V):
    rng = np.random.default_rng(seed)
    cache = {}

    def table(prefix):
        if prefix not in cache:
            zt = rng.normal(0.0, 1.5, V)
            cache[prefix] = (zt, zt + rng.normal(0.0, 1.2, V))
        return cache[prefix]
    return table


@pytest.mark.parametrize("parent,V,lam,T,space,seed", [
    ([0, 0, 0], 3, 0.0, 1.0, "prob", 61),            # a star: three sibling retries
    ([0, 0, 0], 3, 0.4, 0.8, "logit", 62),
    ([0, 0, 1, 1, 2, 2], 2, 0.3, 1.2, "prob", 63),   # two levels of two children
])
def test_multi_exact_enumeration_is_lossless(parent, V, lam, T, space, seed):
    """Each emitted token, given the tokens before it, follows p~ of its prefix
    (the target alone for the bonus after a leaf): the multi-branch walk keeps
    the chain's lossless property ([SD] "修改的拒绝采样", [EAGLE] section 1)."""
    table = _prefix_table(seed, V)
    law = _enumerate_tree(parent, V, table, lam, T, space)
    _check_conditional_laws(law, parent, table, lam, T, space, V)

