"""Pins of the oracle's excusal rules and degenerate-case readings.

Parity with the GPU excuses a request only when one of its draws lies within
1e-6 of the boundary it is compared with; these tests pin that predicate and
the two degenerate readings the parity tests lean on:

* the boundary band: an acceptance uniform u_i within 1e-6 of a_i < 1 (for a
  position at or before the first rejection), or a sampling uniform within
  1e-6 of F(token - 1) or F(token), flags the request; farther away it does
  not.  The boundaries are computed here from scipy's softmax and numpy's
  cumsum, not read from the oracle;
* q(x) = 0 (a draft the drafter could not have drawn): accepted iff
  p~(x) > 0, which is the limit of min(1, p~(x) / q(x)) as q(x) -> 0 ([SD]
  "修改的拒绝采样": accept outright when p >= q);
* zero residual mass after a rejection: the token is drawn from p~ of that
  row, which exact enumeration over the fp32 uniform grid confirms ([EAGLE]
  section "1. 为什么无损": the residual max(0, p~ - q) is undefined when it
  vanishes everywhere; the reading keeps the output law p~).

Each check is also run against copies of the oracle with a planted mistake (a
wider band, an inverted comparison, a fallback from the wrong law, ...); every
planted mistake must make a check fail.
"""
import importlib.util
import os
import sys

import numpy as np
import pytest
import scipy.special

import oracle.verify as ov

GRID = 2 ** 24
NEAR, FAR = 5e-7, 2e-6          # inside and outside the 1e-6 band


def f32(x):
    return float(np.float32(x))


def sm(z, T=1.0):
    return scipy.special.softmax(np.asarray(z, dtype=np.float64) / f32(T))


def cdf(w):
    w = np.asarray(w, dtype=np.float64)
    return np.cumsum(w) / w.sum()


def resid(pm, q):
    w = np.maximum(0.0, pm - q)
    return w / w.sum()


def far_uniform(*laws):
    """A uniform at least 1e-3 away from every boundary of every law (their CDFs)."""
    cands = np.linspace(0.011, 0.989, 979)
    bounds = np.concatenate([[0.0]] + [cdf(w) for w in laws])
    dist = np.min(np.abs(cands[:, None] - bounds[None, :]), axis=1)
    u = float(cands[int(np.argmax(dist))])
    assert dist.max() > 1e-3
    return f32(u)


def count_true(pred):
    """#grid points m in [0, GRID) with pred(m / GRID); pred True then False."""
    lo, hi = 0, GRID
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid / GRID):
            lo = mid + 1
        else:
            hi = mid
    return lo


def token_law(draw, V):
    """Law of the token draw(u) over the fp32 uniform grid (draw monotone in u)."""
    law = np.zeros(V)
    prev = 0
    for v in range(V):
        cnt = count_true(lambda u, v=v: draw(u) <= v)
        law[v] = (cnt - prev) / GRID
        prev = cnt
    return law


# ---------------------------------------------------------------------------
# the checks, each taking the oracle module (or a mutant of it)
# ---------------------------------------------------------------------------


def _chain_rows(seed, V=6):
    rng = np.random.default_rng(seed)
    zt = rng.normal(0.0, 1.5, (3, V))
    zq = zt[:2] + rng.normal(0.0, 1.0, (2, V))
    return zt, zq


def check_chain_acceptance_band(m):
    for seed, lam in ((1, 0.0), (2, 0.3), (3, 0.0)):
        zt, zq = _chain_rows(seed)
        lam32 = f32(lam)
        p, q = sm(zt[0]), sm(zq[0])
        pm = (1.0 - lam32) * p + lam32 * q
        x = int(np.argmax(q / pm))                       # p~(x) < q(x): a < 1
        a = pm[x] / q[x]
        assert 1e-3 < a < 1.0 - 1e-3
        # the bonus (accepted) and residual (rejected) laws: u_s far from both
        us = far_uniform(sm(zt[1]), resid(pm, q))
        for d, want in ((NEAR, True), (-NEAR, True), (FAR, False), (-FAR, False)):
            u = f32(a + d)
            r = m.chain_verify_one(zt[:2], zq[:1], [x], [u], us, lam, 1.0)
            assert r.accepted == (1 if u < a else 0)
            assert r.flagged == want, (seed, d, r.a[0], u)


def check_chain_band_ignores_undrawn_positions(m):
    zt, zq = _chain_rows(4)
    p0, q0, p1, q1 = sm(zt[0]), sm(zq[0]), sm(zt[1]), sm(zq[1])
    x0, x1 = int(np.argmax(q0 / p0)), int(np.argmax(q1 / p1))
    a0, a1 = p0[x0] / q0[x0], p1[x1] / q1[x1]
    assert a0 < 0.9 and a1 < 0.999
    us = far_uniform(resid(p0, q0))
    # rejected at position 0: position 1's uniform is never compared
    r = m.chain_verify_one(zt, zq, [x0, x1], [f32(a0 + 0.05), f32(a1 + NEAR)], us, 0.0, 1.0)
    assert r.accepted == 0 and not r.flagged
    # accepted at 0: now position 1 is compared and its uniform is in the band
    us = far_uniform(resid(p1, q1), sm(zt[2]))
    r = m.chain_verify_one(zt, zq, [x0, x1], [f32(a0 - 0.05), f32(a1 + NEAR)], us, 0.0, 1.0)
    assert r.accepted == 1 and r.flagged


def check_chain_band_needs_ratio_below_one(m):
    zt, zq = _chain_rows(5)
    p, q = sm(zt[0]), sm(zq[0])
    x = int(np.argmax(p / q))                            # p(x) > q(x): a = 1
    us = far_uniform(sm(zt[1]))
    r = m.chain_verify_one(zt[:2], zq[:1], [x], [f32(1.0 - 2.0 ** -24)], us, 0.0, 1.0)
    assert r.a[0] == 1.0 and r.accepted == 1 and not r.flagged


def check_chain_sample_band(m):
    # K = 0: one draw from the target row
    rng = np.random.default_rng(6)
    zt = rng.normal(0.0, 1.0, (1, 7))
    F = cdf(sm(zt[0]))
    j = 1 + int(np.argmax(np.diff(F)))                   # widest interval, not the first token
    cases = ((F[j] - NEAR, True), (F[j] - FAR, False), (F[j - 1] + NEAR, True),
             (F[j - 1] + FAR, False))
    for us, want in cases:
        r = m.chain_verify_one(zt, np.zeros((0, 7)), [], [], f32(us), 0.0, 1.0)
        assert r.tokens == [j]
        assert r.flagged == want, (us, F[j - 1], F[j])
    # a residual draw after a rejection at position 0
    zt, zq = _chain_rows(7)
    p, q = sm(zt[0], 0.8), sm(zq[0], 0.8)
    x = int(np.argmax(q / p))
    a = p[x] / q[x]
    F = cdf(resid(p, q))
    j = int(np.argmax(np.diff(np.concatenate([[0.0], F]))))
    lo = F[j - 1] if j > 0 else 0.0
    for us, want in ((F[j] - NEAR, True), (F[j] - FAR, False), (lo + NEAR, True), (lo + FAR, False)):
        r = m.chain_verify_one(zt[:2], zq[:1], [x], [f32(min(a + 0.05, 0.999))], f32(us), 0.0, 0.8)
        assert r.accepted == 0 and r.tokens == [j]
        assert r.flagged == want, (us, lo, F[j])


def _multi_case():
    """Root with two children whose acceptance ratios a1 (against p~) and a2
    (against the normalised residual) both lie well inside (0, 1)."""
    V, lam, T = 6, 0.25, 1.0
    for seed in range(200):
        rng = np.random.default_rng(1000 + seed)
        zt = rng.normal(0.0, 1.5, (3, V))
        zq = zt + rng.normal(0.0, 1.0, (3, V))
        lam32 = f32(lam)
        q = sm(zq[0], T)
        pm = (1.0 - lam32) * sm(zt[0], T) + lam32 * q
        r1 = resid(pm, q)
        r2w = np.maximum(0.0, r1 - q)
        x1 = int(np.argmax(q / pm))
        for x2 in range(V):
            a1, a2 = pm[x1] / q[x1], r1[x2] / q[x2]
            if 0.05 < a1 < 0.95 and 0.05 < a2 < 0.95 and r2w.sum() > 0.05:
                return dict(zt=zt, zq=zq, x=[x1, x2], a1=a1, a2=a2, pm=pm, q=q, r1=r1,
                            r2=r2w / r2w.sum(), lam=lam, T=T)
    raise AssertionError("no tree case found")


def check_multi_bands(m):
    c = _multi_case()
    parent = [0, 0]
    zt, zq, x, lam, T = c["zt"], c["zq"], c["x"], c["lam"], c["T"]
    bonus1, bonus2 = sm(zt[1], T), sm(zt[2], T)
    us = far_uniform(bonus1, bonus2, c["r2"])
    # first child, acceptance band
    for d, want in ((NEAR, True), (-NEAR, True), (FAR, False), (-FAR, False)):
        u1 = f32(c["a1"] + d)
        r = m.tree_multi_one(zt, zq, parent, x, [u1, 0.999], us, lam, T)
        assert r.accepted == (1 if u1 < c["a1"] else 0)
        assert r.flagged == want, (d, r.a, u1)
    # first child rejected far from its band; the second child's band
    u1 = f32(min(c["a1"] + 0.03, 0.999))
    for d, want in ((NEAR, True), (-NEAR, True), (FAR, False), (-FAR, False)):
        u2 = f32(c["a2"] + d)
        r = m.tree_multi_one(zt, zq, parent, x, [u1, u2], us, lam, T)
        assert r.tested == [1, 2]
        assert r.accepted == (1 if u2 < c["a2"] else 0)
        assert r.flagged == want, (d, r.a, u2)
    # both rejected: the draw from the second residual, at its CDF boundaries
    u2 = f32(min(c["a2"] + 0.03, 0.999))
    F = cdf(c["r2"])
    j = int(np.argmax(np.diff(np.concatenate([[0.0], F]))))
    lo = F[j - 1] if j > 0 else 0.0
    cases = [(F[j] - NEAR, True), (F[j] - FAR, False), (lo + FAR, False)]
    if j > 0:
        cases.append((lo + NEAR, True))
    for s, want in cases:
        r = m.tree_multi_one(zt, zq, parent, x, [u1, u2], f32(s), lam, T)
        assert r.accepted == 0 and r.tokens == [j]
        assert r.flagged == want, (s, lo, F[j])
    # first child accepted: the bonus draw from its own row
    F = cdf(bonus1)
    j = int(np.argmax(np.diff(np.concatenate([[0.0], F]))))
    for s, want in ((F[j] - NEAR, True), (F[j] - FAR, False)):
        r = m.tree_multi_one(zt, zq, parent, x, [f32(c["a1"] - 0.03), 0.5], f32(s), lam, T)
        assert r.accepted == 1 and r.bonus and r.tokens == [x[0], j]
        assert r.flagged == want


def check_zero_q_reading(m):
    rng = np.random.default_rng(8)
    V = 6
    zt = rng.normal(0.0, 1.0, (2, V))
    zq = zt[:1] + rng.normal(0.0, 1.0, (1, V))
    x = 2
    for lam in (0.0, 0.4):
        # q(x) = 0 < p~(x): accepted whatever the uniform; the limit q(x) -> 0+ agrees
        zq0 = zq.copy()
        zq0[0, x] = -np.inf
        r = m.chain_verify_one(zt, zq0, [x], [f32(1.0 - 2.0 ** -24)], 0.5, lam, 1.0)
        assert r.a[0] == 1.0 and r.accepted == 1
        zq_lim = zq.copy()
        zq_lim[0, x] = -600.0                          # q(x) ~ e^-600 > 0 in fp64
        assert m.chain_verify_one(zt, zq_lim, [x], [0.5], 0.5, lam, 1.0).a[0] == 1.0
        # q(x) = 0 = p~(x) (the target rules x out too): rejected, even at u = 0
        zt0 = zt.copy()
        zt0[0, x] = -np.inf
        r = m.chain_verify_one(zt0, zq0, [x], [0.0], 0.5, lam, 1.0)
        assert r.a[0] == 0.0 and r.accepted == 0
        # at lambda = 0 the limit p~(x) = 0 < q(x) -> 0+ gives the same answer (for
        # lambda > 0 that limit is lambda: 0/0 has no limit to follow, the reading decides)
        if lam == 0.0:
            assert m.chain_verify_one(zt0, zq_lim, [x], [0.0], 0.5, lam, 1.0).a[0] == 0.0
    # logit space: a -inf draft logit makes the mixed logit -inf, so p~(x) = 0
    zq0 = zq.copy()
    zq0[0, x] = -np.inf
    r = m.chain_verify_one(zt, zq0, [x], [0.0], 0.5, 0.4, 1.0, space="logit")
    assert r.a[0] == 0.0 and r.accepted == 0


def check_zero_residual_fallback(m):
    V = 5
    rng = np.random.default_rng(9)
    zt = rng.normal(0.0, 1.5, (2, V))
    zq = rng.normal(0.0, 1.5, (1, V))
    x = 1
    zq[0, x] = -np.inf
    q = sm(zq[0], 0.9)
    assert np.abs(q - sm(zt[0], 0.9)).max() > 0.05     # p_t differs from q
    # lambda = 1: p~ = q, a = [p~(x) > 0] = 0, residual max(0, q - q) = 0 -> draw from q
    r = m.chain_verify_one(zt, zq, [x], [0.5], 0.5, 1.0, 0.9)
    assert r.accepted == 0 and r.fallback
    law = token_law(lambda u: m.chain_verify_one(zt, zq, [x], [0.5], u, 1.0, 0.9).tokens[-1], V)
    np.testing.assert_allclose(law, q, atol=2.0 / GRID)
    # identical rows with q(x) = 0 = p~(x), lambda = 0.4: same fallback, law q = p~
    z = zq.copy()
    zt2 = np.concatenate([z, rng.normal(0.0, 1.0, (1, V))])
    r = m.chain_verify_one(zt2, z, [x], [0.5], 0.5, 0.4, 0.9)
    assert r.accepted == 0 and r.fallback
    law = token_law(lambda u: m.chain_verify_one(zt2, z, [x], [0.5], u, 0.4, 0.9).tokens[-1], V)
    np.testing.assert_allclose(law, q, atol=2.0 / GRID)
    # the same in logit space: the mixed logits of identical rows are the rows
    r = m.chain_verify_one(zt2, z, [x], [0.5], 0.5, 0.4, 0.9, space="logit")
    assert r.accepted == 0 and r.fallback
    law = token_law(lambda u: m.chain_verify_one(zt2, z, [x], [0.5], u, 0.4, 0.9,
                                                 space="logit").tokens[-1], V)
    np.testing.assert_allclose(law, q, atol=2.0 / GRID)
    # and over a wider row, where the expanded mixed logits (1 - lam) z + lam z
    # would round away from z on many elements
    zw = rng.normal(0.0, 3.0, (2, 50))
    zw[0, 7] = -np.inf
    for lam in (0.4, 0.3, 0.7):
        r = m.chain_verify_one(zw, zw[:1], [7], [0.5], 0.5, lam, 0.9, space="logit")
        assert r.accepted == 0 and r.fallback, lam
    # multi-branch, identical rows at the root, lambda = 0.4: same fallback
    res = m.tree_multi_one(zt2[:1].repeat(2, 0), z.repeat(2, 0), [0], [x], [0.5], 0.5, 0.4, 0.9)
    assert res.accepted == 0 and res.fallback
    # multi-branch: lambda = 1, the only child has q(x) = 0 -> draw from r = p~ = q
    zt3, zq3 = zt, np.concatenate([zq, zq])      # root and its one child
    res = m.tree_multi_one(zt3, zq3, [0], [x], [0.5], 0.5, 1.0, 0.9)
    assert res.accepted == 0 and res.fallback
    law = token_law(lambda u: m.tree_multi_one(zt3, zq3, [0], [x], [0.5], u, 1.0, 0.9).tokens[-1], V)
    np.testing.assert_allclose(law, q, atol=2.0 / GRID)


CHECKS = [check_chain_acceptance_band, check_chain_band_ignores_undrawn_positions,
          check_chain_band_needs_ratio_below_one, check_chain_sample_band, check_multi_bands,
          check_zero_q_reading, check_zero_residual_fallback]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_oracle(check):
    check(ov)


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one check fail
# ---------------------------------------------------------------------------

_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                    "verify.py")


def mutant(old, new, count=1):
    """A copy of the oracle module with `old` replaced by `new` in its source."""
    with open(_SRC, encoding="utf-8") as f:
        src = f.read()
    assert src.count(old) == count, (old, src.count(old))
    name = f"_oracle_mutant_{abs(hash((old, new)))}"
    spec = importlib.util.spec_from_loader(name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod                     # dataclasses look their module up
    try:
        exec(compile(src.replace(old, new), _SRC, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


MUTANTS = {
    "band 1e-3": ("FLAG_BAND = 1e-6", "FLAG_BAND = 1e-3", 1),
    "band 1e-9": ("FLAG_BAND = 1e-6", "FLAG_BAND = 1e-9", 1),
    "chain acceptance test inverted": ("abs(u - a[i]) < FLAG_BAND", "abs(u - a[i]) > FLAG_BAND", 1),
    "chain flags a == 1 too": ("if a[i] < 1.0 and abs(u - a[i])", "if abs(u - a[i])", 1),
    "chain flags every position": ("for i in range(min(n + 1, k)):", "for i in range(k):", 1),
    "chain ignores the rejected position": ("for i in range(min(n + 1, k)):",
                                            "for i in range(min(n, k)):", 1),
    "sample band one-sided": ("if (u_s - F_lo) < FLAG_BAND or (F_hi - u_s) < FLAG_BAND:\n        flagged = True\n\n    tokens = [int(t) for t in x[:n]]",
                              "if (F_hi - u_s) < FLAG_BAND:\n        flagged = True\n\n    tokens = [int(t) for t in x[:n]]", 1),
    "sample band inverted": ("(F_hi - u_s) < FLAG_BAND", "(F_hi - u_s) > FLAG_BAND", 2),
    "multi child test unflagged": ("if a < 1.0 and abs(uc - a) < FLAG_BAND:",
                                   "if a < 1.0 and abs(uc - a) < 0.0:", 1),
    "q = 0 always accepts": ("return 1.0 if p_mix_x > 0.0 else 0.0", "return 1.0", 1),
    "q = 0 always rejects": ("return 1.0 if p_mix_x > 0.0 else 0.0", "return 0.0", 1),
    "chain fallback from the target": ("w = p_mix_rows[n]", "w = softmax_T(zt[n], T)", 1),
    "chain fallback never taken": ("if not w.sum() > 0.0:", "if False:", 1),
    "excess in expanded form": ("return (1.0 - lam) * (p_t - q)", "return (1.0 - lam) * p_t + lam * q - q", 1),
    "multi fallback from the target": ("fallback = True\n                break",
                                       "fallback = True\n                r = softmax_T(zt[u], T)\n                break", 1),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new, count = MUTANTS[name]
    m = mutant(old, new, count)
    failed = []
    for check in CHECKS:
        try:
            check(m)
        except (AssertionError, ValueError, ZeroDivisionError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, f"planted mistake '{name}' passed every check"
