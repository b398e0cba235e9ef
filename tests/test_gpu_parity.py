"""Parity of the HIP path (through the C ABI) with the fp64 oracle on MI355X.

Bar: accepted counts and emitted tokens bit-exact for every request whose
draws all lie outside the 1e-6 boundary band (flagged requests are counted and
printed, not hidden); acceptance probabilities within 1e-5 absolute for every
drafted position; greedy trees bit-exact.
"""
import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle
from sampling_spec_verify_amd import specverify as sv
from sampling_spec_verify_amd import synth
from tests.gpu_util import (ACCEPT_PROB_TOL, chain_call, compare_chain, dev, dev_logits,
                            flag_limit, oracle_chain, path_lengths,
                            run_chain, run_greedy, run_path, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    sv.lib()


def report(name, stats):
    print(f"[parity] {name}: {stats}", flush=True)


# ---------------------------------------------------------------------------
# the five named workloads at full size
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3", "c4"])
def test_chain_workload(cfg):
    print(f"[parity] generating {cfg}", flush=True)
    x = synth.config(cfg)
    g = run_chain(x)
    assert int(g.status[0]) == 0, sv.decode_flags(int(g.status[0]))
    stats = compare_chain(x, g, oracle_chain(x))
    report(cfg, stats)
    if x.B == 1:                     # a single request is checked outright, never excused
        assert stats["flagged"] == 0


def test_tree_workload_greedy():
    x = synth.config("c5")
    g = run_greedy(x)
    assert int(g.status[0]) == 0
    acc, out, nodes = oracle.tree_greedy(x.widened(x.target), x.parent, x.node_token, x.Dmax)
    np.testing.assert_array_equal(g.accepted, acc)
    np.testing.assert_array_equal(g.out_tokens, out)
    np.testing.assert_array_equal(g.accepted_nodes, nodes)
    report("c5 greedy", {"accepted": acc.tolist()})


def test_tree_workload_path():
    x = synth.config("c5")
    g = run_path(x)
    assert int(g.status[0]) == 0
    ref = oracle.tree_path(x.widened(x.target), x.widened(x.draft), x.node_token, x.path,
                           x.u_accept, x.u_sample, x.lam, x.temperature)
    stats = compare_chain(x, g, ref, lengths=path_lengths(x))
    report("c5 path", stats)


@pytest.mark.parametrize("seed_offset", [1, 2, 3])
def test_c2_more_seeds(seed_offset):
    x = synth.config("c2", seed_offset)
    stats = compare_chain(x, run_chain(x), oracle_chain(x))
    report(f"c2/{seed_offset}", stats)
    assert stats["flagged"] == 0


# ---------------------------------------------------------------------------
# smaller shapes: several tiles, ragged tails, padded rows, both dtypes
# ---------------------------------------------------------------------------

SMALL = [
    # seed, B, K, V, dtype, lam, T, ragged, ld
    (1, 3, 4, 1000, "fp32", 0.0, 1.0, False, None),
    (2, 5, 3, 8200, "bf16", 0.3, 0.7, True, None),
    (3, 2, 8, 33000, "bf16", 0.0, 1.3, False, None),
    (4, 4, 2, 4097, "fp32", 0.5, 1.0, True, 4100),
    (5, 3, 5, 1001, "bf16", 0.1, 0.9, True, 1008),
    (6, 7, 1, 7, "fp32", 0.0, 1.0, False, 8),
    (7, 2, 6, 1, "bf16", 0.2, 1.0, False, 8),
    (8, 6, 0, 5000, "bf16", 0.0, 0.8, False, None),
    (9, 2, 64, 300, "fp32", 0.0, 1.0, False, None),
    (10, 9, 8, 20000, "fp32", 0.9, 2.0, True, None),
    (11, 40, 4, 2048, "bf16", 0.0, 1.0, True, None),
    # ragged batches on either side of the packed job order's 256-request limit
    (12, 256, 3, 1500, "fp32", 0.2, 0.8, True, None),
    (13, 257, 3, 2000, "bf16", 0.0, 1.0, True, None),
    (14, 300, 2, 1200, "bf16", 0.6, 1.1, True, None),
    # a large batch: thousands of blocks in every launch, the unpacked job order
    (17, 4096, 4, 1000, "fp32", 0.2, 0.9, True, None),
    # the largest vocabularies the validator accepts (bf16 2^21, fp32 2^20): LDS
    # staging is off, and the locate holds 16 piece masses per thread
    (15, 2, 3, 1 << 21, "bf16", 0.0, 1.0, False, None),
    (16, 2, 2, 1 << 20, "fp32", 0.3, 0.9, False, None),
]


@pytest.mark.parametrize("seed,B,K,V,dtype,lam,T,ragged,ld", SMALL)
def test_chain_small(seed, B, K, V, dtype, lam, T, ragged, ld):
    x = synth.make_chain(100 + seed, B, K, V, dtype, sigma_t=2.0, sigma_q=(0.3, 2.0),
                         zipf=V > 16, lam=lam, temperature=T, ragged=ragged, k_min=0)
    g = run_chain(x, ld)
    assert int(g.status[0]) == 0, sv.decode_flags(int(g.status[0]))
    report(f"small{seed}", compare_chain(x, g, oracle_chain(x)))


def test_identical_rows_accept_every_draft():
    x = synth.make_chain(201, 6, 5, 3000, "bf16", lam=0.4)
    x.draft = np.ascontiguousarray(x.target[:, :5, :])
    g = run_chain(x)
    assert np.all(g.accepted == 5)
    assert np.all(g.accept_prob == 1.0)
    report("p==q", compare_chain(x, g, oracle_chain(x)))


def test_lambda_one_accepts_every_draft():
    x = synth.make_chain(202, 4, 6, 2000, "fp32", lam=1.0, sigma_q=3.0)
    g = run_chain(x)
    assert np.all(g.accepted == 6)
    compare_chain(x, g, oracle_chain(x))


def test_masked_vocabulary():
    x = synth.make_chain(203, 4, 4, 9000, "fp32", sigma_q=1.0, temperature=0.8)
    x.target[:, :, 5000:] = -np.inf             # target rules out the upper vocabulary
    x.draft[:, :, 7000:] = -np.inf
    x.tokens = np.minimum(x.tokens, 6999)
    g = run_chain(x)
    assert int(g.status[0]) == 0
    report("masked", compare_chain(x, g, oracle_chain(x)))
    assert np.all(g.out_tokens[g.out_tokens >= 0] < 7000)


def test_stage_calls_equal_full_call():
    x = synth.make_chain(204, 5, 4, 12000, "bf16", ragged=True, lam=0.2)
    call = chain_call(x)
    full = to_host(call.run())
    call.row_stats()
    split = to_host(call.accept_resample())
    for a, b in zip(full, split):
        np.testing.assert_array_equal(a, b)


def test_resample_stage_repeats_on_the_same_statistics():
    """One row-statistics launch, then the accept / resample launch twice with
    different uniforms written in place: each run matches the oracle for its
    own uniforms (the hand-over counters of the draw reset themselves)."""
    x = synth.make_chain(206, 7, 4, 30000, "bf16", ragged=True, lam=0.2, sigma_q=(0.3, 2.0))
    call = chain_call(x)
    call.row_stats()
    rng = np.random.default_rng(207)
    for rep in range(3):
        if rep:
            x.u_accept = rng.random(x.u_accept.shape, dtype=np.float32)
            x.u_sample = rng.random(x.u_sample.shape, dtype=np.float32)
            call.inputs[4].copy_(torch.from_numpy(x.u_accept).to(call.inputs[4].device))
            call.inputs[5].copy_(torch.from_numpy(x.u_sample).to(call.inputs[5].device))
        g = to_host(call.accept_resample())
        report(f"repeat{rep}", compare_chain(x, g, oracle_chain(x)))


def test_bitwise_deterministic():
    x = synth.make_chain(205, 16, 8, 50000, "bf16", ragged=True, lam=0.3)
    a = run_chain(x)
    b = run_chain(x)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


# ---------------------------------------------------------------------------
# data errors reported in the status word
# ---------------------------------------------------------------------------


def test_status_bad_token_and_length():
    x = synth.make_chain(206, 3, 4, 1000, "fp32")
    x.tokens[1, 2] = 1000 + 5
    x.draft_len = np.array([4, 4, 9], dtype=np.int32)
    g = run_chain(x)
    flags = sv.decode_flags(int(g.status[0]))
    assert "BAD_TOKEN" in flags and "BAD_LENGTH" in flags
    assert g.accepted[1] <= 2 and g.accept_prob[1, 2] == 0.0
    # request 2 is clamped to K = 4 and otherwise normal
    x2 = synth.make_chain(206, 3, 4, 1000, "fp32")
    ref = oracle_chain(x2, requests=[2])
    if not ref.flagged[2]:
        assert g.accepted[2] == ref.accepted[2]
        np.testing.assert_array_equal(g.out_tokens[2], ref.out_tokens[2])


def test_status_bad_row():
    x = synth.make_chain(207, 2, 3, 1000, "fp32")
    x.target[0, 1, 10] = np.nan
    g = run_chain(x)
    assert "BAD_ROW" in sv.decode_flags(int(g.status[0]))
    assert g.accepted[0] <= 1
    ref = oracle_chain(x, requests=[1])
    compare_chain(x, g, ref, requests=[1])


# ---------------------------------------------------------------------------
# greedy and path tree verification on small random trees
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("seed,B,N,V,dtype,ints", [
    (1, 6, 12, 50, "fp32", True), (2, 4, 30, 20000, "fp32", True), (3, 5, 20, 9000, "bf16", False),
    (4, 3, 1, 4, "fp32", True), (5, 2, 200, 100, "bf16", True), (6, 8, 0, 500, "fp32", False),
    (7, 2, 1024, 300, "bf16", False),
    (8, 2048, 12, 500, "bf16", False),
])
def test_greedy_random_trees(seed, B, N, V, dtype, ints):
    x = synth.make_random_tree(300 + seed, B, N, V, dtype, int_logits=ints)
    g = run_greedy(x)
    assert int(g.status[0]) == 0
    acc, out, nodes = oracle.tree_greedy(x.widened(x.target), x.parent, x.node_token, x.Dmax)
    np.testing.assert_array_equal(g.accepted, acc)
    np.testing.assert_array_equal(g.out_tokens, out)
    np.testing.assert_array_equal(g.accepted_nodes, nodes)


def test_greedy_depth_cut_and_bad_parent():
    x = synth.make_random_tree(311, 2, 10, 64, "fp32", int_logits=True, sharp=1e-4)
    x.parent[0] = np.arange(10)                 # a chain: accepted as deep as tokens match
    g = run_greedy(x, Dmax=2)
    acc, out, nodes = oracle.tree_greedy(x.widened(x.target), x.parent, x.node_token, 12)
    for b in range(2):
        keep = min(acc[b], 2)
        assert g.accepted[b] == keep
        np.testing.assert_array_equal(g.accepted_nodes[b, :keep], nodes[b, :keep])
    x.parent[1, 3] = 7                          # parent not below the node
    g = run_greedy(x)
    assert "BAD_TREE" in sv.decode_flags(int(g.status[0]))


def test_greedy_special_values():
    """NaN rows are reported, never argmax'd; -inf rows, signed zeros and +inf
    in the partial last vector follow the oracle's first-maximum rule."""
    x = synth.make_random_tree(321, 5, 6, 3001, "bf16", int_logits=True)
    t = x.target                                 # bf16 bit patterns
    t[0, 2, 1500] = 0x7FC0                       # quiet NaN
    t[1, 0, :] = 0xFF80                          # a row of -inf: argmax is 0
    t[2, 0, :] = 0xFF80
    t[2, 0, 17] = 0x8000                         # -0 ties +0: the lower index wins
    t[2, 0, 2999] = 0x0000
    t[3, 0, 3000] = 0x7F80                       # +inf at the last element (partial vector)
    t[4, 1, 5] = 0x7F81                          # signalling-NaN bit pattern
    x.node_token[1:4, 0] = [0, 17, 3000]         # node 1 (a root child) matches row 0's argmax
    g = run_greedy(x)
    assert "BAD_ROW" in sv.decode_flags(int(g.status[0]))
    zt = x.widened(t)
    for b in (1, 2, 3):
        r = oracle.tree_greedy_one(zt[b], x.parent[b], x.node_token[b])
        assert r.accepted >= 1
        assert g.accepted[b] == r.accepted
        np.testing.assert_array_equal(g.out_tokens[b, :r.accepted + 1], r.tokens)
    assert oracle.tree_greedy_one(zt[1], x.parent[1], x.node_token[1]).argmax[0] == 0
    assert oracle.tree_greedy_one(zt[2], x.parent[2], x.node_token[2]).argmax[0] == 17
    assert oracle.tree_greedy_one(zt[3], x.parent[3], x.node_token[3]).argmax[0] == 3000
    for b in (0, 4):                             # the oracle refuses these requests
        # (widening the signalling-NaN pattern raises numpy's invalid-cast flag)
        with pytest.raises(oracle.InvalidRow), np.errstate(invalid="ignore"):
            oracle.tree_greedy_one(zt[b], x.parent[b], x.node_token[b])


def test_greedy_split_calls_equal_full_call():
    x = synth.make_random_tree(322, 4, 20, 20000, "bf16", int_logits=True)
    call = sv.TreeGreedyCall(dev_logits(x.target, x.dtype), dev(x.parent), dev(x.node_token), x.Dmax)
    full = to_host(call.run())
    call.row_argmax()
    split = to_host(call.walk())
    for a, b in zip(full, split):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("seed,B,N,V,dtype,lam,T", [
    (1, 6, 12, 3000, "fp32", 0.0, 1.0), (2, 4, 40, 20000, "bf16", 0.3, 0.8),
    (3, 3, 5, 17, "fp32", 0.5, 1.2),
    (4, 2, 1024, 300, "fp32", 0.2, 1.0),        # the most nodes a tree may have: one per resolve thread
])
def test_path_random_trees(seed, B, N, V, dtype, lam, T):
    x = synth.make_random_tree(400 + seed, B, N, V, dtype, sharp=1.0, lam=lam, temperature=T)
    # path tokens must be draws of the draft at each path node's parent row for
    # the law to hold; parity holds for any tokens
    g = run_path(x)
    assert int(g.status[0]) == 0
    ref = oracle.tree_path(x.widened(x.target), x.widened(x.draft), x.node_token, x.path,
                           x.u_accept, x.u_sample, x.lam, x.temperature)
    report(f"path{seed}", compare_chain(x, g, ref, lengths=path_lengths(x)))


# ---------------------------------------------------------------------------
# the output law on the GPU: 10^6 requests at V = 6
# ---------------------------------------------------------------------------


def test_gpu_output_law_monte_carlo():
    V, K, lam, T, n = 6, 2, 0.3, 0.8, 1_000_000
    rng = np.random.default_rng(77)
    zt = rng.normal(0.0, 1.5, (K + 1, V))
    zq = zt[:K] + rng.normal(0.0, 1.0, (K, V))
    zt[1, 2] = -np.inf
    zt32, zq32 = zt.astype(np.float32), zq.astype(np.float32)
    q = [scipy.special.softmax(zq32[i].astype(np.float64) / np.float32(T)) for i in range(K)]
    p = [scipy.special.softmax(zt32[i].astype(np.float64) / np.float32(T)) for i in range(K + 1)]
    tokens = np.stack([rng.choice(V, size=n, p=q[i]) for i in range(K)], axis=1).astype(np.int32)
    x = synth.ChainInputs("mc", "fp32", np.broadcast_to(zt32, (n, K + 1, V)).copy(),
                          np.broadcast_to(zq32, (n, K, V)).copy(), tokens, None,
                          rng.random((n, K), dtype=np.float32), rng.random(n, dtype=np.float32),
                          lam, T)
    g = run_chain(x, ld=8)
    lam32 = float(np.float32(lam))
    pm = [(1 - lam32) * p[j] + lam32 * q[j] for j in range(K)]
    alpha = [np.minimum(pm[j], q[j]).sum() for j in range(K)]

    def chisq(obs, prob):
        keep = prob > 0
        assert np.all(obs[~keep] == 0)
        exp = prob[keep] / prob[keep].sum() * obs[keep].sum()
        return scipy.stats.chisquare(obs[keep], exp).pvalue

    first = np.bincount(g.out_tokens[:, 0], minlength=V)
    sel = g.accepted >= 1
    second = np.bincount(g.out_tokens[sel, 1], minlength=V)
    bonus = np.bincount(g.out_tokens[g.accepted == K, K], minlength=V)
    nh = np.bincount(g.accepted, minlength=K + 1)
    law_n = np.array([1 - alpha[0], alpha[0] * (1 - alpha[1]), alpha[0] * alpha[1]])
    pv = [chisq(first, pm[0]), chisq(second, pm[1]), chisq(bonus, p[K]), chisq(nh, law_n)]
    print(f"[parity] MC p-values {pv}", flush=True)
    assert min(pv) > 0.01


# ---------------------------------------------------------------------------
# tree-attention mask (bit-exact against the oracle)
# ---------------------------------------------------------------------------


def _mask_case(parent: np.ndarray, words=None):
    B, N = parent.shape
    W = (N + 32) // 32 if words is None else words
    g = sv.tree_attention_mask(dev(parent.astype(np.int32)), N, W)
    torch.cuda.synchronize()
    mask = g.mask.cpu().numpy().view(np.uint32)
    depth = g.depth.cpu().numpy()
    ref_mask, ref_depth, bad = oracle.tree_attention_mask(parent, W)
    np.testing.assert_array_equal(mask, ref_mask)
    np.testing.assert_array_equal(depth, ref_depth)
    return int(g.status[0].item()), bad


def test_mask_tree_workload():
    x = synth.config("c5")
    st, bad = _mask_case(x.parent)
    assert st == 0 and not bad.any()


@pytest.mark.parametrize("seed,B,N,words", [
    (1, 5, 0, None), (2, 3, 1, None), (3, 7, 31, None), (4, 4, 32, None), (5, 6, 33, 3),
    (6, 2, 200, None), (7, 3, 1024, None), (8, 9, 70, 40),
])
def test_mask_random_trees(seed, B, N, words):
    rng = np.random.default_rng(500 + seed)
    parent = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        shape = b % 3
        for i in range(1, N + 1):
            if shape == 0:
                parent[b, i - 1] = i - 1                    # chain: causal mask, deepest walks
            elif shape == 1:
                parent[b, i - 1] = int(rng.integers(0, i))  # uniform random recursive tree
            else:
                parent[b, i - 1] = int(rng.integers(max(0, i - 3), i))  # deep, narrow
    st, bad = _mask_case(parent, words)
    assert st == 0 and not bad.any()


def test_mask_bad_parent_is_reported_and_read_as_root_child():
    parent = np.array([[0, 1, 7, 2, -3, 4], [0, 0, 1, 1, 2, 2]], dtype=np.int32)
    st, bad = _mask_case(parent)
    assert bad.tolist() == [True, False]
    assert "BAD_TREE" in sv.decode_flags(st)


# ---------------------------------------------------------------------------
# logit-space mixture (the RAPID pseudocode's form)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("cfg,lam", [("c3", None), ("c4", 0.3), ("c2", 0.5)])
def test_logit_mixture_workload(cfg, lam):
    x = synth.config(cfg)
    if lam is not None:
        x.lam = lam
    g = run_chain(x, space="logit")
    assert int(g.status[0]) == 0, sv.decode_flags(int(g.status[0]))
    stats = compare_chain(x, g, oracle_chain(x, space="logit"))
    report(f"{cfg} logit", stats)


LOGIT_SMALL = [
    # seed, B, K, V, dtype, lam, T, ragged, ld
    (21, 3, 4, 1000, "fp32", 0.3, 1.0, False, None),
    (22, 5, 3, 8200, "bf16", 0.7, 0.7, True, None),
    (23, 2, 8, 33000, "bf16", 0.05, 1.3, False, None),
    (24, 4, 2, 4097, "fp32", 0.5, 1.0, True, 4100),
    (25, 7, 1, 7, "fp32", 0.4, 1.0, False, 8),
    (26, 6, 0, 5000, "bf16", 0.2, 0.8, False, None),
    (27, 2, 64, 300, "fp32", 0.6, 1.0, False, None),
    (28, 40, 4, 2048, "bf16", 0.95, 1.0, True, None),
    (29, 300, 3, 1500, "bf16", 0.3, 1.0, True, None),
    (30, 2, 2, 1 << 21, "bf16", 0.5, 1.0, False, None),
]


@pytest.mark.parametrize("seed,B,K,V,dtype,lam,T,ragged,ld", LOGIT_SMALL)
def test_logit_mixture_small(seed, B, K, V, dtype, lam, T, ragged, ld):
    x = synth.make_chain(100 + seed, B, K, V, dtype, sigma_t=2.0, sigma_q=(0.3, 2.0),
                         zipf=V > 16, lam=lam, temperature=T, ragged=ragged, k_min=0)
    g = run_chain(x, ld, space="logit")
    assert int(g.status[0]) == 0, sv.decode_flags(int(g.status[0]))
    report(f"logit{seed}", compare_chain(x, g, oracle_chain(x, space="logit")))


@pytest.mark.parametrize("lam", [0.0, 1.0])
def test_logit_mixture_at_the_ends_equals_probability_space(lam):
    x = synth.make_chain(231, 5, 4, 6000, "bf16", lam=lam, sigma_q=1.5, ragged=True)
    a = run_chain(x, space="logit")
    b = run_chain(x)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    compare_chain(x, a, oracle_chain(x, space="logit"))


def test_logit_mixture_identical_rows_and_stage_calls():
    x = synth.make_chain(232, 4, 5, 3000, "fp32", lam=0.45)
    x.draft = np.ascontiguousarray(x.target[:, :5, :])
    g = run_chain(x, space="logit")
    assert np.all(g.accepted == 5)
    x = synth.make_chain(233, 5, 4, 12000, "bf16", ragged=True, lam=0.35)
    call = chain_call(x, space="logit")
    full = to_host(call.run())
    call.row_stats()
    split = to_host(call.accept_resample())
    for u, v in zip(full, split):
        np.testing.assert_array_equal(u, v)
    compare_chain(x, full, oracle_chain(x, space="logit"))


def test_logit_mixture_path_mode():
    x = synth.make_random_tree(433, 5, 30, 9000, "bf16", sharp=1.0, lam=0.4, temperature=0.9)
    g = run_path(x, space="logit")
    assert int(g.status[0]) == 0
    ref = oracle.tree_path(x.widened(x.target), x.widened(x.draft), x.node_token, x.path,
                           x.u_accept, x.u_sample, x.lam, x.temperature, space="logit")
    report("path logit", compare_chain(x, g, ref, lengths=path_lengths(x)))


@pytest.mark.parametrize("dtype,V,space", [("fp32", 3000, "prob"), ("bf16", 3001, "prob"),
                                           ("bf16", 3001, "logit"), ("fp32", 70001, "logit")])
def test_lambda_one_with_unreachable_draft_samples_the_draft(dtype, V, space):
    """lambda = 1 and q(x) = 0: the draft is rejected and, the residual
    max(0, p~ - q) being zero, the token is drawn from p~ = q by the
    fallback scan (both mixture spaces, a partial last vector, and a row of
    several pages)."""
    x = synth.make_chain(234, 6, 3, V, dtype, lam=1.0, sigma_q=2.0)
    neg_inf = np.float32(-np.inf)
    for b in range(x.B):                             # position 1's draft cannot produce x
        if dtype == "bf16":
            x.draft[b, 1, x.tokens[b, 1]] = 0xFF80
        else:
            x.draft[b, 1, x.tokens[b, 1]] = neg_inf
    g = run_chain(x, space=space)
    flags = sv.decode_flags(int(g.status[0]))
    assert "ZERO_Q" in flags and "FALLBACK" in flags
    assert np.all(g.accepted == 1)
    report(f"lambda=1 q(x)=0 {dtype} {space}", compare_chain(x, g, oracle_chain(x, space=space)))


# ---------------------------------------------------------------------------
# acceptance-rate telemetry: alpha_i = sum_v min(p~, q), within 1e-5
# ---------------------------------------------------------------------------

ALPHA_TOL = 1e-5


def _alpha_case(x, space="prob", ld=None):
    alpha, status = sv.chain_acceptance_rate(dev_logits(x.target, x.dtype, ld),
                                             dev_logits(x.draft, x.dtype, ld), x.lam,
                                             x.temperature, dev(x.draft_len), space=space)
    torch.cuda.synchronize()
    g = alpha.cpu().numpy().astype(np.float64)
    ref = oracle_chain(x, space=space)
    lens = x.lengths()
    err = 0.0
    for b in range(x.B):
        k = int(lens[b])
        if k:
            err = max(err, float(np.abs(g[b, :k] - ref.details[b].alpha).max()))
        assert np.all(g[b, k:] == 0.0)
    assert err <= ALPHA_TOL, err
    return int(status[0].item()), err


@pytest.mark.parametrize("cfg,space", [("c3", "prob"), ("c3", "logit"), ("c4", "prob"),
                                       ("c1", "prob"), ("c2", "prob")])
def test_acceptance_rate_workload(cfg, space):
    x = synth.config(cfg)
    st, err = _alpha_case(x, space)
    assert st == 0
    report(f"alpha {cfg} {space}", {"max_abs_err": err})


@pytest.mark.parametrize("seed,B,K,V,dtype,lam,T,ragged,ld,space", [
    (41, 3, 4, 1000, "fp32", 0.0, 1.0, False, None, "prob"),
    (42, 5, 3, 8200, "bf16", 0.3, 0.7, True, None, "prob"),
    (43, 4, 2, 4097, "fp32", 0.5, 1.0, True, 4100, "logit"),
    (44, 7, 1, 7, "fp32", 0.4, 1.0, False, 8, "logit"),
    (45, 2, 64, 300, "fp32", 0.6, 1.0, False, None, "prob"),
    (46, 6, 5, 33000, "bf16", 0.8, 1.5, True, None, "logit"),
    (47, 300, 3, 1500, "bf16", 0.0, 1.0, True, None, "prob"),
    (48, 2, 3, 1 << 21, "bf16", 0.3, 1.0, True, None, "logit"),
])
def test_acceptance_rate_small(seed, B, K, V, dtype, lam, T, ragged, ld, space):
    x = synth.make_chain(100 + seed, B, K, V, dtype, sigma_t=2.0, sigma_q=(0.3, 2.0),
                         zipf=V > 16, lam=lam, temperature=T, ragged=ragged, k_min=0)
    st, err = _alpha_case(x, space, ld)
    assert st == 0
    report(f"alpha small{seed}", {"max_abs_err": err})


@pytest.mark.parametrize("lam,space", [(0.0, "prob"), (0.3, "prob"), (0.4, "logit")])
def test_acceptance_rate_bad_row_is_nan_and_flagged(lam, space):
    """A NaN in a drafted target or draft row makes that position's alpha NaN and
    sets SV_DATA_BAD_ROW; the other positions keep the oracle's values (each of
    the kernel's three forms of the sum: two probabilities, and the single
    exponential of the logit space and of lambda = 0)."""
    x = synth.make_chain(261, 3, 3, 3000, "fp32", lam=lam)
    x.target[0, 1, 17] = np.nan
    x.draft[2, 0, 2999] = np.nan
    alpha, status = sv.chain_acceptance_rate(dev_logits(x.target, x.dtype),
                                             dev_logits(x.draft, x.dtype), x.lam, x.temperature,
                                             space=space)
    torch.cuda.synchronize()
    g = alpha.cpu().numpy()
    assert int(status[0].item()) & 0x02
    assert np.isnan(g[0, 1]) and np.isnan(g[2, 0])
    good = np.isfinite(g)
    assert good.sum() == g.size - 2
    y = synth.make_chain(261, 3, 3, 3000, "fp32", lam=lam)
    ref = oracle_chain(y, space=space)
    for b in range(3):
        for i in range(3):
            if good[b, i]:
                assert abs(g[b, i] - ref.details[b].alpha[i]) <= ALPHA_TOL


def test_acceptance_rate_identical_rows_and_lambda_one_are_one():
    x = synth.make_chain(247, 4, 3, 5000, "bf16", lam=0.3)
    x.draft = np.ascontiguousarray(x.target[:, :3, :])
    _alpha_case(x)
    alpha, _ = sv.chain_acceptance_rate(dev_logits(x.target, x.dtype), dev_logits(x.draft, x.dtype),
                                        x.lam, x.temperature)
    np.testing.assert_allclose(alpha.cpu().numpy(), 1.0, atol=ALPHA_TOL)
    x = synth.make_chain(248, 3, 4, 2000, "fp32", lam=1.0, sigma_q=2.0)
    alpha, _ = sv.chain_acceptance_rate(dev_logits(x.target, x.dtype), dev_logits(x.draft, x.dtype),
                                        x.lam, x.temperature)
    np.testing.assert_allclose(alpha.cpu().numpy(), 1.0, atol=ALPHA_TOL)


# ---------------------------------------------------------------------------
# multi-branch stochastic tree verification (sibling retries)
# ---------------------------------------------------------------------------


def _multi_case(x, Dmax=None, space="prob", label="multi", blocks_per_tree=0):
    Dmax = x.Dmax if Dmax is None else Dmax
    g = sv.tree_verify_multi(dev_logits(x.target, x.dtype), dev_logits(x.draft, x.dtype),
                             dev(x.parent), dev(x.node_token), dev(x.u_node), dev(x.u_sample), Dmax,
                             x.lam, x.temperature, space, blocks_per_tree=blocks_per_tree)
    return compare_multi(x, to_host(g), Dmax, space, label)


def compare_multi(x, g, Dmax, space="prob", label="multi"):
    """Host outputs g of a multi-branch call against the oracle: bitwise equal
    outside requests whose draws the oracle flags, acceptance values within
    ACCEPT_PROB_TOL; the flagged count bounded."""
    acc, out, nodes, ap, flag, det = oracle.tree_multi(
        x.widened(x.target), x.widened(x.draft), x.parent, x.node_token, x.u_node, x.u_sample,
        x.lam, x.temperature, Dmax, space)
    stats = {"requests": x.B, "flagged": 0, "flagged_mismatch": 0, "max_a_err": 0.0,
             "tested": 0}
    for b in range(x.B):
        tested = ap[b] >= 0.0
        stats["tested"] += int(tested.sum())
        same = (g.accepted[b] == acc[b] and np.array_equal(g.out_tokens[b], out[b])
                and np.array_equal(g.accepted_nodes[b], nodes[b]))
        if flag[b]:
            stats["flagged"] += 1
            stats["flagged_mismatch"] += int(not same)
            continue
        assert same, (f"request {b}: gpu {g.accepted[b]} {g.out_tokens[b].tolist()} "
                      f"oracle {acc[b]} {out[b].tolist()}")
        np.testing.assert_array_equal(g.accept_prob[b] >= 0.0, tested)
        if tested.any():
            err = float(np.abs(g.accept_prob[b][tested] - ap[b][tested]).max())
            stats["max_a_err"] = max(stats["max_a_err"], err)
            assert err <= ACCEPT_PROB_TOL, (b, err)
    report(label, stats)
    assert stats["flagged"] <= flag_limit(x.B), stats
    return g, stats


@pytest.mark.parametrize("lam,space", [(0.0, "prob"), (0.3, "prob"), (0.3, "logit")])
def test_multi_tree_workload(lam, space):
    x = synth.config("c5")
    x.lam = lam
    g, stats = _multi_case(x, space=space, label=f"c5 multi {space} {lam}")
    assert int(g.status[0]) == 0
    assert stats["flagged"] <= 2


@pytest.mark.parametrize("seed,B,N,V,dtype,lam,T,space,Dmax", [
    (1, 6, 12, 3000, "fp32", 0.0, 1.0, "prob", None),
    (2, 4, 40, 20000, "bf16", 0.3, 0.8, "prob", None),
    (3, 3, 5, 17, "fp32", 0.5, 1.2, "logit", None),
    (4, 5, 30, 9000, "bf16", 0.2, 1.0, "logit", 3),
    (5, 2, 200, 500, "fp32", 0.0, 1.5, "prob", None),
    (6, 4, 0, 700, "bf16", 0.0, 1.0, "prob", None),
    (7, 1, 1024, 256, "fp32", 0.3, 1.0, "prob", None),
])
def test_multi_random_trees(seed, B, N, V, dtype, lam, T, space, Dmax):
    # loose draft rows (sigma 2) so that rejections and sibling retries are common
    x = synth.make_random_tree(600 + seed, B, N, V, dtype, sharp=1.0, sigma_q=2.0, lam=lam,
                               temperature=T)
    g, _ = _multi_case(x, Dmax=Dmax, space=space, label=f"multi random {seed}")
    assert int(g.status[0]) == 0


def test_multi_barrier_slots_under_alternating_batches():
    """Two batches of trees alternate 60 times on one workspace.  The blocks of
    a tree exchange values through rotating slots that each call starts empty;
    a value read from the previous call or from an earlier barrier of the same
    call would change an output, and a slot never filled would raise
    SV_DATA_SYNC.  B = 3 puts a tree's blocks on different XCDs."""
    xs = [synth.make_random_tree(seed, 3, 30, 20000, "bf16", sharp=1.0, sigma_q=2.0, lam=lam,
                                 temperature=T) for seed, lam, T in ((631, 0.0, 1.0), (637, 0.3, 0.8))]
    B, N, V = 3, 30, 20000
    ws = torch.empty(int(sv.lib().sv_tree_multi_workspace_bytes(B, N, V)), dtype=torch.uint8,
                     device="cuda:0")
    refs = [oracle.tree_multi(x.widened(x.target), x.widened(x.draft), x.parent, x.node_token,
                              x.u_node, x.u_sample, x.lam, x.temperature, x.Dmax, "prob") for x in xs]
    args = [(dev_logits(x.target, x.dtype), dev_logits(x.draft, x.dtype), dev(x.parent),
             dev(x.node_token), dev(x.u_node), dev(x.u_sample), x.Dmax, x.lam, x.temperature, "prob")
            for x in xs]
    reps = 60
    hist = [[] for _ in xs]
    for _ in range(reps):
        for j in range(len(xs)):
            out = sv.tree_verify_multi(*args[j], workspace=ws)
            hist[j].append((out.status.clone(), out.accepted.clone(), out.out_tokens.clone()))
    torch.cuda.synchronize()
    for j, ref in enumerate(refs):
        acc, toks, flag = ref[0], ref[1], ref[4]
        for st, a, o in hist[j]:
            assert int(st[0]) & 0x80 == 0
            a, o = a.cpu().numpy(), o.cpu().numpy()
            for b in range(B):
                if not flag[b]:
                    assert a[b] == acc[b] and np.array_equal(o[b], toks[b])
    report("multi slots", {"calls": 2 * reps, "trees": B})


def test_multi_on_chain_shaped_trees_matches_path_mode():
    x = synth.make_random_tree(621, 5, 7, 4000, "fp32", sharp=1.0, sigma_q=1.5, lam=0.2)
    x.parent[:] = np.arange(7)
    x.path = np.tile(np.arange(1, 8, dtype=np.int32), (5, 1))
    x.u_accept = x.u_node.copy()                # the same uniform per node in both calls
    g, _ = _multi_case(x, Dmax=7)
    p = run_path(x)
    np.testing.assert_array_equal(g.accepted, p.accepted)
    np.testing.assert_array_equal(g.out_tokens, p.out_tokens)


def test_multi_bad_parent_and_token_are_reported():
    x = synth.make_random_tree(622, 3, 10, 500, "fp32", sharp=1.0, sigma_q=2.0)
    x.parent[0, 4] = 9                          # node 5's parent is not below it
    x.node_token[1, :] = 600                    # tokens outside [0, V)
    g = sv.tree_verify_multi(dev_logits(x.target, x.dtype), dev_logits(x.draft, x.dtype),
                             dev(x.parent), dev(x.node_token), dev(x.u_node), dev(x.u_sample),
                             x.Dmax)
    flags = sv.decode_flags(int(to_host(g).status[0]))
    assert "BAD_TREE" in flags and "BAD_TOKEN" in flags


@pytest.mark.parametrize("space", ["prob", "logit"])
def test_gpu_multi_output_law_monte_carlo(space):
    """2 x 10^5 trees (root with three children, each with one child) whose rows
    depend only on the token prefix and whose node tokens are independent
    draws from the parent's q: the first emitted token follows p~ of the
    root, the second p~ of its prefix, the bonus the target (chi-square
    p > 0.01)."""
    V, lam, T, n = 5, 0.3, 0.9, 200_000
    parent = np.array([0, 0, 0, 1, 2, 3], dtype=np.int32)
    rng = np.random.default_rng(78)
    table = {(): (rng.normal(0, 1.5, V), None)}
    for t1 in range(V):
        table[(t1,)] = (rng.normal(0, 1.5, V), None)
        for t2 in range(V):
            table[(t1, t2)] = (rng.normal(0, 1.5, V), None)
    for k in table:                                   # draft rows: target + noise
        zt = table[k][0].astype(np.float32)
        table[k] = (zt, (zt + rng.normal(0, 1.0, V)).astype(np.float32))
    T32, l32 = float(np.float32(T)), float(np.float32(lam))

    def q_of(k):
        return scipy.special.softmax(table[k][1].astype(np.float64) / T32)

    def pmix(k):
        zt, zq = (a.astype(np.float64) for a in table[k])
        if space == "prob":
            return (1 - l32) * scipy.special.softmax(zt / T32) + l32 * scipy.special.softmax(zq / T32)
        return scipy.special.softmax(((1 - l32) * zt + l32 * zq) / T32)

    tok1 = np.stack([rng.choice(V, size=n, p=q_of(())) for _ in range(3)], axis=1)
    tok2 = np.zeros_like(tok1)
    for j in range(3):
        for t in range(V):
            sel = tok1[:, j] == t
            tok2[sel, j] = rng.choice(V, size=int(sel.sum()), p=q_of((t,)))
    node_token = np.concatenate([tok1, tok2], axis=1).astype(np.int32)
    zt = np.zeros((n, 7, V), dtype=np.float32)
    zq = np.zeros((n, 7, V), dtype=np.float32)
    zt[:, 0], zq[:, 0] = table[()]
    for t1 in range(V):
        rows_t = np.stack([table[(t1,)][0]] + [table[(t1, t2)][0] for t2 in range(V)])
        rows_q = np.stack([table[(t1,)][1]] + [table[(t1, t2)][1] for t2 in range(V)])
        for j in range(3):
            sel = tok1[:, j] == t1
            zt[sel, 1 + j], zq[sel, 1 + j] = rows_t[0], rows_q[0]
            zt[sel, 4 + j] = rows_t[1 + tok2[sel, j]]
            zq[sel, 4 + j] = rows_q[1 + tok2[sel, j]]
    u_node = rng.random((n, 6), dtype=np.float32)
    u_s = rng.random(n, dtype=np.float32)
    g = to_host(sv.tree_verify_multi(dev_logits(zt, "fp32", 8), dev_logits(zq, "fp32", 8),
                                     dev(np.broadcast_to(parent, (n, 6)).copy()), dev(node_token),
                                     dev(u_node), dev(u_s), 2, lam, T, space))
    assert int(g.status[0]) == 0

    def chisq(obs, prob):
        keep = prob > 0
        assert np.all(obs[~keep] == 0)
        exp = prob[keep] / prob[keep].sum() * obs[keep].sum()
        return scipy.stats.chisquare(obs[keep], exp).pvalue

    pv = [chisq(np.bincount(g.out_tokens[:, 0], minlength=V), pmix(()))]
    for t1 in range(V):
        sel = (g.accepted >= 1) & (g.out_tokens[:, 0] == t1)
        if sel.sum() > 2000:
            pv.append(chisq(np.bincount(g.out_tokens[sel, 1], minlength=V), pmix((t1,))))
        for t2 in range(V):
            sel2 = (g.accepted == 2) & (g.out_tokens[:, 0] == t1) & (g.out_tokens[:, 1] == t2)
            if sel2.sum() > 2000:
                pbonus = scipy.special.softmax(table[(t1, t2)][0].astype(np.float64) / T32)
                pv.append(chisq(np.bincount(g.out_tokens[sel2, 2], minlength=V), pbonus))
    print(f"[parity] multi MC {space}: {len(pv)} laws, min p {min(pv):.4f}, "
          f"depths {np.bincount(g.accepted).tolist()}", flush=True)
    assert len(pv) >= 8
    assert min(pv) > 0.01 / len(pv)            # Bonferroni over the tested laws


# ---------------------------------------------------------------------------
# the hand-over of chunk records between the mass blocks of a request
# ---------------------------------------------------------------------------


def test_handover_between_mass_blocks_under_alternating_inputs():
    """Two batches alternate 300 times on one workspace.  Each request's four
    mass blocks land on different XCDs (B = 7 is not a multiple of 8), and a
    record read before its writer's store landed would carry the other batch's
    value, so any such read changes an output token."""
    B, K, V = 7, 4, 50000
    xs = [synth.make_chain(seed, B, K, V, "bf16", sigma_t=2.0, sigma_q=(0.3, 2.0), lam=lam,
                           temperature=T, ragged=True)
          for seed, lam, T in ((705, 0.0, 1.0), (709, 0.3, 0.8))]
    ws = torch.empty(sv.chain_workspace_bytes(B, K, V), dtype=torch.uint8, device="cuda:0")
    calls = [sv.ChainCall(dev_logits(x.target, x.dtype), dev_logits(x.draft, x.dtype), dev(x.tokens),
                          dev(x.u_accept), dev(x.u_sample), x.lam, x.temperature, dev(x.draft_len),
                          workspace=ws) for x in xs]
    refs = [oracle_chain(x) for x in xs]
    reps = 300
    hist = [torch.empty((reps, B, K + 1), dtype=torch.int32, device="cuda:0") for _ in xs]
    acc = [torch.empty((reps, B), dtype=torch.int32, device="cuda:0") for _ in xs]
    for i in range(reps):
        for j, c in enumerate(calls):
            out = c.run()
            hist[j][i].copy_(out.out_tokens)
            acc[j][i].copy_(out.accepted)
    torch.cuda.synchronize()
    for j, (x, ref) in enumerate(zip(xs, refs)):
        assert not ref.flagged.any()
        assert int(calls[j].out.status[0]) == 0
        h, a = hist[j].cpu().numpy(), acc[j].cpu().numpy()
        assert (a == ref.accepted[None, :]).all(), np.argwhere(a != ref.accepted[None, :])[:5]
        assert (h == ref.out_tokens[None]).all(), np.argwhere(h != ref.out_tokens[None])[:5]
    report("handover", {"calls": 2 * reps, "requests": B})
