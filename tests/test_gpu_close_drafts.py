"""Parity where the draft is close to the target (high acceptance).

A good drafter's rows nearly equal the target's, so a rejection leaves a
residual max(0, p~ - q) of small total mass W, and the normalised residual of
the EAGLE page (section "1. 为什么无损") amplifies any error in forming it by
1 / W.  These cases draw the draft logits as target + N(0, sigma^2) with
sigma in {0.01, 0.03, 0.1} (in bf16 most logits then round to the target's
own value) and raise the acceptance uniforms into [1 - eps, 1), so that most
requests reject a draft and draw from that small residual.  The bar is the
usual one: counts and tokens bit-exact outside draws within 1e-6 of their
boundary (at most a couple flagged), a_i within 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
from sampling_spec_verify_amd import specverify as sv
from sampling_spec_verify_amd import synth
from tests.gpu_util import compare_chain, oracle_chain, path_lengths, run_chain, run_path
from tests.test_gpu_parity import _multi_case, report

pytestmark = pytest.mark.gpu

SIGMAS = [0.01, 0.03, 0.1]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    sv.lib()


def _residual_share(ref, lens):
    """Fraction of requests whose last token came from a residual draw."""
    return float(np.mean([ref.accepted[b] < lens[b] for b in range(len(lens))]))


def _run(x, eps, label, space="prob"):
    x.u_accept = synth.raise_uniforms(x.u_accept, eps)
    print(f"[close] {label}: B={x.B} K={x.K} V={x.V} {x.dtype} lam={x.lam} T={x.temperature} "
          f"eps={eps} {space}", flush=True)
    g = run_chain(x, space=space)
    assert int(g.status[0]) == 0, sv.decode_flags(int(g.status[0]))
    ref = oracle_chain(x, space=space)
    stats = compare_chain(x, g, ref)
    stats["residual_share"] = _residual_share(ref, x.lengths())
    report(label, stats)
    return stats


@pytest.mark.parametrize("sigma", SIGMAS)
def test_close_single_request_shape(sigma):
    """The single-request Llama-3-vocabulary shape (K = 8, V = 128256, bf16), 16 requests."""
    x = synth.make_chain(7100 + int(sigma * 1000), 16, 8, 128256, "bf16", sigma_t=3.0,
                         sigma_q=sigma, lam=0.0, temperature=1.0, name="close-c2")
    stats = _run(x, 0.05, f"close c2-shape sigma={sigma}")
    assert stats["residual_share"] >= 0.25


@pytest.mark.parametrize("sigma", SIGMAS)
def test_close_ragged_batch_shape(sigma):
    """The ragged 64-request batch (K_b in 1..8, V = 128256, bf16, T = 0.7)."""
    x = synth.make_chain(7200 + int(sigma * 1000), 64, 8, 128256, "bf16", sigma_t=3.0,
                         sigma_q=sigma, lam=0.0, temperature=0.7, ragged=True, k_min=1,
                         name="close-c4")
    stats = _run(x, 0.05, f"close c4-shape sigma={sigma}")
    assert stats["residual_share"] >= 0.25


@pytest.mark.parametrize("sigma,lam,space", [(0.01, 0.3, "prob"), (0.03, 0.3, "logit"),
                                             (0.1, 0.5, "logit")])
def test_close_mixture(sigma, lam, space):
    """RAPID's mixture with a close draft, both mixture spaces (V = 151936, bf16)."""
    x = synth.make_chain(7300 + int(sigma * 1000), 16, 8, 151936, "bf16", sigma_t=3.0,
                         sigma_q=sigma, lam=lam, temperature=1.0, name="close-c3")
    stats = _run(x, 0.02, f"close mixture sigma={sigma} lam={lam} {space}", space=space)
    assert stats["residual_share"] >= 0.1


@pytest.mark.parametrize("sigma", [0.01, 0.001])
def test_close_fp32(sigma):
    """fp32 logits: no bf16 ties, every element's logit moves a little."""
    x = synth.make_chain(7400 + int(sigma * 10000), 24, 6, 50000, "fp32", sigma_t=3.0,
                         sigma_q=sigma, lam=0.0, temperature=0.9, name="close-fp32")
    stats = _run(x, sigma, f"close fp32 sigma={sigma}")
    assert stats["residual_share"] >= 0.25


def test_identical_rows_rejecting_an_undrawable_draft():
    """p_t == q with drafted tokens of probability 0: the residual is zero
    everywhere, so the call takes the fallback to p~ (= q) in both mixture
    spaces, as the oracle's reading does."""
    x = synth.make_chain(7500, 6, 3, 5000, "bf16", lam=0.4)
    x.draft = np.ascontiguousarray(x.target[:, :3, :])
    ninf = synth.f32_to_bf16_bits(np.array([-np.inf], dtype=np.float32))[0]
    for b in range(x.B):
        x.target[b, 0, x.tokens[b, 0]] = ninf
        x.draft[b, 0, x.tokens[b, 0]] = ninf
    for space in ("prob", "logit"):
        g = run_chain(x, space=space)
        assert np.all(g.accepted == 0)
        ref = oracle_chain(x, space=space)
        assert all(d.fallback for d in ref.details)
        report(f"identical rows, q(x) = 0, {space}",
               compare_chain(x, g, ref))


@pytest.mark.parametrize("sigma", [0.01, 0.1])
def test_close_tree_path_and_multi(sigma):
    """Draft trees with a close draft: the seeded-path chain and the
    multi-branch walk (whose first residual at a node is formed the same way)."""
    x = synth.make_tree(7600 + int(sigma * 1000), 8, 26, 128256, "bf16", sigma_q=sigma)
    x.u_accept = synth.raise_uniforms(x.u_accept, 0.05)
    x.u_node = synth.raise_uniforms(x.u_node, 0.05)
    gp = run_path(x)
    assert int(gp.status[0]) == 0
    rp = oracle.tree_path(x.widened(x.target), x.widened(x.draft), x.node_token, x.path,
                          x.u_accept, x.u_sample, x.lam, x.temperature)
    report(f"close path sigma={sigma}", compare_chain(x, gp, rp, lengths=path_lengths(x)))
    gm, stats = _multi_case(x, label=f"close multi sigma={sigma}")
    assert int(gm.status[0]) == 0
