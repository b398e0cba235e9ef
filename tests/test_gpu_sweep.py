"""A seeded sweep of random call shapes through every verify entry point, each
checked against the fp64 oracle to the same bar as the named cases.

Chain cases draw batch sizes on both sides of the packed job order's limit
(256 requests), vocabularies across vector and tile boundaries, both dtypes,
padded row strides, ragged and full batches, both mixture spaces, and lambda
and temperature across their ranges; each runs the verify call and the
acceptance-rate call.  Tree cases draw random recursive trees of several
sizes (with tied integer logits in some) and run greedy, path, multi-branch
and mask calls on each.  Every case prints its parameters before it runs."""
import numpy as np
import pytest
import torch

import oracle
from sampling_spec_verify_amd import specverify as sv
from sampling_spec_verify_amd import synth
from tests.gpu_util import compare_chain, oracle_chain, path_lengths, run_chain, run_greedy, run_path
from tests.test_gpu_parity import _alpha_case, _mask_case, _multi_case, report

pytestmark = pytest.mark.gpu

N_CHAIN = 40
N_TREE = 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    sv.lib()


def chain_params(i):
    rng = np.random.default_rng(9000 + i)
    B = int(rng.choice([1, 2, 5, 17, 64, 255, 256, 257, 300]))
    K = int(rng.integers(0, 11))
    V = int(rng.choice([1, 7, 8, 9, 511, 4095, 4096, 4097, 30011, 65536, 131075]))
    if B * (K + 1) * V > 40_000_000:     # keeps the oracle's share of the sweep to seconds
        V = 4097
    dtype = str(rng.choice(["bf16", "fp32"]))
    lam = float(rng.choice([0.0, 0.0, 0.2, 0.5, 0.9, 1.0]))
    T = float(rng.choice([0.3, 0.7, 1.0, 1.7]))
    ragged = bool(rng.integers(0, 2))
    per = 8 if dtype == "bf16" else 4
    ld = None if rng.integers(0, 3) else (-(-V // per) + int(rng.integers(1, 3))) * per
    space = str(rng.choice(["prob", "logit"]))
    return B, K, V, dtype, lam, T, ragged, ld, space


def tree_params(i):
    rng = np.random.default_rng(9500 + i)
    B = int(rng.choice([1, 3, 8, 33]))
    N = int(rng.choice([1, 2, 5, 26, 63, 200]))
    V = int(rng.choice([2, 9, 1000, 4097, 50000]))
    if B * (N + 1) * V > 20_000_000:
        V = 1000
    dtype = str(rng.choice(["bf16", "fp32"]))
    lam = float(rng.choice([0.0, 0.3, 0.8]))
    T = float(rng.choice([0.5, 1.0, 1.5]))
    space = str(rng.choice(["prob", "logit"]))
    ints = bool(rng.integers(0, 3) == 0)
    return B, N, V, dtype, lam, T, space, ints


@pytest.mark.parametrize("i", range(N_CHAIN))
def test_chain_sweep(i):
    B, K, V, dtype, lam, T, ragged, ld, space = chain_params(i)
    print(f"[sweep] chain {i}: B={B} K={K} V={V} {dtype} lam={lam} T={T} ragged={ragged} "
          f"ld={ld} {space}", flush=True)
    x = synth.make_chain(9100 + i, B, K, V, dtype, sigma_t=2.0, sigma_q=(0.3, 2.0),
                         zipf=V > 16, lam=lam, temperature=T, ragged=ragged, k_min=0)
    g = run_chain(x, ld, space)
    assert int(g.status[0]) == 0, sv.decode_flags(int(g.status[0]))
    report(f"sweep chain {i}", compare_chain(x, g, oracle_chain(x, space=space)))
    if K > 0:
        st, err = _alpha_case(x, space, ld)
        assert st == 0
        report(f"sweep alpha {i}", {"max_abs_err": err})


@pytest.mark.parametrize("i", range(N_TREE))
def test_tree_sweep(i):
    B, N, V, dtype, lam, T, space, ints = tree_params(i)
    print(f"[sweep] tree {i}: B={B} N={N} V={V} {dtype} lam={lam} T={T} {space} "
          f"int_logits={ints}", flush=True)
    x = synth.make_random_tree(9600 + i, B, N, V, dtype, int_logits=ints, sharp=1.0,
                               sigma_q=2.0, lam=lam, temperature=T)
    g = run_greedy(x)
    assert int(g.status[0]) == 0
    acc, out, nodes = oracle.tree_greedy(x.widened(x.target), x.parent, x.node_token, x.Dmax)
    np.testing.assert_array_equal(g.accepted, acc)
    np.testing.assert_array_equal(g.out_tokens, out)
    np.testing.assert_array_equal(g.accepted_nodes, nodes)
    gp = run_path(x, space=space)
    assert int(gp.status[0]) == 0
    rp = oracle.tree_path(x.widened(x.target), x.widened(x.draft), x.node_token, x.path,
                          x.u_accept, x.u_sample, x.lam, x.temperature, space=space)
    report(f"sweep path {i}", compare_chain(x, gp, rp, lengths=path_lengths(x)))
    gm, _ = _multi_case(x, space=space, label=f"sweep multi {i}")
    assert int(gm.status[0]) == 0
    st, bad = _mask_case(x.parent)
    assert st == 0 and not bad.any()
