"""Helpers of the GPU parity tests: move seeded inputs to the device, run the
library through its C ABI, and compare with the fp64 oracle request by request."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from sampling_spec_verify_amd import specverify as sv
from sampling_spec_verify_amd.synth import ChainInputs, TreeInputs

DEV = "cuda:0"
ACCEPT_PROB_TOL = 1e-5      # per-position acceptance probability, absolute


def dev_logits(arr: np.ndarray, dtype: str, ld: int | None = None) -> torch.Tensor:
    """[B, R, V] logits (fp32, or bf16 bits) as a device view over a [B, R, ld] buffer."""
    B, R, V = arr.shape
    if ld is None:                       # rows must start on 16-byte boundaries
        per = 8 if dtype == "bf16" else 4
        ld = -(-V // per) * per
    if dtype == "bf16":
        buf = torch.zeros((B, R, ld), dtype=torch.int16)
        buf[:, :, :V] = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
        t = buf.to(DEV).view(torch.bfloat16)
    else:
        buf = torch.zeros((B, R, ld), dtype=torch.float32)
        buf[:, :, :V] = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
        t = buf.to(DEV)
    return t[:, :, :V]


def dev(a: np.ndarray | None):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def chain_call(x: ChainInputs, ld: int | None = None, space: str = "prob") -> sv.ChainCall:
    return sv.ChainCall(dev_logits(x.target, x.dtype, ld), dev_logits(x.draft, x.dtype, ld),
                        dev(x.tokens), dev(x.u_accept), dev(x.u_sample), x.lam, x.temperature,
                        dev(x.draft_len), space=space)


def to_host(out):
    torch.cuda.synchronize()
    return type(out)(*[t.cpu().numpy() for t in out])


def run_chain(x: ChainInputs, ld: int | None = None, space: str = "prob"):
    return to_host(chain_call(x, ld, space).run())


def oracle_chain(x: ChainInputs, requests=None, space: str = "prob"):
    return oracle.chain_verify(x.widened(x.target), x.widened(x.draft), x.tokens, x.draft_len,
                               x.u_accept, x.u_sample, x.lam, x.temperature, requests, space)


def flag_limit(requests: int) -> int:
    """Most boundary-flagged requests a comparison may excuse: 1 + requests / 16.
    An acceptance draw falls in the 1e-6 band of its ratio with probability
    2e-6; a sampling draw falls in the band of some CDF boundary with
    probability up to 2e-6 per token of the law's support (about 1 % at
    V = 1500, more where many tokens carry under 2e-6 of mass each).  A band of
    1e-3, or an inverted test, would flag nearly every request."""
    return 1 + requests // 16


def compare_chain(x: ChainInputs, g, ref, requests=None, lengths=None):
    """Bit-exact counts and tokens outside flagged draws; a_i within 1e-5; at
    most flag_limit() flagged requests."""
    lens = x.lengths() if lengths is None else lengths
    req = range(x.B) if requests is None else requests
    stats = {"requests": 0, "flagged": 0, "flagged_mismatch": 0, "max_a_err": 0.0}
    for b in req:
        k = int(lens[b])
        err = np.abs(g.accept_prob[b, :k].astype(np.float64) - ref.accept_prob[b, :k])
        stats["max_a_err"] = max(stats["max_a_err"], float(err.max()) if k else 0.0)
        assert np.all(err <= ACCEPT_PROB_TOL), (b, err.max())
        assert np.all(g.accept_prob[b, k:] == 0.0)
        same = g.accepted[b] == ref.accepted[b] and np.array_equal(g.out_tokens[b], ref.out_tokens[b])
        stats["requests"] += 1
        if ref.flagged[b]:
            stats["flagged"] += 1
            stats["flagged_mismatch"] += int(not same)
        else:
            assert same, (f"request {b}: gpu n={g.accepted[b]} {g.out_tokens[b].tolist()} "
                          f"oracle n={ref.accepted[b]} {ref.out_tokens[b].tolist()}")
    assert stats["flagged"] <= flag_limit(stats["requests"]), stats
    return stats


def run_greedy(x: TreeInputs, Dmax: int | None = None, ld: int | None = None):
    Dmax = x.Dmax if Dmax is None else Dmax
    out = sv.tree_verify_greedy(dev_logits(x.target, x.dtype, ld), dev(x.parent),
                                dev(x.node_token), Dmax)
    return to_host(out)


def run_path(x: TreeInputs, ld: int | None = None, space: str = "prob"):
    out = sv.tree_verify_path(dev_logits(x.target, x.dtype, ld), dev_logits(x.draft, x.dtype, ld),
                              dev(x.node_token), dev(x.path), dev(x.u_accept), dev(x.u_sample),
                              x.lam, x.temperature, space=space)
    return to_host(out)


def path_lengths(x: TreeInputs) -> np.ndarray:
    return np.array([len(oracle.path_rows(x.path[b])) for b in range(x.B)], dtype=np.int32)
