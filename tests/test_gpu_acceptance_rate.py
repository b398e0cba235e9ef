"""The acceptance-rate call's hand-over between waves, against the oracle
([SD] and [EAGLE]: the acceptance rate of a position is sum_v min(p~, q)).

Each position's chunk sums reach the wave of its last chunk as tagged records,
which that wave clears after reading, and the statistics launch sets every
alpha to 0 first.  These cases check:

* one workspace serves calls of changing geometry in turn, and a workspace
  full of random bytes serves a first call: no record of another call is
  taken for this call's, and alpha past each draft length reads 0 whatever
  the output held;
* rows of more than 64 chunks (a summing lane takes several chunks) and of
  one chunk (no records at all);
* replays of one captured call (the same tag every replay) with new logits
  written between replays follow the oracle every time;
* the status word is cleared by each call: a clean call after a flagged one
  on the same status buffer reads 0.
"""
import numpy as np
import pytest
import torch

from sampling_spec_verify_amd import specverify as sv
from sampling_spec_verify_amd import synth
from tests.gpu_util import dev, dev_logits, oracle_chain

pytestmark = pytest.mark.gpu

ALPHA_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    sv.lib()


def _ref(x, space):
    ref = oracle_chain(x, space=space)
    lens = x.lengths()
    out = np.zeros((x.B, x.K))
    for b in range(x.B):
        out[b, :int(lens[b])] = ref.details[b].alpha
    return out


def _check(x, alpha, ref):
    g = alpha.cpu().numpy().astype(np.float64)
    lens = x.lengths()
    for b in range(x.B):
        k = int(lens[b])
        assert np.all(g[b, k:] == 0.0), b
    err = float(np.abs(g - ref).max()) if g.size else 0.0
    assert err <= ALPHA_TOL, err
    return err


def _call(x, space, workspace=None, stream=None, tensors=None):
    t, d = tensors if tensors is not None else (dev_logits(x.target, x.dtype), dev_logits(x.draft, x.dtype))
    return sv.AcceptanceRateCall(t, d, x.lam, x.temperature, dev(x.draft_len), stream=stream,
                                 workspace=workspace, space=space)


SHAPES = [
    # seed, B, K, V, dtype, lam, T, ragged, space
    (1, 16, 8, 151936, "bf16", 0.3, 1.0, False, "prob"),
    (2, 5, 3, 1 << 20, "fp32", 0.0, 0.7, True, "prob"),    # more than 64 chunks per row
    (3, 7, 4, 300, "fp32", 0.5, 1.0, True, "logit"),       # one chunk per row
    (4, 300, 2, 2000, "bf16", 0.0, 1.0, True, "prob"),     # more than 256 requests
    (5, 9, 6, 40001, "bf16", 0.4, 1.3, True, "logit"),
]


def test_one_workspace_across_geometries_and_random_bytes():
    xs = [synth.make_chain(9800 + s, B, K, V, dt, sigma_t=2.0, sigma_q=(0.3, 2.0), zipf=True, lam=lam,
                           temperature=T, ragged=rg, k_min=0)
          for s, B, K, V, dt, lam, T, rg, _ in SHAPES]
    spaces = [c[-1] for c in SHAPES]
    size = max(int(sv.lib().sv_chain_acceptance_workspace_bytes(x.B, x.K, x.V)) for x in xs)
    ws = torch.empty(size, dtype=torch.uint8, device="cuda:0")
    gen = torch.Generator(device="cpu").manual_seed(9810)
    ws.copy_(torch.randint(0, 256, (size,), dtype=torch.uint8, generator=gen).to(ws.device))
    calls = [_call(x, sp, workspace=ws) for x, sp in zip(xs, spaces)]
    refs = [_ref(x, sp) for x, sp in zip(xs, spaces)]
    worst = 0.0
    for rep in range(12):
        if rep == 6:                        # random bytes again, mid-sequence
            ws.copy_(torch.randint(0, 256, (size,), dtype=torch.uint8, generator=gen).to(ws.device))
        for x, c, ref in zip(xs, calls, refs):
            c.alpha.fill_(-7.0)
            alpha, status = c.run()
            torch.cuda.synchronize()
            assert int(status[0].item()) == 0, (rep, sv.decode_flags(int(status[0].item())))
            worst = max(worst, _check(x, alpha, ref))
    print(f"[alpha] 60 calls over 5 geometries on one workspace, max |err| {worst:.2e}", flush=True)


def test_graph_replays_with_new_logits_between_replays():
    """A captured call keeps its tag on every replay; the records a replay
    reads must be its own, so each replay's alpha follows its own logits."""
    B, K, V = 6, 5, 20000
    xs = [synth.make_chain(9900 + k, B, K, V, "bf16", sigma_q=(0.3, 2.0), lam=0.3, ragged=True, k_min=0)
          for k in range(4)]
    for x in xs[1:]:                         # one set of draft lengths, new logits
        x.draft_len[:] = xs[0].draft_len
    refs = [_ref(x, "prob") for x in xs]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        t = dev_logits(xs[0].target, "bf16")
        d = dev_logits(xs[0].draft, "bf16")
        call = _call(xs[0], "prob", stream=s, tensors=(t, d))
        call.run()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call.run()
    for rep in range(8):
        x = xs[rep % 4]
        with torch.cuda.stream(s):
            t.copy_(dev_logits(x.target, "bf16"))
            d.copy_(dev_logits(x.draft, "bf16"))
            call.alpha.fill_(-7.0)
            g.replay()
        s.synchronize()
        print(f"[alpha] graph replay {rep}", flush=True)
        assert int(call.status[0].item()) == 0
        _check(x, call.alpha, refs[rep % 4])


def test_status_is_cleared_by_each_call():
    x = synth.make_chain(9950, 3, 3, 3000, "fp32", lam=0.3)
    bad = x.target.copy()
    bad[1, 2, 5] = np.nan
    t = dev_logits(bad, x.dtype)
    call = _call(x, "prob", tensors=(t, dev_logits(x.draft, x.dtype)))
    ref = _ref(x, "prob")
    for rep in range(3):
        t.copy_(dev_logits(bad, x.dtype))
        alpha, status = call.run()
        torch.cuda.synchronize()
        assert sv.decode_flags(int(status[0].item())) == ["BAD_ROW"], int(status[0].item())
        a = alpha.cpu().numpy()
        assert np.isnan(a[1, 2]) and np.isfinite(a).sum() == a.size - 1
        t.copy_(dev_logits(x.target, x.dtype))
        alpha, status = call.run()
        torch.cuda.synchronize()
        assert int(status[0].item()) == 0
        _check(x, alpha, ref)
