"""sv_chain_verify_noalloc (the chain call on the library's own per-GPU
scratch array) against sv_chain_verify (caller workspace) on the same inputs:
outputs bitwise equal, over calls in a row whose sizes shrink and grow again,
so that whatever one call leaves in the shared array cannot leak into the next."""
import numpy as np
import pytest
import torch

from sampling_spec_verify_amd import specverify as sv
from sampling_spec_verify_amd import synth
from tests.gpu_util import chain_call, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    sv.lib()


def _both(x, label):
    print(f"[noalloc] {label}: B={x.B} K={x.K} V={x.V} {x.dtype}", flush=True)
    ref = to_host(chain_call(x).run())
    call = chain_call(x)
    for o in call.out:
        o.fill_(-7)
    got = to_host(sv.chain_verify_noalloc(call))
    for name, a, b in zip(ref._fields, ref, got):
        np.testing.assert_array_equal(a, b, err_msg=f"{label}: {name}")
    return ref


def test_noalloc_matches_workspace_call_shrinking_then_growing():
    big = synth.config("c4")                        # 64 ragged requests, V = 128256
    small = synth.make_chain(8100, 3, 5, 20000, "fp32", lam=0.2, temperature=0.9,
                             ragged=True, k_min=0)
    r1 = _both(big, "ragged 64-request batch")
    r2 = _both(small, "3 fp32 requests, V = 20000")
    r3 = _both(big, "ragged 64-request batch again")
    for a, b in zip(r1, r3):
        np.testing.assert_array_equal(a, b)
    assert int(r2.status[0]) == 0

