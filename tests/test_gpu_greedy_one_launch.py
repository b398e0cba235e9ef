"""The greedy tree call's one-launch form against its two-launch form and the
oracle ([EAGLE] "核心思路" step 3: keep a draft equal to the target's most
likely token; [SD] "Tree Speculation").

Trees of at most 64 nodes in batches of at most 1024 take one launch, whose
waves hand chunk and row results over through tagged, self-clearing records;
everything else takes the row-argmax launch and the walk launch.  These cases
check:

* the one launch gives bitwise the two launches' outputs (sv_tree_row_argmax
  then sv_tree_greedy_walk), and the oracle's, on both sides of its size
  limits and with more than 64 chunks per row;
* one workspace serves calls of changing geometry in turn, and a workspace
  full of random bytes serves a first call: no record of another call is
  taken for this call's;
* replays of one captured launch (the same tag every replay) with new logits
  written between replays follow the oracle every time;
* the status word is written by the call itself: a clean call after a flagged
  one reads 0, and a flag raised by any one tree reaches it.
"""
import numpy as np
import pytest
import torch

import oracle
from sampling_spec_verify_amd import specverify as sv
from sampling_spec_verify_amd import synth
from tests.gpu_util import dev, dev_logits, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    sv.lib()


def _call(x, workspace=None):
    return sv.TreeGreedyCall(dev_logits(x.target, x.dtype), dev(x.parent), dev(x.node_token), x.Dmax,
                             workspace=workspace)


def _check_oracle(x, g, Dmax=None):
    Dmax = x.Dmax if Dmax is None else Dmax
    acc, out, nodes = oracle.tree_greedy(x.widened(x.target), x.parent, x.node_token, Dmax)
    np.testing.assert_array_equal(g.accepted, acc)
    np.testing.assert_array_equal(g.out_tokens, out)
    np.testing.assert_array_equal(g.accepted_nodes, nodes)


CASES = [
    # seed, B, N, V, dtype, integer logits (ties)
    (1, 8, 26, 128256, "bf16", False),      # the tree workload's shape
    (2, 3, 63, 5000, "bf16", True),         # 64 nodes: the largest one-launch tree
    (3, 3, 64, 5000, "bf16", True),         # 65 nodes: two launches
    (4, 1024, 5, 700, "fp32", True),        # the largest one-launch batch
    (5, 1025, 5, 700, "fp32", True),        # two launches
    (6, 1, 3, 300001, "bf16", False),       # more than 64 chunks per row
    (7, 5, 0, 900, "fp32", False),          # root only
    (8, 4, 9, 1, "bf16", True),             # V = 1
    (9, 2, 40, 33, "fp32", True),           # one chunk per row: no chunk records
]


@pytest.mark.parametrize("seed,B,N,V,dtype,ints", CASES, ids=[f"B{c[1]}-N{c[2]}-V{c[3]}" for c in CASES])
def test_one_launch_equals_two_launches_and_the_oracle(seed, B, N, V, dtype, ints):
    x = synth.make_random_tree(9400 + seed, B, N, V, dtype, int_logits=ints)
    print(f"[greedy one-launch] B={B} N={N} V={V} {dtype}", flush=True)
    call = _call(x)
    for o in call.out:
        o.fill_(-7)
    full = to_host(call.run())
    for o in call.out:
        o.fill_(-7)
    call.row_argmax()
    split = to_host(call.walk())
    for f, a, b in zip(full._fields, full, split):
        np.testing.assert_array_equal(a, b, err_msg=f)
    assert int(full.status[0]) == 0
    _check_oracle(x, full)


def test_one_workspace_across_geometries_and_random_bytes():
    xs = [synth.make_random_tree(9500, 9, 30, 40000, "bf16"),
          synth.make_random_tree(9501, 4, 12, 70001, "fp32", int_logits=True),
          synth.make_random_tree(9502, 13, 63, 2500, "bf16", int_logits=True),
          synth.make_tree(9503, 8, 26, 128256, "bf16")]
    size = max(sv.tree_workspace_bytes(x.B, x.N, x.V) for x in xs)
    ws = torch.empty(size, dtype=torch.uint8, device="cuda:0")
    gen = torch.Generator(device="cpu").manual_seed(9504)
    ws.copy_(torch.randint(0, 256, (size,), dtype=torch.uint8, generator=gen).to(ws.device))
    calls = [_call(x, workspace=ws) for x in xs]
    refs = [oracle.tree_greedy(x.widened(x.target), x.parent, x.node_token, x.Dmax) for x in xs]
    for rep in range(30):
        if rep == 15:                       # random bytes again, mid-sequence
            ws.copy_(torch.randint(0, 256, (size,), dtype=torch.uint8, generator=gen).to(ws.device))
        for c, (acc, out, nodes) in zip(calls, refs):
            for o in c.out:
                o.fill_(-7)
            g = to_host(c.run())
            assert int(g.status[0]) == 0, (rep, sv.decode_flags(int(g.status[0])))
            np.testing.assert_array_equal(g.accepted, acc)
            np.testing.assert_array_equal(g.out_tokens, out)
            np.testing.assert_array_equal(g.accepted_nodes, nodes)
    print("[greedy one-launch] 120 calls over 4 geometries on one workspace", flush=True)


def test_graph_replays_with_new_logits_between_replays():
    """A captured launch keeps its tag on every replay; the records a replay
    reads must be its own, so each replay's outputs follow its own logits."""
    B, N, V = 6, 30, 20000
    xs = [synth.make_random_tree(9600 + k, B, N, V, "bf16", int_logits=True) for k in range(4)]
    for x in xs[1:]:                         # one tree shape, new logits
        x.parent[:] = xs[0].parent
        x.node_token[:] = xs[0].node_token
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        tgt = dev_logits(xs[0].target, "bf16")
        call = sv.TreeGreedyCall(tgt, dev(xs[0].parent), dev(xs[0].node_token), xs[0].Dmax, stream=s)
        call.run()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call.run()
    for rep in range(8):
        x = xs[rep % 4]
        with torch.cuda.stream(s):
            tgt.copy_(dev_logits(x.target, "bf16"))
            for o in call.out:
                o.fill_(-7)
            g.replay()
        s.synchronize()
        out = to_host(call.out)
        print(f"[greedy one-launch] graph replay {rep}", flush=True)
        assert int(out.status[0]) == 0
        _check_oracle(x, out, Dmax=xs[0].Dmax)     # the captured call's Dmax


def test_status_is_written_by_the_call():
    """The one launch stores the status once, from the last tree to finish:
    a clean call after a flagged one reads 0 on the same status buffer, and a
    flag raised by any one tree reaches it."""
    x = synth.make_random_tree(9700, 6, 10, 3000, "fp32", int_logits=True)
    bad_parent = x.parent.copy()
    bad_parent[0, 4] = 9                     # node 5 of tree 0: a parent not below it
    call = _call(x)
    par = call.inputs[1]
    for rep in range(3):
        par.copy_(torch.from_numpy(bad_parent).to(par.device))
        gb = to_host(call.run())
        assert sv.decode_flags(int(gb.status[0])) == ["BAD_TREE"], int(gb.status[0])
        par.copy_(torch.from_numpy(x.parent).to(par.device))
        go = to_host(call.run())
        assert int(go.status[0]) == 0
        _check_oracle(x, go)
    for t in (5, 3, 0):
        y = synth.make_random_tree(9701, 6, 10, 3000, "fp32", int_logits=True)
        y.node_token[t, 0] = 3000            # out of range: BAD_TOKEN
        g = to_host(_call(y).run())
        assert sv.decode_flags(int(g.status[0])) == ["BAD_TOKEN"], (t, int(g.status[0]))
