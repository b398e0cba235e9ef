"""The multi-branch walk at every number of blocks per tree, and on a grid
wider than the GPU.

A tree's blocks wait for one another at its barriers.  Each block takes its
(tree, slice) role from a start-order ticket, so the walk needs only one
tree's blocks on the GPU at once: a grid of more blocks than the compute units
hold runs its trees in rounds.  These cases check that every choice of blocks
per tree, that wide grid included, gives the oracle's walk ([SD] "Tree
Speculation", the chain rule of [EAGLE] section 1 applied to what a rejection
leaves) with the status word clear, and that replays of one captured call on
one workspace follow the oracle with new logits each time.
"""
import numpy as np
import pytest
import torch

from sampling_spec_verify_amd import specverify as sv
from sampling_spec_verify_amd import synth
from tests.gpu_util import dev, dev_logits, to_host
from tests.test_gpu_parity import _multi_case, compare_multi

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    sv.lib()


@pytest.mark.parametrize("blocks", [1, 2, 5, 16, 32])
def test_multi_every_block_count_matches_the_oracle(blocks):
    x = synth.config("c5")
    x.lam = 0.3
    print(f"[multi blocks] c5 trees, lam 0.3, {blocks} blocks per tree", flush=True)
    g, stats = _multi_case(x, label=f"c5 multi, {blocks} blocks per tree", blocks_per_tree=blocks)
    assert int(g.status[0]) == 0


def test_multi_grid_wider_than_the_gpu():
    """64 trees at 16 blocks each: 1024 walk blocks, four times what the
    compute units hold at once (one 512-thread walk block per unit)."""
    props = torch.cuda.get_device_properties(0)
    x = synth.make_tree(9100, 64, 26, 65536, "bf16", lam=0.2)
    assert 64 * 16 > props.multi_processor_count
    print(f"[multi blocks] 64 trees x 16 blocks on {props.multi_processor_count} units", flush=True)
    for space in ("prob", "logit"):
        g, stats = _multi_case(x, space=space, label=f"64 trees x 16 blocks, {space}", blocks_per_tree=16)
        assert int(g.status[0]) == 0, sv.decode_flags(int(g.status[0]))


def test_multi_block_counts_agree_with_each_other():
    """The walk's decisions do not depend on the block count: the same trees at
    1 and 16 blocks emit the same tokens outside draws near a boundary."""
    x = synth.make_tree(9200, 12, 40, 128256, "bf16", lam=0.0)
    g1, s1 = _multi_case(x, label="12 trees, 1 block", blocks_per_tree=1)
    g16, s16 = _multi_case(x, label="12 trees, 16 blocks", blocks_per_tree=16)
    if s1["flagged"] == 0 and s16["flagged"] == 0:
        np.testing.assert_array_equal(g1.out_tokens, g16.out_tokens)
        np.testing.assert_array_equal(g1.accepted_nodes, g16.accepted_nodes)
    tested = g1.accept_prob >= 0
    np.testing.assert_array_equal(tested, g16.accept_prob >= 0)
    assert float(np.abs(g1.accept_prob[tested] - g16.accept_prob[tested]).max(initial=0.0)) <= 1e-6


def test_graph_replays_with_new_logits_between_replays():
    """Replays of one captured call (the statistics launch and the walk) on one
    workspace, with new logits written between replays, follow the oracle every
    time: the statistics launch empties the walk's barrier slots, resets its
    ticket counter and clears the status word on every replay."""
    B, N, V = 6, 20, 20000
    xs = [synth.make_random_tree(9800 + k, B, N, V, "bf16", sharp=1.0, sigma_q=2.0, lam=0.2)
          for k in range(4)]
    for x in xs[1:]:                         # one tree shape and one set of uniforms
        x.parent[:] = xs[0].parent
        x.node_token[:] = xs[0].node_token
        x.u_node[:] = xs[0].u_node
        x.u_sample[:] = xs[0].u_sample
    x0 = xs[0]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        t = dev_logits(x0.target, "bf16")
        d = dev_logits(x0.draft, "bf16")
        par, tok, un, us = dev(x0.parent), dev(x0.node_token), dev(x0.u_node), dev(x0.u_sample)
        ws = torch.empty(int(sv.lib().sv_tree_multi_workspace_bytes(B, N, V)), dtype=torch.uint8,
                         device="cuda:0")
        sv.tree_verify_multi(t, d, par, tok, un, us, x0.Dmax, x0.lam, x0.temperature, "prob",
                             stream=s, workspace=ws)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        out = sv.tree_verify_multi(t, d, par, tok, un, us, x0.Dmax, x0.lam, x0.temperature, "prob",
                                   stream=s, workspace=ws)
    for rep in range(8):
        x = xs[rep % 4]
        with torch.cuda.stream(s):
            t.copy_(dev_logits(x.target, "bf16"))
            d.copy_(dev_logits(x.draft, "bf16"))
            for o in out:
                o.fill_(-7)
            g.replay()
        s.synchronize()
        print(f"[multi blocks] graph replay {rep}", flush=True)
        h = to_host(out)
        assert int(h.status[0]) == 0, sv.decode_flags(int(h.status[0]))
        compare_multi(x, h, x0.Dmax, label=f"multi graph replay {rep}")


@pytest.mark.parametrize("B,N,V,dtype", [
    (2, 31, 128256, "bf16"),     # 2 x 32 rows x 32 chunks = 2048 partials: the table's limit
    (2, 32, 128256, "bf16"),     # 2112 partials: combined on the way
    (3, 62, 3000, "fp32"),       # 63 nodes
    (3, 63, 3000, "fp32"),       # 64 nodes: the largest tabled tree
    (3, 64, 3000, "fp32"),       # 65 nodes: combined on the way
], ids=["N31-at-parts-limit", "N32-past-parts-limit", "N62", "N63-at-node-limit", "N64-past-node-limit"])
def test_statistics_table_limits(B, N, V, dtype):
    """A tree of at most 64 nodes whose rows' chunk partials fit the table has
    every node's statistics, logits and first-child test formed at its start;
    a larger one combines them on the way.  Both sides of both limits follow
    the oracle, in both spaces."""
    for space, lam in (("prob", 0.0), ("logit", 0.3)):
        if V > 100000:      # the tree workload's recipe (peaked rows: draws far from boundaries)
            x = synth.make_tree(9900 + N, B, N, V, dtype, lam=lam, sigma_q=1.5)
        else:
            x = synth.make_random_tree(9900 + N, B, N, V, dtype, sharp=1.0, sigma_q=2.0, lam=lam)
        g, _ = _multi_case(x, space=space, label=f"table limits N={N} V={V} {space}")
        assert int(g.status[0]) == 0
