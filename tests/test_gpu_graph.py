"""Calls of the library captured in a HIP graph and replayed, and the read-stream
calibration kernel.

One graph holds a ragged batched chain call (c4's shapes at a smaller
vocabulary), a logit-space chain call and a greedy tree call; another holds
path-mode calls in both mixture spaces and a tree-mask call; each is bound to
one side stream.
Every replay is checked against the fp64 oracle, with eager work on the same
stream between replays (the outputs are overwritten, and the uniforms are
replaced in place, so each replay must read its inputs afresh).
"""
import numpy as np
import pytest
import torch

import oracle
from sampling_spec_verify_amd import specverify as sv
from sampling_spec_verify_amd import synth
from tests.gpu_util import compare_chain, dev, dev_logits, oracle_chain, path_lengths

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    sv.lib()


def _host(out):
    return type(out)(*[t.cpu().numpy() for t in out])


def test_graph_replays_follow_the_oracle():
    xa = synth.make_chain(seed=4101, B=24, K=8, V=5003, dtype="bf16", lam=0.0, temperature=0.7,
                          ragged=True)
    xb = synth.make_chain(seed=4102, B=6, K=5, V=3001, dtype="fp32", lam=0.4, temperature=1.3)
    xt = synth.make_random_tree(seed=4103, B=4, N=19, V=2048, dtype="bf16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ua_a, us_a = dev(xa.u_accept), dev(xa.u_sample)
        ua_b, us_b = dev(xb.u_accept), dev(xb.u_sample)
        ca = sv.ChainCall(dev_logits(xa.target, xa.dtype), dev_logits(xa.draft, xa.dtype),
                          dev(xa.tokens), ua_a, us_a, xa.lam, xa.temperature, dev(xa.draft_len),
                          stream=s)
        cb = sv.ChainCall(dev_logits(xb.target, xb.dtype), dev_logits(xb.draft, xb.dtype),
                          dev(xb.tokens), ua_b, us_b, xb.lam, xb.temperature, None, stream=s,
                          space="logit")
        ct = sv.TreeGreedyCall(dev_logits(xt.target, xt.dtype), dev(xt.parent),
                               dev(xt.node_token), xt.Dmax, stream=s)
        for c in (ca, cb, ct):          # eager first run: the kernels are loaded before capture
            c.run()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ca.run()
        cb.run()
        ct.run()
    t_acc, t_tok, t_nodes = oracle.tree_greedy(xt.widened(xt.target), xt.parent, xt.node_token,
                                               xt.Dmax)
    rng = np.random.default_rng(4104)
    for rep in range(4):
        if rep >= 2:                    # new uniforms, written in place on the graph's stream
            xa.u_accept = rng.random(xa.u_accept.shape, dtype=np.float32)
            xa.u_sample = rng.random(xa.u_sample.shape, dtype=np.float32)
            xb.u_accept = rng.random(xb.u_accept.shape, dtype=np.float32)
            xb.u_sample = rng.random(xb.u_sample.shape, dtype=np.float32)
        with torch.cuda.stream(s):
            if rep >= 2:
                ua_a.copy_(torch.from_numpy(xa.u_accept).to("cuda:0", non_blocking=False))
                us_a.copy_(torch.from_numpy(xa.u_sample).to("cuda:0", non_blocking=False))
                ua_b.copy_(torch.from_numpy(xb.u_accept).to("cuda:0", non_blocking=False))
                us_b.copy_(torch.from_numpy(xb.u_sample).to("cuda:0", non_blocking=False))
            for c in (ca, cb, ct):
                for o in c.out:
                    o.fill_(-7)
            g.replay()
        s.synchronize()
        print(f"[graph] replay {rep}", flush=True)
        ga, gb, gt = _host(ca.out), _host(cb.out), _host(ct.out)
        assert ga.status[0] == 0 and gb.status[0] == 0 and gt.status[0] == 0
        compare_chain(xa, ga, oracle_chain(xa))
        compare_chain(xb, gb, oracle_chain(xb, space="logit"))
        assert np.array_equal(gt.accepted, t_acc)
        assert np.array_equal(gt.out_tokens, t_tok)
        assert np.array_equal(gt.accepted_nodes, t_nodes)


def test_graph_replays_path_and_mask_follow_the_oracle():
    """Path-mode calls (both mixture spaces) and a mask call in one graph.  From
    the third replay on, new uniforms and new node tokens are written in place
    between replays: each replay must read the path's tokens afresh."""
    xp = synth.make_random_tree(seed=4111, B=5, N=40, V=4099, dtype="bf16", sharp=1.0, lam=0.3,
                                temperature=0.9)
    xq = synth.make_random_tree(seed=4112, B=3, N=12, V=2048, dtype="fp32", sharp=1.0, lam=0.4,
                                temperature=1.2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ins = []
        calls = []
        for x, space in ((xp, "prob"), (xq, "logit")):
            ua, us, tok = dev(x.u_accept), dev(x.u_sample), dev(x.node_token)
            ins.append((ua, us, tok))
            calls.append(sv.TreePathCall(dev_logits(x.target, x.dtype), dev_logits(x.draft, x.dtype), tok,
                                         dev(x.path), ua, us, x.lam, x.temperature, stream=s, space=space))
        cm = sv.TreeMaskCall(dev(xp.parent), stream=s)
        for c in (*calls, cm):           # eager first run: the kernels are loaded before capture
            c.run()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in (*calls, cm):
            c.run()
    W = cm.out.mask.shape[2]
    ref_mask, ref_depth, bad = oracle.tree_attention_mask(xp.parent, W)
    assert not bad.any()
    rng = np.random.default_rng(4113)
    for rep in range(4):
        with torch.cuda.stream(s):
            if rep >= 2:
                for x, (ua, us, tok) in zip((xp, xq), ins):
                    x.u_accept = rng.random(x.u_accept.shape, dtype=np.float32)
                    x.u_sample = rng.random(x.u_sample.shape, dtype=np.float32)
                    x.node_token = rng.integers(0, x.V, x.node_token.shape, dtype=np.int32)
                    ua.copy_(torch.from_numpy(x.u_accept).to("cuda:0", non_blocking=False))
                    us.copy_(torch.from_numpy(x.u_sample).to("cuda:0", non_blocking=False))
                    tok.copy_(torch.from_numpy(x.node_token).to("cuda:0", non_blocking=False))
            for c in calls:
                for o in c.out:
                    o.fill_(-7)
            cm.out.mask.fill_(-7)
            cm.out.depth.fill_(-7)
            g.replay()
        s.synchronize()
        print(f"[graph] path and mask replay {rep}", flush=True)
        for c, x, space in zip(calls, (xp, xq), ("prob", "logit")):
            got = _host(c.out)
            assert got.status[0] == 0, (rep, space, sv.decode_flags(int(got.status[0])))
            ref = oracle.tree_path(x.widened(x.target), x.widened(x.draft), x.node_token, x.path,
                                   x.u_accept, x.u_sample, x.lam, x.temperature, space=space)
            compare_chain(x, got, ref, lengths=path_lengths(x))
        np.testing.assert_array_equal(cm.out.mask.cpu().numpy().view(np.uint32), ref_mask)
        np.testing.assert_array_equal(cm.out.depth.cpu().numpy(), ref_depth)
        assert int(cm.out.status[0].item()) == 0


def test_read_stream_reads_its_bytes():
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    zeros = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda:0")
    sv.read_stream(zeros, zeros.numel(), sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    # a single vector whose words fold to the kernel's fixed word: the sink is written
    word = np.array([0x9E3779B9, 0, 0, 0], dtype=np.uint32)
    one = torch.from_numpy(word.view(np.uint8).copy()).to("cuda:0")
    sv.read_stream(one, 16, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == 0x9E3779B9
    # the fold of a ragged tail (one job and a part) covers the last vector too
    n_vec = 512 + 37
    buf = np.zeros((n_vec, 4), dtype=np.uint32)
    buf[n_vec - 1] = word
    sink.zero_()
    t = torch.from_numpy(buf.view(np.uint8).reshape(-1).copy()).to("cuda:0")
    sv.read_stream(t, n_vec * 16, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == 0x9E3779B9
