"""Seeded synthetic inputs for the speculative-decoding verify step.

This module only *draws* inputs: logits, drafted tokens, uniforms, draft trees
and tree paths.  It holds none of the verify arithmetic (no softmax, no
mixture, no acceptance ratio, no residual, no inverse CDF).  Drafted tokens are
drawn with the Gumbel-max trick, ``argmax(z / T + G)`` with ``G`` standard
Gumbel noise, which yields an exact sample of ``softmax(z / T)`` without
evaluating that softmax.

Both the HIP path and the CPU oracle consume what this module returns; it is
the only code the two share.

Workloads (seeded, one ``numpy.random.SeedSequence(1000 + c)`` per config):

* ``c1`` tiny linear chain: B=1, K=4, V=1000, fp32; target ~ N(0, 2^2),
  draft = target + N(0, 1); lambda 0, T 1.
* ``c2`` single request, Llama-3 vocabulary: B=1, K=8, V=128256, bf16;
  target ~ N(0, 3^2) + Zipf-like rank bias, draft = target + N(0, 1).
* ``c3`` RAPID mixture, batched: B=16, K=8, V=151936 (Qwen2.5 vocabulary),
  bf16; draft = target + N(0, 0.5^2); lambda 0.3, T 1.
* ``c4`` ragged batch: B=64, K_b ~ U{1..8}, V=128256, bf16, T 0.7; per request
  draft noise sigma_b ~ U[0.3, 2.0].
* ``c5`` draft trees: B=8, 26 nodes each (depth 6, per-depth child caps
  4/3/2/1/1/1), target and draft [8, 27, 128256] bf16.

The Zipf-like bias gives the token of rank r (r = 1..V, a fresh seeded
permutation per row) the additive logit ``-1.1 * ln(r)``.  Logits are formed
in fp32 and rounded to bf16 with round-to-nearest-even on the bit pattern.
Uniforms are fp32 multiples of 2^-24 in [0, 1).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# ---------------------------------------------------------------------------
# primitives
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); uint16 bits.

    NaN inputs stay NaN (quiet); infinities stay infinite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    t = u >> 16
    t &= 1
    t += 0x7FFF
    t += u                       # no uint32 overflow for finite inputs
    t >>= 16
    r = t.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    """fp32 uniforms on the 2^-24 grid in [0, 1)."""
    return rng.random(shape, dtype=np.float32)


def raise_uniforms(u: np.ndarray, eps: float) -> np.ndarray:
    """Map grid uniforms u in [0, 1) onto the top of the interval, [1 - eps, 1):
    1 - m 2^-24 with m = max(1, round(eps (1 - u) 2^24)), still on the grid.
    Acceptance uniforms this high reject most drafts whose ratio is below one,
    which makes a close draft produce residual draws."""
    k = np.rint((1.0 - np.asarray(u, dtype=np.float64)) * 2.0 ** 24)
    m = np.maximum(1.0, np.rint(eps * k))
    return (1.0 - m * 2.0 ** -24).astype(np.float32)


def zipf_bias(rng: np.random.Generator, rows: int, V: int, slope: float = 1.1) -> np.ndarray:
    """[rows, V] fp32: rank r (1-based) of a fresh permutation gets -slope*ln(r)."""
    ranks = -slope * np.log(np.arange(1, V + 1, dtype=np.float64))
    out = np.empty((rows, V), dtype=np.float32)
    for i in range(rows):
        perm = rng.permutation(V)
        out[i, perm] = ranks
    return out


def gumbel_max_sample(rng: np.random.Generator, logits: np.ndarray, T: float) -> np.ndarray:
    """One exact draw from softmax(logits / T) per row via argmax(z/T + Gumbel).

    ``logits`` is [..., V] (any float type; widened to fp64).  Returns int32.
    """
    z = np.asarray(logits, dtype=np.float64)
    g = rng.gumbel(size=z.shape)
    return np.argmax(z / float(T) + g, axis=-1).astype(np.int32)


# ---------------------------------------------------------------------------
# containers
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class ChainInputs:
    """Inputs of one linear-chain verify call.

    target  [B, K+1, V]  fp32 array, or uint16 bf16 bits when dtype == "bf16"
    draft   [B, K, V]    same dtype as target
    tokens  [B, K]       int32 drafted tokens (entries >= draft_len[b] unused)
    draft_len [B] int32 or None (None: every request drafts K tokens)
    u_accept [B, K] fp32, u_sample [B] fp32
    """

    name: str
    dtype: str
    target: np.ndarray
    draft: np.ndarray
    tokens: np.ndarray
    draft_len: Optional[np.ndarray]
    u_accept: np.ndarray
    u_sample: np.ndarray
    lam: float
    temperature: float

    @property
    def B(self) -> int:
        return self.target.shape[0]

    @property
    def K(self) -> int:
        return self.draft.shape[1]

    @property
    def V(self) -> int:
        return self.target.shape[2]

    def lengths(self) -> np.ndarray:
        if self.draft_len is None:
            return np.full(self.B, self.K, dtype=np.int32)
        return self.draft_len

    def positions(self) -> int:
        """Number of verified draft positions (sum of K_b)."""
        return int(self.lengths().sum())

    def widened(self, a: np.ndarray) -> np.ndarray:
        """fp32 view of a logits array (exact for bf16)."""
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else a


@dataclasses.dataclass
class TreeInputs:
    """Inputs of one draft-tree verify call (greedy and path modes).

    target [B, N+1, V], draft [B, N+1, V] (fp32, or bf16 bits)
    parent [B, N] int32: parent of node i+1 (0 = root), parent < i+1
    node_token [B, N] int32: token of node i+1
    path [B, Dmax] int32: root->leaf node ids (1-based), -1 terminated
    u_accept [B, Dmax], u_sample [B] fp32
    u_node [B, N] fp32: one acceptance uniform per node (multi-branch walks)
    """

    name: str
    dtype: str
    target: np.ndarray
    draft: np.ndarray
    parent: np.ndarray
    node_token: np.ndarray
    path: np.ndarray
    u_accept: np.ndarray
    u_sample: np.ndarray
    lam: float
    temperature: float
    u_node: Optional[np.ndarray] = None

    @property
    def B(self) -> int:
        return self.target.shape[0]

    @property
    def N(self) -> int:
        return self.parent.shape[1]

    @property
    def V(self) -> int:
        return self.target.shape[2]

    @property
    def Dmax(self) -> int:
        return self.path.shape[1]

    def widened(self, a: np.ndarray) -> np.ndarray:
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else a


# ---------------------------------------------------------------------------
# generic chain generator
# ---------------------------------------------------------------------------

# new streams go at the end: spawned children keep their index, so the
# earlier streams (and every input drawn from them) stay as they were
_STREAMS = ("target", "noise", "perm", "sigma_k", "draft_tok", "u_accept", "u_sample",
            "tree_shape", "tree_path", "u_node")


def _streams(seed: int):
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {n: np.random.Generator(np.random.PCG64(k)) for n, k in zip(_STREAMS, kids)}


def make_chain(seed: int, B: int, K: int, V: int, dtype: str = "bf16", *,
               sigma_t: float = 3.0, sigma_q=1.0, zipf: bool = True,
               lam: float = 0.0, temperature: float = 1.0,
               ragged: bool = False, k_min: int = 1, name: str = "chain") -> ChainInputs:
    """Seeded chain inputs.

    ``sigma_q`` is a float (one draft-noise scale) or a (lo, hi) pair, in which
    case every request draws its own scale uniformly from [lo, hi].
    ``ragged`` draws K_b uniformly from {k_min..K} per request.
    """
    assert dtype in ("bf16", "fp32")
    s = _streams(seed)
    zt = (s["target"].standard_normal((B, K + 1, V), dtype=np.float32) * np.float32(sigma_t))
    if zipf:
        zt += zipf_bias(s["perm"], B * (K + 1), V).reshape(B, K + 1, V)
    if isinstance(sigma_q, tuple):
        sig = s["sigma_k"].uniform(sigma_q[0], sigma_q[1], size=B).astype(np.float32)
    else:
        sig = np.full(B, sigma_q, dtype=np.float32)
    zq = zt[:, :K, :] + s["noise"].standard_normal((B, K, V), dtype=np.float32) * sig[:, None, None]
    if ragged:
        draft_len = s["sigma_k"].integers(k_min, K + 1, size=B).astype(np.int32)
    else:
        draft_len = None
    if dtype == "bf16":
        t_arr = f32_to_bf16_bits(zt)
        q_arr = f32_to_bf16_bits(zq)
        q_w = bf16_bits_to_f32(q_arr)
    else:
        t_arr = np.ascontiguousarray(zt, dtype=np.float32)
        q_arr = np.ascontiguousarray(zq, dtype=np.float32)
        q_w = q_arr
    del zt, zq
    tokens = np.zeros((B, K), dtype=np.int32)
    for b in range(B):
        tokens[b] = gumbel_max_sample(s["draft_tok"], q_w[b], temperature)
    u_acc = uniforms(s["u_accept"], (B, K))
    u_smp = uniforms(s["u_sample"], (B,))
    return ChainInputs(name, dtype, t_arr, q_arr, tokens, draft_len, u_acc, u_smp,
                       float(lam), float(temperature))


# ---------------------------------------------------------------------------
# draft trees
# ---------------------------------------------------------------------------

#: child caps per depth for the c5 tree (root 4, depth 1: 3, depth 2: 2,
#: depths 3..5: 1, depth 6: leaves)
TREE_CAPS = (4, 3, 2, 1, 1, 1, 0)


def make_tree_shape(rng: np.random.Generator, n_nodes: int = 26, depth: int = 6,
                    caps=TREE_CAPS) -> np.ndarray:
    """Random tree with a guaranteed root->depth spine, nodes renumbered so parent < child.

    Returns ``parent`` [n_nodes] int32 where ``parent[i]`` is the parent of node i+1
    (node 0 is the root).  Nodes are numbered in breadth-first order.
    """
    par = [-1]
    dep = [0]
    nchild = [0]
    for d in range(1, depth + 1):          # the spine 0 -> 1 -> ... -> depth
        par.append(d - 1)
        dep.append(d)
        nchild.append(0)
        nchild[d - 1] += 1
    while len(par) < n_nodes + 1:
        open_nodes = [i for i in range(len(par)) if nchild[i] < caps[dep[i]]]
        if not open_nodes:
            raise ValueError("tree caps cannot hold the requested node count")
        p = open_nodes[int(rng.integers(len(open_nodes)))]
        par.append(p)
        dep.append(dep[p] + 1)
        nchild.append(0)
        nchild[p] += 1
    # breadth-first renumbering (children in creation order)
    children = [[] for _ in par]
    for i in range(1, len(par)):
        children[par[i]].append(i)
    order = [0]
    head = 0
    while head < len(order):
        order.extend(children[order[head]])
        head += 1
    new_id = {old: new for new, old in enumerate(order)}
    parent = np.zeros(n_nodes, dtype=np.int32)
    for old in range(1, len(par)):
        parent[new_id[old] - 1] = new_id[par[old]]
    return parent


def tree_depths(parent: np.ndarray) -> np.ndarray:
    d = np.zeros(len(parent) + 1, dtype=np.int32)
    for i in range(1, len(parent) + 1):
        d[i] = d[parent[i - 1]] + 1
    return d


def seeded_path(rng: np.random.Generator, parent: np.ndarray, Dmax: int) -> np.ndarray:
    """Root->leaf path: from each node take child floor(u * n_children)."""
    N = len(parent)
    children = [[] for _ in range(N + 1)]
    for i in range(1, N + 1):
        children[parent[i - 1]].append(i)
    path = np.full(Dmax, -1, dtype=np.int32)
    node, d = 0, 0
    while children[node]:
        u = float(rng.random(dtype=np.float32))
        node = children[node][int(u * len(children[node]))]
        if d >= Dmax:
            raise ValueError("path longer than Dmax")
        path[d] = node
        d += 1
    return path


def make_tree(seed: int, B: int, N: int, V: int, dtype: str = "bf16", *,
              depth: int = 6, caps=TREE_CAPS, sigma_t: float = 3.0, sigma_q: float = 1.0,
              zipf: bool = True, lam: float = 0.0, temperature: float = 1.0,
              Dmax: Optional[int] = None, name: str = "tree") -> TreeInputs:
    """Seeded draft trees; each child's token is drawn from the draft row of its parent."""
    s = _streams(seed)
    Dmax = depth if Dmax is None else Dmax
    zt = s["target"].standard_normal((B, N + 1, V), dtype=np.float32) * np.float32(sigma_t)
    if zipf:
        zt += zipf_bias(s["perm"], B * (N + 1), V).reshape(B, N + 1, V)
    zq = zt + s["noise"].standard_normal((B, N + 1, V), dtype=np.float32) * np.float32(sigma_q)
    if dtype == "bf16":
        t_arr, q_arr = f32_to_bf16_bits(zt), f32_to_bf16_bits(zq)
        q_w = bf16_bits_to_f32(q_arr)
    else:
        t_arr, q_arr = zt.astype(np.float32), zq.astype(np.float32)
        q_w = q_arr
    parent = np.zeros((B, N), dtype=np.int32)
    node_token = np.zeros((B, N), dtype=np.int32)
    path = np.full((B, Dmax), -1, dtype=np.int32)
    for b in range(B):
        parent[b] = make_tree_shape(s["tree_shape"], N, depth, caps)
        # a child's token is a draw from its parent's draft row; siblings draw
        # independently (duplicates allowed)
        for i in range(1, N + 1):
            p = parent[b, i - 1]
            node_token[b, i - 1] = gumbel_max_sample(s["draft_tok"], q_w[b, p], temperature)
        path[b] = seeded_path(s["tree_path"], parent[b], Dmax)
    u_acc = uniforms(s["u_accept"], (B, Dmax))
    u_smp = uniforms(s["u_sample"], (B,))
    return TreeInputs(name, dtype, t_arr, q_arr, parent, node_token, path, u_acc, u_smp,
                      float(lam), float(temperature), uniforms(s["u_node"], (B, N)))


# ---------------------------------------------------------------------------
# the five named workloads
# ---------------------------------------------------------------------------

CONFIGS = {
    "c1": "tiny linear chain: B=1, K=4, V=1000, fp32, lambda=0, T=1",
    "c2": "single-request Llama-3-vocab chain: B=1, K=8, V=128256, bf16, lambda=0, T=1",
    "c3": "RAPID mixture batch: B=16, K=8, V=151936, bf16, lambda=0.3, T=1",
    "c4": "ragged batch: B=64, K_b~U{1..8}, V=128256, bf16, lambda=0, T=0.7",
    "c5": "draft trees: B=8, N=26 (depth 6, caps 4/3/2/1/1/1), V=128256, bf16",
}


def config(name: str, seed_offset: int = 0):
    """Inputs of a named workload; ``seed_offset`` selects another seeded draw."""
    c = int(name[1:])
    seed = 1000 + c + 7919 * seed_offset
    if name == "c1":
        return make_chain(seed, 1, 4, 1000, "fp32", sigma_t=2.0, sigma_q=1.0, zipf=False,
                          lam=0.0, temperature=1.0, name="c1")
    if name == "c2":
        return make_chain(seed, 1, 8, 128256, "bf16", sigma_t=3.0, sigma_q=1.0,
                          lam=0.0, temperature=1.0, name="c2")
    if name == "c3":
        return make_chain(seed, 16, 8, 151936, "bf16", sigma_t=3.0, sigma_q=0.5,
                          lam=0.3, temperature=1.0, name="c3")
    if name == "c4":
        return make_chain(seed, 64, 8, 128256, "bf16", sigma_t=3.0, sigma_q=(0.3, 2.0),
                          lam=0.0, temperature=0.7, ragged=True, k_min=1, name="c4")
    if name == "c5":
        return make_tree(seed, 8, 26, 128256, "bf16", depth=6, sigma_t=3.0, sigma_q=1.0,
                         lam=0.0, temperature=1.0, name="c5")
    raise KeyError(name)


def make_random_tree(seed: int, B: int, N: int, V: int, dtype: str = "fp32", *,
                     int_logits: bool = False, sharp: float = 0.05, sigma_q: float = 1.0,
                     lam: float = 0.0, temperature: float = 1.0, name: str = "rtree") -> TreeInputs:
    """Small random trees for edge cases: parent[i] ~ U{0..i}, node tokens drawn
    from the parent's target row at a low temperature ``sharp`` (so they often
    hit that row's most likely token).  ``int_logits`` draws integer logits in
    [-3, 3] to create many equal maxima."""
    s = _streams(seed)
    if int_logits:
        zt = s["target"].integers(-3, 4, size=(B, N + 1, V)).astype(np.float32)
    else:
        zt = s["target"].standard_normal((B, N + 1, V), dtype=np.float32) * np.float32(2.0)
    zq = zt + s["noise"].standard_normal((B, N + 1, V), dtype=np.float32) * np.float32(sigma_q)
    if dtype == "bf16":
        t_arr, q_arr = f32_to_bf16_bits(zt), f32_to_bf16_bits(zq)
        t_w = bf16_bits_to_f32(t_arr)
    else:
        t_arr, q_arr = zt, zq.astype(np.float32)
        t_w = t_arr
    parent = np.zeros((B, N), dtype=np.int32)
    node_token = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        for i in range(1, N + 1):
            parent[b, i - 1] = int(s["tree_shape"].integers(0, i))
            node_token[b, i - 1] = gumbel_max_sample(s["draft_tok"], t_w[b, parent[b, i - 1]], sharp)
    Dmax = max(1, max(int(tree_depths(parent[b]).max()) for b in range(B)))
    path = np.stack([seeded_path(s["tree_path"], parent[b], Dmax) for b in range(B)])
    u_acc = uniforms(s["u_accept"], (B, Dmax))
    u_smp = uniforms(s["u_sample"], (B,))
    return TreeInputs(name, dtype, t_arr, q_arr, parent, node_token, path, u_acc, u_smp,
                      float(lam), float(temperature), uniforms(s["u_node"], (B, N)))
