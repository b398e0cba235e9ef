"""fp64 CPU oracle of the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library
and its Python binding never import, call or link it, and it imports nothing
from them.

It is the plain, slow, sequential algorithm, one request at a time, in float64
on the exact widening of the inputs (bf16 and fp32 logits widen exactly; the
scalars lambda, T and the uniforms are the fp32 values the library receives,
widened).  Each function names the passage of the source pages it follows:

* [RAPID] "RAPID：基于检索增强的推测解码长上下文推理" (explainer of arXiv
  2502.20330), sections "2) 推理时知识迁移" (the mixture equation) and
  "3) 候选验证机制（伪代码）" (the verify loop).
* [SD] "大模型推理的Speculative Decoding原理详解", section "修改的拒绝采样"
  (two-branch rejection rule), "加速效果分析" (expected tokens per step),
  "批量投机" and "Tree Speculation".
* [EAGLE] "投机解码（EAGLE）：让小模型猜、大模型验，无损加速 LLM 生成",
  section "1. 为什么无损：接受概率的精巧设计" (residual max(0, p - q)),
  "核心思路" step 3 (greedy match) and "3. 验证阶段树形attention".

Readings where the pages are silent or disagree (temperature, bonus token,
uniform layout, tie rules, the tree encoding) are listed in the design notes;
each is marked "reading" below.

All functions are pinned by ``tests/test_oracle_pins.py``; the boundary-band
predicate that decides which requests a parity comparison may excuse, the
q(x) = 0 reading and the zero-residual fallback are pinned by
``tests/test_oracle_excusal.py``.  None is "parity unpinned".
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

#: half-width of the band around an acceptance ratio or a CDF boundary inside
#: which a uniform draw is reported as a boundary draw
FLAG_BAND = 1e-6


class InvalidRow(ValueError):
    """A logits row whose softmax is undefined (NaN, +inf, or every entry -inf)."""


def as_f32_scalar(x: float) -> float:
    """The fp32 value the library receives for a scalar argument, widened."""
    return float(np.float32(x))


# ---------------------------------------------------------------------------
# distributions
# ---------------------------------------------------------------------------


def softmax_T(z: np.ndarray, T: float) -> np.ndarray:
    """softmax(z / T) in fp64.

    [RAPID] pseudocode applies a softmax to each position's target and draft
    logits; the temperature T (reading) divides the logits of both models
    before that softmax.  The maximum is subtracted for range only; it cancels
    in the ratio.
    """
    y = np.asarray(z, dtype=np.float64) / float(T)
    m = y.max()                      # NaN anywhere makes the max NaN
    if not np.isfinite(m):
        raise InvalidRow("row holds NaN or +inf, or is all -inf")
    e = np.exp(y - m)
    return e / e.sum()


def mixture(p_t: np.ndarray, q: np.ndarray, lam: float) -> np.ndarray:
    """RAPID's inference-time knowledge transfer: p~ = (1 - lam) p_t + lam q.

    [RAPID] section "2) 推理时知识迁移", mixture equation; mixed in probability
    space (the pseudocode's logit-space form is the other reading, not taken).
    """
    return (1.0 - lam) * p_t + lam * q


def mixture_excess(p_t: np.ndarray, q: np.ndarray, lam: float) -> np.ndarray:
    """p~ - q of the probability-space mixture, written as (1 - lam)(p_t - q).

    [RAPID] section "2) 推理时知识迁移": p~ = (1 - lam) p_t + lam q, so
    p~ - q = (1 - lam)(p_t - q) exactly.  This form is exactly zero wherever
    p_t == q, as the mathematics says; the expanded form leaves rounding
    residue there, which a normalisation would turn into a spurious law.
    """
    return (1.0 - lam) * (p_t - q)


def enhanced_logits(zt: np.ndarray, zq: np.ndarray, lam: float) -> np.ndarray:
    """The RAPID pseudocode's logit-space mixture: (1 - lam) z_t + lam z_q.

    [RAPID] "3) 候选验证机制（伪代码）": ``enhanced_target = (1 - λ) *
    target_logits + λ * draft_logits``, then a softmax per position.  At
    lam = 0 and lam = 1 the other model's logits carry weight 0 and are left
    out (so a -inf there does not turn into NaN).  Where both logits are
    finite it is evaluated as z_q + (1 - lam)(z_t - z_q), the same number,
    which equals z_q exactly when z_t == z_q (the mixture of a model with
    itself is that model); elsewhere the expression as written.
    """
    zt = np.asarray(zt, dtype=np.float64)
    zq = np.asarray(zq, dtype=np.float64)
    if lam == 0.0:
        return zt.copy()
    if lam == 1.0:
        return zq.copy()
    fin = np.isfinite(zt) & np.isfinite(zq)
    with np.errstate(invalid="ignore"):
        return np.where(fin, zq + (1.0 - lam) * (zt - zq), (1.0 - lam) * zt + lam * zq)


def accept_prob(p_mix_x: float, q_x: float) -> float:
    """Acceptance probability of a drafted token x: min(1, p~(x) / q(x)).

    [RAPID] pseudocode ``accept_prob``; [SD] "修改的拒绝采样" and [EAGLE]
    section 1 state the same rule in two branches (p >= q accepts outright,
    otherwise accept with probability p / q).  Reading for q(x) = 0 (the draft
    could not have drawn x): accept iff p~(x) > 0.
    """
    if q_x == 0.0:
        return 1.0 if p_mix_x > 0.0 else 0.0
    return min(1.0, p_mix_x / q_x)


def residual_weights(p_mix: np.ndarray, q: np.ndarray, excess: Optional[np.ndarray] = None) -> np.ndarray:
    """Unnormalised law resampled after a rejection: max(0, p~ - q).

    [EAGLE] section 1 (resample from max(0, p - q)); [SD] "修改的拒绝采样"
    calls it the (p - q) distribution; the RAPID pseudocode's ``p_t - p_q`` is
    read as the same clipped difference, with p~ in place of p.  ``excess``,
    when given, is p~ - q already formed (``mixture_excess``).
    """
    return np.maximum(0.0, p_mix - q if excess is None else excess)


def inverse_cdf(w: np.ndarray, u: float):
    """Categorical draw from weights w with one uniform u in [0, 1).

    token = min{ j : F(j) > u },  F(j) = sum_{v <= j} w(v) / sum_v w(v).
    Zero-weight tokens are never chosen (F does not rise there).  Returns
    (token, F(token - 1), F(token)) with F(-1) = 0.
    """
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    total = c[-1]
    if not total > 0.0:
        raise ValueError("inverse_cdf: no positive weight")
    F = c / total
    hits = np.nonzero(F > u)[0]
    if len(hits):
        j = int(hits[0])
    else:                                    # u at or above F's last step by rounding
        j = int(np.nonzero(w > 0.0)[0][-1])
    lo = float(F[j - 1]) if j > 0 else 0.0
    return j, lo, float(F[j])


# ---------------------------------------------------------------------------
# one request
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class ChainResult:
    accepted: int              # accepted drafts n (0..k)
    tokens: List[int]          # n accepted drafts + 1 corrected or bonus token
    a: np.ndarray              # [k] acceptance probability of every position
    alpha: np.ndarray          # [k] sum_v min(p~, q): expected acceptance at each position
    bonus: bool                # True when every draft was accepted
    sample_row: int            # position whose distribution produced the last token
    F_lo: float                # F(token - 1) of that draw
    F_hi: float                # F(token)
    fallback: bool             # residual mass was zero; sampled p~ instead
    flagged: bool              # some draw lies within FLAG_BAND of its boundary


MIX_SPACES = ("prob", "logit")


def chain_verify_one(zt: np.ndarray, zq: np.ndarray, x, u_acc, u_s: float,
                     lam: float, T: float, space: str = "prob") -> ChainResult:
    """Verify one request's linear chain of k drafts.

    zt [k+1, V] target logits (row k serves the bonus token), zq [k, V] draft
    logits, x [k] drafted tokens, u_acc [k] acceptance uniforms, u_s the
    sampling uniform.

    [RAPID] "3) 候选验证机制（伪代码）": per position, softmax both rows, mix,
    test a uniform against min(1, p~/q), stop at the first rejection and
    resample there.  Reading: the comparison is strict (u < a); every position
    below k gets its acceptance probability reported, also past the first
    rejection; when all k drafts pass, one bonus token is drawn from the
    target's row k at temperature T (its draft row does not exist, so no
    mixture applies there); the one sampling uniform u_s serves whichever of
    the residual or bonus draws happens.

    ``space`` picks where the two models mix: "prob" is the mixture equation
    of [RAPID] section 2, p~ = (1 - lam) p_t + lam q; "logit" is the form the
    [RAPID] pseudocode writes, p~ = softmax(((1 - lam) z_t + lam z_q) / T).
    Either p~ then takes the target's place in the acceptance ratio, the
    residual and the fallback.
    """
    if space not in MIX_SPACES:
        raise ValueError(f"unknown mixture space {space!r}")
    lam = as_f32_scalar(lam)
    T = as_f32_scalar(T)
    u_s = float(np.float32(u_s))
    k = len(x)
    zt = np.asarray(zt, dtype=np.float64)
    zq = np.asarray(zq, dtype=np.float64)
    V = zt.shape[1]
    a = np.zeros(k)
    alpha = np.zeros(k)
    p_mix_rows, excess_rows = [], []
    for i in range(k):
        xi = int(x[i])
        if not 0 <= xi < V:
            raise ValueError(f"drafted token {xi} outside [0, {V})")
        q = softmax_T(zq[i], T)
        if space == "prob":
            p_t = softmax_T(zt[i], T)
            p_mix = mixture(p_t, q, lam)
            excess = mixture_excess(p_t, q, lam)
        else:
            p_mix = softmax_T(enhanced_logits(zt[i], zq[i], lam), T)
            excess = p_mix - q
        a[i] = accept_prob(p_mix[xi], q[xi])
        alpha[i] = np.minimum(p_mix, q).sum()
        p_mix_rows.append(p_mix)
        excess_rows.append(excess)

    n = k
    for i in range(k):
        if not float(np.float32(u_acc[i])) < a[i]:
            n = i
            break

    fallback = False
    if n < k:
        w = residual_weights(None, None, excess_rows[n])
        if not w.sum() > 0.0:                # reading: zero residual mass -> draw from p~
            w = p_mix_rows[n]
            fallback = True
    else:
        w = softmax_T(zt[k], T)
    tok, F_lo, F_hi = inverse_cdf(w, u_s)

    flagged = False
    for i in range(min(n + 1, k)):
        u = float(np.float32(u_acc[i]))
        if a[i] < 1.0 and abs(u - a[i]) < FLAG_BAND:
            flagged = True
    if (u_s - F_lo) < FLAG_BAND or (F_hi - u_s) < FLAG_BAND:
        flagged = True

    tokens = [int(t) for t in x[:n]] + [tok]
    return ChainResult(n, tokens, a, alpha, n == k, n, F_lo, F_hi, fallback, flagged)


@dataclasses.dataclass
class GreedyResult:
    accepted: int              # depth of the deepest accepted node
    tokens: List[int]          # tokens along the accepted path + the bonus argmax
    nodes: List[int]           # accepted node ids, root excluded, root -> leaf
    argmax: np.ndarray         # [N+1] target argmax of every row


def tree_greedy_one(zt: np.ndarray, parent, node_token) -> GreedyResult:
    """Greedy verification of one draft tree.

    [EAGLE] "核心思路" step 3: a draft is kept when it is the target's most
    likely token; [SD] "Tree Speculation" and [EAGLE] "3. 验证阶段树形attention":
    the whole tree is scored at once and a node sees only its ancestors.

    Encoding (reading): node 0 is the root; node i (1..N) has token
    node_token[i-1], parent parent[i-1] < i and target row i.  Row r holds the
    target's logits for the token that follows node r.  Node i is accepted iff
    its parent is accepted and its token equals the argmax of its parent's row
    (lowest token id on ties).  The deepest accepted node wins (lowest node id
    on ties); the bonus token is the argmax of its row.
    """
    zt = np.asarray(zt, dtype=np.float64)
    N = len(parent)
    for r in range(N + 1):
        if np.isnan(zt[r]).any():
            raise InvalidRow(f"row {r} holds NaN")
    am = np.array([int(np.argmax(zt[r])) for r in range(N + 1)])
    ok = [True] + [False] * N
    depth = [0] * (N + 1)
    for i in range(1, N + 1):
        p = int(parent[i - 1])
        if not 0 <= p < i:
            raise ValueError(f"parent of node {i} is {p}, not in [0, {i})")
        depth[i] = depth[p] + 1
        ok[i] = ok[p] and int(node_token[i - 1]) == int(am[p])
    best = 0
    for i in range(1, N + 1):
        if ok[i] and depth[i] > depth[best]:
            best = i
    nodes = []
    v = best
    while v != 0:
        nodes.append(v)
        v = int(parent[v - 1])
    nodes.reverse()
    tokens = [int(node_token[v - 1]) for v in nodes] + [int(am[best])]
    return GreedyResult(len(nodes), tokens, nodes, am)


def path_rows(path) -> List[int]:
    """Leading node ids of a -1 terminated path."""
    out = []
    for v in path:
        if int(v) < 0:
            break
        out.append(int(v))
    return out


def tree_path_one(zt: np.ndarray, zq: np.ndarray, node_token, path, u_acc, u_s: float,
                  lam: float, T: float, space: str = "prob") -> ChainResult:
    """Stochastic verification along one root->leaf path of a draft tree.

    Reading: chain acceptance ([RAPID] verify loop) along the nodes
    n_1..n_d of ``path``.  Position j drafts the token of node n_{j+1}, drawn
    from the draft row of its parent n_j (n_0 = root); it is tested against
    target row n_j and draft row n_j.  The bonus row is target row n_d.
    """
    nodes = path_rows(path)
    d = len(nodes)
    rows = [0] + nodes
    x = [int(node_token[v - 1]) for v in nodes]
    return chain_verify_one(np.asarray(zt)[rows], np.asarray(zq)[rows[:d]], x,
                            np.asarray(u_acc)[:d], u_s, lam, T, space)


@dataclasses.dataclass
class TreeMask:
    mask: np.ndarray           # [N+1, N+1] bool: row i may attend to column j
    depth: np.ndarray          # [N+1] int: edges from the root
    bad: bool                  # some parent was out of range


def tree_attention_mask_one(parent) -> TreeMask:
    """Tree-attention mask of one draft tree.

    [EAGLE] "3. 验证阶段树形attention": to verify a whole tree in one target
    pass, every candidate token may only see its own ancestor path.  Reading:
    position i (node i; 0 is the root) sees itself and every ancestor, the
    root included; depth[i] is the number of edges from the root (the offset
    of node i's position after the root).  A node whose parent is not in
    [0, i) is read as a child of the root and reported as bad.
    """
    N = len(parent)
    mask = np.zeros((N + 1, N + 1), dtype=bool)
    depth = np.zeros(N + 1, dtype=np.int64)
    par = [-1] + [int(p) for p in parent]
    bad = False
    for i in range(1, N + 1):
        if not 0 <= par[i] < i:
            par[i] = 0
            bad = True
    for i in range(N + 1):
        v = i
        while v >= 0:                 # walk to the root; parents decrease, so this ends
            mask[i, v] = True
            v = par[v]
        depth[i] = mask[i].sum() - 1
    return TreeMask(mask, depth, bad)


def pack_mask_rows(mask: np.ndarray, words: int) -> np.ndarray:
    """Bit j of 32-bit word j // 32 of a row holds column j (little-endian)."""
    R, C = mask.shape
    out = np.zeros((R, words), dtype=np.uint32)
    for j in range(C):
        out[:, j // 32] |= mask[:, j].astype(np.uint32) << np.uint32(j % 32)
    return out


@dataclasses.dataclass
class MultiResult:
    accepted: int              # depth of the deepest accepted node
    tokens: List[int]          # accepted nodes' tokens + the final (residual or bonus) token
    nodes: List[int]           # accepted node ids, root -> deepest
    a: np.ndarray              # [N] acceptance probability of each tested node, -1 if untested
    tested: List[int]          # node ids in the order they were tested
    bonus: bool                # the walk ended at a node without (visible) children
    fallback: bool             # a residual had zero mass; its current target was sampled instead
    flagged: bool              # some draw lies within FLAG_BAND of its boundary


def tree_multi_one(zt: np.ndarray, zq: np.ndarray, parent, node_token, u_acc, u_s: float,
                   lam: float, T: float, space: str = "prob",
                   Dmax: Optional[int] = None) -> MultiResult:
    """Stochastic verification of a whole draft tree, retrying siblings.

    [SD] "Tree Speculation": several candidates per position are verified
    together, so when one branch is rejected another may still be accepted;
    the pages give no rule for this.  Reading (the chain rule applied again
    to what a rejection leaves): at node u with target r = p~ at row u (either
    mixture space) and draft q at row u, the children are tested in node order;
    child c with token x is accepted iff u_acc[c-1] < min(1, r(x) / q(x)) (the
    chain test, same q(x) = 0 reading); after a rejection
    r <- max(0, r - q) / sum max(0, r - q) (the chain's residual, now the
    target of the next child).  The first accepted child becomes u; if every
    child is rejected one token is drawn from the final r by inverse CDF with
    u_s; at a node without children (or at depth Dmax) the bonus token is
    drawn from the target's own softmax(z_t[u] / T).  When the children's
    tokens are independent draws from q of their parent, every retry is a
    fresh chain step aimed at the residual, so the emitted token follows p~
    (the same argument as the chain's).  Zero residual mass (rounding only):
    draw from the current r and report a fallback.
    """
    if space not in MIX_SPACES:
        raise ValueError(f"unknown mixture space {space!r}")
    lam = as_f32_scalar(lam)
    T = as_f32_scalar(T)
    u_s = float(np.float32(u_s))
    zt = np.asarray(zt, dtype=np.float64)
    zq = np.asarray(zq, dtype=np.float64)
    N = len(parent)
    V = zt.shape[1]
    children = [[] for _ in range(N + 1)]
    for i in range(1, N + 1):
        p = int(parent[i - 1])
        if not 0 <= p < i:
            raise ValueError(f"parent of node {i} is {p}, not in [0, {i})")
        children[p].append(i)
    a_out = np.full(N, -1.0)
    tested, nodes = [], []
    flagged = fallback = False
    u, depth = 0, 0
    while True:
        kids = children[u] if (Dmax is None or depth < Dmax) else []
        if not kids:
            tok, F_lo, F_hi = inverse_cdf(softmax_T(zt[u], T), u_s)
            bonus = True
            break
        q = softmax_T(zq[u], T)
        if space == "prob":
            p_t = softmax_T(zt[u], T)
            r = mixture(p_t, q, lam)
            excess = mixture_excess(p_t, q, lam)        # r - q while r is p~
        else:
            r = softmax_T(enhanced_logits(zt[u], zq[u], lam), T)
            excess = r - q
        nxt = None
        for c in kids:
            x = int(node_token[c - 1])
            if not 0 <= x < V:
                raise ValueError(f"token {x} of node {c} outside [0, {V})")
            a = accept_prob(r[x], q[x])
            a_out[c - 1] = a
            tested.append(c)
            uc = float(np.float32(u_acc[c - 1]))
            if a < 1.0 and abs(uc - a) < FLAG_BAND:
                flagged = True
            if uc < a:
                nxt = c
                break
            w = residual_weights(r, q, excess)
            excess = None                               # later residuals: r - q itself
            W = w.sum()
            if not W > 0.0:
                fallback = True
                break
            r = w / W
        if nxt is not None:
            nodes.append(nxt)
            u, depth = nxt, depth + 1
            continue
        tok, F_lo, F_hi = inverse_cdf(r, u_s)
        bonus = False
        break
    if (u_s - F_lo) < FLAG_BAND or (F_hi - u_s) < FLAG_BAND:
        flagged = True
    tokens = [int(node_token[c - 1]) for c in nodes] + [tok]
    return MultiResult(len(nodes), tokens, nodes, a_out, tested, bonus, fallback, flagged)


# ---------------------------------------------------------------------------
# batches ([SD] "批量投机": every request is verified independently)
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class BatchResult:
    accepted: np.ndarray       # [B] int32
    out_tokens: np.ndarray     # [B, W] int32, -1 padded
    accept_prob: np.ndarray    # [B, K] float64, 0 beyond each request's length
    flagged: np.ndarray        # [B] bool
    details: list


def chain_verify(target, draft, tokens, draft_len: Optional[np.ndarray], u_accept, u_sample,
                 lam: float, T: float, requests=None, space: str = "prob") -> BatchResult:
    """All requests of a chain batch.  target [B,K+1,V], draft [B,K,V] (float arrays)."""
    B, K = tokens.shape
    req = range(B) if requests is None else requests
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, K + 1), -1, dtype=np.int32)
    ap = np.zeros((B, K))
    flag = np.zeros(B, dtype=bool)
    det = [None] * B
    for b in req:
        k = K if draft_len is None else int(draft_len[b])
        r = chain_verify_one(target[b, :k + 1], draft[b, :k], tokens[b, :k], u_accept[b, :k],
                             u_sample[b], lam, T, space)
        acc[b] = r.accepted
        out[b, :len(r.tokens)] = r.tokens
        ap[b, :k] = r.a
        flag[b] = r.flagged
        det[b] = r
    return BatchResult(acc, out, ap, flag, det)


def tree_greedy(target, parent, node_token, Dmax: int, requests=None):
    """Greedy verification of a batch of trees; returns (accepted, out_tokens, nodes)."""
    B, N = parent.shape
    req = range(B) if requests is None else requests
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, Dmax + 1), -1, dtype=np.int32)
    nodes = np.full((B, Dmax), -1, dtype=np.int32)
    for b in req:
        r = tree_greedy_one(target[b], parent[b], node_token[b])
        acc[b] = r.accepted
        out[b, :len(r.tokens)] = r.tokens
        nodes[b, :len(r.nodes)] = r.nodes
    return acc, out, nodes


def tree_path(target, draft, node_token, path, u_accept, u_sample, lam, T,
              requests=None, space: str = "prob") -> BatchResult:
    B, Dmax = path.shape
    req = range(B) if requests is None else requests
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, Dmax + 1), -1, dtype=np.int32)
    ap = np.zeros((B, Dmax))
    flag = np.zeros(B, dtype=bool)
    det = [None] * B
    for b in req:
        r = tree_path_one(target[b], draft[b], node_token[b], path[b], u_accept[b],
                          u_sample[b], lam, T, space)
        acc[b] = r.accepted
        out[b, :len(r.tokens)] = r.tokens
        ap[b, :len(r.a)] = r.a
        flag[b] = r.flagged
        det[b] = r
    return BatchResult(acc, out, ap, flag, det)


def tree_attention_mask(parent, words: int):
    """A batch of trees: (mask [B, N+1, words] uint32, depth [B, N+1], bad [B])."""
    B, N = parent.shape
    mask = np.zeros((B, N + 1, words), dtype=np.uint32)
    depth = np.zeros((B, N + 1), dtype=np.int64)
    bad = np.zeros(B, dtype=bool)
    for b in range(B):
        r = tree_attention_mask_one(parent[b])
        mask[b] = pack_mask_rows(r.mask, words)
        depth[b] = r.depth
        bad[b] = r.bad
    return mask, depth, bad


def tree_multi(target, draft, parent, node_token, u_accept, u_sample, lam, T, Dmax: int,
               space: str = "prob", requests=None):
    """A batch of multi-branch tree verifications: (accepted, out_tokens [B, Dmax+1],
    nodes [B, Dmax], accept_prob [B, N], flagged [B], details)."""
    B, N = parent.shape
    req = range(B) if requests is None else requests
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, Dmax + 1), -1, dtype=np.int32)
    nodes = np.full((B, Dmax), -1, dtype=np.int32)
    ap = np.full((B, N), -1.0)
    flag = np.zeros(B, dtype=bool)
    det = [None] * B
    for b in req:
        r = tree_multi_one(target[b], draft[b], parent[b], node_token[b], u_accept[b],
                           u_sample[b], lam, T, space, Dmax)
        acc[b] = r.accepted
        out[b, :len(r.tokens)] = r.tokens
        nodes[b, :len(r.nodes)] = r.nodes
        ap[b] = r.a
        flag[b] = r.flagged
        det[b] = r
    return acc, out, nodes, ap, flag, det

