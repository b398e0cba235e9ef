// Multi-branch stochastic verification of draft trees on gfx950.
//
// Method (cited by page title and section):
//   "大模型推理的Speculative Decoding原理详解", "Tree Speculation": a tree of
//     candidates is verified together, so a rejected branch may leave a
//     sibling accepted (the page gives no rule).
//   Same page, "修改的拒绝采样", and the EAGLE explainer, "1. 为什么无损": a
//     draft x ~ q is kept with probability min(1, p(x)/q(x)), else the token
//     is drawn from max(0, p - q) normalised.
//   RAPID explainer (arXiv 2502.20330), "2) 推理时知识迁移" and
//     "3) 候选验证机制（伪代码）": p is the mixture p~ (probability or logit
//     space).
//
// Rule (applying the chain rule again to what a rejection leaves): at node u
// the children are tested in node order against a target r, first p~ of
// row u; after a rejection r <- max(0, r - q) / sum, the next child's
// target.  The first accepted child becomes u; if every child is rejected one
// token is drawn from the last residual; a node without children (or at depth
// Dmax) emits the bonus token from the target's own softmax(z/T).
//
// G cooperating 512-thread blocks walk each tree (G up to
// SV_MAX_BLOCKS_PER_TREE, as many as fit the GPU with the other trees'
// blocks), block g owning vocabulary slice g.
// Every block takes every decision of the walk from the same combined values.
// The row statistics of every tree row (but the draft rows of childless
// nodes, which no test reads) come from a row-statistics launch before the
// walk (chunk partials, combined by the walk in fp64): a small
// tree combines all its rows, loads every node's logits at its parent's rows
// and forms each first child's test when it starts; a larger one combines a
// node's children's rows while the first child is tested.  Each step that
// needs a sum over the vocabulary is a pass of every block over its slice of
// the node's two rows, combined at a barrier of the tree's blocks: the
// residual after a rejection (written to a ping-pong fp32 buffer of the
// workspace with its fp64 mass), and an inverse CDF over slice totals, then
// within the slice holding the draw.  Acceptance of a first child uses the
// gathered logits in fp64; a later child forms the residual at its token again
// with the residual pass's own operations (bitwise the stored value), so no
// block reads another block's slice of the residual.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "sv_common.hpp"
#include "sv_device.hpp"

namespace sv {

constexpr int kMB = 512;                  // threads of a walk block (1024 spilled registers)
constexpr int kMW = kMB / kWave;          // its waves
constexpr int kMU = 2;                    // tiles of a pass in flight per thread
constexpr int kMNodes = SV_MAX_TREE_NODES + 1;
constexpr int kSpec = (kMB / 64 - 2) / 2;  // statistics slots filled ahead of need (waves 2 and up, two per node)
constexpr int kTabNodes = 64;              // trees of at most this many nodes ...
constexpr int kTabParts = 2048;            // ... and chunk partials: every node's statistics at the start
constexpr int kMaxG = SV_MAX_BLOCKS_PER_TREE;   // blocks per tree at most
constexpr int kSlot = 4;                  // doubles a block publishes per barrier
constexpr int kSpinLimit = 1 << 20;       // polls of a barrier before it is given up (about 1 s)

struct MultiArgs {
    const char *tgt, *drf;
    int64_t ld_t, ld_q;
    int elem;
    int B, N, V, Dmax;
    const int32_t *parent, *node_token;
    const float *u_accept, *u_sample;
    float lam, c_hi, c_lo;
    double c_d, al, be;                   // log2(e)/T; logit space: (1 - lambda) c, lambda c
    float d_hi, d_lo;                     // c (or (1 - lambda) c in logit space) as hi + lo
    int space;                            // 0 probability space, 1 logit space
    int32_t *accepted, *out_tokens, *accepted_nodes;
    float *accept_prob;                   // [B, N] or NULL
    int32_t *status;
    float *buf;                           // [B, 2, Vp] residual ping-pong
    int Vp;                               // residual row stride: V rounded up to 8 floats
    int G;                                // blocks per tree; block g owns vocabulary slice g
    unsigned long long *pub;              // [B, G, 3, kSlot] values published at a barrier (bit patterns)
    unsigned *ticket;                     // start-order counter that assigns each block its (tree, slice)
    const Part *part1;                    // [B, N+1, 2, C1]: chunk partials of every row's statistics
    int C1;
    float mx[4];                          // logit space: (1 - lambda) c and lambda c as hi + lo
};

struct MultiShared {
    int par[kMNodes];                     // parent of each node (as given)
    int head[kMNodes];                    // first child of a node (node order), -1: none
    int next[kMNodes];                    // next sibling, -1: none
    int tok[kMNodes];
    double zs[kMNodes];                   // residual masses of the current node, in order
    float czt[kMNodes], czq[kMNodes];     // target / draft logit of each child's token at its parent's rows
    float ua[kMNodes];                    // acceptance uniform of each node's draft
    int path[SV_MAX_POSITIONS + 1];
    double red[kMW];
    float redf[kMW];
    int redi[kMW];
    double sA, SA, sB, SB;                // statistics of the two rows (A: target or mixed)
    double iA, iB;                        // 1 / SA, 1 / SB
    float k0;                             // q(v) / A(v) = 2^((z_q - z_t) d + k0)
    double gath[kMaxG][kSlot];            // every block's published values after a barrier
    // statistics combined ahead of need: slot k holds the rows (A, B) of node
    // spec_node[k] (-1: none) as shift and sum
    int spec_node[kSpec];
    double spec_s[kSpec][2], spec_S[kSpec][2];
    int spec_hit;
    // small trees: every row's chunk partials staged, then every node's rows
    float tab_ps[kTabParts];
    double tab_pS[kTabParts];
    double tab_s[kTabNodes][2], tab_S[kTabNodes][2];
    double tab_iA[kTabNodes], tab_iB[kTabNodes];    // 1 / S of each row
    float tab_k0[kTabNodes];
    double tab_acc[kTabNodes];            // a first child's acceptance probability at its parent
    int tab_fl[kTabNodes];                // and the flags its test raises
    int flags, decision, token, broken;
    int tree, slice;                      // this block's role, from its start-order ticket
};

// ---- block reductions (every thread calls; results uniform) ---------------

__device__ __forceinline__ float mblock_max(float v, MultiShared &sh) {
    v = wave_max(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) sh.redf[w] = v;
    __syncthreads();
    float r = sh.redf[0];
    for (int i = 1; i < kMW; ++i) r = fmaxf(r, sh.redf[i]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ int mblock_max_i(int v, MultiShared &sh) {
    v = -wave_min_i(-v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) sh.redi[w] = v;
    __syncthreads();
    int r = sh.redi[0];
    for (int i = 1; i < kMW; ++i) r = max(r, sh.redi[i]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ double mblock_sum(double v, MultiShared &sh) {
    v = wave_sum_d(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) sh.red[w] = v;
    __syncthreads();
    double r = 0.0;
    for (int i = 0; i < kMW; ++i) r += sh.red[i];
    __syncthreads();
    return r;
}

// Inclusive / exclusive scan of one double per thread in thread order,
// offset by carry; every exclusive prefix is bitwise the previous thread's
// inclusive one (the wave bases are formed by the same additions).
__device__ __forceinline__ Scan mblock_scan(double v, double carry, MultiShared &sh) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const double x = wave_scan_d(v);
    if (lane == kWave - 1) sh.red[w] = x;
    __syncthreads();
    double base = 0.0, tot = 0.0;
    for (int i = 0; i < kMW; ++i) {
        if (i == w) base = tot;
        tot = tot + sh.red[i];
    }
    const double prev = dpp_shift_d<kDppWaveShr1, 0xF, 0xF>(x);
    Scan s;
    s.incl = carry + (base + x);
    s.excl = carry + ((lane == 0) ? base : (base + prev));
    s.total = carry + tot;
    __syncthreads();
    return s;
}

// ---- the blocks of one tree -------------------------------------------------
//
// Block g of a tree owns the contiguous vocabulary slice g (whole 16-byte
// vectors, in index order) for every pass.  The blocks take the same
// decisions from the same combined values, so they meet the same barriers.
// Values cross blocks only through agent-scope relaxed atomics (write-through
// stores, coherent loads), and every published value marks its own arrival:
// a block's slot reads as an empty marker (a signalling-NaN bit pattern that
// no arithmetic produces) until the block writes the value, and the readers
// poll the values themselves, one thread per value, so a barrier costs one
// store and one load round trip.  Slots rotate over three barriers: after
// barrier k a block empties the slot it filled for barrier k - 1 (every
// reader has consumed it, since each reader published for barrier k after
// reading it) for use at barrier k + 2, and it drains that store before it
// publishes for barrier k + 1, so a reader that has passed barrier k + 1
// finds the slot empty or holding the barrier-(k + 2) value.
//
// A block's role (tree, slice) is not its grid index but the ticket it takes
// from a counter when it starts: ticket k is tree k / G, slice k % G.  Only
// running blocks hold tickets and tickets are handed out in order, so every
// tree below the newest ticket's has all its blocks running or done, and at
// most one tree is still missing blocks.  The complete trees finish and free
// their compute units, and the next blocks to start complete the last tree:
// the walk progresses whenever G blocks fit on the GPU beside other work,
// whatever the grid size (a grid wider than the GPU runs its trees in
// rounds).  A poll still gives up after kSpinLimit rounds, marking the block
// broken (SV_DATA_SYNC), so every wave ends in any case.

struct Slice {
    int lo, hi;                            // vectors [lo, hi)
};

__device__ __forceinline__ Slice my_slice(const MultiArgs &a, const MultiShared &sh, int nvec) {
    const int g = sh.slice;
    const int per = (nvec + a.G - 1) / a.G;
    Slice s;
    s.lo = min(g * per, nvec);
    s.hi = min(s.lo + per, nvec);
    return s;
}

constexpr unsigned long long kEmpty = 0x7FF0DEAD5EED1234ull;   // an empty slot (a signalling NaN)
constexpr int kRot = 3;                                            // slots per block, used in rotation

__device__ __forceinline__ unsigned long long *pub_slot(const MultiArgs &a, const MultiShared &sh, int g,
                                                        int phase) {
    const int b = sh.tree;
    return a.pub + ((int64_t(b) * a.G + g) * kRot + (phase % kRot)) * kSlot;
}

// Thread 0 publishes v[0..n) for the barrier that ends phase + 1, once its
// earlier stores (the emptying of this slot) have drained.
__device__ __forceinline__ void publish_vals(const MultiArgs &a, const MultiShared &sh, int phase, const double *v,
                                             int n) {
    if (threadIdx.x != 0) return;
    unsigned long long *p = pub_slot(a, sh, sh.slice, phase + 1);
    __builtin_amdgcn_s_waitcnt(0);
    for (int j = 0; j < n; ++j)
        __hip_atomic_store(&p[j], static_cast<unsigned long long>(__double_as_longlong(v[j])), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// The tree's barrier; then sh.gath holds every block's published values.
// Every thread calls it with the same phase count, which it advances.  It
// starts with a block barrier: the polling threads overwrite sh.gath, which
// other waves of the block may still be reading from the barrier before.
__device__ void tree_barrier(const MultiArgs &a, MultiShared &sh, int &phase, int n) {
    __syncthreads();
    ++phase;
    if (static_cast<int>(threadIdx.x) < a.G * n) {
        const int g = static_cast<int>(threadIdx.x) / n, j = static_cast<int>(threadIdx.x) % n;
        const unsigned long long *p = &pub_slot(a, sh, g, phase)[j];
        unsigned long long w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int polls = 0;
        while (w == kEmpty && !sh.broken) {
            __builtin_amdgcn_s_sleep(1);
            if (++polls > kSpinLimit) {
                sh.broken = 1;
                break;
            }
            w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        sh.gath[g][j] = __longlong_as_double(static_cast<long long>(w));
    }
    __syncthreads();
    // every block has read this block's slot of the barrier before this one:
    // empty it for the barrier after the next
    if (threadIdx.x == 0) {
        unsigned long long *mine = pub_slot(a, sh, sh.slice, phase + 2);
        for (int j = 0; j < kSlot; ++j) __hip_atomic_store(&mine[j], kEmpty, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---- element values -----------------------------------------------------

template <class DT>
struct RowPair {
    const char *t, *q;
    int V;
};

// 2^(z c - s) with c = c_hi + c_lo
__device__ __forceinline__ float m_pow2(float z, float c_hi, float c_lo, float s) {
    return __builtin_amdgcn_exp2f(fmaf(z, c_lo, fmaf(z, c_hi, -s)));
}
// 2^(alpha z_t + beta z_q - s), the exponent formed as the row-statistics
// launch forms it (so the node's sums and its elements agree)
__device__ __forceinline__ float m_pow2_mixed(float zt, float zq, const float (&mx)[4], float s) {
    return __builtin_amdgcn_exp2f(mixed_expo(zt, zq, mx, s));
}

// p~(v) and q(v) of one element from its logits and the node's statistics
template <class DT>
__device__ __forceinline__ void m_probs(const MultiArgs &a, const MultiShared &sh, float zt, float zq,
                                        double &pm, double &q) {
    const double iA = sh.iA, iB = sh.iB;
    q = static_cast<double>(m_pow2(zq, a.c_hi, a.c_lo, static_cast<float>(sh.sB))) * iB;
    if (a.space == 1) {
        pm = static_cast<double>(m_pow2_mixed(zt, zq, a.mx, static_cast<float>(sh.sA))) * iA;
    } else {
        const double pt = static_cast<double>(m_pow2(zt, a.c_hi, a.c_lo, static_cast<float>(sh.sA))) * iA;
        pm = (1.0 - static_cast<double>(a.lam)) * pt + static_cast<double>(a.lam) * q;
    }
}

// The first residual at a node, max(0, p~(v) - q(v)), as an fp32 weight:
// (1 - lambda) p_t(v) max(0, 1 - q(v)/p_t(v)) in probability space (the
// mixture equation gives p~ - q = (1 - lambda)(p_t - q)), p~(v) max(0,
// 1 - q(v)/p~(v)) in logit space, with the ratio 2^e, e = (z_q - z_t) d + k0
// (sv_device one_minus_exp2: error relative to the weight, however close the
// rows are).  The residual pass and the child tests both form it here.
__device__ __forceinline__ float first_residual(const MultiArgs &a, const MultiShared &sh, float zt, float zq) {
    const float d = zq - zt;
    const float g = one_minus_exp2(fmaf(d, a.d_hi, fmaf(d, a.d_lo, sh.k0)));
    if (a.space == 1)
        return static_cast<float>(static_cast<double>(m_pow2_mixed(zt, zq, a.mx, static_cast<float>(sh.sA))) *
                                  sh.iA * static_cast<double>(g));
    const double pt = static_cast<double>(m_pow2(zt, a.c_hi, a.c_lo, static_cast<float>(sh.sA))) * sh.iA;
    return static_cast<float>((1.0 - static_cast<double>(a.lam)) * pt * static_cast<double>(g));
}

// ---- passes ----------------------------------------------------------------

// Row statistics of the node's rows: A = target (probability space) or the
// mixed logits (logit space), B = draft; with target_only, A alone (the bonus
// row).  Per thread a running integer shift and fp64 sum, then block-wide.
template <class DT>
__device__ void pass_stats(const MultiArgs &a, MultiShared &sh, int &phase, const char *row_t,
                           const char *row_q, bool target_only) {
    constexpr int VEC = DT::kVec;
    const int V = a.V;
    const int nvec = (V + VEC - 1) / VEC;
    const Slice sl = my_slice(a, sh, nvec);
    float sa = -INFINITY, sb = -INFINITY;
    double aa = 0.0, ab = 0.0;
    const bool mixed = !target_only && a.space == 1;
    for (int g0 = sl.lo; g0 < sl.hi; g0 += kMB * kMU) {
        u32x4 dt[kMU], dq[kMU];
#pragma unroll
        for (int k = 0; k < kMU; ++k) {
            // vectors past the slice read as -inf (their weights are 0)
            const int gv = g0 + k * kMB + static_cast<int>(threadIdx.x);
            dt[k] = load_row_vec<DT, false>(row_t, gv < sl.hi ? gv : nvec, V);
            if (!target_only) dq[k] = load_row_vec<DT, false>(row_q, gv < sl.hi ? gv : nvec, V);
        }
#pragma unroll
        for (int k = 0; k < kMU; ++k) {
            float ft[VEC], fq[VEC];
            DT::unpack(dt[k], ft);
            float mt = -INFINITY, mq = -INFINITY;
            for (int e = 0; e < VEC; ++e) mt = fmaxf(mt, ft[e]);
            if (!target_only) {
                DT::unpack(dq[k], fq);
                for (int e = 0; e < VEC; ++e) mq = fmaxf(mq, fq[e]);
            }
            // row A
            float cand;
            if (mixed) {
                cand = (mt == -INFINITY || mq == -INFINITY)
                           ? -INFINITY
                           : static_cast<float>(ceil(a.al * static_cast<double>(mt) + a.be * static_cast<double>(mq)));
            } else {
                cand = (mt == -INFINITY) ? -INFINITY : ceilf(mt * a.c_hi);
            }
            float sn = fmaxf(sa, cand);
            aa *= pow2_shift_d(sa == -INFINITY ? 0.0 : static_cast<double>(sa) - static_cast<double>(sn));
            sa = sn;
            const float su = (sa == -INFINITY) ? 0.0f : sa;
            float acc = 0.0f;
            for (int e = 0; e < VEC; ++e)
                acc += mixed ? m_pow2_mixed(ft[e], fq[e], a.mx, su) : m_pow2(ft[e], a.c_hi, a.c_lo, su);
            aa += static_cast<double>(acc);
            if (!target_only) {
                const float cq = (mq == -INFINITY) ? -INFINITY : ceilf(mq * a.c_hi);
                sn = fmaxf(sb, cq);
                ab *= pow2_shift_d(sb == -INFINITY ? 0.0 : static_cast<double>(sb) - static_cast<double>(sn));
                sb = sn;
                const float sq = (sb == -INFINITY) ? 0.0f : sb;
                float accq = 0.0f;
                for (int e = 0; e < VEC; ++e) accq += m_pow2(fq[e], a.c_hi, a.c_lo, sq);
                ab += static_cast<double>(accq);
            }
        }
    }
    const float ma = mblock_max(sa, sh);
    const double SA = mblock_sum(sa == -INFINITY ? 0.0 : aa * pow2_shift_d(static_cast<double>(sa) - static_cast<double>(ma)), sh);
    double SB = 1.0;
    float mb = 0.0f;
    if (!target_only) {
        mb = mblock_max(sb, sh);
        SB = mblock_sum(sb == -INFINITY ? 0.0 : ab * pow2_shift_d(static_cast<double>(sb) - static_cast<double>(mb)), sh);
    }
    // the tree's rows: combine the blocks' (shift, sum) pairs in slice order
    const double mine[kSlot] = {static_cast<double>(ma), SA, static_cast<double>(mb), SB};
    publish_vals(a, sh, phase, mine, 4);
    tree_barrier(a, sh, phase, 4);
    double tA = -INFINITY, tB = -INFINITY;
    for (int g = 0; g < a.G; ++g) {
        tA = fmax(tA, sh.gath[g][0]);
        tB = fmax(tB, sh.gath[g][2]);
    }
    double SAt = 0.0, SBt = 0.0;
    for (int g = 0; g < a.G; ++g) {
        if (sh.gath[g][0] != -INFINITY) SAt += sh.gath[g][1] * pow2_shift_d(sh.gath[g][0] - tA);
        if (sh.gath[g][2] != -INFINITY) SBt += sh.gath[g][3] * pow2_shift_d(sh.gath[g][2] - tB);
    }
    if (threadIdx.x == 0) {
        sh.sA = tA;
        sh.SA = SAt;
        sh.sB = target_only ? 0.0 : tB;
        sh.SB = target_only ? 1.0 : SBt;
        sh.iA = 1.0 / SAt;
        sh.iB = target_only ? 1.0 : 1.0 / SBt;
        sh.k0 = target_only ? 0.0f : static_cast<float>((tA - tB) + log2(SAt / SBt));
    }
    __syncthreads();
}

// The statistics of node u's rows from the chunk partials of the row-statistics
// launch that precedes the walk (one position per row of the tree): wave 0
// combines row A (the target, or the logit-space mixture), wave 1 the draft
// row, in fp64 over the chunks in order.  No barrier between the tree's blocks:
// each combines the same partials the same way.  target_only: row A alone.
// One row's (shift, sum) from its chunk partials, by one whole wave (results
// uniform over the wave): row 0 is A, row 1 is B of node u.
__device__ __forceinline__ void row_combine(const MultiArgs &a, int b, int u, int row, float &smax_out,
                                            double &S_out) {
    const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
    const Part *p = a.part1 + ((int64_t(b) * (a.N + 1) + u) * 2 + row) * a.C1;
    float smax = -INFINITY;
    for (int c = lane; c < a.C1; c += kWave) smax = fmaxf(smax, p[c].s);
    smax = wave_max(smax);
    double S = 0.0;
    for (int c = lane; c < a.C1; c += kWave) {
        const Part q = p[c];
        if (q.s != -INFINITY) S += q.S * pow2_shift_d(static_cast<double>(q.s) - static_cast<double>(smax));
    }
    smax_out = smax;
    S_out = wave_sum_d(S);
}

// The node's statistics in shared memory from its rows' (shift, sum); one thread.
__device__ __forceinline__ void set_stats(MultiShared &sh, double tA, double SAt, double tB, double SBt,
                                          bool target_only) {
    if (target_only) {
        tB = 0.0;
        SBt = 1.0;
    }
    sh.sA = tA;
    sh.SA = SAt;
    sh.sB = tB;
    sh.SB = SBt;
    sh.iA = 1.0 / SAt;
    sh.iB = 1.0 / SBt;
    sh.k0 = target_only ? 0.0f : static_cast<float>((tA - tB) + log2(SAt / SBt));
}

__device__ void load_stats(const MultiArgs &a, MultiShared &sh, int b, int u, bool target_only) {
    const int wv = static_cast<int>(threadIdx.x) / kWave, lane = static_cast<int>(threadIdx.x) & (kWave - 1);
    if (wv == 0 || (wv == 1 && !target_only)) {
        float smax;
        double S;
        row_combine(a, b, u, wv, smax, S);
        if (lane == 0) {
            sh.red[wv] = S;
            sh.redf[wv] = smax;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0)
        set_stats(sh, sh.redf[0], sh.red[0], target_only ? 0.0 : static_cast<double>(sh.redf[1]),
                  target_only ? 1.0 : sh.red[1], target_only);
    __syncthreads();
}

// Statistics ahead of need: waves 2 .. 2 kSpec + 1 combine the rows of the
// given nodes (two waves per node) into the slots, with no barrier: the
// caller's next block barrier publishes them.  Thread 0 records the nodes.
__device__ __forceinline__ void spec_stats(const MultiArgs &a, MultiShared &sh, int b, const int (&nodes)[kSpec]) {
    const int wv = static_cast<int>(threadIdx.x) / kWave, lane = static_cast<int>(threadIdx.x) & (kWave - 1);
    if (threadIdx.x == 0)
        for (int k = 0; k < kSpec; ++k) sh.spec_node[k] = nodes[k];
    if (wv >= 2 && wv < 2 + 2 * kSpec) {
        const int k = (wv - 2) >> 1, row = (wv - 2) & 1;
        if (nodes[k] >= 0) {
            float smax;
            double S;
            row_combine(a, b, nodes[k], row, smax, S);
            if (lane == 0) {
                sh.spec_s[k][row] = static_cast<double>(smax);
                sh.spec_S[k][row] = S;
            }
        }
    }
}

// Maximum and sum over the 8 lanes of an aligned group (lane moves xor 1,
// xor 2, then the mirror within 8 lanes); every lane of the group gets the
// same result.  The maximum orders floats by integer keys, as wave_max.
__device__ __forceinline__ float octet_max(float v) {
    const int b = i_of(v);
    int k = b ^ ((b >> 31) & 0x7fffffff);
    k = max(k, dpp<kDppXor1>(k));
    k = max(k, dpp<kDppXor2>(k));
    k = max(k, dpp<kDppHalfMirror>(k));
    return f_of(k ^ ((k >> 31) & 0x7fffffff));
}
__device__ __forceinline__ double octet_sum_d(double v) {
    v += dpp_d<kDppXor1>(v);
    v += dpp_d<kDppXor2>(v);
    v += dpp_d<kDppHalfMirror>(v);
    return v;
}

// Every row of a small tree from its staged partials: row j (node j / 2, row
// j % 2) by the 8 lanes of group j of the block, each lane taking chunks
// l, l + 8, ... in order (the row_combine operations on the same values, in
// a fixed order of its own).  Every thread calls it.
__device__ __forceinline__ void tab_combine_all(MultiShared &sh, int C1, int rows) {
    const int t = static_cast<int>(threadIdx.x);
    const int l8 = t & 7;
    for (int j0 = 0; j0 < rows; j0 += kMB / 8) {
        const int j = j0 + t / 8;
        const bool on = j < rows;
        const float *ps = sh.tab_ps + (on ? j : 0) * C1;
        const double *pS = sh.tab_pS + (on ? j : 0) * C1;
        float smax = -INFINITY;
        for (int c = l8; c < C1; c += 8) smax = fmaxf(smax, ps[c]);
        smax = octet_max(smax);
        double S = 0.0;
        for (int c = l8; c < C1; c += 8) {
            const float sc = ps[c];
            if (sc != -INFINITY) S += pS[c] * pow2_shift_d(static_cast<double>(sc) - static_cast<double>(smax));
        }
        S = octet_sum_d(S);
        if (on && l8 == 0) {
            sh.tab_s[j >> 1][j & 1] = static_cast<double>(smax);
            sh.tab_S[j >> 1][j & 1] = S;
        }
    }
}

// Node u's statistics from the small tree's table, or from a slot filled
// ahead of need if one holds it (the same values load_stats would set);
// every slot is emptied.  Block barrier.
__device__ __forceinline__ bool take_spec(MultiShared &sh, int u, bool target_only, bool tab) {
    if (threadIdx.x == 0) {
        int hit = 0;
        if (tab) {
            // the values set_stats forms, computed once per node at the start
            sh.sA = sh.tab_s[u][0];
            sh.SA = sh.tab_S[u][0];
            sh.iA = sh.tab_iA[u];
            sh.sB = target_only ? 0.0 : sh.tab_s[u][1];
            sh.SB = target_only ? 1.0 : sh.tab_S[u][1];
            sh.iB = target_only ? 1.0 : sh.tab_iB[u];
            sh.k0 = target_only ? 0.0f : sh.tab_k0[u];
            hit = 1;
        }
        for (int k = 0; k < kSpec; ++k) {
            if (!hit && sh.spec_node[k] == u) {
                set_stats(sh, sh.spec_s[k][0], sh.spec_S[k][0], sh.spec_s[k][1], sh.spec_S[k][1], target_only);
                hit = 1;
            }
            sh.spec_node[k] = -1;
        }
        sh.spec_hit = hit;
    }
    __syncthreads();
    return sh.spec_hit != 0;
}

// The VEC fp32 values of vector gv of a residual row (16-byte loads; the
// row stride Vp keeps every vector aligned), and their store.
template <int VEC>
__device__ __forceinline__ void load_res_vec(const float *row, int gv, float (&f)[VEC]) {
#pragma unroll
    for (int h = 0; h < VEC / 4; ++h) {
        const u32x4 d = *reinterpret_cast<const u32x4 *>(row + int64_t(gv) * VEC + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) f[4 * h + j] = __uint_as_float(d[j]);
    }
}
template <int VEC>
__device__ __forceinline__ void store_res_vec(float *row, int gv, const float (&f)[VEC]) {
#pragma unroll
    for (int h = 0; h < VEC / 4; ++h) {
        u32x4 d;
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = __float_as_uint(f[4 * h + j]);
        *reinterpret_cast<u32x4 *>(row + int64_t(gv) * VEC + 4 * h) = d;
    }
}

// Residual after a rejection: w(v) = max(0, r(v) - q(v)) with r = p~ (first
// rejection, from the logits: first_residual) or the previous residual
// in[v] / Zin; w is
// stored (fp32) in out, where only this block reads it again (its slice), and
// its fp64 sum over the tree's slices returned.  The child tests form w at a
// child's token again from the same values and operations.  Each thread
// loads all its vectors (logits and the previous residual) before any
// arithmetic, forms each vector's weights in registers and stores them as
// whole vectors (0 past V, inside the padded row).  draw_next: the draw from
// this residual follows (the node's last child was rejected), so the pass
// also forms what the draw's first pass would from the stored values (the
// slice's tile-scan total and last positive weight) and publishes them with
// the mass at the same barrier: sh.gath[g] = {mass, total, last}.
template <class DT>
__device__ double pass_residual(const MultiArgs &a, MultiShared &sh, int &phase, const char *row_t,
                                const char *row_q, const float *in, double Zin, float *out, bool draw_next) {
    constexpr int VEC = DT::kVec;
    const int V = a.V;
    const int nvec = (V + VEC - 1) / VEC;
    const Slice sl = my_slice(a, sh, nvec);
    double tot = 0.0;
    double carry = 0.0;
    int last = -1;
    for (int g0 = sl.lo; g0 < sl.hi; g0 += kMB * kMU) {
        u32x4 dt[kMU], dq[kMU];
        float pin[kMU][VEC];
#pragma unroll
        for (int k = 0; k < kMU; ++k) {
            const int gv = g0 + k * kMB + static_cast<int>(threadIdx.x);
            dt[k] = load_row_vec<DT, false>(row_t, gv < sl.hi ? gv : nvec, V);
            dq[k] = load_row_vec<DT, false>(row_q, gv < sl.hi ? gv : nvec, V);
            if (in != nullptr) load_res_vec<VEC>(in, gv < sl.hi ? gv : sl.lo, pin[k]);
        }
#pragma unroll
        for (int k = 0; k < kMU; ++k) {
            const int gv = g0 + k * kMB + static_cast<int>(threadIdx.x);
            double vsum = 0.0;
            if (gv < sl.hi) {
                float ft[VEC], fq[VEC], w[VEC];
                DT::unpack(dt[k], ft);
                DT::unpack(dq[k], fq);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float we;
                    if (in == nullptr) {
                        we = first_residual(a, sh, ft[e], fq[e]);
                    } else {
                        double pm, q;
                        m_probs<DT>(a, sh, ft[e], fq[e], pm, q);
                        we = static_cast<float>(fmax(0.0, static_cast<double>(pin[k][e]) / Zin - q));
                    }
                    w[e] = (gv * VEC + e < V) ? we : 0.0f;
                }
                store_res_vec<VEC>(out, gv, w);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    tot += static_cast<double>(w[e]);
                    // the draw's tile weight of the stored value (tile_weights)
                    double wd = static_cast<double>(w[e]);
                    if (!(wd > 0.0)) wd = 0.0;
                    vsum += wd;
                    if (wd > 0.0) last = gv * VEC + e;
                }
            }
            // the draw's tiles: kMB vectors from the slice's start (uniform)
            if (draw_next && g0 + k * kMB < sl.hi) carry = mblock_scan(vsum, carry, sh).total;
        }
    }
    const double msum = mblock_sum(tot, sh);
    if (draw_next) {
        last = mblock_max_i(last, sh);
        const double mine[kSlot] = {msum, carry, static_cast<double>(last), 0.0};
        publish_vals(a, sh, phase, mine, 3);
        tree_barrier(a, sh, phase, 3);
    } else {
        const double mine[kSlot] = {msum, 0.0, 0.0, 0.0};
        publish_vals(a, sh, phase, mine, 1);
        tree_barrier(a, sh, phase, 1);
    }
    double Z = 0.0;
    for (int g = 0; g < a.G; ++g) Z += sh.gath[g][0];
    return Z;
}

enum MultiDraw { kDrawBonus = 0, kDrawBuffer = 1, kDrawMixture = 2 };

// Weight of an element for a draw: the bonus 2^(z_t c - s) (unnormalised),
// or p~ itself (a stored residual is read as whole vectors by tile_weights).
template <class DT, int KIND>
__device__ __forceinline__ double draw_weight(const MultiArgs &a, const MultiShared &sh, float zt, float zq) {
    if constexpr (KIND == kDrawBonus) {
        return static_cast<double>(m_pow2(zt, a.c_hi, a.c_lo, static_cast<float>(sh.sA)));
    } else {
        double pm, q;
        m_probs<DT>(a, sh, zt, zq, pm, q);
        return pm;
    }
}

// Weights of vector gv of the slice ending at vector hi (0 past it), their
// sum in element order, and the last element with a positive weight.
template <class DT, int KIND>
__device__ __forceinline__ double tile_weights(const MultiArgs &a, const MultiShared &sh, const char *row_t,
                                              const char *row_q, const float *buf, int gv, int hi,
                                              double (&w)[DT::kVec], int &last) {
    constexpr int VEC = DT::kVec;
    const int V = a.V;
    const int gl = (gv < hi) ? gv : (V + VEC - 1) / VEC;      // past the slice: a -inf vector
    float ft[VEC], fq[VEC], fb[VEC];
    if (KIND != kDrawBuffer) DT::unpack(load_row_vec<DT, false>(row_t, gl, V), ft);
    if (KIND == kDrawMixture) DT::unpack(load_row_vec<DT, false>(row_q, gl, V), fq);
    if (KIND == kDrawBuffer) load_res_vec<VEC>(buf, (gv < hi) ? gv : hi - 1, fb);
    double sum = 0.0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const int v = gv * VEC + e;
        double we;
        if constexpr (KIND == kDrawBuffer) we = static_cast<double>(fb[e]);
        else we = draw_weight<DT, KIND>(a, sh, ft[e], fq[e]);
        w[e] = (gv < hi && v < V) ? we : 0.0;
        if (!(w[e] > 0.0)) w[e] = 0.0;
        sum += w[e];
        if (w[e] > 0.0) last = v;
    }
    return sum;
}

// Inverse CDF in index order: the token min{v : F(v) > u * W}, with the last
// positive weight when rounding leaves no crossing; -1 when the total is not
// positive.  Every block first sums its slice in tiles of kMB vectors (a
// block scan per tile) and publishes the total; the slice totals in slice
// order give each slice its base and W.  The block whose [base, base + total)
// holds u * W walks its slice again with the same tile scans from base and
// publishes the token.
template <class DT, int KIND>
__device__ int pass_draw(const MultiArgs &a, MultiShared &sh, int &phase, const char *row_t,
                         const char *row_q, const float *buf, double u, bool given = false) {
    constexpr int VEC = DT::kVec;
    const int nvec = (a.V + VEC - 1) / VEC;
    const Slice sl = my_slice(a, sh, nvec);
    const int g = sh.slice;
    // given: the residual pass that wrote buf published the slice totals and
    // last positive weights already (sh.gath[i][1], sh.gath[i][2])
    const int ic = given ? 1 : 0, il = given ? 2 : 1;
    if (!given) {
        double carry = 0.0;
        int last = -1;
        for (int g0 = sl.lo; g0 < sl.hi; g0 += kMB) {
            double w[VEC];
            const double sum = tile_weights<DT, KIND>(a, sh, row_t, row_q, buf,
                                                      g0 + static_cast<int>(threadIdx.x), sl.hi, w, last);
            carry = mblock_scan(sum, carry, sh).total;
        }
        last = mblock_max_i(last, sh);
        const double mine[kSlot] = {carry, static_cast<double>(last), 0.0, 0.0};
        publish_vals(a, sh, phase, mine, 2);
        tree_barrier(a, sh, phase, 2);
    }
    double base = 0.0, W = 0.0;
    int glast = -1;
    for (int i = 0; i < a.G; ++i) {
        if (i == g) base = W;
        W += sh.gath[i][ic];
        glast = max(glast, static_cast<int>(sh.gath[i][il]));
    }
    const double mytot = sh.gath[g][ic];
    if (!(W > 0.0) || !isfinite(W)) return -1;                 // the same in every block
    const double t = u * W;
    int mytok = -1;
    if (mytot > 0.0 && base <= t && t < base + mytot) {        // uniform over the block
        if (threadIdx.x == 0) sh.token = -1;
        __syncthreads();
        double c2 = base;
        for (int g0 = sl.lo; g0 < sl.hi; g0 += kMB) {
            const int gv = g0 + static_cast<int>(threadIdx.x);
            double w[VEC];
            int dummy = -1;
            const double sum = tile_weights<DT, KIND>(a, sh, row_t, row_q, buf, gv, sl.hi, w, dummy);
            const Scan s = mblock_scan(sum, c2, sh);
            if (s.excl <= t && t < s.incl) {
                double cum = s.excl;
                int pick = -1, lastpos = -1;
                for (int e = 0; e < VEC; ++e) {
                    if (w[e] > 0.0) {
                        lastpos = gv * VEC + e;
                        cum += w[e];
                        if (pick < 0 && cum > t) pick = gv * VEC + e;
                    }
                }
                sh.token = (pick >= 0) ? pick : lastpos;
            }
            c2 = s.total;
            __syncthreads();
            if (sh.token >= 0) break;
        }
        // t rounded past this slice's last prefix: its last positive weight
        mytok = (sh.token >= 0) ? sh.token : static_cast<int>(sh.gath[g][il]);
        __syncthreads();
    }
    const double mt[kSlot] = {static_cast<double>(mytok), 0.0, 0.0, 0.0};
    publish_vals(a, sh, phase, mt, 1);
    tree_barrier(a, sh, phase, 1);
    int tok = -1;
    for (int i = 0; i < a.G; ++i) tok = max(tok, static_cast<int>(sh.gath[i][0]));
    return (tok >= 0) ? tok : glast;        // t rounded to the very top: the last positive weight
}

// Acceptance probability of child token x (logits zt, zq at its parent's
// rows) while no residual has been formed at the parent: min(1, p~(x) / q(x))
// in fp64 from the parent's row statistics; q(x) = 0 accepts iff p~(x) > 0.
// fl gets SV_DATA_BAD_TOKEN or SV_DATA_ZERO_Q.
__device__ __forceinline__ double first_child_acc(const MultiArgs &a, double sA, double SA, double sB, double SB,
                                                  int x, float zt, float zq, int &fl) {
    if (x < 0 || x >= a.V) {
        fl |= SV_DATA_BAD_TOKEN;
        return 0.0;
    }
    const double q = (zq == -INFINITY) ? 0.0 : exp2_d(static_cast<double>(zq) * a.c_d - sB) / SB;
    double r;
    if (a.space == 1) {
        r = (zt == -INFINITY || zq == -INFINITY)
                ? 0.0
                : exp2_d(a.al * static_cast<double>(zt) + a.be * static_cast<double>(zq) - sA) / SA;
    } else {
        const double pt = (zt == -INFINITY) ? 0.0 : exp2_d(static_cast<double>(zt) * a.c_d - sA) / SA;
        r = (1.0 - static_cast<double>(a.lam)) * pt + static_cast<double>(a.lam) * q;
    }
    if (q == 0.0) {
        fl |= SV_DATA_ZERO_Q;
        return (r > 0.0) ? 1.0 : 0.0;
    }
    return fmin(1.0, r / q);
}

// ---- the walk ----------------------------------------------------------------

template <class DT>
__global__ __launch_bounds__(kMB) void k_tree_multi(MultiArgs a) {
    __shared__ MultiShared sh;
    const int t = threadIdx.x;
    if (t == 0) {
        const unsigned k = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh.tree = static_cast<int>(k / static_cast<unsigned>(a.G));
        sh.slice = static_cast<int>(k % static_cast<unsigned>(a.G));
    }
    __syncthreads();
    const int b = sh.tree;
    const int g = sh.slice;     // block 0 of the tree writes the outputs
    int phase = 0;
    const int N = a.N, V = a.V;
    for (int i = t; i <= N; i += kMB) {
        sh.head[i] = -1;
        sh.next[i] = -1;
        sh.tok[i] = (i > 0) ? a.node_token[int64_t(b) * N + i - 1] : -1;
        sh.par[i] = (i > 0) ? a.parent[int64_t(b) * N + i - 1] : -1;
        sh.ua[i] = (i > 0) ? a.u_accept[int64_t(b) * N + i - 1] : 0.0f;
    }
    // a small tree: every row's chunk partials, staged while the tree is read
    const int n_parts = 2 * (N + 1) * a.C1;
    const bool tab = (N + 1 <= kTabNodes) && (n_parts <= kTabParts);
    if (tab) {
        const Part *pp = a.part1 + int64_t(b) * n_parts;
        for (int i = t; i < n_parts; i += kMB) {
            const Part q = pp[i];
            sh.tab_ps[i] = q.s;
            sh.tab_pS[i] = q.S;
        }
    } else {
        // the root's statistics, combined while the tree is read
        int nodes[kSpec];
        for (int k = 0; k < kSpec; ++k) nodes[k] = (k == 0) ? 0 : -1;
        spec_stats(a, sh, b, nodes);
    }
    if (a.accept_prob != nullptr && g == 0)
        for (int i = t; i < N; i += kMB) a.accept_prob[int64_t(b) * N + i] = -1.0f;
    if (t == 0) {
        sh.flags = 0;
        sh.broken = 0;
    }
    __syncthreads();
    if (tab) {
        // children lists in node order, one node per thread: node i's first
        // child and its next sibling are the first later nodes whose parent
        // is i, and is i's parent (the lists the serial linking below forms)
        for (int i = t; i <= N; i += kMB) {
            const int p = sh.par[i];
            const bool linked = i >= 1 && p >= 0 && p < i;
            if (i >= 1 && !linked) atomicOr(&sh.flags, SV_DATA_BAD_TREE);   // never tested
            int hd = -1, nx = -1;
            for (int j = i + 1; j <= N; ++j) {
                const int pj = sh.par[j];
                if (hd < 0 && pj == i) hd = j;
                if (linked && nx < 0 && pj == p) nx = j;
            }
            sh.head[i] = hd;
            sh.next[i] = nx;
        }
    } else if (t == 0) {
        // children lists in node order: link from the last node down
        for (int i = N; i >= 1; --i) {
            const int p = sh.par[i];
            if (p < 0 || p >= i) {
                sh.flags |= SV_DATA_BAD_TREE;       // never tested
                continue;
            }
            sh.next[i] = sh.head[p];
            sh.head[p] = i;
        }
    }
    const char *tb = a.tgt + int64_t(b) * (N + 1) * a.ld_t * a.elem;
    const char *qb = a.drf + int64_t(b) * (N + 1) * a.ld_q * a.elem;
    if (tab) {
        // every node's two logits at its parent's rows (node i by thread
        // i + 64), and every node's two rows
        const int i = t - kWave;
        float zt = 0.0f, zq = 0.0f;
        const bool mine = i >= 1 && i <= N && sh.par[i] >= 0 && sh.par[i] <= N;
        if (mine) {
            const int x = sh.tok[i];
            if (x >= 0 && x < V) {
                zt = DT::load1(tb + int64_t(sh.par[i]) * a.ld_t * a.elem, x);
                zq = DT::load1(qb + int64_t(sh.par[i]) * a.ld_q * a.elem, x);
            }
        }
        tab_combine_all(sh, a.C1, 2 * (N + 1));
        if (mine) {
            sh.czt[i] = zt;
            sh.czq[i] = zq;
        }
    }
    __syncthreads();
    if (tab) {
        // every node's derived statistics (as set_stats forms them), and each
        // first child's test at its parent, one thread per node
        for (int v = t; v <= N; v += kMB) {
            const double SAv = sh.tab_S[v][0], SBv = sh.tab_S[v][1];
            sh.tab_iA[v] = 1.0 / SAv;
            sh.tab_iB[v] = 1.0 / SBv;
            sh.tab_k0[v] = static_cast<float>((sh.tab_s[v][0] - sh.tab_s[v][1]) + log2(SAv / SBv));
            const int p = (v >= 1) ? sh.par[v] : -1;
            if (p >= 0 && p < v && sh.head[p] == v) {
                int fl = 0;
                sh.tab_acc[v] = first_child_acc(a, sh.tab_s[p][0], sh.tab_S[p][0], sh.tab_s[p][1], sh.tab_S[p][1],
                                                sh.tok[v], sh.czt[v], sh.czq[v], fl);
                sh.tab_fl[v] = fl;
            }
        }
        __syncthreads();
    }

    float *buf0 = a.buf + int64_t(b) * 2 * a.Vp;
    float *buf1 = buf0 + a.Vp;
    const double us = static_cast<double>(a.u_sample[b]);
    int u = 0, depth = 0, tok = -1;
    bool done = false;
    bool kids_ready = tab;              // the children's logits of node u are in sh.czt / sh.czq
    while (!done) {
        if (tab) {
            // a small tree's accepted first children need no block barrier:
            // every thread follows them through the table (the same values
            // in every block), down to the first node whose first child is
            // rejected, has a row the walk must flag, or is absent
            for (;;) {
                const int c = (depth < a.Dmax) ? sh.head[u] : -1;
                if (c < 0) break;
                const double SAu = sh.tab_S[u][0], SBu = sh.tab_S[u][1];
                if (!(SAu > 0.0) || !isfinite(SAu) || !(SBu > 0.0) || !isfinite(SBu) ||
                    !isfinite(sh.tab_s[u][0]) || !isfinite(sh.tab_s[u][1]))
                    break;
                const double acc_p = sh.tab_acc[c];
                if (!(static_cast<double>(sh.ua[c]) < acc_p)) break;
                if (t == 0) {
                    sh.flags |= sh.tab_fl[c];
                    if (a.accept_prob != nullptr && g == 0)
                        a.accept_prob[int64_t(b) * N + c - 1] = static_cast<float>(acc_p);
                    if (depth < SV_MAX_POSITIONS) sh.path[depth] = c;
                }
                u = c;
                ++depth;
            }
        }
        const char *rt = tb + int64_t(u) * a.ld_t * a.elem;
        const char *rq = qb + int64_t(u) * a.ld_q * a.elem;
        const int first = (depth < a.Dmax) ? sh.head[u] : -1;
        // the node's statistics, when combined ahead of need
        const bool have = take_spec(sh, u, first < 0, tab);
        if (first < 0) {
            // bonus: the target's own softmax(z/T) at this node (in logit
            // space the precomputed row A is the mixture: a pass of its own)
            if (a.space == 1) pass_stats<DT>(a, sh, phase, rt, rq, true);
            else if (!have) load_stats(a, sh, b, u, true);
            tok = pass_draw<DT, kDrawBonus>(a, sh, phase, rt, rq, nullptr, us);
            if (tok < 0 && t == 0) sh.flags |= SV_DATA_BAD_ROW;
            break;
        }
        // the children's two logits, for thread 0's child tests: loaded by
        // the threads of their node ids while the statistics combine, unless
        // the parent's visit loaded them already (see below)
        constexpr int kPre = (kMNodes + kMB - 1) / kMB;
        if (!kids_ready) {
            float pzt[kPre], pzq[kPre];
#pragma unroll
            for (int k = 0; k < kPre; ++k) {
                const int i = t + k * kMB;
                pzt[k] = pzq[k] = 0.0f;
                if (i >= 1 && i <= N && sh.par[i] == u) {
                    const int x = sh.tok[i];
                    if (x >= 0 && x < V) {
                        pzt[k] = DT::load1(rt, x);
                        pzq[k] = DT::load1(rq, x);
                    }
                }
            }
            if (!have) load_stats(a, sh, b, u, false);
#pragma unroll
            for (int k = 0; k < kPre; ++k) {
                const int i = t + k * kMB;
                if (i >= 1 && i <= N && sh.par[i] == u) {
                    sh.czt[i] = pzt[k];
                    sh.czq[i] = pzq[k];
                }
            }
        } else if (!have) {
            load_stats(a, sh, b, u, false);
        }
        if (!kids_ready || !have) __syncthreads();       // (uniform) shared values were written
        if (!(sh.SA > 0.0) || !isfinite(sh.SA) || !(sh.SB > 0.0) || !isfinite(sh.SB) ||
            !isfinite(sh.sA) || !isfinite(sh.sB)) {
            if (t == 0) sh.flags |= SV_DATA_BAD_ROW;
            tok = -1;
            break;
        }
        // test the children in node order
        float *cur = nullptr;            // stored residual (NULL: r = p~)
        double Z = 1.0;
        int nrej = 0;                    // residuals formed at this node; their masses in sh.zs
        int c = first, nxt = -1;
        bool drawn = false;
        {
            // the first children's statistics, combined while thread 0
            // tests the first child (the test's barrier publishes them);
            // a small tree has every node's in its table already
            if (!tab) {
                int nodes[kSpec];
                int cc = first;
                for (int k = 0; k < kSpec; ++k) {
                    nodes[k] = cc;
                    cc = (cc >= 0) ? sh.next[cc] : -1;
                }
                spec_stats(a, sh, b, nodes);
            }
            // and the grandchildren's two logits at their parents' rows, for
            // the tests at whichever child is accepted; node i is taken by
            // thread i + 64, so that wave 0 (thread 0 tests) loads nothing
            // for trees of fewer than kMB - 64 nodes (a small tree has
            // every node's already)
            constexpr int kPre2 = (kMNodes + kWave + kMB - 1) / kMB;
#pragma unroll
            for (int k = 0; k < (tab ? 0 : kPre2); ++k) {
                const int i = t - kWave + k * kMB;
                if (i < 1 || i > N) continue;
                const int pi = sh.par[i];
                if (pi < 1 || pi > N || sh.par[pi] != u) continue;
                const int x = sh.tok[i];
                float zt = 0.0f, zq = 0.0f;
                if (x >= 0 && x < V) {
                    zt = DT::load1(tb + int64_t(pi) * a.ld_t * a.elem, x);
                    zq = DT::load1(qb + int64_t(pi) * a.ld_q * a.elem, x);
                }
                sh.czt[i] = zt;
                sh.czq[i] = zq;
            }
        }
        while (c >= 0) {
            if (t == 0) {
                const int x = sh.tok[c];
                double acc_p = 0.0;
                if (cur == nullptr) {
                    // fp64 from the gathered logits (a small tree's first
                    // children: computed with the tree's table)
                    int fl = 0;
                    if (tab && c == first) {
                        acc_p = sh.tab_acc[c];
                        fl = sh.tab_fl[c];
                    } else {
                        acc_p = first_child_acc(a, sh.sA, sh.SA, sh.sB, sh.SB, x, sh.czt[c], sh.czq[c], fl);
                    }
                    sh.flags |= fl;
                } else if (x < 0 || x >= V) {
                    sh.flags |= SV_DATA_BAD_TOKEN;
                } else {
                    // the stored residual at x, formed again with the residual
                    // pass's own operations from the logits, q(x) and the masses
                    const float zt = sh.czt[c];
                    const float zq = sh.czq[c];
                    double pm, q;
                    m_probs<DT>(a, sh, zt, zq, pm, q);
                    double r = static_cast<double>(first_residual(a, sh, zt, zq)) / sh.zs[1];
                    for (int j = 2; j <= nrej; ++j)
                        r = static_cast<double>(static_cast<float>(fmax(0.0, r - q))) / sh.zs[j];
                    if (q == 0.0) {
                        sh.flags |= SV_DATA_ZERO_Q;
                        acc_p = (r > 0.0) ? 1.0 : 0.0;
                    } else {
                        acc_p = fmin(1.0, r / q);
                    }
                }
                if (a.accept_prob != nullptr && g == 0)
                    a.accept_prob[int64_t(b) * N + c - 1] = static_cast<float>(acc_p);
                const float uc = sh.ua[c];
                sh.decision = (static_cast<double>(uc) < acc_p) ? 1 : 0;
            }
            __syncthreads();
            if (sh.decision) {
                nxt = c;
                break;
            }
            // rejected: the residual becomes the next child's target
            float *out = (cur == buf0) ? buf1 : buf0;
            const bool last_child = sh.next[c] < 0;
            const double Zn = pass_residual<DT>(a, sh, phase, rt, rq, cur, Z, out, last_child);
            if (!(Zn > 0.0) || !isfinite(Zn)) {
                // zero residual mass (rounding): draw from the current target
                if (t == 0) sh.flags |= SV_DATA_FALLBACK;
                tok = (cur == nullptr) ? pass_draw<DT, kDrawMixture>(a, sh, phase, rt, rq, nullptr, us)
                                       : pass_draw<DT, kDrawBuffer>(a, sh, phase, rt, rq, cur, us);
                drawn = true;
                break;
            }
            cur = out;
            Z = Zn;
            ++nrej;
            if (t == 0) sh.zs[nrej] = Zn;
            c = sh.next[c];
            __syncthreads();
        }
        if (drawn) break;
        if (nxt >= 0) {
            if (t == 0 && depth < SV_MAX_POSITIONS) sh.path[depth] = nxt;
            u = nxt;
            ++depth;
            kids_ready = true;
            continue;               // the next node's first barrier follows its statistics
        }
        // every child rejected: draw from the last residual, whose pass
        // published the draw's slice totals
        tok = pass_draw<DT, kDrawBuffer>(a, sh, phase, rt, rq, cur, us, true);
        if (tok < 0 && t == 0) sh.flags |= SV_DATA_BAD_ROW;
        done = true;
    }
    __syncthreads();
    if (t == 0 && sh.broken) atomicOr(a.status, SV_DATA_SYNC);
    if (g != 0) return;
    const int keep = min(depth, a.Dmax);
    for (int i = t; i <= a.Dmax; i += kMB) {
        int v = -1;
        if (i < keep) v = sh.tok[sh.path[i]];
        else if (i == keep) v = tok;
        a.out_tokens[int64_t(b) * (a.Dmax + 1) + i] = v;
        if (i < a.Dmax) a.accepted_nodes[int64_t(b) * a.Dmax + i] = (i < keep) ? sh.path[i] : -1;
    }
    if (t == 0) {
        a.accepted[b] = keep;
        if (sh.flags) atomicOr(a.status, sh.flags);
    }
}

}  // namespace sv

namespace {

using namespace sv;

// status word (when the caller passes none) at 0 and the ticket counter at 64,
// published slots [B, kMaxG, 3, kSlot], residual rows [B, 2, Vp] (Vp = V rounded up to 8), the row
// statistics' chunk partials [B, N+1, 2, C1] and their launch's counters [B]
constexpr int64_t kTicketOffset = 64;
int64_t multi_layout_pub() { return 256; }
int64_t multi_layout_buf(int B) {
    return multi_layout_pub() + align256(int64_t(B) * kMaxG * kRot * kSlot * int64_t(sizeof(double)));
}
int64_t multi_residual_stride(int V) { return (int64_t(V) + 7) / 8 * 8; }
int64_t multi_layout_part(int B, int V) {
    return multi_layout_buf(B) + align256(int64_t(B) * 2 * multi_residual_stride(V) * int64_t(sizeof(float)));
}
int64_t multi_layout_count(int B, int N, int V) {
    return multi_layout_part(B, V) +
           align256(int64_t(B) * (N + 1) * 2 * c1_for(V, kMinNV, kMinVec) * int64_t(sizeof(Part)));
}
int64_t multi_layout_total(int B, int N, int V) {
    return multi_layout_count(B, N, V) + align256(int64_t(B) * int64_t(sizeof(int)));
}

// Blocks per tree: each block keeps at least one tile of the row; by default
// the trees share the GPU's resident walk blocks, so that every tree runs in
// the first round; `want` in 1..kMaxG asks for that many.
int choose_g(int B, int V, int vec, int units, int want) {
    const int nvec = (V + vec - 1) / vec;
    const int cap = (want > 0) ? want : units / std::max(B, 1);
    return std::max(1, std::min({kMaxG, cap, (nvec + kMB - 1) / kMB}));
}

sv_status verify_multi(const void *target_logits, int64_t ld_t, const void *draft_logits, int64_t ld_q,
                       sv_dtype dtype, int B, int N, int V, const int32_t *parent, const int32_t *node_token,
                       const float *u_accept, const float *u_sample, float lambda, float temperature,
                       int mix_space, int32_t *accepted, int32_t *out_tokens, int32_t *accepted_nodes,
                       float *accept_prob, int Dmax, int32_t *status, void *workspace, size_t workspace_bytes,
                       hipStream_t stream, int blocks_per_tree) {
    if (mix_space != SV_MIX_PROB && mix_space != SV_MIX_LOGIT) return SV_EINVAL;
    if (blocks_per_tree < 0 || blocks_per_tree > kMaxG) return SV_EINVAL;
    const int eb = elem_bytes(dtype);
    if (eb == 0) return SV_EDTYPE;
    if (B < 0 || N < 0 || N > SV_MAX_TREE_NODES || V < 1 || Dmax < 0 || Dmax > SV_MAX_POSITIONS ||
        B > (1 << 30) || int64_t(V) > (int64_t(1) << 28) ||
        int64_t(B) * (N + 1) * 2 * c1_for(V, kMinNV, kMinVec) >= (int64_t(1) << 31))
        return SV_EINVAL;
    sv_status st = check_scalars(lambda, temperature);
    if (st != SV_OK) return st;
    if (B == 0) return SV_OK;
    if (!u_sample || !accepted || !out_tokens || (Dmax > 0 && !accepted_nodes)) return SV_ENULL;
    if (N > 0 && (!parent || !node_token || !u_accept)) return SV_ENULL;
    if ((st = check_logits(target_logits, ld_t, V, eb)) != SV_OK) return st;
    if ((st = check_logits(draft_logits, ld_q, V, eb)) != SV_OK) return st;
    if (!workspace || !aligned16(workspace) ||
        workspace_bytes < static_cast<size_t>(multi_layout_total(B, N, V)))
        return SV_EWORKSPACE;
    MultiArgs a;
    a.tgt = static_cast<const char *>(target_logits);
    a.drf = static_cast<const char *>(draft_logits);
    a.ld_t = ld_t;
    a.ld_q = ld_q;
    a.elem = eb;
    a.B = B;
    a.N = N;
    a.V = V;
    a.Dmax = Dmax;
    a.parent = parent;
    a.node_token = node_token;
    a.u_accept = u_accept;
    a.u_sample = u_sample;
    a.lam = lambda;
    temperature_split(temperature, &a.c_hi, &a.c_lo, &a.c_d);
    a.space = (mix_space == SV_MIX_LOGIT && lambda > 0.0f && lambda < 1.0f) ? 1 : 0;
    a.al = (1.0 - static_cast<double>(lambda)) * a.c_d;
    a.be = static_cast<double>(lambda) * a.c_d;
    a.mx[0] = a.mx[1] = a.mx[2] = a.mx[3] = 0.0f;
    if (a.space == 1) {
        split_positive(a.al, &a.d_hi, &a.d_lo);
        split_positive(a.al, &a.mx[0], &a.mx[1]);
        split_positive(a.be, &a.mx[2], &a.mx[3]);
    } else {
        a.d_hi = a.c_hi;
        a.d_lo = a.c_lo;
    }
    a.accepted = accepted;
    a.out_tokens = out_tokens;
    a.accepted_nodes = accepted_nodes;
    a.accept_prob = accept_prob;
    char *ws = static_cast<char *>(workspace);
    a.status = status ? status : reinterpret_cast<int32_t *>(ws);
    a.pub = reinterpret_cast<unsigned long long *>(ws + multi_layout_pub());
    a.buf = reinterpret_cast<float *>(ws + multi_layout_buf(B));
    a.Vp = static_cast<int>(multi_residual_stride(V));
    a.ticket = reinterpret_cast<unsigned *>(ws + kTicketOffset);
    a.part1 = reinterpret_cast<const Part *>(ws + multi_layout_part(B, V));
    a.C1 = rows_stats_chunks(B, N + 1, V, dtype, a.space);
    // A tree's blocks wait for one another; the start-order tickets make any
    // grid progress as long as G blocks fit at once.  By default B * G stays
    // within the resident capacity, so every tree runs in the first round.  An
    // ordinary launch: a cooperative one costs about 20 us per call here
    const void *kern = dtype == SV_BF16 ? reinterpret_cast<const void *>(k_tree_multi<Bf16>)
                                        : reinterpret_cast<const void *>(k_tree_multi<F32>);
    int dev = 0, units = 0, per_unit = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&units, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_unit, kern, kMB, 0) != hipSuccess)
        return SV_EHIP;
    a.G = choose_g(B, V, 16 / eb, units * std::max(per_unit, 0), blocks_per_tree);
    const int64_t n_slots = int64_t(B) * a.G * kRot * kSlot;
    // every row's statistics in one streaming launch over the whole GPU: the
    // walk then combines a node's chunk partials instead of a pass and a
    // barrier of its own.  The launch also clears the status word, empties
    // the walk's barrier slots and resets its ticket counter.
    st = rows_stats(target_logits, ld_t, draft_logits, ld_q, dtype, B, N + 1, V, lambda, temperature, a.space,
                    reinterpret_cast<Part *>(ws + multi_layout_part(B, V)),
                    reinterpret_cast<int *>(ws + multi_layout_count(B, N, V)), a.status, stream, a.pub, n_slots,
                    kEmpty, a.ticket, parent);
    if (st != SV_OK) return st;
    const dim3 grid(static_cast<unsigned>(int64_t(B) * a.G));
    if (dtype == SV_BF16) {
        hipLaunchKernelGGL(k_tree_multi<Bf16>, grid, dim3(kMB), 0, stream, a);
    } else {
        hipLaunchKernelGGL(k_tree_multi<F32>, grid, dim3(kMB), 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

}  // namespace

extern "C" {

size_t sv_tree_multi_workspace_bytes(int B, int N, int V) {
    if (B < 0 || N < 0 || N > SV_MAX_TREE_NODES || V < 1) return 0;
    return static_cast<size_t>(multi_layout_total(B, N, V));
}

sv_status sv_tree_verify_multi(const void *target_logits, int64_t ld_t, const void *draft_logits,
                               int64_t ld_q, sv_dtype dtype, int B, int N, int V,
                               const int32_t *parent, const int32_t *node_token,
                               const float *u_accept, const float *u_sample, float lambda,
                               float temperature, int mix_space, int32_t *accepted,
                               int32_t *out_tokens, int32_t *accepted_nodes, float *accept_prob,
                               int Dmax, int32_t *status, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    return verify_multi(target_logits, ld_t, draft_logits, ld_q, dtype, B, N, V, parent, node_token, u_accept,
                        u_sample, lambda, temperature, mix_space, accepted, out_tokens, accepted_nodes,
                        accept_prob, Dmax, status, workspace, workspace_bytes, stream, 0);
}

sv_status sv_tree_verify_multi_ex(const void *target_logits, int64_t ld_t, const void *draft_logits,
                                  int64_t ld_q, sv_dtype dtype, int B, int N, int V,
                                  const int32_t *parent, const int32_t *node_token,
                                  const float *u_accept, const float *u_sample, float lambda,
                                  float temperature, int mix_space, int32_t *accepted,
                                  int32_t *out_tokens, int32_t *accepted_nodes, float *accept_prob,
                                  int Dmax, int32_t *status, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream, int blocks_per_tree) {
    return verify_multi(target_logits, ld_t, draft_logits, ld_q, dtype, B, N, V, parent, node_token, u_accept,
                        u_sample, lambda, temperature, mix_space, accepted, out_tokens, accepted_nodes,
                        accept_prob, Dmax, status, workspace, workspace_bytes, stream, blocks_per_tree);
}

}  // extern "C"
