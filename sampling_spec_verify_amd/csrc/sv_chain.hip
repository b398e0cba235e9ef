// Linear-chain and tree-path verification on gfx950.
//
// Method (cited by page title and section):
//   RAPID explainer (arXiv 2502.20330), "2) 推理时知识迁移": the target law is
//     replaced by the mixture p~ = (1 - lambda) p_t + lambda q.
//   RAPID explainer, "3) 候选验证机制（伪代码）": per drafted position, softmax
//     both rows, accept with probability min(1, p~(x)/q(x)), stop at the first
//     rejection and resample there.
//   "大模型推理的Speculative Decoding原理详解", "修改的拒绝采样", and the EAGLE
//     explainer, "1. 为什么无损": the resample law is max(0, p - q), normalised.
//
// Two launches per call:
//
//  1. k_row_stats: one wavefront per (request, position, tensor, chunk) streams
//     64 lanes x NV x 16 bytes of one drafted row with coalesced 16-byte loads
//     and reduces it to (shift s, S = sum 2^(z c - s)) with c = log2(e)/T and
//     s an integer, so partials combine by exact powers of two; the wave whose
//     chunk holds the drafted token also records its logit.  Every
//     drafted target and draft row is read exactly once.  Waves are
//     independent (no LDS, no barrier); the launch also clears the status word
//     and the per-request counters of launch 2.
//
//  2. k_resolve_mass: grid (B requests, C2 chunks) of 1024-thread blocks.
//     Every block stages its request's row partials in LDS, combines them in
//     fp64, computes every a_i in fp64 from the ratio
//     p_t(x) / q(x) = 2^((z_t(x) - z_q(x)) c - (s_t - s_q)) S_q / S_t (no
//     logarithms) and ballots the first rejection n;
//     block 0 writes every output but the sampled token.  Each block then
//     reduces its chunk of the sampling row: the residual max(0, p_t - q) at
//     row n (the same normalised law as max(0, p~ - q), since
//     p~ - q = (1 - lambda)(p_t - q)), or the bonus softmax(z/T) at the
//     request's last target row, to fp64 sums of its 16 * NV2 pieces, and
//     publishes them as agent-scope atomic stores.  Every block then counts
//     itself done (one atomic counter per request); wave 0 of the last of
//     the request's C2 blocks draws the token alone: it loads every piece
//     mass in one round (runs of consecutive pieces per lane, staged in LDS),
//     scales them to a common frame, finds the run and then the piece holding
//     u * W with two fp64 wave scans, reloads that piece's 64 vectors and
//     finds the token with a third.
//
// The only data that crosses blocks inside a launch are those piece masses:
// written and read as relaxed agent-scope atomics (write-through stores,
// coherent loads), drained before the counter is bumped, so no device-wide
// cache writeback is needed.  A separate launch for the draw costs about as
// much as the draw itself on this GPU (every kernel carries a fixed cost of
// a few microseconds).  The draw itself is all wave-level scans, ballots and
// lane reads, with no block barrier.  Every reduction has a fixed order
// (bitwise reproducible): which block draws does not change the result.
//
// Path mode reuses both launches with a row indirection: position j of a
// request uses target and draft row n_j of its draft tree (n_0 = root).
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include <algorithm>
#include <mutex>

#include "sv_common.hpp"
#include "sv_device.hpp"

namespace sv {

// ---------------------------------------------------------------------------
// request geometry
// ---------------------------------------------------------------------------

// Whether position i of request b is drafted (cheaper than counting them all).
__device__ __forceinline__ bool geo_position_valid(const Geo &g, int b, int i) {
    if (g.path == nullptr) {
        if (g.draft_len == nullptr) return i < g.P;
        const int k = g.draft_len[b];
        return i < min(max(k, 0), g.P);
    }
    for (int d = 0; d <= i; ++d) {
        const int v = g.path[int64_t(b) * g.P + d];
        if (v < 1 || v > g.N) return false;
    }
    return true;
}

// Row (within the request) of position i, for 0 <= i <= positions.
__device__ __forceinline__ int geo_row(const Geo &g, int b, int i) {
    if (g.path == nullptr) return i;
    return i == 0 ? 0 : g.path[int64_t(b) * g.P + i - 1];
}

// Drafted token of position i < positions.
__device__ __forceinline__ int geo_token(const Geo &g, int b, int i) {
    if (g.path == nullptr) return g.tokens[int64_t(b) * g.P + i];
    const int v = g.path[int64_t(b) * g.P + i];
    return g.tokens[int64_t(b) * g.N + v - 1];
}

// Requests the packed order covers, kWave per draft_len load.
constexpr int kPackChunks = 4;

// The r-th drafted position of a ragged chain batch in (request, position)
// order.  With it the jobs of drafted rows take the front of a statistics
// launch and the undrafted remainder its tail, where whole blocks exit at
// once, instead of idle waves sitting between busy ones in every block.
// Called with r uniform over the wave; b and i come out uniform.  False past
// the last drafted position.
__device__ __forceinline__ bool packed_position(const Geo &g, int B, int r, int &b, int &i) {
    const int lane = threadIdx.x & (kWave - 1);
    int k[kPackChunks];
#pragma unroll
    for (int t = 0; t < kPackChunks; ++t) {
        const int req = t * kWave + lane;
        k[t] = (req < B) ? min(max(g.draft_len[req], 0), g.P) : 0;
    }
    int base = 0;
#pragma unroll
    for (int t = 0; t < kPackChunks; ++t) {
        const int incl = wave_scan_i(k[t]);
        const int tot = __builtin_amdgcn_readlane(incl, kWave - 1);
        if (r < base + tot) {
            const int rr = r - base;
            // requests before the owner end at or before rr; lanes past B carry
            // the chunk total, which exceeds rr
            const int owner = __popcll(__ballot(incl <= rr));
            const int before = (owner > 0) ? __builtin_amdgcn_readlane(incl, owner - 1) : 0;
            b = t * kWave + owner;
            i = rr - before;
            return true;
        }
        base += tot;
    }
    return false;
}

// (request, position) held by position slot r of a statistics launch; false
// when the slot holds no drafted position.
__device__ __forceinline__ bool slot_position(const ChainArgs &a, int r, int &b, int &i) {
    if (a.packed) return packed_position(a.g, a.B, r, b, i);
    i = r % a.g.Pcap;
    b = r / a.g.Pcap;
    return geo_position_valid(a.g, b, i);
}

__device__ __forceinline__ const char *row_ptr(const Geo &g, int tensor, int b, int r) {
    if (tensor == 0)
        return g.tgt + (int64_t(b) * g.req_t * g.ld_t + int64_t(r) * g.ld_t) * g.elem;
    return g.drf + (int64_t(b) * g.req_q * g.ld_q + int64_t(r) * g.ld_q) * g.elem;
}

// ---------------------------------------------------------------------------
// launch 1: row statistics
// ---------------------------------------------------------------------------

// Whether node i of tree b is some node's parent (tree rows, one per node:
// a.leaf_par [B, leaf_N]); one ballot per 64 parents, uniform over the wave.
__device__ __forceinline__ bool node_has_child(const ChainArgs &a, int b, int i) {
    const int32_t *par = a.leaf_par + int64_t(b) * a.leaf_N;
    const int lane = threadIdx.x & (kWave - 1);
    bool has = false;
    for (int j0 = 0; j0 < a.leaf_N; j0 += kWave) {
        const int j = j0 + lane;
        const int pj = (j < a.leaf_N) ? par[j] : -1;
        has = has || (__ballot(pj == i) != 0ull);
    }
    return has;
}

// An empty partial (no element, sum 0) for chunk c of slot `slot` of (b, i).
__device__ __forceinline__ void empty_partial(const ChainArgs &a, int b, int i, int slot, int c) {
    Part p;
    p.s = -INFINITY;
    p.z = 0.0f;
    p.S = 0.0;
    a.part1[(int64_t(b) * a.g.Pcap + i) * 2 * a.C1 + int64_t(slot) * a.C1 + c] = p;
}

// One job: wave-chunk c of one drafted row, reduced by one wavefront.
// LEAF (tree rows, one per node): the draft row of a node that no node names
// as its parent is never read, so its wave stores an empty partial instead.
template <class DT, int NV, bool LEAF = false>
__device__ __forceinline__ void row_chunk_stats(const ChainArgs &a, unsigned job) {
    const unsigned C1 = static_cast<unsigned>(a.C1);
    const int c = static_cast<int>(job % C1);
    const unsigned rest = job / C1;
    const int tensor = static_cast<int>(rest & 1u);
    int b, i;
    if (!slot_position(a, static_cast<int>(rest >> 1), b, i)) return;
    if (LEAF && tensor == 1 && !node_has_child(a, b, i)) {
        if ((threadIdx.x & (kWave - 1)) == 0) empty_partial(a, b, i, 1, c);
        return;
    }
    const char *row = row_ptr(a.g, tensor, b, geo_row(a.g, b, i));
    // the wave whose chunk holds the drafted token also gathers its logit
    // no drafted tokens (the acceptance-rate call): nothing to gather
    const int x = (a.g.tokens != nullptr) ? geo_token(a.g, b, i) : -1;
    const bool own_x = x >= 0 && x < a.g.V && x / a.ch1 == c;

    constexpr int VEC = DT::kVec;
    const int lane = threadIdx.x & (kWave - 1);
    const int V = a.g.V;
    const int v0 = c * (kWave * NV);

    u32x4 d[NV];
    load_chunk<DT, NV>(row, v0, lane, V, d);
    // the loads are out: back to the base issue priority for the fold
    __builtin_amdgcn_s_setprio(0);
    float f[NV][VEC];
#pragma unroll
    for (int n = 0; n < NV; ++n) DT::unpack(d[n], f[n]);
    float m = -INFINITY;
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int e = 0; e < VEC; ++e) m = fmaxf(m, f[n][e]);

    const float c_hi = a.c_hi, c_lo = a.c_lo;
    // integer shift at or above the lane's largest z * c_hi: every weight is
    // at most about 1 and lanes rescale by exact powers of two
    const float s_lane = (m == -INFINITY) ? -INFINITY : ceilf(m * c_hi);
    const float s_use = (m == -INFINITY) ? 0.0f : s_lane;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            acc[e] += __builtin_amdgcn_exp2f(fmaf(f[n][e], c_lo, fmaf(f[n][e], c_hi, -s_use)));
    float S_lane = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) S_lane += acc[e];

    const float s_w = wave_max(s_lane);
    const float fac = (s_lane == -INFINITY) ? 0.0f : pow2_shift(s_lane - s_w);
    const double S_w = wave_sum_d(static_cast<double>(S_lane) * static_cast<double>(fac));
    if (lane == 0) {
        Part p;
        p.s = s_w;
        p.z = own_x ? DT::load1(row, x) : 0.0f;
        p.S = S_w;
        a.part1[(int64_t(b) * a.g.Pcap + i) * 2 * a.C1 + int64_t(tensor) * a.C1 + c] = p;
    }
}

// Zeroes the per-request counters of the mass blocks (launch 2), so that
// every call starts from zero whatever the workspace held.  The block size is
// the compile-time THREADS: reading blockDim would cost every wave a load
// from the dispatch packet before it can retire.
template <int THREADS>
__device__ __forceinline__ void clear_counts(const ChainArgs &a) {
    for (int i = static_cast<int>(blockIdx.x) * THREADS + static_cast<int>(threadIdx.x); i < a.B;
         i += static_cast<int>(gridDim.x) * THREADS)
        a.count[i] = 0;
    if (a.fill != nullptr) {
        for (int64_t i = int64_t(blockIdx.x) * THREADS + threadIdx.x; i < a.fill_n; i += int64_t(gridDim.x) * THREADS)
            a.fill[i] = a.fill_val;
        if (blockIdx.x == 0 && threadIdx.x == 0) *a.zero_word = 0u;
    }
    if (a.zero_f != nullptr) {
        for (int64_t i = int64_t(blockIdx.x) * THREADS + threadIdx.x; i < a.zero_f_n; i += int64_t(gridDim.x) * THREADS)
            a.zero_f[i] = 0.0f;
    }
}

// One wavefront per job; the job index is made wave-uniform so that its
// decode runs as 32-bit scalar arithmetic.  Jobs of undrafted positions exit
// after a few instructions.  Two waves per block in both row-statistics
// kernels: on a ragged batch the last busy blocks finish sooner than with
// four (26.1-26.3 against 26.5-27.0 us on a ragged batch of 64 requests of
// 1-8 positions at V = 128256), and the logit-space kernel gains a little on a
// full one (17.3 against 17.6 us on 16 requests of 8 positions at V = 151936).
constexpr int kStatsWaves = 2;

// Issue priority for a long row stream: when the grid spans at least two
// rounds of resident waves (256 CUs x 28 waves of this kernel), a wave starts
// at raised priority, so that a newly started wave decodes its job and issues
// its loads ahead of the folds of the waves already resident, and drops back
// once its loads are out.  On the ragged 64-request batch (32,768 jobs) this
// took the kernel from 26.1-26.3 to 25.1-25.2 us; on the full 16-request
// batch at V = 151936 (9,728 jobs, 1.4 rounds) it cost 1.2 us, so shorter
// grids keep one priority.
constexpr int kPrioJobs = 2 * 256 * 28;

template <class DT, int NV, bool PRIO, bool LEAF = false>
__global__ __launch_bounds__(kStatsWaves * kWave) void k_row_stats(ChainArgs a, int n_jobs) {
    if (PRIO) __builtin_amdgcn_s_setprio(3);
    const int job = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kStatsWaves +
                                                   static_cast<int>(threadIdx.x) / kWave);
    if (job < n_jobs) row_chunk_stats<DT, NV, LEAF>(a, static_cast<unsigned>(job));
    // cleared last: a store ahead of the job's reads would keep the compiler
    // from issuing them as scalar loads
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.status = 0;
    clear_counts<kStatsWaves * kWave>(a);
}

// Logit-space mixture (the RAPID pseudocode mixes logits, enhanced =
// (1 - lambda) z_t + lambda z_q, then takes a softmax): one job is wave-chunk
// c of drafted position i with its target and draft chunks together, so each
// drafted row is still read once.  Slot 0 of the position receives the
// enhanced row's partial: its exponent y = alpha z_t + beta z_q - s
// (alpha = (1 - lambda) c, beta = lambda c) comes from mixed_expo, four fp32
// fmas of the split constants; the lane shift ceil(alpha m_t + beta m_q),
// formed in fp64 once per lane, bounds the lane's largest
// alpha z_t + beta z_q from above (alpha, beta >= 0), and the slot carries the
// drafted token's target logit.  Slot 1 receives the draft row's partial
// exactly as in probability space.
// LEAF (tree rows, one per node): a node without children is never tested
// from, and its bonus row is the target's own softmax, which the walk forms
// itself in logit space; its wave stores empty partials for both slots.
template <class DT, int NV, bool LEAF = false>
__device__ __forceinline__ void row_chunk_stats_logit(const ChainArgs &a, unsigned job) {
    const unsigned C1 = static_cast<unsigned>(a.C1);
    const int c = static_cast<int>(job % C1);
    int b, i;
    if (!slot_position(a, static_cast<int>(job / C1), b, i)) return;
    if (LEAF && !node_has_child(a, b, i)) {
        if ((threadIdx.x & (kWave - 1)) == 0) {
            empty_partial(a, b, i, 0, c);
            empty_partial(a, b, i, 1, c);
        }
        return;
    }
    const int r = geo_row(a.g, b, i);
    const char *row_t = row_ptr(a.g, 0, b, r);
    const char *row_q = row_ptr(a.g, 1, b, r);
    const int x = (a.g.tokens != nullptr) ? geo_token(a.g, b, i) : -1;
    const bool own_x = x >= 0 && x < a.g.V && x / a.ch1 == c;

    constexpr int VEC = DT::kVec;
    const int lane = threadIdx.x & (kWave - 1);
    const int V = a.g.V;
    const int v0 = c * (kWave * NV);
    u32x4 dt[NV], dq[NV];
    load_chunk<DT, NV>(row_t, v0, lane, V, dt);
    load_chunk<DT, NV>(row_q, v0, lane, V, dq);
    float ft[NV][VEC], fq[NV][VEC];
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        DT::unpack(dt[n], ft[n]);
        DT::unpack(dq[n], fq[n]);
    }
    float mt = -INFINITY, mq = -INFINITY;
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            mt = fmaxf(mt, ft[n][e]);
            mq = fmaxf(mq, fq[n][e]);
        }
    const float c_hi = a.c_hi, c_lo = a.c_lo;
    const double al = a.alpha_c, be = a.beta_c;
    const float mx[4] = {a.al_hi, a.al_lo, a.be_hi, a.be_lo};
    // draft row, as in probability space
    const float sq_lane = (mq == -INFINITY) ? -INFINITY : ceilf(mq * c_hi);
    const float sq_use = (mq == -INFINITY) ? 0.0f : sq_lane;
    // enhanced row: -inf in either model leaves every mixed logit of the lane at -inf
    const bool e_none = (mt == -INFINITY) || (mq == -INFINITY);
    const float se_lane = e_none ? -INFINITY
                                 : static_cast<float>(ceil(al * static_cast<double>(mt) +
                                                           be * static_cast<double>(mq)));
    const double se_use = e_none ? 0.0 : static_cast<double>(se_lane);
    float accq[VEC], acce[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) accq[e] = acce[e] = 0.0f;
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            accq[e] += __builtin_amdgcn_exp2f(fmaf(fq[n][e], c_lo, fmaf(fq[n][e], c_hi, -sq_use)));
            acce[e] += __builtin_amdgcn_exp2f(mixed_expo(ft[n][e], fq[n][e], mx, static_cast<float>(se_use)));
        }
    float Sq_lane = 0.0f, Se_lane = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        Sq_lane += accq[e];
        Se_lane += acce[e];
    }
    const float sq_w = wave_max(sq_lane);
    const float se_w = wave_max(se_lane);
    const float fq_ = (sq_lane == -INFINITY) ? 0.0f : pow2_shift(sq_lane - sq_w);
    const float fe_ = (se_lane == -INFINITY) ? 0.0f : pow2_shift(se_lane - se_w);
    const double Sq_w = wave_sum_d(static_cast<double>(Sq_lane) * static_cast<double>(fq_));
    const double Se_w = wave_sum_d(static_cast<double>(Se_lane) * static_cast<double>(fe_));
    if (lane == 0) {
        Part* dst = a.part1 + (int64_t(b) * a.g.Pcap + i) * 2 * a.C1;
        Part pe, pq;
        pe.s = se_w;
        pe.z = own_x ? DT::load1(row_t, x) : 0.0f;
        pe.S = Se_w;
        pq.s = sq_w;
        pq.z = own_x ? DT::load1(row_q, x) : 0.0f;
        pq.S = Sq_w;
        dst[c] = pe;
        dst[a.C1 + c] = pq;
    }
}

template <class DT, int NV, bool LEAF = false>
__global__ __launch_bounds__(kStatsWaves * kWave) void k_row_stats_logit(ChainArgs a, int n_jobs) {
    const int job = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kStatsWaves +
                                                   static_cast<int>(threadIdx.x) / kWave);
    if (job < n_jobs) row_chunk_stats_logit<DT, NV, LEAF>(a, static_cast<unsigned>(job));
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.status = 0;
    clear_counts<kStatsWaves * kWave>(a);
}

// ---------------------------------------------------------------------------
// launch 2: resolve + chunk masses, then the inverse-CDF draw in the last block
// ---------------------------------------------------------------------------

// kResidualLogit: the residual max(0, p~ - q) of the logit-space mixture,
// p~ = softmax of the mixed logits (the target slot of the record holds its
// shift and 1 / sum).
enum SampleMode { kResidual = 0, kBonus = 1, kResidualLogit = 2 };

struct SampleCtx {
    const char *row_t;      // target row of the sampling position
    const char *row_q;      // draft row (residual / mixture)
    float c_hi, c_lo;
    float st, it;           // target row: p_t(v) = 2^(z c - st) * it
    float sq, iq;           // draft row:  q(v)   = 2^(z c - sq) * iq
    float w_t, w_q;         // mixture weights (1 - lambda, lambda)
    float mx[4];            // logit space: (1 - lambda) c and lambda c, each as hi + lo
    float d_hi, d_lo;       // residual: q(v) / p(v) = 2^((z_q - z_t) (d_hi + d_lo) + k0)
    float k0;               //   (d = c, or (1 - lambda) c in logit space)
    int logit;              // the target-slot statistics are those of the mixed logits
    int V;
};

// 2^(z c - s) with c = c_hi + c_lo, the argument formed with two fmas
__device__ __forceinline__ float pow2_logit(float z, float c_hi, float c_lo, float s) {
    return __builtin_amdgcn_exp2f(fmaf(z, c_lo, fmaf(z, c_hi, -s)));
}

// 2^(alpha z_t + beta z_q - s) of the logit-space mixture
__device__ __forceinline__ float pow2_mixed(float zt, float zq, const float (&m)[4], float s) {
    return __builtin_amdgcn_exp2f(mixed_expo(zt, zq, m, s));
}

// The sampling row is cut into chunks of kBlock2 lanes x NV2 vectors, one
// chunk per block of launch 2.  Wave w of the block owns the contiguous
// vectors [w * 64 * NV2, (w+1) * 64 * NV2) of the chunk and its lane l holds
// vectors n * 64 + l, n < NV2 (coalesced per n).  A "piece" is one such
// vector row (chunk, w, n): 64 contiguous vectors.  The inverse CDF runs in
// element order: chunk, wave, n, lane, element.
template <int NV2>
__device__ __forceinline__ int64_t piece_vec(int chunk, int wv, int n, int lane) {
    return int64_t(chunk) * (kBlock2 * NV2) + int64_t(wv) * (kWave * NV2) + int64_t(n) * kWave + lane;
}

template <class DT, int MODE>
__device__ __forceinline__ void load_vec(const SampleCtx &S, int64_t gv, u32x4 &dt, u32x4 &dq) {
    dt = load_row_vec<DT, false>(S.row_t, static_cast<int>(gv), S.V);
    if (MODE != kBonus) dq = load_row_vec<DT, false>(S.row_q, static_cast<int>(gv), S.V);
}

// Weights of one 16-byte vector; elements past V hold -inf logits and weigh 0.
// `s_use` is the bonus shift.
//
// Residual: max(0, p(v) - q(v)) = p(v) max(0, 1 - q(v) / p(v)), with p = p_t
// (or the logit-space p~) and q(v) / p(v) = 2^e(v),
// e(v) = (z_q(v) - z_t(v)) d + k0, k0 = (s_p - s_q) + log2(S_p / S_q) formed in
// fp64 once per request.  Every factor carries a few fp32 ulps of error
// relative to the weight itself, however close p and q are: subtracting the
// two probabilities would leave an error relative to p instead, which grows
// without bound relative to the residual mass as the draft approaches the
// target.  The common factor 1 / S_p is left out (the law is normalised).
template <class DT, int MODE>
__device__ __forceinline__ void vec_weights(const SampleCtx &S, const u32x4 &dt, const u32x4 &dq,
                                            float s_use, float *w) {
    constexpr int VEC = DT::kVec;
    float ft[VEC], fq[VEC];
    DT::unpack(dt, ft);
    if (MODE != kBonus) DT::unpack(dq, fq);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        if (MODE == kBonus) {
            w[e] = pow2_logit(ft[e], S.c_hi, S.c_lo, s_use);
        } else {
            const float ep = (MODE == kResidualLogit) ? pow2_mixed(ft[e], fq[e], S.mx, S.st)
                                                      : pow2_logit(ft[e], S.c_hi, S.c_lo, S.st);
            const float d = fq[e] - ft[e];
            w[e] = ep * one_minus_exp2(fmaf(d, S.d_hi, fmaf(d, S.d_lo, S.k0)));
        }
    }
}

// Sum of one vector's weights: a pairwise fp32 tree (adjacent pairs first),
// widened once.  The weights are non-negative, so its relative error stays
// below 3 * 2^-24 of the vector's own mass.
template <int VEC>
__device__ __forceinline__ double vec_sum(const float *w) {
    float p[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) p[e] = w[e];
#pragma unroll
    for (int h = 1; h < VEC; h *= 2)
#pragma unroll
        for (int e = 0; e + h < VEC; e += 2 * h) p[e] = p[e] + p[e + h];
    return static_cast<double>(p[0]);
}

// ---------------------------------------------------------------------------
// acceptance rate alpha_i = sum_v min(p~(v), q(v)) of every drafted position
// ---------------------------------------------------------------------------

// Row statistics (shift s, 1 / S) of one row from its C1 chunk partials, by
// one wavefront, in fp64 and in a fixed order; S = 0 or non-finite marks the
// row bad (1 / S is then NaN).
// Row statistics from the chunk partials: the shift s and 1 / S, and also
// off = s + log2 S, so that log2 p(v) = z c - off (NaN for a bad row).
// first: p[lane] when lane < C1, loaded by the caller ahead of other loads.
__device__ __forceinline__ void combine_row(const Part *p, int C1, const Part &first, float &s_out,
                                            float &inv_out, float &off_out) {
    const int lane = threadIdx.x & (kWave - 1);
    float smax = -INFINITY;
    if (lane < C1) smax = fmaxf(smax, first.s);
    for (int c = lane + kWave; c < C1; c += kWave) smax = fmaxf(smax, p[c].s);
    smax = wave_max(smax);
    double S = 0.0;
    if (lane < C1 && first.s != -INFINITY)
        S += first.S * pow2_shift_d(static_cast<double>(first.s) - static_cast<double>(smax));
    for (int c = lane + kWave; c < C1; c += kWave) {
        const Part q = p[c];
        if (q.s != -INFINITY) S += q.S * pow2_shift_d(static_cast<double>(q.s) - static_cast<double>(smax));
    }
    S = wave_sum_d(S);
    s_out = smax;
    const bool ok = S > 0.0 && isfinite(S) && isfinite(smax);
    inv_out = ok ? static_cast<float>(1.0 / S) : NAN;
    off_out = ok ? static_cast<float>(static_cast<double>(smax) + log2(S)) : NAN;
}

// alpha of one position, by the wave of its last chunk (own: that chunk's
// sum): the other chunks' tagged sums, one lane per chunk, each lane adding
// its chunks in chunk order, then a fixed-order wave sum.  The position's
// blocks are dispatched before the block of its last chunk, so the wave waits
// only for waves already started; a wave that gives up stores NaN and sets
// SV_DATA_SYNC.  A NaN sum (a bad row) sets SV_DATA_BAD_ROW.
__device__ __forceinline__ void alpha_fold(const ChainArgs &a, unsigned long long *rec, double own, int64_t pos) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t tag = a.tag;
    int flags = 0;
    double s = 0.0;
    for (int c0 = 0; c0 < a.C1; c0 += kWave) {
        const int c = c0 + lane;
        if (c == a.C1 - 1) {
            s += own;
        } else if (c < a.C1 - 1) {
            unsigned long long w0 = ld_agent(rec + 2 * c), w1 = ld_agent(rec + 2 * c + 1);
            poll_pair(rec + 2 * c, tag, w0, w1, flags);
            s += __longlong_as_double(static_cast<long long>((w1 << 32) | (w0 & 0xFFFFFFFFull)));
        }
    }
    s = wave_sum_d(s);
    const bool sync = __ballot(flags != 0) != 0ull;
    if (lane == 0) {
        const float out = sync ? NAN : static_cast<float>(s);
        a.alpha[pos] = out;
        const int f = (sync ? SV_DATA_SYNC : 0) | (!(out == out) && !sync ? SV_DATA_BAD_ROW : 0);
        if (f) atomicOr(a.status, f);
    }
}

// One block per (request, position, group of 4 chunks): wave 0 combines the
// target (or mixed, in logit space) row's statistics and wave 1 the draft
// row's, then wave w reduces chunk 4 g + w to the fp64 sum of
// min(p~(v), q(v)) over its elements.  Per element (probability space)
// p~ = (1 - lambda) p_t + lambda q with p(v) = 2^(z c - s) / S; in logit
// space p~(v) = 2^(alpha z_t + beta z_q - s_e) / S_e.
//
// MODE 0 (probability space, lambda > 0) forms both probabilities.  Where p~
// is itself one softmax (MODE 1: logit space; MODE 2: lambda = 0, p~ = p_t),
// min(p~, q) = 2^min(log2 p~, log2 q) with log2 p(v) = z c - (s + log2 S):
// one exponential per element instead of two.
template <class DT, int NV, int MODE>
__global__ __launch_bounds__(kBlock) void k_alpha_mass(ChainArgs a) {
    __shared__ float st_s, st_i, sq_s, sq_i, st_o, sq_o;
    const int groups = (a.C1 + kWaves - 1) / kWaves;
    const int job = blockIdx.x;
    const int grp = job % groups;
    int b, i;
    if (!slot_position(a, job / groups, b, i)) return;     // uniform over the block
    const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    // waves 0 and 1 load their row's first 64 chunk partials first (they
    // return first), then every wave its chunk of both rows, which does not
    // depend on the row statistics: the partials are combined while the
    // chunks are in flight
    const int c = grp * kWaves + wv;
    constexpr int VEC = DT::kVec;
    const int V = a.g.V;
    const Part *parts = a.part1 + (int64_t(b) * a.g.Pcap + i) * 2 * a.C1;
    Part first;
    if (wv < 2 && lane < a.C1) first = parts[wv * a.C1 + lane];
    const int r = geo_row(a.g, b, i);
    const char *row_t = row_ptr(a.g, 0, b, r);
    const char *row_q = row_ptr(a.g, 1, b, r);
    const int v0 = min(c, a.C1 - 1) * (kWave * NV);
    u32x4 dt[NV], dq[NV];
    load_chunk_clamped<DT, NV>(row_t, v0, lane, V, dt);
    load_chunk_clamped<DT, NV>(row_q, v0, lane, V, dq);
    if (wv < 2) {
        float s_, inv_, off_;
        combine_row(parts + wv * a.C1, a.C1, first, s_, inv_, off_);
        if (lane == 0) {
            if (wv == 0) {
                st_s = s_;
                st_i = inv_;
                st_o = off_;
            } else {
                sq_s = s_;
                sq_i = inv_;
                sq_o = off_;
            }
        }
    }
    __syncthreads();
    if (c >= a.C1) return;
    mask_chunk<DT, NV>(v0, lane, V, dt);
    mask_chunk<DT, NV>(v0, lane, V, dq);
    const float c_hi = a.c_hi, c_lo = a.c_lo;
    const float ts = st_s, ti = st_i, qs = sq_s, qi = sq_i;
    const float w_t = 1.0f - a.lam, w_q = a.lam;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
    const float ot = st_o, oq = sq_o;
    const float mx[4] = {a.al_hi, a.al_lo, a.be_hi, a.be_lo};
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        float ft[VEC], fq[VEC];
        DT::unpack(dt[n], ft);
        DT::unpack(dq[n], fq);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if (MODE == 0) {
                const float q = pow2_logit(fq[e], c_hi, c_lo, qs) * qi;
                const float pm = fmaf(w_t, pow2_logit(ft[e], c_hi, c_lo, ts) * ti, w_q * q);
                acc[e] += fminf(pm, q);
            } else {
                const float yq = fmaf(fq[e], c_lo, fmaf(fq[e], c_hi, -oq));
                const float yp = (MODE == 1) ? mixed_expo(ft[e], fq[e], mx, ot)
                                             : fmaf(ft[e], c_lo, fmaf(ft[e], c_hi, -ot));
                acc[e] += __builtin_amdgcn_exp2f(fminf(yp, yq));
            }
        }
    }
    double tot = wave_sum_d(vec_sum<VEC>(acc));
    // a bad row (its statistics are NaN) makes alpha NaN; fminf alone would
    // drop a NaN probability in favour of the other one
    if (!(ti == ti && qi == qi)) tot = NAN;
    unsigned long long *rec = a.alpha_rec + (int64_t(b) * a.g.Pcap + i) * a.C1 * 2;
    if (c != a.C1 - 1) {
        if (lane == 0) {
            const unsigned long long tagw = static_cast<unsigned long long>(a.tag) << 32;
            const unsigned long long bits = static_cast<unsigned long long>(__double_as_longlong(tot));
            st_agent(rec + 2 * c, tagw | (bits & 0xFFFFFFFFull));
            st_agent(rec + 2 * c + 1, tagw | (bits >> 32));
        }
        return;
    }
    alpha_fold(a, rec, tot, int64_t(b) * a.g.P + i);
}

struct ResolveShared {
    float s[2 * SV_MAX_POSITIONS];      // row shift
    double S[2 * SV_MAX_POSITIONS];     // row sum of 2^(z c - s)
    float zx[2 * SV_MAX_POSITIONS];     // logit of the drafted token
    int row_bad[2 * SV_MAX_POSITIONS];
    double a[SV_MAX_POSITIONS];
    int x[SV_MAX_POSITIONS];
    int rowi[SV_MAX_POSITIONS + 1];     // request row of position i (i <= K)
    int pathv[SV_MAX_POSITIONS];
    int tokn[SV_MAX_TREE_NODES];        // path mode: every node's drafted token
    float u[SV_MAX_POSITIONS];
    float f[kWaves2];
    int K, n, flags;
};

// Every drafted row's (shift, sum) from its C1 chunk partials, one wave per
// row, in fp64 and a fixed order, with the drafted token's logit; STAGED reads
// the partials from shared memory, otherwise from the workspace.
template <bool STAGED>
__device__ __forceinline__ void combine_rows(const ChainArgs &a, const Geo &g, ResolveShared &sh, int K, int C1,
                                             int64_t pbase, const float *ps, const double *pS, const float *pz) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
#pragma unroll 1
    for (int j = wv; j < 2 * K; j += kWaves2) {
        float smax = -INFINITY;
#pragma unroll 1
        for (int c = lane; c < C1; c += kWave)
            smax = fmaxf(smax, STAGED ? ps[j * C1 + c] : a.part1[pbase + int64_t(j) * C1 + c].s);
        smax = wave_max(smax);
        double S = 0.0;
#pragma unroll 1
        for (int c = lane; c < C1; c += kWave) {
            float s;
            double Sc;
            if (STAGED) {
                s = ps[j * C1 + c];
                Sc = pS[j * C1 + c];
            } else {
                const Part p = a.part1[pbase + int64_t(j) * C1 + c];
                s = p.s;
                Sc = p.S;
            }
            if (s != -INFINITY) S += Sc * pow2_shift_d(static_cast<double>(s) - static_cast<double>(smax));
        }
        S = wave_sum_d(S);
        if (lane == 0) {
            const int x = sh.x[j >> 1];
            float zx = NAN;
            if (x >= 0 && x < g.V) {
                const int cx = x / a.ch1;
                zx = STAGED ? pz[j * C1 + cx] : a.part1[pbase + int64_t(j) * C1 + cx].z;
            }
            sh.zx[j] = zx;
            sh.s[j] = smax;
            sh.S[j] = S;
            sh.row_bad[j] = !(S > 0.0) || !isfinite(S) || !isfinite(smax);
        }
    }
}

// Resolve request b: positions, row statistics (from the staged partials of
// launch 1, which also carry the drafted token's logit), acceptance
// probabilities and the first rejection.  One parallel load round.
template <class DT>
__device__ __forceinline__ void resolve_request(const ChainArgs &a, int b, ResolveShared &sh,
                                                float *ps, double *pS, float *pz, bool staged) {
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wv = t / kWave;
    const Geo &g = a.g;
    const int P = g.P, Pc = g.Pcap, C1 = a.C1;
    const int64_t pbase = int64_t(b) * Pc * 2 * C1;
    // Every load of the first round goes out before any value is used: the
    // partials, the position's uniform and token (or path node) and the
    // draft length are read into registers, then stored to shared memory.
    // (Stored as they arrived, a loop's waits would hold back the loads after
    // it: three round trips instead of one.)
    static_assert(kStageMax % kBlock2 == 0, "whole staging rounds");
    constexpr int kStageIter = kStageMax / kBlock2;
    const int n_stage = staged ? 2 * Pc * C1 : 0;
    Part pr[kStageIter];
#pragma unroll
    for (int k = 0; k < kStageIter; ++k) {
        const int idx = t + k * kBlock2;
        if (idx < n_stage) pr[k] = a.part1[pbase + idx];
    }
    float uv = 0.0f;
    int xv = 0;
    if (t < Pc) {
        uv = a.u_accept[int64_t(b) * P + t];
        xv = (g.path == nullptr) ? g.tokens[int64_t(b) * P + t] : g.path[int64_t(b) * P + t];
    }
    // path mode: every node's token (the path picks them after the walk)
    static_assert(SV_MAX_TREE_NODES <= kBlock2, "one node per thread");
    int tn = 0;
    if (g.path != nullptr && t < g.N) tn = g.tokens[int64_t(b) * g.N + t];
    const bool lead = t == 0 && g.path == nullptr;
    int k_len = P;
    if (lead && g.draft_len != nullptr) k_len = g.draft_len[b];
#pragma unroll
    for (int k = 0; k < kStageIter; ++k) {
        const int idx = t + k * kBlock2;
        if (idx < n_stage) {
            ps[idx] = pr[k].s;
            pz[idx] = pr[k].z;
            pS[idx] = pr[k].S;
        }
    }
    if (t < Pc) {
        sh.u[t] = uv;
        if (g.path == nullptr) sh.x[t] = xv;
        else sh.pathv[t] = xv;
    }
    if (g.path != nullptr && t < g.N) sh.tokn[t] = tn;
    if (lead) {
        int fl = 0;
        if (k_len < 0 || k_len > P) {
            fl |= SV_DATA_BAD_LENGTH;
            k_len = min(max(k_len, 0), P);
        }
        sh.K = k_len;
        sh.flags = fl;
    }
    __syncthreads();
    if (g.path != nullptr) {
        if (t == 0) {
            int d = 0, fl = 0;
            for (; d < Pc; ++d) {
                const int v = sh.pathv[d];
                if (v == -1) break;
                if (v < 1 || v > g.N) {
                    fl |= SV_DATA_BAD_TREE;
                    break;
                }
            }
            sh.K = d;
            sh.flags = fl;
        }
        __syncthreads();
        if (t < sh.K) sh.x[t] = sh.tokn[sh.pathv[t] - 1];
        if (t <= sh.K) sh.rowi[t] = (t == 0) ? 0 : sh.pathv[t - 1];
    } else if (t <= Pc) {
        sh.rowi[t] = t;
    }
    __syncthreads();
    const int K = sh.K;
    // row statistics: combine the C1 chunk partials of every row in fp64
    // (two loops, so that the staged one reads shared memory only)
    if (staged) combine_rows<true>(a, g, sh, K, C1, pbase, ps, pS, pz);
    else combine_rows<false>(a, g, sh, K, C1, pbase, ps, pS, pz);
    __syncthreads();
    if (wv == 0) {
        bool rej = false;
        int fl = 0;
        if (lane < K) {
            const int i = lane;
            const float zt = sh.zx[2 * i], zq = sh.zx[2 * i + 1];
            double acc_p;
            if (!(sh.x[i] >= 0 && sh.x[i] < g.V)) {
                fl |= SV_DATA_BAD_TOKEN;
                acc_p = 0.0;
            } else if (sh.row_bad[2 * i] || sh.row_bad[2 * i + 1]) {
                fl |= SV_DATA_BAD_ROW;
                acc_p = 0.0;
            } else if (zq == -INFINITY) {
                // q(x) = 0: accept iff p~(x) > 0.  In logit space the mixed
                // logit of x is -inf too, so p~(x) = 0.
                fl |= SV_DATA_ZERO_Q;
                acc_p = (a.space == 0 && a.lam < 1.0f && zt != -INFINITY) ? 1.0 : 0.0;
            } else if (a.lam >= 1.0f) {
                acc_p = 1.0;
            } else if (a.space == 1) {
                // slot 0 holds the mixed row (shift s_e, sum S_e) and z_t(x):
                // p~(x) / q(x) = 2^E S_q / S_e with
                // E = (alpha z_t(x) + beta z_q(x)) - c z_q(x) - (s_e - s_q)
                //   = alpha (z_t(x) - z_q(x)) - (s_e - s_q), as alpha + beta = c
                const double E = a.alpha_c * (static_cast<double>(zt) - static_cast<double>(zq)) -
                                 (static_cast<double>(sh.s[2 * i]) - static_cast<double>(sh.s[2 * i + 1]));
                const double ratio = exp2_d(E) * (sh.S[2 * i + 1] / sh.S[2 * i]);
                acc_p = fmin(1.0, ratio);
            } else {
                // p(x) = 2^(z(x) c - s) / S for either model, so
                // p_t(x) / q(x) = 2^E S_q / S_t with E = (z_t(x) - z_q(x)) c - (s_t - s_q)
                const double E = (static_cast<double>(zt) - static_cast<double>(zq)) * a.c_d -
                                 (static_cast<double>(sh.s[2 * i]) - static_cast<double>(sh.s[2 * i + 1]));
                const double ratio = exp2_d(E) * (sh.S[2 * i + 1] / sh.S[2 * i]);
                if (ratio >= 1.0) {
                    acc_p = 1.0;
                } else {
                    const double lam = static_cast<double>(a.lam);
                    acc_p = fmin(1.0, (1.0 - lam) * ratio + lam);
                }
            }
            sh.a[i] = acc_p;
            rej = !(static_cast<double>(sh.u[i]) < acc_p);
        }
        const unsigned long long mask = __ballot(rej);
        const int fl_all = wave_or8(fl);
        if (lane == 0) {
            sh.n = mask ? (__ffsll(static_cast<long long>(mask)) - 1) : K;
            sh.flags |= fl_all;
        }
    }
    __syncthreads();
}

// Hand-over of the chunk records between the mass blocks of one request,
// which may run on different XCDs (each with its own L2): every record is
// written and read as an agent-scope relaxed atomic (write-through stores and
// coherent loads), and a writer drains its stores (s_waitcnt) before the
// block counts itself done, so the last block sees every record without a
// device-wide cache writeback.
__device__ __forceinline__ void publish(double *p, double v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double collect(const double *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sampling context of request b from its hand-over record.
__device__ __forceinline__ SampleCtx sample_ctx(const ChainArgs &a, int b, const ReqRecord &r) {
    SampleCtx S;
    S.V = a.g.V;
    S.c_hi = a.c_hi;
    S.c_lo = a.c_lo;
    S.w_t = 1.0f - a.lam;
    S.w_q = a.lam;
    S.mx[0] = a.al_hi;
    S.mx[1] = a.al_lo;
    S.mx[2] = a.be_hi;
    S.mx[3] = a.be_lo;
    S.logit = a.space;
    S.d_hi = a.space ? a.al_hi : a.c_hi;
    S.d_lo = a.space ? a.al_lo : a.c_lo;
    S.k0 = r.k0;
    S.row_t = row_ptr(a.g, 0, b, r.row);
    S.row_q = (r.mode != kBonus) ? row_ptr(a.g, 1, b, r.row) : nullptr;
    S.st = r.st;
    S.it = r.it;
    S.sq = r.sq;
    S.iq = r.iq;
    return S;
}

// Chunk c of the sampling row: the bonus shift (largest logit times c_hi,
// block-wide) and the fp64 wave sum of every piece, written to the chunk
// record: [shift, unused, piece sums (wave-major)].  Every thread must call this.
template <class DT, int MODE, int NV2>
__device__ __forceinline__ void chunk_pieces(const SampleCtx &S, int c, double *rec, float *f16) {
    constexpr int VEC = DT::kVec;
    const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    u32x4 dt[NV2], dq[NV2];
#pragma unroll
    for (int n = 0; n < NV2; ++n) load_vec<DT, MODE>(S, piece_vec<NV2>(c, wv, n, lane), dt[n], dq[n]);
    float s_use = 0.0f, s_rec = 0.0f;
    if (MODE == kBonus) {
        float m = -INFINITY;
#pragma unroll
        for (int n = 0; n < NV2; ++n) {
            float f[VEC];
            DT::unpack(dt[n], f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) m = fmaxf(m, f[e]);
        }
        m = wave_max(m);
        if (lane == 0) f16[wv] = m;
        __syncthreads();
        m = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves2; ++w) m = fmaxf(m, f16[w]);
        s_rec = (m == -INFINITY) ? -INFINITY : ceilf(m * S.c_hi);   // integer: chunks rescale exactly
        s_use = (m == -INFINITY) ? 0.0f : s_rec;
    }
#pragma unroll
    for (int n = 0; n < NV2; ++n) {
        float w[VEC];
        vec_weights<DT, MODE>(S, dt[n], dq[n], s_use, w);
        const double ws = wave_sum_d(vec_sum<VEC>(w));
        if (lane == 0) publish(&rec[2 + wv * NV2 + n], ws);
    }
    if (threadIdx.x == 0) publish(&rec[0], static_cast<double>(s_rec));
}

// The draw runs on one wavefront: wave 0 of the block that counts its
// request's mass blocks complete.  Every step below is a wave-level scan, ballot or lane
// read; the only memory round trips are the piece masses (coherent loads)
// and the reload of the chosen piece.
//
// Intervals: the pieces of the sampling row, in index order, are cut into
// 64 runs of pp consecutive pieces, one run per lane.  The lanes' run masses
// are scanned in lane order, so the lane intervals [excl, incl) tile [0, W);
// inside the run that holds t = u * W the pieces are scanned again, one per
// lane, from the run's lower bound, and the run's last piece ends at the
// run's upper bound, so the piece intervals tile the run.  Rounding can still
// leave t past the last piece's lower bound with no owner: then the run's
// last positive piece is taken.  Every sum has a fixed order, so the draw is
// bitwise reproducible.

// Wave-level inverse CDF over the request's piece masses (staged in LDS:
// np doubles, then np floats of chunk shifts for the bonus row), then over
// the chosen piece's 64 vectors.  Returns -1 when the row has no positive
// mass.  All lanes of the wave must call this; the result is wave-uniform.
template <class DT, int MODE, int NV2>
__device__ __forceinline__ int locate_wave(const ChainArgs &a, int b, const SampleCtx &S, double u,
                                           double *stage) {
    constexpr int VEC = DT::kVec;
    constexpr int kPieces = kWaves2 * NV2;
    const int lane = threadIdx.x & (kWave - 1);
    const double *cr = a.chunks + int64_t(b) * a.C2 * a.rec_stride;
    const int np = a.C2 * kPieces;
    const int pp = (np + kWave - 1) / kWave;        // pieces per lane run, <= kMaxPieces / 64
    float *sstage = reinterpret_cast<float *>(stage + np);
    const int p0 = lane * pp;
    // 1. this lane's run: piece masses (and, for the bonus row, chunk shifts)
    double tot = 0.0;
    float sm = -INFINITY;
    // batches of 8 pieces with every load in flight: the loads are not
    // guarded (an index past the row's pieces reads the last one, unused),
    // so no branch separates them
    for (int j0 = 0; j0 < pp; j0 += 8) {
        double mv[8];
        float sv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int p = min(p0 + j0 + k, np - 1);
            const double *rc = cr + int64_t(p / kPieces) * a.rec_stride;
            mv[k] = collect(&rc[2 + p % kPieces]);
            if (MODE == kBonus) sv[k] = static_cast<float>(collect(&rc[0]));
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int p = p0 + j0 + k;
            if (j0 + k < pp && p < np) {
                stage[p] = mv[k];
                if (MODE == kBonus) {
                    sstage[p] = sv[k];
                    sm = fmaxf(sm, sv[k]);
                } else {
                    tot += mv[k];                    // residual chunks share shift 0
                }
            }
        }
    }
    // 2. bonus row: every piece to the common frame 2^(-largest chunk shift)
    float smax = 0.0f;
    if (MODE == kBonus) {
        smax = wave_max(sm);
#pragma unroll 4
        for (int j = 0; j < pp; ++j) {
            const int p = p0 + j;
            if (p < np) {
                const float sp = sstage[p];
                const double sc = (sp == -INFINITY) ? 0.0 : pow2_shift_d(static_cast<double>(sp) - static_cast<double>(smax));
                const double m = stage[p] * sc;
                stage[p] = m;
                tot += m;
            }
        }
    }
    // 3. the run holding t
    const double incl = wave_scan_d(tot);
    const double excl = dpp_shift_d<kDppWaveShr1, 0xF, 0xF>(incl);   // 0 at lane 0
    const double W = readlane_d(incl, kWave - 1);
    if (!(W > 0.0) || !isfinite(W)) return -1;
    const double t = u * W;
    const unsigned long long run = __ballot(excl <= t && t < incl);
    if (run == 0ull) return -1;                       // t outside [0, W): u outside [0, 1)
    const int ol = __ffsll(static_cast<long long>(run)) - 1;
    const double run_lo = readlane_d(excl, ol), run_hi = readlane_d(incl, ol);
    // 4. the piece holding t inside that run, one piece per lane (the run's
    // masses were written by lane ol: order the wave's LDS accesses)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int q = ol * pp + lane;
    const double mj = (lane < pp && q < np) ? stage[q] : 0.0;
    const double x2 = wave_scan_d(mj);
    const double lo = run_lo + dpp_shift_d<kDppWaveShr1, 0xF, 0xF>(x2);
    const double hi = (lane == pp - 1) ? run_hi : run_lo + x2;
    const unsigned long long hit = __ballot(mj > 0.0 && lo <= t && t < hi);
    const unsigned long long posm = __ballot(mj > 0.0);
    if (posm == 0ull) return -1;                      // not reached: the run has positive mass
    const int js = hit ? (__ffsll(static_cast<long long>(hit)) - 1)
                       : (63 - __clzll(static_cast<long long>(posm)));
    const int ps = ol * pp + js;
    const double lo_s = readlane_d(lo, js);
    const int cs = ps / kPieces, wsv = (ps % kPieces) / NV2, ns = ps % NV2;
    float spick = 0.0f;
    double scale = 1.0;
    if (MODE == kBonus) {
        spick = sstage[ps];
        scale = (spick == -INFINITY) ? 0.0 : pow2_shift_d(static_cast<double>(spick) - static_cast<double>(smax));
    }
    const double tp = (t - lo_s) / scale;            // target inside the piece, chunk frame
    // the chosen piece's own chunk shift, as the mass kernel used it
    const float s_use = (MODE == kBonus && spick != -INFINITY) ? spick : 0.0f;
    // 5. the token inside the piece: its 64 vectors, one per lane
    const int64_t gv = piece_vec<NV2>(cs, wsv, ns, lane);
    u32x4 dt, dq;
    load_vec<DT, MODE>(S, gv, dt, dq);
    float w[VEC];
    vec_weights<DT, MODE>(S, dt, dq, s_use, w);
    const double x = wave_scan_d(vec_sum<VEC>(w));
    const double ex = dpp_shift_d<kDppWaveShr1, 0xF, 0xF>(x);     // 0 at lane 0
    int last = -1;
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        if (w[e] > 0.0f) last = e;
    int pick = -1;
    if (ex <= tp && tp < x) {
        double cum = ex;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if (w[e] > 0.0f) {
                cum += static_cast<double>(w[e]);
                if (pick < 0 && cum > tp) pick = e;
            }
        }
        if (pick < 0) pick = last;
    }
    // The lanes hold the piece's vectors in index order.  The token is the
    // pick of the lowest lane whose interval holds tp (the intervals tile the
    // piece, so there is at most one such lane); rounding can hide the
    // crossing, and then the last positive weight of the highest lane that
    // has one is taken.  Ballots and lane reads, not LDS atomics: an atomic
    // from every lane runs as a serial loop over the lanes.
    const int base = static_cast<int>(gv * VEC);
    const unsigned long long own = __ballot(pick >= 0);
    const unsigned long long pos = __ballot(last >= 0);
    if (own) return __builtin_amdgcn_readlane(base + pick, __ffsll(static_cast<long long>(own)) - 1);
    if (pos) return __builtin_amdgcn_readlane(base + last, 63 - __clzll(static_cast<long long>(pos)));
    return -1;
}

// Zero residual mass after a rejection (reachable only through rounding):
// draw from p~ = (1 - lambda) p_t + lambda q at that row instead.  Two passes
// over the row in pages of 64 vectors (one per lane) in index order, the
// first for the total W, the second for the page, lane and element where the
// running sum first exceeds u * W (rare path: small code rather than speed).
// All lanes must call this; the result is wave-uniform.
template <class DT>
__device__ __forceinline__ int sample_mixture_wave(const SampleCtx &S, double u) {
    constexpr int VEC = DT::kVec;
    const int lane = threadIdx.x & (kWave - 1);
    const int V = S.V;
    const int nvec = (V + VEC - 1) / VEC;
    auto weights = [&](int gv, float (&w)[VEC]) {
        float ft[VEC], fq[VEC];
        DT::unpack(load_row_vec<DT, false>(S.row_t, gv, V), ft);
        DT::unpack(load_row_vec<DT, false>(S.row_q, gv, V), fq);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if (S.logit) {
                w[e] = pow2_mixed(ft[e], fq[e], S.mx, S.st) * S.it;          // p~ itself
            } else {
                const float pt = pow2_logit(ft[e], S.c_hi, S.c_lo, S.st) * S.it;
                const float pq = pow2_logit(fq[e], S.c_hi, S.c_lo, S.sq) * S.iq;
                w[e] = fmaf(S.w_t, pt, S.w_q * pq);
            }
        }
    };
    double carry = 0.0;
#pragma unroll 1
    for (int base = 0; base < nvec; base += kWave) {
        float w[VEC];
        weights(base + lane, w);                      // vectors past the row read as -inf: weight 0
        carry += readlane_d(wave_scan_d(vec_sum<VEC>(w)), kWave - 1);
    }
    const double W = carry;
    if (!(W > 0.0) || !isfinite(W)) return -1;
    const double t = u * W;
    carry = 0.0;
    int last_tok = -1;
#pragma unroll 1
    for (int base = 0; base < nvec; base += kWave) {
        float w[VEC];
        weights(base + lane, w);
        const double x = wave_scan_d(vec_sum<VEC>(w));
        const double lo = carry + dpp_shift_d<kDppWaveShr1, 0xF, 0xF>(x);
        const double hi = carry + x;
        int last = -1;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            if (w[e] > 0.0f) last = e;
        int pick = -1;
        if (lo <= t && t < hi) {                      // this lane's interval of the page holds t
            double cum = lo;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                if (w[e] > 0.0f) {
                    cum += static_cast<double>(w[e]);
                    if (pick < 0 && cum > t) pick = e;
                }
            }
            if (pick < 0) pick = last;
        }
        const unsigned long long own = __ballot(pick >= 0);
        if (own) return __builtin_amdgcn_readlane((base + lane) * VEC + pick, __ffsll(static_cast<long long>(own)) - 1);
        const unsigned long long pos = __ballot(last >= 0);
        if (pos) last_tok = __builtin_amdgcn_readlane((base + lane) * VEC + last, 63 - __clzll(static_cast<long long>(pos)));
        carry += readlane_d(x, kWave - 1);
    }
    return last_tok;                                  // t at the very top by rounding: last positive weight
}

// The sampled (corrected or bonus) token of request b, written at position
// r.n by wave 0 of the block that completed the request's mass blocks.
template <class DT, int NV2>
__device__ __forceinline__ void draw_request(const ChainArgs &a, int b, const ReqRecord &r,
                                             const SampleCtx &S, double *stage, float u_s) {
    const double u = static_cast<double>(u_s);
    int flags = 0;
    // At lambda = 1, p~ = q and the residual max(0, p~ - q) is identically
    // zero (a rejection there means q(x) = 0): straight to the fallback, p~.
    // The chunk records hold max(0, p_t - q), which is no longer the same law.
    int tok;
    if (r.mode == kResidual)
        tok = (a.lam >= 1.0f) ? -1 : locate_wave<DT, kResidual, NV2>(a, b, S, u, stage);
    else if (r.mode == kResidualLogit)
        tok = locate_wave<DT, kResidualLogit, NV2>(a, b, S, u, stage);
    else
        tok = locate_wave<DT, kBonus, NV2>(a, b, S, u, stage);
    if (tok < 0 && r.mode != kBonus && r.rows_ok) {
        flags |= SV_DATA_FALLBACK;
        tok = sample_mixture_wave<DT>(S, u);
    }
    if (tok < 0) {
        tok = -1;
        flags |= SV_DATA_BAD_ROW;
    }
    if ((threadIdx.x & (kWave - 1)) == 0) {
        a.out_tokens[int64_t(b) * (a.g.P + 1) + r.n] = tok;
        if (flags) atomicOr(a.status, flags);
    }
}


template <class DT, int NV2>
__global__ __launch_bounds__(kBlock2) void k_resolve_mass(ChainArgs a, int staged) {
    __shared__ ResolveShared sh;
    __shared__ int last;
    extern __shared__ double dyn[];
    const int b = blockIdx.x;
    const int c = blockIdx.y;
    const int stage_n = staged ? 2 * a.g.Pcap * a.C1 : 0;
    double *pS = dyn;
    float *ps = reinterpret_cast<float *>(dyn + stage_n);
    float *pz = ps + stage_n;
    // the draw's uniform, read now so that the drawing wave does not wait for it
    const float u_s = a.u_sample[b];
    resolve_request<DT>(a, b, sh, ps, pS, pz, staged != 0);

    const int n = sh.n, K = sh.K;
    ReqRecord r;
    r.n = n;
    r.st = r.sq = r.it = r.iq = r.k0 = 0.0f;
    if (n < K) {
        r.mode = (a.space == 1) ? kResidualLogit : kResidual;
        r.row = sh.rowi[n];
        r.rows_ok = !sh.row_bad[2 * n] && !sh.row_bad[2 * n + 1];
        // p(v) = 2^(z c - s) / S
        r.st = sh.s[2 * n];
        r.sq = sh.s[2 * n + 1];
        r.it = static_cast<float>(1.0 / sh.S[2 * n]);
        r.iq = static_cast<float>(1.0 / sh.S[2 * n + 1]);
        // q(v) / p(v) = 2^((z_q - z_t) d + k0): the shifts are integers, the
        // sums fp64; 0 exactly for two identical rows
        r.k0 = static_cast<float>((static_cast<double>(sh.s[2 * n]) - static_cast<double>(sh.s[2 * n + 1])) +
                                  log2(sh.S[2 * n] / sh.S[2 * n + 1]));
    } else {
        r.mode = kBonus;
        r.row = sh.rowi[K];
        r.rows_ok = 1;
    }
    if (c == 0) {
        // every output but the sampled token
        const int P = a.g.P;
        const int t = threadIdx.x;
        if (t <= P && t != n) a.out_tokens[int64_t(b) * (P + 1) + t] = (t < n) ? sh.x[t] : -1;
        if (a.accept_prob != nullptr && t < P)
            a.accept_prob[int64_t(b) * P + t] = (t < K) ? static_cast<float>(sh.a[t]) : 0.0f;
        if (t == 0) {
            a.accepted[b] = n;
            if (sh.flags) atomicOr(a.status, sh.flags);
        }
    }
    const SampleCtx S = sample_ctx(a, b, r);
    double *cr = a.chunks + (int64_t(b) * a.C2 + c) * a.rec_stride;
    if (r.mode == kResidual) chunk_pieces<DT, kResidual, NV2>(S, c, cr, sh.f);
    else if (r.mode == kResidualLogit) chunk_pieces<DT, kResidualLogit, NV2>(S, c, cr, sh.f);
    else chunk_pieces<DT, kBonus, NV2>(S, c, cr, sh.f);

    // The block counts itself done once every thread's record stores have
    // drained (one atomic per block: an atomic per wave on the request's one
    // counter serialises, 30 against 15 us on the ragged 64-request batch); wave 0 of the
    // block that brings the count to C2 sees every record of the request and
    // draws the token alone.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (a.C2 > 1) {
        if (threadIdx.x == 0) {
            last = __hip_atomic_fetch_add(&a.count[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   a.C2 - 1;
            // every block of the request has counted: zero again, so that this
            // launch may be repeated on the same statistics (new uniforms)
            if (last) __hip_atomic_store(&a.count[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!last) return;                         // uniform
    }
    // (a row of one chunk: the request's only block draws, with no count)
    if (threadIdx.x >= kWave) return;              // whole waves
    // the resolve staging area is free again: it holds the piece masses
    draw_request<DT, NV2>(a, b, r, S, dyn, u_s);
}

}  // namespace sv

// ===========================================================================
// host entry points
// ===========================================================================

namespace {

using namespace sv;

struct ChainReq {
    const void *tgt;
    int64_t ld_t;
    const void *drf;
    int64_t ld_q;
    sv_dtype dtype;
    int B, P, V, N;
    bool path_mode;
    const int32_t *tokens, *draft_len, *path;
    const float *u_accept, *u_sample;
    float lam, T;
    int32_t *accepted, *out_tokens;
    float *accept_prob;
    int32_t *status;
    void *ws;
    size_t ws_bytes;
    hipStream_t stream;
    hipEvent_t ev_start, ev_stop;   // optional: attached to the row-statistics launch
    int space;                      // 1: logit-space mixture (only for 0 < lambda < 1)
    float *zero_f;                  // optional: floats the row-statistics launch sets to 0
    int64_t zero_f_n;
};

int choose_nv(int B, int P, int V, int vec) { return choose_stream_nv(2LL * B * P, V, vec); }


int pcap(const ChainReq &q) { return q.path_mode ? std::min(q.P, q.N) : q.P; }

// Vectors per lane and tensor of a row-stats job.  Logit-space jobs read the
// target and draft chunks together: 4 vectors of each (8 KB per wave) unless
// that leaves fewer than 2048 jobs, then 2.  Depends only on the call's sizes
// and mode, so both launches of a call agree on the chunk geometry.
int choose_nv_mode(const ChainReq &q, int vec) {
    if (q.space == 1) return int64_t(q.B) * pcap(q) * c1_for(q.V, 4, vec) < 2048 ? 2 : 4;
    return choose_nv(q.B, pcap(q), q.V, vec);
}

// Everything but the workspace.
sv_status validate_args(const ChainReq &q) {
    const int eb = elem_bytes(q.dtype);
    if (eb == 0) return SV_EDTYPE;
    if (q.B < 0 || q.P < 0 || q.P > SV_MAX_POSITIONS || q.V < 1 || q.N < 0 ||
        q.N > SV_MAX_TREE_NODES || q.B > (1 << 30) || c2_for(q.V, 16 / eb, 2) > kMaxC2)
        return SV_EINVAL;
    sv_status st = check_scalars(q.lam, q.T);
    if (st != SV_OK) return st;
    if (q.B == 0) return SV_OK;
    if (!q.u_sample || !q.accepted || !q.out_tokens) return SV_ENULL;
    if ((st = check_logits(q.tgt, q.ld_t, q.V, eb)) != SV_OK) return st;
    if (q.P > 0) {
        if (!q.u_accept) return SV_ENULL;
        if ((st = check_logits(q.drf, q.ld_q, q.V, eb)) != SV_OK) return st;
        if (q.path_mode) {
            if (!q.path || (q.N > 0 && !q.tokens)) return SV_ENULL;
        } else if (!q.tokens) {
            return SV_ENULL;
        }
    }
    if (int64_t(q.B) * pcap(q) * 2 * c1_for(q.V, kMinNV, kMinVec) >= (int64_t(1) << 31)) return SV_EINVAL;
    return SV_OK;
}

sv_status validate(const ChainReq &q) {
    const sv_status st = validate_args(q);
    if (st != SV_OK || q.B == 0) return st;
    const ChainLayout L = chain_layout(q.B, pcap(q), q.V);
    if (!q.ws || !aligned16(q.ws) || q.ws_bytes < static_cast<size_t>(L.total)) return SV_EWORKSPACE;
    return SV_OK;
}

ChainArgs make_args(const ChainReq &q, int vec, int nv) {
    const ChainLayout L = chain_layout(q.B, pcap(q), q.V);
    char *ws = static_cast<char *>(q.ws);
    ChainArgs a;
    a.g.tgt = static_cast<const char *>(q.tgt);
    a.g.drf = static_cast<const char *>(q.drf);
    a.g.ld_t = q.ld_t;
    a.g.ld_q = q.ld_q;
    a.g.req_t = q.path_mode ? q.N + 1 : q.P + 1;
    a.g.req_q = q.path_mode ? q.N + 1 : q.P;
    a.g.elem = elem_bytes(q.dtype);
    a.g.V = q.V;
    a.g.P = q.P;
    a.g.Pcap = q.path_mode ? std::min(q.P, q.N) : q.P;
    a.g.N = q.N;
    a.g.tokens = q.tokens;
    a.g.draft_len = q.path_mode ? nullptr : q.draft_len;
    a.g.path = q.path_mode ? q.path : nullptr;
    a.packed = (a.g.draft_len != nullptr && q.B <= kPackChunks * kWave) ? 1 : 0;
    a.B = q.B;
    a.u_accept = q.u_accept;
    a.u_sample = q.u_sample;
    a.lam = q.lam;
    temperature_split(q.T, &a.c_hi, &a.c_lo, &a.c_d);
    a.accepted = q.accepted;
    a.out_tokens = q.out_tokens;
    a.accept_prob = q.accept_prob;
    a.status = q.status ? q.status : reinterpret_cast<int32_t *>(ws + L.status);
    a.part1 = reinterpret_cast<Part *>(ws + L.part1);
    a.count = reinterpret_cast<int *>(ws + L.count);
    a.chunks = reinterpret_cast<double *>(ws + L.chunks);
    a.C1 = c1_for(q.V, nv, vec);
    a.ch1 = 64 * nv * vec;
    a.NV2 = choose_nv2(q.B, q.V, vec);
    a.C2 = c2_for(q.V, vec, a.NV2);
    a.rec_stride = chunk_rec_doubles(a.NV2);
    a.fill = nullptr;
    a.fill_n = 0;
    a.fill_val = 0;
    a.zero_word = nullptr;
    a.zero_f = q.zero_f;
    a.zero_f_n = q.zero_f_n;
    a.leaf_par = nullptr;
    a.leaf_N = 0;
    a.alpha_rec = nullptr;
    a.tag = 0;
    a.space = q.space;
    a.alpha_c = (1.0 - static_cast<double>(q.lam)) * a.c_d;
    a.beta_c = static_cast<double>(q.lam) * a.c_d;
    split_positive(a.alpha_c, &a.al_hi, &a.al_lo);
    split_positive(a.beta_c, &a.be_hi, &a.be_lo);
    return a;
}

template <class DT>
sv_status run_typed(const ChainReq &q, int which) {
    const int nv = choose_nv_mode(q, DT::kVec);
    const ChainArgs a = make_args(q, DT::kVec, nv);
    // the draw stages at most kMaxPieces piece masses in LDS (always true for
    // the vocabularies validate() accepts; checked before any launch)
    const int64_t n_pieces = int64_t(a.C2) * kWaves2 * a.NV2;
    if (n_pieces > kMaxPieces) return SV_EINVAL;
    if ((which & 1) && a.space == 1) {
        const int jobs = static_cast<int>(int64_t(q.B) * a.g.Pcap * a.C1);
        const dim3 grid(static_cast<unsigned>(jobs > 0 ? cdiv(jobs, kStatsWaves) : 1));
        const dim3 block(kStatsWaves * kWave);
        if (nv == 4)
            launch_timed(k_row_stats_logit<DT, 4>, grid, block, 0, q.stream, q.ev_start, q.ev_stop, a, jobs);
        else
            launch_timed(k_row_stats_logit<DT, 2>, grid, block, 0, q.stream, q.ev_start, q.ev_stop, a, jobs);
        if (hipGetLastError() != hipSuccess) return SV_EHIP;
    } else if (which & 1) {
        const int jobs = static_cast<int>(int64_t(q.B) * a.g.Pcap * 2 * a.C1);
        const dim3 grid(static_cast<unsigned>(jobs > 0 ? cdiv(jobs, kStatsWaves) : 1));
        const dim3 block(kStatsWaves * kWave);
        if (nv == 8 && jobs >= kPrioJobs)
            launch_timed(k_row_stats<DT, 8, true>, grid, block, 0, q.stream, q.ev_start, q.ev_stop, a, jobs);
        else if (nv == 8)
            launch_timed(k_row_stats<DT, 8, false>, grid, block, 0, q.stream, q.ev_start, q.ev_stop, a, jobs);
        else if (nv == 4)
            launch_timed(k_row_stats<DT, 4, false>, grid, block, 0, q.stream, q.ev_start, q.ev_stop, a, jobs);
        else
            launch_timed(k_row_stats<DT, 2, false>, grid, block, 0, q.stream, q.ev_start, q.ev_stop, a, jobs);
        if (hipGetLastError() != hipSuccess) return SV_EHIP;
    }
    if (which & 2) {
        const int64_t stage_n = int64_t(2) * a.g.Pcap * a.C1;
        const int staged = stage_n <= kStageMax ? 1 : 0;
        // the resolve staging area, reused by the draw for the piece masses
        // (a double and a float each)
        const size_t lds = std::max(staged ? static_cast<size_t>(stage_n) * (sizeof(double) + 2 * sizeof(float)) : 0,
                                    static_cast<size_t>(n_pieces) * (sizeof(double) + sizeof(float)));
        const dim3 grid(static_cast<unsigned>(q.B), static_cast<unsigned>(a.C2));
        // the events time the call's first launch: this one when it runs alone
        hipEvent_t e0 = (which & 1) ? nullptr : q.ev_start, e1 = (which & 1) ? nullptr : q.ev_stop;
        const uint32_t ldsb = static_cast<uint32_t>(lds);
        if (a.NV2 == 8) {
            launch_timed(k_resolve_mass<DT, 8>, grid, dim3(kBlock2), ldsb, q.stream, e0, e1, a, staged);
        } else if (a.NV2 == 4) {
            launch_timed(k_resolve_mass<DT, 4>, grid, dim3(kBlock2), ldsb, q.stream, e0, e1, a, staged);
        } else if (a.NV2 == 2) {
            launch_timed(k_resolve_mass<DT, 2>, grid, dim3(kBlock2), ldsb, q.stream, e0, e1, a, staged);
        } else {
            launch_timed(k_resolve_mass<DT, 1>, grid, dim3(kBlock2), ldsb, q.stream, e0, e1, a, staged);
        }
        if (hipGetLastError() != hipSuccess) return SV_EHIP;
    }
    return SV_OK;
}

// Row statistics of rows 0 .. R-1 of every request of [B, R, V] target and
// draft logits: the first launch of a chain call with one position per row and
// no drafted tokens.
template <class DT>
sv_status rows_stats_typed(ChainArgs a, hipStream_t stream, int nv) {
    const int jobs = static_cast<int>(int64_t(a.B) * a.g.Pcap * (a.space == 1 ? 1 : 2) * a.C1);
    const dim3 grid(static_cast<unsigned>(jobs > 0 ? cdiv(jobs, kStatsWaves) : 1));
    const dim3 block(kStatsWaves * kWave);
    if (a.space == 1 && a.leaf_par != nullptr) {
        if (nv == 4) hipLaunchKernelGGL((k_row_stats_logit<DT, 4, true>), grid, block, 0, stream, a, jobs);
        else hipLaunchKernelGGL((k_row_stats_logit<DT, 2, true>), grid, block, 0, stream, a, jobs);
    } else if (a.space == 1) {
        if (nv == 4) hipLaunchKernelGGL((k_row_stats_logit<DT, 4>), grid, block, 0, stream, a, jobs);
        else hipLaunchKernelGGL((k_row_stats_logit<DT, 2>), grid, block, 0, stream, a, jobs);
    } else if (a.leaf_par != nullptr) {
        if (nv == 8) hipLaunchKernelGGL((k_row_stats<DT, 8, false, true>), grid, block, 0, stream, a, jobs);
        else if (nv == 4) hipLaunchKernelGGL((k_row_stats<DT, 4, false, true>), grid, block, 0, stream, a, jobs);
        else hipLaunchKernelGGL((k_row_stats<DT, 2, false, true>), grid, block, 0, stream, a, jobs);
    } else if (nv == 8 && jobs >= kPrioJobs) {
        hipLaunchKernelGGL((k_row_stats<DT, 8, true>), grid, block, 0, stream, a, jobs);
    } else if (nv == 8) {
        hipLaunchKernelGGL((k_row_stats<DT, 8, false>), grid, block, 0, stream, a, jobs);
    } else if (nv == 4) {
        hipLaunchKernelGGL((k_row_stats<DT, 4, false>), grid, block, 0, stream, a, jobs);
    } else {
        hipLaunchKernelGGL((k_row_stats<DT, 2, false>), grid, block, 0, stream, a, jobs);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

template <class DT, int NV>
void launch_alpha(const ChainArgs &a, hipStream_t stream) {
    const int groups = (a.C1 + kWaves - 1) / kWaves;
    const dim3 grid(static_cast<unsigned>(int64_t(a.B) * a.g.Pcap * groups));
    if (a.space == 1)
        hipLaunchKernelGGL((k_alpha_mass<DT, NV, 1>), grid, dim3(kBlock), 0, stream, a);
    else if (a.lam == 0.0f)
        hipLaunchKernelGGL((k_alpha_mass<DT, NV, 2>), grid, dim3(kBlock), 0, stream, a);
    else
        hipLaunchKernelGGL((k_alpha_mass<DT, NV, 0>), grid, dim3(kBlock), 0, stream, a);
}

// The acceptance-rate call: row statistics (as the verify call's first
// launch, no drafted tokens, which also clears alpha), then the per-chunk
// min(p~, q) masses, each position summed by the wave of its last chunk.
template <class DT>
sv_status run_alpha_typed(const ChainReq &q, float *alpha) {
    const int nv = choose_nv_mode(q, DT::kVec);
    ChainArgs a = make_args(q, DT::kVec, nv);
    a.alpha_rec = reinterpret_cast<unsigned long long *>(static_cast<char *>(q.ws) +
                                                         alpha_layout_parts(q.B, pcap(q), q.V));
    a.tag = next_call_tag();
    a.alpha = alpha;
    // the statistics launch also clears every alpha (undrafted positions stay 0)
    ChainReq qs = q;
    qs.zero_f = alpha;
    qs.zero_f_n = int64_t(q.B) * q.P;
    sv_status st = run_typed<DT>(qs, 1);
    if (st != SV_OK) return st;
    if (a.g.Pcap > 0) {
        if (nv == 8) launch_alpha<DT, 8>(a, q.stream);
        else if (nv == 4) launch_alpha<DT, 4>(a, q.stream);
        else launch_alpha<DT, 2>(a, q.stream);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

sv_status run_chain(const ChainReq &q, int which) {
    const sv_status st = validate(q);
    if (st != SV_OK || q.B == 0) return st;
    return q.dtype == SV_BF16 ? run_typed<Bf16>(q, which) : run_typed<F32>(q, which);
}

ChainReq chain_req(const void *t, int64_t ld_t, const void *d, int64_t ld_q, sv_dtype dt, int B,
                   int K, int V, const int32_t *tok, const int32_t *dl, const float *ua,
                   const float *us, float lam, float T, int32_t *acc, int32_t *out, float *ap,
                   int32_t *status, void *ws, size_t wsb, hipStream_t s) {
    ChainReq q;
    q.tgt = t;
    q.ld_t = ld_t;
    q.drf = d;
    q.ld_q = ld_q;
    q.dtype = dt;
    q.B = B;
    q.P = K;
    q.V = V;
    q.N = 0;
    q.path_mode = false;
    q.tokens = tok;
    q.draft_len = dl;
    q.path = nullptr;
    q.u_accept = ua;
    q.u_sample = us;
    q.lam = lam;
    q.T = T;
    q.accepted = acc;
    q.out_tokens = out;
    q.accept_prob = ap;
    q.status = status;
    q.ws = ws;
    q.ws_bytes = wsb;
    q.stream = s;
    q.ev_start = nullptr;
    q.ev_stop = nullptr;
    q.space = 0;
    q.zero_f = nullptr;
    q.zero_f_n = 0;
    return q;
}

}  // namespace

// Workspace of sv_chain_verify_noalloc: one copy per GPU, held until the
// process ends.  Its name is a host-side stand-in in host code; the kernels
// get the device address that hipGetSymbolAddress returns for the current
// device.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];      // device address of `scratch`, per device, once looked up

// The current device's copy of `scratch`, looked up on the first call made
// with that device current.
sv_status scratch_for_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SV_EHIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SV_OK;
}

}  // namespace

namespace sv {

int rows_stats_chunks(int B, int R, int V, sv_dtype dtype, int space) {
    const int vec = 16 / elem_bytes(dtype);
    const int nv = (space == 1) ? (int64_t(B) * R * c1_for(V, 4, vec) < 2048 ? 2 : 4)
                                : choose_stream_nv(2LL * B * R, V, vec);
    return c1_for(V, nv, vec);
}

sv_status rows_stats(const void *tgt, int64_t ld_t, const void *drf, int64_t ld_q, sv_dtype dtype, int B, int R,
                     int V, float lam, float T, int space, Part *part1, int *count, int32_t *status,
                     hipStream_t stream, unsigned long long *fill, int64_t fill_n, unsigned long long fill_val,
                     unsigned *zero_word, const int32_t *leaf_par) {
    const int eb = elem_bytes(dtype);
    const int vec = 16 / eb;
    const int nv = (space == 1) ? (int64_t(B) * R * c1_for(V, 4, vec) < 2048 ? 2 : 4)
                                : choose_stream_nv(2LL * B * R, V, vec);
    ChainArgs a{};
    a.g.tgt = static_cast<const char *>(tgt);
    a.g.drf = static_cast<const char *>(drf);
    a.g.ld_t = ld_t;
    a.g.ld_q = ld_q;
    a.g.req_t = R;
    a.g.req_q = R;
    a.g.elem = eb;
    a.g.V = V;
    a.g.P = R;
    a.g.Pcap = R;
    a.g.N = 0;
    a.g.tokens = nullptr;
    a.g.draft_len = nullptr;
    a.g.path = nullptr;
    a.packed = 0;
    a.B = B;
    a.lam = lam;
    temperature_split(T, &a.c_hi, &a.c_lo, &a.c_d);
    a.status = status;
    a.part1 = part1;
    a.count = count;
    a.C1 = c1_for(V, nv, vec);
    a.ch1 = 64 * nv * vec;
    a.space = space;
    a.alpha_c = (1.0 - static_cast<double>(lam)) * a.c_d;
    a.beta_c = static_cast<double>(lam) * a.c_d;
    split_positive(a.alpha_c, &a.al_hi, &a.al_lo);
    split_positive(a.beta_c, &a.be_hi, &a.be_lo);
    a.fill = fill;
    a.fill_n = fill_n;
    a.fill_val = fill_val;
    a.zero_word = zero_word;
    a.leaf_par = leaf_par;
    a.leaf_N = R - 1;
    return dtype == SV_BF16 ? rows_stats_typed<Bf16>(a, stream, nv) : rows_stats_typed<F32>(a, stream, nv);
}

}  // namespace sv

extern "C" {

const char *sv_status_string(sv_status s) {
    switch (s) {
        case SV_OK: return "SV_OK: success";
        case SV_EINVAL: return "SV_EINVAL: size or scalar argument out of range";
        case SV_ENULL: return "SV_ENULL: required pointer is NULL";
        case SV_EALIGN: return "SV_EALIGN: logits pointer or row stride not 16-byte aligned, or ld < V";
        case SV_EWORKSPACE: return "SV_EWORKSPACE: workspace missing, misaligned or too small";
        case SV_EDTYPE: return "SV_EDTYPE: unknown dtype";
        case SV_EHIP: return "SV_EHIP: kernel launch failed";
        case SV_ETOOBIG: return "SV_ETOOBIG: the call needs more scratch than sv_chain_verify_noalloc holds";
        default: break;
    }
    return "unknown sv_status";
}

size_t sv_chain_workspace_bytes(int B, int K, int V) {
    if (B < 0 || K < 0 || K > SV_MAX_POSITIONS || V < 1) return 0;
    return static_cast<size_t>(chain_layout(B, K, V).total);
}

sv_status sv_chain_verify(const void *target_logits, int64_t ld_t, const void *draft_logits,
                          int64_t ld_q, sv_dtype dtype, int B, int K, int V,
                          const int32_t *draft_tokens, const int32_t *draft_len,
                          const float *u_accept, const float *u_sample, float lambda,
                          float temperature, int32_t *accepted, int32_t *out_tokens,
                          float *accept_prob, int32_t *status, void *workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    return run_chain(chain_req(target_logits, ld_t, draft_logits, ld_q, dtype, B, K, V,
                               draft_tokens, draft_len, u_accept, u_sample, lambda, temperature,
                               accepted, out_tokens, accept_prob, status, workspace,
                               workspace_bytes, stream),
                     3);
}

sv_status sv_chain_verify_noalloc(const void *target_logits, int64_t ld_t, const void *draft_logits,
                                  int64_t ld_q, sv_dtype dtype, int B, int K, int V,
                                  const int32_t *draft_tokens, const int32_t *draft_len,
                                  const float *u_accept, const float *u_sample, float lambda,
                                  float temperature, int32_t *accepted, int32_t *out_tokens,
                                  float *accept_prob, int32_t *status, hipStream_t stream) {
    ChainReq q = chain_req(target_logits, ld_t, draft_logits, ld_q, dtype, B, K, V, draft_tokens,
                           draft_len, u_accept, u_sample, lambda, temperature, accepted,
                           out_tokens, accept_prob, status, nullptr, 0, stream);
    sv_status st = validate_args(q);
    if (st != SV_OK || q.B == 0) return st;
    if (chain_layout(q.B, pcap(q), q.V).total > static_cast<int64_t>(SV_NOALLOC_SCRATCH_BYTES))
        return SV_ETOOBIG;
    if ((st = scratch_for_current_device(&q.ws)) != SV_OK) return st;
    q.ws_bytes = SV_NOALLOC_SCRATCH_BYTES;
    return q.dtype == SV_BF16 ? run_typed<Bf16>(q, 3) : run_typed<F32>(q, 3);
}

sv_status sv_chain_row_stats(const void *target_logits, int64_t ld_t, const void *draft_logits,
                             int64_t ld_q, sv_dtype dtype, int B, int K, int V,
                             const int32_t *draft_tokens, const int32_t *draft_len,
                             const float *u_accept, const float *u_sample, float lambda,
                             float temperature, int32_t *accepted, int32_t *out_tokens,
                             float *accept_prob, int32_t *status, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    return run_chain(chain_req(target_logits, ld_t, draft_logits, ld_q, dtype, B, K, V,
                               draft_tokens, draft_len, u_accept, u_sample, lambda, temperature,
                               accepted, out_tokens, accept_prob, status, workspace,
                               workspace_bytes, stream),
                     1);
}

sv_status sv_chain_row_stats_timed(const void *target_logits, int64_t ld_t,
                                   const void *draft_logits, int64_t ld_q, sv_dtype dtype, int B,
                                   int K, int V, const int32_t *draft_tokens,
                                   const int32_t *draft_len, const float *u_accept,
                                   const float *u_sample, float lambda, float temperature,
                                   int32_t *accepted, int32_t *out_tokens, float *accept_prob,
                                   int32_t *status, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream, hipEvent_t kernel_start,
                                   hipEvent_t kernel_stop) {
    ChainReq q = chain_req(target_logits, ld_t, draft_logits, ld_q, dtype, B, K, V, draft_tokens,
                           draft_len, u_accept, u_sample, lambda, temperature, accepted,
                           out_tokens, accept_prob, status, workspace, workspace_bytes, stream);
    q.ev_start = kernel_start;
    q.ev_stop = kernel_stop;
    return run_chain(q, 1);
}

sv_status sv_chain_verify_ex(const void *target_logits, int64_t ld_t, const void *draft_logits,
                             int64_t ld_q, sv_dtype dtype, int B, int K, int V,
                             const int32_t *draft_tokens, const int32_t *draft_len,
                             const float *u_accept, const float *u_sample, float lambda,
                             float temperature, int32_t *accepted, int32_t *out_tokens,
                             float *accept_prob, int32_t *status, void *workspace,
                             size_t workspace_bytes, hipStream_t stream, int mix_space, int stages,
                             hipEvent_t kernel_start, hipEvent_t kernel_stop) {
    if ((mix_space != SV_MIX_PROB && mix_space != SV_MIX_LOGIT) || stages < 1 || stages > 3)
        return SV_EINVAL;
    ChainReq q = chain_req(target_logits, ld_t, draft_logits, ld_q, dtype, B, K, V, draft_tokens,
                           draft_len, u_accept, u_sample, lambda, temperature, accepted,
                           out_tokens, accept_prob, status, workspace, workspace_bytes, stream);
    // at lambda = 0 or 1 the logit mixture is one model's own logits: the
    // probability-space path computes exactly that
    q.space = (mix_space == SV_MIX_LOGIT && lambda > 0.0f && lambda < 1.0f) ? 1 : 0;
    q.ev_start = kernel_start;
    q.ev_stop = kernel_stop;
    return run_chain(q, stages);
}

size_t sv_chain_acceptance_workspace_bytes(int B, int K, int V) {
    if (B < 0 || K < 0 || K > SV_MAX_POSITIONS || V < 1) return 0;
    return static_cast<size_t>(alpha_layout_total(B, K, V));
}

sv_status sv_chain_acceptance_rate(const void *target_logits, int64_t ld_t, const void *draft_logits,
                                   int64_t ld_q, sv_dtype dtype, int B, int K, int V,
                                   const int32_t *draft_len, float lambda, float temperature,
                                   int mix_space, float *alpha, int32_t *status, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    if (mix_space != SV_MIX_PROB && mix_space != SV_MIX_LOGIT) return SV_EINVAL;
    const int eb = elem_bytes(dtype);
    if (eb == 0) return SV_EDTYPE;
    if (B < 0 || K < 0 || K > SV_MAX_POSITIONS || V < 1 || B > (1 << 30)) return SV_EINVAL;
    sv_status st = check_scalars(lambda, temperature);
    if (st != SV_OK) return st;
    if (B == 0 || K == 0) return SV_OK;
    if (!alpha) return SV_ENULL;
    if ((st = check_logits(target_logits, ld_t, V, eb)) != SV_OK) return st;
    if ((st = check_logits(draft_logits, ld_q, V, eb)) != SV_OK) return st;
    if (int64_t(B) * K * 2 * c1_for(V, kMinNV, kMinVec) >= (int64_t(1) << 31)) return SV_EINVAL;
    if (!workspace || !aligned16(workspace) ||
        workspace_bytes < static_cast<size_t>(alpha_layout_total(B, K, V)))
        return SV_EWORKSPACE;
    ChainReq q = chain_req(target_logits, ld_t, draft_logits, ld_q, dtype, B, K, V, nullptr,
                           draft_len, nullptr, nullptr, lambda, temperature, nullptr, nullptr,
                           nullptr, status, workspace, workspace_bytes, stream);
    q.space = (mix_space == SV_MIX_LOGIT && lambda > 0.0f && lambda < 1.0f) ? 1 : 0;
    return dtype == SV_BF16 ? run_alpha_typed<Bf16>(q, alpha) : run_alpha_typed<F32>(q, alpha);
}

sv_status sv_chain_accept_resample(const void *target_logits, int64_t ld_t,
                                   const void *draft_logits, int64_t ld_q, sv_dtype dtype, int B,
                                   int K, int V, const int32_t *draft_tokens,
                                   const int32_t *draft_len, const float *u_accept,
                                   const float *u_sample, float lambda, float temperature,
                                   int32_t *accepted, int32_t *out_tokens, float *accept_prob,
                                   int32_t *status, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
    return run_chain(chain_req(target_logits, ld_t, draft_logits, ld_q, dtype, B, K, V,
                               draft_tokens, draft_len, u_accept, u_sample, lambda, temperature,
                               accepted, out_tokens, accept_prob, status, workspace,
                               workspace_bytes, stream),
                     2);
}

sv_status sv_tree_verify_path(const void *target_logits, int64_t ld_t, const void *draft_logits,
                              int64_t ld_q, sv_dtype dtype, int B, int N, int V,
                              const int32_t *node_token, const int32_t *path, int Dmax,
                              const float *u_accept, const float *u_sample, float lambda,
                              float temperature, int32_t *accepted, int32_t *out_tokens,
                              float *accept_prob, int32_t *status, void *workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    if (N < 0 || N > SV_MAX_TREE_NODES || Dmax < 0 || Dmax > SV_MAX_POSITIONS) return SV_EINVAL;
    ChainReq q = chain_req(target_logits, ld_t, draft_logits, ld_q, dtype, B, Dmax, V, node_token,
                           nullptr, u_accept, u_sample, lambda, temperature, accepted, out_tokens,
                           accept_prob, status, workspace, workspace_bytes, stream);
    q.N = N;
    q.path_mode = true;
    q.path = path;
    return run_chain(q, 3);
}

sv_status sv_tree_verify_path_ex(const void *target_logits, int64_t ld_t, const void *draft_logits,
                                 int64_t ld_q, sv_dtype dtype, int B, int N, int V,
                                 const int32_t *node_token, const int32_t *path, int Dmax,
                                 const float *u_accept, const float *u_sample, float lambda,
                                 float temperature, int32_t *accepted, int32_t *out_tokens,
                                 float *accept_prob, int32_t *status, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream, int mix_space) {
    if (mix_space != SV_MIX_PROB && mix_space != SV_MIX_LOGIT) return SV_EINVAL;
    if (N < 0 || N > SV_MAX_TREE_NODES || Dmax < 0 || Dmax > SV_MAX_POSITIONS) return SV_EINVAL;
    ChainReq q = chain_req(target_logits, ld_t, draft_logits, ld_q, dtype, B, Dmax, V, node_token,
                           nullptr, u_accept, u_sample, lambda, temperature, accepted, out_tokens,
                           accept_prob, status, workspace, workspace_bytes, stream);
    q.N = N;
    q.path_mode = true;
    q.path = path;
    q.space = (mix_space == SV_MIX_LOGIT && lambda > 0.0f && lambda < 1.0f) ? 1 : 0;
    return run_chain(q, 3);
}

}  // extern "C"
