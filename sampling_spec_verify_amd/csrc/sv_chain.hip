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
//     and reduces it to (shift s, S = sum 2^(z c - s)) with c = log2(e)/T.
//     Every drafted target and draft row is read exactly once.  Waves are
//     independent (no LDS, no barrier); block 0 also clears the per-request
//     completion counters and the status word used by launch 2.
//
//  2. k_accept_resample: grid (C2 chunks, B requests), 256 threads.  Every
//     block first resolves its request (combines the row partials in fp64,
//     gathers z(x_i), computes a_i in fp64, ballots the first rejection n),
//     then reduces its chunk of the sampling row: the residual
//     max(0, p_t - q) at row n (the same normalised law as max(0, p~ - q),
//     since p~ - q = (1 - lambda)(p_t - q)), or the bonus softmax(z/T) at the
//     request's last target row.  Chunk masses go to the workspace; the last
//     block of the request (integer done-counter) scans them in fp64, finds
//     the chunk holding u * W, re-reads that chunk (L2 / MALL resident),
//     scans it in LDS and writes the outputs.
//
// Path mode reuses both launches with a row indirection: position j of a
// request uses target and draft row n_j of its draft tree (n_0 = root).
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>

#include "sv_common.hpp"
#include "sv_device.hpp"

namespace sv {

// ---------------------------------------------------------------------------
// request geometry
// ---------------------------------------------------------------------------

// Number of drafted positions of request b; data errors OR-ed into *flags.
__device__ __forceinline__ int geo_positions(const Geo &g, int b, int *flags) {
    if (g.path == nullptr) {
        if (g.draft_len == nullptr) return g.P;
        int k = g.draft_len[b];
        if (k < 0 || k > g.P) {
            *flags |= SV_DATA_BAD_LENGTH;
            k = min(max(k, 0), g.P);
        }
        return k;
    }
    int d = 0;
    for (; d < g.Pcap; ++d) {
        const int v = g.path[int64_t(b) * g.P + d];
        if (v == -1) break;
        if (v < 1 || v > g.N) {
            *flags |= SV_DATA_BAD_TREE;
            break;
        }
    }
    return d;
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

__device__ __forceinline__ const char *row_ptr(const Geo &g, int tensor, int b, int r) {
    if (tensor == 0)
        return g.tgt + (int64_t(b) * g.req_t * g.ld_t + int64_t(r) * g.ld_t) * g.elem;
    return g.drf + (int64_t(b) * g.req_q * g.ld_q + int64_t(r) * g.ld_q) * g.elem;
}

// ---------------------------------------------------------------------------
// launch 1: row statistics
// ---------------------------------------------------------------------------

template <class DT, int NV>
__global__ __launch_bounds__(kBlock) void k_row_stats(ChainArgs a, int64_t n_jobs) {
    if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < a.B; i += kBlock) a.counters[i] = 0;
        if (threadIdx.x == 0) *a.status = 0;
    }
    const int64_t job = int64_t(blockIdx.x) * kWaves + (threadIdx.x / kWave);
    if (job >= n_jobs) return;
    const int C1 = a.C1;
    const int c = static_cast<int>(job % C1);
    int64_t rest = job / C1;
    const int tensor = static_cast<int>(rest & 1);
    rest >>= 1;
    const int i = static_cast<int>(rest % a.g.Pcap);
    const int b = static_cast<int>(rest / a.g.Pcap);
    int flags = 0;
    if (i >= geo_positions(a.g, b, &flags)) return;
    const char *row = row_ptr(a.g, tensor, b, geo_row(a.g, b, i));

    constexpr int VEC = DT::kVec;
    const int lane = threadIdx.x & (kWave - 1);
    const int V = a.g.V;
    const int64_t v0 = int64_t(c) * (kWave * NV);

    u32x4 d[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        const int64_t gv = v0 + n * kWave + lane;
        if (gv * VEC < V) {
            d[n] = load16(row + gv * 16);
        } else {
            d[n] = u32x4{DT::kNegInfWord, DT::kNegInfWord, DT::kNegInfWord, DT::kNegInfWord};
        }
    }
    float f[NV][VEC];
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        DT::unpack(d[n], f[n]);
        const int64_t lim = int64_t(V) - (v0 + n * kWave + lane) * VEC;
        if (lim < VEC) {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if (e >= lim) f[n][e] = -INFINITY;
        }
    }
    float m = -INFINITY;
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int e = 0; e < VEC; ++e) m = fmaxf(m, f[n][e]);

    const float c_hi = a.c_hi, c_lo = a.c_lo;
    const float s_lane = (m == -INFINITY) ? -INFINITY : m * c_hi;
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
    const float fac = (s_lane == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s_lane - s_w);
    const double S_w = wave_sum_d(static_cast<double>(S_lane) * static_cast<double>(fac));
    if (lane == 0) {
        Part p;
        p.s = s_w;
        p.pad = 0.0f;
        p.S = S_w;
        a.part1[((int64_t(b) * a.g.Pcap + i) * 2 + tensor) * C1 + c] = p;
    }
}

// ---------------------------------------------------------------------------
// launch 2: resolve + resample
// ---------------------------------------------------------------------------

enum SampleMode { kResidual = 0, kBonus = 1, kMixture = 2 };

struct SampleCtx {
    int mode;
    const char *row_t;      // target row of the sampling position
    const char *row_q;      // draft row (residual / mixture)
    float c_hi, c_lo;
    float st_hi, st_lo;     // log2-domain normaliser shift of the target row
    float sq_hi, sq_lo;     // ... of the draft row
    float w_t, w_q;         // mixture weights (1 - lambda, lambda)
    int V;
};

__device__ __forceinline__ float log2_prob(float z, float c_hi, float c_lo, float s_hi, float s_lo) {
    return fmaf(z, c_lo, fmaf(z, c_hi, -s_hi)) - s_lo;
}

// Weights of this thread's NV2 vectors of chunk `chunk` (elements past V get 0).
// In bonus mode the block first finds the chunk maximum and uses the shift
// s = max * c_hi (returned in *s_chunk; -inf when the chunk has no finite
// element).  Every thread of the block must call this.
template <class DT>
__device__ void chunk_weights(const SampleCtx &S, int chunk, float (&w)[kNV2][DT::kVec],
                              float *sh4, float *s_chunk) {
    constexpr int VEC = DT::kVec;
    const int64_t v0 = int64_t(chunk) * (kBlock * kNV2);
    u32x4 dt[kNV2], dq[kNV2];
#pragma unroll
    for (int n = 0; n < kNV2; ++n) {
        const int64_t gv = v0 + n * kBlock + threadIdx.x;
        const bool ok = gv * VEC < S.V;
        dt[n] = ok ? load16(S.row_t + gv * 16)
                   : u32x4{DT::kNegInfWord, DT::kNegInfWord, DT::kNegInfWord, DT::kNegInfWord};
        if (S.mode != kBonus)
            dq[n] = ok ? load16(S.row_q + gv * 16)
                       : u32x4{DT::kNegInfWord, DT::kNegInfWord, DT::kNegInfWord, DT::kNegInfWord};
    }
    float ft[kNV2][VEC], fq[kNV2][VEC];
#pragma unroll
    for (int n = 0; n < kNV2; ++n) {
        DT::unpack(dt[n], ft[n]);
        if (S.mode != kBonus) DT::unpack(dq[n], fq[n]);
        const int64_t lim = int64_t(S.V) - (v0 + n * kBlock + threadIdx.x) * VEC;
        if (lim < VEC) {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if (e >= lim) {
                    ft[n][e] = -INFINITY;
                    fq[n][e] = -INFINITY;
                }
        }
    }
    if (S.mode == kBonus) {
        float m = -INFINITY;
#pragma unroll
        for (int n = 0; n < kNV2; ++n)
#pragma unroll
            for (int e = 0; e < VEC; ++e) m = fmaxf(m, ft[n][e]);
        m = block_max(m, sh4);
        const float s = (m == -INFINITY) ? -INFINITY : m * S.c_hi;
        const float s_use = (m == -INFINITY) ? 0.0f : s;
        *s_chunk = s;
#pragma unroll
        for (int n = 0; n < kNV2; ++n)
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                w[n][e] = __builtin_amdgcn_exp2f(fmaf(ft[n][e], S.c_lo, fmaf(ft[n][e], S.c_hi, -s_use)));
        return;
    }
    *s_chunk = 0.0f;
#pragma unroll
    for (int n = 0; n < kNV2; ++n)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float pt = __builtin_amdgcn_exp2f(log2_prob(ft[n][e], S.c_hi, S.c_lo, S.st_hi, S.st_lo));
            const float pq = __builtin_amdgcn_exp2f(log2_prob(fq[n][e], S.c_hi, S.c_lo, S.sq_hi, S.sq_lo));
            w[n][e] = (S.mode == kResidual) ? fmaxf(pt - pq, 0.0f) : fmaf(S.w_t, pt, S.w_q * pq);
        }
}

template <int VEC>
__device__ __forceinline__ double vec_sum(const float *w) {
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) s += static_cast<double>(w[e]);
    return s;
}

// Mass of a chunk: the paged block scan's total (the same arithmetic the
// locate step repeats, so both agree bitwise).
template <class DT>
__device__ double chunk_mass(const float (&w)[kNV2][DT::kVec], double *shd) {
    double carry = 0.0;
#pragma unroll
    for (int n = 0; n < kNV2; ++n) carry = block_scan_d(vec_sum<DT::kVec>(w[n]), carry, shd).total;
    return carry;
}

struct Resolve {
    int K;          // drafted positions of the request
    int n;          // accepted drafts
    int flags;
};

// Shared state of launch 2.
struct ResolveShared {
    float s[2 * SV_MAX_POSITIONS];
    double S[2 * SV_MAX_POSITIONS];
    float zx[2 * SV_MAX_POSITIONS];
    double a[SV_MAX_POSITIONS];
    int x[SV_MAX_POSITIONS];
    int row_bad[2 * SV_MAX_POSITIONS];
    int n;
    int flags;
};

// Resolve request b: row statistics, acceptance probabilities, first rejection.
template <class DT>
__device__ Resolve resolve_request(const ChainArgs &a, int b, ResolveShared &sh) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    int flags = 0;
    const int K = geo_positions(a.g, b, &flags);
    const int V = a.g.V;
    for (int j = wv; j < 2 * K; j += kWaves) {
        const int i = j >> 1, tensor = j & 1;
        const Part *p = a.part1 + ((int64_t(b) * a.g.Pcap + i) * 2 + tensor) * a.C1;
        float smax = -INFINITY;
        for (int c = lane; c < a.C1; c += kWave) smax = fmaxf(smax, p[c].s);
        smax = wave_max(smax);
        double S = 0.0;
        for (int c = lane; c < a.C1; c += kWave) {
            const Part q = p[c];
            if (q.s != -INFINITY) S += q.S * exp2(static_cast<double>(q.s) - static_cast<double>(smax));
        }
        S = wave_sum_d(S);
        if (lane == 0) {
            sh.s[j] = smax;
            sh.S[j] = S;
            const int x = geo_token(a.g, b, i);
            const bool tok_ok = x >= 0 && x < V;
            const char *row = row_ptr(a.g, tensor, b, geo_row(a.g, b, i));
            sh.zx[j] = tok_ok ? DT::load1(row, x) : NAN;
            if (tensor == 0) sh.x[i] = x;
            sh.row_bad[j] = !(S > 0.0) || !isfinite(S) || !isfinite(smax);
        }
    }
    __syncthreads();
    if (wv == 0) {
        bool rej = false;
        int fl = 0;
        if (lane < K) {
            const int i = lane;
            const float zt = sh.zx[2 * i], zq = sh.zx[2 * i + 1];
            double acc_p;
            if (!(sh.x[i] >= 0 && sh.x[i] < V)) {
                fl |= SV_DATA_BAD_TOKEN;
                acc_p = 0.0;
            } else if (sh.row_bad[2 * i] || sh.row_bad[2 * i + 1]) {
                fl |= SV_DATA_BAD_ROW;
                acc_p = 0.0;
            } else if (zq == -INFINITY) {
                fl |= SV_DATA_ZERO_Q;
                acc_p = (a.lam < 1.0f && zt != -INFINITY) ? 1.0 : 0.0;
            } else if (a.lam >= 1.0f) {
                acc_p = 1.0;
            } else {
                // log2 p(x) = z(x) c - s - log2 S for either model
                const double lt = static_cast<double>(zt) * a.c_d - static_cast<double>(sh.s[2 * i]) - log2(sh.S[2 * i]);
                const double lq = static_cast<double>(zq) * a.c_d - static_cast<double>(sh.s[2 * i + 1]) - log2(sh.S[2 * i + 1]);
                if (lt >= lq) {
                    acc_p = 1.0;
                } else {
                    const double lam = static_cast<double>(a.lam);
                    acc_p = fmin(1.0, (1.0 - lam) * exp2(lt - lq) + lam);
                }
            }
            sh.a[i] = acc_p;
            const double u = static_cast<double>(a.u_accept[int64_t(b) * a.g.P + i]);
            rej = !(u < acc_p);
        }
        const unsigned long long mask = __ballot(rej);
        // OR the per-lane flags
        int fl_all = fl;
        for (int off = 1; off < kWave; off <<= 1) fl_all |= __shfl_xor(fl_all, off, kWave);
        if (lane == 0) {
            sh.n = mask ? (__ffsll(static_cast<long long>(mask)) - 1) : K;
            sh.flags = flags | fl_all;
        }
    }
    __syncthreads();
    Resolve r;
    r.K = K;
    r.n = sh.n;
    r.flags = sh.flags;
    return r;
}

// Sampling context of request b after the resolve.
template <class DT>
__device__ SampleCtx make_ctx(const ChainArgs &a, int b, const Resolve &r, const ResolveShared &sh) {
    SampleCtx S;
    S.V = a.g.V;
    S.c_hi = a.c_hi;
    S.c_lo = a.c_lo;
    S.w_t = 1.0f - a.lam;
    S.w_q = a.lam;
    S.st_hi = S.st_lo = S.sq_hi = S.sq_lo = 0.0f;
    if (r.n < r.K) {
        const int row = geo_row(a.g, b, r.n);
        S.mode = kResidual;
        S.row_t = row_ptr(a.g, 0, b, row);
        S.row_q = row_ptr(a.g, 1, b, row);
        // p(v) = 2^(z c - sigma), sigma = s + log2 S, split into hi + lo floats
        const double st = static_cast<double>(sh.s[2 * r.n]) + log2(sh.S[2 * r.n]);
        const double sq = static_cast<double>(sh.s[2 * r.n + 1]) + log2(sh.S[2 * r.n + 1]);
        S.st_hi = static_cast<float>(st);
        S.st_lo = static_cast<float>(st - static_cast<double>(S.st_hi));
        S.sq_hi = static_cast<float>(sq);
        S.sq_lo = static_cast<float>(sq - static_cast<double>(S.sq_hi));
    } else {
        S.mode = kBonus;
        S.row_t = row_ptr(a.g, 0, b, geo_row(a.g, b, r.K));
        S.row_q = nullptr;
    }
    return S;
}

struct LocateShared {
    float f4[kWaves];
    double d4[kWaves];
    int found;
    int lastpos;
    double excl;
    double scale;
};

// Total sampling mass W of request b from its chunk records, and (when
// t >= 0) the chunk c* whose prefix interval holds t.
__device__ double chunk_scan(const ChainArgs &a, int b, double t, LocateShared &L) {
    const Part *rec = a.part2 + int64_t(b) * a.C2;
    float smax = -INFINITY;
    for (int c = threadIdx.x; c < a.C2; c += kBlock) smax = fmaxf(smax, rec[c].s);
    smax = block_max(smax, L.f4);
    double carry = 0.0;
    for (int base = 0; base < a.C2; base += kBlock) {
        const int c = base + threadIdx.x;
        double m = 0.0, scale = 0.0;
        if (c < a.C2) {
            const Part p = rec[c];
            if (p.s != -INFINITY) {
                scale = exp2(static_cast<double>(p.s) - static_cast<double>(smax));
                m = p.S * scale;
            }
        }
        const Scan sc = block_scan_d(m, carry, L.d4);
        if (t >= 0.0 && c < a.C2 && sc.excl <= t && t < sc.incl) {
            L.found = c;
            L.excl = sc.excl;
            L.scale = scale;
        }
        carry = sc.total;
    }
    __syncthreads();
    return carry;
}

// Token of the sampling row: the first index whose running mass exceeds
// u * W.  Returns -1 when the row has no positive finite mass.
template <class DT>
__device__ int locate(const ChainArgs &a, const SampleCtx &S, int b, double u, LocateShared &L) {
    constexpr int VEC = DT::kVec;
    if (threadIdx.x == 0) {
        L.found = -1;
        L.lastpos = -1;
    }
    __syncthreads();
    const double W = chunk_scan(a, b, -1.0, L);
    if (!(W > 0.0) || !isfinite(W)) return -1;
    const double t = u * W;
    chunk_scan(a, b, t, L);
    const int cs = L.found;
    if (cs < 0) return -1;
    const double tc = (t - L.excl) / L.scale;
    float w[kNV2][VEC];
    float s_unused;
    chunk_weights<DT>(S, cs, w, L.f4, &s_unused);
    if (threadIdx.x == 0) L.found = INT_MAX;
    __syncthreads();
    const int64_t v0 = int64_t(cs) * (kBlock * kNV2);
    double carry = 0.0;
    int mylast = -1;
#pragma unroll
    for (int n = 0; n < kNV2; ++n) {
        const Scan sc = block_scan_d(vec_sum<VEC>(w[n]), carry, L.d4);
        const int64_t e0 = (v0 + n * kBlock + threadIdx.x) * VEC;
        if (sc.excl <= tc && tc < sc.incl) {
            double cum = sc.excl;
            int pick = -1, last = -1;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                if (w[n][e] > 0.0f) {
                    last = e;
                    cum += static_cast<double>(w[n][e]);
                    if (pick < 0 && cum > tc) pick = e;
                }
            }
            if (pick < 0) pick = last;
            if (pick >= 0) atomicMin(&L.found, static_cast<int>(e0 + pick));
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            if (w[n][e] > 0.0f) mylast = static_cast<int>(e0 + e);
        carry = sc.total;
    }
    if (mylast >= 0) atomicMax(&L.lastpos, mylast);
    __syncthreads();
    const int tok = (L.found != INT_MAX) ? L.found : L.lastpos;
    __syncthreads();
    return tok;
}

template <class DT>
__global__ __launch_bounds__(kBlock) void k_accept_resample(ChainArgs a) {
    __shared__ ResolveShared sh;
    __shared__ LocateShared L;
    __shared__ int sh_last;
    const int b = blockIdx.x;
    const int c = blockIdx.y;
    const Resolve r = resolve_request<DT>(a, b, sh);
    SampleCtx S = make_ctx<DT>(a, b, r, sh);

    float w[kNV2][DT::kVec];
    float s_chunk;
    chunk_weights<DT>(S, c, w, L.f4, &s_chunk);
    const double M = chunk_mass<DT>(w, L.d4);
    if (threadIdx.x == 0) {
        Part p;
        p.s = s_chunk;
        p.pad = 0.0f;
        p.S = M;
        a.part2[int64_t(b) * a.C2 + c] = p;
        __threadfence();
        const int prev = atomicAdd(&a.counters[b], 1);
        sh_last = (prev == a.C2 - 1);
    }
    __syncthreads();
    if (!sh_last) return;
    __threadfence();

    int flags = r.flags;
    const double u = static_cast<double>(a.u_sample[b]);
    int tok = locate<DT>(a, S, b, u, L);
    if (tok < 0 && S.mode == kResidual) {
        // Zero residual mass after a rejection (possible only through
        // rounding): draw from p~ at that row instead.
        const bool rows_ok = !sh.row_bad[2 * r.n] && !sh.row_bad[2 * r.n + 1];
        if (rows_ok) {
            flags |= SV_DATA_FALLBACK;
            S.mode = kMixture;
            for (int cc = 0; cc < a.C2; ++cc) {
                chunk_weights<DT>(S, cc, w, L.f4, &s_chunk);
                const double Mc = chunk_mass<DT>(w, L.d4);
                if (threadIdx.x == 0) {
                    Part p;
                    p.s = 0.0f;
                    p.pad = 0.0f;
                    p.S = Mc;
                    a.part2[int64_t(b) * a.C2 + cc] = p;
                }
            }
            __threadfence();
            __syncthreads();
            tok = locate<DT>(a, S, b, u, L);
        }
    }
    if (tok < 0) flags |= SV_DATA_BAD_ROW;

    const int P = a.g.P;
    const int t = threadIdx.x;
    if (t <= P) {
        const int v = (t < r.n) ? sh.x[t] : (t == r.n ? tok : -1);
        a.out_tokens[int64_t(b) * (P + 1) + t] = v;
    }
    if (a.accept_prob != nullptr && t < P)
        a.accept_prob[int64_t(b) * P + t] = (t < r.K) ? static_cast<float>(sh.a[t]) : 0.0f;
    if (t == 0) {
        a.accepted[b] = r.n;
        if (flags) atomicOr(a.status, flags);
    }
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
};

int choose_nv(int B, int P, int V, int vec) {
    const int64_t rows = 2LL * B * P;
    int nv = 8;
    while (nv > kMinNV && rows * c1_for(V, nv, vec) < 8192) nv >>= 1;
    return nv;
}

int pcap(const ChainReq &q) { return q.path_mode ? std::min(q.P, q.N) : q.P; }

sv_status validate(const ChainReq &q) {
    const int eb = elem_bytes(q.dtype);
    if (eb == 0) return SV_EDTYPE;
    if (q.B < 0 || q.P < 0 || q.P > SV_MAX_POSITIONS || q.V < 1 || q.N < 0 ||
        q.N > SV_MAX_TREE_NODES || q.B > (1 << 30))
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
    a.B = q.B;
    a.u_accept = q.u_accept;
    a.u_sample = q.u_sample;
    a.lam = q.lam;
    temperature_split(q.T, &a.c_hi, &a.c_lo, &a.c_d);
    a.accepted = q.accepted;
    a.out_tokens = q.out_tokens;
    a.accept_prob = q.accept_prob;
    a.counters = reinterpret_cast<int32_t *>(ws + L.counters);
    a.status = q.status ? q.status : reinterpret_cast<int32_t *>(ws + L.status);
    a.part1 = reinterpret_cast<Part *>(ws + L.part1);
    a.part2 = reinterpret_cast<Part *>(ws + L.part2);
    a.C1 = c1_for(q.V, nv, vec);
    a.C2 = c2_for(q.V, vec);
    return a;
}

template <class DT>
sv_status run_typed(const ChainReq &q, int which) {
    const int nv = choose_nv(q.B, pcap(q), q.V, DT::kVec);
    const ChainArgs a = make_args(q, DT::kVec, nv);
    if (which & 1) {
        const int64_t jobs = int64_t(q.B) * a.g.Pcap * 2 * a.C1;
        const int64_t blocks = jobs > 0 ? cdiv(jobs, kWaves) : 1;
        if (blocks > 0x7fffffffLL) return SV_EINVAL;
        const dim3 grid(static_cast<unsigned>(blocks));
        if (nv == 8)
            hipLaunchKernelGGL((k_row_stats<DT, 8>), grid, dim3(kBlock), 0, q.stream, a, jobs);
        else if (nv == 4)
            hipLaunchKernelGGL((k_row_stats<DT, 4>), grid, dim3(kBlock), 0, q.stream, a, jobs);
        else
            hipLaunchKernelGGL((k_row_stats<DT, 2>), grid, dim3(kBlock), 0, q.stream, a, jobs);
        if (hipGetLastError() != hipSuccess) return SV_EHIP;
    }
    if (which & 2) {
        const dim3 grid(static_cast<unsigned>(q.B), static_cast<unsigned>(a.C2));
        hipLaunchKernelGGL((k_accept_resample<DT>), grid, dim3(kBlock), 0, q.stream, a);
        if (hipGetLastError() != hipSuccess) return SV_EHIP;
    }
    return SV_OK;
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
    return q;
}

}  // namespace

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

}  // extern "C"
