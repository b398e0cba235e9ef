// Host/device definitions shared by the chain, path and tree kernels:
// argument records, workspace layout, temperature constants and argument
// validation.  Validation runs on the host before any HIP call.
#pragma once

#include <atomic>
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

// Partial reduction of one wave-chunk of a row: the sum S of 2^(z*c - s) over
// the chunk's elements, relative to the shift s, an integer (held as a float:
// the ceiling of the chunk's largest logit times c_hi), so that partials
// rescale exactly by powers of two.  s = -inf marks a chunk without any finite
// element.
struct alignas(16) Part {
    float s;
    float z;        // the drafted token's logit, in the partial of the chunk holding it
    double S;
};

// Per-chunk argmax partial (greedy trees).
struct alignas(16) ArgPart {
    float val;
    int idx;
    int nan;
    int pad;
};

// Per-request record of launch 2 of a chain call: the accepted count and the
// sampling row with its statistics.
struct alignas(16) ReqRecord {
    int n;          // accepted drafts
    int mode;       // the sampling row's law: residual, logit-space residual or bonus
    int row;        // request row of the sampling position
    int rows_ok;    // the residual rows have valid statistics
    float st, sq;   // integer shifts of the target and draft rows: p(v) = 2^(z c - s) / S
    float it, iq;   // 1 / S of the target and draft rows
    float k0;       // residual: q(v) / p(v) = 2^((z_q(v) - z_t(v)) d + k0)
};

// Request geometry of the chain and path calls.
struct Geo {
    const char *tgt;              // target logits base
    const char *drf;              // draft logits base
    int64_t ld_t, ld_q;           // row strides (elements)
    int64_t req_t, req_q;         // rows per request
    int elem;                     // bytes per element
    int V;                        // vocabulary
    int P;                        // positions capacity (chain K, path Dmax): output strides
    int Pcap;                     // positions a request can hold (chain K, path min(Dmax, N)):
                                  // stride of the row-partial workspace
    int N;                        // tree nodes (path mode)
    const int32_t *tokens;        // chain: draft_tokens [B, K]; path: node_token [B, N]
    const int32_t *draft_len;     // chain only, may be NULL
    const int32_t *path;          // path mode; NULL for a chain
};

struct ChainArgs {
    Geo g;
    int B;
    const float *u_accept;        // [B, P]
    const float *u_sample;        // [B]
    float lam;
    float c_hi, c_lo;             // log2(e)/T = c_hi + c_lo, c_hi > 0, c_lo > 0
    double c_d;                   // log2(e)/T in double
    int32_t *accepted;            // [B]
    int32_t *out_tokens;          // [B, P+1]
    float *accept_prob;           // [B, P] or NULL
    int32_t *status;              // [1]
    Part *part1;                  // [B, Pcap, 2, C1] workspace: row partials
    int *count;                   // [B] workspace: mass blocks of the request done (cleared by launch 1)
    double *chunks;               // [B, C2, rec_stride] workspace: sampling-chunk records
    int C1;                       // wave-chunks per row in the row-stats pass
    int ch1;                      // elements per row-stats chunk
    int NV2;                      // vectors per lane per sampling chunk (2, 4 or 8)
    int C2;                       // chunks per row in the sampling pass
    int rec_stride;               // doubles per chunk record: shift, pad, 16 * NV2 piece sums
    int packed;                   // 1: position slots of the statistics launches follow the
                                  // packed order of drafted positions (ragged chain, B <= 256)
    int space;                    // 0: probability-space mixture; 1: logit space (0 < lambda < 1)
    double alpha_c, beta_c;       // logit space: (1 - lambda) c and lambda c, c = log2(e)/T, fp64
    float al_hi, al_lo, be_hi, be_lo;   // the same split as hi + lo, each part > 0 (fp32 exponents)
    // [B, Pcap, C1, 2] workspace: each chunk's sum of min(p~, q) as a tagged
    // word pair (low, high half of the double), and the call's tag
    unsigned long long *alpha_rec;
    uint32_t tag;
    // words the row-statistics launch also sets for a caller that runs after
    // it (the multi-branch walk's barrier slots and ticket; the
    // acceptance-rate output, every position of which starts at 0); NULL: none
    unsigned long long *fill;
    int64_t fill_n;
    unsigned long long fill_val;
    unsigned *zero_word;
    float *zero_f;
    int64_t zero_f_n;
    // tree rows (one position per node): the parent array [B, leaf_N] whose
    // childless nodes' draft rows are skipped; NULL: every row
    const int32_t *leaf_par;
    int leaf_N;
    float *alpha;                 // [B, P] out: expected acceptance of each drafted position
};

struct TreeArgs {
    const char *tgt;
    int64_t ld_t;
    int elem;
    int B, N, V, Dmax, C1;
    const int32_t *parent;
    const int32_t *node_token;
    int32_t *accepted;
    int32_t *out_tokens;
    int32_t *accepted_nodes;
    int32_t *status;
    ArgPart *part;                // [B, N+1, C1]
    // one-launch call: the same slots as tagged record pairs, row and tree
    // words, and the call's tag
    unsigned long long *rec;      // [B, N+1, C1, 2]
    unsigned long long *rowword;  // [B, N+1]: each row's argmax
    unsigned long long *treeflag; // [B]: each tree's flags
    uint32_t tag;
};

// ---------------------------------------------------------------------------
// tiling
// ---------------------------------------------------------------------------

constexpr int kBlock2 = 1024;                 // threads of a resolve / mass block
constexpr int kWaves2 = kBlock2 / 64;
constexpr int kMaxC2 = 128;                   // sampling chunks per row at NV2 = 2 (bounds V)
constexpr int kMinVec = 4;                    // fp32: 4 elements per 16-byte vector
constexpr int kMinNV = 2;                     // smallest row-stats vectors per lane
constexpr int kStageMax = 2048;               // row partials staged in LDS per request
constexpr int kMaxPieces = 4096;             // piece masses of one sampling row (staged in LDS by the draw)
constexpr int kGreedyStageMax = 2048;         // argmax partials staged in LDS per tree

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Row-stats wave-chunk: 64 lanes x NV vectors x VEC elements.
inline int c1_for(int V, int NV, int vec) { return static_cast<int>(cdiv(V, 64LL * NV * vec)); }
// Vectors per lane of a streaming wave-job: 8 (8 KB of bf16 per wave) unless
// that leaves fewer than 512 jobs (two per compute unit), then 4 or 2.  Below
// that, smaller jobs only multiply the partials the resolve combines: on one
// request of 8 positions at V = 128256 a threshold of 2048 jobs gave 2 KB jobs
// and a 15.7 us call, 512 gives 8 KB jobs and 15.2 us.
inline int choose_stream_nv(int64_t rows, int V, int vec) {
    int nv = 8;
    while (nv > kMinNV && rows * c1_for(V, nv, vec) < 512) nv >>= 1;
    return nv;
}

inline int c2_for(int V, int vec, int nv2) {
    return static_cast<int>(cdiv(V, int64_t(kBlock2) * nv2 * vec));
}

// Vectors per lane of a sampling chunk: the smallest of 1, 2, 4, 8 that keeps
// the chunk grid of launch 2 within one block per compute unit (256), as far
// as larger chunks still help.  Small batches take one vector: their sampling
// rows then spread over twice the compute units, which halves each wave's
// residual weights (one request of 8 positions at V = 128256: 16 blocks).
inline int choose_nv2(int B, int V, int vec) {
    int nv2 = (c2_for(V, vec, 1) <= kMaxC2) ? 1 : 2;
    while (nv2 < 8 && int64_t(B) * c2_for(V, vec, nv2) > 256 &&
           c2_for(V, vec, 2 * nv2) < c2_for(V, vec, nv2))
        nv2 *= 2;
    return nv2;
}

inline int chunk_rec_doubles(int nv2) { return 2 + 16 * nv2; }

// Bytes of the chunk records for either element type.
inline int64_t chunk_bytes(int B, int V) {
    int64_t m = 0;
    for (int vec = 4; vec <= 8; vec += 4) {
        const int nv2 = choose_nv2(B, V, vec);
        const int64_t b = int64_t(B) * c2_for(V, vec, nv2) * chunk_rec_doubles(nv2) * 8;
        m = b > m ? b : m;
    }
    return m;
}

struct ChainLayout {
    int64_t status, count, chunks, part1, total;
};

inline ChainLayout chain_layout(int B, int P, int V) {
    ChainLayout L;
    const int64_t c1max = c1_for(V, kMinNV, kMinVec);
    L.status = 0;
    L.count = 256;
    L.chunks = L.count + align256(int64_t(B) * int64_t(sizeof(int)));
    L.part1 = L.chunks + align256(chunk_bytes(B, V));
    L.total = L.part1 + align256(int64_t(B) * P * 2 * c1max * int64_t(sizeof(Part)));
    return L;
}

// The acceptance-rate call: the chain layout, then the per-chunk partial sums
// of min(p~, q), one tagged word pair (16 bytes) per (request, position, chunk).
inline int64_t alpha_layout_parts(int B, int P, int V) { return chain_layout(B, P, V).total; }
inline int64_t alpha_layout_total(int B, int P, int V) {
    return alpha_layout_parts(B, P, V) + align256(int64_t(B) * P * c1_for(V, kMinNV, kMinVec) * 16);
}

struct TreeLayout {
    int64_t status, part, rowword, treeflag, total;
};

inline TreeLayout tree_layout(int B, int N, int V) {
    TreeLayout L;
    const int64_t c1max = c1_for(V, kMinNV, kMinVec);
    L.status = 0;
    L.part = 256;
    L.rowword = L.part + align256(int64_t(B) * (N + 1) * c1max * int64_t(sizeof(ArgPart)));
    L.treeflag = L.rowword + align256(int64_t(B) * (N + 1) * 8);
    L.total = L.treeflag + align256(int64_t(B) * 8);
    return L;
}

// Temperature constants: c = log2(e) / T split as c_hi + c_lo with both parts
// strictly positive, so that (-inf) * c_hi + (-inf) * c_lo stays -inf.
inline bool temperature_split(float T, float *c_hi, float *c_lo, double *c_d) {
    const double c = 1.4426950408889634074 / static_cast<double>(T);
    if (!(c > 0.0 && c < 1.0e38)) return false;
    float hi = static_cast<float>(c);
    if (static_cast<double>(hi) >= c) hi = nextafterf(hi, 0.0f);
    float lo = static_cast<float>(c - static_cast<double>(hi));
    if (!(hi > 0.0f) || !(lo >= 1.1754944e-38f) || !isfinite(hi) || !isfinite(lo)) return false;
    *c_hi = hi;
    *c_lo = lo;
    *c_d = static_cast<double>(hi) + static_cast<double>(lo);
    return true;
}

// x > 0 as hi + lo in fp32 with hi < x the largest float below it and lo > 0,
// so that (-inf) * hi + (-inf) * lo stays -inf.  x = 0 gives 0 + 0.
inline void split_positive(double x, float *hi, float *lo) {
    if (!(x > 0.0)) {
        *hi = 0.0f;
        *lo = 0.0f;
        return;
    }
    float h = static_cast<float>(x);
    if (static_cast<double>(h) >= x) h = nextafterf(h, 0.0f);
    *hi = h;
    *lo = static_cast<float>(x - static_cast<double>(h));
}

// Launches `kernel` on `stream`; when either event is given, the launch
// records them at the kernel's own begin and end (the dispatch timestamps),
// so their elapsed time is the kernel duration without queueing gaps.
template <typename Kernel, typename... Args>
inline void launch_timed(Kernel kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop, Args... args) {
    if (ev_start != nullptr || ev_stop != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ev_start, ev_stop, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
}

// A tag for the records one call hands between its waves: the top bit set
// (so no untagged value, index or zero word matches it) and a process-wide
// count below it (so no other call's records carry it).
inline uint32_t next_call_tag() {
    static std::atomic<uint32_t> calls{0};
    return 0x80000000u | (calls.fetch_add(1u, std::memory_order_relaxed) & 0x7FFFFFFFu);
}

// Row statistics of rows 0 .. R-1 of every request of [B, R, V] target and
// draft logits (the chain's first launch, one position per row): partials
// [B, R, 2, C1] into part1, C1 = rows_stats_chunks(...).  Space 1: slot 0 of
// a row holds the logit-space mixture's statistics, as in the chain.  count
// (B ints) is cleared, status cleared, fill[0 .. fill_n) set to fill_val and
// *zero_word to 0 (when given).  leaf_par: the [B, R - 1] parent array of
// trees whose row r belongs to node r; the draft row of a node without
// children is then skipped (its partials read as an empty row).  Host code;
// enqueued on stream.
int rows_stats_chunks(int B, int R, int V, sv_dtype dtype, int space);
sv_status rows_stats(const void *tgt, int64_t ld_t, const void *drf, int64_t ld_q, sv_dtype dtype, int B, int R,
                     int V, float lam, float T, int space, Part *part1, int *count, int32_t *status,
                     hipStream_t stream, unsigned long long *fill = nullptr, int64_t fill_n = 0,
                     unsigned long long fill_val = 0, unsigned *zero_word = nullptr,
                     const int32_t *leaf_par = nullptr);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int elem_bytes(sv_dtype d) { return d == SV_BF16 ? 2 : (d == SV_F32 ? 4 : 0); }

inline sv_status check_logits(const void *p, int64_t ld, int V, int eb) {
    if (!p) return SV_ENULL;
    if (ld < V || !aligned16(p) || ((ld * eb) & 15) != 0) return SV_EALIGN;
    return SV_OK;
}

inline sv_status check_scalars(float lam, float T) {
    if (!(lam >= 0.0f && lam <= 1.0f)) return SV_EINVAL;
    if (!(T > 0.0f) || !isfinite(T)) return SV_EINVAL;
    float a, b;
    double c;
    if (!temperature_split(T, &a, &b, &c)) return SV_EINVAL;
    return SV_OK;
}

}  // namespace sv
