// Device helpers shared by the libspecverify kernels (gfx950, wave64).
//
//  * 16-byte row loads and bf16/fp32 unpacking,
//  * wavefront reductions built from DPP lane moves (quad_perm, row mirrors)
//    plus one ds_swizzle across the 16-lane rows and a readlane pair across
//    the two 32-lane halves,
//  * a block-wide (256-thread) inclusive/exclusive scan of doubles whose
//    inclusive values form a monotone sequence: every item's exclusive prefix
//    is bitwise the previous item's inclusive prefix, so "first item whose
//    inclusive prefix exceeds t" is always unique.
//
// Every reduction runs in a fixed order, so results are bitwise reproducible;
// no floating-point atomics are used anywhere in the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;

// ---------------------------------------------------------------------------
// element types
// ---------------------------------------------------------------------------

struct Bf16 {
    static constexpr int kVec = 8;     // elements per 16-byte vector
    static constexpr int kBytes = 2;
    static constexpr unsigned kNegInfWord = 0xff80ff80u;
    __device__ static __forceinline__ void unpack(const u32x4 &d, float *f) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = __uint_as_float(d[j] << 16);
            f[2 * j + 1] = __uint_as_float(d[j] & 0xffff0000u);
        }
    }
    __device__ static __forceinline__ float load1(const char *row, int64_t i) {
        const unsigned short h = reinterpret_cast<const unsigned short *>(row)[i];
        return __uint_as_float(static_cast<unsigned>(h) << 16);
    }
};

struct F32 {
    static constexpr int kVec = 4;
    static constexpr int kBytes = 4;
    static constexpr unsigned kNegInfWord = 0xff800000u;
    __device__ static __forceinline__ void unpack(const u32x4 &d, float *f) {
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(d[j]);
    }
    __device__ static __forceinline__ float load1(const char *row, int64_t i) {
        return reinterpret_cast<const float *>(row)[i];
    }
};

// One 16-byte load.  NT marks it non-temporal: the single-use stream over the
// drafted rows.  Reads of rows that were streamed just before (the sampling
// row) or that the same block reads again (the tree walk) use ordinary loads.
template <bool NT = true>
__device__ __forceinline__ u32x4 load16(const char *p) {
    if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return *reinterpret_cast<const u32x4 *>(p);
}

// 16-byte vector gv (in units of DT::kVec elements) of a row of V elements:
// vectors past the row read as -inf; in the one partial vector the elements
// past V are set to -inf on the packed words.  The partial-vector test only
// runs when V is not a multiple of kVec (a wave-uniform condition).
template <class DT, bool NT = true>
__device__ __forceinline__ u32x4 load_row_vec(const char *row, int gv, int V) {
    constexpr int VEC = DT::kVec;
    const int nvec = (V + VEC - 1) / VEC;
    u32x4 d = (gv < nvec) ? load16<NT>(row + int64_t(gv) * 16)
                          : u32x4{DT::kNegInfWord, DT::kNegInfWord, DT::kNegInfWord, DT::kNegInfWord};
    if ((V % VEC) != 0 && gv == nvec - 1) {
        const int valid = V - gv * VEC;             // 1 .. VEC-1 elements stay
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (DT::kVec == 8) {
                if (2 * j >= valid) d[j] = 0xff80ff80u;
                else if (2 * j + 1 >= valid) d[j] = (d[j] & 0x0000ffffu) | 0xff800000u;
            } else if (j >= valid) {
                d[j] = 0xff800000u;
            }
        }
    }
    return d;
}

// The NV vectors v0 + n * 64 + lane (n < NV) of a row, as load_row_vec reads
// them.  When the whole chunk lies inside the row's full vectors (v0 is
// wave-uniform, so the test is too; it holds for every chunk but a row's
// last), the loads go out without per-vector guards or masking.
template <class DT, int NV>
__device__ __forceinline__ void load_chunk(const char *row, int v0, int lane, int V, u32x4 (&d)[NV]) {
    if (v0 + NV * kWave <= V / DT::kVec) {
#pragma unroll
        for (int n = 0; n < NV; ++n) d[n] = load16(row + int64_t(v0 + n * kWave + lane) * 16);
    } else {
#pragma unroll
        for (int n = 0; n < NV; ++n) d[n] = load_row_vec<DT>(row, v0 + n * kWave + lane, V);
    }
}

// load_chunk's vectors as two steps, for a kernel that uses other loads issued
// before the chunk while the chunk is in flight: the loads go out in straight
// code (lanes past the row read its last vector again), so that waiting for
// those earlier loads does not wait for the chunk; mask_chunk then gives the
// elements past the row -inf (a wave-uniform test: only a row's last chunk).
template <class DT, int NV>
__device__ __forceinline__ void load_chunk_clamped(const char *row, int v0, int lane, int V, u32x4 (&d)[NV]) {
    const int last = (V + DT::kVec - 1) / DT::kVec - 1;
#pragma unroll
    for (int n = 0; n < NV; ++n) d[n] = load16(row + int64_t(min(v0 + n * kWave + lane, last)) * 16);
}

template <class DT, int NV>
__device__ __forceinline__ void mask_chunk(int v0, int lane, int V, u32x4 (&d)[NV]) {
    if (v0 + NV * kWave <= V / DT::kVec) return;
    const int last = (V + DT::kVec - 1) / DT::kVec - 1;
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        const int gv = v0 + n * kWave + lane;
        if (gv > last) {
            d[n] = u32x4{DT::kNegInfWord, DT::kNegInfWord, DT::kNegInfWord, DT::kNegInfWord};
        } else if ((V % DT::kVec) != 0 && gv == last) {
            const int valid = V - gv * DT::kVec;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (DT::kVec == 8) {
                    if (2 * j >= valid) d[n][j] = 0xff80ff80u;
                    else if (2 * j + 1 >= valid) d[n][j] = (d[n][j] & 0x0000ffffu) | 0xff800000u;
                } else if (j >= valid) {
                    d[n][j] = 0xff800000u;
                }
            }
        }
    }
}

// 2^d for an integer-valued d <= 0 (a difference of two integer shifts),
// exactly; 0 below the smallest subnormal.
__device__ __forceinline__ float pow2_shift(float d) {
    return d < -149.0f ? 0.0f : ldexpf(1.0f, static_cast<int>(d));
}
__device__ __forceinline__ double pow2_shift_d(double d) {
    return d < -1074.0 ? 0.0 : ldexp(1.0, static_cast<int>(d));
}

// 2^x in fp64: x = k + f with k = floor(x), 2^f = sqrt(2) e^y with
// y = (f - 1/2) ln 2 in [-0.35, 0.35], e^y by its Taylor series through y^13
// (truncation below 2e-16 relative).  0 below -1100, +inf above 1100, NaN
// passes through.
__device__ __forceinline__ double exp2_d(double x) {
    if (x != x) return x;
    if (x < -1100.0) return 0.0;
    if (x > 1100.0) return INFINITY;
    const double k = floor(x);
    const double y = (x - k - 0.5) * 0.69314718055994530942;
    double p = 1.0 / 6227020800.0;                    // 1/13!
    p = fma(p, y, 1.0 / 479001600.0);                 // 1/12!
    p = fma(p, y, 1.0 / 39916800.0);
    p = fma(p, y, 1.0 / 3628800.0);
    p = fma(p, y, 1.0 / 362880.0);
    p = fma(p, y, 1.0 / 40320.0);
    p = fma(p, y, 1.0 / 5040.0);
    p = fma(p, y, 1.0 / 720.0);
    p = fma(p, y, 1.0 / 120.0);
    p = fma(p, y, 1.0 / 24.0);
    p = fma(p, y, 1.0 / 6.0);
    p = fma(p, y, 0.5);
    p = fma(p, y, 1.0);
    p = fma(p, y, 1.0);
    return ldexp(1.41421356237309504880 * p, static_cast<int>(k));
}

// alpha z_t + beta z_q - s in fp32 with alpha = m[0] + m[1], beta = m[2] + m[3]
// (the hi + lo splits): the large products first, each fma rounding once,
// then the two small corrections.  Near the largest mixed logit (the terms
// that carry the mass) the result is within about 1e-7 of the exact value.
__device__ __forceinline__ float mixed_expo(float zt, float zq, const float (&m)[4], float s) {
    return fmaf(zq, m[3], fmaf(zt, m[1], fmaf(zq, m[2], fmaf(zt, m[0], -s))));
}

// max(0, 1 - 2^e) in fp32 with an error of a few ulps relative to the result
// itself, also where 2^e is close to 1 (the residual weight of an element whose
// two probabilities nearly agree).  0 for e >= 0 and for NaN.  For
// -1/2 <= e < 0 it is -expm1(e ln 2) by its Taylor series c1 e + ... + c7 e^7,
// c_k = (ln 2)^k / k! (truncation below 1.6e-8 relative; 2 ulps in all, as
// measured against fp64 over the interval); below -1/2 it is 1 - 2^e, where
// 2^e < 0.71 and the subtraction loses under two bits.
__device__ __forceinline__ float one_minus_exp2(float e) {
    float p = 1.5252733804059841e-05f;              // (ln 2)^7 / 7!
    p = fmaf(p, e, 1.5403530393381608e-04f);
    p = fmaf(p, e, 1.3333558146428443e-03f);
    p = fmaf(p, e, 9.6181291076284772e-03f);
    p = fmaf(p, e, 5.5504108664821580e-02f);
    p = fmaf(p, e, 2.4022650695910071e-01f);
    p = fmaf(p, e, 6.9314718055994531e-01f);        // ln 2
    const float small = -e * p;
    const float large = 1.0f - __builtin_amdgcn_exp2f(e);
    return fmaxf((e < -0.5f) ? large : small, 0.0f);  // e >= 0 gives small <= 0; NaN gives 0
}

// ---------------------------------------------------------------------------
// tagged hand-over words between the waves of one launch
// ---------------------------------------------------------------------------
//
// A 64-bit word carries the call's tag in its high half and 32 bits of payload
// in its low half.  It is written as an agent-scope relaxed atomic store
// (write-through, so visible to every XCD's L2) and read as an agent-scope
// atomic load.  A reader polls until the tag appears and then clears the word,
// so a later call (or a replay of the same captured launch, which keeps its
// tag) never takes it for its own.

constexpr int kPollSpin = 1 << 20;          // polls of one word before the wave gives up

__device__ __forceinline__ unsigned long long ld_agent(const unsigned long long *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(unsigned long long *p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tagged(unsigned long long w, uint32_t tag) {
    return static_cast<uint32_t>(w >> 32) == tag;
}

// Polls the word pair at p until both carry the tag (w0, w1: the words
// already loaded); clears them.  A wave that gives up sets SV_DATA_SYNC.
__device__ __forceinline__ void poll_pair(unsigned long long *p, uint32_t tag, unsigned long long &w0,
                                          unsigned long long &w1, int &flags) {
    int polls = 0;
    while (!tagged(w0, tag) || !tagged(w1, tag)) {
        if (++polls > kPollSpin) {
            flags |= SV_DATA_SYNC;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        w0 = ld_agent(p);
        w1 = ld_agent(p + 1);
    }
    st_agent(p, 0ull);
    st_agent(p + 1, 0ull);
}

// ---------------------------------------------------------------------------
// lane moves
// ---------------------------------------------------------------------------

// DPP controls (GFX9 encoding)
constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
// ds_swizzle bitmask mode: and 0x1f, or 0, xor 0x10 -> lane ^ 16 within 32
constexpr int kSwzXor16 = 0x401F;

// Lane permutations whose every lane has a source lane (quad perms and
// mirrors), so no lane keeps an old value.
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int swz16(int v) { return __builtin_amdgcn_ds_swizzle(v, kSwzXor16); }

__device__ __forceinline__ float f_of(int v) { return __int_as_float(v); }
__device__ __forceinline__ int i_of(float v) { return __float_as_int(v); }

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const int lo = dpp<CTRL>(__double2loint(v));
    const int hi = dpp<CTRL>(__double2hiint(v));
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double swz16_d(double v) {
    const int lo = swz16(__double2loint(v));
    const int hi = swz16(__double2hiint(v));
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double readlane_d(double v, int lane) {
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), lane);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), lane);
    return __hiloint2double(hi, lo);
}

// ---------------------------------------------------------------------------
// wavefront reductions (result is wave-uniform)
// ---------------------------------------------------------------------------

__device__ __forceinline__ int wave_max_i(int v);

// Maximum over the wave of non-NaN floats, through integer keys: the key
// flips the magnitude bits of negative values, so signed integer order is
// float order (-0 and +0 map to -1 and 0 and come back unchanged).  Integer
// maxima fuse with the lane moves, where a float maximum would first
// canonicalise every moved value.
__device__ __forceinline__ float wave_max(float v) {
    const int b = i_of(v);
    const int k = wave_max_i(b ^ ((b >> 31) & 0x7fffffff));
    return f_of(k ^ ((k >> 31) & 0x7fffffff));
}

__device__ __forceinline__ int wave_max_i(int v) {
    v = max(v, dpp<kDppXor1>(v));
    v = max(v, dpp<kDppXor2>(v));
    v = max(v, dpp<kDppHalfMirror>(v));
    v = max(v, dpp<kDppMirror>(v));
    v = max(v, swz16(v));
    return max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 32));
}

__device__ __forceinline__ int wave_min_i(int v) {
    v = min(v, dpp<kDppXor1>(v));
    v = min(v, dpp<kDppXor2>(v));
    v = min(v, dpp<kDppHalfMirror>(v));
    v = min(v, dpp<kDppMirror>(v));
    v = min(v, swz16(v));
    return min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 32));
}

// Lane l of a wave receives v of lane l - n within its 16-lane row (row_shr),
// of lane l - 1 across the wave (wave_shr), or lane 15 / 31 broadcast to the
// following rows (row_bcast), only where the row mask (rows 0..3) and bank
// mask allow; every other lane receives 0.
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ double dpp_shift_d(double v) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROW_MASK, BANK_MASK, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROW_MASK, BANK_MASK, false);
    return __hiloint2double(hi, lo);
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;
constexpr int kDppWaveShr1 = 0x138;    // whole wave, lane l receives lane l - 1

// Inclusive scan of one double per lane, in lane order (log-step: shifts by
// 1, 2, 4, 8 inside each 16-lane row, then lane 15 into rows 1 and 3, then
// lane 31 into rows 2 and 3).
__device__ __forceinline__ double wave_scan_d(double v) {
    v += dpp_shift_d<kDppRowShr1, 0xF, 0xF>(v);
    v += dpp_shift_d<kDppRowShr2, 0xF, 0xF>(v);
    v += dpp_shift_d<kDppRowShr4, 0xF, 0xF>(v);
    v += dpp_shift_d<kDppRowShr8, 0xF, 0xF>(v);
    v += dpp_shift_d<kDppRowBcast15, 0xA, 0xF>(v);
    v += dpp_shift_d<kDppRowBcast31, 0xC, 0xF>(v);
    return v;
}

// Inclusive scan of one int per lane, in lane order, by the same shift steps.
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ int dpp_shift_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, BANK_MASK, false);
}
__device__ __forceinline__ int wave_scan_i(int v) {
    v += dpp_shift_i<kDppRowShr1, 0xF, 0xF>(v);
    v += dpp_shift_i<kDppRowShr2, 0xF, 0xF>(v);
    v += dpp_shift_i<kDppRowShr4, 0xF, 0xF>(v);
    v += dpp_shift_i<kDppRowShr8, 0xF, 0xF>(v);
    v += dpp_shift_i<kDppRowBcast15, 0xA, 0xF>(v);
    v += dpp_shift_i<kDppRowBcast31, 0xC, 0xF>(v);
    return v;
}

// OR of an 8-bit flag word over the wave, one ballot per bit (a shuffle
// butterfly would take six LDS round trips).
__device__ __forceinline__ int wave_or8(int v) {
    int r = 0;
#pragma unroll
    for (int bit = 0; bit < 8; ++bit)
        if (__ballot((v >> bit) & 1)) r |= 1 << bit;
    return r;
}

__device__ __forceinline__ double wave_sum_d(double v) {
    v += dpp_d<kDppXor1>(v);
    v += dpp_d<kDppXor2>(v);
    v += dpp_d<kDppHalfMirror>(v);
    v += dpp_d<kDppMirror>(v);
    v += swz16_d(v);
    return readlane_d(v, 0) + readlane_d(v, 32);
}

// ---------------------------------------------------------------------------
// block (256 threads) helpers; every thread of the block must call them
// ---------------------------------------------------------------------------

__device__ __forceinline__ float block_max(float v, float *sh4) {
    v = wave_max(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) sh4[w] = v;
    __syncthreads();
    const float r = fmaxf(fmaxf(sh4[0], sh4[1]), fmaxf(sh4[2], sh4[3]));
    __syncthreads();
    return r;
}

struct Scan {
    double incl;    // prefix including this thread's item
    double excl;    // prefix before it (bitwise the previous item's incl)
    double total;   // prefix of the whole block (bitwise the last item's incl)
};

// Inclusive scan of one double per thread, in thread order, offset by `carry`.
__device__ __forceinline__ Scan block_scan_d(double v, double carry, double *sh4) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const double x = wave_scan_d(v);
    if (lane == kWave - 1) sh4[w] = x;
    __syncthreads();
    const double b1 = sh4[0];
    const double b2 = b1 + sh4[1];
    const double b3 = b2 + sh4[2];
    const double tot = b3 + sh4[3];
    const double base = (w == 0) ? 0.0 : (w == 1) ? b1 : (w == 2) ? b2 : b3;
    const double prev = dpp_shift_d<kDppWaveShr1, 0xF, 0xF>(x);   // lane l - 1 (0 at lane 0)
    Scan s;
    s.incl = carry + (base + x);
    s.excl = carry + ((lane == 0) ? base : (base + prev));
    s.total = carry + tot;
    __syncthreads();
    return s;
}

}  // namespace sv
