// Greedy draft-tree verification on gfx950.
//
// Method (cited by page title and section):
//   EAGLE explainer "投机解码（EAGLE）：让小模型猜、大模型验，无损加速 LLM 生成",
//     "核心思路" step 3: a draft token is kept when it is the target's most
//     likely token; "3. 验证阶段树形attention": the whole tree is scored in one
//     target pass and each node sees only its ancestors.
//   "大模型推理的Speculative Decoding原理详解", "Tree Speculation": several
//     candidate branches per position, verified together.
//
// Row argmax: one wavefront per (request, row, chunk) streams 64 lanes x NV x
// 16 bytes of a target row and keeps the largest value with its lowest index
// (no exponentials: argmax is temperature-free).  Walk: the chunk results give
// the argmax of each row, then ok[i] = ok[parent[i]] and token[i] ==
// argmax[parent[i]]; the deepest ok node (lowest id on ties) and its root path
// are emitted, followed by the argmax of its row as the bonus token.
//
// Trees of at most 64 nodes (the root included) take one launch,
// k_greedy_fold: the wave of each tree's last job walks that tree in
// registers, one lane per node, once the tree's chunk records are in.  Larger
// trees take two: k_row_argmax, then k_greedy_walk, one 1024-thread block per
// tree.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "sv_common.hpp"
#include "sv_device.hpp"

namespace sv {

// One job: the largest value (lowest index among equals) of wave-chunk c of
// one target row, by one wavefront.  Maximum first, position second: every
// lane reduces each of its 16-byte vectors to a maximum, the wave takes the
// maximum of those, and only then does each lane look for its first element
// equal to it (a lane's vectors, and the elements inside one, are in index
// order).  The lane maxima use the NaN-propagating maximum (v_maximum3_f32),
// so a NaN anywhere in a lane shows up in that lane's maximum and marks the
// whole row bad (the chunk's maximum and index then do not matter).  Signed zeros
// compare equal in the position search, as in the first-maximum rule.
// Elements past V read as -inf and sit above every valid index, so they never
// win a tie.
struct ChunkMax {
    float val;      // the chunk's largest value
    int idx;        // its lowest index (INT_MAX: none)
    bool nan;       // a NaN in the chunk
};

template <class DT, int NV>
__device__ __forceinline__ ChunkMax chunk_argmax(const TreeArgs &a, unsigned job) {
    const int c = static_cast<int>(job % static_cast<unsigned>(a.C1));
    const int64_t row_id = job / static_cast<unsigned>(a.C1);   // b * (N+1) + r
    const char *row = a.tgt + row_id * a.ld_t * a.elem;

    constexpr int VEC = DT::kVec;
    const int lane = threadIdx.x & (kWave - 1);
    const int V = a.V;
    const int v0 = c * (kWave * NV);
    u32x4 d[NV];
    load_chunk<DT, NV>(row, v0, lane, V, d);
    float vm[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        float f[VEC];
        DT::unpack(d[n], f);
        float m = f[0];
#pragma unroll
        for (int e = 1; e < VEC; ++e) m = __builtin_elementwise_maximum(m, f[e]);
        vm[n] = m;
    }
    float lm = vm[0];
#pragma unroll
    for (int n = 1; n < NV; ++n) lm = __builtin_elementwise_maximum(lm, vm[n]);
    const bool nan = (lm != lm);
    const float wm = wave_max(lm);
    // this lane's first vector, then first element, equal to the wave maximum
    int nsel = -1;
#pragma unroll
    for (int n = NV - 1; n >= 0; --n)
        if (vm[n] == wm) nsel = n;
    int idx = INT_MAX;
    if (nsel >= 0) {
        u32x4 dv = d[0];
#pragma unroll
        for (int n = 1; n < NV; ++n)
            if (nsel == n) dv = d[n];
        float f[VEC];
        DT::unpack(dv, f);
        int esel = VEC - 1;
#pragma unroll
        for (int e = VEC - 1; e >= 0; --e)
            if (f[e] == wm) esel = e;
        idx = (v0 + nsel * kWave + lane) * VEC + esel;
    }
    ChunkMax r;
    r.val = wm;
    r.idx = wave_min_i(idx);
    r.nan = __ballot(nan) != 0ull;
    return r;
}

template <class DT, int NV>
__device__ __forceinline__ void row_chunk_argmax(const TreeArgs &a, unsigned job) {
    const ChunkMax r = chunk_argmax<DT, NV>(a, job);
    if ((threadIdx.x & (kWave - 1)) == 0) {
        ArgPart p;
        p.val = r.val;
        p.idx = r.idx;
        p.nan = r.nan ? 1 : 0;
        p.pad = 0;
        a.part[job] = p;     // job = (b * (N+1) + r) * C1 + c
    }
}

// One wavefront per job (wave-uniform index, 32-bit scalar decode).
template <class DT, int NV>
__global__ __launch_bounds__(kBlock) void k_row_argmax(TreeArgs a, int n_jobs) {
    const int job = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kWaves +
                                                   static_cast<int>(threadIdx.x) / kWave);
    if (job < n_jobs) row_chunk_argmax<DT, NV>(a, static_cast<unsigned>(job));
    // cleared last (a store ahead of the reads would keep them off the scalar path)
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.status = 0;
}

// One 1024-thread block per request.  All of the request's chunk partials,
// parents and node tokens arrive in one parallel load round (partials staged
// in LDS when they fit) and sixteen waves combine the rows.  The walk is
// parallel over nodes: node i matches when its parent is valid and its token
// is the argmax of the parent's row; ok[i] (every node from i up to the root
// matches) and depth[i] come from pointer jumping, O(log depth) rounds over
// (ancestor, value) pairs where the value is the depth while every node
// passed so far matched and a large negative number once one did not.  The
// deepest ok node (lowest id on ties) is a block maximum of
// depth * 2048 + (2047 - i); only its own root path is walked serially.
constexpr int kNodes = SV_MAX_TREE_NODES + 1;
constexpr int kRejected = -(1 << 20);       // below any sum of <= kNodes depths

// Every row's argmax from its C1 chunk partials (rows 0..N at p + base, C1
// each), one wave per row; a row with no value or a NaN gets -1 and flags
// the call.
__device__ __forceinline__ void argmax_rows(const ArgPart *parts, int64_t base, int C1, int N, int *am,
                                            int *flags) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
#pragma unroll 1
    for (int r = wv; r <= N; r += kWaves2) {
        const ArgPart *p = parts + base + int64_t(r) * C1;
        float v = -INFINITY;
#pragma unroll 1
        for (int c = lane; c < C1; c += kWave) v = fmaxf(v, p[c].val);
        v = wave_max(v);
        int idx = INT_MAX;
        int nan = 0;
#pragma unroll 1
        for (int c = lane; c < C1; c += kWave) {
            const ArgPart q = p[c];
            if (q.val == v) idx = min(idx, q.idx);
            nan |= q.nan;
        }
        idx = wave_min_i(idx);
        const bool anynan = __ballot(nan != 0) != 0ull;
        if (lane == 0) {
            am[r] = (idx == INT_MAX || anynan) ? -1 : idx;
            if (idx == INT_MAX || anynan) atomicOr(flags, SV_DATA_BAD_ROW);
        }
    }
}

__global__ __launch_bounds__(kBlock2) void k_greedy_walk(TreeArgs a, int staged) {
    __shared__ int am[kNodes];
    __shared__ int par[kNodes];
    __shared__ int tok[kNodes];
    __shared__ int path[kNodes];        // ancestor buffer of the jumps, then the output path
    __shared__ int anc[kNodes];
    __shared__ int dep[2][kNodes];
    __shared__ int wkey[kWaves2];
    __shared__ int sh_flags;
    extern __shared__ ArgPart stage[];
    const int b = blockIdx.x;
    const int N = a.N;
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wv = t / kWave;
    const int64_t pbase = int64_t(b) * (N + 1) * a.C1;
    if (t == 0) sh_flags = 0;
    if (staged)
        for (int idx = t; idx < (N + 1) * a.C1; idx += kBlock2) stage[idx] = a.part[pbase + idx];
    for (int i = t; i < N; i += kBlock2) {
        par[i + 1] = a.parent[int64_t(b) * N + i];
        tok[i + 1] = a.node_token[int64_t(b) * N + i];
    }
    __syncthreads();

    // argmax of every row: largest value, lowest index among equals (two
    // loops, so that the staged one reads shared memory only)
    if (staged) argmax_rows(stage, 0, a.C1, N, am, &sh_flags);
    else argmax_rows(a.part, pbase, a.C1, N, am, &sh_flags);
    __syncthreads();

    // one edge per node: parent and whether the node's token matches
    int flags = 0;
    for (int i = t; i <= N; i += kBlock2) {
        int up = 0, val = 0;                 // the root: depth 0, ok
        if (i > 0) {
            const int p = par[i];
            val = kRejected;
            if (p < 0 || p >= i) {
                flags |= SV_DATA_BAD_TREE;   // never followed: treated as a rejected root child
            } else {
                up = p;
                if (tok[i] < 0 || tok[i] >= a.V) flags |= SV_DATA_BAD_TOKEN;
                else if (am[p] >= 0 && tok[i] == am[p]) val = 1;
            }
        }
        anc[i] = up;
        dep[0][i] = val;
    }
    // pointer jumping: (anc, dep) -> (anc[anc], dep + dep[anc]) until every
    // chain reaches the root; anc and path alternate as the ancestor buffer
    int cur = 0;
    int *A0 = anc, *A1 = path;
    bool more = true;
#pragma unroll 1
    while (more) {
        __syncthreads();
        bool any = false;
        for (int i = t; i <= N; i += kBlock2) {
            const int u = A0[i];
            int d = dep[cur][i], nu = 0;
            if (u != 0) {
                d += dep[cur][u];
                nu = A0[u];
            }
            A1[i] = nu;
            dep[cur ^ 1][i] = d;
            any |= (nu != 0);
        }
        more = __syncthreads_or(any) != 0;
        cur ^= 1;
        int *tmp = A0;
        A0 = A1;
        A1 = tmp;
    }
    // deepest ok node, lowest id on ties (node ids are < 2048)
    int key = -1;
    for (int i = t; i <= N; i += kBlock2) {
        const int d = dep[cur][i];
        if (d >= 0) key = max(key, d * 2048 + (2047 - i));
    }
    key = -wave_min_i(-key);
    const unsigned long long fl_mask = __ballot(flags != 0);
    if (lane == 0) wkey[wv] = key;
    if (fl_mask) {
        const int fl_all = wave_or8(flags);
        if (lane == 0) atomicOr(&sh_flags, fl_all);
    }
    __syncthreads();
    int best_key = wkey[0];
#pragma unroll
    for (int w = 1; w < kWaves2; ++w) best_key = max(best_key, wkey[w]);
    const int best = 2047 - best_key % 2048;
    const int best_d = best_key / 2048;
    const int Dmax = a.Dmax;
    const int keep = min(best_d, Dmax);
    if (t == 0) {
        // nodes root -> best (path[d] = node at depth d), cut to Dmax nodes
        int v = best;
        for (int d = best_d; d >= 1; --d) {
            if (d <= keep) path[d] = v;
            v = par[v];
        }
        if (best_d > Dmax) sh_flags |= SV_DATA_DEPTH;
    }
    __syncthreads();
    const int last = keep > 0 ? path[keep] : 0;
    const int bonus = am[last];
    for (int i = t; i <= Dmax; i += kBlock2) {
        int v = -1;
        if (i < keep) v = tok[path[i + 1]];
        else if (i == keep) v = bonus;
        a.out_tokens[int64_t(b) * (Dmax + 1) + i] = v;
        if (i < Dmax) a.accepted_nodes[int64_t(b) * Dmax + i] = (i < keep) ? path[i + 1] : -1;
    }
    if (t == 0) {
        a.accepted[b] = keep;
        if (sh_flags) atomicOr(a.status, sh_flags);
    }
}

// ---- one launch for trees of at most 64 nodes --------------------------------
//
// Records cross waves as agent-scope relaxed atomics (write-through: the
// reading wave may run on another XCD), each 64-bit word carrying the call's
// tag in its high half.  The tag has its top bit set and changes every call,
// so neither an untagged partial nor a record another call left in the
// workspace passes for this call's.  Every record has one reader, which clears
// it after reading: a replay of the same launch (same tag) finds it empty.
//
//  * A chunk's record: (tag, value bits), (tag, index | nan << 31).
//  * The wave of a row's last chunk combines the row: lane c polls chunk c's
//    record until both words carry the tag (its own chunk it has in
//    registers), then the wave takes the row's argmax and publishes it as the
//    row's word (tag, argmax), -1 for a row with a NaN or no index.
//  * The wave of a tree's last chunk (row N) polls the other rows' words
//    while it combines its own row, and walks the tree in registers, one lane
//    per node.
//  * The status word is stored once, by the wave of the batch's last tree
//    (the grid's last job): every other walking wave stores its tree's flags
//    as a word (tag, flags), and the last one polls those words while it
//    combines its own row, so that its whole tail is one round trip.
//
// A wave waits only for waves of earlier jobs, dispatched before it.  Every
// poll is bounded (about a second); a wave that gives up sets SV_DATA_SYNC
// (outputs invalid) and goes on, so every wave ends.

constexpr int kFoldNodes = kWave;           // N + 1 at most: one lane per node
constexpr int kFoldTrees = 1024;            // trees per one-launch call at most (flag words polled by one wave)

// The argmax of the row whose last chunk this wave holds (own): its other
// chunks' records, one lane per chunk, combined as the two-launch walk does
// (the largest value, then the lowest index among the chunks holding it);
// -1 for a row with a NaN or no index.  `pre`: loads to issue first, so that
// their round trip overlaps this one (the tree walker's row words).
__device__ __forceinline__ int fold_row(const TreeArgs &a, int64_t row_id, const ChunkMax &own, int &flags) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t tag = a.tag;
    unsigned long long *rec = a.rec + 2 * row_id * a.C1;
    float best = -INFINITY;
    int bidx = INT_MAX;
    bool nan = false;
    for (int c0 = 0; c0 < a.C1; c0 += kWave) {
        const int c = c0 + lane;
        float v = -INFINITY;
        int i = INT_MAX;
        bool n = false;
        if (c == a.C1 - 1) {
            v = own.val;
            i = own.idx;
            n = own.nan;
        } else if (c < a.C1 - 1) {
            unsigned long long w0 = ld_agent(rec + 2 * c), w1 = ld_agent(rec + 2 * c + 1);
            poll_pair(rec + 2 * c, tag, w0, w1, flags);
            v = __uint_as_float(static_cast<uint32_t>(w0));
            const uint32_t lo = static_cast<uint32_t>(w1);
            i = static_cast<int>(lo & 0x7FFFFFFFu);
            n = (lo >> 31) != 0u;
        }
        // the chunk maxima ignore a NaN value: such a chunk carries the flag
        const float m = wave_max(v == v ? v : -INFINITY);
        const int mi = wave_min_i((v == m) ? i : INT_MAX);
        nan |= __ballot(n) != 0ull;
        if (m > best) {
            best = m;
            bidx = mi;
        } else if (m == best) {
            bidx = min(bidx, mi);
        }
    }
    if (bidx == INT_MAX || nan) {
        flags |= SV_DATA_BAD_ROW;
        return -1;
    }
    return bidx;
}

// The walk of tree b by one wavefront, lane i holding node i (N + 1 <= 64).
__device__ void fold_walk(const TreeArgs &a, int b, const ChunkMax &own) {
    const int lane = threadIdx.x & (kWave - 1);
    const int N = a.N;
    const uint32_t tag = a.tag;
    int flags = 0;
    // the other rows' words, in flight while this wave combines row N
    unsigned long long *rw = a.rowword + int64_t(b) * (N + 1);
    unsigned long long w = (lane < N) ? ld_agent(rw + lane) : 0ull;
    // the batch's last tree: the other trees' flag words, also in flight
    const bool last_tree = (b == a.B - 1);
    unsigned long long fw = (last_tree && lane < b) ? ld_agent(a.treeflag + lane) : 0ull;
    const int am_n = fold_row(a, int64_t(b) * (N + 1) + N, own, flags);
    int am = am_n;
    if (lane < N) {
        int polls = 0;
        while (!tagged(w, tag)) {
            if (++polls > kPollSpin) {
                flags |= SV_DATA_SYNC;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            w = ld_agent(rw + lane);
        }
        st_agent(rw + lane, 0ull);
        am = static_cast<int>(static_cast<uint32_t>(w));
        if (am == -2) {                     // its row combine gave up waiting
            flags |= SV_DATA_SYNC;
            am = -1;
        } else if (am < 0) {
            flags |= SV_DATA_BAD_ROW;
        }
    }
    int par = -1, tok = -1;
    if (lane >= 1 && lane <= N) {
        par = a.parent[int64_t(b) * N + lane - 1];
        tok = a.node_token[int64_t(b) * N + lane - 1];
    }
    const bool par_ok = lane >= 1 && lane <= N && par >= 0 && par < lane;
    const int am_par = __shfl(am, par_ok ? par : 0);
    // (ancestor, value): the depth while every node passed so far matched, a
    // large negative number once one did not (the root: depth 0, ok)
    int up = 0, dep = (lane <= N) ? 0 : kRejected;
    if (lane >= 1 && lane <= N) {
        dep = kRejected;
        if (!par_ok) {
            flags |= SV_DATA_BAD_TREE;       // never followed: a rejected root child
        } else {
            up = par;
            if (tok < 0 || tok >= a.V) flags |= SV_DATA_BAD_TOKEN;
            else if (am_par >= 0 && tok == am_par) dep = 1;
        }
    }
    while (__ballot(up != 0) != 0ull) {
        const int du = __shfl(dep, up);
        const int uu = __shfl(up, up);
        if (up != 0) {
            dep += du;
            up = uu;
        }
    }
    const int key = (lane <= N && dep >= 0) ? dep * 2048 + (2047 - lane) : -1;
    const int best_key = wave_max_i(key);         // the root's key is at least 2047
    const int best = 2047 - best_key % 2048;
    const int best_d = best_key / 2048;
    const int keep = min(best_d, a.Dmax);
    if (best_d > a.Dmax) flags |= SV_DATA_DEPTH;
    // the root path of best: lane d holds the node at depth d
    int mypath = 0;
    {
        int v = best;
        for (int d = best_d; d >= 1; --d) {
            if (lane == d) mypath = v;
            v = __builtin_amdgcn_readlane(par, v);
        }
    }
    const int p_next = __shfl(mypath, (lane + 1) & (kWave - 1));   // path[lane + 1]
    const int tok_next = __shfl(tok, p_next & (kWave - 1));
    const int last = keep > 0 ? __builtin_amdgcn_readlane(mypath, keep) : 0;
    const int bonus = __builtin_amdgcn_readlane(am, last);
    for (int i = lane; i <= a.Dmax; i += kWave) {
        int v = -1;
        if (i < keep) v = tok_next;
        else if (i == keep) v = bonus;
        a.out_tokens[int64_t(b) * (a.Dmax + 1) + i] = v;
        if (i < a.Dmax) a.accepted_nodes[int64_t(b) * a.Dmax + i] = (i < keep) ? p_next : -1;
    }
    if (lane == 0) a.accepted[b] = keep;
    if (!last_tree) {
        const int fl = wave_or8(flags);
        if (lane == 0) st_agent(a.treeflag + b, (static_cast<unsigned long long>(tag) << 32) | static_cast<uint32_t>(fl));
        return;
    }
    // the status: this tree's flags and every other tree's flag word
    int other = 0;
    for (int t0 = 0; t0 < b; t0 += kWave) {
        const int t = t0 + lane;
        if (t < b) {
            if (t0 > 0) fw = ld_agent(a.treeflag + t);
            int polls = 0;
            while (!tagged(fw, tag)) {
                if (++polls > kPollSpin) {
                    flags |= SV_DATA_SYNC;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                fw = ld_agent(a.treeflag + t);
            }
            st_agent(a.treeflag + t, 0ull);
            other |= static_cast<int>(static_cast<uint32_t>(fw));
        }
    }
    const int fl = wave_or8(flags | (other & 0xFF));
    if (lane == 0) *a.status = fl;
}

// Row argmax; the wave of a row's last chunk combines the row, and the wave
// of a tree's last chunk walks the tree.
template <class DT, int NV>
__global__ __launch_bounds__(kBlock) void k_greedy_fold(TreeArgs a, int n_jobs) {
    const int job = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kWaves +
                                                   static_cast<int>(threadIdx.x) / kWave);
    if (job >= n_jobs) return;
    const ChunkMax r = chunk_argmax<DT, NV>(a, static_cast<unsigned>(job));
    const int64_t row_id = job / a.C1;
    if ((job + 1) % a.C1 != 0) {
        if ((threadIdx.x & (kWave - 1)) == 0) {
            const unsigned long long tagw = static_cast<unsigned long long>(a.tag) << 32;
            st_agent(a.rec + 2 * int64_t(job), tagw | __float_as_uint(r.val));
            st_agent(a.rec + 2 * int64_t(job) + 1,
                     tagw | (static_cast<uint32_t>(r.idx) & 0x7FFFFFFFu) | (r.nan ? 0x80000000u : 0u));
        }
        return;
    }
    const int b = static_cast<int>(row_id / (a.N + 1));
    if (row_id % (a.N + 1) != a.N) {
        int flags = 0;
        const int am = fold_row(a, row_id, r, flags);
        if ((threadIdx.x & (kWave - 1)) == 0) {
            // a SYNC failure marks the row (its argmax is then not trusted) as -1 with the flag
            const unsigned long long tagw = static_cast<unsigned long long>(a.tag) << 32;
            st_agent(a.rowword + row_id, tagw | static_cast<uint32_t>((flags & SV_DATA_SYNC) ? -2 : am));
        }
        return;
    }
    fold_walk(a, b, r);
}

// Tree-attention mask (EAGLE explainer, "3. 验证阶段树形attention": to verify
// a tree in one target pass each candidate may attend only to its ancestor
// path).  Grid (request, slice): every block stages its request's parent
// array in LDS (an out-of-range parent reads as the root), then each thread
// produces whole 32-bit mask words: word w of row i holds, at bit j, whether
// node 32 w + j is i or an ancestor of i.  Parents are smaller than their
// children, so a node's ancestors decrease along the walk: the walk first
// climbs past the word's range, then sets at most 32 bits and stops below it.
// The word-0 walk reaches the root and also gives the node's depth.
constexpr int kMaskBlock = 256;

__global__ __launch_bounds__(kMaskBlock) void k_tree_mask(const int32_t *parent, int N,
                                                          uint32_t *mask, int W, int32_t *depth,
                                                          int32_t *status) {
    __shared__ int par[kNodes];
    __shared__ int sh_bad;
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    if (t == 0) sh_bad = 0;
    __syncthreads();
    int bad = 0;
    for (int i = t; i <= N; i += kMaskBlock) {
        int p = -1;
        if (i > 0) {
            p = parent[int64_t(b) * N + i - 1];
            if (p < 0 || p >= i) {
                bad = 1;
                p = 0;
            }
        }
        par[i] = p;
    }
    if (bad) atomicOr(&sh_bad, 1);
    __syncthreads();
    const int64_t items = int64_t(N + 1) * W;
    uint32_t *out = mask + int64_t(b) * items;
    for (int64_t it = int64_t(blockIdx.y) * kMaskBlock + t; it < items;
         it += int64_t(gridDim.y) * kMaskBlock) {
        const int i = static_cast<int>(it / W);
        const int w = static_cast<int>(it - int64_t(i) * W);
        const int lo = 32 * w;
        int a = i, steps = 0;
        uint32_t bits = 0;
        while (a >= lo + 32) {           // the root's parent is -1, so this ends
            a = par[a];
            ++steps;
        }
        while (a >= lo) {
            bits |= 1u << (a - lo);
            a = par[a];
            ++steps;
        }
        out[it] = bits;
        if (w == 0 && depth != nullptr) depth[int64_t(b) * (N + 1) + i] = steps - 1;
    }
    if (t == 0 && blockIdx.y == 0 && sh_bad && status != nullptr) atomicOr(status, SV_DATA_BAD_TREE);
}

}  // namespace sv

namespace {

using namespace sv;

template <class DT>
sv_status run_tree(const TreeArgs &a0, hipStream_t stream, int which, hipEvent_t ev_start,
                   hipEvent_t ev_stop) {
    TreeArgs a = a0;
    const int64_t rows = int64_t(a.B) * (a.N + 1);
    const int nv = choose_stream_nv(rows, a.V, DT::kVec);
    a.C1 = c1_for(a.V, nv, DT::kVec);
    if (rows * a.C1 >= (int64_t(1) << 31)) return SV_EINVAL;
    if (which == 3 && a.N + 1 <= kFoldNodes && a.B <= kFoldTrees) {
        // one launch: the walk in the argmax launch's tail
        a.tag = next_call_tag();
        const int jobs = static_cast<int>(rows * a.C1);
        const dim3 grid(static_cast<unsigned>(std::max<int64_t>(1, cdiv(jobs, kWaves))));
        if (nv == 8)
            launch_timed(k_greedy_fold<DT, 8>, grid, dim3(kBlock), 0, stream, ev_start, ev_stop, a, jobs);
        else if (nv == 4)
            launch_timed(k_greedy_fold<DT, 4>, grid, dim3(kBlock), 0, stream, ev_start, ev_stop, a, jobs);
        else
            launch_timed(k_greedy_fold<DT, 2>, grid, dim3(kBlock), 0, stream, ev_start, ev_stop, a, jobs);
        return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
    }
    if (which & 1) {
        const int jobs = static_cast<int>(rows * a.C1);
        const dim3 grid(static_cast<unsigned>(std::max<int64_t>(1, cdiv(jobs, kWaves))));
        if (nv == 8)
            launch_timed(k_row_argmax<DT, 8>, grid, dim3(kBlock), 0, stream, ev_start, ev_stop, a, jobs);
        else if (nv == 4)
            launch_timed(k_row_argmax<DT, 4>, grid, dim3(kBlock), 0, stream, ev_start, ev_stop, a, jobs);
        else
            launch_timed(k_row_argmax<DT, 2>, grid, dim3(kBlock), 0, stream, ev_start, ev_stop, a, jobs);
        if (hipGetLastError() != hipSuccess) return SV_EHIP;
    }
    if (which & 2) {
        const int64_t stage_n = int64_t(a.N + 1) * a.C1;
        const int staged = stage_n <= kGreedyStageMax ? 1 : 0;
        const size_t lds = staged ? static_cast<size_t>(stage_n) * sizeof(ArgPart) : 0;
        hipLaunchKernelGGL(k_greedy_walk, dim3(static_cast<unsigned>(a.B)), dim3(kBlock2), lds,
                           stream, a, staged);
        if (hipGetLastError() != hipSuccess) return SV_EHIP;
    }
    return SV_OK;
}

// Validates the greedy call and runs the launches in `which` (1: row argmax,
// 2: walk, 3: the whole call, in one launch for trees of at most 64 nodes).
// Argument errors return before any HIP call.
sv_status greedy_call(const void *target_logits, int64_t ld_t, sv_dtype dtype, int B, int N,
                      int V, const int32_t *parent, const int32_t *node_token, int32_t *accepted,
                      int32_t *out_tokens, int32_t *accepted_nodes, int Dmax, int32_t *status,
                      void *workspace, size_t workspace_bytes, hipStream_t stream, int which,
                      hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr) {
    const int eb = elem_bytes(dtype);
    if (eb == 0) return SV_EDTYPE;
    if (B < 0 || N < 0 || N > SV_MAX_TREE_NODES || V < 1 || Dmax < 0 || B > (1 << 30))
        return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!accepted || !out_tokens || (Dmax > 0 && !accepted_nodes)) return SV_ENULL;
    if (N > 0 && (!parent || !node_token)) return SV_ENULL;
    const sv_status st = check_logits(target_logits, ld_t, V, eb);
    if (st != SV_OK) return st;
    const TreeLayout L = tree_layout(B, N, V);
    if (!workspace || !aligned16(workspace) || workspace_bytes < static_cast<size_t>(L.total))
        return SV_EWORKSPACE;
    char *ws = static_cast<char *>(workspace);
    TreeArgs a;
    a.tgt = static_cast<const char *>(target_logits);
    a.ld_t = ld_t;
    a.elem = eb;
    a.B = B;
    a.N = N;
    a.V = V;
    a.Dmax = Dmax;
    a.C1 = 0;
    a.parent = parent;
    a.node_token = node_token;
    a.accepted = accepted;
    a.out_tokens = out_tokens;
    a.accepted_nodes = accepted_nodes;
    a.status = status ? status : reinterpret_cast<int32_t *>(ws + L.status);
    a.part = reinterpret_cast<ArgPart *>(ws + L.part);
    a.rec = reinterpret_cast<unsigned long long *>(ws + L.part);
    a.rowword = reinterpret_cast<unsigned long long *>(ws + L.rowword);
    a.treeflag = reinterpret_cast<unsigned long long *>(ws + L.treeflag);
    a.tag = 0;
    return dtype == SV_BF16 ? run_tree<Bf16>(a, stream, which, ev_start, ev_stop)
                            : run_tree<F32>(a, stream, which, ev_start, ev_stop);
}

}  // namespace

extern "C" {

size_t sv_tree_workspace_bytes(int B, int N, int V) {
    if (B < 0 || N < 0 || N > SV_MAX_TREE_NODES || V < 1) return 0;
    const int64_t greedy = tree_layout(B, N, V).total;
    const int64_t path = chain_layout(B, N < SV_MAX_POSITIONS ? N : SV_MAX_POSITIONS, V).total;
    return static_cast<size_t>(greedy > path ? greedy : path);
}

sv_status sv_tree_verify_greedy(const void *target_logits, int64_t ld_t, sv_dtype dtype, int B,
                                int N, int V, const int32_t *parent, const int32_t *node_token,
                                int32_t *accepted, int32_t *out_tokens, int32_t *accepted_nodes,
                                int Dmax, int32_t *status, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    return greedy_call(target_logits, ld_t, dtype, B, N, V, parent, node_token, accepted, out_tokens,
                       accepted_nodes, Dmax, status, workspace, workspace_bytes, stream, 3);
}

sv_status sv_tree_row_argmax(const void *target_logits, int64_t ld_t, sv_dtype dtype, int B, int N,
                             int V, const int32_t *parent, const int32_t *node_token,
                             int32_t *accepted, int32_t *out_tokens, int32_t *accepted_nodes,
                             int Dmax, int32_t *status, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    return greedy_call(target_logits, ld_t, dtype, B, N, V, parent, node_token, accepted, out_tokens,
                       accepted_nodes, Dmax, status, workspace, workspace_bytes, stream, 1);
}

sv_status sv_tree_verify_greedy_timed(const void *target_logits, int64_t ld_t, sv_dtype dtype, int B,
                                      int N, int V, const int32_t *parent, const int32_t *node_token,
                                      int32_t *accepted, int32_t *out_tokens, int32_t *accepted_nodes,
                                      int Dmax, int32_t *status, void *workspace, size_t workspace_bytes,
                                      hipStream_t stream, hipEvent_t kernel_start, hipEvent_t kernel_stop) {
    return greedy_call(target_logits, ld_t, dtype, B, N, V, parent, node_token, accepted, out_tokens,
                       accepted_nodes, Dmax, status, workspace, workspace_bytes, stream, 3, kernel_start,
                       kernel_stop);
}

sv_status sv_tree_row_argmax_timed(const void *target_logits, int64_t ld_t, sv_dtype dtype, int B,
                                   int N, int V, const int32_t *parent, const int32_t *node_token,
                                   int32_t *accepted, int32_t *out_tokens,
                                   int32_t *accepted_nodes, int Dmax, int32_t *status,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream,
                                   hipEvent_t kernel_start, hipEvent_t kernel_stop) {
    return greedy_call(target_logits, ld_t, dtype, B, N, V, parent, node_token, accepted, out_tokens,
                       accepted_nodes, Dmax, status, workspace, workspace_bytes, stream, 1,
                       kernel_start, kernel_stop);
}

sv_status sv_tree_attention_mask_timed(const int32_t *parent, int B, int N, uint32_t *mask,
                                       int mask_words, int32_t *depth, int32_t *status,
                                       hipStream_t stream, hipEvent_t kernel_start,
                                       hipEvent_t kernel_stop) {
    if (B < 0 || N < 0 || N > SV_MAX_TREE_NODES || B > (1 << 30) || mask_words < (N + 32) / 32 ||
        mask_words > (1 << 20))
        return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!mask || (N > 0 && !parent)) return SV_ENULL;
    const int64_t items = int64_t(N + 1) * mask_words;
    const int slices = static_cast<int>(std::min<int64_t>(64, cdiv(items, kMaskBlock)));
    launch_timed(k_tree_mask, dim3(static_cast<unsigned>(B), static_cast<unsigned>(slices)),
                 dim3(kMaskBlock), 0, stream, kernel_start, kernel_stop, parent, N, mask,
                 mask_words, depth, status);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

sv_status sv_tree_attention_mask(const int32_t *parent, int B, int N, uint32_t *mask, int mask_words,
                                 int32_t *depth, int32_t *status, hipStream_t stream) {
    return sv_tree_attention_mask_timed(parent, B, N, mask, mask_words, depth, status, stream,
                                        nullptr, nullptr);
}

sv_status sv_tree_greedy_walk(const void *target_logits, int64_t ld_t, sv_dtype dtype, int B, int N,
                              int V, const int32_t *parent, const int32_t *node_token,
                              int32_t *accepted, int32_t *out_tokens, int32_t *accepted_nodes,
                              int Dmax, int32_t *status, void *workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    return greedy_call(target_logits, ld_t, dtype, B, N, V, parent, node_token, accepted, out_tokens,
                       accepted_nodes, Dmax, status, workspace, workspace_bytes, stream, 2);
}

}  // extern "C"
