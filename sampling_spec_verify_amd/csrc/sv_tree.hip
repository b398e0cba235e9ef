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
// Two launches:
//  1. k_row_argmax: one wavefront per (request, row, chunk) streams 64 lanes x
//     NV x 16 bytes of a target row and keeps the largest value with its
//     lowest index (no exponentials: argmax is temperature-free).
//  2. k_greedy_walk: one 1024-thread block per request combines the chunk partials into
//     the argmax of each row, then walks the parent array in node order:
//     ok[i] = ok[parent[i]] and token[i] == argmax[parent[i]]; the deepest ok
//     node (lowest id on ties) and its root path are emitted, followed by the
//     argmax of its row as the bonus token.
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
template <class DT, int NV>
__device__ __forceinline__ void row_chunk_argmax(const TreeArgs &a, unsigned job) {
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
    const int widx = wave_min_i(idx);
    const bool wnan = __ballot(nan) != 0ull;
    if (lane == 0) {
        ArgPart p;
        p.val = wm;
        p.idx = widx;
        p.nan = wnan ? 1 : 0;
        p.pad = 0;
        a.part[row_id * a.C1 + c] = p;
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

    // argmax of every row: largest value, lowest index among equals
#pragma unroll 1
    for (int r = wv; r <= N; r += kWaves2) {
        const ArgPart *p = staged ? stage + r * a.C1 : a.part + pbase + int64_t(r) * a.C1;
        float v = -INFINITY;
#pragma unroll 1
        for (int c = lane; c < a.C1; c += kWave) v = fmaxf(v, p[c].val);
        v = wave_max(v);
        int idx = INT_MAX;
        int nan = 0;
#pragma unroll 1
        for (int c = lane; c < a.C1; c += kWave) {
            const ArgPart q = p[c];
            if (q.val == v) idx = min(idx, q.idx);
            nan |= q.nan;
        }
        idx = wave_min_i(idx);
        const bool anynan = __ballot(nan != 0) != 0ull;
        if (lane == 0) {
            am[r] = (idx == INT_MAX || anynan) ? -1 : idx;
            if (idx == INT_MAX || anynan) atomicOr(&sh_flags, SV_DATA_BAD_ROW);
        }
    }
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
// 2: walk).  Argument errors return before any HIP call.
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
