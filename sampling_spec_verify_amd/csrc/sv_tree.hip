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
// one target row, by one wavefront.
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
#pragma unroll
    for (int n = 0; n < NV; ++n) d[n] = load_row_vec<DT>(row, v0 + n * kWave + lane, V);
    // elements past V read as -inf and sit above every valid index, so they
    // never win: a lane keeps the first index of its largest value
    float best = -INFINITY;
    int best_i = INT_MAX;
    bool nan = false;
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        float f[VEC];
        DT::unpack(d[n], f);
        const int i0 = (v0 + n * kWave + lane) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            nan |= (f[e] != f[e]);
            if (f[e] > best || best_i == INT_MAX) {
                best = (f[e] != f[e]) ? best : f[e];
                best_i = (f[e] != f[e]) ? best_i : i0 + e;
            }
        }
    }
    const float wbest = wave_max(best);
    const int widx = wave_min_i(best == wbest ? best_i : INT_MAX);
    const bool wnan = __ballot(nan) != 0ull;
    if (lane == 0) {
        ArgPart p;
        p.val = wbest;
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
// in LDS when they fit), sixteen waves combine the rows, then one thread walks
// the parent array.
__global__ __launch_bounds__(kBlock2) void k_greedy_walk(TreeArgs a, int staged) {
    __shared__ int am[SV_MAX_TREE_NODES + 1];
    __shared__ int par[SV_MAX_TREE_NODES + 1];
    __shared__ int tok[SV_MAX_TREE_NODES + 1];
    __shared__ int path[SV_MAX_TREE_NODES + 1];
    __shared__ int sh_flags, sh_depth, sh_best;
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

    if (t == 0) {
        // ok / depth packed into path[] (reused): depth+1 when ok, 0 otherwise
        int flags = 0;
        path[0] = 1;                         // root: ok, depth 0
        int best = 0, best_d = 0;
        for (int i = 1; i <= N; ++i) {
            const int p = par[i];
            int st = 0;
            if (p < 0 || p >= i) {
                flags |= SV_DATA_BAD_TREE;
            } else if (tok[i] < 0 || tok[i] >= a.V) {
                flags |= SV_DATA_BAD_TOKEN;
            } else if (path[p] > 0 && am[p] >= 0 && tok[i] == am[p]) {
                st = path[p] + 1;
            }
            path[i] = st;
            if (st - 1 > best_d) {
                best_d = st - 1;
                best = i;
            }
        }
        // nodes root -> best (path[d] = node at depth d), cut to Dmax nodes
        int v = best;
        for (int d = best_d; d >= 1; --d) {
            path[d] = v;
            v = par[v];
        }
        if (best_d > a.Dmax) flags |= SV_DATA_DEPTH;
        sh_best = best;
        sh_depth = best_d;
        sh_flags |= flags;
    }
    __syncthreads();
    const int Dmax = a.Dmax;
    const int keep = min(sh_depth, Dmax);
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

}  // namespace sv

namespace {

using namespace sv;

template <class DT>
sv_status run_tree(const TreeArgs &a0, hipStream_t stream) {
    TreeArgs a = a0;
    const int64_t rows = int64_t(a.B) * (a.N + 1);
    const int nv = choose_stream_nv(rows, a.V, DT::kVec);
    a.C1 = c1_for(a.V, nv, DT::kVec);
    if (rows * a.C1 >= (int64_t(1) << 31)) return SV_EINVAL;
    const int jobs = static_cast<int>(rows * a.C1);
    const dim3 grid(static_cast<unsigned>(std::max<int64_t>(1, cdiv(jobs, kWaves))));
    if (nv == 8)
        hipLaunchKernelGGL((k_row_argmax<DT, 8>), grid, dim3(kBlock), 0, stream, a, jobs);
    else if (nv == 4)
        hipLaunchKernelGGL((k_row_argmax<DT, 4>), grid, dim3(kBlock), 0, stream, a, jobs);
    else
        hipLaunchKernelGGL((k_row_argmax<DT, 2>), grid, dim3(kBlock), 0, stream, a, jobs);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
    const int64_t stage_n = int64_t(a.N + 1) * a.C1;
    const int staged = stage_n <= kGreedyStageMax ? 1 : 0;
    const size_t lds = staged ? static_cast<size_t>(stage_n) * sizeof(ArgPart) : 0;
    hipLaunchKernelGGL(k_greedy_walk, dim3(static_cast<unsigned>(a.B)), dim3(kBlock2), lds, stream, a,
                       staged);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
    return SV_OK;
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
    return dtype == SV_BF16 ? run_tree<Bf16>(a, stream) : run_tree<F32>(a, stream);
}

}  // extern "C"
