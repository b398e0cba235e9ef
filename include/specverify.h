/*
 * libspecverify: the verify step of speculative decoding on MI355X (gfx950).
 *
 * Sources the operations follow (cited by page title and section):
 *   [RAPID] "RAPID：基于检索增强的推测解码长上下文推理" (explainer of arXiv
 *           2502.20330): section "2) 推理时知识迁移" gives the mixture
 *           p~ = (1 - lambda) p_t + lambda q; section "3) 候选验证机制（伪代码）"
 *           gives the per-position accept / first-rejection / resample loop.
 *   [SD]    "大模型推理的Speculative Decoding原理详解": section "修改的拒绝采样"
 *           (accept outright when p >= q, else with probability p/q), sections
 *           "批量投机" (many requests verified in one batch) and
 *           "Tree Speculation" (a tree of candidates checked in one pass).
 *   [EAGLE] "投机解码（EAGLE）：让小模型猜、大模型验，无损加速 LLM 生成":
 *           section "1. 为什么无损" (resample from max(0, p - q)), "核心思路"
 *           step 3 (greedy: keep a draft equal to the target's most likely
 *           token) and "3. 验证阶段树形attention" (a node sees its ancestors).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer argument is DEVICE memory owned by the caller, except where
 *    stated.  The library never allocates, frees or synchronises; all work is
 *    enqueued on `stream` and outputs are valid once the stream reaches it.
 *  - Logits are bf16 (SV_BF16) or fp32 (SV_F32).  A logits tensor is laid out
 *    [B, R, V] with R rows per request; row r of request b starts at element
 *    (b * R + r) * ld.  `ld` >= V, `ld * sizeof(elem)` must be a multiple of
 *    16 bytes and the base pointer 16-byte aligned (rows are streamed with
 *    16-byte loads).
 *  - Temperature T (> 0, finite) divides both models' logits before the
 *    softmax.  lambda is in [0, 1].
 *  - Uniforms are fp32 in [0, 1).  A draft is accepted iff u < a, with
 *    a = min(1, p~(x) / q(x)).  One sampling uniform per request drives the
 *    inverse-CDF draw, token = min{ j : F(j) > u }, from the normalised
 *    residual max(0, p~ - q) after a rejection, or from the target's own
 *    softmax(z/T) (the bonus token) when every draft is accepted.
 *  - Argument errors are returned synchronously, before any HIP call.  Data
 *    errors found on the device are OR-ed into the int32 word `*status`
 *    (SV_DATA_* bits; the call first clears it); the caller reads it when
 *    convenient.  HIP launch failures return SV_EHIP.
 *  - `workspace` is caller-owned device scratch of at least the size the
 *    matching *_workspace_bytes() reports, 16-byte aligned, and not shared by
 *    calls that may run concurrently.  Its contents need no initialisation.
 *  - The library keeps no state and is thread-safe, apart from the per-device
 *    address of the fixed scratch array of sv_chain_verify_noalloc, looked up
 *    once per device under a lock.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SV_OK = 0,
    SV_EINVAL = 1,      /* a size or scalar is out of range (B < 0, K > SV_MAX_POSITIONS, T <= 0, ...) */
    SV_ENULL = 2,       /* a required pointer is NULL */
    SV_EALIGN = 3,      /* a logits pointer or row stride is not 16-byte aligned, or ld < V */
    SV_EWORKSPACE = 4,  /* workspace NULL, misaligned or smaller than required */
    SV_EDTYPE = 5,      /* unknown sv_dtype */
    SV_EHIP = 6,        /* a kernel launch failed */
    SV_ETOOBIG = 7,     /* sv_chain_verify_noalloc: the sizes need more than its fixed scratch */
    /* Not codes: they give the type the range of int, so that any int a C
     * caller passes (sv_status_string(99)) is a value of the type in C++ too. */
    SV_STATUS_INT_MIN_ = -0x7fffffff - 1,
    SV_STATUS_INT_MAX_ = 0x7fffffff
} sv_status;

typedef enum {
    SV_BF16 = 0,
    SV_F32 = 1,
    /* not dtypes: the range of int, as for sv_status (an unknown dtype returns SV_EDTYPE) */
    SV_DTYPE_INT_MIN_ = -0x7fffffff - 1,
    SV_DTYPE_INT_MAX_ = 0x7fffffff
} sv_dtype;

/* Where the target and draft models are mixed ([RAPID]): SV_MIX_PROB is the
 * mixture equation of section "2) 推理时知识迁移", p~ = (1 - lambda) p_t +
 * lambda q; SV_MIX_LOGIT is the form of the section-3 pseudocode, p~ =
 * softmax(((1 - lambda) z_t + lambda z_q) / T).  Either p~ takes the target's
 * place in the acceptance ratio min(1, p~(x) / q(x)), in the residual
 * max(0, p~ - q) and in the zero-residual fallback; the bonus token is always
 * drawn from the target's own softmax(z/T).  At lambda = 0 or 1 the two
 * coincide. */
typedef enum { SV_MIX_PROB = 0, SV_MIX_LOGIT = 1 } sv_mix_space;

/* Largest number of drafted positions per request (chain K, tree path Dmax). */
#define SV_MAX_POSITIONS 64
/* Largest number of non-root nodes of a draft tree. */
#define SV_MAX_TREE_NODES 1024
/* Largest vocabulary of the chain and path calls, by dtype (their draw
 * stages at most 4096 piece masses of a sampling row in LDS); a larger V
 * returns SV_EINVAL.  The acceptance-rate, greedy and multi-branch calls
 * accept larger vocabularies. */
#define SV_MAX_VOCAB_BF16 2097152
#define SV_MAX_VOCAB_F32 1048576
/* Largest number of cooperating blocks per tree of the multi-branch call. */
#define SV_MAX_BLOCKS_PER_TREE 32

/* Bits of the device-side status word. */
#define SV_DATA_BAD_TOKEN   0x01 /* a drafted or node token outside [0, V): that draft is rejected */
#define SV_DATA_BAD_ROW     0x02 /* a used row has NaN / +inf or is all -inf: rejected there; a
                                    sampled token from such a row is -1 */
#define SV_DATA_ZERO_Q      0x04 /* a drafted token has draft probability 0: accepted iff p~(x) > 0 */
#define SV_DATA_BAD_LENGTH  0x08 /* draft_len[b] outside [0, K]: clamped */
#define SV_DATA_BAD_TREE    0x10 /* parent or path entry invalid: node never accepted / path cut */
#define SV_DATA_FALLBACK    0x20 /* residual mass was zero after a rejection: sampled p~ instead */
#define SV_DATA_DEPTH       0x40 /* accepted tree path deeper than Dmax: cut at Dmax nodes */
#define SV_DATA_SYNC        0x80 /* sv_tree_verify_multi, one-launch sv_tree_verify_greedy,
                                    sv_chain_acceptance_rate: a wait for another block's or wave's
                                    values gave up (other work held the GPU's compute units); the
                                    call's outputs are invalid */

/* Human-readable name of a status code (static storage, host memory). */
const char *sv_status_string(sv_status s);

/* ------------------------------------------------------------------------
 * Linear chain ([RAPID] verify loop, [SD] batched speculation)
 * ------------------------------------------------------------------------ */

/* Workspace bytes for sv_chain_verify with these sizes (either dtype).
 * Returns 0 for invalid sizes. */
size_t sv_chain_workspace_bytes(int B, int K, int V);

/*
 * Verify B requests of up to K drafts each.
 *
 *  target_logits  [B, K+1, V], row stride ld_t elements; row k of a request
 *                 with K_b drafts is the target's prediction for position k,
 *                 row K_b serves the bonus token.
 *  draft_logits   [B, K, V], row stride ld_q.
 *  draft_tokens   [B, K] int32, token drafted at each position.
 *  draft_len      [B] int32 K_b in [0, K], or NULL (every request drafts K).
 *  u_accept       [B, K] fp32 acceptance uniforms, u_sample [B] fp32.
 *  lambda, temperature: host scalars.
 *  accepted       [B] int32 out: number n_b of accepted drafts (0..K_b).
 *  out_tokens     [B, K+1] int32 out: the n_b accepted drafts, then the
 *                 resampled (n_b < K_b) or bonus (n_b = K_b) token, then -1.
 *  accept_prob    [B, K] fp32 out or NULL: a_i for every i < K_b (also past
 *                 the first rejection); 0 for i >= K_b.
 *  status         [1] int32 out (device) or NULL.
 *  K = 0 is valid: each request then samples one token from target row 0.
 */
sv_status sv_chain_verify(const void *target_logits, int64_t ld_t,
                          const void *draft_logits, int64_t ld_q,
                          sv_dtype dtype, int B, int K, int V,
                          const int32_t *draft_tokens, const int32_t *draft_len,
                          const float *u_accept, const float *u_sample,
                          float lambda, float temperature,
                          int32_t *accepted, int32_t *out_tokens, float *accept_prob,
                          int32_t *status, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Bytes of the device scratch array that sv_chain_verify_noalloc uses in
 * place of a workspace (one array per GPU, held until the process ends). */
#define SV_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * sv_chain_verify for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results as sv_chain_verify, without the workspace: the
 * call uses a file-scope device array of SV_NOALLOC_SCRATCH_BYTES bytes,
 * whose address on the current device it looks up once (hipGetSymbolAddress)
 * on its first call there.  It calls no hipMalloc, hipFree or other
 * allocating routine.  Sizes whose workspace (sv_chain_workspace_bytes)
 * exceeds that array return SV_ETOOBIG before any HIP call; other argument
 * errors as sv_chain_verify.  Every call on one GPU shares that GPU's array
 * and nothing in it needs to start cleared (each call re-initialises what it
 * reads); calls that may overlap on one GPU (other streams, other host
 * threads) race on it and must be serialised by the caller.
 */
sv_status sv_chain_verify_noalloc(const void *target_logits, int64_t ld_t,
                                  const void *draft_logits, int64_t ld_q,
                                  sv_dtype dtype, int B, int K, int V,
                                  const int32_t *draft_tokens, const int32_t *draft_len,
                                  const float *u_accept, const float *u_sample,
                                  float lambda, float temperature,
                                  int32_t *accepted, int32_t *out_tokens, float *accept_prob,
                                  int32_t *status, hipStream_t stream);

/*
 * The two launches sv_chain_verify makes, exposed so that a caller can time or
 * interleave them.  Same arguments and meaning; sv_chain_row_stats streams the
 * drafted rows once and reduces each to (max, sum of exponentials);
 * sv_chain_accept_resample must follow it on the same stream with the same
 * workspace and resolves acceptance, resamples and writes the outputs; it
 * may be repeated on the same statistics (for instance with new uniforms).
 */
sv_status sv_chain_row_stats(const void *target_logits, int64_t ld_t,
                             const void *draft_logits, int64_t ld_q,
                             sv_dtype dtype, int B, int K, int V,
                             const int32_t *draft_tokens, const int32_t *draft_len,
                             const float *u_accept, const float *u_sample,
                             float lambda, float temperature,
                             int32_t *accepted, int32_t *out_tokens, float *accept_prob,
                             int32_t *status, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);
sv_status sv_chain_accept_resample(const void *target_logits, int64_t ld_t,
                                   const void *draft_logits, int64_t ld_q,
                                   sv_dtype dtype, int B, int K, int V,
                                   const int32_t *draft_tokens, const int32_t *draft_len,
                                   const float *u_accept, const float *u_sample,
                                   float lambda, float temperature,
                                   int32_t *accepted, int32_t *out_tokens, float *accept_prob,
                                   int32_t *status, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * sv_chain_row_stats with the row-statistics kernel timed: the launch records
 * kernel_start at the kernel's first wave and kernel_stop after its last (the
 * dispatch's own begin and end timestamps), so hipEventElapsedTime on the pair
 * gives the kernel duration without launch gaps or queueing.  Either event may
 * be NULL (then neither is recorded).  The events are owned by the caller,
 * created with hipEventCreate on the device that runs the stream; errors as
 * sv_chain_row_stats.
 */
sv_status sv_chain_row_stats_timed(const void *target_logits, int64_t ld_t,
                                   const void *draft_logits, int64_t ld_q,
                                   sv_dtype dtype, int B, int K, int V,
                                   const int32_t *draft_tokens, const int32_t *draft_len,
                                   const float *u_accept, const float *u_sample,
                                   float lambda, float temperature,
                                   int32_t *accepted, int32_t *out_tokens, float *accept_prob,
                                   int32_t *status, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream, hipEvent_t kernel_start,
                                   hipEvent_t kernel_stop);

/*
 * sv_chain_verify with the mixture space chosen (mix_space, an sv_mix_space)
 * and the launches selected: stages = 1 runs the row-statistics launch,
 * 2 the accept / resample launches (after a stage-1 call of the same
 * arguments on the same stream and workspace), 3 both.  kernel_start /
 * kernel_stop (either may be NULL) time the call's first launch as in
 * sv_chain_row_stats_timed: the row-statistics kernel for stages 1 and 3,
 * the accept / resample kernel for stages = 2.  In logit space a row-statistics job reads the
 * target and draft chunks of a position together, so each drafted row is
 * still read once.  SV_EINVAL also for an unknown mix_space or stages.
 */
sv_status sv_chain_verify_ex(const void *target_logits, int64_t ld_t,
                             const void *draft_logits, int64_t ld_q,
                             sv_dtype dtype, int B, int K, int V,
                             const int32_t *draft_tokens, const int32_t *draft_len,
                             const float *u_accept, const float *u_sample,
                             float lambda, float temperature,
                             int32_t *accepted, int32_t *out_tokens, float *accept_prob,
                             int32_t *status, void *workspace, size_t workspace_bytes,
                             hipStream_t stream, int mix_space, int stages,
                             hipEvent_t kernel_start, hipEvent_t kernel_stop);

/*
 * Acceptance rate of every drafted position: alpha[b, i] = sum_v
 * min(p~(v), q(v)), the probability that position i accepts a draft drawn
 * from q ([SD] and [EAGLE] define the acceptance rate as the share of drafts
 * the target keeps; with the rule min(1, p~/q) its expectation under q is
 * this sum).  It needs no drafted tokens or uniforms.  Telemetry for a host
 * policy that adapts the draft length or lambda ([EAGLE] "4. 草稿长度和接受率
 * 的权衡"; [RAPID] section 2: lambda is schedulable).  Costs one more read of
 * every drafted row: two launches (row statistics, which also set every
 * alpha to 0; per-chunk min masses, each position's chunks summed in a fixed
 * order by the wave of its last chunk, from tagged records that the reader
 * clears).
 *
 *  Arguments as sv_chain_verify (draft_len may be NULL); mix_space an
 *  sv_mix_space.  alpha [B, K] float out (0 past draft_len[b]; NaN where a
 *  row is bad, with SV_DATA_BAD_ROW in *status).  workspace of at least
 *  sv_chain_acceptance_workspace_bytes(B, K, V) bytes.  A position's summing
 *  wave waits only for blocks dispatched before its own; if that wait gives
 *  up (about a second), its alpha is NaN and SV_DATA_SYNC is set.
 */
size_t sv_chain_acceptance_workspace_bytes(int B, int K, int V);
sv_status sv_chain_acceptance_rate(const void *target_logits, int64_t ld_t,
                                   const void *draft_logits, int64_t ld_q,
                                   sv_dtype dtype, int B, int K, int V,
                                   const int32_t *draft_len, float lambda, float temperature,
                                   int mix_space, float *alpha, int32_t *status,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Draft trees ([SD] "Tree Speculation", [EAGLE] greedy match + tree attention)
 *
 * Node 0 is the root; node i (1..N) has token node_token[b, i-1] and parent
 * parent[b, i-1] in [0, i-1].  Row r of a request's [N+1, V] logits belongs to
 * node r: the target's (or draft's) prediction of the token after node r.
 * ------------------------------------------------------------------------ */

/* Workspace bytes for either tree call with these sizes; 0 for invalid sizes. */
size_t sv_tree_workspace_bytes(int B, int N, int V);

/*
 * Greedy verification: node i is accepted iff its parent is accepted and its
 * token equals the argmax of the parent's target row (lowest token id on
 * ties).  The deepest accepted node wins (lowest node id on ties).
 *
 *  target_logits  [B, N+1, V], stride ld_t.   parent, node_token [B, N] int32.
 *  accepted       [B] out: depth of the winning node (accepted draft count).
 *  out_tokens     [B, Dmax+1] out: tokens of the accepted nodes root->leaf,
 *                 then the argmax of the winning node's row, then -1.
 *  accepted_nodes [B, Dmax] out: accepted node ids root->leaf, then -1.
 *  lambda and temperature do not enter (argmax is temperature-free).
 *
 * Launches.  Trees of at most 64 nodes (N <= 63, the root included) in
 * batches of at most 1024 trees take one launch: the wave that streams a
 * tree's last row chunk walks that tree once the tree's other chunk and row
 * records (tagged with the call, write-through) are in; it waits only for
 * waves of earlier jobs, dispatched before it.  The status word is stored once,
 * by the wave of the batch's last tree.  Other sizes take the two launches below.  In
 * the one-launch form every wait is bounded (about a second): a wave that
 * gives up sets SV_DATA_SYNC, and the call's outputs are then invalid.
 */
sv_status sv_tree_verify_greedy(const void *target_logits, int64_t ld_t, sv_dtype dtype,
                                int B, int N, int V,
                                const int32_t *parent, const int32_t *node_token,
                                int32_t *accepted, int32_t *out_tokens, int32_t *accepted_nodes,
                                int Dmax, int32_t *status, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * The two launches sv_tree_verify_greedy makes for larger trees, exposed so
 * that a caller can time or interleave them (at any size).  Same arguments
 * and meaning; sv_tree_row_argmax
 * streams every target row once and reduces it to per-chunk (max, lowest
 * index) partials; sv_tree_greedy_walk must follow it on the same stream with
 * the same workspace, combines the partials into row argmaxes, walks the
 * parent array and writes the outputs.
 */
sv_status sv_tree_row_argmax(const void *target_logits, int64_t ld_t, sv_dtype dtype,
                             int B, int N, int V,
                             const int32_t *parent, const int32_t *node_token,
                             int32_t *accepted, int32_t *out_tokens, int32_t *accepted_nodes,
                             int Dmax, int32_t *status, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);
sv_status sv_tree_greedy_walk(const void *target_logits, int64_t ld_t, sv_dtype dtype,
                              int B, int N, int V,
                              const int32_t *parent, const int32_t *node_token,
                              int32_t *accepted, int32_t *out_tokens, int32_t *accepted_nodes,
                              int Dmax, int32_t *status, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * sv_tree_verify_greedy with its first launch (the one launch, for the trees
 * it covers; else the row argmax) timed by kernel_start / kernel_stop, events
 * attached to the launch itself as in sv_chain_row_stats_timed.
 */
sv_status sv_tree_verify_greedy_timed(const void *target_logits, int64_t ld_t, sv_dtype dtype,
                                      int B, int N, int V,
                                      const int32_t *parent, const int32_t *node_token,
                                      int32_t *accepted, int32_t *out_tokens,
                                      int32_t *accepted_nodes, int Dmax, int32_t *status,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream,
                                      hipEvent_t kernel_start, hipEvent_t kernel_stop);

/*
 * sv_tree_row_argmax with the row-argmax kernel timed by kernel_start /
 * kernel_stop, exactly as sv_chain_row_stats_timed times its kernel.
 */
sv_status sv_tree_row_argmax_timed(const void *target_logits, int64_t ld_t, sv_dtype dtype,
                                   int B, int N, int V,
                                   const int32_t *parent, const int32_t *node_token,
                                   int32_t *accepted, int32_t *out_tokens,
                                   int32_t *accepted_nodes, int Dmax, int32_t *status,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream,
                                   hipEvent_t kernel_start, hipEvent_t kernel_stop);

/*
 * Tree-attention mask of a batch of draft trees ([EAGLE] "3. 验证阶段树形
 * attention": to verify a whole tree in one target pass, each candidate token
 * may attend only to its ancestor path).  Node i (0 = root) may attend to
 * node j iff j == i or j is an ancestor of i; the root is an ancestor of
 * every node.
 *
 *  parent [B, N] int32 as in the tree calls (node i has parent parent[b, i-1]
 *         in [0, i-1]); may be NULL when N == 0.
 *  mask   [B, N+1, mask_words] uint32 out: bit j % 32 of word j / 32 of row i
 *         is set iff node i may attend to node j; mask_words >= (N + 32) / 32
 *         (words past column N are written as 0).
 *  depth  [B, N+1] int32 out or NULL: edges from the root to node i (the
 *         offset of node i's position after the root's).
 *  status [1] int32 or NULL: OR-ed with SV_DATA_BAD_TREE when a parent is out
 *         of range (that node is then treated as a child of the root).  Unlike
 *         the verify calls, this call does not clear *status first.
 *
 * Errors: SV_EINVAL for B < 0, N outside [0, SV_MAX_TREE_NODES] or too few
 * mask_words; SV_ENULL for a missing mask (or parent when N > 0); SV_EHIP.
 * Needs no workspace.
 */
sv_status sv_tree_attention_mask(const int32_t *parent, int B, int N,
                                 uint32_t *mask, int mask_words, int32_t *depth,
                                 int32_t *status, hipStream_t stream);

/* sv_tree_attention_mask with its kernel timed by kernel_start / kernel_stop,
 * exactly as sv_chain_row_stats_timed times its kernel. */
sv_status sv_tree_attention_mask_timed(const int32_t *parent, int B, int N,
                                       uint32_t *mask, int mask_words, int32_t *depth,
                                       int32_t *status, hipStream_t stream,
                                       hipEvent_t kernel_start, hipEvent_t kernel_stop);

/*
 * Stochastic verification along one caller-chosen root->leaf path: chain
 * acceptance (as sv_chain_verify) where position j drafts node n_{j+1}'s token
 * and is tested on target row n_j and draft row n_j (n_0 = root); the bonus
 * row is target row n_d.
 *
 *  target_logits, draft_logits [B, N+1, V].   node_token [B, N].
 *  path     [B, Dmax] int32 node ids n_1..n_d in [1, N], then -1 (or full).
 *  u_accept [B, Dmax], u_sample [B].
 *  accepted [B], out_tokens [B, Dmax+1], accept_prob [B, Dmax] (or NULL).
 */
sv_status sv_tree_verify_path(const void *target_logits, int64_t ld_t,
                              const void *draft_logits, int64_t ld_q,
                              sv_dtype dtype, int B, int N, int V,
                              const int32_t *node_token, const int32_t *path, int Dmax,
                              const float *u_accept, const float *u_sample,
                              float lambda, float temperature,
                              int32_t *accepted, int32_t *out_tokens, float *accept_prob,
                              int32_t *status, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* sv_tree_verify_path with the mixture space chosen (mix_space, an
 * sv_mix_space); SV_EINVAL also for an unknown mix_space. */
sv_status sv_tree_verify_path_ex(const void *target_logits, int64_t ld_t,
                                 const void *draft_logits, int64_t ld_q,
                                 sv_dtype dtype, int B, int N, int V,
                                 const int32_t *node_token, const int32_t *path, int Dmax,
                                 const float *u_accept, const float *u_sample,
                                 float lambda, float temperature,
                                 int32_t *accepted, int32_t *out_tokens, float *accept_prob,
                                 int32_t *status, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream, int mix_space);

/*
 * Multi-branch stochastic verification of a whole draft tree ([SD] "Tree
 * Speculation": when one branch is rejected another may still be accepted).
 * The pages give no rule; the one used applies the chain rule again to what a
 * rejection leaves.  At node u (starting at the root) the children are tested
 * in node order against a target r, first p~ at row u (mix_space as in
 * sv_chain_verify_ex) with the draft q at row u: child c with token x is
 * accepted iff u_accept[b, c-1] < min(1, r(x) / q(x)) (q(x) = 0: accepted iff
 * r(x) > 0); after a rejection r <- max(0, r - q) normalised, the next child's
 * target.  The first accepted child becomes u.  If every child is rejected,
 * one token is drawn from the last r by inverse CDF with u_sample[b]; at a
 * node without children, or at depth Dmax, the bonus token is drawn from the
 * target's own softmax(z_t/T) at that node.  When each child's token is an
 * independent draw from its parent's q, the emitted tokens follow p~.
 *
 *  target_logits, draft_logits [B, N+1, V]; parent, node_token [B, N] as in
 *  the tree calls; u_accept [B, N] one uniform per node; u_sample [B].
 *  accepted [B] out: depth of the last accepted node (<= Dmax).
 *  out_tokens [B, Dmax+1] out: the accepted nodes' tokens, then the drawn
 *  token, then -1.  accepted_nodes [B, Dmax] out: node ids, -1 padded.
 *  accept_prob [B, N] out or NULL: min(1, r(x)/q(x)) of every tested node,
 *  -1 for nodes never tested.  Dmax in [0, SV_MAX_POSITIONS].
 *  status: cleared, then SV_DATA_* bits (BAD_TREE: a node with an invalid
 *  parent is never tested; BAD_TOKEN: rejected; ZERO_Q; FALLBACK: a residual
 *  had zero mass and its current target was drawn from; BAD_ROW).
 *  workspace: sv_tree_multi_workspace_bytes(B, N, V) bytes (two fp32
 *  residual rows per request, the barrier slots, and the chunk partials of
 *  every tree row).
 *
 * Launches: a row-statistics launch over the rows of every tree (all but
 * those of childless nodes that no step reads), then the walk.
 * Each tree is walked by G cooperating 512-thread blocks (G up to
 * SV_MAX_BLOCKS_PER_TREE; by default as many as let all B * G blocks fit the
 * GPU at once), each owning a slice of the vocabulary: every sum over the
 * vocabulary is a pass of the blocks over their slices, combined at a barrier
 * of the tree's blocks.  The walk is bound by that chain of passes rather than
 * by HBM bandwidth.
 *
 * Residency contract.  A tree's blocks wait for one another.  Each block takes
 * its tree and slice from a start-order ticket, so a block only ever waits for
 * blocks of a tree whose earlier blocks are already running: the call
 * progresses whenever G of its blocks fit on the GPU at once (one per compute
 * unit), whatever else runs there, and a grid wider than the GPU runs its
 * trees in rounds.  SV_DATA_SYNC (outputs invalid; rerun the call) is set only
 * if other work keeps a started tree's remaining blocks from starting for
 * about a second.  G = 1 (sv_tree_verify_multi_ex) has no waits between
 * blocks at all, at the cost of one compute unit's speed per tree.
 */
size_t sv_tree_multi_workspace_bytes(int B, int N, int V);
sv_status sv_tree_verify_multi(const void *target_logits, int64_t ld_t,
                               const void *draft_logits, int64_t ld_q,
                               sv_dtype dtype, int B, int N, int V,
                               const int32_t *parent, const int32_t *node_token,
                               const float *u_accept, const float *u_sample,
                               float lambda, float temperature, int mix_space,
                               int32_t *accepted, int32_t *out_tokens,
                               int32_t *accepted_nodes, float *accept_prob, int Dmax,
                               int32_t *status, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* sv_tree_verify_multi with the number of blocks per tree chosen by the
 * caller: blocks_per_tree 0 is the automatic choice above, 1 ..
 * SV_MAX_BLOCKS_PER_TREE asks for that many (fewer when the row has fewer
 * 512-vector tiles than that); outside that range (and 0) returns SV_EINVAL.  Outputs follow the same rule for every choice; the
 * acceptance values may differ in the last bits, since the per-slice sums are
 * combined in another grouping. */
sv_status sv_tree_verify_multi_ex(const void *target_logits, int64_t ld_t,
                                  const void *draft_logits, int64_t ld_q,
                                  sv_dtype dtype, int B, int N, int V,
                                  const int32_t *parent, const int32_t *node_token,
                                  const float *u_accept, const float *u_sample,
                                  float lambda, float temperature, int mix_space,
                                  int32_t *accepted, int32_t *out_tokens,
                                  int32_t *accepted_nodes, float *accept_prob, int Dmax,
                                  int32_t *status, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream, int blocks_per_tree);

/* ------------------------------------------------------------------------
 * Measurement utility (not a step of the method)
 * ------------------------------------------------------------------------ */

/*
 * Read-stream calibration: reads bytes of device memory at buf once, with
 * the access pattern of the row streams above (one wavefront per 8 KB job,
 * 16-byte non-temporal loads, 256-thread blocks), and folds them with XOR;
 * no other arithmetic.  Its duration over the same byte count as a verify
 * kernel's stream is the practical read ceiling that kernel is compared with.
 *
 *  buf    device memory, 16-byte aligned, owned by the caller.
 *  bytes  a positive multiple of 16.
 *  sink   one device uint32 the kernel writes only when the fold equals a
 *         fixed word (it keeps the loads from being elided); its value means
 *         nothing.
 *  kernel_start, kernel_stop  events recorded at the kernel's own begin and
 *         end (hipExtLaunchKernelGGL), or NULL for an untimed launch.
 * Returns SV_EINVAL (null pointer, bytes 0 or not a multiple of 16, buf not
 * 16-byte aligned, more than 2^31 - 1 blocks) before any HIP call, SV_EHIP
 * when the launch fails.
 */
sv_status sv_read_stream(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream,
                         hipEvent_t kernel_start, hipEvent_t kernel_stop);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
