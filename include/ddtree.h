/*
 * libddtree -- DDTree tree-parallel verify step for AMD MI355X (gfx950).
 *
 * One verify step of tree speculative decoding, for a batch of B requests on
 * one GPU, as described in the blog pages on DDTree ("The Architecture of
 * Speculative Decoding: Dissecting DDTree's Tree-Parallel Evaluation
 * Strategy", Sections 1-3; "The Pivot Point", "The Design Constraint: Load
 * Contexts Once"; "Implementing Temperature-Aware Tree Sampling for DDTree",
 * "Path B"; "The Tree That Couldn't Branch", "Hypothesis 3" and "Hypothesis 4"):
 *
 *   ddtree_draft_topk      draft logits  ->  per-depth top-k tokens and their
 *                          full-vocabulary log-probs (the input of the build)
 *   ddtree_build           per-depth draft top-k  ->  best-first token tree
 *   ddtree_tree_attention  every tree node attends to its request's context
 *                          (streamed from HBM once, shared by all nodes) and
 *                          to its own ancestors (ddtree_tree_attention_ranges:
 *                          the same with per-request context row ranges;
 *                          ..._ranges_capped: lengths read on the device)
 *   ddtree_vocab_reduce    per-node argmax / max / log-sum-exp and, for
 *                          sampling, the exact integer softmax total R
 *   ddtree_verify_greedy   greedy verified-tree walk -> accept length, bonus
 *   ddtree_vocab_verify_greedy  ddtree_vocab_reduce (greedy) and
 *                          ddtree_verify_greedy in one call (one launch fewer)
 *   ddtree_verify_sample   temperature-T tree rejection sampling walk
 *   ddtree_verify_sample_lazy  the same walk, reducing only the rows it visits
 *   ddtree_vocab_top_p     per-node top-p nucleus of the integer target law
 *   ddtree_verify_sample_top_p  the sampled walk on the top-p nuclei
 *   ddtree_verify_linear_sample  linear speculative sampling with draft probabilities
 *   ddtree_commit          the accepted path's K/V rows into the context cache;
 *                          the next step's prefix length and root token
 *
 * Conventions shared by every call
 *   - Every data pointer is device-accessible memory owned by the caller
 *     (unless named *_host): device memory, or pinned host memory mapped for
 *     the device (e.g. the walks' accept_len / bonus, which the host reads
 *     every step).  The library allocates nothing and keeps no state between
 *     calls; workspaces are passed in and sized by the *_workspace_size calls.
 *   - Every call enqueues its kernels on `stream` and returns without waiting.
 *   - The returned status covers argument validation (done on the host before
 *     anything is launched: nothing is enqueued on a non-OK status) and launch
 *     errors (DDTREE_EDEVICE).  ddtree_last_error() gives a thread-local message
 *     for the last non-OK status of the calling thread.
 *   - Preconditions not checked (undefined results otherwise): inputs are
 *     finite (draft log-probs may be -inf, e.g. masked tokens); draft
 *     log-probs are non-increasing along the top-k axis; the draft tokens of
 *     one (request, depth) are distinct; host copies of context offsets and
 *     lengths (the *_host arrays) hold the same values as the device arrays.
 *   - Tensors are dense, row-major, with 16-byte aligned base pointers.
 *   - Calls are thread-safe (no shared state); calls on one stream are ordered.
 *   - Walk results without a stream synchronisation: every walk
 *     (ddtree_verify_greedy, ddtree_vocab_verify_greedy, ddtree_verify_sample,
 *     ddtree_verify_sample_lazy, ddtree_verify_sample_top_p,
 *     ddtree_verify_linear_sample) stores accept_len[b] last, after request b's
 *     other outputs and a system-scope release.  A host that places accept_len
 *     (and the other outputs it wants to read) in mapped pinned host memory,
 *     fills accept_len with a negative value before enqueuing the step, and
 *     polls it may read request b's bonus, out_tokens and path_nodes as soon
 *     as accept_len[b] >= 0, without waiting for the kernels to end.  Later
 *     work on the stream still runs after the walk has ended.
 */
#ifndef DDTREE_H
#define DDTREE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DDTREE_OK = 0,
  DDTREE_EINVAL = 1,       /* bad argument (null pointer, size out of range, ...) */
  DDTREE_EUNSUPPORTED = 2, /* valid but not implemented (e.g. head_dim 96) */
  DDTREE_EDEVICE = 3       /* a HIP launch or runtime call failed */
} ddtree_status;

/* Element type codes.  The type is a plain 32-bit integer, not an enum, so
 * that any value a caller passes is well defined on both sides of the ABI;
 * values other than these two are rejected with DDTREE_EINVAL. */
typedef int32_t ddtree_dtype;
enum { DDTREE_F32 = 0, DDTREE_BF16 = 1 };

/* Size limits (validated). */
#define DDTREE_MAX_NODES 128  /* N = budget + 1 */
#define DDTREE_MAX_DEPTH 64   /* D */
#define DDTREE_MAX_TOPK 64    /* K */
#define DDTREE_R_BLOCK 32768  /* tokens per block of the sampling weight sums (R_blocks) */

/*
 * The token tree of a batch: structure-of-arrays, one row of N = budget + 1
 * entries per request, root at index 0, nodes numbered in the order the
 * best-first build takes them (so parent[i] < i).  All arrays are device
 * memory of the shapes given; entries n >= num_nodes[b] are padding
 * (integer fields -1, score -inf, vis 0).
 */
typedef struct {
  int32_t* token;        /* [B, N] draft token of the node (root: the anchor token) */
  int32_t* parent;       /* [B, N] parent index, -1 for the root */
  int32_t* depth;        /* [B, N] 0 for the root */
  int32_t* rank;         /* [B, N] rank of the token in its depth's top-k, -1 for the root */
  int32_t* position;     /* [B, N] prefix_len[b] + depth */
  int32_t* first_child;  /* [B, N] lowest-rank child, -1 if none */
  int32_t* next_sibling; /* [B, N] next-rank sibling, -1 if none */
  float* score;          /* [B, N] cumulative draft log-prob (fp32 sum), root 0 */
  uint64_t* vis;         /* [B, N, W] bit j of row i: node i sees node j (ancestors and itself) */
  int32_t* num_nodes;    /* [B] 1 + number of nodes taken (<= N) */
  int32_t B, N, D, K, W; /* W = (N + 63) / 64 */
  int32_t* max_depth;    /* [B] depth of the deepest node taken (0 if only the root), or
                            NULL: written by ddtree_build when set, read by nothing else */
} ddtree_tree;

/*
 * ddtree_draft_topk -- per-depth top-k of the draft head.
 * Source: "Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 1
 * step 1 (from every depth position of the draft forward, the top-k candidate
 * tokens and their log-probs, which step 2 turns into cumulative scores).
 * Readings: the log-prob is the log-softmax of the whole row at temperature 1
 * (not renormalised over the top-k); candidates are ordered by logit,
 * descending, equal logits by lower token id.
 *   logits     [rows, V] bf16 or fp32 (rows = requests x depths, any order;
 *              typically the [B, D, V] draft outputs viewed as B*D rows)
 *   K          1 <= K <= min(V, 64)
 *   tokens     [rows, K] int32   rank-ordered token ids
 *   logprobs   [rows, K] fp32    logit - log-sum-exp of the row (computed in
 *              fp32: within ~1e-5 of the exact value for V = 163840)
 *   workspace  ddtree_draft_topk_workspace_size(rows, V, K) bytes (may be 0),
 *              16-byte aligned device scratch; contents need no
 *              initialisation and are garbage afterwards (calls sharing it
 *              must not overlap).
 * The tokens are exact (pure comparisons of the given logits).
 * Errors: DDTREE_EINVAL (null pointers, sizes, K out of range, dtype),
 *         DDTREE_EUNSUPPORTED (rows > 65535).
 */
size_t ddtree_draft_topk_workspace_size(int32_t rows, int32_t V, int32_t K);

ddtree_status ddtree_draft_topk(const void* logits, ddtree_dtype dtype, int32_t rows, int32_t V,
                                int32_t K, int32_t* tokens, float* logprobs, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * ddtree_build -- best-first tree from per-depth top-k draft log-probs.
 * Source: "Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 1,
 * steps 2-3 (heap on cumulative log-prob: take the best entry, add it, offer
 * its best child and next sibling, until `budget` nodes; visibility = the
 * ancestors); "The Tree That Couldn't Branch", "Hypothesis 3" (position =
 * prefix length + depth) and "Hypothesis 4" (every depth-d node draws its
 * children from the same depth-d top-k).
 *   draft_lp   [B, D, K] fp32  log-prob of the rank-r token at depth d+1
 *   draft_tok  [B, D, K] int32 the token itself
 *   root_tok   [B] int32, prefix_len [B] int32
 *   budget     nodes to take besides the root, 1 <= budget <= 127;
 *              tree->N must equal budget + 1 and tree->B/D/K/W match.
 * Order: larger cumulative score first (score(child) = fp32(score(parent) +
 * draft_lp), one rounded add), ties by smaller parent index then smaller rank.
 * tree->max_depth, when not NULL, receives each request's deepest depth: the
 * statistic that tells whether the budget went to breadth before the tree
 * reached the drafter's last depth ("The Tree That Couldn't Branch",
 * "Hypothesis 1: Best-First Search Exhaustion"; read beside node counts and
 * accepted depths in "The Experiment: budget=7, topk_cap=1").
 * Errors: DDTREE_EINVAL for null pointers or out-of-range sizes.
 */
ddtree_status ddtree_build(const float* draft_lp, const int32_t* draft_tok,
                           const int32_t* root_tok, const int32_t* prefix_len, int32_t B,
                           int32_t D, int32_t K, int32_t budget, const ddtree_tree* tree,
                           hipStream_t stream);

/*
 * ddtree_tree_attention -- tree attention with the context loaded once.
 * Source: "Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 1
 * step 4 and Section 2; "The Pivot Point", "The Design Constraint: Load
 * Contexts Once": every tree node of request b attends to all L_b context
 * keys and to the tree keys its vis row marks; each context K/V element is
 * read from HBM once and used by every tree query.
 *   q            [B, N, Hq, Dh]        dtype
 *   k_ctx, v_ctx [ctx_offsets[B], Hkv, Dh] dtype; request b owns rows
 *                [ctx_offsets[b], ctx_offsets[b+1])
 *   ctx_offsets  [B+1] int32 device;  ctx_offsets_host: the same values in host memory
 *   k_tree, v_tree [B, N, Hkv, Dh]    dtype (the tree tokens' own K/V)
 *   tree         from ddtree_build (uses vis, num_nodes)
 *   Hq % Hkv == 0, query head h reads KV head h / (Hq / Hkv); Dh in {64, 128};
 *   M = N * Hq / Hkv <= 1024 query rows per KV head.  Up to 128 rows share
 *   one pass over the context; larger M is processed in 128-row slices, each
 *   of which reads the context once more.
 *   scale        score scale > 0, or 0 for 1/sqrt(Dh) (the pages give no scale;
 *                1/sqrt(Dh) is the usual one)
 *   out          [B, N, Hq, Dh] dtype; padding nodes get 0
 *   lse          [B, N, Hq] fp32 natural-log softmax denominator, or NULL
 *   workspace    device scratch of at least
 *                ddtree_tree_attention_workspace_size(...) bytes (contents
 *                need no initialisation and are garbage afterwards)
 * Context lengths: the host copy decides the work split and the grid.  For
 * B <= 64 the kernels take every context range from the host copy (the device
 * array is not read), so a call captured in a HIP graph keeps the ranges it
 * was captured with (ddtree_tree_attention_ranges_capped reads the lengths on
 * the device instead, for captured steps over growing caches).  For B > 64 the kernels look their ranges up in the
 * device array, which must then hold the host copy's values; if it does not,
 * the output is undefined but no workspace access leaves the planned splits.
 * Errors: DDTREE_EINVAL (null pointers, sizes, small workspace),
 *         DDTREE_EUNSUPPORTED (other Dh, too many query rows per KV head).
 */
size_t ddtree_tree_attention_workspace_size(int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                                            int32_t Dh, const int32_t* ctx_offsets_host);

ddtree_status ddtree_tree_attention(const void* q, const void* k_ctx, const void* v_ctx,
                                    const int32_t* ctx_offsets, const int32_t* ctx_offsets_host,
                                    const void* k_tree, const void* v_tree,
                                    const ddtree_tree* tree, int32_t Hq, int32_t Hkv, int32_t Dh,
                                    ddtree_dtype dtype, float scale, void* out, float* lse,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ddtree_tree_attention_tuned -- ddtree_tree_attention with its work split
 * chosen by the caller instead of planned (a tuning and test entry point: the
 * split size changes the order in which partial sums meet, so outputs differ
 * from the planned call's within rounding).  Source: as ddtree_tree_attention.
 *   tuning->split_keys  context keys per workgroup, rounded up to whole
 *                       key tiles; 0 keeps the planned size
 *   tuning->stages      LDS ring depth of the bf16 head_dim-128 kernel when the
 *                       query rows of a KV head fit four waves (2, 3 or 4);
 *                       0 keeps 2
 *   workspace           ddtree_tree_attention_tuned_workspace_size(..., tuning)
 * tuning == NULL is ddtree_tree_attention.  Every other argument as there.
 * Errors: as ddtree_tree_attention; DDTREE_EINVAL for negative split_keys or a
 *         stage count other than 0, 2, 3, 4.
 */
typedef struct {
  int32_t split_keys;
  int32_t stages;
} ddtree_attention_tuning;

size_t ddtree_tree_attention_tuned_workspace_size(int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                                                  int32_t Dh, const int32_t* ctx_offsets_host,
                                                  const ddtree_attention_tuning* tuning);

ddtree_status ddtree_tree_attention_tuned(const void* q, const void* k_ctx, const void* v_ctx,
                                          const int32_t* ctx_offsets,
                                          const int32_t* ctx_offsets_host, const void* k_tree,
                                          const void* v_tree, const ddtree_tree* tree, int32_t Hq,
                                          int32_t Hkv, int32_t Dh, ddtree_dtype dtype, float scale,
                                          void* out, float* lse, void* workspace,
                                          size_t workspace_bytes,
                                          const ddtree_attention_tuning* tuning,
                                          hipStream_t stream);

/*
 * ddtree_tree_attention_noalloc -- ddtree_tree_attention for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same kernels, split plan and
 * outputs, bit for bit, with the split partials kept in a device array of the
 * library instead of a caller workspace.  The call itself allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); the first call on a
 * device looks the array's address up on that device.
 *   Every argument except the workspace: as ddtree_tree_attention.
 *   The array holds DDTREE_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU for the life
 *   of the process; a call whose split partials need more (see
 *   ddtree_tree_attention_workspace_size; the five reference workloads need at
 *   most ~41 MB) is rejected with DDTREE_EUNSUPPORTED before any launch.
 *   Every call on one GPU uses that GPU's one array: calls that overlap on a
 *   GPU (different streams or host threads without ordering between them)
 *   race and give undefined outputs; calls ordered on one stream do not.  The
 *   kernels need no initialised contents (every partial they read was written
 *   by the same call).
 * Errors: as ddtree_tree_attention; DDTREE_EUNSUPPORTED when the partials do
 *         not fit; DDTREE_EDEVICE when the array's address cannot be obtained.
 */
#define DDTREE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

ddtree_status ddtree_tree_attention_noalloc(const void* q, const void* k_ctx, const void* v_ctx,
                                            const int32_t* ctx_offsets,
                                            const int32_t* ctx_offsets_host, const void* k_tree,
                                            const void* v_tree, const ddtree_tree* tree,
                                            int32_t Hq, int32_t Hkv, int32_t Dh,
                                            ddtree_dtype dtype, float scale, void* out,
                                            float* lse, hipStream_t stream);

/*
 * ddtree_tree_attention_ranges -- the same tree attention with each request's
 * context given as a (start, length) range of rows instead of packed offsets,
 * so that a batch can keep its caches in per-request slabs that grow in place
 * (ddtree_commit appends the accepted path at row cache_base[b] + position;
 * the next step then passes ctx_start = cache_base, ctx_len = next_prefix_len).
 * Source: as ddtree_tree_attention; "Dissecting DDTree's Tree-Parallel
 * Evaluation Strategy", Section 2 (the cache that later steps read once grows
 * by the committed tokens).
 *   ctx_start, ctx_len  [B] int32 device: request b's context is rows
 *                [ctx_start[b], ctx_start[b] + ctx_len[b]) of k_ctx / v_ctx
 *                (ranges may leave gaps; rows outside every range are not read)
 *   ctx_start_host, ctx_len_host  the same values in host memory (the split
 *                plan is made on the host)
 *   workspace    ddtree_tree_attention_ranges_workspace_size(...) bytes
 * Every other argument, the outputs and the numerics are those of
 * ddtree_tree_attention.
 * Errors: as ddtree_tree_attention; DDTREE_EINVAL also for a negative start or
 *         length, or start + length beyond INT32_MAX.
 */
size_t ddtree_tree_attention_ranges_workspace_size(int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                                                   int32_t Dh, const int32_t* ctx_len_host);

ddtree_status ddtree_tree_attention_ranges(const void* q, const void* k_ctx, const void* v_ctx,
                                           const int32_t* ctx_start, const int32_t* ctx_len,
                                           const int32_t* ctx_start_host,
                                           const int32_t* ctx_len_host, const void* k_tree,
                                           const void* v_tree, const ddtree_tree* tree,
                                           int32_t Hq, int32_t Hkv, int32_t Dh,
                                           ddtree_dtype dtype, float scale, void* out,
                                           float* lse, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream);

/*
 * ddtree_tree_attention_ranges_capped -- ddtree_tree_attention_ranges with the
 * context lengths read from device memory when the kernels run: the host
 * gives only an upper bound per request, so one call captured in a HIP graph
 * stays valid while the caches grow (a decode loop replays the captured step
 * while ddtree_commit advances ctx_len on the device).
 * Source: as ddtree_tree_attention_ranges ("Dissecting DDTree's Tree-Parallel
 * Evaluation Strategy", Section 2: the cache grows by the committed tokens).
 *   ctx_start      [B] int32 device, as in ddtree_tree_attention_ranges
 *   ctx_len        [B] int32 device: the lengths, read when the kernels run;
 *                  a length above its bound is read as the bound, a negative
 *                  one as 0
 *   ctx_start_host [B] the starts in host memory
 *   ctx_cap_host   [B] host upper bounds of the lengths: they fix the work split,
 *                  the grid and the workspace (the splits past a request's
 *                  current length stay idle)
 *   workspace      ddtree_tree_attention_ranges_workspace_size(..., ctx_cap_host)
 *                  bytes
 * Every other argument and the outputs are those of ddtree_tree_attention_ranges;
 * results equal that call's with ctx_len_host = ctx_cap_host's split size, i.e.
 * within the attention tolerance of the exact-length call.
 * Errors: as ddtree_tree_attention_ranges, with the bounds checked as the
 *         lengths are there; DDTREE_EUNSUPPORTED for B > 64.
 */
ddtree_status ddtree_tree_attention_ranges_capped(
    const void* q, const void* k_ctx, const void* v_ctx, const int32_t* ctx_start,
    const int32_t* ctx_len, const int32_t* ctx_start_host, const int32_t* ctx_cap_host,
    const void* k_tree, const void* v_tree, const ddtree_tree* tree, int32_t Hq, int32_t Hkv,
    int32_t Dh, ddtree_dtype dtype, float scale, void* out, float* lse, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * ddtree_vocab_reduce -- one pass over the target logits of every tree node.
 * Source: "Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 1
 * step 4 (argmax at every node in parallel) and Section 3 (softmax at
 * temperature T over the verify logits).
 *   logits    [B, N, V] dtype (row b, n: the target's prediction after node n)
 *   num_nodes [B] rows n >= num_nodes[b] are skipped (argmax -1, maxv -inf, R 0,
 *             lse -inf)
 *   argmax    [B, N] int32, lowest token id among equal maxima
 *   maxv      [B, N] fp32, the logit at argmax (+0.0 for a zero)
 *   temperature  0 => greedy only; > 0 => also R
 *   R         [B, N] uint64 (required iff temperature > 0): exact sum over the
 *             row of the integer weights w(l) = floor(p * 2^(32+k)) where
 *             y = (l - maxv) * c, c = fp32(log2(e) / T), k = rint(y),
 *             f = y - k, p = degree-6 Taylor polynomial of 2^f in fp32 with
 *             separately rounded multiplies and adds, coefficients
 *             fp32((ln 2)^n / n!), and w = 0 when y < -32.  w/R is the
 *             temperature-T softmax to ~1e-6 relative; ddtree_verify_sample
 *             recomputes the same w.  Sampling rows need V <= 64 * DDTREE_R_BLOCK.
 *   R_blocks  [B, N, ceil(V / DDTREE_R_BLOCK)] uint64 or NULL: the same weights
 *             summed over each block of DDTREE_R_BLOCK consecutive tokens
 *             (R is their sum); ddtree_verify_sample uses them to find the
 *             block of its residual draw without re-weighing the whole row.
 *             Written only when temperature > 0 (padding rows: 0).
 *   lse       [B, N] fp32 natural-log log-sum-exp of the raw logits, or NULL
 *   workspace ddtree_vocab_reduce_workspace_size(B, N, V) bytes (may be 0),
 *             16-byte aligned device scratch; contents need no
 *             initialisation and are garbage afterwards (calls sharing it
 *             must not overlap).  Required when greedy and that size is
 *             non-zero.  Unused when sampling (may be NULL): a workgroup
 *             takes each row whole, bf16 rows without lse held in registers.
 * Errors: DDTREE_EINVAL (null pointers, sizes, temperature < 0 or NaN),
 *         DDTREE_EUNSUPPORTED (sampling with V > 64 * DDTREE_R_BLOCK).
 */
size_t ddtree_vocab_reduce_workspace_size(int32_t B, int32_t N, int32_t V);

ddtree_status ddtree_vocab_reduce(const void* logits, ddtree_dtype dtype, int32_t B, int32_t N,
                                  int32_t V, const int32_t* num_nodes, float temperature,
                                  int32_t* argmax, float* maxv, uint64_t* R, uint64_t* R_blocks,
                                  float* lse, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * ddtree_verify_greedy -- greedy verified-tree walk.
 * Source: "Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 1
 * step 5: from the root take the child whose token equals the argmax at the
 * current node; stop when none does; the bonus is the argmax at the last node.
 *   argmax      [B, N] from ddtree_vocab_reduce
 *   accept_len  [B]          number of accepted draft tokens (0..D)
 *   path_nodes  [B, D+1]     root, then the accepted nodes, then -1
 *   out_tokens  [B, D+1]     the accepted draft tokens, then the bonus, then -1
 *   bonus       [B]
 * Errors: DDTREE_EINVAL (null pointers, tree sizes).
 */
ddtree_status ddtree_verify_greedy(const ddtree_tree* tree, const int32_t* argmax,
                                   int32_t* accept_len, int32_t* path_nodes, int32_t* out_tokens,
                                   int32_t* bonus, hipStream_t stream);

/*
 * ddtree_vocab_verify_greedy -- the greedy vocabulary reduction and the
 * greedy walk in one call: the same argmax, maxv, accept_len, path_nodes,
 * out_tokens and bonus as ddtree_vocab_reduce (temperature 0, no lse)
 * followed by ddtree_verify_greedy, bit for bit.  The per-row merge of the
 * vocabulary slices and the walk share one launch (one workgroup per
 * request), which saves a dependent kernel launch at small batch.
 * Source: as ddtree_vocab_reduce ("Dissecting DDTree's Tree-Parallel
 * Evaluation Strategy", Section 1 step 4: argmax at every node) and
 * ddtree_verify_greedy (Section 1 step 5).
 *   logits      [B, N, V] row-major, dtype bf16 or f32; B and N from `tree`
 *   argmax, maxv  [B, N] outputs as ddtree_vocab_reduce's (padding rows:
 *               -1 and -inf)
 *   accept_len, path_nodes, out_tokens, bonus: as ddtree_verify_greedy
 *   workspace   ddtree_vocab_reduce_workspace_size(B, N, V) bytes, 16-byte
 *               aligned (may be null when that size is 0); caller-owned
 * Errors: DDTREE_EINVAL (null pointers, tree sizes, V < 1, unknown dtype,
 *         workspace missing or too small).
 */
ddtree_status ddtree_vocab_verify_greedy(const void* logits, ddtree_dtype dtype, int32_t V,
                                         const ddtree_tree* tree, int32_t* argmax, float* maxv,
                                         int32_t* accept_len, int32_t* path_nodes,
                                         int32_t* out_tokens, int32_t* bonus, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/*
 * ddtree_verify_sample -- temperature-T tree rejection sampling walk.
 * Source: "Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 3
 * (tree-structured rejection sampling: test the children, renormalise the
 * residual on rejection, draw the bonus from the residual and stop);
 * "Implementing Temperature-Aware Tree Sampling for DDTree", "Path B".
 * The children are the deterministic top-k, so child c is accepted with the
 * residual target probability of its token: with t = floor(u * R_res / 2^64),
 * c is accepted iff t < w(c); on rejection R_res -= w(c) and the token is
 * excluded.  Children are tried in rank order.  When no child is accepted (or
 * the node is a leaf), the bonus is the smallest token x whose running sum of
 * non-excluded weights exceeds floor(u' * R_res / 2^64).
 *   logits [B, N, V] dtype, maxv [B, N], R [B, N] and R_blocks
 *   [B, N, ceil(V / DDTREE_R_BLOCK)] from ddtree_vocab_reduce with the same
 *   temperature; uniforms [B, N, 2] uint64: slot 0 = the node's accept test,
 *   slot 1 = its bonus draw.  Outputs as ddtree_verify_greedy.
 *   The residual draw subtracts the rejected tokens' weights from their
 *   blocks, picks the block holding the draw, and weighs only that block.
 * Errors: DDTREE_EINVAL (null pointers, sizes, temperature <= 0 or NaN),
 *         DDTREE_EUNSUPPORTED (V > 64 * DDTREE_R_BLOCK).
 */
ddtree_status ddtree_verify_sample(const ddtree_tree* tree, const void* logits,
                                   ddtree_dtype dtype, int32_t V, const float* maxv,
                                   const uint64_t* R, const uint64_t* R_blocks, float temperature,
                                   const uint64_t* uniforms,
                                   int32_t* accept_len, int32_t* path_nodes, int32_t* out_tokens,
                                   int32_t* bonus, hipStream_t stream);

/*
 * ddtree_verify_sample_lazy -- the sampled walk, with the target rows reduced
 * only when the walk reaches them.
 * Source: "Implementing Temperature-Aware Tree Sampling for DDTree", "Path B:
 * CPU-Side Tree Rejection Sampling" (the target softmax computed lazily, for
 * the nodes the rejection walk visits only), with the walk of
 * ddtree_verify_sample.  Computes exactly what ddtree_vocab_reduce
 * (temperature) followed by ddtree_verify_sample computes (bit-identical
 * accept_len, path_nodes, out_tokens, bonus), but reads and weighs only the
 * accept_len + 1 rows the walk visits instead of all N rows of every request:
 * one 1024-thread workgroup per request, row after row.  Worth it when accept
 * lengths are short next to the tree size; needs no maxv, R or workspace.
 *   logits, uniforms, outputs, temperature: as for ddtree_verify_sample.
 * Errors: DDTREE_EINVAL (null pointers, tree sizes, temperature <= 0, dtype),
 *         DDTREE_EUNSUPPORTED (V > 64 * DDTREE_R_BLOCK).
 */
ddtree_status ddtree_verify_sample_lazy(const ddtree_tree* tree, const void* logits,
                                        ddtree_dtype dtype, int32_t V, float temperature,
                                        const uint64_t* uniforms, int32_t* accept_len,
                                        int32_t* path_nodes, int32_t* out_tokens, int32_t* bonus,
                                        hipStream_t stream);

/*
 * ddtree_vocab_top_p -- the top-p (nucleus) truncation of every node's target
 * law, for ddtree_verify_sample_top_p.
 * Source: "Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 3
 * (temperature and top_p threaded through to the verify walk).
 * Readings: tokens are ordered by their integer weight w (see
 * ddtree_vocab_reduce) descending, equal weights by id ascending; the nucleus
 * is the shortest prefix whose weight sum S satisfies 2^32 * S >= P * R with
 * P = rint(top_p * 2^32) clamped to [1, 2^32].  It is described by its last
 * token (weight thr_w, id thr_id): a token is kept iff w > thr_w, or
 * w == thr_w and id <= thr_id.
 *   logits [B, N, V] dtype; num_nodes [B]; maxv, R [B, N] from
 *   ddtree_vocab_reduce at the same temperature (temperature > 0)
 *   top_p in (0, 1]
 *   thr_w [B, N] uint64, thr_id [B, N] int32, Rp [B, N] uint64 (the kept
 *   total), Rp_blocks [B, N, ceil(V / DDTREE_R_BLOCK)] uint64 (kept weight per
 *   token block).  Padding rows: 0, -1, 0, 0.
 * One 1024-thread workgroup per row; a few passes over the row and then an
 * LDS-resident search while the candidates fit (8192 tokens), row passes
 * otherwise.
 * Errors: DDTREE_EINVAL (null pointers, sizes, temperature, top_p, dtype),
 *         DDTREE_EUNSUPPORTED (V > 64 * DDTREE_R_BLOCK).
 */
ddtree_status ddtree_vocab_top_p(const void* logits, ddtree_dtype dtype, int32_t B, int32_t N,
                                 int32_t V, const int32_t* num_nodes, const float* maxv,
                                 const uint64_t* R, float temperature, float top_p,
                                 uint64_t* thr_w, int32_t* thr_id, uint64_t* Rp,
                                 uint64_t* Rp_blocks, hipStream_t stream);

/*
 * ddtree_verify_sample_top_p -- the sampled walk of ddtree_verify_sample on
 * the rows' top-p nuclei: every weight outside its row's nucleus counts as 0
 * (accept tests, residual totals and the residual draw alike).
 * Source: as ddtree_verify_sample; "Dissecting DDTree's Tree-Parallel
 * Evaluation Strategy", Section 3 (top_p threaded through to the walk).
 *   maxv from ddtree_vocab_reduce; Rp, Rp_blocks, thr_w, thr_id from
 *   ddtree_vocab_top_p; every other argument and output as ddtree_verify_sample.
 * Errors: as ddtree_verify_sample.
 */
ddtree_status ddtree_verify_sample_top_p(const ddtree_tree* tree, const void* logits,
                                         ddtree_dtype dtype, int32_t V, const float* maxv,
                                         const uint64_t* Rp, const uint64_t* Rp_blocks,
                                         const uint64_t* thr_w, const int32_t* thr_id,
                                         float temperature, const uint64_t* uniforms,
                                         int32_t* accept_len, int32_t* path_nodes,
                                         int32_t* out_tokens, int32_t* bonus,
                                         hipStream_t stream);

/*
 * ddtree_verify_linear_sample -- linear speculative sampling with the draft's
 * own probabilities (a chain of D drafted tokens, no tree).
 * Source: "Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 3
 * (linear DFlash at temperature T: accept the drafted token with probability
 * min(1, p_target / p_draft), else draw from the residual and stop) and
 * "Mistakes and Incorrect Assumptions" (the draft's full probability of the
 * sampled token is needed, not only its top-k log-prob).
 * Readings: the drafted tokens were drawn from the draft's softmax at the same
 * T; the residual is max(0, q - p) renormalised; q and p are the exact integer
 * laws w / R (see ddtree_vocab_reduce), so position k accepts its token x iff
 * floor(u0 * wp(x) * Rq / 2^64) < wq(x) * Rp, a rejection draws
 * t = floor(u1 * Rr / 2^64) over r(y) = max(0, wq(y) Rp - wp(y) Rq) (from q if
 * Rr = 0), and after D acceptances the bonus is drawn from target row D.
 *   target_logits [B, D+1, V]  row k: the target's distribution for position k+1
 *   draft_logits  [B, D, V]    row k: the draft distribution token k was drawn from
 *   draft_tokens  [B, D] int32
 *   maxq, Rq, Rq_blocks  ddtree_vocab_reduce(target_logits as [B, D+1, V],
 *                  num_nodes = D+1, temperature): [B, D+1], [B, D+1], [B, D+1, nb]
 *   maxp, Rp       ddtree_vocab_reduce(draft_logits as [B, D, V], num_nodes = D,
 *                  temperature): [B, D], [B, D]
 *   uniforms       [B, D+1, 2] raw 64-bit: slot 0 = accept test of position k,
 *                  slot 1 = residual draw at k (or the bonus draw at k = D)
 *   accept_len [B], out_tokens [B, D+1] (accepted tokens, then the residual or
 *   bonus token, then -1), bonus [B]
 * One 1024-thread workgroup per request; a residual is summed over the whole
 * row pair (ALU work of the order of a vocabulary pass over two rows).
 * Errors: DDTREE_EINVAL (null pointers, sizes, temperature <= 0, dtype),
 *         DDTREE_EUNSUPPORTED (V > 64 * DDTREE_R_BLOCK).
 */
ddtree_status ddtree_verify_linear_sample(const void* target_logits, const void* draft_logits,
                                          ddtree_dtype dtype, int32_t B, int32_t D, int32_t V,
                                          const int32_t* draft_tokens, const float* maxq,
                                          const uint64_t* Rq, const uint64_t* Rq_blocks,
                                          const float* maxp, const uint64_t* Rp,
                                          float temperature, const uint64_t* uniforms,
                                          int32_t* accept_len, int32_t* out_tokens,
                                          int32_t* bonus, hipStream_t stream);

/*
 * ddtree_commit -- commit the accepted path into the context KV cache.
 * Source: "Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 1
 * step 5 and its summary (the single longest verified path is committed) and
 * Section 2 (the context cache grows by the committed tokens and is read once
 * by later steps).
 * Readings: the rows committed are the verify pass's K/V of the root and of the
 * accepted nodes (path_nodes[b][0 .. accept_len[b]]); node n goes to its tree
 * position (tree->position, = prefix_len + depth); the bonus token has no K/V
 * yet and becomes the next root.
 *   tree        the build's outputs (position is read)
 *   accept_len, path_nodes [B, D+1], bonus   from a verify walk
 *   k_tree, v_tree [B, N, Hkv, Dh] (dtype): the tree's keys and values, as
 *               passed to ddtree_tree_attention
 *   k_cache, v_cache [cache_rows, Hkv, Dh] (dtype): the cache; request b's
 *               position p is row cache_base[b] + p (for one request, the
 *               packed context of ddtree_tree_attention with ctx_offsets
 *               {0, prefix_len}; for several, per-request slabs)
 *   cache_base  [B] int64 device array
 *   capacity    positions per request: a row whose position is >= capacity,
 *               or whose row index falls outside [0, cache_rows), is not
 *               written (no error; compare next_prefix_len with capacity)
 *   next_prefix_len [B]  position[b][0] + accept_len[b] + 1, or -1 when
 *               accept_len[b] is outside [0, D] (nothing is written then)
 *   next_root   [B]      the bonus token
 * next_prefix_len / next_root may alias the build's prefix_len / root_tok
 * inputs (not accept_len or path_nodes); the cache must not overlap k_tree /
 * v_tree.
 * Errors: DDTREE_EINVAL (null pointers, sizes, dtype, alignment),
 *         DDTREE_EUNSUPPORTED (Hkv * Dh * element size not a multiple of 16).
 */
ddtree_status ddtree_commit(const ddtree_tree* tree, const int32_t* accept_len,
                            const int32_t* path_nodes, const int32_t* bonus, const void* k_tree,
                            const void* v_tree, int32_t Hkv, int32_t Dh, ddtree_dtype dtype,
                            void* k_cache, void* v_cache, const int64_t* cache_base,
                            int64_t cache_rows, int32_t capacity, int32_t* next_prefix_len,
                            int32_t* next_root, hipStream_t stream);

/* Host-only helper: the constants the sampling weights use for temperature T
 * (c = fp32(log2(e)/T) and a[0..6] = fp32((ln 2)^n / n!)).  No GPU needed. */
ddtree_status ddtree_sampling_constants(float temperature, float* c, float* a7);

/* Thread-local message for the last non-OK status returned on this thread. */
const char* ddtree_last_error(void);

/* Library version string. */
const char* ddtree_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DDTREE_H */
