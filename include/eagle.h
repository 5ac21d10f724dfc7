/*
 * eagle.h - C ABI of the EAGLE-2 draft-and-verify hot path for AMD MI355X
 * (gfx950).
 *
 * One cycle of EAGLE-2 speculative decoding over a dynamic draft tree:
 * build the tree's ancestor mask, run tree-masked attention of the tree nodes
 * against a KV prefix, project features through the LM head with softmax
 * statistics and top-k, grow and prune the tree by cumulative log-probability,
 * and accept the longest verified path (greedy, or speculative sampling).
 *
 * The method is described on the pages
 *   [G] "EAGLE-2: Feature-Level Speculative Decoding Guide" (aifetchly blog),
 *   [D] "Support Eagle-3 Speculative Decoding in llama.cpp" (discussion #15902),
 *   [P] "EAGLE-2 Speculative Decoding Support for llama.cpp - Phase 1"
 *       (PR #13908).
 * Each entry point below names the passage that defines its operation.
 *
 * Conventions shared by every call
 *   - Every pointer is a DEVICE pointer unless marked (host).  The caller owns
 *     all memory; the library never allocates, frees or keeps a pointer after
 *     the call returns.  Workspaces are caller-provided scratch whose size the
 *     matching *_workspace() query returns; their contents need no
 *     initialisation and are garbage afterwards, except the projection
 *     workspaces, whose first 64 KiB hold counters that must start at zero
 *     and are left at zero (decoder-layer section).
 *   - Single sequence (batch 1), as [P] "Implementation Characteristics"
 *     states.
 *   - Arguments are validated on the host before anything is enqueued; a bad
 *     argument returns EAGLE_EINVAL (or EAGLE_EUNSUPPORTED for a valid shape
 *     this build does not implement) and enqueues nothing.
 *   - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *     without synchronising.  A launch failure returns EAGLE_EHIP.
 *   - Errors in device data (a parent that is not an earlier node, a token
 *     outside [0, V), ...) cannot be seen on the host; kernels OR an
 *     EAGLE_DEV_* bit into *dev_status when dev_status is non-null and then
 *     finish with a defined (but meaningless) output.  dev_status is never
 *     cleared by the library.
 *   - Calls keep no global state and are reentrant; calls on different streams
 *     may overlap if their buffers do not.
 *   - Element types: EAGLE_BF16 = bfloat16 (round-to-nearest-even), EAGLE_F32.
 *     Accumulation is always fp32.
 */
#ifndef EAGLE_H_
#define EAGLE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EAGLE_ABI_VERSION 6

typedef enum {
  EAGLE_OK = 0,
  EAGLE_EINVAL = -1,        /* bad argument (null pointer, size, alignment)  */
  EAGLE_EUNSUPPORTED = -2,  /* valid but not implemented (e.g. hd = 96)      */
  EAGLE_EWORKSPACE = -3,    /* workspace smaller than the query's answer     */
  EAGLE_EHIP = -4           /* a HIP launch or runtime call failed           */
} eagle_status;

typedef enum { EAGLE_F32 = 0, EAGLE_BF16 = 1 } eagle_dtype;

enum { EAGLE_EXPAND = 0, EAGLE_RERANK = 1 };
enum { EAGLE_GREEDY = 0, EAGLE_SAMPLE = 1 };

/* Bits OR-ed into *dev_status by kernels. */
enum {
  EAGLE_DEV_BAD_PARENT = 1,     /* parents[i] not -1 and not in [0, i)        */
  EAGLE_DEV_BAD_ROOT = 2,       /* node 0 not the single root (acceptance)    */
  EAGLE_DEV_BAD_TOKEN = 4,      /* token outside [0, V)                       */
  EAGLE_DEV_BAD_INDEX = 8,      /* frontier / mask-row index out of range     */
  EAGLE_DEV_ORPHAN = 16,        /* rerank kept an entry without its parent    */
  EAGLE_DEV_PATH_TRUNC = 32,    /* accepted path longer than max_path         */
  EAGLE_DEV_TIMEOUT = 64        /* a bounded wait for the other workgroups of
                                   one launch expired (eagle_accept_q: the GPU
                                   was shared); outputs are not valid         */
};

/* Limits of this build. */
#define EAGLE_MAX_TREE 256      /* T, Tk: tree nodes per call (words <= 4)    */
#define EAGLE_MAX_TOPK 64       /* k of eagle_lmhead_topk                     */
#define EAGLE_MAX_POOL 8192     /* candidate-pool entries of expand/rerank    */
#define EAGLE_MAX_APPEND 4096   /* kf * k entries appended by one EXPAND      */

int eagle_abi_version(void);
const char* eagle_status_string(int status);   /* static string, never NULL */

/*
 * eagle_build_tree_mask - ancestor-only visibility of a draft tree.
 *
 * [G] Key Architectural Mechanics 3 (Single-Pass Tree Verification): a tree
 * token attends to the tokens on its own branch and never to another branch;
 * a node also sees itself, so a chain gives the causal mask ([G] section 1).
 *
 *   parents  int32[T]       parent of node i, -1 for a root; a valid parent
 *                           precedes its child (parents[i] < i).  Several
 *                           roots (a forest) are allowed here.
 *   T        1..256         nodes.
 *   words    >= ceil(T/64), <= 4: uint64 words per mask row.
 *   mask     uint64[T][words] out: bit (j % 64) of word (j / 64) of row i is
 *                           set iff node j is i or an ancestor of i; bits >= T
 *                           are zero.
 *   depth    int32[T]       out: edges from i to its root.
 *   dev_status int32[1] or NULL: EAGLE_DEV_BAD_PARENT on a bad parent (the
 *                           walk stops there).
 */
int eagle_build_tree_mask(const int32_t* parents, int32_t T, int32_t words,
                          uint64_t* mask, int32_t* depth, int32_t* dev_status,
                          hipStream_t stream);

/*
 * eagle_tree_attn - tree-masked attention of tree nodes against a KV prefix.
 *
 * [G] Key Architectural Mechanics 3: the target scores every tree node in one
 * batched pass under the tree mask.  [D] LlamaAttention printout: grouped-
 * query attention (q 4096 -> 32 heads, k/v 4096 -> 8 heads of 128).
 *
 * For query row i and head h (KV head g = h / (Hq / Hkv)):
 *   visible = prefix positions 0..L-1, plus tree nodes j < Tk whose bit is set
 *             in mask row m(i) (m(i) = q_mask_row[i], or i when NULL);
 *   out[i][h] = sum_j softmax_j(scale * q[i][h] . k_j) v_j over visible j.
 *
 *   q        [Tq][Hq][hd] in_dt (RoPE already applied).
 *   k_cache, v_cache [Hkv][ld_cache][hd] in_dt, rows 0..L-1 used; L >= 0.
 *   k_tree, v_tree   [Hkv][ld_tree][hd] in_dt, rows 0..Tk-1 used.
 *   mask     uint64[mask_rows][words] (eagle_build_tree_mask layout).
 *   q_mask_row int32[Tq] or NULL; entries outside [0, mask_rows) set
 *            EAGLE_DEV_BAD_INDEX and the row sees the prefix only.
 *   Tq 1..256, Tk 1..256, Hq % Hkv == 0, hd in {64, 128}; every row must see
 *   at least one position (L > 0, or its own node in the tree).
 *   scale    score scale (1/sqrt(hd) for standard attention).
 *   in_dt    EAGLE_BF16 or EAGLE_F32; out_dt EAGLE_BF16 or EAGLE_F32.
 *   out      [Tq][Hq][hd] out_dt.
 *   workspace >= eagle_tree_attn_workspace(...) bytes, 256-byte aligned.
 *   Rows of K/V, q and out must be 16-byte aligned (hd contiguous).
 */
size_t eagle_tree_attn_workspace(int32_t Tq, int32_t Hq, int32_t Hkv, int32_t hd,
                                 int64_t L, int32_t Tk, eagle_dtype in_dt);
int eagle_tree_attn(const void* q,
                    const void* k_cache, const void* v_cache, int64_t L, int64_t ld_cache,
                    const void* k_tree, const void* v_tree, int32_t Tk, int32_t ld_tree,
                    const uint64_t* mask, int32_t words, int32_t mask_rows,
                    const int32_t* q_mask_row, int32_t Tq,
                    int32_t Hq, int32_t Hkv, int32_t hd, float scale,
                    eagle_dtype in_dt, eagle_dtype out_dt, void* out,
                    void* workspace, size_t ws_bytes, int32_t* dev_status,
                    hipStream_t stream);

/*
 * eagle_lmhead_topk - LM head, softmax statistics and top-k.
 *
 * [G] Key Architectural Mechanics 1: P = softmax(W_LM f) with the target's own
 * LM head; section 2: the confidence C = P(y_(1))/P(y_(2)) of the two most
 * likely tokens, which equals exp(topk_logp[t][0] - topk_logp[t][1]).
 * [D] printout: no bias.
 *
 *   f        [T][d] dt, row t is one feature: final norm already applied, or
 *            deferred (in_ssq [in_parts][T] f32 or NULL, in_eps; see the
 *            decoder-layer section).
 *   W        [V][d] dt, one row per vocabulary entry.
 *   T 1..256, d % 128 == 0 (bf16) or any d >= 1 (f32), 0 <= k <= min(V, 64);
 *            k = 0 computes lse (and logits) only, e.g. for sampling
 *            acceptance, which reads the logits.
 *   topk_id  int32[T][k] out: the k largest logits of row t, larger first,
 *            the lower vocabulary index first among equal logits (NULL when
 *            k = 0).
 *   topk_logp f32[T][k] out: logit - lse (temperature 1) (NULL when k = 0).
 *   lse      f32[T] out: log sum_v exp(logit[t][v]).
 *   logits   f32[T][V] out, or NULL: the fp32 logits.
 *   workspace >= eagle_lmhead_topk_workspace(...) bytes, 256-byte aligned.
 *            bf16: the first 2 KiB hold one 64-bit key bound per feature
 *            row, raised by the partial lists as they finish so that later
 *            lists skip keys below it.  They must be zero before the first
 *            call that uses the buffer (allocate it zeroed); every call leaves
 *            them zero, so the buffer can be reused by later calls on the same
 *            stream, also under graph capture.  The results do not depend on
 *            the order in which the lists finish.
 */
size_t eagle_lmhead_topk_workspace(int32_t T, int32_t d, int32_t V, int32_t k, eagle_dtype dt);
int eagle_lmhead_topk(const void* f, const void* W, int32_t T, int32_t d, int32_t V,
                      int32_t k, eagle_dtype dt, const float* in_ssq, int32_t in_parts,
                      float in_eps, int32_t* topk_id, float* topk_logp, float* lse,
                      float* logits, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * eagle_lmhead_topk_noalloc - eagle_lmhead_topk without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments, outputs, kernels and results as eagle_lmhead_topk, minus
 * workspace/ws_bytes.  The partial lists (or the fp32 logits of the f32 path
 * when logits is NULL) live in a scratch array the library holds on every
 * GPU it runs on, EAGLE_LMHEAD_SCRATCH_BYTES bytes, kept until the process
 * ends; its address is looked up once per device on the first call made
 * with that device current.  The call itself allocates nothing.
 *   Limit: eagle_lmhead_topk_workspace(T, d, V, k, dt) must not exceed
 *   EAGLE_LMHEAD_SCRATCH_BYTES (else EAGLE_EWORKSPACE, before any HIP call);
 *   e.g. T = 128, V = 128256, k = 10 in bf16 needs 11.3 MB.
 *   stream must belong to the current device (else EAGLE_EINVAL).
 * Every call on one GPU shares that GPU's scratch.  It starts zeroed (static
 * device memory), and every call leaves its key bounds (see the workspace of
 * eagle_lmhead_topk) zero again.  Calls that overlap in time on one GPU (two
 * streams, or two host threads) race on it: serialise them.
 */
#define EAGLE_LMHEAD_SCRATCH_BYTES ((size_t)16 << 20)
int eagle_lmhead_topk_noalloc(const void* f, const void* W, int32_t T, int32_t d, int32_t V,
                              int32_t k, eagle_dtype dt, const float* in_ssq, int32_t in_parts,
                              float in_eps, int32_t* topk_id, float* topk_logp, float* lse,
                              float* logits, hipStream_t stream);

/*
 * eagle_expand_rerank - grow the dynamic draft tree and prune it.
 *
 * [D] (reply on static vs dynamic trees): the draft's confidence approximates
 * acceptance; the tree is grown from it and pruned at the end of drafting.
 * [G] section 2: the token budget goes where confidence is high.  Reading:
 * confidence = cumulative log-probability, value[child] =
 * fp32(value[parent] + logp), root value 0; ties go to the lower pool index.
 *
 * The candidate pool is four parallel device arrays (token, parent, depth,
 * value) of capacity pool_cap; entry 0 is the root.  pool_n (host) is the
 * number of valid entries before this call.
 *
 * EXPAND: for frontier slot s < kf and child rank j < k (s-major) append
 *   entry pool_n + s*k + j = {child_id[s][j], frontier[s],
 *   depth[frontier[s]] + 1, fp32(value[frontier[s]] + child_logp[s][j])};
 *   new_frontier[0..k_select) = the k_select best appended entries by
 *   (value desc, index asc), in ascending pool index.
 *   Needs pool_n + kf*k <= pool_cap, kf*k <= 4096, 1 <= k_select <= kf*k.
 * RERANK: keep the root and the T-1 best non-root entries by (value desc,
 *   index asc; +0.0 equals -0.0, a NaN value ranks last); write them in
 *   ascending pool index as node_token, node_parent (index into this list,
 *   -1 for the root), node_depth and node_pool_idx.  Needs
 *   1 <= T <= min(pool_n, 256), pool_n <= 8192.
 * Unused pointers of the other mode may be NULL.
 */
int eagle_expand_rerank(int32_t mode,
                        int32_t* pool_token, int32_t* pool_parent, int32_t* pool_depth,
                        float* pool_value, int32_t pool_n, int32_t pool_cap,
                        const int32_t* frontier, int32_t kf,
                        const int32_t* child_id, const float* child_logp, int32_t k,
                        int32_t k_select, int32_t* new_frontier,
                        int32_t T, int32_t* node_token, int32_t* node_parent,
                        int32_t* node_depth, int32_t* node_pool_idx,
                        int32_t* dev_status, hipStream_t stream);

/*
 * eagle_gate_children - confidence-gated branching of drafted nodes.
 *
 * [G] Key Architectural Mechanics 2: a drafted node's confidence is
 * C = P(y_(1)) / P(y_(2)); above a threshold tau the draft deepens a linear
 * chain, at or below it the node branches into 2 to 4 children (tau = 2.0 in
 * [G]'s Reference Implementation).  Reading: child j (logp sorted
 * descending) is kept while fewer than max_branch are kept and
 * logp_j - logp_0 >= -ln(tau), i.e. P_j >= P_(1) / tau: one child exactly when
 * C > tau.  Children not kept get log-probability -inf, so EXPAND gives them
 * value -inf and they rank below every kept candidate.
 *
 * logp f32[rows][k] device (eagle_lmhead_topk's topk_logp) -> out_logp
 * f32[rows][k] (may be logp itself); kept int32[rows] (nullable): children
 * kept; confidence f32[rows] (nullable): exp(logp_0 - logp_1), +inf for
 * k = 1.  The compare is one fp32 subtraction with ln(tau) computed in fp64
 * and rounded once to fp32.
 * Errors: rows < 1, k outside [1, EAGLE_MAX_TOPK], max_branch < 1, tau < 1
 * or not finite, null logp/out_logp -> EAGLE_EINVAL.
 */
int eagle_gate_children(const float* logp, int32_t rows, int32_t k, float tau,
                        int32_t max_branch, float* out_logp, int32_t* kept,
                        float* confidence, hipStream_t stream);

/*
 * eagle_logits_process - mixed-sampling processing (temperature, top-k,
 * top-p) of the target's logits before eagle_accept(SAMPLE).
 *
 * [P] test setup: the speedups are measured under mixed sampling
 * (temperature, top_k, top_p); [G] Key Architectural Mechanics 3: a greedy or
 * nucleus-sampling verifier walks the tree.  Reading: top-k keeps the
 * k = min(top_k, V) tokens ranked first by (logit descending, index
 * ascending), top_k = 0 keeps all V; top-p (top_p < 1) then keeps, in that
 * order, the shortest prefix whose mass under exp((l - l_max) / temperature)
 * (fp64, summed in rank order) reaches top_p times the mass of the k; a
 * token stays while the mass before it is below that.  Removed tokens become
 * -inf, so eagle_accept(SAMPLE) with the same temperature samples the
 * renormalised processed distribution.
 *
 * logits f32[T][V] device -> out f32[T][V] (may be logits itself); kept
 * int32[T] device or NULL: tokens kept per row.  Logits must be finite.
 * workspace >= eagle_logits_process_workspace(T, V, top_k) bytes, 256-byte
 * aligned, all zero before its first use (it starts with per-row arrival
 * counters, which every call leaves zero again; calls that share one
 * workspace must not overlap).  The query returns 0, and workspace may be
 * NULL, when the k kept by top-k are too many for the chunked path: then one
 * workgroup per row streams the row once per radix pass.
 * Errors: null pointers, T or V < 1, top_k < 0, temperature not in
 * (0, inf), top_p not in (0, 1] -> EAGLE_EINVAL; top_p < 1 with more than
 * 1024 tokens left by top-k -> EAGLE_EUNSUPPORTED; small or null workspace
 * when one is needed -> EAGLE_EWORKSPACE.
 */
size_t eagle_logits_process_workspace(int32_t T, int32_t V, int32_t top_k);
int eagle_logits_process(const float* logits, int32_t T, int32_t V, float temperature,
                         int32_t top_k, float top_p, float* out, int32_t* kept,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * eagle_accept - accept the longest verified path through the tree.
 *
 * [G] Key Architectural Mechanics 3: a greedy or sampling verifier walks the
 * tree from the root and accepts matching tokens until the first discrepancy;
 * the output equals plain decoding.  [G] The Problem 1 and [D] opening post:
 * speculative sampling's accept/reject rule (Leviathan et al., Chen et al.).
 *
 * Tree: node_token/node_parent int32[T], node 0 the single root, parents
 * before children.
 * GREEDY (target_top1: the target's argmax at each node, node i's at element
 *   i * top1_stride; top1_stride = 1 for an int32[T] array, or k to read
 *   column 0 of eagle_lmhead_topk's topk_id[T][k] in place): node c matches
 *   when node_token[c] == top1(parent(c)); the path ends at the deepest node
 *   whose whole root path matches (lowest index among equally deep ones);
 *   bonus = top1(end).  top1_stride < 1 -> EAGLE_EINVAL.
 * SAMPLE (target_logits f32[T][V], temperature > 0, uniforms f32[2T] in
 *   [0,1)): at node u, p = exp((l_u - max l_u) / temperature) in fp64 and
 *   Z_res = sum p minus the mass of tokens already rejected at u; children
 *   in ascending index: a child whose token was rejected is rejected,
 *   otherwise child c with token x is accepted iff uniforms[c] * Z_res < p[x]
 *   (the walk moves to c), else x is rejected.  When all children are
 *   rejected or u is a leaf, bonus = the smallest token i whose running sum of
 *   non-rejected p exceeds uniforms[T + u] * Z_res.  The division by the
 *   temperature is a product with its fp64 reciprocal (exact at 1) and sums
 *   run in chunks of 4096 tokens, so results can differ from a sequential
 *   fp64 evaluation only where a decision's margin is a few ulp of Z.
 *   workspace >= eagle_accept_workspace(T, V) bytes (SAMPLE only).
 * Outputs: path int32[max_path] = node ids from the root (path[0] = 0), the
 *   rest -1; n_accepted int32[1] = accepted draft nodes (path length - 1);
 *   bonus_token int32[1].  A path longer than max_path is cut and sets
 *   EAGLE_DEV_PATH_TRUNC.
 */
size_t eagle_accept_workspace(int32_t T, int32_t V);
int eagle_accept(int32_t mode, int32_t T, const int32_t* node_token,
                 const int32_t* node_parent, const int32_t* target_top1,
                 int32_t top1_stride, const float* target_logits, int32_t V, float temperature,
                 const float* uniforms, int32_t max_path, int32_t* path,
                 int32_t* n_accepted, int32_t* bonus_token,
                 void* workspace, size_t ws_bytes, int32_t* dev_status,
                 hipStream_t stream);

/*
 * eagle_kv_commit - append the accepted path's K/V rows to the caches.
 *
 * [D] reply on how large the draft's context grows: the target keeps KV
 * entries only for accepted tokens, the draft keeps them for every candidate
 * and needs eviction.  [G] Key Architectural Mechanics 3: the accepted tokens
 * are the longest verified root path.  After acceptance, source rows
 * rows[0], rows[1], ... (eagle_accept's path: node ids, root first; or the
 * draft's slot ids of the same nodes) become cache positions L, L + 1, ...
 * of every layer and KV head; every other candidate's rows are dropped.
 *
 * src_k, src_v:  [layers][Hkv][ld_src][hd] (layer stride src_layer_stride
 *                elements); valid source rows are [0, src_rows).
 * rows:          int32[max_rows] device.
 * n_accepted:    int32[1] device or NULL.  Rows copied: n_accepted[0] + 1
 *                (the root and the accepted nodes), or max_rows if NULL.  A
 *                count above max_rows is cut to max_rows and sets
 *                EAGLE_DEV_PATH_TRUNC; a negative n_accepted sets
 *                EAGLE_DEV_BAD_INDEX and copies nothing.
 * cache_k, cache_v: [layers][Hkv][ld_cache][hd] (layer stride
 *                cache_layer_stride elements); rows L .. L + n - 1 are
 *                written, nothing else.
 * Every source row of a (layer, head) is read before any of its cache rows is
 * written, so the source may lie inside the cache (tree rows stored right
 * after the prefix: src_k = cache_k + L hd, ld_src = ld_cache); K and V, and
 * distinct layers and heads, must not overlap.
 * Host errors: L < 0, L + max_rows > ld_cache, max_rows outside
 * [1, EAGLE_MAX_TREE], src_rows outside [1, ld_src], layers < 1, a layer
 * stride below one layer's size when layers > 1, misaligned (16-byte)
 * pointers -> EAGLE_EINVAL; hd not 64 or 128, or max_rows * hd * element size
 * above 64 KiB -> EAGLE_EUNSUPPORTED.  Device errors: a source row outside
 * [0, src_rows) sets EAGLE_DEV_BAD_INDEX and its cache row is left unchanged.
 */
int eagle_kv_commit(const void* src_k, const void* src_v, int32_t ld_src, int32_t src_rows,
                    int64_t src_layer_stride, const int32_t* rows, const int32_t* n_accepted,
                    int32_t max_rows, void* cache_k, void* cache_v, int64_t L,
                    int64_t ld_cache, int64_t cache_layer_stride, int32_t layers,
                    int32_t Hkv, int32_t hd, eagle_dtype dt, int32_t* dev_status,
                    hipStream_t stream);

/*
 * eagle_path_slots - the draft's rows of the accepted path, for the draft's
 * KV eviction.
 *
 * [D] reply on the draft's context: the draft keeps K/V for every candidate
 * it ran, so after acceptance the rows of the accepted tokens are kept and
 * the rest dropped.  The draft ran a node (and wrote its K/V at a slot) only
 * if it expanded it; on the accepted path that is every node but possibly the
 * last, which may be a leaf.
 *   path, n_accepted: eagle_accept's outputs (node ids, root first; count
 *                 n_accepted[0] + 1, cut to max_path).
 *   node_pool_idx int32[T]: eagle_expand_rerank's pool entry of each node.
 *   slot_of_pool  int32[pool_cap]: the draft slot of each pool entry, or -1
 *                 for an entry never expanded.
 *   slot_rows     int32[max_path] out: slot_of_pool[node_pool_idx[path[j]]]
 *                 for j < n, then -1; n = the leading path nodes that have a
 *                 slot in [0, n_slots).
 *   n_rows_minus_one int32[1] out: n - 1, the count convention of
 *                 eagle_kv_commit's n_accepted, so the two calls chain.
 * Device errors: a path node outside [0, T) or a pool index outside
 * [0, pool_cap) sets EAGLE_DEV_BAD_INDEX and ends the rows there; a root with
 * no slot (n = 0) sets it too.  Host errors: null pointers, max_path or T
 * outside [1, EAGLE_MAX_TREE], pool_cap or n_slots < 1 -> EAGLE_EINVAL.
 */
int eagle_path_slots(const int32_t* path, const int32_t* n_accepted, int32_t max_path,
                     const int32_t* node_pool_idx, int32_t T, const int32_t* slot_of_pool,
                     int32_t pool_cap, int32_t n_slots, int32_t* slot_rows,
                     int32_t* n_rows_minus_one, int32_t* dev_status, hipStream_t stream);

/*
 * eagle_kv_commit_pair - both commits of a cycle in one launch, for one layer
 * each: eagle_kv_commit of the target's tree rows (rows = path, n_accepted)
 * and eagle_kv_commit of the draft's rows of the same nodes, with those rows
 * found as eagle_path_slots finds them (path[0 .. max_path), node_pool_idx
 * [T], slot_of_pool [pool_cap], the draft's n_slots = d_src_rows).  Both
 * caches take the rows at position L and share Hkv, hd and dt; sources and
 * caches are [Hkv][ld][hd] (ld = *_ld_src, *_ld_cache rows).  max_path <=
 * max_rows <= 256.  Status codes as for the two calls it replaces.
 */
int eagle_kv_commit_pair(const void* t_src_k, const void* t_src_v, int32_t t_ld_src,
                         int32_t t_src_rows, void* t_cache_k, void* t_cache_v,
                         int64_t t_ld_cache, const void* d_src_k, const void* d_src_v,
                         int32_t d_ld_src, int32_t d_src_rows, void* d_cache_k, void* d_cache_v,
                         int64_t d_ld_cache, int64_t L, const int32_t* path,
                         const int32_t* n_accepted, int32_t max_rows,
                         const int32_t* node_pool_idx, int32_t T, const int32_t* slot_of_pool,
                         int32_t pool_cap, int32_t max_path, int32_t Hkv, int32_t hd,
                         eagle_dtype dt, int32_t* dev_status, hipStream_t stream);

/*
 * eagle_accept_q - speculative sampling over the tree with the draft's own
 * distribution instead of a point mass.
 *
 * [G] The Problem 1 (accept or reject draft tokens against the target's
 * distribution) and Key Architectural Mechanics 3 (the verifier walks the
 * tree).  Reading for a sampled draft: the children of node u are draws from
 * q_u = softmax(draft_logits[u] / temperature) without replacement and are
 * verified by recursive rejection sampling.  With p_1 = p_u (target, same
 * temperature) and q_1 = q_u: child i (ascending index) with token x is
 * accepted iff uniforms[c] * q_i(x) < p_i(x) (probability min(1, p_i / q_i))
 * and the walk moves to it; on rejection p_(i+1) = max(p_i - q_i, 0)
 * renormalised and q_(i+1) = q_i without x, renormalised (q counts as 0 once
 * no draft mass is left).  A child whose token was already rejected at u is
 * skipped.  When all children are rejected, or u is a leaf, the bonus is the
 * smallest token whose running sum of the last residual exceeds
 * uniforms[T + u] times its total.  fp64 from fp32 logits; sums in a fixed
 * order (results can differ from a sequential fp64 evaluation only where a
 * decision's margin is a few ulp).  One launch of up to 256 workgroups (one
 * per CU, each owning a slice of the vocabulary) walks the tree together:
 * every workgroup takes every decision itself, and they meet at a grid
 * barrier only for the sums over the vocabulary (a visited node's row
 * statistics, each rejection's residual mass, the bonus draw); a barrier is
 * an all-gather of tagged records in the workspace, which every workgroup
 * combines itself in the same fixed order.  The whole
 * grid must be resident at once: the call assumes the GPU is not shared with
 * other work holding CUs; a barrier that never fills sets EAGLE_DEV_TIMEOUT
 * after about a second instead of hanging (the outputs are then not valid).
 *
 * target_logits, draft_logits f32[T][V]; uniforms f32[2T] in [0, 1);
 * workspace >= eagle_accept_q_workspace(T, V) bytes, 256-byte aligned, zero
 * before its first use (it holds a generation number that every call
 * advances and the tagged barrier records; keep the buffer for later calls
 * on the same stream, or zero it again before handing it over).
 * Outputs and device errors as eagle_accept.  Host errors: null pointers, T
 * outside [1, EAGLE_MAX_TREE], V or max_path < 1, temperature not in
 * (0, 3e38], a misaligned workspace -> EAGLE_EINVAL; V above 524288 ->
 * EAGLE_EUNSUPPORTED; small workspace -> EAGLE_EWORKSPACE.
 */
size_t eagle_accept_q_workspace(int32_t T, int32_t V);
int eagle_accept_q(int32_t T, const int32_t* node_token, const int32_t* node_parent,
                   const float* target_logits, const float* draft_logits, int32_t V,
                   float temperature, const float* uniforms, int32_t max_path, int32_t* path,
                   int32_t* n_accepted, int32_t* bonus_token, void* workspace, size_t ws_bytes,
                   int32_t* dev_status, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decoder-layer support for the draft rounds and the verify pass.
 *
 * [G] Key Architectural Mechanics 1: each draft step fuses the previous
 * feature with the current token's embedding, h = W_fuse [f ; Emb(y)], runs one
 * transformer decoder layer, f' = TransformerLayer(h), and scores f' with the
 * target's LM head.  [D] yuhuili/EAGLE3-LLaMA3.1-Instruct-8B printout: the
 * layer is a Llama decoder layer (RMSNorm eps 1e-5, q/k/v/o projections,
 * SiLU-gated MLP, rotary embedding, no biases) and the draft shares the
 * target's embedding table.  Weights are [out][in] bf16 (nn.Linear layout).
 *
 * Projection workspaces (eagle_linear*, sizes from eagle_linear_workspace and
 * eagle_linear_rows_workspace): when the product is split over k to occupy the
 * whole GPU, fp32 partial tiles are kept there and summed in a fixed order.
 * With M <= 16 the sum and the epilogue run inside the one projection kernel:
 * the last workgroup to finish a column block (counted in the first 64 KiB of
 * the workspace) does them.  Those 64 KiB must be zero before the first call
 * that uses the buffer (allocate it zeroed); every call leaves them zero, so a
 * buffer can be reused by later calls on the same stream, also under graph
 * capture.  Calls that run concurrently must not share a workspace.
 *
 * Deferred RMSNorm.  Every norm of the layer feeds a product, and the row
 * scale 1 / sqrt(mean(y[m]^2) + eps) factors out of it:
 *   RMSNorm(y)[m] W^T = (y[m] * gamma) W^T / sqrt(mean(y[m]^2) + eps).
 * eagle_linear_rmsnorm_deferred therefore hands over xg = y * gamma (bf16,
 * elementwise, needs no whole row) and partial sums of squares ssq[p][m]
 * (p < eagle_linear_norm_parts(M, K, N), each over a disjoint set of columns);
 * the consumers (eagle_linear_swiglu, eagle_linear_rope_qkv,
 * eagle_lmhead_topk) take the optional triple (in_ssq, in_parts, in_eps),
 * add the partials in p order, and scale their fp32 results of row m by
 * 1 / sqrt(sum_p in_ssq[p][m] / K + in_eps) before their own epilogue.  With
 * in_ssq NULL the input is used as given.  The only difference from applying
 * the norm first is where the bf16 rounding of the input falls (relative error
 * 2^-9 either way).
 * ------------------------------------------------------------------------ */

/*
 * eagle_linear - out[m][n] = sum_k x[m][k] W[n][k] (+ residual[m][n]).
 *   x [M][K] bf16 (M 1..256, K % 128 == 0), W [N][K] bf16, residual [M][N] f32
 *   or NULL (may alias out when out_dt is f32), out [M][N] out_dt.
 *   workspace >= eagle_linear_workspace(M, K, N, 0) bytes (16-byte aligned,
 *   zeroed before first use; may be NULL when that size is 0).
 */
size_t eagle_linear_workspace(int32_t M, int32_t K, int32_t N, int32_t swiglu);
int eagle_linear(const void* x, int32_t M, int32_t K, const void* W, int32_t N,
                 const float* residual, void* out, eagle_dtype out_dt, void* workspace,
                 size_t ws_bytes, hipStream_t stream);

/*
 * eagle_fuse3 - Eagle-3 feature fusion: out[m][n] = sum_k x[m][k] W[n][k] with
 * x[m] = [h_low[m] ; h_mid[m] ; h_high[m]] (K = 3 d), read from the three
 * buffers directly.
 *
 * [D] opening post: the target's hidden states after its first, middle and
 * last decoder layers are recorded; [D] replies: a single FC layer maps the
 * three to one feature g, which feeds the draft's decoder layer.  Reading: the
 * segments are concatenated in the order low, middle, high.
 *   h_low, h_mid, h_high [M][d] bf16 (M 1..16, d % 128 == 0), W [N][3 d] bf16,
 *   out [M][N] out_dt; workspace >= eagle_linear_workspace(M, 3 d, N, 0)
 *   bytes, with the zeroing rule of the projection workspaces.
 *   Errors: null or misaligned (16-byte) pointers, M, d or N < 1 ->
 *   EAGLE_EINVAL; M > 16 or d % 128 != 0 -> EAGLE_EUNSUPPORTED; small
 *   workspace -> EAGLE_EWORKSPACE.
 */
int eagle_fuse3(const void* h_low, const void* h_mid, const void* h_high, int32_t M,
                int32_t d, const void* W, int32_t N, void* out, eagle_dtype out_dt,
                void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * eagle_linear_swiglu - out[m][n] = silu(x W_gate^T)[m][n] * (x W_up^T)[m][n],
 * the LlamaMLP hidden activation.  x [M][K] bf16 (with an optional deferred
 * RMSNorm: in_ssq [in_parts][M] or NULL, in_eps), W_gate/W_up [N][K] bf16,
 * out [M][N] bf16, workspace >= eagle_linear_workspace(M, K, N, 1) bytes.
 */
int eagle_linear_swiglu(const void* x, int32_t M, int32_t K, const float* in_ssq,
                        int32_t in_parts, float in_eps, const void* w_gate, const void* w_up,
                        int32_t N, void* out, void* workspace, size_t ws_bytes,
                        hipStream_t stream);

/*
 * eagle_linear_rmsnorm - a projection whose result feeds an RMSNorm, in two
 * launches: out[m] = x[m] W^T + residual[m] (f32, residual may be NULL or
 * alias out) and norm_out[m] = out[m] / sqrt(mean(out[m]^2) + eps) * gamma
 * (bf16).  N % 4 == 0, N <= 8192.
 *   workspace >= eagle_linear_rows_workspace(M, K, N) bytes.
 */
size_t eagle_linear_rows_workspace(int32_t M, int32_t K, int32_t N);
int eagle_linear_rmsnorm(const void* x, int32_t M, int32_t K, const void* W, int32_t N,
                         const float* residual, float* out, const float* gamma, float eps,
                         void* norm_out, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * eagle_linear_rmsnorm_deferred - the same product and residual add, with the
 * norm deferred to the consumer (one launch for M <= 16, two otherwise):
 * out[m] = x[m] W^T + residual[m] (f32), xg_out[m] = out[m] * gamma (bf16,
 * [M][N]) and ssq_out [P][M] f32, P = eagle_linear_norm_parts(M, K, N):
 * sums of out[m][n]^2 over disjoint column sets (64 columns each for
 * M <= 16, 1024 otherwise).  Used for the layer's
 * residual adds, each of which is followed by a norm that feeds a product.
 * N % 4 == 0, N <= 8192; workspace >= eagle_linear_rows_workspace(M, K, N).
 */
int32_t eagle_linear_norm_parts(int32_t M, int32_t K, int32_t N);
int eagle_linear_rmsnorm_deferred(const void* x, int32_t M, int32_t K, const void* W, int32_t N,
                                  const float* residual, float* out, const float* gamma,
                                  void* xg_out, float* ssq_out, void* workspace,
                                  size_t ws_bytes, hipStream_t stream);

/*
 * eagle_linear_rope_qkv - the q/k/v projection followed by eagle_rope_qkv's
 * rotation and placement (one launch for M <= 16 and hd % 64 == 0, two
 * otherwise): x [M][K] bf16 (optional deferred RMSNorm: in_ssq, in_parts,
 * in_eps), w_qkv
 * [(Hq + 2 Hkv) hd][K] bf16 (q rows, then k, then v); outputs and the other
 * arguments as eagle_rope_qkv.  (Hq + 2 Hkv) hd <= 16384, hd % 8 == 0.
 *   workspace >= eagle_linear_rows_workspace(M, K, (Hq + 2 Hkv) hd) bytes.
 */
int eagle_linear_rope_qkv(const void* x, int32_t M, int32_t K, const float* in_ssq,
                          int32_t in_parts, float in_eps, const void* w_qkv, int32_t Hq,
                          int32_t Hkv, int32_t hd, const int32_t* depth, int64_t pos_base,
                          float theta, const int32_t* row_slot, int32_t slot_cap, void* q_out,
                          void* k_tree, void* v_tree, int32_t ld_tree, void* workspace,
                          size_t ws_bytes, int32_t* dev_status, hipStream_t stream);

/*
 * eagle_rmsnorm - out[m] = x[m] / sqrt(mean(x[m]^2) + eps) * gamma.
 *   x [M][N] f32, gamma [N] f32, out [M][N] bf16.
 */
int eagle_rmsnorm(const float* x, const float* gamma, int32_t M, int32_t N, float eps,
                  void* out, hipStream_t stream);

/*
 * eagle_rope_qkv - rotary embedding of q and k, and placement of k/v in the
 * tree K/V buffers.  qkv [M][(Hq + 2 Hkv) hd] f32 (q heads, then k, then v);
 * row m sits at position pos_base + depth[m] (reading: a tree node's position
 * is the prefix length plus its depth); dims i and i + hd/2 turn by
 * position * theta^(-2i/hd).  q_out [M][Hq][hd] bf16; k (rotated) and v go to
 * k_tree/v_tree [Hkv][ld_tree][hd] bf16 at row row_slot[m] (m when NULL);
 * a slot outside [0, slot_cap) sets EAGLE_DEV_BAD_INDEX and is skipped.
 */
int eagle_rope_qkv(const float* qkv, int32_t M, int32_t Hq, int32_t Hkv, int32_t hd,
                   const int32_t* depth, int64_t pos_base, float theta, const int32_t* row_slot,
                   int32_t slot_cap, void* q_out, void* k_tree, void* v_tree, int32_t ld_tree,
                   int32_t* dev_status, hipStream_t stream);

/*
 * eagle_draft_prepare - everything one draft round needs before its layer,
 * for the rows frontier[0..kf) (pool entries; see eagle_expand_rerank):
 *   - row j gets draft slot slot_base + j, which holds its K/V, its output
 *     feature and its mask row; slot_of_pool[frontier[j]] is set to it and
 *     slot_parent[slot] to the slot of the entry's parent (-1 for the root);
 *   - row_token, row_depth (pool depth), row_slot and row_src (the parent's
 *     slot, whose output feature predicted this row's token and is paired with
 *     it: [G] Reference Implementation, the feature and the token it produced
 *     step together);
 *   - slot_mask [slot_cap][words] (or NULL): the slot's ancestor mask row, its
 *     parent slot's row plus its own bit (eagle_build_tree_mask layout);
 *   - x_in [kf][2d] bf16 (or NULL): the fused input [f ; Emb(y)] =
 *     [bf16(feat[row_src]) (root_feat for the root) ; embed[row_token]],
 *     feat [slot_cap][d] f32, root_feat [d] f32, embed [V][d] bf16.
 * slot_of_pool [pool capacity] must hold the slots of earlier rounds.  A
 * frontier entry or parent slot out of range sets EAGLE_DEV_BAD_INDEX, a token
 * outside [0, V) EAGLE_DEV_BAD_TOKEN.
 */
int eagle_draft_prepare(const int32_t* frontier, int32_t kf, const int32_t* pool_token,
                        const int32_t* pool_parent, const int32_t* pool_depth, int32_t pool_n,
                        int32_t* slot_of_pool, int32_t slot_base, int32_t slot_cap,
                        int32_t* slot_parent, uint64_t* slot_mask, int32_t words,
                        int32_t* row_token, int32_t* row_depth, int32_t* row_slot,
                        int32_t* row_src, const float* feat, const float* root_feat,
                        const void* embed, int32_t V, int32_t d, void* x_in,
                        int32_t* dev_status, hipStream_t stream);

/* eagle_embed - out[m] = embed[token[m]] as f32 ([M][d]); embed [V][d] bf16. */
int eagle_embed(int32_t M, const int32_t* token, const void* embed, int32_t V, int32_t d,
                float* out, int32_t* dev_status, hipStream_t stream);

/*
 * eagle_embed_deferred - eagle_embed with the RMSNorm that follows it
 * deferred to the next product (see "Deferred RMSNorm" above): out[m] =
 * embed[token[m]] as f32 ([M][d]), xg_out[m] = bf16(out[m] * gamma) ([M][d])
 * and ssq_out[m] = sum_n out[m][n]^2 ([1][M] f32: one part).  d % 8 == 0;
 * embed, gamma, out and xg_out 16-byte aligned.  A token outside [0, V) sets
 * EAGLE_DEV_BAD_TOKEN and reads row 0.
 */
int eagle_embed_deferred(int32_t M, const int32_t* token, const void* embed, int32_t V,
                         int32_t d, const float* gamma, float* out, void* xg_out, float* ssq_out,
                         int32_t* dev_status, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* EAGLE_H_ */
