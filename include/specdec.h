/*
 * specdec.h -- C ABI of the speculative-decoding verification step on MI355X (gfx950).
 *
 * The verification step scores the gamma+1 positions of every sequence in one
 * pass over the LM-head weights, then runs the modified rejection sampling
 * rule on the target and draft distributions.  Sources, cited by title and
 * section (four web articles):
 *   [LLMI] "LLM Inference & Speculative Decoding: From Roofline Physics to
 *          Lossless Acceleration" (arman1o1.github.io)
 *   [MATH] "Speculative Decoding: Mathematical Foundations, Distribution
 *          Preservation Proofs, Tree-Structured Verification, and
 *          Memory-Bandwidth Amortization" (llms.blog)
 *   [LESS] "Speculative decoding." lesson (gtadkapally.com, learn-cs)
 *   [PREP] "Speculative Decoding: Draft, Verify, Accept" (vanos001.github.io)
 *
 * Conventions for every entry point
 *   - Pointers named as device buffers are device memory owned by the caller;
 *     the library never allocates, frees, or synchronises.  Work is enqueued
 *     on `stream` (a hipStream_t; NULL is the null stream) and the call
 *     returns at once.  Kernel faults surface at the caller's next stream
 *     synchronisation.
 *   - Sizes are element counts.  Arrays are dense and row-major.
 *   - Invalid arguments are reported by the return value (a specdec_status)
 *     before anything is launched: null required pointer, bad size, pointer
 *     not 16-byte aligned where 128-bit accesses need it, temperature < 0 or
 *     NaN, workspace too small.  Token ids in device buffers cannot be
 *     checked from the host: ids outside [0, V) are clamped into range by the
 *     kernels, never used to index out of bounds.
 *   - The library keeps no state between calls and may be called from several
 *     host threads; calls on different streams must use different outputs and
 *     workspaces.
 *   - Numeric degenerate cases are defined behaviour, not errors: q(x) is
 *     floored at 1e-12 before dividing ([LLMI] section 2 listing); a residual
 *     with no mass falls back to p ([PREP] demo); T == 0 selects the greedy
 *     rule ([LLMI] section 4, failure mode 1).
 */
#ifndef SPECDEC_H
#define SPECDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPECDEC_OK = 0,
  SPECDEC_ERR_NULL = 1,        /* a required pointer is NULL                        */
  SPECDEC_ERR_SHAPE = 2,       /* a size is out of range                            */
  SPECDEC_ERR_ALIGN = 3,       /* a pointer or row pitch is not 16-byte aligned     */
  SPECDEC_ERR_TEMPERATURE = 4, /* temperature < 0 or NaN                            */
  SPECDEC_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required           */
  SPECDEC_ERR_LAUNCH = 6,      /* the HIP runtime refused a launch                  */
  SPECDEC_ERR_ARG = 7,         /* an enumerated argument has an unknown value       */
  SPECDEC_ERR_SCRATCH = 8,     /* the shape's workspace exceeds the static buffer   */
  SPECDEC_ERR_DEVICE = 9       /* the runtime gave no current device or buffer      */
} specdec_status;

/* How the draft distribution is given. */
#define SPECDEC_DRAFT_LOGITS 0 /* q = softmax(draft / T), formed on the device      */
#define SPECDEC_DRAFT_PROBS 1  /* q used as given (one-hot, lookup or any vector)   */
#define SPECDEC_DRAFT_ONEHOT 2 /* q = e_x, one-hot at each drafted token (greedy or
                                  prompt-lookup drafts, [LESS] "Where drafts come
                                  from"); no draft array is read                  */

/* Element type of the scores written by specdec_verify_logits. */
#define SPECDEC_OUT_F32 0
#define SPECDEC_OUT_BF16 1

/* Memory layout of the weights W. */
#define SPECDEC_WEIGHTS_ROW_MAJOR 0 /* W [V, d] row-major, as a model stores it      */
#define SPECDEC_WEIGHTS_PACKED 1    /* the tile layout written by specdec_pack_weights */

/* Largest number of drafted tokens per sequence. */
#define SPECDEC_MAX_GAMMA 63

/* Largest number of nodes of one draft tree (the root included). */
#define SPECDEC_MAX_TREE_NODES 64

/* Human-readable name of a status code; never NULL. */
const char* specdec_status_string(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int specdec_version(void);

/* Bytes of device workspace that specdec_reject_sample and specdec_verify_step
 * need for B sequences of gamma drafts over a vocabulary of V entries.  The
 * workspace holds per-chunk softmax partials, per-row normalisers and
 * per-sequence decisions; its contents need no initialisation and are
 * meaningless after the call.  Returns 0 for invalid sizes. */
size_t specdec_workspace_bytes(int64_t B, int64_t gamma, int64_t V);

/* Bytes of device workspace that specdec_verify_logits needs for N positions,
 * hidden size d, V outputs and the given weight layout, on the current
 * device.  0 means none (the workspace argument may then be NULL).  With
 * packed weights, at most 16 positions, V >= 65536 and d <= 4096 it is 256
 * bytes: the counter of the queue from which the workgroups take vocabulary
 * tiles (initialised by the call itself).  When the
 * output rows are too few to occupy every compute unit, or X is too large to
 * stage whole, the k range is split into groups whose fp32 partial sums are
 * kept here and then added in group order.  For many positions with packed
 * weights (past 128 positions, d % 128 == 0) it also holds a copy of X in the
 * packed layout (ceil(N/16)*16*d bf16), which the kernel for that regime
 * reads.  Returns 0 for invalid sizes. */
size_t specdec_logits_workspace_bytes(int64_t N, int64_t d, int64_t V, int weight_layout);

/* Bytes of device workspace that specdec_verify_step needs: the larger of
 * specdec_logits_workspace_bytes(B*(gamma+1), d, V, weight_layout) and
 * specdec_workspace_bytes(B, gamma, V) rounded up to 256 bytes plus, with
 * packed weights past 64 positions (d % 128 == 0), the packed copy of X that
 * the scoring kernel reads while it also forms the softmax statistics (or,
 * where specdec_logits_workspace_bytes names the tile queue, its 256 bytes).  The
 * unfused path runs the two stages one after the other in the same bytes.
 * Returns 0 for invalid sizes. */
size_t specdec_step_workspace_bytes(int64_t B, int64_t gamma, int64_t d, int64_t V, int weight_layout);

/* How specdec_verify_step runs for a shape on the current device, as a set of
 * flags (0 for invalid sizes):
 *   SPECDEC_STEP_FUSED_STATISTICS    the scoring kernel forms the softmax
 *       (or argmax) partials of every target row as it writes the logits, so
 *       the sampling stage does not read the logits back (packed weights)
 *   SPECDEC_STEP_GREEDY_WITHOUT_LOGITS  at T == 0 the step may be given
 *       logits == NULL: the scoring kernel takes every row's argmax itself and
 *       stores no scores ([LLMI] section 4, failure mode 1: greedy decoding
 *       needs only the argmax; [MATH] "Greedy Decoding Equivalence")
 * The same flags hold for specdec_tree_verify_step with B trees of M nodes
 * (pass gamma = M - 1). */
#define SPECDEC_STEP_FUSED_STATISTICS 1
#define SPECDEC_STEP_GREEDY_WITHOUT_LOGITS 2
int specdec_step_options(int64_t B, int64_t gamma, int64_t d, int64_t V, int weight_layout);

/* Name of the kernel that computes the scores of this shape on the current
 * device ("sweep_kernel", "panel_kernel", "deep_kernel" or "tiled_kernel"),
 * for matching profiler records; "" for invalid sizes.  Never NULL. */
const char* specdec_scoring_kernel(int64_t N, int64_t d, int64_t V, int weight_layout);

/* Bytes of the packed weight layout of a [V, d] bf16 matrix (d % 32 == 0):
 * ceil(V/16)*16*d*2.  Returns 0 for invalid sizes. */
size_t specdec_packed_weight_bytes(int64_t V, int64_t d);

/* Rewrites W [V, d] (device, bf16, row-major) into the packed tile layout in
 * W_packed (device, specdec_packed_weight_bytes(V, d) bytes, caller-owned,
 * must not overlap W).  Inside 16-row tile t, the 32 k values of k-step s
 * form one contiguous 1 KB block holding, for lane l = 16g + m of a wave,
 * W[16t + m][32s + 8g .. 32s + 8g + 7]; rows past V are zero.  This is the
 * operand order of the gfx950 bf16 matrix instruction, so the scoring kernels
 * read each W byte once in fully contiguous 1 KB pieces.  A one-time
 * preparation of the weights (as at model load); the scores it produces are
 * identical to the row-major ones.  Requires d % 32 == 0. */
int specdec_pack_weights(const void* W, void* W_packed, int64_t V, int64_t d, void* stream);

/* Scores: Y = X W^T, the one pass of the target's output layer over all
 * N = B*(gamma+1) positions ([LLMI] section 0, the linear layer Y = XW over N
 * tokens; [MATH] "Prefill vs. Verification Arithmetic Intensity").
 *   X  device, bf16 [N, d]: hidden states, row n = b*(gamma+1) + i
 *   W  device, bf16 [V, d]: weights, one row per output entry (so Y = X W^T;
 *      the pages write the same map as X times a d x V matrix), in
 *      weight_layout SPECDEC_WEIGHTS_ROW_MAJOR, or the same matrix after
 *      specdec_pack_weights (SPECDEC_WEIGHTS_PACKED, needs d % 32 == 0)
 *   Y  device, [N, V]: fp32 (out_dtype SPECDEC_OUT_F32) or bf16 rounded to
 *      nearest even (SPECDEC_OUT_BF16)
 *   workspace  device, at least specdec_logits_workspace_bytes(N, d, V,
 *      weight_layout) bytes, 16-byte aligned (may be NULL when that is 0);
 *      needs no initialisation, meaningless after the call
 * Products are exact and accumulate in fp32 (in k order within a k-group;
 * k-groups, when the shape uses them, are added in order).  Requires N >= 1,
 * d >= 8 with d % 8 == 0, V >= 1; X and W 16-byte aligned.  Y needs 16-byte
 * alignment (8 for bf16) when V % 4 == 0; other V use element stores. */
int specdec_verify_logits(const void* X, const void* W, void* Y, int64_t N, int64_t d, int64_t V, int out_dtype,
                          int weight_layout, void* workspace, size_t workspace_bytes, void* stream);

/* The rejection-sampling rule on given target logits ([LLMI] section 2,
 * acceptance rule, residual distribution and bonus token; [MATH] "The
 * Modified Rejection Sampling Algorithm" and "Greedy Decoding Equivalence";
 * [LESS] "Draft, then verify" and "The acceptance rule").
 *   target_logits device fp32 [B, gamma+1, V]: row i scores the position after
 *                 the i-th drafted token; row gamma is the bonus row
 *   draft         device fp32 [B, gamma, V]: draft logits (draft_kind
 *                 SPECDEC_DRAFT_LOGITS) or probabilities (SPECDEC_DRAFT_PROBS);
 *                 unused (may be NULL) when temperature == 0, gamma == 0 or
 *                 draft_kind is SPECDEC_DRAFT_ONEHOT (then row i keeps x_i
 *                 iff u < p_i(x_i), and a rejection draws from p_i without x_i)
 *   draft_tokens  device int32 [B, gamma]: the drafted ids x_i
 *   temperature   T >= 0.  T > 0: p = softmax(target / T) and, for logits,
 *                 q = softmax(draft / T) ([LESS] "First: what an output
 *                 distribution is"; temperature is applied to both, per
 *                 [LESS] "Why the output is exactly p").  T == 0: greedy rule.
 *   uniforms      device fp32 [B, gamma+1, 2], each in [0, 1): [b, i, 0]
 *                 decides the accept test at row i, [b, i, 1] drives the draw
 *                 if the step ends at row i.  Unused (may be NULL) at T == 0.
 *   out_tokens    device int32 [B, gamma+1]: emitted tokens, -1 after the last
 *   out_num_emitted device int32 [B]: 1 .. gamma+1
 *   out_probs     optional device fp32 [B, gamma, 2]: p_i(x_i), q_i(x_i) for
 *                 every drafted row (NULL to skip; unused at T == 0)
 *   workspace     device, at least specdec_workspace_bytes(B, gamma, V) bytes,
 *                 16-byte aligned
 * Row i keeps x_i iff u[b,i,0] < min(1, p_i(x_i) / max(q_i(x_i), 1e-12)); the
 * step emits x_0 .. x_{k-1} for the first rejected row k, then one token drawn
 * by inverse CDF (smallest v with u[b,k,1] * S < C_v, C the running sum in
 * vocabulary order) from (p_k - q_k)+, or from p_gamma when all gamma are
 * kept.  p, q, (p - q)+ and p/q are fp32 values; normalisers and running sums
 * are accumulated in fp64.  At T == 0 row i keeps x_i iff x_i is the row's
 * argmax (lowest index on ties); the first mismatch, or the bonus row, emits
 * the argmax.  Requires B >= 1, 0 <= gamma <= SPECDEC_MAX_GAMMA, V >= 1. */
int specdec_reject_sample(const float* target_logits, const float* draft, int draft_kind,
                          const int32_t* draft_tokens, float temperature, const float* uniforms, int64_t B,
                          int64_t gamma, int64_t V, int32_t* out_tokens, int32_t* out_num_emitted,
                          float* out_probs, void* workspace, size_t workspace_bytes, void* stream);

/* The whole step: specdec_verify_logits (fp32 scores into `logits`) followed by
 * specdec_reject_sample, enqueued on one stream.
 *   X [B*(gamma+1), d] and W [V, d] bf16 in weight_layout, as in
 *            specdec_verify_logits
 *   logits   device fp32 [B*(gamma+1), V]: caller scratch that receives the
 *            target logits.  May be NULL at temperature == 0 when
 *            specdec_step_options reports SPECDEC_STEP_GREEDY_WITHOUT_LOGITS
 *            for the shape: the scoring kernel then takes every row's argmax
 *            and no scores are written or read back (SPECDEC_ERR_NULL
 *            otherwise)
 *   workspace at least specdec_step_workspace_bytes(B, gamma, d, V,
 *            weight_layout) bytes, shared by the two stages
 * Other arguments as in specdec_reject_sample. */
int specdec_verify_step(const void* X, const void* W, int weight_layout, const float* draft, int draft_kind,
                        const int32_t* draft_tokens, float temperature, const float* uniforms, int64_t B,
                        int64_t gamma, int64_t d, int64_t V, float* logits, int32_t* out_tokens,
                        int32_t* out_num_emitted, float* out_probs, void* workspace, size_t workspace_bytes,
                        void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * specdec_verify_step with the library's own static workspace instead of a
 * caller-provided one.  The workspace is a file-scope device array of
 * SPECDEC_NOALLOC_MAX_WORKSPACE bytes, one copy on every GPU the library runs
 * on, held until the process ends; its device address is looked up once per
 * device, on the first call made with that device current.  The call itself
 * allocates nothing and frees nothing.
 *   Arguments as in specdec_verify_step, without the workspace; the caller
 *   still provides every input and output (logits as in specdec_verify_step).
 *   SPECDEC_ERR_SCRATCH (before any device call) when
 *   specdec_step_workspace_bytes(B, gamma, d, V, weight_layout) exceeds
 *   SPECDEC_NOALLOC_MAX_WORKSPACE (32 MiB: up to about 512 positions of a
 *   Llama-sized head); SPECDEC_ERR_DEVICE when the runtime cannot report the
 *   current device or the buffer's address.
 * Every call on one GPU uses that GPU's one buffer, which keeps the last
 * call's contents (nothing in it needs to start at zero: each call
 * initialises what it reads).  Calls that overlap in time on one GPU (from
 * several host threads, or on several streams) race on it: order them on one
 * stream, or give each its own workspace through specdec_verify_step. */
#define SPECDEC_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)
int specdec_verify_step_noalloc(const void* X, const void* W, int weight_layout, const float* draft, int draft_kind,
                                const int32_t* draft_tokens, float temperature, const float* uniforms, int64_t B,
                                int64_t gamma, int64_t d, int64_t V, float* logits, int32_t* out_tokens,
                                int32_t* out_num_emitted, float* out_probs, void* stream);

/* Top-k / top-p warping before the rule ([LESS] "Why the output is exactly p":
 * the sampling settings reshape p, and q before drafting, and the rule then
 * reproduces the reshaped p; [PREP] "Correctness").  At T > 0 every target row
 * and every draft-logits row is warped after temperature: entries are ranked
 * by logit (larger first, ties by lower index); top-k keeps the first top_k;
 * top-p then keeps the shortest prefix of those whose probability mass reaches
 * top_p (at least one entry); the kept entries are renormalised and the rest
 * have probability 0.  Draft probabilities and one-hot drafts are used as
 * given.  At T == 0 the settings are ignored (the argmax is always kept).
 *   top_k  >= 0; 0 (or >= V) turns top-k off
 *   top_p  in (0, 1]; 1 turns top-p off.  Masses are summed exactly as
 *          integers with 40 fraction bits (fp32 exp((z - max z) / T)), so the
 *          top-p cut may differ from an fp64 one only where the cumulative
 *          mass is within a few 1e-6 of top_p.
 * Requires V <= 2^23 when either setting is active (SPECDEC_ERR_SHAPE).
 * Other arguments, the workspace and the rule as in specdec_reject_sample
 * (SPECDEC_ERR_ARG for settings out of range).  Logits must not be NaN. */
int specdec_reject_sample_warped(const float* target_logits, const float* draft, int draft_kind,
                                 const int32_t* draft_tokens, float temperature, int64_t top_k, float top_p,
                                 const float* uniforms, int64_t B, int64_t gamma, int64_t V, int32_t* out_tokens,
                                 int32_t* out_num_emitted, float* out_probs, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* specdec_verify_step with top-k / top-p warping as in
 * specdec_reject_sample_warped (same workspace size as specdec_verify_step). */
int specdec_verify_step_warped(const void* X, const void* W, int weight_layout, const float* draft, int draft_kind,
                               const int32_t* draft_tokens, float temperature, int64_t top_k, float top_p,
                               const float* uniforms, int64_t B, int64_t gamma, int64_t d, int64_t V, float* logits,
                               int32_t* out_tokens, int32_t* out_num_emitted, float* out_probs, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Tree verification ([LLMI] section 3, multi-draft tree speculation: the tree
 * attention mask and depth offsets; [MATH] "SpecInfer and Tree-Based
 * Verification": every node of the tree is scored in one pass and the longest
 * accepted path is kept).  A tree of M nodes is flattened so that every parent
 * comes before its children: node 0 is the root (the last token already in the
 * text; its parent entry is ignored) and node i >= 1 has parents[i] in
 * [0, i).  A node whose parent entry is outside [0, i) is detached: it is its
 * own only ancestor, has depth 0 and is never accepted.  M <= 64. */

/* Ancestor masks and depths of B trees.
 *   parents       device int32 [B, M]
 *   out_mask      device uint64 [B, M]: bit j of [b, i] set iff node j is an
 *                 ancestor of node i or i itself (the attention pattern)
 *   out_depth     device int32 [B, M]: edges from the root (the RoPE position
 *                 offset of the node)
 *   out_additive  optional device fp32 [B, M, M]: 0 where node i may attend
 *                 to node j, -inf elsewhere (NULL to skip) */
int specdec_tree_mask(const int32_t* parents, int64_t B, int64_t M, uint64_t* out_mask, int32_t* out_depth,
                      float* out_additive, void* stream);

/* Bytes of device workspace for specdec_tree_verify_greedy (0 for invalid sizes). */
size_t specdec_tree_workspace_bytes(int64_t B, int64_t M, int64_t V);

/* Greedy (T = 0) verification of B trees on given logits.
 *   target_logits device fp32 [B, M, V]: row i scores the position after
 *                 node i along its path from the root
 *   parents, node_tokens  device int32 [B, M]: node i's parent and token
 *                 (ids outside [0, V) never match an argmax)
 *   out_tokens    device int32 [B, M]: the tokens of the kept path after the
 *                 root, then the argmax of the last kept node's row, then -1
 *   out_num_emitted device int32 [B]: length of the kept path (root
 *                 excluded) + 1, in 1 .. M
 *   out_nodes     device int32 [B, M]: the kept path's node indices from the
 *                 root (the positions whose keys and values survive), then -1
 * Node i >= 1 is accepted iff its parent is and node_tokens[i] is the argmax
 * of its parent's row (lowest index on ties); the deepest accepted node
 * (lowest index among equals) ends the kept path.  With a chain (parents[i] =
 * i - 1) this is the greedy rule of specdec_reject_sample. */
int specdec_tree_verify_greedy(const float* target_logits, const int32_t* parents, const int32_t* node_tokens,
                               int64_t B, int64_t M, int64_t V, int32_t* out_tokens, int32_t* out_num_emitted,
                               int32_t* out_nodes, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace for specdec_tree_verify_step, composed as for
 * specdec_step_workspace_bytes with specdec_tree_workspace_bytes(B, M, V) as
 * the sampling part (0 for invalid sizes). */
size_t specdec_tree_step_workspace_bytes(int64_t B, int64_t M, int64_t d, int64_t V, int weight_layout);

/* The whole tree step: scores of all B*M nodes (X [B*M, d] bf16, row b*M + i
 * the hidden state of node i of tree b; W as in specdec_verify_logits) into
 * `logits` fp32 [B*M, V], then specdec_tree_verify_greedy on them.  With
 * packed weights the scoring kernel forms the rows' argmax partials itself;
 * then `logits` may be NULL where specdec_step_options(B, M - 1, d, V,
 * weight_layout) reports SPECDEC_STEP_GREEDY_WITHOUT_LOGITS (no scores are
 * written; SPECDEC_ERR_NULL otherwise). */
int specdec_tree_verify_step(const void* X, const void* W, int weight_layout, const int32_t* parents,
                             const int32_t* node_tokens, int64_t B, int64_t M, int64_t d, int64_t V, float* logits,
                             int32_t* out_tokens, int32_t* out_num_emitted, int32_t* out_nodes, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Paged KV cache with speculative rollback ([LLMI] section 1, paged block
 * allocation: keys and values in fixed-size physical blocks reached through a
 * per-request block table, so rejected speculative tokens are dropped by
 * shortening a length and returning blocks, without moving data; [LESS] "The
 * KV cache has to forget": after a round the cache is cut back to the true
 * text).  All state is caller-owned device memory:
 *   k_pool, v_pool  [num_blocks][heads][block_size][head_dim] elements of
 *                   elem_bytes (2 or 4) each; head_dim * elem_bytes % 16 == 0
 *   block_tables    int32 [R][max_blocks]: physical block of each logical block
 *   seq_lens        int32 [R]: tokens held; request r uses
 *                   ceil(seq_lens[r] / block_size) logical blocks, token t sits
 *                   in logical block t / block_size at offset t % block_size
 *   free_stack      int32 [num_blocks] and free_top int32 [1]: the free blocks
 *                   are free_stack[0 .. free_top-1], the top of the stack last
 *   status          int32 [1], written by append (0 ok; 1 not enough free
 *                   blocks; 2 a request would exceed max_blocks; on 1 or 2
 *                   nothing changes) and by rollback (0 ok; 3 some request was
 *                   asked to grow or to go below 0 and was left as it is)
 * A batch is served in request order, exactly as one request after another
 * would be: allocation takes blocks from the top of the free stack, rollback
 * pushes a request's trailing blocks back, its last logical block first.
 * Block ids read from a table are checked against num_blocks: an
 * inconsistent table never makes a kernel access outside the pool. */

/* Fresh state: free_stack = num_blocks-1, ..., 1, 0 (the first block handed
 * out is 0), free_top = num_blocks, seq_lens = 0. */
int specdec_kv_init(int32_t* free_stack, int32_t* free_top, int32_t* seq_lens, int64_t R, int64_t num_blocks,
                    void* stream);

/* Bytes of device workspace for specdec_kv_append (0 for invalid sizes). */
size_t specdec_kv_workspace_bytes(int64_t R);

/* Appends n_new tokens to every request: k_new, v_new device
 * [R][heads][n_new][head_dim] (16-byte aligned).  Allocates the logical
 * blocks the new lengths need, then writes the keys and values through the
 * tables; all or nothing (see status). */
int specdec_kv_append(void* k_pool, void* v_pool, int32_t* block_tables, int32_t* seq_lens, int32_t* free_stack,
                      int32_t* free_top, int32_t* status, const void* k_new, const void* v_new, int64_t R,
                      int64_t n_new, int64_t num_blocks, int64_t heads, int64_t block_size, int64_t head_dim,
                      int64_t elem_bytes, int64_t max_blocks, void* workspace, size_t workspace_bytes, void* stream);

/* Rolls request r back to keep_lens[r] tokens (device int32 [R]), returning
 * the blocks it no longer needs.  No key or value moves. */
int specdec_kv_rollback(int32_t* block_tables, int32_t* seq_lens, int32_t* free_stack, int32_t* free_top,
                        int32_t* status, const int32_t* keep_lens, int64_t R, int64_t num_blocks, int64_t block_size,
                        int64_t max_blocks, void* stream);

/* The rollback after a verification step, driven by its num_emitted (device
 * int32 [R]): the step appended the gamma+1 positions it scored (the last
 * token of the text and the gamma drafts); the text grew by num_emitted
 * tokens, of which the last (correction or bonus) is not yet in the cache.
 * So request r keeps seq_lens[r] - (gamma + 1) + num_emitted[r] tokens. */
int specdec_kv_rollback_after_verify(int32_t* block_tables, int32_t* seq_lens, int32_t* free_stack,
                                     int32_t* free_top, int32_t* status, const int32_t* num_emitted, int64_t gamma,
                                     int64_t R, int64_t num_blocks, int64_t block_size, int64_t max_blocks,
                                     void* stream);

/* Contiguous keys and values: k_out, v_out device [R][heads][max_len][head_dim];
 * entries t < min(seq_lens[r], max_len) are written, the rest left as they are.
 * max_len <= 2^24 and max_len * head_dim * elem_bytes <= 2^34 (SPECDEC_ERR_SHAPE
 * otherwise). */
int specdec_kv_gather(const void* k_pool, const void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                      int64_t R, int64_t num_blocks, int64_t heads, int64_t block_size, int64_t head_dim,
                      int64_t elem_bytes, int64_t max_blocks, int64_t max_len, void* k_out, void* v_out,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECDEC_H */
