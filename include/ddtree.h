/*
 * ddtree.h -- C ABI of libddtree.so, the DDTree tree-verify step on
 * AMD Instinct MI355X (gfx950).
 *
 * The step verifies a budget-sized draft token tree against the committed
 * state of a hybrid linear-attention target in one pass, then accepts the
 * longest draft path that agrees with the target's greedy choice and rolls
 * the linear-attention state forward to it.  Sources:
 *   [P1] Luce-Org/lucebox-hub README (bittide copy), section
 *        "02 · DFlash DDtree Qwen3.5 & Qwen3.6 27B GGUF on RTX 3090":
 *        "Algorithms used" (DDTree tree-structured verify beats chain verify
 *        at the same budget), "Implemented here" (tree-aware SSM state
 *        rollback kernels ssm_conv_tree, gated_delta_net_tree and
 *        gated_delta_net_tree_persist; budget 22), "Retune per GPU".
 *   [P2] codehub view of lucebox-hub@main: "Run the Server" / "Making
 *        requests" (greedy decoding), "Server flags" (--ddtree,
 *        --ddtree-budget 22, --fa-window 0 = full attention),
 *        "GPU draft top-K & verify-argmax (DFlash)" (verify argmax read in
 *        place from device logits, result validated).
 *   [P3] Luce-Org/lucebox README, "Inference Engine Optimizations" (paged
 *        attention, concurrent serving).
 * The recurrence of the linear-attention layers is the gated delta rule
 * (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", 2024).
 *
 * Conventions shared by every call
 * --------------------------------
 * - All pointers named "device" are HIP device pointers owned by the caller;
 *   the library never allocates, frees or keeps a pointer past the call.
 * - Every call that takes `stream` validates its host-visible arguments,
 *   then enqueues kernels on that hipStream_t (passed as void*, NULL = the
 *   null stream) and returns without synchronising.  On any validation
 *   error it returns a negative DDT_E_* code and enqueues nothing.
 * - Problems that only the device can see (a malformed parent array, a draft
 *   token outside the vocabulary, ...) are reported as DDT_ST_* bits in the
 *   per-sequence device status word plan->status[b]; kernels never read
 *   outside their buffers on such input.  The caller reads the status words
 *   (a few bytes) after the step and discards results of flagged sequences.
 *   There is no silent CPU fallback.
 * - Several sequences are verified together (continuous batching, [P3]):
 *   their trees are concatenated; node ids inside a tree are local
 *   (0 = root), and "global" node g = tree_off[b] + local id indexes the
 *   per-node arrays.
 * - Calls on different streams are thread-safe; calls that share output
 *   buffers must be ordered by the caller.
 */
#ifndef DDTREE_H
#define DDTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DDT_VERSION 2

/* return codes */
#define DDT_OK 0
#define DDT_E_ARG (-1)    /* null pointer or bad enum / flag               */
#define DDT_E_TREE (-2)   /* malformed tree (host-side plan only)           */
#define DDT_E_SHAPE (-3)  /* unsupported or inconsistent sizes              */
#define DDT_E_DTYPE (-4)  /* unsupported storage type                       */
#define DDT_E_RANGE (-5)  /* value out of range (host-side checks)          */
#define DDT_E_WS (-6)     /* workspace too small                            */
#define DDT_E_HIP (-7)    /* a HIP launch failed; see ddt_status_str        */

/* device status bits, OR-ed into plan->status[b] */
#define DDT_ST_TREE 1u    /* parent array of sequence b malformed           */
#define DDT_ST_LEVELS 2u  /* tree deeper than the level cap                 */
#define DDT_ST_TOKEN 4u   /* a draft token is outside [0, V)                */
#define DDT_ST_ARGMAX 8u  /* verify argmax failed validation                */
#define DDT_ST_CTX 16u    /* context length / page table cannot hold it     */
#define DDT_ST_COMMIT 32u /* commit descriptor incomplete                   */

/* storage types */
#define DDT_F32 0
#define DDT_F16 1
#define DDT_BF16 2

#define DDT_MAX_NODES 64 /* nodes per tree, root included                  */
#define DDT_MAX_W 8      /* conv width                                      */
#define DDT_PAGE 16      /* tokens per KV page                              */

/*
 * Plan of a batch of draft trees.  Host struct holding device pointers
 * (host pointers for ddt_tree_plan_host).  The caller allocates every array
 * with the stated size; ddt_tree_plan fills the outputs.
 *
 * Tree encoding ([P1] "Algorithms used"; [P2] --ddtree-budget): parent
 * pointers, parent[root] = -1, 0 <= parent[i] < i, so index order is
 * topological.  The root is the last committed token (the previous step's
 * bonus), not yet in the cache or the state; the budget counts it.
 */
typedef struct ddt_plan {
  int32_t B;       /* sequences, >= 1                                      */
  int32_t n_total; /* nodes over all sequences = tree_off[B]               */
  int32_t n_max;   /* largest tree, 1..DDT_MAX_NODES                       */
  int32_t W;       /* conv width the windows are built for, 1..DDT_MAX_W   */
  const int32_t *tree_off; /* [B+1] node offsets, tree_off[0] = 0; with B = 1
                              the layer kernels do not read it (the tree is
                              nodes 0..n_total-1) and the device plan flags
                              DDT_ST_TREE if it says otherwise             */
  const int32_t *parent;   /* [n_total] local parent ids                    */
  int32_t *depth;  /* out [n_total] edge depth (root 0)                    */
  uint64_t *anc;   /* out [n_total] bit j = local node j on the root path  */
  int32_t *win;    /* out [n_total][max(W-1,1)]: entry j-1 = j-th previous
                      token on prefix ++ root path: local node id >= 0, or
                      -(s+1) for committed prefix slot s (0 = oldest)     */
  int32_t *status; /* out [B] device status word, DDT_ST_* bits          */
} ddt_plan;

int ddt_version(void);
const char *ddt_status_str(int code);

/*
 * sha256 (64 lowercase hex digits) of the sources this library was built
 * from: include/ddtree.h and every file of the package's csrc/ directory,
 * taken in name order as "<relative path>\0<bytes>" records.  A caller can
 * hash its checked-out sources the same way to confirm which build it runs.
 * The string is static; the caller must not free it.
 */
const char *ddt_source_hash(void);

/*
 * Tree plan on the host: same outputs as ddt_tree_plan, all pointers in
 * `plan` are host pointers.  Returns DDT_E_TREE on a malformed tree (any
 * parent[0] != -1, parent[i] outside [0, i), tree size outside
 * [1, DDT_MAX_NODES] or above n_max) and DDT_E_RANGE when a tree has more
 * than max_levels levels (levels count the nodes on a root path).  Outputs
 * are written only on DDT_OK.
 */
int ddt_tree_plan_host(const ddt_plan *plan, int32_t max_levels);

/*
 * Tree plan on the device (one wavefront per sequence).  Reads
 * plan->tree_off and plan->parent, writes depth, anc, win and resets
 * status[b] to the sequence's DDT_ST_TREE / DDT_ST_LEVELS bits.  A
 * malformed tree is flagged and replaced by a safe plan (invalid parents
 * read as the root) so later kernels stay in bounds.  Must run before the
 * other calls of a step.
 */
int ddt_tree_plan(const ddt_plan *plan, int32_t max_levels, void *stream);

/*
 * Tree-aware causal depthwise conv1d ([P1] "Implemented here",
 * ssm_conv_tree).  For every node i and channel c:
 *   y[i][c] = act( sum_{t=0}^{W-1} w[c][W-1-t] * tok_t(i)[c] )
 * where tok_0 = x[i] and tok_j (j >= 1) is window entry j-1 of the plan
 * (an ancestor's x, or a committed prefix token).  No bias.
 *   x      device [n_total][C]        dtype
 *   prefix device [B][W-1][C]         dtype, oldest first (read only)
 *   w      device [C][W]              dtype, tap W-1 = current token
 *   y      device [n_total][C]        fp32
 *   act    0 = identity, 1 = SiLU;  dtype DDT_F32 or DDT_BF16;  C % 64 == 0.
 */
int ddt_tree_conv(const ddt_plan *plan, const void *x, const void *prefix, const void *w,
                  int32_t C, int32_t act, int32_t dtype, float *y, void *stream);

/*
 * Tree gated delta-net ([P1] "Implemented here", gated_delta_net_tree
 * and its _persist variant).  For value head h (key head g = h / (Hv/Hk)),
 * every node n starts from its parent's state (the root from S_c[b][h]):
 *   S_n = alpha_n S_p (I - beta_n k_n k_n^T) + beta_n v_n k_n^T
 *   out_n = scale * S_n q_n
 * S is dv x dk (row r of S maps keys to value channel r).
 *   q, k        device [n_total][Hk][dk]   dtype
 *   v           device [n_total][Hv][dv]   dtype
 *   alpha, beta device [n_total][Hv]       dtype
 *   S_c         device [B][Hv][dv][dk]     fp32, read only
 *   out         device [n_total][Hv][dv]   fp32
 *   node_states device [n_total][Hv][dv][dk] fp32 or NULL: when given, every
 *               node's state is stored ("persist"), so the commit can
 *               select the accepted node's state instead of replaying.
 *   node_u      device [n_total][Hv][dv] fp32 or NULL: when given, every
 *               node's u_n = beta_n (v_n - alpha_n S_p k_n) is stored (the
 *               state update is S_n = alpha_n S_p + u_n k_n^T), so the commit
 *               can rebuild the accepted node's state from S_c with one
 *               rank-L update (DDT_COMMIT_UPDATE), 46x less than node_states.
 * Requires Hv % Hk == 0, dk in {16, 32, 64, 128}, dv % 16 == 0, dtype
 * DDT_F32 or DDT_BF16; q, k, v rows 16-byte aligned.  Outputs of nodes on
 * the same root path are consistent to the last bit: the state a node gets
 * here, in a replay of its path, or in an update from the saved u is the
 * same.
 */
int ddt_tree_gdn(const ddt_plan *plan, const void *q, const void *k, const void *v,
                 const void *alpha, const void *beta, const float *S_c, int32_t Hk, int32_t Hv,
                 int32_t dk, int32_t dv, float scale, int32_t dtype, float *out,
                 float *node_states, float *node_u, void *stream);

/*
 * Tree-masked attention over the committed KV cache.  Node i, query
 * head h (KV head g = h / (Hq/Hkv)) attends to all T[b] committed tokens of
 * its sequence plus the draft tokens on its own root path, itself included
 * (plan->anc); full attention, no window ([P2] --fa-window 0):
 *   out[i][h] = softmax(scale * K q_ih)^T V
 * The cache is paged ([P3]); a page holds DDT_PAGE tokens of every KV head:
 *   Kc device [P][Hkv][DDT_PAGE][D]   token t at page_table[b][t/16], row t%16
 *   Vc device [P][Hkv][D][DDT_PAGE]   same page, column t%16 (channel-major
 *                                     inside a page)
 *   page_table device [B][max_pages] int32, or NULL for B == 1 with page
 *              t/16 (a contiguous cache).
 *   T          device [B] committed lengths; each must be <= T_max (host).
 *   q          device [n_total][Hq][D];  Kt, Vt device [n_total][Hkv][D]
 *              (the tree's draft keys/values, not yet in the cache)
 *   out        device [n_total][Hq][D] fp32
 *   ws         device workspace of ddt_tree_attn_workspace() bytes (split
 *              partials; its contents need not be initialised: a call reads
 *              only the slots it has written).  The workspace query returns
 *              0 when the small path runs, which needs none.
 * dtype: DDT_F16 (D in {128, 256} on matrix cores; D in {16, 32, 64} on the
 * small path) or DDT_F32 (D in {16, 32, 64}).  Hq % Hkv == 0.  n_splits: number of
 * context splits per KV head (and group of up to 192 query rows), 0 = automatic
 * (about one workgroup per compute unit, splits of at least 256 keys).  One
 * sequence has them all; the sequences of a larger batch share them: each
 * takes one, and the rest are dealt in proportion to each sequence's 32-key
 * tiles (cache and tree), at most one per 256 of its committed keys, so a
 * batch of B sequences uses at least B splits (matrix-core path: B <= 1024,
 * else DDT_E_SHAPE).  A sequence whose T[b] exceeds T_max or its page table is
 * flagged DDT_ST_CTX and only its first T_max tokens are read.
 * Precision (matrix-core path): scores and value sums accumulate in fp32,
 * probabilities enter the value product as fp16 (as the fp16 values do);
 * each context split's output rows, divided by their own sums, pass through
 * fp16 in the workspace (at most 2^-11 relative) before the fp32 merge.
 */
size_t ddt_tree_attn_workspace(const ddt_plan *plan, int32_t Hq, int32_t Hkv, int32_t D,
                               int32_t T_max, int32_t n_splits);
int ddt_tree_attn(const ddt_plan *plan, const void *q, const void *Kc, const void *Vc,
                  const int32_t *page_table, int32_t max_pages, const int32_t *T, int32_t T_max,
                  const void *Kt, const void *Vt, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                  int32_t dtype, int32_t n_splits, float *out, void *ws, size_t ws_bytes,
                  void *stream);

/*
 * Variant of ddt_tree_attn: tree-masked attention over an 8-bit KV cache ([P1] keeps its
 * cache quantized to fit long contexts).  Same operation, layouts of pages
 * and arguments as ddt_tree_attn, with the cache stored as
 *   Kq  device [P][Hkv][DDT_PAGE][D] int8     Vq  device [P][Hkv][D][DDT_PAGE] int8
 *   Ksc device [P][Hkv][DDT_PAGE] fp16        Vsc device [P][Hkv][DDT_PAGE] fp16
 * one scale per token and KV head for K and for V.  The cache value of an
 * entry q with scale s is fp16(q * s): the exact product rounded once to
 * fp16 (round to nearest even); attention is over those values exactly as
 * over an fp16 cache.  q, Kt, Vt fp16; D in {128, 256}; the workspace is
 * ddt_tree_attn_workspace() bytes.  Errors as ddt_tree_attn; DDT_E_SHAPE for
 * another D.
 */
int ddt_tree_attn_q8(const ddt_plan *plan, const void *q, const int8_t *Kq, const void *Ksc,
                     const int8_t *Vq, const void *Vsc, const int32_t *page_table, int32_t max_pages,
                     const int32_t *T, int32_t T_max, const void *Kt, const void *Vt, int32_t Hq,
                     int32_t Hkv, int32_t D, float scale, int32_t n_splits, float *out, void *ws,
                     size_t ws_bytes, void *stream);

/*
 * Verify argmax and greedy acceptance walk ([P2] "Making requests":
 * greedy decoding; "GPU draft top-K & verify-argmax": the argmax is read in
 * place from the device logits and validated).
 *   argmax[i] = smallest v maximising logits[i][v] (NaN never wins)
 *   path: start at the root; while some child c of the last node has
 *   draft_tok[c] == argmax[last], append the smallest such c.
 *   logits    device [n_total][V]  DDT_F32 or DDT_BF16
 *   draft_tok device [n_total] int32 (the root's entry is not compared)
 *   argmax    device out [n_total] int32
 *   path      device out [B][n_max] int32 local ids, padded with -1
 *   L         device out [B] path length (tokens emitted = L: L-1 drafts
 *             plus the bonus token)
 *   bonus     device out [B] argmax of the last path node
 *   ws        device workspace of ddt_accept_walk_workspace() bytes.
 * A draft token outside [0, V) sets DDT_ST_TOKEN (it can never match).
 */
size_t ddt_accept_walk_workspace(const ddt_plan *plan, int32_t V);
int ddt_accept_walk(const ddt_plan *plan, const void *logits, int32_t dtype, int32_t V,
                    const int32_t *draft_tok, int32_t *argmax, int32_t *path, int32_t *L,
                    int32_t *bonus, void *ws, size_t ws_bytes, void *stream);

/*
 * The verify argmax and walk on the host: the fall-back of the validated
 * device walk (codehub lucebox-hub@main, "GPU draft top-K & verify-argmax
 * (DFlash)": the device result is checked, and the host computes it when the
 * check fails).  The device walk reports a failed check as DDT_ST_ARGMAX in
 * the plan's status word; the caller then copies that step's logits and draft
 * tokens to the host and calls this.  Results are those of ddt_accept_walk,
 * bit for bit (same ties, NaN and -0 rules).
 *   plan      host struct with HOST pointers: tree_off, parent (read) and
 *             status (DDT_ST_TOKEN OR-ed in for a draft token outside
 *             [0, V), which can never match); depth, anc, win unused
 *   logits    host [n_total][V]  DDT_F32 or DDT_BF16
 *   draft_tok host [n_total] int32 (the root's entry is not compared)
 *   argmax, path, L, bonus  host outputs, laid out as for ddt_accept_walk
 * Errors: DDT_E_ARG (null pointer), DDT_E_SHAPE (B, n_total, n_max, V),
 * DDT_E_DTYPE, DDT_E_TREE (the trees are checked as ddt_tree_plan_host checks
 * them); nothing is written then.  Runs on the calling thread; no HIP call.
 */
int ddt_accept_walk_host(const ddt_plan *plan, const void *logits, int32_t dtype, int32_t V,
                         const int32_t *draft_tok, int32_t *argmax, int32_t *path, int32_t *L,
                         int32_t *bonus);

/*
 * The same verify argmax and walk for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops, and
 * harnesses that forbid allocation.  Arguments and results are those of
 * ddt_accept_walk, without the workspace: the chunk maxima go to a static
 * device array of DDT_NOALLOC_MAX_NODES * 16 keys (512 KiB) that the library
 * holds on every GPU it runs on until the process ends.  The call allocates
 * and frees nothing.  Every key it reads is first written by the same call,
 * so the array needs no clearing; but all calls on one GPU share it, so two
 * calls that overlap on one GPU (different streams, not ordered) race and
 * must be ordered by the caller.
 * Errors: as ddt_accept_walk, plus DDT_E_SHAPE for n_total above
 * DDT_NOALLOC_MAX_NODES and DDT_E_HIP if the array's device address cannot
 * be found; nothing is launched then.
 */
#define DDT_NOALLOC_MAX_NODES 4096
int ddt_accept_walk_noalloc(const ddt_plan *plan, const void *logits, int32_t dtype, int32_t V,
                            const int32_t *draft_tok, int32_t *argmax, int32_t *path, int32_t *L,
                            int32_t *bonus, void *stream);

/*
 * Stochastic acceptance (temperature > 0).  Requests without a temperature
 * are sampled with the model card's settings (temperature 1.0, top_p 0.95,
 * top_k 20; codehub lucebox-hub@main, "Making requests"); the pages give no
 * rule for accepting a tree then.  Reading: every node's target
 * distribution is its logits / T, cut to the top_k tokens (ties to the lower
 * index, NaN and -inf never kept), softmaxed, cut to the smallest prefix in
 * descending order with c_i >= top_p * total (inclusive cumulative masses),
 * renormalised; the node's sample is the first kept token with
 * c_i > u * R (R the kept mass, u the node's uniform).  The walk is the
 * greedy walk with the samples in place of the argmax: every emitted token
 * is a draw from the target, which is what recursive rejection sampling
 * gives for deterministic candidates.
 *   logits, dtype, V, draft_tok, path, L, bonus  as for ddt_accept_walk
 *   uniforms  device [n_total] float in [0, 1): one draw per node (input;
 *             the caller's random numbers)
 *   temperature > 0 and finite; top_k 1..32; top_p in (0, 1]
 *   sample    device out [n_total] int32: every node's sample (0 and
 *             DDT_ST_ARGMAX for a row with no finite logit)
 *   ws        device workspace of ddt_accept_sample_workspace() bytes.
 * Samples are computed in fp32: a draw whose u * R lies within rounding
 * distance of a cumulative mass may differ from an exact evaluation by the
 * neighbouring token.
 * Errors: DDT_E_ARG, DDT_E_SHAPE (V, top_k; V up to 393216), DDT_E_RANGE
 * (temperature, top_p), DDT_E_DTYPE, DDT_E_WS; nothing is launched then.
 */
size_t ddt_accept_sample_workspace(const ddt_plan *plan, int32_t V, int32_t top_k);
int ddt_accept_sample(const ddt_plan *plan, const void *logits, int32_t dtype, int32_t V,
                      const int32_t *draft_tok, const float *uniforms, float temperature, int32_t top_k,
                      float top_p, int32_t *sample, int32_t *path, int32_t *L, int32_t *bonus, void *ws,
                      size_t ws_bytes, void *stream);

/*
 * Commit of the accepted path ([P1] "Implemented here": tree-aware SSM
 * state rollback; "Why GGUF": the DDTree verify state).  In one launch, for
 * every sequence b with accepted local path p_0 = 0, ..., p_{L-1}:
 *  - each gated delta-net layer: S_c[b] <- state of node p_{L-1}.
 *    mode DDT_COMMIT_REPLAY re-runs the rule along the path from S_c;
 *    mode DDT_COMMIT_SELECT copies the persisted node state (node_states of
 *    that layer must be non-NULL); mode DDT_COMMIT_UPDATE applies
 *    S_c <- a_i P_i S_c + sum_a a_i w(a,i) u_a k_a^T + u_i k_i^T over the
 *    path, with the u saved by ddt_tree_gdn (node_u must be non-NULL; P_i is
 *    the product of the gates of i's ancestors, w(a,i) of those strictly
 *    between a and i).  All three give bitwise the same state.  A layer
 *    without the buffer its mode needs sets DDT_ST_COMMIT and is left as is.
 *  - each conv: prefix[b] <- last W-1 rows of prefix[b] ++ x[path].
 *  - each attention layer: the path's Kt/Vt are written to cache positions
 *    T[b] .. T[b]+L-1 (the page table must already map them), and finally
 *    T[b] += L.
 * Cache capacity (when n_attn > 0): page_table is [B][max_pages]; for a
 * contiguous cache (page_table NULL, B == 1) max_pages is the number of
 * DDT_PAGE-token pages each layer's Kc / Vc holds.  Either way max_pages >= 1
 * (else DDT_E_SHAPE) and sequence b fits when 0 <= T[b] and
 * T[b] + L[b] <= DDT_PAGE * max_pages.  A sequence that does not fit is not
 * committed at all -- its delta-net states, conv prefixes, cache and T[b]
 * are left as they were -- and DDT_ST_CTX is set in its status word, so its
 * layers never move ahead of its cache.  With n_attn == 0 there is no cache
 * and every sequence is committed.
 * The layer descriptor arrays live in DEVICE memory (the caller builds them
 * once); their shapes are given here.  Per-layer fields may be NULL where
 * noted.
 */
#define DDT_COMMIT_REPLAY 0
#define DDT_COMMIT_SELECT 1
#define DDT_COMMIT_UPDATE 2

typedef struct ddt_gdn_layer {
  const void *q, *k, *v, *alpha, *beta; /* this step's tree inputs (ddt_tree_gdn) */
  float *S_c;                           /* [B][Hv][dv][dk], updated in place */
  const float *node_states;             /* SELECT source, or NULL            */
  const float *node_u;                  /* UPDATE source, or NULL            */
  const void *x;                        /* conv input [n_total][C], NULL = no conv */
  void *prefix;                         /* [B][W-1][C], updated in place     */
} ddt_gdn_layer;

typedef struct ddt_attn_layer {
  const void *Kt, *Vt; /* [n_total][Hkv][D] draft keys / values */
  void *Kc, *Vc;       /* the layer's page pools                */
} ddt_attn_layer;

int ddt_commit_state(const ddt_plan *plan, const int32_t *path, const int32_t *L, int32_t mode,
                     const ddt_gdn_layer *gdn_layers, int32_t n_gdn, int32_t Hk, int32_t Hv,
                     int32_t dk, int32_t dv, int32_t gdn_dtype, int32_t C, int32_t conv_dtype,
                     const ddt_attn_layer *attn_layers, int32_t n_attn, int32_t Hkv, int32_t D,
                     int32_t kv_dtype, const int32_t *page_table, int32_t max_pages, int32_t *T,
                     void *stream);

/* ---------------------------------------------------------------------------
 * Fused linear-attention layer: tree conv -> SiLU -> split -> L2 norm ->
 * tree gated delta-net in one launch (the pages' single-dispatch forward,
 * lucebox-hub README, "01 · Megakernel", applied to the verify layers of
 * "02 · DFlash DDtree", "Implemented here"; the layer stage is the Gated
 * DeltaNet one: short conv with SiLU, L2-normalised q and k).
 *   y_n  = SiLU(tree conv of x over prefix ++ root path of n)   (as a2, act 1)
 *   y_n  = [q (Hk*dk) | k (Hk*dk) | v (Hv*dv)], head-major
 *   q, k <- x / sqrt(sum x^2 + 1e-6) per head;  v as is
 *   out  = the a3 rule on (q, k, v, alpha, beta) from S_c
 *   x         device [n_total][C], C = 2*Hk*dk + Hv*dv, dtype DDT_BF16 or
 *             DDT_F32, rows and base 16-byte aligned
 *   prefix    device [B][W-1][C] dtype, oldest first (read only; may be NULL
 *             when plan->W == 1);  w device [C][W] dtype, tap W-1 = current
 *   alpha, beta device [n_total][Hv] fp32 (gates)
 *   S_c       device [B][Hv][dv][dk] fp32, read only
 *   out       device [n_total][Hv][dv] fp32
 *   q_out, k_out device [n_total][Hk][dk] fp32 or NULL: the normalised q, k
 *             exactly as the kernel uses them (rounded to 16 significand
 *             bits, within 2^-16 of the normalised values plus one fp32 ulp
 *             of the reciprocal square root); the commit's
 *             UPDATE needs k, REPLAY q, k and v
 *   v_out     device [n_total][Hv][dv] fp32 or NULL: v after SiLU
 *   node_states, node_u  as for ddt_tree_gdn (node_u: the saved u for UPDATE)
 * A layer committed with DDT_COMMIT_UPDATE or SELECT takes k_out as its k,
 * the fp32 gates, and gdn_dtype DDT_F32; UPDATE and SELECT then give
 * bitwise the node state this call computes.  REPLAY (from q_out, k_out,
 * v_out) forms its products in fp32 and agrees within rounding only.
 * Same shape rules as ddt_tree_gdn, with Hv and dv at most 65535; the
 * workgroup's LDS, ddt_tree_conv_gdn_lds(n_max, dk) bytes, must fit in
 * 160 KiB (it does for every n_max <= 64 at dk <= 128).
 * Errors: DDT_E_ARG, DDT_E_SHAPE, DDT_E_DTYPE, plan errors; nothing is
 * launched then.
 */
size_t ddt_tree_conv_gdn_lds(int32_t n_max, int32_t dk);
int ddt_tree_conv_gdn(const ddt_plan *plan, const void *x, const void *prefix, const void *w, int32_t dtype,
                      const float *alpha, const float *beta, const float *S_c, int32_t Hk, int32_t Hv,
                      int32_t dk, int32_t dv, float scale, float *out, float *q_out, float *k_out,
                      float *v_out, float *node_states, float *node_u, void *stream);

/* ---------------------------------------------------------------------------
 * Ahead of the verify step: draft top-K / log-sum-exp and tree construction.
 *
 * ddt_draft_topk: the draft model's K most likely tokens (1 <= K <= 8) and
 * the log-sum-exp of every draft position, read from the draft logits on
 * the device (codehub lucebox-hub@main, "GPU draft top-K & verify-argmax
 * (DFlash)").
 *   logits      device, [B][L][V], DDT_BF16 or DDT_F32 (16-byte aligned rows
 *               use vector reads; any other layout is read element-wise).
 *   topk_idx    device out [B][L][K] int32: indices by descending logit,
 *               ties to the lower index; -1 past the row's finite logits.
 *   topk_logit  device out [B][L][K] float: their logits (-inf where -1).
 *   lse         device out [B][L] float: log-sum-exp of the finite logits
 *               (-inf if there are none).  NaN logits count as -inf.
 *   workspace   device, at least ddt_draft_topk_workspace(B, L, V, K)
 *               bytes, owned by the caller (0 for invalid sizes).
 * Errors: DDT_E_ARG (null pointer), DDT_E_SHAPE (B, L outside [1, 65535],
 * V outside [1, 1572864], K outside [1, 8]), DDT_E_DTYPE, DDT_E_WS; nothing
 * is launched then.
 *
 * ddt_tree_build: DDTree's budget-N tree from those candidates (lucebox-hub
 * README, "02 · DFlash DDtree", "Algorithms used"; the pages give no
 * selection rule).  Reading: a node at depth d has as candidate children
 * the top-K tokens of draft position d (0-based; the root, the last
 * committed token, has depth 0); log p = logit - lse; a node's score is the
 * sum of log p along its root path; the tree is the root plus the N-1 best
 * nodes under (score descending, then the candidate ranks along the path
 * lexicographically, a prefix before its extensions), numbered in that
 * order, so every parent precedes its children.  Scores are summed in fp32
 * root first.
 *   topk_idx, topk_logit, lse   device, as written by ddt_draft_topk: each
 *               row's entries by non-increasing logit, absent ones (-1)
 *               last; rows in another order give an unspecified tree.
 *   L           draft positions, 1..16;  K as above;  N budget 1..64.
 *   root_token  device [B] int32: the root's token (the last committed one).
 *   parent, tok device out [B][N] int32: tree b is rows b*N .. b*N+n-1, node
 *               ids local to the tree, parent[root] = -1; with every
 *               n_nodes[b] == N the arrays feed ddt_tree_plan directly with
 *               tree_off[b] = b*N.
 *   score       device out [B][N] float: node scores (0 for the root).
 *   n_nodes     device out [B] int32: nodes built (< N only when fewer
 *               candidates exist, e.g. K = 1 or positions without finite
 *               logits).
 * Errors: DDT_E_ARG, DDT_E_SHAPE; nothing is launched then.
 */
size_t ddt_draft_topk_workspace(int32_t B, int32_t L, int32_t V, int32_t K);
int ddt_draft_topk(const void *logits, int32_t B, int32_t L, int32_t V, int32_t dtype, int32_t K,
                   int32_t *topk_idx, float *topk_logit, float *lse, void *workspace, size_t ws_bytes,
                   void *stream);
int ddt_tree_build(const int32_t *topk_idx, const float *topk_logit, const float *lse, int32_t B, int32_t L,
                   int32_t K, int32_t N, const int32_t *root_token, int32_t *parent, int32_t *tok, float *score,
                   int32_t *n_nodes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DDTREE_H */
