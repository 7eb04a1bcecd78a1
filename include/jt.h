/*
 * jt.h -- C ABI of the tree speculative-decoding verify step on AMD MI355X
 * (gfx950).  Each operation is a thin host entry point that validates its
 * arguments and enqueues HIP kernels on the caller's stream:
 *
 *   jt_build_tree      candidate tree from the draft's per-depth logits
 *   jt_tree_meta       per-node ancestor bitmasks (the tree-causal mask)
 *   jt_tree_attention  paged tree-causal attention of every tree node
 *   jt_accept          greedy acceptance of the longest matching path
 *   jt_accept_margin   acceptance under a probability-ratio margin
 *   jt_commit_kv       move the accepted path's K/V next to the prefix
 *   jt_accept_stochastic  lossless verification at temperature T > 0
 *                      (top-W siblings, or children sampled from the draft)
 *   jt_build_tree_variant  tree build under the alternative expansions and
 *                      priorities (node-block, entropy / mixed)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is DEVICE memory unless marked [host].  The caller
 *   allocates and owns all buffers, including the workspace; the library
 *   allocates nothing and keeps no mutable global state, so calls are
 *   re-entrant and thread-safe.  Calls that share a workspace buffer must be
 *   ordered on one stream.
 * - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *   stream).  Every call only enqueues work and returns; nothing synchronises
 *   with the host.  Per-sequence counts (n_nodes, prefix_len) stay on the
 *   device and are read there.
 * - Host-side argument checks run before anything is enqueued.  A call that
 *   returns anything but JT_OK has enqueued nothing and written nothing.
 *   JT_ERR_LAUNCH means a kernel launch itself failed (the stream state is then
 *   whatever HIP reports).
 * - Invalid DEVICE data (which the host cannot see) is reported through the
 *   optional `err` word: kernels atomically OR the JT_DERR_* bits below into
 *   *err and skip the offending item without reading out of bounds.  Outputs
 *   of a skipped item are unspecified.  Pass NULL to skip error reporting.
 * - Layouts are dense, row-major, in the order the brackets give.
 * - Node numbering: node 0 is the root (the last accepted token).  Drafted
 *   nodes 1..n_nodes-1 are numbered in best-first pop order, so
 *   parent[j] < j for every j >= 1 and parent[0] = -1.  A tree of budget B
 *   has at most max_nodes = B + 1 nodes.
 */
#ifndef JT_H
#define JT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every enum below also lists its type's full int32 range (the _RANGE_
 * members are never valid arguments): any int a caller passes is then a
 * value of the type, which the library rejects with JT_ERR_INVALID_ARG,
 * rather than an out-of-range enum value that C++ leaves undefined. */
typedef enum {
  JT_STATUS_RANGE_MIN_ = INT32_MIN,
  JT_OK = 0,
  JT_ERR_INVALID_ARG = 1,  /* a null pointer, a negative or inconsistent size */
  JT_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels implement    */
  JT_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than the query says    */
  JT_ERR_LAUNCH = 4,       /* a HIP kernel launch failed                       */
  JT_ERR_SCRATCH = 5,      /* inputs exceed jt_accept_noalloc's static scratch */
  JT_STATUS_RANGE_MAX_ = INT32_MAX
} jt_status;

typedef enum {
  JT_DTYPE_RANGE_MIN_ = INT32_MIN,
  JT_F32 = 0,
  JT_BF16 = 1,
  JT_DTYPE_RANGE_MAX_ = INT32_MAX
} jt_dtype;

/* Tree expansion of jt_build_tree_variant. */
typedef enum {
  JT_EXPAND_RANGE_MIN_ = INT32_MIN,
  JT_EXPAND_CANDIDATE = 0,
  JT_EXPAND_NODE_BLOCK = 1,
  JT_EXPAND_RANGE_MAX_ = INT32_MAX
} jt_expand;

/* How the drafted tokens of a tree were proposed (jt_accept_stochastic). */
typedef enum {
  JT_DRAFT_RANGE_MIN_ = INT32_MIN,
  JT_DRAFT_TOPW = 0,    /* siblings are distinct chosen tokens (jt_build_tree's top-W) */
  JT_DRAFT_SAMPLED = 1, /* every child drawn i.i.d. from softmax(draft row / T)        */
  JT_DRAFT_RANGE_MAX_ = INT32_MAX
} jt_draft_mode;

/* Device error bits (OR-ed into *err). */
#define JT_DERR_BAD_LOGIT 1   /* NaN or +inf logit, or a draft row without a finite entry */
#define JT_DERR_BAD_PARENT 2  /* parent[0] != -1, or parent[j] outside [0, j)              */
#define JT_DERR_BAD_NNODES 4  /* n_nodes outside [1, max_nodes]                             */
#define JT_DERR_BAD_PAGE 8    /* a page id outside [0, num_pages)                           */
#define JT_DERR_BAD_PREFIX 16 /* prefix_len < 0, or prefix_len + n_nodes > pages * 16       */
#define JT_DERR_BAD_DEPTH 32  /* depth[j] != depth[parent[j]] + 1, or deeper than depth_n   */
#define JT_DERR_BAD_TOKEN 64  /* a token id outside [0, vocab)                              */
#define JT_DERR_BAD_PATH 128  /* accept_len outside [0, depth_n], or accept_nodes not a     */
                              /* strictly increasing list of node ids in [1, n_nodes)       */
#define JT_DERR_BAD_UNIFORM 256 /* a uniform draw outside [0, 1) (or NaN)                   */

/* [host] Static, NUL-terminated description of a status code. */
const char* jt_status_string(jt_status s);

/* [host] Library ABI version (major * 100 + minor). */
int jt_version(void);

/* ------------------------------------------------------------------------
 * jt_build_tree -- per-depth top-W candidates, then best-first expansion.
 *
 * Defined by the JetSpec news piece (mlqm.cn/news/158889), paragraph on
 * building the candidate tree (depth N, width W, budget B; top-W per depth;
 * greedy expansion by cumulative draft log-probability until the budget is
 * full) and the JetSpec explainer (techwalker.com, "加速AI思考…"), section 五
 * (priority queue of candidate nodes keyed by the path's cumulative
 * log-probability, at most W children per popped node, stop at B nodes).
 *
 * Readings fixed here (the pages state no tie rules and no arithmetic):
 *  - The drafter's logits are per depth: row d-1 of a sequence holds depth d,
 *    and every depth-d node's children are the same top-W tokens of that row
 *    (logit descending, then token id ascending).
 *  - One queue pop adds one candidate (parent node, rank) to the tree; a
 *    popped node shallower than N then offers its W children.  Pops stop after
 *    B nodes or when no candidate is left, so
 *    n_nodes = 1 + min(B, W + W^2 + ... + W^N).
 *  - score(v) = raw(v) - S_depth(v), where raw is the fp64 sum of the fp32
 *    logits along the path (root to node), S_d = lse_1 + ... + lse_d (fp64,
 *    added in depth order) and lse_d the fp64 log-sum-exp of row d.
 *  - Queue order: score descending, then parent node index ascending, then
 *    candidate rank ascending.
 * The per-depth log-sum-exp is an fp64 reduction whose summation order
 * differs from a sequential one in the last bits, so two candidates of
 * different depths whose scores are within ~1e-13 may be ordered differently
 * from a sequential fp64 implementation; parent/token/depth are otherwise an
 * exact function of the inputs.
 *
 *   draft_logits  [batch, depth_n, vocab]   dt = JT_F32 or JT_BF16.  Entries
 *                                            must be finite or -inf; each row
 *                                            needs one finite entry.
 *   root_token    [batch] int32             token of node 0.
 *   parent, token, depth  [batch, budget_b + 1] int32 (out).  Rows past
 *                                            n_nodes hold -1.
 *   score         [batch, budget_b + 1] f64 (out, nullable); -inf padded.
 *   n_nodes       [batch] int32 (out).
 *   err           int32 (nullable): JT_DERR_BAD_LOGIT.
 * Limits: batch >= 0, 1 <= depth_n <= 64, 1 <= width_w <= min(vocab, 16),
 * 0 <= budget_b <= 1023, vocab >= 1; the per-sequence selection state must
 * fit one workgroup's LDS (JT_ERR_UNSUPPORTED otherwise; fine for N=16, B=256,
 * W=8).
 * ---------------------------------------------------------------------- */
size_t jt_build_tree_workspace(int batch, int depth_n, int vocab, int width_w, int budget_b);
jt_status jt_build_tree(const void* draft_logits, jt_dtype dt, int batch, int depth_n,
                        int vocab, int width_w, int budget_b, const int32_t* root_token,
                        int32_t* parent, int32_t* token, int32_t* depth, double* score,
                        int32_t* n_nodes, int32_t* err, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * jt_build_tree_variant -- the tree build under the alternative expansion and
 * priority rules.
 *
 * JetSpec explainer (techwalker.com), section 五: a priority queue whose best
 * entry is popped and given up to W children until B nodes are placed; the
 * same section compares the cumulative log-probability priority with the
 * per-position entropy and with weighted mixes of the two.
 *
 * Priority, with a = entropy_weight in [0, 1]:
 *   key = (1 - a) * score - a * H_d     (a == 1: key = -H_d)
 * where score is the cumulative draft log-probability (as jt_build_tree) and
 * H_d = -sum p log p of softmax(draft row d) (fp64, nats) for the depth d of
 * the node being ranked (lower entropy ranks higher).  The key is evaluated
 * in fp64 without fused multiply-adds.
 * expand_mode:
 *   JT_EXPAND_CANDIDATE   the queue holds candidates (placed node, rank); a
 *                         pop places one node; ties go to the lower parent
 *                         index, then the lower rank.  With a = 0 the result
 *                         equals jt_build_tree.
 *   JT_EXPAND_NODE_BLOCK  the queue holds placed nodes shallower than N (the
 *                         root first); a pop attaches all W children of that
 *                         node (rank order, consecutive node indices), cut
 *                         short at B; ties go to the lower node index.
 * Candidates, node numbering (parent[j] < j), outputs, err bits, workspace
 * (jt_build_tree_workspace) and limits are those of jt_build_tree, except that
 * no LDS limit applies.  The per-depth lse and entropy are fp64 reductions in
 * another order than a sequential one: priorities that differ by ~1e-13 may
 * be ordered differently from a sequential fp64 implementation.
 * One workgroup per sequence runs the B pops one after another (a workgroup
 * argmax each); jt_build_tree remains the fast path for the default rule.
 *   entropy_weight  in [0, 1] (JT_ERR_INVALID_ARG otherwise, NaN included).
 * ---------------------------------------------------------------------- */
jt_status jt_build_tree_variant(const void* draft_logits, jt_dtype dt, int batch, int depth_n,
                                int vocab, int width_w, int budget_b, jt_expand expand_mode,
                                double entropy_weight, const int32_t* root_token,
                                int32_t* parent, int32_t* token, int32_t* depth, double* score,
                                int32_t* n_nodes, int32_t* err, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * jt_tree_meta -- ancestor-or-self bitmasks of every node.
 *
 * The tree-causal rule: a node attends to the prefix and to the nodes of its
 * own root-to-node branch -- never to siblings' branches or to descendants
 * (JetSpec news piece, paragraph on the one-forward solution and the
 * tree-causal attention mask; explainer section 三).  Self-visibility is this
 * library's reading.
 *
 *   parent    [batch, max_nodes] int32      parent[0] = -1, parent[j] in [0, j).
 *   n_nodes   [batch] int32                 1 <= n_nodes <= max_nodes.
 *   anc_mask  [batch, max_nodes, ceil(max_nodes / 32)] uint32 (out):
 *             bit (j % 32) of word j / 32 of row i is set iff node j is i or
 *             an ancestor of i.  Rows >= n_nodes are zero.
 *   err       JT_DERR_BAD_PARENT, JT_DERR_BAD_NNODES (that sequence's rows are
 *             then all zero).
 * Limits: batch >= 0, 1 <= max_nodes <= 1024.
 * ---------------------------------------------------------------------- */
jt_status jt_tree_meta(const int32_t* parent, const int32_t* n_nodes, int batch, int max_nodes,
                       uint32_t* anc_mask, int32_t* err, void* stream);

/* ------------------------------------------------------------------------
 * jt_tree_attention -- paged tree-causal attention, one pass over the tree.
 *
 * For sequence s, node i < n_nodes[s] and query head h (KV head
 * g = h / (num_q_heads / num_kv_heads)): the visible keys are the prefix
 * positions t < P = prefix_len[s] and the tree-tail positions P + j for every
 * j set in anc_mask row i.  o = softmax(scale * q.k over visible keys) @ v,
 * lse = natural log of the softmax normaliser.  JetSpec explainer section 七
 * (paged tree attention: tree mask staged on chip, tree-tail masking, no dense
 * mask), section 三 (all candidate paths verified in one target forward).
 *
 *   q         [batch, max_nodes, num_q_heads, head_dim]  dt (RoPE already
 *             applied by the caller).
 *   k_pool, v_pool [num_pages, num_kv_heads, page_size, head_dim]  dt.
 *             Logical position t of sequence s lives in page
 *             page_table[s, t / page_size], slot t % page_size.  The tree tail:
 *             node j's K/V are at position P + j (node-index order) and must be
 *             finite; slots at or past P + n_nodes are never used (they may
 *             hold anything, NaN included).
 *   n_nodes, prefix_len [batch] int32.
 *   page_table [batch, max_pages_per_seq] int32; entries past
 *             ceil((P + n_nodes) / page_size) are not read.
 *   anc_mask  as written by jt_tree_meta for the same max_nodes.
 *   scale     > 0 and finite (e.g. 1/sqrt(head_dim) if q is unscaled).
 *   out       [batch, max_nodes, num_q_heads, head_dim]  dt (out); rows
 *             >= n_nodes are not written.
 *   lse       [batch, max_nodes, num_q_heads] f32 (out, nullable).
 *   err       JT_DERR_BAD_NNODES, JT_DERR_BAD_PREFIX (sequence skipped),
 *             JT_DERR_BAD_PAGE (that page's keys read as zero).
 * Arithmetic: bf16 inputs use bf16 MFMA with fp32 accumulation, probabilities
 * rounded to bf16 for the PV product, output rounded to bf16.  Rows whose keys
 * are split over several workgroups are merged from normalised partial rows
 * kept in the workspace in fp16 (relative rounding 2^-11, finer than the bf16
 * output) with fp32 log-sum-exps.  f32 inputs are computed in fp32
 * throughout.
 * Limits: head_dim in {64, 128}, page_size == 16, num_q_heads a multiple of
 * num_kv_heads with num_q_heads / num_kv_heads <= 16, 1 <= max_nodes <= 1024,
 * max_pages_per_seq >= 1, num_pages >= 1.
 * ---------------------------------------------------------------------- */
size_t jt_tree_attention_workspace(int batch, int max_nodes, int num_q_heads, int num_kv_heads,
                                   int head_dim, int max_pages_per_seq, int page_size,
                                   jt_dtype dt);
jt_status jt_tree_attention(const void* q, const void* k_pool, const void* v_pool, jt_dtype dt,
                            int batch, int max_nodes, int num_q_heads, int num_kv_heads,
                            int head_dim, const int32_t* n_nodes, const int32_t* prefix_len,
                            const int32_t* page_table, int max_pages_per_seq, int num_pages,
                            int page_size, const uint32_t* anc_mask, float scale, void* out,
                            float* lse, int32_t* err, void* workspace, size_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------------------
 * jt_accept -- greedy acceptance of the longest consistent path.
 *
 * Row r of a sequence's target logits is the target's next-token prediction
 * after node r; a_r = its argmax (ties to the lowest token id).  The root is
 * accepted; node v >= 1 is accepted iff its parent is accepted and
 * token[v] == a_{parent[v]}.  The path ends at the deepest accepted node
 * (lowest index among equals).  JetSpec news piece (the target verifies the
 * tree and keeps the longest consistent prefix under the SD acceptance rule);
 * explainer section 三; SD overview (chooseai.io/news/6515), section on when
 * lossless decoding fails (temperature 0: a draft token is accepted only if
 * it equals the target's choice).
 *
 *   target_logits [batch, max_nodes, vocab]  dt; rows >= n_nodes not read.
 *   parent, token, depth [batch, max_nodes] int32 (as from jt_build_tree).
 *   n_nodes   [batch] int32.
 *   accept_len   [batch] int32 (out): depth of the deepest accepted node.
 *   accept_nodes [batch, depth_n] int32 (out): node indices of the accepted
 *                path (root excluded), -1 padded.
 *   bonus_token  [batch] int32 (out): a at the deepest accepted node.
 *   err       JT_DERR_BAD_LOGIT (NaN), JT_DERR_BAD_NNODES, JT_DERR_BAD_PARENT,
 *             JT_DERR_BAD_DEPTH (that sequence's outputs are then zero / -1).
 * Limits: batch >= 0, 1 <= max_nodes <= 1024, vocab >= 1, 1 <= depth_n <= 64.
 * ---------------------------------------------------------------------- */
size_t jt_accept_workspace(int batch, int max_nodes, int vocab);
jt_status jt_accept(const void* target_logits, jt_dtype dt, int batch, int max_nodes, int vocab,
                    int depth_n, const int32_t* parent, const int32_t* token,
                    const int32_t* depth, const int32_t* n_nodes, int32_t* accept_len,
                    int32_t* accept_nodes, int32_t* bonus_token, int32_t* err, void* workspace,
                    size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * jt_accept_noalloc -- jt_accept for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).
 *
 * Same arguments, outputs, rule and error bits as jt_accept, without the
 * workspace: the argmax partials (8 bytes per (row, vocabulary chunk)) live
 * in a static device array of JT_ACCEPT_SCRATCH_BYTES that each GPU the
 * library runs on holds until the process ends.  The call allocates nothing
 * (no hipMalloc / hipFree); its first call on a device looks up that
 * device's copy of the array.  Inputs whose partials need more than the
 * array (jt_accept_workspace(batch, max_nodes, vocab) > the limit, e.g.
 * batch * max_nodes above about 64K rows) return JT_ERR_SCRATCH before
 * anything is enqueued.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (concurrent streams or host threads) race
 * and must be ordered by the caller.  Nothing in the array needs clearing
 * between calls (every partial read is written first by the same call).
 * ---------------------------------------------------------------------- */
#define JT_ACCEPT_SCRATCH_BYTES (4u << 20)
jt_status jt_accept_noalloc(const void* target_logits, jt_dtype dt, int batch, int max_nodes,
                            int vocab, int depth_n, const int32_t* parent, const int32_t* token,
                            const int32_t* depth, const int32_t* n_nodes, int32_t* accept_len,
                            int32_t* accept_nodes, int32_t* bonus_token, int32_t* err,
                            void* stream);

/* ------------------------------------------------------------------------
 * jt_accept_margin -- acceptance under the per-step margin rule.
 *
 * AdaptiveSpec page (kongchang.com, "AdaptiveSpec：免训练推测解码方案提速56%的
 * 技术解析"), section on the per-step margin rule: a drafted token is kept when
 * the target's probability of it divided by the target's top-1 probability
 * reaches a threshold theta, even when it is not the top-1 token (the page's
 * example keeps a token at 0.30 against a top-1 at 0.35 with theta = 0.8).
 * With p = softmax(L / T) that ratio is exp((L[x] - max L) / T), so the rule is
 * L[x] - max L >= T * ln(theta); the library forms that logit margin on the
 * host in fp64.
 *
 * Same arguments, outputs and walk as jt_accept, except the per-node test:
 * node v >= 1 is accepted iff its parent is accepted and
 *   (double)L[parent(v)][token[v]] - (double)max_x L[parent(v)][x]
 *       >= temperature * log(theta)
 * evaluated in fp64 on the stored logit values.  Several siblings may pass;
 * the path ends at the deepest accepted node (lowest index among equals) and
 * bonus_token is the argmax (lowest id) of that node's row.
 *   theta        in (0, 1] (1 keeps only tokens tied with the maximum).
 *   temperature  > 0 and finite.
 *   err          as jt_accept, plus JT_DERR_BAD_TOKEN (a token id outside
 *                [0, vocab): that sequence's outputs are then zero / -1).
 * ---------------------------------------------------------------------- */
jt_status jt_accept_margin(const void* target_logits, jt_dtype dt, int batch, int max_nodes,
                           int vocab, int depth_n, const int32_t* parent, const int32_t* token,
                           const int32_t* depth, const int32_t* n_nodes, double theta,
                           double temperature, int32_t* accept_len, int32_t* accept_nodes,
                           int32_t* bonus_token, int32_t* err, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * jt_commit_kv -- commit the accepted path to the KV cache.
 *
 * After acceptance the next decode step starts from the accepted state
 * (JetSpec news piece, mlqm.cn/news/158889, tree-construction paragraph).
 * With the tree tail at positions P + j (jt_tree_attention), the k-th accepted
 * node a_k (k = 1..accept_len, depth order, as jt_accept writes them) moves
 * from position P + a_k to P + k in every KV head of both pools; the root
 * (position P) and positions past P + accept_len are not written; then
 * prefix_len += 1 + accept_len (root plus accepted nodes).  All source rows of
 * a sequence are read before any row is written, so overlapping sources and
 * destinations are fine.  Afterwards, decode attention of node a_L over the
 * new prefix equals its tree attention before the commit.
 *
 *   k_pool, v_pool  [num_pages, num_kv_heads, page_size, head_dim]  dt (in/out).
 *   page_table      [batch, max_pages_per_seq] int32 (as jt_tree_attention).
 *                   Tail pages must not be shared between sequences.
 *   n_nodes         [batch] int32 (the tree's node count).
 *   parent          [batch, max_nodes] int32 (nullable): the tree's parent
 *                   array; when given, accept_nodes must also be the chain
 *                   root -> a_1 -> ... -> a_L (parent[a_1] = 0,
 *                   parent[a_k] = a_{k-1}).
 *   accept_len      [batch] int32; accept_nodes [batch, depth_n] int32 (as
 *                   from jt_accept / jt_accept_margin).
 *   prefix_len      [batch] int32 (in/out).
 *   err             JT_DERR_BAD_PATH (accept_len outside [0, min(depth_n,
 *                   n_nodes - 1)], accept_nodes not strictly increasing in
 *                   [1, n_nodes) or, with parent, not a root-to-node chain,
 *                   n_nodes or prefix_len invalid), JT_DERR_BAD_PAGE (a page
 *                   id of a moved row's source or destination outside
 *                   [0, num_pages)).  Such a sequence is left unchanged: its
 *                   pools and its prefix_len are not written.
 * Limits: page_size == 16, head_dim * element size a multiple of 16 bytes,
 * 1 <= depth_n <= 64 with 2 * depth_n * head_dim * element size <= 64 KiB,
 * 1 <= max_nodes <= 1024.
 * ---------------------------------------------------------------------- */
jt_status jt_commit_kv(void* k_pool, void* v_pool, jt_dtype dt, int batch, int num_kv_heads,
                       int head_dim, const int32_t* page_table, int max_pages_per_seq,
                       int num_pages, int page_size, const int32_t* n_nodes,
                       const int32_t* parent, int max_nodes, int depth_n,
                       const int32_t* accept_len, const int32_t* accept_nodes,
                       int32_t* prefix_len, int32_t* err, void* stream);

/* ------------------------------------------------------------------------
 * jt_accept_stochastic -- lossless verification at temperature T > 0.
 *
 * Single-token rule (SD overview, chooseai.io/news/6515, section on what
 * speculative decoding is; AdaptiveSpec page, kongchang.com, section on the
 * strict token-matching rule): with draft distribution q and target
 * distribution p, a drafted token x is accepted with probability
 * min(1, p(x) / q(x)); on rejection the next token is drawn from
 * norm(max(0, p - q)), which leaves the output distributed as the target's
 * provided x was proposed from q.  The proposal is named by draft_mode:
 *
 *  JT_DRAFT_TOPW     the siblings are chosen tokens, as jt_build_tree makes
 *                    them (the top-W draft tokens of each depth: JetSpec news
 *                    piece, tree-construction paragraph; explainer section
 *                    五).  Each sibling's proposal is the point mass on its
 *                    token, so x is accepted with probability p(x) and a
 *                    rejection removes x from p and renormalises.  The output
 *                    follows the target distribution for any fixed tree.
 *                    draft_logits is not read (may be NULL).
 *  JT_DRAFT_SAMPLED  every child of a node was drawn independently from
 *                    q = softmax(draft row of its depth / T): x is accepted
 *                    iff u * q(x) < p(x) and a rejection sets
 *                    p = norm(max(0, p - q)) with the same q for the next
 *                    sibling.  Lossless only under that sampling assumption;
 *                    on jt_build_tree's deterministic siblings it is NOT.
 *
 * Tree walk (the pages state the rule for one token):
 *  - p at node u = softmax(target row u / T).
 *  - Starting at the root, the current node's children are tried in node-index
 *    order: child v (token x) is accepted iff u_accept[v] < p(x) (TOPW) or
 *    u_accept[v] * q(x) < p(x) (SAMPLED), p being the current distribution;
 *    a rejection replaces p by its residual and the next child is tried; if
 *    that residual has no mass the remaining children are skipped and p stays
 *    as it was.  An accepted child becomes the current node.
 *  - When no child is accepted the walk stops; bonus_token is the smallest
 *    y with sum_{i <= y} p(i) > u_sample * sum_i p(i) (index order).
 * Arithmetic: fp64 on the stored logit values (exp of the device math
 * library); different summation orders from a sequential fp64 reference only
 * move decisions whose margin is at the rounding level (~1e-13 relative).
 *
 *   target_logits [batch, max_nodes, vocab]  dt; rows >= n_nodes not read.
 *   draft_logits  [batch, depth_n, vocab]    dt (row d-1 = depth d); SAMPLED
 *                 only.
 *   parent, token, depth, n_nodes   as jt_accept.
 *   temperature   > 0 and finite.
 *   u_accept  [batch, max_nodes] f32: uniform in [0, 1) per node (entry 0 and
 *             entries >= n_nodes are not read).
 *   u_sample  [batch] f32: uniform in [0, 1).
 *   accept_len, accept_nodes, bonus_token  (out) as jt_accept.
 *   err       JT_DERR_BAD_LOGIT (NaN / +inf, or a row with no finite entry),
 *             JT_DERR_BAD_NNODES, JT_DERR_BAD_PARENT, JT_DERR_BAD_DEPTH,
 *             JT_DERR_BAD_TOKEN, JT_DERR_BAD_UNIFORM (that sequence's outputs
 *             are then zero / -1).
 *   workspace  jt_accept_stochastic_workspace(batch, vocab) bytes (2 * vocab
 *             doubles per sequence: the exponentials of the current target
 *             row and, SAMPLED, of the children's draft row; then 20 bytes per
 *             4096-entry chunk of the root's target row and the depth-1 draft
 *             row, whose statistics are computed up front).  TOPW writes
 *             zeros into the cached target row for rejected tokens.
 * Limits: batch >= 0, 1 <= max_nodes <= 1024, vocab >= 1, 1 <= depth_n <= 64.
 * Two short pre-pass kernels over every sequence's first rows, then one
 * workgroup per sequence for the walk.
 * ---------------------------------------------------------------------- */
size_t jt_accept_stochastic_workspace(int batch, int vocab);
jt_status jt_accept_stochastic(const void* target_logits, const void* draft_logits, jt_dtype dt,
                               int batch, int max_nodes, int vocab, int depth_n,
                               const int32_t* parent, const int32_t* token, const int32_t* depth,
                               const int32_t* n_nodes, float temperature,
                               jt_draft_mode draft_mode, const float* u_accept,
                               const float* u_sample, int32_t* accept_len, int32_t* accept_nodes,
                               int32_t* bonus_token, int32_t* err, void* workspace,
                               size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* JT_H */
