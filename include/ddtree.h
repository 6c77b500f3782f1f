/*
 * ddtree.h -- C ABI of libddtree.so: draft-tree construction on MI355X (gfx950).
 *
 * The library turns a block drafter's per-position logits into the draft
 * tree that DDTree verifies in one target pass, and walks the verified tree.
 * Operations and where the pages define them:
 *
 *  - ddtree_build: the tree of the B most probable draft prefixes under the
 *    drafter's factorised distribution. DDTree explainer ("DDTree Explained:
 *    From Block Diffusion to Optimal Diffusion Draft Trees"), section 2
 *    (objective), section 3 (Proposition 2: the top-B prefixes form the
 *    optimal tree; Lemma 1: the top K = min(B, V) tokens per position
 *    suffice) and section 5 (build_tree returns the tree's tokens and
 *    parent indices); SparklingTree post, sections "Step 1" (per-row top-K
 *    and log-sum-exp) and "Step 3" (best-first order of the nodes).
 *  - ddtree_mask: the ancestor-only attention mask. SparklingTree post,
 *    section "Step 4: Creating the tree mask"; DDTree explainer, section 5.
 *  - ddtree_accept: the greedy verifier walk. DDTree explainer, section 5;
 *    TreeSpark README, item 4 (argmax-following acceptance walk).
 *  - ddtree_row_topk: stage 1 alone (row log-sum-exp and sorted top-K).
 *  - treespark_expand: TreeSpark's parent-conditioned tree. TreeSpark README,
 *    item 1 (z_d(u) = l_d + W e(t_u), branching k over depths, global top-N
 *    packing) and item 2 (per-parent top-k expansion, joint path-score
 *    frontier pruning, global top-N packing).
 *    SparklingTree post, section "Step 1".
 *  - sparkling_build: SparklingTree's conditioned best-first tree.
 *    SparklingTree post, sections "Building SparklingTree" (top-C pre-filter
 *    of every drafter row, low-rank first-order Markov head) and "Solving
 *    the candidate tree construction" (the head looks back one token, so the
 *    deltas between consecutive rows' candidates form a table computed up
 *    front; best-first growth on the conditioned rows).
 *  - sparkling_beam: a fixed-branching beam tree on SparklingTree's rows.
 *    SparklingTree post, section "Future Ideas", item 4.
 *  - dspark_budget: DSpark's survival-ranked verification budget. DSpark
 *    explainer, section "Hardware aware prefix scheduler"; DSpark guide,
 *    sections "Survival probability" and "Picking the budget".
 *  - ddtree_select: stage 2 alone, from stage 1's tables. DDTree explainer,
 *    sections 3-4; SparklingTree post, section "Step 3".
 *    ddtree_build = ddtree_row_topk + ddtree_select in one call.
 *
 * Conventions shared by every call:
 *  - Device pointers. Every array argument is device memory owned by the
 *    caller; the library never allocates, frees or retains memory.
 *  - Streams. Work is enqueued on `stream` (a hipStream_t; NULL is the null
 *    stream) and runs asynchronously. Outputs are valid once the stream has
 *    reached that point. No call synchronises with the host.
 *  - Errors. Arguments are checked on the host before anything is enqueued:
 *    DDT_EINVAL for null pointers or bad sizes, DDT_ENOTSUP for sizes outside
 *    the supported region, DDT_EWORKSPACE for a workspace that is too small;
 *    nothing is enqueued then. DDT_EHIP reports a failed launch. Device-side
 *    contents (token ids, parent indices) are not validated.
 *  - Layouts are row-major and contiguous. Node numbering: node 0 is the
 *    root (the bonus token, which is not an output); node j+1 is the j-th
 *    emitted node, and nodes are emitted in best-first order, so a parent
 *    always precedes its children.
 *  - Threading: the library keeps no state; concurrent calls need separate
 *    workspaces.
 */
#ifndef DDTREE_H
#define DDTREE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DDT_OK = 0,
  DDT_EINVAL = -1,     /* null pointer or invalid size */
  DDT_ENOTSUP = -2,    /* valid but outside the supported region */
  DDT_EWORKSPACE = -3, /* workspace smaller than the matching *_workspace_size() */
  DDT_EHIP = -4        /* a HIP launch failed */
};

enum { DDT_BF16 = 0, DDT_F32 = 1 };

/* Supported region. */
#define DDT_MAX_B 512   /* node budget */
#define DDT_MAX_L 32    /* draft positions (tree depth) */
#define DDT_MAX_LK 8192 /* L * min(B, V) */

int ddt_abi_version(void);
const char* ddt_status_string(int status);

/*
 * Workspace. ddtree_build and ddtree_row_topk need a device scratch buffer of
 * at least the size the matching *_workspace_size() returns. Its contents on
 * entry are ignored: every record a launch reads was written earlier in the
 * same call, so an abandoned or failed call leaves nothing behind that a
 * later call depends on. A workspace must not be used by two calls that can
 * run concurrently (two streams, or two host threads on one stream without
 * ordering): they would overwrite each other's records.
 */
size_t ddtree_build_workspace_size(int64_t batch, int32_t L, int64_t V, int32_t B, int dtype);
size_t ddtree_row_topk_workspace_size(int64_t rows, int64_t V, int32_t K, int dtype);

/*
 * ddtree_build -- stages 1 and 2 (and optionally 3) for a batch of requests.
 *
 * logits       [batch][L][V] drafter logits, bf16 (DDT_BF16) or float32
 *              (DDT_F32), 16-byte aligned (DDT_EINVAL otherwise). Row d of a
 *              request is draft position d+1. Finite values of magnitude
 *              below 2^22 only (the normaliser's exponent arguments are
 *              float32; beyond that its offset can fall short by one
 *              float32 unit of x * log2(e), and the result is undefined).
 * B            node budget, 1 <= B <= DDT_MAX_B. K = min(B, V) tokens per
 *              row are ranked; 1 <= L <= DDT_MAX_L; L*K <= DDT_MAX_LK; and
 *              L * ceil(log2 K) <= 122.
 * Outputs, per request b:
 *  tree_tokens [batch][B] int32  token of node j+1;
 *  parents     [batch][B] int32  node number of node j+1's parent (0 = root);
 *  logq        [batch][B] float  node's prefix log-probability;
 *  depths      [batch][B] int32  node depth 1..L (may be NULL);
 *  num_nodes   [batch]    int32  number of nodes emitted, min(B, number of
 *              prefixes of length <= L over the top-K tokens);
 *  mask        [batch][B+1][ceil((B+1)/64)] uint64 or NULL: the ancestor
 *              mask of ddtree_mask, written by the same launch.
 *  Entries j >= num_nodes hold token -1, parent -1, depth 0, logq -inf.
 *
 * Node selection. With z_d the log-sum-exp of row d and x_d[t] the logit of
 * token t, a prefix (t_1..t_d) scores S - Z with S = x_1[t_1] + ... +
 * x_d[t_d] and Z = z_1 + ... + z_d (float64, left to right), capped at its
 * parent's score. The emitted nodes are the B highest-scoring prefixes; ties
 * go to the lexicographically smaller tuple of per-row ranks (a prefix before
 * its extensions), and tokens of equal logit within a row rank by lower id.
 * The row normalisers are computed in float32/float64 on the device, so
 * prefixes of different depths whose scores differ by less than about 1e-6
 * may order differently than in exact arithmetic.
 */
int ddtree_build(const void* logits, int dtype, int64_t batch, int32_t L, int64_t V, int32_t B,
                 int32_t* tree_tokens, int32_t* parents, float* logq, int32_t* depths,
                 int32_t* num_nodes, uint64_t* mask, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/*
 * ddtree_build_noalloc -- ddtree_build without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Arguments and
 * outputs as ddtree_build. The scratch space is a static 16 MiB device array
 * of the library (one per GPU, held until the process ends), so no call
 * allocates anything. Shapes whose ddtree_build_workspace_size() exceeds
 * 16 MiB return DDT_ENOTSUP before anything is enqueued (the batch-256,
 * B = 256 workload needs 7.5 MiB). Every call on one GPU shares that GPU's
 * array: calls that can overlap on one GPU (two streams, or two host threads)
 * race and give undefined results. No kernel reads scratch it did not write
 * in the same call, so nothing needs clearing between calls. DDT_EHIP if the
 * array's device address cannot be obtained.
 */
int ddtree_build_noalloc(const void* logits, int dtype, int64_t batch, int32_t L, int64_t V,
                         int32_t B, int32_t* tree_tokens, int32_t* parents, float* logq,
                         int32_t* depths, int32_t* num_nodes, uint64_t* mask,
                         hipStream_t stream);

/*
 * ddtree_select -- stage 2 alone (plus the optional fused mask): the tree of
 * ddtree_build from per-row tables, e.g. those of ddtree_row_topk.
 * vals [batch][L][K] float and ids [batch][L][K] int32: each row's K largest
 *      logits in descending order (equal values by ascending id) and their
 *      token ids; lse [batch][L] double: the rows' log-sum-exp.
 * 1 <= K <= DDT_MAX_B, L*K <= DDT_MAX_LK, L * ceil(log2 K) <= 122; with
 * K = min(B, V) the result equals ddtree_build's (Lemma 1). Outputs and
 * selection rule as in ddtree_build.
 */
int ddtree_select(const float* vals, const int32_t* ids, const double* lse, int64_t batch,
                  int32_t L, int32_t K, int32_t B, int32_t* tree_tokens, int32_t* parents,
                  float* logq, int32_t* depths, int32_t* num_nodes, uint64_t* mask,
                  hipStream_t stream);

/*
 * ddtree_mask -- stage 3. Row i of request b has bit j (word j/64, bit j%64,
 * LSB first) set iff node j is node i or one of its ancestors; node 0 (the
 * root) is visible to every node. Rows i > num_nodes[b] are zero.
 * parents   [batch][B] int32, as written by ddtree_build (parents[j] <= j);
 * num_nodes [batch] int32 in [0, B];
 * mask      [batch][B+1][ceil((B+1)/64)] uint64 output.
 */
int ddtree_mask(const int32_t* parents, const int32_t* num_nodes, int64_t batch, int32_t B,
                uint64_t* mask, hipStream_t stream);

/*
 * ddtree_accept -- stage 4, the greedy walk. From the root, repeatedly move to
 * the child whose token equals the target's choice at the current node, until
 * no child matches. Siblings carry distinct tokens, so the walk is unique.
 * target_tokens  [batch][B+1] int32: the target's argmax at each node
 *                (index 0 = root);
 * accepted_nodes [batch][L] int32: node numbers along the accepted path,
 *                padded with -1;
 * accept_len     [batch] int32: number of accepted draft tokens;
 * next_token     [batch] int32: the target's token at the last accepted node
 *                (the new bonus token). Committed tokens = accept_len + 1.
 */
int ddtree_accept(const int32_t* tree_tokens, const int32_t* parents, const int32_t* num_nodes,
                  const int32_t* target_tokens, int64_t batch, int32_t B, int32_t L,
                  int32_t* accepted_nodes, int32_t* accept_len, int32_t* next_token,
                  hipStream_t stream);

/*
 * ddtree_compact_kv -- KV-cache compaction to the accepted path (DDTree
 * explainer, section 5, "KV cache management": after each round only the
 * accepted path's cache is kept). The verification pass wrote the rows of
 * the root (the bonus token) and of nodes 1..B at positions past_len[b] + j.
 * For every layer and KV head, rows past_len[b] + i, i = 1..accept_len[b],
 * take the rows at past_len[b] + accepted_nodes[b][i-1]; every other row is
 * left as it was. In place; the caches are not reallocated.
 * k_cache, v_cache [layers][batch][heads][cap][row_bytes] (row_bytes = head
 *                  dim x element size; any element type, copied bit for bit),
 *                  16-byte aligned;
 * past_len       [batch] int32: cache length before the verified block;
 * accepted_nodes [batch][L], accept_len [batch]: as written by ddtree_accept
 *                (node numbers increase along the path, a_i >= i);
 * new_len        [batch] int32 output (nullable): past_len + accept_len + 1.
 * Supported: row_bytes a multiple of 16 and <= 1024, 1 <= L <= DDT_MAX_L;
 * otherwise DDT_ENOTSUP. Device contents are not validated beyond skipping
 * rows whose source or destination falls outside [0, cap).
 */
int ddtree_compact_kv(void* k_cache, void* v_cache, int64_t layers, int64_t batch,
                      int32_t heads, int64_t cap, int32_t row_bytes, const int32_t* past_len,
                      const int32_t* accepted_nodes, const int32_t* accept_len, int32_t L,
                      int32_t* new_len, hipStream_t stream);

/*
 * ddtree_row_topk -- stage 1 alone over `rows` independent rows of length V
 * (logits as in ddtree_build: 16-byte aligned, finite).
 * ids  [rows][K] int32 and vals [rows][K] float: the K largest logits of each
 *      row in descending order, equal values by ascending id (-0 equals +0);
 *      vals are the exact input values.
 * lse  [rows] double: log sum_v exp(x[v]); per-element exponentials in
 *      float32, sums combined in float64 (absolute error ~1e-6).
 * 1 <= K <= min(V, DDT_MAX_B).
 */
int ddtree_row_topk(const void* logits, int dtype, int64_t rows, int64_t V, int32_t K,
                    int32_t* ids, float* vals, double* lse, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * treespark_expand -- TreeSpark's parent-conditioned expansion (TreeSpark
 * README, items 1-2). For request b with anchor token a_b (the root, score
 * 0) and depths d = 1..D: every frontier parent u (token t_u) gets
 *   z = backbone[b][d-1] + W . E[t_u]          (over the whole vocabulary)
 * and its top k = min(k, V) tokens by (z desc, id asc) become children
 * scored score(u) + z[t] - logsumexp(z), rank tuple = u's + (j). The frontier
 * of depth d+1 is the best F children of depth d; after depth D the best N
 * of all candidates are packed. Order: score desc, then rank tuple
 * lexicographic asc (a prefix before its extensions).
 * backbone [batch][D][V] bf16 backbone logits; W, E [V][H] bf16 (head weight
 *          and embedding table, 16-byte aligned); anchor [batch] int32 in
 *          [0, V) (not validated on the device).
 * Outputs [batch][N]: tree_tokens, parents (packed position of the parent,
 *          0 = the anchor), logq (float path log-prob), depths (nullable);
 *          num_nodes [batch] = min(N, candidates); the tail is padded with
 *          -1, -1, -inf, 0. ddtree_mask builds the mask from parents.
 * z accumulates in float32 (bf16 MFMA), log-sum-exp combines in float64.
 * Supported: 1 <= D <= 16, 1 <= k <= 8, 1 <= F <= 8, 1 <= N <= 4096,
 * H a positive multiple of 64, V < 2^31, V * H * 2 < 2^32 (the embedding
 * table is addressed with 32-bit byte offsets); otherwise DDT_ENOTSUP.
 * The workspace (treespark_workspace_size bytes, no zero-fill needed) holds
 * per-depth partial records and the candidates.
 */
size_t treespark_workspace_size(int64_t batch, int32_t D, int64_t V, int32_t H, int32_t k,
                                int32_t F, int32_t N);
int treespark_expand(const void* backbone, const void* W, const void* E, const int32_t* anchor,
                     int64_t batch, int32_t D, int64_t V, int32_t H, int32_t k, int32_t F,
                     int32_t N, int32_t* tree_tokens, int32_t* parents, float* logq,
                     int32_t* depths, int32_t* num_nodes, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * sparkling_build -- SparklingTree's conditioned best-first tree (SparklingTree
 * post, "Building SparklingTree" and "Solving the candidate tree
 * construction"). For request b with drafter rows x_1..x_L (logits [b][d][:]):
 *  1. c_d = the top C tokens of x_d by (value desc, id asc) (the pre-filter);
 *  2. row 1 (children of the root): lp_j = x_1[c_1j] - logsumexp over the C
 *     candidates (depth 1 is not conditioned);
 *     row d >= 2 for a parent holding candidate token p of depth d-1:
 *     s_j = x_d[c_dj] + W1[p] . W2t[c_dj] (the rank-R Markov head,
 *     W1 [V][R] extraction, W2t [V][R] projection transposed), lp_j = s_j -
 *     logsumexp(s) over the C candidates; children order by (lp desc, id asc);
 *  3. the B best prefixes, score = sum of lp along the path (float64 left to
 *     right from float32 lp), ordered by (score desc, rank tuple lexicographic
 *     asc, a prefix before its extensions) -- the order of the post's
 *     best-first heap (pop, push the best child and the next sibling).
 * logits [batch][L][V], dtype DDT_BF16 or DDT_F32, 16-byte aligned;
 * W1, W2t [V][R] bf16, 16-byte aligned; token ids < V come from step 1.
 * Outputs as ddtree_build ([batch][B] tree_tokens, parents, logq, depths
 * (nullable); num_nodes [batch] = min(B, prefixes); mask [batch][B+1][W]
 * (nullable), W = ceil((B+1)/64)); the tail is padded with -1, -1, -inf, 0.
 * The Markov dot products accumulate bf16 products in float32 (MFMA); row
 * normalisation is float32; path scores are float64.
 * Supported: 1 <= C <= min(128, V), R a multiple of 64 up to 256,
 * 1 <= L <= DDT_MAX_L, B <= DDT_MAX_B, L * ceil(log2 C) <= 122, V < 2^31;
 * otherwise DDT_ENOTSUP (C > V: DDT_EINVAL).
 * The workspace (sparkling_build_workspace_size bytes, no zero-fill needed)
 * holds the top-C tables and the conditioned rows ([batch][L-1][C][C] float
 * log-probs, each row's best child); 0 means unsupported sizes.
 */
size_t sparkling_build_workspace_size(int64_t batch, int32_t L, int64_t V, int32_t C,
                                      int32_t R, int32_t B, int dtype);
int sparkling_build(const void* logits, int dtype, const uint16_t* W1, const uint16_t* W2t,
                    int64_t batch, int32_t L, int64_t V, int32_t C, int32_t R, int32_t B,
                    int32_t* tree_tokens, int32_t* parents, float* logq, int32_t* depths,
                    int32_t* num_nodes, uint64_t* mask, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * dspark_budget -- DSpark's hardware-aware prefix scheduler (DSpark explainer,
 * "Hardware aware prefix scheduler"; DSpark guide, "Survival probability",
 * "Picking the budget"). For the R = batch active requests with block
 * confidences conf[b][p] (the chance guess p survives if every earlier one
 * did; clamped into [0, 1], NaN as 0):
 *   survival[b][p] = conf[b][0] * ... * conf[b][p] (float64, left to right);
 *   every slot ranks by survival desc, then request asc, then position asc;
 *   keeping the first n slots costs cost_ms[R + n] (one target step over
 *   R + n tokens: each request's last token plus its kept guesses) and is
 *   expected to yield R + (sum of the kept survivals) tokens;
 *   n = the count maximising expected tokens / cost over n = 0..min(R*P,
 *   n_cost-1-R) (the smallest such n among equal maxima).
 * conf [batch][P] float, cost_ms [n_cost] float (positive; n_cost > batch),
 * both device memory.
 * Outputs: keep [batch] int32 (each request keeps the first keep[b] guesses
 * of its block), n_keep [1] int32 = n, survival [batch][P] float64
 * (nullable), expected_tokens [1] float64 (nullable), objective [1] float64
 * expected tokens per ms (nullable).
 * The scan of expected tokens sums in a tree order: within about 1e-15
 * relative of a sequential sum, so n can differ from a sequential
 * evaluation only between counts whose objectives agree that closely.
 * Supported: batch * P <= 4096 (DDT_ENOTSUP otherwise). One workgroup; no
 * workspace.
 */
int dspark_budget(const float* conf, int64_t batch, int32_t P, const float* cost_ms,
                  int32_t n_cost, int32_t* keep, double* survival, int32_t* n_keep,
                  double* expected_tokens, double* objective, hipStream_t stream);

/*
 * sparkling_beam -- a fixed-branching beam tree on SparklingTree's conditioned
 * rows (SparklingTree post, "Future Ideas", item 4: a beam with a fixed
 * branching budget in place of the best-first heap; evenly spread branches).
 * Rows as sparkling_build (top C candidates per row, the rank-R Markov head,
 * log-probs over the C candidates). widths [L] is a HOST array, or NULL for
 * the evenly spread schedule of `budget` nodes: floor(budget / L) per depth,
 * one more on the first budget mod L depths. With widths given, budget must
 * be 0 or their sum (DDT_EINVAL otherwise). Depth 1 keeps
 * the widths[0] best children of the root; depth d+1 the widths[d] best of all
 * children of depth d's beam; best = score (sum of lp along the path,
 * float64) desc, then rank tuple lexicographic asc (a child's rank = its
 * position in its row by lp desc, token asc). A width above the number of
 * candidates keeps them all; a zero width ends the tree.
 * Nodes are emitted depth by depth, each depth in beam order: node j+1 is the
 * j-th, parents[j] its parent's node number (0 = the root).
 * Outputs [batch][B] with B = sum of widths (tree_tokens, parents, logq,
 * depths nullable), num_nodes [batch], mask [batch][B+1][ceil((B+1)/64)]
 * (nullable); the tail is padded with -1, -1, -inf, 0.
 * Supported: each width <= 64, B <= DDT_MAX_B, and sparkling_build's limits
 * on C, R, L and V (DDT_ENOTSUP); a negative width or B = 0: DDT_EINVAL.
 * Workspace: sparkling_build_workspace_size(batch, L, V, C, R, B, dtype) bytes.
 */
/*
 * ddtree_read_probe -- measurement probe: the practical read ceiling of stage
 * 1 (SparklingTree post, "Step 1": every drafter row is read once). Streams
 * rows x row_bytes bytes from src (device, 16-byte aligned, row_bytes a
 * multiple of 16) with stage 1's launch geometry and load path (one
 * 256-thread workgroup per row, nontemporal 16-byte buffer loads, double
 * buffered) and computes nothing but an XOR of the words, written to
 * sink[rows][4] (device uint32, one word per wave) so the loads stay live.
 * Its rate is what the stage-1 kernel's bandwidth is reported against.
 * DDT_EINVAL for null or misaligned pointers and bad sizes; DDT_ENOTSUP for
 * rows or row_bytes above 2^31 - 1.
 */
int ddtree_read_probe(const void* src, int64_t rows, int64_t row_bytes, uint32_t* sink,
                      hipStream_t stream);

/*
 * ddtree_ts_load_probe -- measurement probe: the loads of one TreeSpark head
 * evaluation (TreeSpark README, item 1: z_d(u) = l_d + W . e(t_u) streams the
 * head weight W once per depth while every vocabulary tile re-reads its
 * parents' embedding rows) with nothing computed. W and E: device bf16
 * [V][H], 16-byte aligned, H a multiple of 64; ptok: device int32 [128]
 * parent tokens (each < V; a token past the table reads zeros); sink:
 * device uint32 [256], written only on an impossible XOR value (the loads
 * stay live). Launch geometry, LDS ring, wait and barrier per step are
 * ts_gemm_kernel's. variant: 0 W alone (nontemporal), 1 W + the parents'
 * rows 16 bytes of 32 rows per instruction (the MFMA B layout), 2 W + the
 * rows as whole 128-byte lines, 3 as 2 with W at system-scope nontemporal,
 * 4 W alone at system-scope nontemporal, 5 as 2 for only the first 16
 * parents of each 32 (half the rows' traffic), 6 as 2 with 256-row tiles
 * (eight waves, one workgroup per CU, each pair of waves sharing its 32
 * parents' lines: half the rows' traffic per W byte), 7 as 6 with one
 * persistent workgroup per CU streaming its tiles as one step sequence.
 * DDT_EINVAL for null or misaligned
 * pointers, bad sizes or variants; DDT_ENOTSUP for V x H x 2 >= 4 GiB.
 */
int ddtree_ts_load_probe(const void* W, const void* E, const int32_t* ptok, int64_t V, int32_t H,
                         int32_t variant, uint32_t* sink, hipStream_t stream);

int sparkling_beam(const void* logits, int dtype, const uint16_t* W1, const uint16_t* W2t,
                   int64_t batch, int32_t L, int64_t V, int32_t C, int32_t R,
                   const int32_t* widths, int32_t budget, int32_t* tree_tokens,
                   int32_t* parents, float* logq,
                   int32_t* depths, int32_t* num_nodes, uint64_t* mask, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DDTREE_H */
