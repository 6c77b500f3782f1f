/*
 * ddtree_oracle.c -- CPU oracle for draft-tree construction.
 *
 * TEST INFRASTRUCTURE. This is a plain, slow, obviously correct float64
 * implementation of what the draft-tree hot path computes. Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg load it. It
 * shares no source, header, table or helper with the HIP library, and the
 * HIP library never calls it.
 *
 * Sources (the pages; no line numbers):
 *  - SparklingTree post, section "Step 1: Sorting the DFlash marginals":
 *    per row, upcast the drafter logits, keep the top K = min(budget, V)
 *    tokens in sorted order and the row's log-sum-exp; the depth limit is
 *    the number of rows.
 *  - SparklingTree post, section "Step 3: The best-first heap algorithm",
 *    and the DDTree explainer, section 4 "Best-first heap algorithm
 *    (Algorithm 1)": prefixes are indexed by rank tuples; a max-heap seeded
 *    with the top-1 token at depth 1 pops the best prefix, emits it as the
 *    next tree node, and pushes its next sibling (last rank + 1) and its
 *    first child (append rank 0), until the budget is spent or the heap is
 *    empty.
 *  - SparklingTree post, section "Step 4: Creating the tree mask": each
 *    mask row is its parent's row plus the diagonal.
 *  - DDTree explainer, section 5 "Implementation highlights": the verifier
 *    walk follows, from the bonus token, the child whose token equals the
 *    target's choice, and returns the accepted path and a new bonus token.
 *
 * Readings where the pages leave a step open (each also listed in the
 * design notes):
 *  - Ties inside a row go to the lower token id; -0 equals +0.
 *  - Prefix score. With x_i the logits of row i and z_i = log sum_v
 *    exp(x_i[v]), a prefix rho of depth d scores
 *        raw(rho) = S(rho) - Z_d,   S = x_1[t_1] + ... + x_d[t_d],
 *        Z_d = z_1 + ... + z_d,
 *    both sums taken left to right in float64. Equal-probability prefixes of
 *    one depth then score exactly equal, whatever z's rounding. The score
 *    used for ordering is score(rho) = min(score(parent), raw(rho)) with the
 *    root at 0. Mathematically raw never exceeds the parent's score (every
 *    log-probability is <= 0); the min only pins down float64 rounding for
 *    rows whose normaliser equals their maximum to float64 precision.
 *  - Order. A prefix comes before another if its score is higher; on equal
 *    scores the lexicographically smaller rank tuple comes first, and a
 *    proper prefix comes before its extensions (the pages' heap entries are
 *    compared as (-score, rank tuple)).
 *  - Node numbering. Root is node 0; the j-th pop (0-based) is node j+1;
 *    parents[j] is the node number of its parent.
 *  - A budget above the number of prefixes ends when the heap empties; the
 *    tail is padded with token -1, parent -1, depth 0, log-prob -inf.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_BF16 0
#define OR_F32 1
#define OR_MAXL 64

int oracle_abi_version(void) { return 1; }

/* Exact float64 value of element idx of a bf16 (raw bits) or f32 array. */
static double value_at(const void* base, int dtype, size_t idx) {
  if (dtype == OR_BF16) {
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f == 0.0f ? 0.0 : (double)f;
  } else {
    float f = ((const float*)base)[idx];
    return f == 0.0f ? 0.0 : (double)f;
  }
}

/* Row normaliser z = log sum_v exp(x[v]) (Step 1's logsumexp), float64,
 * summed in index order after subtracting the row maximum. */
double oracle_row_lse(const void* row, int dtype, int64_t V) {
  double m = -INFINITY;
  for (int64_t v = 0; v < V; ++v) {
    double x = value_at(row, dtype, (size_t)v);
    if (x > m) m = x;
  }
  double s = 0.0;
  for (int64_t v = 0; v < V; ++v) s += exp(value_at(row, dtype, (size_t)v) - m);
  return m + log(s);
}

typedef struct {
  double x;
  int32_t id;
} ranked;

static int ranked_cmp(const void* pa, const void* pb) {
  const ranked* a = (const ranked*)pa;
  const ranked* b = (const ranked*)pb;
  if (a->x > b->x) return -1;
  if (a->x < b->x) return 1;
  return (a->id < b->id) ? -1 : (a->id > b->id);
}

/* Ranking (Step 1's topk): sort the whole row by (value desc, id asc) and
 * keep the first K. scratch must hold V entries. */
static void rank_row(const void* row, int dtype, int64_t V, int32_t K, ranked* scratch,
                     int32_t* ids, double* vals) {
  for (int64_t v = 0; v < V; ++v) {
    scratch[v].x = value_at(row, dtype, (size_t)v);
    scratch[v].id = (int32_t)v;
  }
  qsort(scratch, (size_t)V, sizeof(ranked), ranked_cmp);
  for (int32_t r = 0; r < K; ++r) {
    ids[r] = scratch[r].id;
    vals[r] = scratch[r].x;
  }
}

int oracle_row_rank(const void* row, int dtype, int64_t V, int32_t K, int32_t* ids,
                    double* vals) {
  if (!row || !ids || !vals || V <= 0 || K <= 0 || K > V) return -1;
  ranked* scratch = (ranked*)malloc(sizeof(ranked) * (size_t)V);
  if (!scratch) return -2;
  rank_row(row, dtype, V, K, scratch, ids, vals);
  free(scratch);
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Best-first heap over rank tuples (Algorithm 1).                         */

typedef struct {
  double score;     /* ordering score (see header) */
  double S;         /* float64 sum of the prefix's logits, left to right */
  double S_par;     /* the parent's S (0 for depth 1) */
  double score_par; /* the parent's score (0 for depth 1) */
  int32_t depth;    /* d >= 1 */
  int32_t parent;   /* node number of the parent, 0 = root */
  int32_t ranks[OR_MAXL];
} entry;

/* a pops before b */
static int before(const entry* a, const entry* b) {
  if (a->score > b->score) return 1;
  if (a->score < b->score) return 0;
  int n = a->depth < b->depth ? a->depth : b->depth;
  for (int i = 0; i < n; ++i)
    if (a->ranks[i] != b->ranks[i]) return a->ranks[i] < b->ranks[i];
  return a->depth < b->depth;
}

typedef struct {
  entry* e;
  int32_t n;
  int32_t cap;
  int32_t max_n;
} heap;

static void heap_push(heap* h, const entry* x) {
  int32_t i = h->n++;
  if (h->n > h->max_n) h->max_n = h->n;
  h->e[i] = *x;
  while (i > 0) {
    int32_t p = (i - 1) / 2;
    if (!before(&h->e[i], &h->e[p])) break;
    entry t = h->e[i];
    h->e[i] = h->e[p];
    h->e[p] = t;
    i = p;
  }
}

static void heap_pop(heap* h, entry* out) {
  *out = h->e[0];
  h->e[0] = h->e[--h->n];
  int32_t i = 0;
  for (;;) {
    int32_t l = 2 * i + 1, r = l + 1, m = i;
    if (l < h->n && before(&h->e[l], &h->e[m])) m = l;
    if (r < h->n && before(&h->e[r], &h->e[m])) m = r;
    if (m == i) break;
    entry t = h->e[i];
    h->e[i] = h->e[m];
    h->e[m] = t;
    i = m;
  }
}

/* Fill a heap entry for rank r at depth d below a parent with (S_par, score_par). */
static void make_entry(entry* e, const entry* par_or_null, int32_t d, int32_t r,
                       int32_t parent_node, const double* vals, int32_t K, const double* Z,
                       int32_t* clamps) {
  e->depth = d;
  e->parent = parent_node;
  if (par_or_null) {
    memcpy(e->ranks, par_or_null->ranks, sizeof(int32_t) * (size_t)(d - 1));
    e->S_par = par_or_null->S;
    e->score_par = par_or_null->score;
  } else {
    e->S_par = 0.0;
    e->score_par = 0.0;
  }
  e->ranks[d - 1] = r;
  e->S = e->S_par + vals[(size_t)(d - 1) * K + r];
  double raw = e->S - Z[d - 1];
  if (raw > e->score_par) {
    e->score = e->score_par;
    if (clamps) ++*clamps;
  } else {
    e->score = raw;
  }
}

/* Stage 2 for one request from its sorted top-K table (vals/ids [L][K],
 * row normalisers z[L]). Outputs as in oracle_build. */
int oracle_select(const double* vals, const int32_t* ids, const double* z, int32_t L,
                  int32_t K, int32_t B, int32_t* tree_tokens, int32_t* parents, float* logq,
                  int32_t* depths, int32_t* num_nodes, double* score64, double* next_score,
                  int32_t* max_heap, int32_t* clamps) {
  if (L <= 0 || L > OR_MAXL || K <= 0 || B <= 0) return -1;
  double Z[OR_MAXL];
  double acc = 0.0;
  for (int32_t d = 0; d < L; ++d) {
    acc += z[d];
    Z[d] = acc;
  }
  heap h;
  h.cap = 2 * B + 2;
  h.n = 0;
  h.max_n = 0;
  h.e = (entry*)malloc(sizeof(entry) * (size_t)h.cap);
  if (!h.e) return -2;
  int32_t nclamp = 0;

  entry first;
  make_entry(&first, NULL, 1, 0, 0, vals, K, Z, &nclamp);
  heap_push(&h, &first);

  int32_t count = 0;
  entry cur, nx;
  while (h.n > 0 && count < B) {
    heap_pop(&h, &cur);
    int32_t d = cur.depth, r = cur.ranks[d - 1];
    tree_tokens[count] = ids[(size_t)(d - 1) * K + r];
    parents[count] = cur.parent;
    depths[count] = d;
    logq[count] = (float)cur.score;
    if (score64) score64[count] = cur.score;
    int32_t node = count + 1;
    ++count;
    if (r + 1 < K) { /* next sibling: same parent, rank r+1 */
      entry par;
      par.S = cur.S_par;
      par.score = cur.score_par;
      memcpy(par.ranks, cur.ranks, sizeof(int32_t) * (size_t)(d - 1));
      make_entry(&nx, &par, d, r + 1, cur.parent, vals, K, Z, &nclamp);
      heap_push(&h, &nx);
    }
    if (d < L) { /* first child: append rank 0 */
      make_entry(&nx, &cur, d + 1, 0, node, vals, K, Z, &nclamp);
      heap_push(&h, &nx);
    }
  }
  *num_nodes = count;
  if (next_score) next_score[0] = h.n > 0 ? h.e[0].score : -INFINITY;
  for (int32_t j = count; j < B; ++j) {
    tree_tokens[j] = -1;
    parents[j] = -1;
    depths[j] = 0;
    logq[j] = -INFINITY;
    if (score64) score64[j] = -INFINITY;
  }
  if (max_heap) *max_heap = h.max_n;
  if (clamps) *clamps = nclamp;
  free(h.e);
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Whole build, threaded over requests (each request is independent).      */

typedef struct {
  const void* logits;
  int dtype;
  int64_t batch;
  int32_t L;
  int64_t V;
  int32_t B;
  int32_t* tree_tokens;
  int32_t* parents;
  float* logq;
  int32_t* depths;
  int32_t* num_nodes;
  double* score64;
  double* next_score;
  double* z_out;
  int32_t* top_ids;
  double* top_vals;
  int32_t* max_heap;
  int32_t* clamps;
  int nthreads;
  int tid;
  int status;
} build_job;

static void* build_worker(void* arg) {
  build_job* J = (build_job*)arg;
  const int32_t L = J->L, B = J->B;
  const int64_t V = J->V;
  const int32_t K = (int32_t)(B < V ? B : V);
  size_t esz = J->dtype == OR_BF16 ? 2 : 4;
  ranked* scratch = (ranked*)malloc(sizeof(ranked) * (size_t)V);
  double* vals = (double*)malloc(sizeof(double) * (size_t)L * K);
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)L * K);
  double* z = (double*)malloc(sizeof(double) * (size_t)L);
  if (!scratch || !vals || !ids || !z) {
    J->status = -2;
    free(scratch); free(vals); free(ids); free(z);
    return NULL;
  }
  for (int64_t b = J->tid; b < J->batch; b += J->nthreads) {
    for (int32_t d = 0; d < L; ++d) {
      const char* row = (const char*)J->logits + ((size_t)b * L + d) * (size_t)V * esz;
      z[d] = oracle_row_lse(row, J->dtype, V);
      rank_row(row, J->dtype, V, K, scratch, ids + (size_t)d * K, vals + (size_t)d * K);
    }
    if (J->z_out) memcpy(J->z_out + (size_t)b * L, z, sizeof(double) * (size_t)L);
    if (J->top_ids) memcpy(J->top_ids + (size_t)b * L * K, ids, sizeof(int32_t) * (size_t)L * K);
    if (J->top_vals) memcpy(J->top_vals + (size_t)b * L * K, vals, sizeof(double) * (size_t)L * K);
    int rc = oracle_select(vals, ids, z, L, K, B, J->tree_tokens + (size_t)b * B,
                           J->parents + (size_t)b * B, J->logq + (size_t)b * B,
                           J->depths + (size_t)b * B, J->num_nodes + b,
                           J->score64 ? J->score64 + (size_t)b * B : NULL,
                           J->next_score ? J->next_score + b : NULL,
                           J->max_heap ? J->max_heap + b : NULL,
                           J->clamps ? J->clamps + b : NULL);
    if (rc) J->status = rc;
  }
  free(scratch); free(vals); free(ids); free(z);
  return NULL;
}

int oracle_build(const void* logits, int dtype, int64_t batch, int32_t L, int64_t V, int32_t B,
                 int32_t* tree_tokens, int32_t* parents, float* logq, int32_t* depths,
                 int32_t* num_nodes, double* score64, double* next_score, double* z_out,
                 int32_t* top_ids, double* top_vals, int32_t* max_heap, int32_t* clamps,
                 int nthreads) {
  if (!logits || !tree_tokens || !parents || !logq || !depths || !num_nodes) return -1;
  if ((dtype != OR_BF16 && dtype != OR_F32) || batch < 0 || L <= 0 || L > OR_MAXL || V <= 0 ||
      B <= 0)
    return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (batch == 0) return 0;
  if (nthreads > batch) nthreads = (int)batch;
  build_job jobs[256];
  pthread_t th[256];
  for (int t = 0; t < nthreads; ++t) {
    build_job j = {logits, dtype, batch, L, V, B, tree_tokens, parents, logq, depths,
                   num_nodes, score64, next_score, z_out, top_ids, top_vals, max_heap,
                   clamps, nthreads, t, 0};
    jobs[t] = j;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, build_worker, &jobs[t]);
  build_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  for (int t = 0; t < nthreads; ++t)
    if (jobs[t].status) return jobs[t].status;
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Stage 3: ancestor-only visibility mask (Step 4), packed LSB-first.       */

int oracle_mask(const int32_t* parents, const int32_t* num_nodes, int64_t batch, int32_t B,
                uint64_t* mask) {
  if (!parents || !num_nodes || !mask || batch < 0 || B <= 0) return -1;
  const int32_t N = B + 1;
  const int32_t W = (N + 63) / 64;
  unsigned char* vis = (unsigned char*)malloc((size_t)N * N);
  if (!vis) return -2;
  for (int64_t b = 0; b < batch; ++b) {
    int32_t n = num_nodes[b];
    if (n < 0 || n > B) { free(vis); return -1; }
    memset(vis, 0, (size_t)N * N);
    vis[0] = 1;
    for (int32_t i = 1; i <= n; ++i) {
      int32_t p = parents[(size_t)b * B + (i - 1)];
      if (p < 0 || p >= i) { free(vis); return -1; }
      memcpy(vis + (size_t)i * N, vis + (size_t)p * N, (size_t)i);
      vis[(size_t)i * N + i] = 1;
    }
    uint64_t* mb = mask + (size_t)b * N * W;
    memset(mb, 0, sizeof(uint64_t) * (size_t)N * W);
    for (int32_t i = 0; i < N; ++i)
      for (int32_t j = 0; j < N; ++j)
        if (vis[(size_t)i * N + j]) mb[(size_t)i * W + j / 64] |= (uint64_t)1 << (j % 64);
  }
  free(vis);
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Stage 4: greedy verifier walk.                                           */

int oracle_accept(const int32_t* tree_tokens, const int32_t* parents, const int32_t* num_nodes,
                  const int32_t* target_tokens, int64_t batch, int32_t B, int32_t L,
                  int32_t* accepted_nodes, int32_t* accept_len, int32_t* next_token) {
  if (!tree_tokens || !parents || !num_nodes || !target_tokens || !accepted_nodes ||
      !accept_len || !next_token || batch < 0 || B <= 0 || L <= 0)
    return -1;
  for (int64_t b = 0; b < batch; ++b) {
    const int32_t* tok = tree_tokens + (size_t)b * B;
    const int32_t* par = parents + (size_t)b * B;
    const int32_t* tgt = target_tokens + (size_t)b * (B + 1);
    int32_t n = num_nodes[b];
    int32_t cur = 0, len = 0;
    for (;;) {
      int32_t want = tgt[cur], found = -1;
      for (int32_t j = 0; j < n; ++j)
        if (par[j] == cur && tok[j] == want) { found = j + 1; break; }
      if (found < 0 || len >= L) break;
      accepted_nodes[(size_t)b * L + len] = found;
      ++len;
      cur = found;
    }
    for (int32_t i = len; i < L; ++i) accepted_nodes[(size_t)b * L + i] = -1;
    accept_len[b] = len;
    next_token[b] = tgt[cur];
  }
  return 0;
}
