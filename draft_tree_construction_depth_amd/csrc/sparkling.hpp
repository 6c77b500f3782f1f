// SparklingTree: conditioned best-first tree from a diffusion drafter's rows
// and a first-order Markov head.
//
// SparklingTree post, "Building SparklingTree" and "Solving the candidate
// tree construction": every drafter row is cut to its top C tokens on the
// device; a low-rank Markov head biases row d by the token chosen at depth
// d-1, delta(p, v) = W1[p] . W2[:, v] (extraction W1 [V][R], projection W2
// [R][V], held transposed as W2t [V][R]); because the head looks back one
// token, the whole table of deltas between consecutive rows' candidates is
// computed up front, and the tree grows best first on conditioned rows.
// Readings (the post leaves them open): depth 1 is not conditioned; a row's
// log-probs are normalised over its C candidates; ties inside a row go to
// the lower token id, prefixes order by (score desc, rank tuple asc).
//
// sp_table_kernel: per request and child row d >= 1, one workgroup forms
//   delta[i][j] = W1[c_{d-1}[i]] . W2t[c_d[j]] for all C x C candidate pairs
//   on MFMA (32x32x16 bf16, float32 accumulate; the child rows of W2t are
//   the A operand, staged in LDS, each wave holds 32 parent rows of W1 as
//   the B operand in registers), so that each lane ends up with half of one
//   parent's row: s_j = x_d[c_j] + delta[i][j], its maximum, sum of
//   exponentials and best child (lp desc, token asc) reduce in registers and
//   one exchange between the two lanes of a parent. lp_j = s_j -
//   logsumexp(s) goes out through an LDS tile as whole 16-byte rows.
//   Rows stay in candidate order: the selection reads them unsorted.
// The selection itself is sp_select_kernel, below.
#pragma once

#include "common.hpp"
#include "select.hpp"
#include "treespark.hpp"  // MFMA fragment types

namespace ddt {

constexpr int kSpThreads = 256;
constexpr int kSpC = 128;     // candidates per row, at most (MFMA tiles of 32)
constexpr int kSpRMax = 256;  // Markov rank, at most (four k-steps of 64 in registers)
constexpr int kSpKT = 64;
constexpr int kSpPitch = kSpRMax + 8;  // bf16 row pitch of the staged W2t rows
constexpr int kSpTile = 132;           // float row pitch of the staged log-prob tile
// With L * ceil(log2 C) <= 122 bits of rank key and C <= 128, L * C <= 17 * 128.
constexpr int kSpMaxLC = 17 * kSpC;

struct SpTableParams {
  const uint16_t* W1;   // [V][R] bf16
  const uint16_t* W2t;  // [V][R] bf16
  const int32_t* ids;   // [batch][L][C] each row's candidate tokens (value desc, id asc)
  const float* vals;    // [batch][L][C] their logits
  int32_t L, C, R;
  float* lp;            // [batch][L-1][C][C]: child row d, parent candidate i, child candidate j
  uint8_t* best;        // [batch][L-1][C]: the best child j of each parent row
  float* blp;           // [batch][L-1][C]: its log-prob
};

// 16-byte aligned so that the fragment reads and the row stores are single
// 16-byte LDS instructions.
struct alignas(16) SpTableSmem {
  union {
    uint16_t w2[kSpC][kSpPitch];  // the child candidates' W2t rows (MFMA A operand)
    float tile[kSpC][kSpTile];    // then the finished log-prob rows
  } u;
  float vals[kSpC];
  int32_t tok[kSpC];
};
static_assert(sizeof(float) * kSpTile == sizeof(uint16_t) * kSpPitch, "tile overlays the rows");

__device__ __forceinline__ bool sp_better(float a, int ta, float b, int tb) {
  return a > b || (a == b && ta < tb);
}

__global__ __launch_bounds__(kSpThreads) void sp_table_kernel(SpTableParams p) {
  __shared__ SpTableSmem sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5;
  const int64_t b = blockIdx.x;
  const int d = blockIdx.y + 1;  // child row
  const int C = p.C, R = p.R, L = p.L;
  const int32_t* pid = p.ids + ((size_t)b * L + d - 1) * C;  // parent candidates
  const int32_t* cid = p.ids + ((size_t)b * L + d) * C;      // child candidates
  // every load in flight before the first wait: this lane's parent row (B
  // operand: parent 32 w + l % 32, k-chunks 8 (l / 32) of each 16), then its
  // share of the child rows (16-byte chunks; half a wave covers one row of
  // 256 bf16)
  const int i = 32 * w + (l & 31);
  const int ptok = pid[i < C ? i : 0];
  const uint16_t* brow = p.W1 + (size_t)ptok * R + 8 * h;
  const int nks = R / kSpKT;
  u32x4 bq[kSpRMax / kSpKT][4];
#pragma unroll
  for (int ks = 0; ks < kSpRMax / kSpKT; ++ks)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      bq[ks][s] = ks < nks ? *(const u32x4*)(brow + ks * kSpKT + 16 * s) : u32x4{0u, 0u, 0u, 0u};
  const int cpr = R >> 3;  // 16-byte chunks per row
  constexpr int kStage = kSpC * (kSpRMax / 8) / kSpThreads;
  u32x4 st[kStage];
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int q = tid + k * kSpThreads;
    const int j = q / cpr, ch = q - j * cpr;
    st[k] = u32x4{0u, 0u, 0u, 0u};
    if (j < C) st[k] = *(const u32x4*)(p.W2t + (size_t)cid[j] * R + 8 * ch);
  }
  if (tid < kSpC) {
    sm.vals[tid] = tid < C ? p.vals[((size_t)b * L + d) * C + tid] : -INFINITY;
    sm.tok[tid] = tid < C ? cid[tid] : 0x7FFFFFFF;
  }
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int q = tid + k * kSpThreads;
    const int j = q / cpr, ch = q - j * cpr;
    if (j < kSpC) *(u32x4*)&sm.u.w2[j][8 * ch] = st[k];
  }
  __syncthreads();
  // acc[m][r] = delta of child 32 m + 8 (r / 4) + 4 (l / 32) + r % 4 for
  // parent 32 w + l % 32
  f32x16 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < kSpRMax / kSpKT; ++ks) {
    if (ks < nks) {
      // the step's A fragments read before its MFMAs
      u32x4 araw[4][4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          araw[s][m] = *(const u32x4*)&sm.u.w2[m * 32 + (l & 31)][ks * kSpKT + 16 * s + 8 * h];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, bq[ks][s]);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, araw[s][m]),
                                                           bv, acc[m], 0, 0, 0);
      }
    }
  }
  // epilogue: this lane's 64 children of parent i, the other 64 in lane l ^ 32
  float mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = m * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      acc[m][r] = j < C ? acc[m][r] + sm.vals[j] : -INFINITY;
      mx = fmaxf(mx, acc[m][r]);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float sum = 0.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[m][r] == -INFINITY ? 0.0f : __expf(acc[m][r] - mx);
  sum += __shfl_xor(sum, 32);
  const float lse = mx + __logf(sum);
  float bv = -INFINITY;
  int bt = 0x7FFFFFFF, bj = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = m * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      const float v = acc[m][r] - lse;
      acc[m][r] = v;
      if (j < C && sp_better(v, sm.tok[j], bv, bt)) {
        bv = v;
        bt = sm.tok[j];
        bj = j;
      }
    }
  {
    const float ov = __shfl_xor(bv, 32);
    const int ot = __shfl_xor(bt, 32), oj = __shfl_xor(bj, 32);
    if (sp_better(ov, ot, bv, bt)) {
      bv = ov;
      bt = ot;
      bj = oj;
    }
  }
  const size_t rowbase = ((size_t)b * (L - 1) + (d - 1)) * C;
  if (h == 0 && i < C) {
    p.best[rowbase + i] = (uint8_t)bj;
    p.blp[rowbase + i] = bv;
  }
  float* dst = p.lp + rowbase * C;  // C rows of C floats, contiguous
  if (C == kSpC) {
    // full tiles: each lane's four consecutive children go out as one
    // 16-byte store (the two lanes of a parent cover 32 contiguous bytes)
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float4 v4;
        v4.x = acc[m][4 * rq + 0];
        v4.y = acc[m][4 * rq + 1];
        v4.z = acc[m][4 * rq + 2];
        v4.w = acc[m][4 * rq + 3];
        *(float4*)(dst + (size_t)i * C + m * 32 + 8 * rq + 4 * h) = v4;
      }
    return;
  }
  __syncthreads();  // every wave has read its A operands: the rows become the tile
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      float4 v4;
      v4.x = acc[m][4 * rq + 0];
      v4.y = acc[m][4 * rq + 1];
      v4.z = acc[m][4 * rq + 2];
      v4.w = acc[m][4 * rq + 3];
      *(float4*)&sm.u.tile[i][m * 32 + 8 * rq + 4 * h] = v4;
    }
  __syncthreads();
  if ((C & 3) == 0) {
    const int cq = C >> 2;  // 16-byte chunks per row
    for (int q = tid; q < C * cq; q += kSpThreads) {
      const int r = q / cq, c4 = q - r * cq;
      *(float4*)(dst + (size_t)r * C + 4 * c4) = *(const float4*)&sm.u.tile[r][4 * c4];
    }
  } else {
    for (int q = tid; q < C * C; q += kSpThreads) {
      const int r = q / C, c = q - r * C;
      dst[(size_t)r * C + c] = sm.u.tile[r][c];
    }
  }
}

// ---------------------------------------------------------------------------
// Selection on conditioned rows: select_kernel's method (an exact threshold
// from the one-deviation prefixes, enumeration of E = {score >= tau} by
// chains, histogram ordering, emission, mask) with a row per (depth, parent
// token) instead of per depth. A node's children live in the row of its
// candidate at the next depth (row 0, the first drafter row renormalised
// over its candidates, for the root); rows are read from global memory in
// candidate order, the best child of every row comes from LDS tables, so a
// chain (rank-0 extensions) is walked without memory waits. Entries carry
// their candidate index in eRank (ranks live in the lexicographic keys).

struct SpTabs {                  // overlays the row-value table (unused here)
  float lp0[kSpC];               // row 0: first drafter row over its candidates
  int32_t spine[kMaxL];          // the spine's candidate at each depth
  int32_t best0;                 // row 0's best candidate (lp desc, token asc)
  int32_t tok[kSpMaxLC];         // [L][C] candidate tokens
  uint8_t best[kSpMaxLC];        // best child of (child row d >= 1, parent candidate)
  float blp[kSpMaxLC];
};
static_assert(sizeof(SpTabs) <= sizeof(float) * kMaxLK, "conditioned tables fit the row table");
static_assert(kSpMaxLC <= kMergeCap, "one-deviation scores fit a merge buffer");

// Conditioned rows of request b: row(d, c) = log-probs of the children at
// depth index d (0-based) of a node holding candidate c at depth index d-1.
struct SpRows {
  const SpTabs* tb;
  const float* lp;     // [L-1][C][C]
  const int32_t* tok;  // [L][C] candidate tokens (LDS)
  int C;
  __device__ const float* row(int d, int c) const {
    return d == 0 ? tb->lp0 : lp + ((size_t)(d - 1) * C + c) * C;
  }
  __device__ int best(int d, int c) const { return d == 0 ? tb->best0 : tb->best[(d - 1) * C + c]; }
  __device__ float best_lp(int d, int c) const {
    return d == 0 ? tb->lp0[tb->best0] : tb->blp[(d - 1) * C + c];
  }
};

// Serial best-first heap (the post's loop) for requests whose enumeration
// overflows: the next sibling is the best child of the row ordered after
// the current one.
__device__ void sp_heap_fallback(const SelectParams& p, SelectSmem& sm, int64_t b, const SpRows& R) {
  SelHeap& h = sm.u.hp;
  const int L = p.L, C = p.K, B = p.B;
  int pool = 0, hn = 0, count = 0;
  // the child of row (d, pc) ordered right after (v, t) (any child when t < 0)
  auto next_after = [&](int d, int pc, float v, int t) -> int {
    const float* r = R.row(d, pc);
    const int32_t* tk = R.tok + (size_t)d * C;
    int bj = -1;
    for (int q = 0; q < C; ++q) {
      const bool after = t < 0 || r[q] < v || (r[q] == v && tk[q] > t);
      if (after && (bj < 0 || r[q] > r[bj] || (r[q] == r[bj] && tk[q] < tk[bj]))) bj = q;
    }
    return bj;
  };
  auto make = [&](int src, double Spar, int d, int rk, int parent_node, int pc, int j) -> int {
    const int e = pool++;
    for (int i = 0; i < d - 1; ++i) h.ranks[e][i] = h.ranks[src][i];
    h.ranks[e][d - 1] = (uint16_t)rk;
    h.dep[e] = (uint8_t)d;
    h.parent[e] = (int16_t)parent_node;
    h.Spar[e] = Spar;
    h.S[e] = Spar + (double)R.row(d - 1, pc)[j];
    h.sc[e] = h.S[e];
    h.cand[e] = (uint8_t)j;
    h.pcand[e] = (uint8_t)pc;
    return e;
  };
  auto push = [&](int e) {
    int i = hn++;
    h.heap[i] = (uint16_t)e;
    while (i > 0) {
      const int pi = (i - 1) >> 1;
      if (!heap_before(h, h.heap[i], h.heap[pi])) break;
      const uint16_t t = h.heap[i];
      h.heap[i] = h.heap[pi];
      h.heap[pi] = t;
      i = pi;
    }
  };
  auto pop = [&]() -> int {
    const int top = h.heap[0];
    h.heap[0] = h.heap[--hn];
    int i = 0;
    for (;;) {
      const int l = 2 * i + 1, r = l + 1;
      int m = i;
      if (l < hn && heap_before(h, h.heap[l], h.heap[m])) m = l;
      if (r < hn && heap_before(h, h.heap[r], h.heap[m])) m = r;
      if (m == i) break;
      const uint16_t t = h.heap[i];
      h.heap[i] = h.heap[m];
      h.heap[m] = t;
      i = m;
    }
    return top;
  };
  push(make(0, 0.0, 1, 0, 0, 0, R.best(0, 0)));
  while (hn > 0 && count < B) {
    const int e = pop();
    const int d = h.dep[e], rk = h.ranks[e][d - 1];
    h.out_e[count] = (int16_t)e;
    const int node = ++count;
    const int j = h.cand[e], pc = h.pcand[e];
    const int sj = next_after(d - 1, pc, R.row(d - 1, pc)[j], R.tok[(size_t)(d - 1) * C + j]);
    if (sj >= 0 && rk + 1 < C) push(make(e, h.Spar[e], d, rk + 1, h.parent[e], pc, sj));  // sibling
    if (d < L) push(make(e, h.S[e], d + 1, 0, node, j, R.best(d, j)));                    // child
  }
  sm.nsel = count;
  for (int q = 0; q < B; ++q) {
    const size_t o = (size_t)b * B + q;
    if (q < count) {
      const int e = h.out_e[q];
      const int d = h.dep[e];
      p.tree_tokens[o] = R.tok[(size_t)(d - 1) * C + h.cand[e]];
      p.parents[o] = h.parent[e];
      p.logq[o] = (float)h.sc[e];
      if (p.depths) p.depths[o] = d;
      sm.opar[q] = h.parent[e];
    } else {
      p.tree_tokens[o] = -1;
      p.parents[o] = -1;
      p.logq[o] = -INFINITY;
      if (p.depths) p.depths[o] = 0;
    }
  }
  p.num_nodes[b] = count;
}

__global__ __launch_bounds__(kSelThreads) void sp_select_kernel(SelectParams p) {
  __shared__ SelectSmem sm;
  SelEnum& en = sm.u.en;
  SpTabs& tb = *reinterpret_cast<SpTabs*>(sm.v);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t b = blockIdx.x;
  const int L = p.L, C = p.K, B = p.B, LC = L * C, bpd = p.bpd;
  SpRows R;
  R.tb = &tb;
  R.lp = p.sp_lp + (size_t)b * (L - 1) * C * C;
  R.tok = tb.tok;
  R.C = C;
  for (int i = tid; i < LC; i += kSelThreads) tb.tok[i] = p.ids[(size_t)b * LC + i];
  for (int i = tid; i < (L - 1) * C; i += kSelThreads) {
    tb.best[i] = p.sp_best[(size_t)b * (L - 1) * C + i];
    tb.blp[i] = p.sp_blp[(size_t)b * (L - 1) * C + i];
  }
  if (wv == 0) {
    // row 0 over its candidates (the table kernel's arithmetic)
    const float* v0 = p.vals + (size_t)b * LC;
    float x[kSpC / kWave];
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < kSpC / kWave; ++q) {
      const int j = lane + q * kWave;
      x[q] = j < C ? v0[j] : -INFINITY;
      mx = fmaxf(mx, x[q]);
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < kSpC / kWave; ++q) sum += x[q] == -INFINITY ? 0.0f : __expf(x[q] - mx);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) sum += __shfl_xor(sum, o);
    const float lse = mx + __logf(sum);
    // its best (rounding can tie distinct logits: ties go to the lower token)
    const int32_t* t0 = p.ids + (size_t)b * LC;  // (the LDS copy is not yet visible)
    float bv = -INFINITY;
    int bt = 0x7FFFFFFF, bj = 0;
#pragma unroll
    for (int q = 0; q < kSpC / kWave; ++q) {
      const int j = lane + q * kWave;
      if (j < C) {
        const float v = x[q] - lse;
        tb.lp0[j] = v;
        if (sp_better(v, t0[j], bv, bt)) {
          bv = v;
          bt = t0[j];
          bj = j;
        }
      }
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const float ov = __shfl_xor(bv, o);
      const int ot = __shfl_xor(bt, o), oj = __shfl_xor(bj, o);
      if (sp_better(ov, ot, bv, bt)) {
        bv = ov;
        bt = ot;
        bj = oj;
      }
    }
    if (lane == 0) tb.best0 = bj;
  }
  __syncthreads();
  if (tid == 0) {
    // the spine: best children all the way down, float64 left to right
    int c = tb.best0;
    double S = (double)tb.lp0[c];
    sm.P0[0] = 0.0;
    sm.sig[0] = 0.0;
    sm.P0[1] = S;
    sm.sig[1] = S;
    tb.spine[0] = c;
    for (int d = 1; d < L; ++d) {
      S += (double)tb.blp[(d - 1) * C + c];
      c = tb.best[(d - 1) * C + c];
      tb.spine[d] = c;
      sm.P0[d + 1] = S;
      sm.sig[d + 1] = S;
    }
    sm.nE = 0;
    sm.ovf = 0;
  }
  __syncthreads();

  // ---- 1. threshold: the spine nodes' rows (root: row 0) give L*C one-
  // deviation prefixes; their minimum is a lower bound with >= B above it
  double tau = -INFINITY;
  if (LC >= B) {
    double* od = sm.u.mt.b;
    for (int i = tid; i < LC; i += kSelThreads) {
      const int d = i / C, j = i - d * C;
      od[i] = sm.P0[d] + (double)R.row(d, d == 0 ? 0 : tb.spine[d - 1])[j];
    }
    __syncthreads();
    tau = sel_tau_hist(sm, LC, B, [&](int i) { return od[i]; },
                       [&](int ln) {
                         double m = INFINITY;
                         for (int i = ln; i < LC; i += kWave) m = od[i] < m ? od[i] : m;
                         return m;
                       });
  }

  // ---- 2. enumerate E = {score >= tau} by chains ----------------------------
  // On overflow the B-th best entry found so far becomes the threshold and
  // the enumeration restarts (as in select_kernel), then the heap.
  for (int attempt = 0;; ++attempt) {
    // spine prefixes reaching tau (the spine's scores do not increase)
    const int D0 = __popcll(__ballot(lane < L && sm.sig[lane + 1] >= tau));
    for (int d = tid; d < D0; d += kSelThreads) {
      en.eS[d] = sm.P0[d + 1];
      en.eSc[d] = sm.sig[d + 1];
      en.ePar[d] = (int16_t)(d - 1);
      en.eRank[d] = (uint16_t)tb.spine[d];
      en.eDep[d] = (uint8_t)(d + 1);
      en.eLh[d] = 0;
      en.eLl[d] = (uint64_t)(d + 1);
    }
    if (tid == 0) sm.nE = D0;
    __syncthreads();
    // Generation g: the chains whose anchors deviate g times. One wave per
    // parent: its row is read once (two floats a lane), a ballot marks the
    // children that deviate (not the row's best) and reach tau, and each such
    // lane appends its chain. A child's rank is 1 (the best child) plus the
    // deviating children ordered before it: every child ordered before a
    // qualifying one scores at least as high, so qualifies too.
    int g0 = 0, g1 = D0, root = 1;
    for (;;) {
      const int np = root + (g1 - g0);
      auto parent = [&](int u, double& S, int& d, int& c, int& pe) {
        S = 0.0;
        d = 0;
        c = 0;
        pe = -1;
        if (!(root && u == 0)) {
          pe = g0 + u - root;
          S = en.eS[pe];
          d = en.eDep[pe];
          c = en.eRank[pe];
        }
      };
      auto load = [&](int u, float& v0, float& v1) {
        v0 = -INFINITY;
        v1 = -INFINITY;
        if (u >= np) return;
        double S;
        int d, c, pe;
        parent(u, S, d, c, pe);
        if (d < L) {
          const float* r = R.row(d, c);
          if (lane < C) v0 = r[lane];
          if (lane + kWave < C) v1 = r[lane + kWave];
        }
      };
      float n0, n1;
      load(wv, n0, n1);
      for (int u = wv; u < np; u += kSelWaves) {
        const float v0 = n0, v1 = n1;
        load(u + kSelWaves, n0, n1);  // the wave's next parent, in flight meanwhile
        double S;
        int d, c, pe;
        parent(u, S, d, c, pe);
        if (d >= L) continue;
        const int bj = R.best(d, c);
        const int j0 = lane, j1 = lane + kWave;
        const bool q0 = j0 < C && j0 != bj && S + (double)v0 >= tau;
        const bool q1 = j1 < C && j1 != bj && S + (double)v1 >= tau;
        const uint64_t m0 = __ballot(q0), m1 = __ballot(q1);
        if ((m0 | m1) == 0) continue;
        const int32_t* tk = tb.tok + d * C;
        const int t0 = j0 < C ? tk[j0] : 0x7FFFFFFF, t1 = j1 < C ? tk[j1] : 0x7FFFFFFF;
        int rk0 = 1, rk1 = 1;
        for (uint64_t m = m0; m; m &= m - 1) {
          const int src = __builtin_ctzll(m);
          const float v = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v0), src));
          const int t = __builtin_amdgcn_readlane(t0, src);
          rk0 += sp_better(v, t, v0, t0) ? 1 : 0;
          rk1 += sp_better(v, t, v1, t1) ? 1 : 0;
        }
        for (uint64_t m = m1; m; m &= m - 1) {
          const int src = __builtin_ctzll(m);
          const float v = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v1), src));
          const int t = __builtin_amdgcn_readlane(t1, src);
          rk0 += sp_better(v, t, v0, t0) ? 1 : 0;
          rk1 += sp_better(v, t, v1, t1) ? 1 : 0;
        }
        uint64_t lh = 0, ll = 0;
        if (pe >= 0) {
          lh = en.eLh[pe];
          ll = en.eLl[pe] & ~63ull;
        }
        // the anchor (child j of the parent, score S + v, rank rk) and its
        // best-child extensions while they reach tau
        auto emit = [&](int j, float v, int rk) {
          const int dn = d + 1;
          const double Sa = S + (double)v;
          uint64_t ah = lh, al = ll;
          lex_set_digit(ah, al, dn, (uint32_t)rk, bpd);
          int ell = 1;
          {
            double S2 = Sa;
            int c2 = j;
            for (int dd = dn + 1; dd <= L; ++dd) {
              S2 += (double)R.best_lp(dd - 1, c2);
              if (S2 < tau) break;
              c2 = R.best(dd - 1, c2);
              ++ell;
            }
          }
          const int pos = atomicAdd(&sm.nE, ell);
          if (pos + ell > kECap) {
            // slots of this chain below the capacity stay unwritten: mark them
            for (int q = pos; q < kECap; ++q) en.eSc[q] = -INFINITY;
            sm.ovf = 1;
            return;
          }
          en.eS[pos] = Sa;
          en.eSc[pos] = Sa;
          en.ePar[pos] = (int16_t)pe;
          en.eRank[pos] = (uint16_t)j;
          en.eDep[pos] = (uint8_t)dn;
          en.eLh[pos] = ah;
          en.eLl[pos] = al | (uint64_t)dn;
          double S2 = Sa;
          int c2 = j;
          for (int k = 1; k < ell; ++k) {
            const int dd = dn + k;
            S2 += (double)R.best_lp(dd - 1, c2);
            c2 = R.best(dd - 1, c2);
            const int q = pos + k;
            en.eS[q] = S2;
            en.eSc[q] = S2;
            en.ePar[q] = (int16_t)(q - 1);
            en.eRank[q] = (uint16_t)c2;
            en.eDep[q] = (uint8_t)dd;
            en.eLh[q] = ah;
            en.eLl[q] = al | (uint64_t)dd;
          }
        };
        if (q0) emit(j0, v0, rk0);
        if (q1) emit(j1, v1, rk1);
      }
      __syncthreads();
      if (sm.ovf) break;
      g0 = g1;
      g1 = sm.nE;
      root = 0;
      __syncthreads();  // every wave has read nE before the next generation appends
      if (g0 == g1) break;
    }
    if (!sm.ovf) break;
    const int n = sm.nE < kECap ? sm.nE : kECap;
    if (attempt == kSelRetries || n < B) break;
    const double t1 = sel_tau_hist(
        sm, n, B, [&](int i) { return en.eSc[i]; }, [&](int) { return tau; },
        reinterpret_cast<double*>(en.eLh), kECap);
    if (!(t1 > tau)) break;
    tau = t1;
    if (tid == 0) sm.ovf = 0;
    __syncthreads();
  }

  if (sm.ovf) {
    __syncthreads();
    if (tid == 0) sp_heap_fallback(p, sm, b, R);
    __syncthreads();
  } else {
    sel_order_emit(p, sm, b, tau);
  }
  sel_mask(p, sm, b);
}

}  // namespace ddt
