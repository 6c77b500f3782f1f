// Stage 2 (+ stage 3): top-B prefix selection and the ancestor mask.
//
// What is computed (DDTree explainer, sections 2-4; SparklingTree post,
// "Step 3"): the B most probable prefixes of the factorised drafter
// distribution, emitted best first. With per-row sorted logits v_d[r] and
// normalisers z_d, a rank tuple (r_1..r_d) scores
//     score = min(score(parent), S - Z_d),  S = v_1[r_1] + ... + v_d[r_d],
//     Z_d = z_1 + ... + z_d   (float64, left to right; root score 0),
// and prefixes are ordered by (score desc, rank tuple lexicographic asc, a
// prefix before its extensions) -- the order in which the pages' best-first
// heap pops them. Scores never increase along a path and siblings are
// ordered, so the first B prefixes in this order form a prefix-closed tree
// (Proposition 2) and every node's parent is emitted before it.
//
// MI355X design: no serial heap on the common path. One 1024-thread
// workgroup per request:
//  1. Threshold. tau = the B-th best score among the L*K prefixes that
//     deviate from the all-rank-0 spine only in their last position (found
//     to ~1e-6 by a block-parallel bisection). These are B valid prefixes,
//     so every one of the true top B scores at least tau.
//  2. Enumerate E = {prefixes with score >= tau} by "chains": a chain is an
//     anchor prefix whose last rank is >= 1 followed by its rank-0
//     extensions, which one thread walks in registers. Generation g holds
//     the chains with g nonzero ranks; a generation's deviating children
//     are counted by binary search over the sorted row, allocated by a block
//     scan and walked in parallel. Drafter trees have <= 3 deviations per
//     path in practice, so this needs a few block-synchronous steps instead
//     of one per tree level.
//  3. Bitonic-sort E (LDS) by (score, 128-bit lexicographic rank key) and
//     emit the first B, mapping parents to output node numbers.
//  4. Write the bit-packed ancestor mask rows from the parents in LDS.
// If E would exceed kECap entries (flat rows with V < B, massive ties), the
// block instead runs the pages' best-first heap in one thread, in LDS:
// exact, slower, and only for such inputs.
#pragma once

#include "common.hpp"

namespace ddt {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kECap = 2048;
constexpr int kMaxLK = 8192;
constexpr int kMaxL = 32;
constexpr int kMaxB = 512;
constexpr int kMaxW = (kMaxB + 1 + 63) / 64;
constexpr int kCPT = kMaxLK / kSelThreads;  // one-deviation prefixes per thread
constexpr int kHeapCap = 2 * kMaxB + 2;

struct SelectParams {
  const float* vals;   // [batch][L][K] sorted logits
  const int32_t* ids;  // [batch][L][K] their token ids
  const double* lse;   // [batch][L] row normalisers
  int64_t batch;
  int32_t L, K, B;
  int32_t bpd;  // bits per lexicographic digit (ceil(log2 K), >= 1)
  int32_t* tree_tokens;
  int32_t* parents;
  float* logq;
  int32_t* depths;  // may be null
  int32_t* num_nodes;
  uint64_t* mask;  // may be null; [batch][B+1][W]
  int32_t W;
};

struct SelEnum {
  double eS[kECap];
  double eSc[kECap];
  uint64_t eLh[kECap];
  uint64_t eLl[kECap];
  int16_t ePar[kECap];
  uint16_t eRank[kECap];
  uint8_t eDep[kECap];
  uint16_t idx[kECap];
  int cnt[kECap + 1];
};

struct SelHeap {
  double sc[kHeapCap];
  double S[kHeapCap];
  double Spar[kHeapCap];
  double scpar[kHeapCap];
  int16_t parent[kHeapCap];  // node number of the parent
  uint8_t dep[kHeapCap];
  uint16_t ranks[kHeapCap][kMaxL];
  uint16_t heap[kHeapCap];  // heap of pool indices
  // emitted nodes
  int16_t out_e[kMaxB];
};

struct SelectSmem {
  float v[kMaxLK];
  double Z[kMaxL];
  double P0[kMaxL + 1];
  double sig[kMaxL + 1];
  union {
    SelEnum en;
    SelHeap hp;
  } u;
  int opar[kMaxB];  // parent node number of output node j+1
  int wsum[kSelWaves];
  int redI[2][kSelWaves];
  double redD[kSelWaves];
  double tau;
  int nE;
  int ovf;
  int nsel;
};

__device__ __forceinline__ void lex_set_digit(uint64_t& hi, uint64_t& lo, int d, uint32_t r,
                                              int bpd) {
  const int s = 128 - d * bpd;  // bit position of the digit's LSB (>= 6)
  if (s >= 64) {
    hi |= (uint64_t)r << (s - 64);
  } else if (s + bpd <= 64) {
    lo |= (uint64_t)r << s;
  } else {
    hi |= (uint64_t)r >> (64 - s);
    lo |= (uint64_t)r << s;
  }
}

__device__ __forceinline__ int sel_block_sum(int v, SelectSmem& sm, int& parity) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sm.redI[parity][threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) t += sm.redI[parity][i];
  parity ^= 1;
  return t;
}

__device__ __forceinline__ double sel_block_min(double v, SelectSmem& sm) {
  v = wave_min(v);
  if ((threadIdx.x & 63) == 0) sm.redD[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = sm.redD[0];
#pragma unroll
  for (int i = 1; i < kSelWaves; ++i) r = r < sm.redD[i] ? r : sm.redD[i];
  __syncthreads();
  return r;
}

__device__ __forceinline__ double sel_block_max(double v, SelectSmem& sm) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) sm.redD[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = sm.redD[0];
#pragma unroll
  for (int i = 1; i < kSelWaves; ++i) r = r > sm.redD[i] ? r : sm.redD[i];
  __syncthreads();
  return r;
}

// e1 strictly before e2 in the output order (PAD = 0xFFFF is last).
__device__ __forceinline__ bool sel_before(const SelEnum& en, int e1, int e2) {
  if (e1 == 0xFFFF) return false;
  if (e2 == 0xFFFF) return true;
  const double a = en.eSc[e1], b = en.eSc[e2];
  if (a != b) return a > b;
  if (en.eLh[e1] != en.eLh[e2]) return en.eLh[e1] < en.eLh[e2];
  return en.eLl[e1] < en.eLl[e2];
}

// ---------------------------------------------------------------------------
// Fallback: best-first heap over rank tuples in one thread (LDS).
__device__ __forceinline__ bool heap_before(const SelHeap& h, int a, int b) {
  if (h.sc[a] != h.sc[b]) return h.sc[a] > h.sc[b];
  const int da = h.dep[a], db = h.dep[b];
  const int n = da < db ? da : db;
  for (int i = 0; i < n; ++i)
    if (h.ranks[a][i] != h.ranks[b][i]) return h.ranks[a][i] < h.ranks[b][i];
  return da < db;
}

__device__ void heap_fallback(const SelectParams& p, SelectSmem& sm, int64_t b) {
  SelHeap& h = sm.u.hp;
  const int L = p.L, K = p.K, B = p.B;
  int pool = 0, hn = 0, count = 0;
  // New pool entry at depth d with last rank r; its first d-1 ranks are
  // copied from pool entry `src` (unused when d == 1).
  auto make = [&](int src, double Spar, double scpar, int d, int r, int parent_node) -> int {
    const int e = pool++;
    for (int i = 0; i < d - 1; ++i) h.ranks[e][i] = h.ranks[src][i];
    h.ranks[e][d - 1] = (uint16_t)r;
    h.dep[e] = (uint8_t)d;
    h.parent[e] = (int16_t)parent_node;
    h.Spar[e] = Spar;
    h.scpar[e] = scpar;
    h.S[e] = Spar + (double)sm.v[(d - 1) * K + r];
    const double raw = h.S[e] - sm.Z[d - 1];
    h.sc[e] = raw > scpar ? scpar : raw;
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
  push(make(0, 0.0, 0.0, 1, 0, 0));
  while (hn > 0 && count < B) {
    const int e = pop();
    const int d = h.dep[e], r = h.ranks[e][d - 1];
    h.out_e[count] = (int16_t)e;
    const int node = ++count;
    if (r + 1 < K) push(make(e, h.Spar[e], h.scpar[e], d, r + 1, h.parent[e]));  // sibling
    if (d < L) push(make(e, h.S[e], h.sc[e], d + 1, 0, node));                   // child
  }
  sm.nsel = count;
  for (int j = 0; j < B; ++j) {
    const size_t o = (size_t)b * B + j;
    if (j < count) {
      const int e = h.out_e[j];
      const int d = h.dep[e], r = h.ranks[e][d - 1];
      p.tree_tokens[o] = p.ids[(size_t)b * L * K + (size_t)(d - 1) * K + r];
      p.parents[o] = h.parent[e];
      p.logq[o] = (float)h.sc[e];
      if (p.depths) p.depths[o] = d;
      sm.opar[j] = h.parent[e];
    } else {
      p.tree_tokens[o] = -1;
      p.parents[o] = -1;
      p.logq[o] = -INFINITY;
      if (p.depths) p.depths[o] = 0;
    }
  }
  p.num_nodes[b] = count;
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams p) {
  __shared__ SelectSmem sm;
  SelEnum& en = sm.u.en;
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int L = p.L, K = p.K, B = p.B, LK = L * K, bpd = p.bpd;
  const float* vals = p.vals + (size_t)b * LK;
  int parity = 0;

  for (int i = tid; i < LK; i += kSelThreads) sm.v[i] = vals[i];
  if (tid == 0) {
    // Z_d and the spine (all ranks 0): float64, left to right.
    double acc = 0.0, S = 0.0, sc = 0.0;
    sm.P0[0] = 0.0;
    sm.sig[0] = 0.0;
    for (int d = 1; d <= L; ++d) {
      acc += p.lse[(size_t)b * L + d - 1];
      sm.Z[d - 1] = acc;
      S += (double)vals[(size_t)(d - 1) * K];
      const double raw = S - acc;
      sc = raw > sc ? sc : raw;
      sm.P0[d] = S;
      sm.sig[d] = sc;
    }
    sm.nE = 0;
    sm.ovf = 0;
  }
  __syncthreads();

  // ---- 1. threshold from the one-deviation prefixes -------------------------
  double sc1[kCPT];
  double lo_l = INFINITY, hi_l = -INFINITY;
#pragma unroll
  for (int i = 0; i < kCPT; ++i) {
    const int c = tid + i * kSelThreads;
    sc1[i] = -INFINITY;
    if (c < LK) {
      const int d = c / K + 1;
      const double raw = (sm.P0[d - 1] + (double)sm.v[c]) - sm.Z[d - 1];
      const double s = raw > sm.sig[d - 1] ? sm.sig[d - 1] : raw;
      sc1[i] = s;
      lo_l = s < lo_l ? s : lo_l;
      hi_l = s > hi_l ? s : hi_l;
    }
  }
  double tau = -INFINITY;
  if (LK >= B) {
    double lo = sel_block_min(lo_l, sm), hi = sel_block_max(hi_l, sm);
    int c_hi = 0;
#pragma unroll
    for (int i = 0; i < kCPT; ++i) c_hi += sc1[i] >= hi ? 1 : 0;
    if (sel_block_sum(c_hi, sm, parity) >= B) {
      lo = hi;
    } else {
      for (int it = 0; it < 24; ++it) {
        const double mid = lo + 0.5 * (hi - lo);
        if (!(mid > lo && mid < hi)) break;
        int c = 0;
#pragma unroll
        for (int i = 0; i < kCPT; ++i) c += sc1[i] >= mid ? 1 : 0;
        if (sel_block_sum(c, sm, parity) >= B) lo = mid;
        else hi = mid;
      }
    }
    tau = lo;
  }

  // ---- 2. enumerate E = {score >= tau} by chains ----------------------------
  int D0 = 0;
  for (int d = 1; d <= L; ++d) D0 += sm.sig[d] >= tau ? 1 : 0;
  if (D0 > kECap) D0 = kECap;  // cannot happen (L <= 32)
  for (int d = tid; d < D0; d += kSelThreads) {
    en.eS[d] = sm.P0[d + 1];
    en.eSc[d] = sm.sig[d + 1];
    en.ePar[d] = (int16_t)(d - 1);
    en.eRank[d] = 0;
    en.eDep[d] = (uint8_t)(d + 1);
    en.eLh[d] = 0;
    en.eLl[d] = (uint64_t)(d + 1);
  }
  if (tid == 0) sm.nE = D0;
  __syncthreads();
  int g0 = 0, g1 = D0, root = 1;
  for (;;) {
    const int np = root + (g1 - g0);
    if (np > kECap) {  // parents must fit the count array
      if (tid == 0) sm.ovf = 1;
      __syncthreads();
      break;
    }
    for (int i = tid; i < np; i += kSelThreads) {
      double S = 0.0;
      int d = 0;
      if (!(root && i == 0)) {
        const int e = g0 + i - root;
        S = en.eS[e];
        d = en.eDep[e];
      }
      int c = 0;
      if (d < L) {
        // number of ranks r >= 1 of row d+1 whose child scores >= tau
        const float* row = sm.v + d * K;
        const double Zd = sm.Z[d];
        int lo = 1, hi = K;  // first failing rank lies in [lo, hi]
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if ((S + (double)row[mid]) - Zd >= tau) lo = mid + 1;
          else hi = mid;
        }
        c = lo - 1;
      }
      en.cnt[i] = c;
    }
    __syncthreads();
    const int A = block_excl_scan<kSelThreads>(en.cnt, np, sm.wsum);
    if (A == 0) break;
    for (int a = tid; a < A; a += kSelThreads) {
      // parent = largest u with offset[u] <= a
      int lo = 0, hi = np - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (en.cnt[mid] <= a) lo = mid;
        else hi = mid - 1;
      }
      const int u = lo;
      const int r = a - en.cnt[u] + 1;
      double Su = 0.0, scu = 0.0;
      int du = 0, pe = -1;
      uint64_t lh = 0, ll = 0;
      if (!(root && u == 0)) {
        pe = g0 + u - root;
        Su = en.eS[pe];
        scu = en.eSc[pe];
        du = en.eDep[pe];
        lh = en.eLh[pe];
        ll = en.eLl[pe] & ~63ull;
      }
      const int d = du + 1;
      const double S = Su + (double)sm.v[(d - 1) * K + r];
      const double raw = S - sm.Z[d - 1];
      const double sc = raw > scu ? scu : raw;
      lex_set_digit(lh, ll, d, (uint32_t)r, bpd);
      int ell = 1;
      {
        double S2 = S, sc2 = sc;
        for (int dd = d + 1; dd <= L; ++dd) {
          S2 += (double)sm.v[(dd - 1) * K];
          const double raw2 = S2 - sm.Z[dd - 1];
          sc2 = raw2 > sc2 ? sc2 : raw2;
          if (sc2 < tau) break;
          ++ell;
        }
      }
      const int pos = atomicAdd(&sm.nE, ell);
      if (pos + ell > kECap) {
        sm.ovf = 1;
        continue;
      }
      en.eS[pos] = S;
      en.eSc[pos] = sc;
      en.ePar[pos] = (int16_t)pe;
      en.eRank[pos] = (uint16_t)r;
      en.eDep[pos] = (uint8_t)d;
      en.eLh[pos] = lh;
      en.eLl[pos] = ll | (uint64_t)d;
      double S2 = S, sc2 = sc;
      for (int i = 1; i < ell; ++i) {
        const int dd = d + i;
        S2 += (double)sm.v[(dd - 1) * K];
        const double raw2 = S2 - sm.Z[dd - 1];
        sc2 = raw2 > sc2 ? sc2 : raw2;
        en.eS[pos + i] = S2;
        en.eSc[pos + i] = sc2;
        en.ePar[pos + i] = (int16_t)(pos + i - 1);
        en.eRank[pos + i] = 0;
        en.eDep[pos + i] = (uint8_t)dd;
        en.eLh[pos + i] = lh;
        en.eLl[pos + i] = ll | (uint64_t)dd;
      }
    }
    __syncthreads();
    if (sm.ovf) break;
    g0 = g1;
    g1 = sm.nE;
    root = 0;
    if (g0 == g1) break;
  }

  if (sm.ovf) {
    __syncthreads();
    if (tid == 0) heap_fallback(p, sm, b);
    __syncthreads();
  } else {
    // ---- 3. sort E and emit the first B -----------------------------------
    const int nE = sm.nE;
    const int N = next_pow2(nE < 1 ? 1 : nE);
    for (int i = tid; i < N; i += kSelThreads) en.idx[i] = (uint16_t)(i < nE ? i : 0xFFFF);
    __syncthreads();
    for (int k = 2; k <= N; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < (N >> 1); i += kSelThreads) {
          const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
          const int hi = lo + j;
          const int x = en.idx[lo], y = en.idx[hi];
          const bool best_first = (lo & k) == 0;
          if (best_first ? sel_before(en, y, x) : sel_before(en, x, y)) {
            en.idx[lo] = (uint16_t)y;
            en.idx[hi] = (uint16_t)x;
          }
        }
        __syncthreads();
      }
    }
    const int nsel = nE < B ? nE : B;
    for (int i = tid; i < nE; i += kSelThreads) en.cnt[i] = -1;
    __syncthreads();
    for (int j = tid; j < nsel; j += kSelThreads) en.cnt[en.idx[j]] = j;
    __syncthreads();
    for (int j = tid; j < B; j += kSelThreads) {
      const size_t o = (size_t)b * B + j;
      if (j < nsel) {
        const int e = en.idx[j];
        const int d = en.eDep[e], r = en.eRank[e], pe = en.ePar[e];
        const int par = pe < 0 ? 0 : en.cnt[pe] + 1;
        p.tree_tokens[o] = p.ids[(size_t)b * LK + (size_t)(d - 1) * K + r];
        p.parents[o] = par;
        p.logq[o] = (float)en.eSc[e];
        if (p.depths) p.depths[o] = d;
        sm.opar[j] = par;
      } else {
        p.tree_tokens[o] = -1;
        p.parents[o] = -1;
        p.logq[o] = -INFINITY;
        if (p.depths) p.depths[o] = 0;
      }
    }
    if (tid == 0) {
      p.num_nodes[b] = nsel;
      sm.nsel = nsel;
    }
    __syncthreads();
  }

  // ---- 4. ancestor mask ------------------------------------------------------
  if (p.mask) {
    const int nsel = sm.nsel, W = p.W;
    for (int i = tid; i <= B; i += kSelThreads) {
      uint64_t m[kMaxW];
#pragma unroll
      for (int q = 0; q < kMaxW; ++q) m[q] = 0;
      if (i <= nsel) {
        int u = i;
        for (int step = 0; step <= kMaxL + 1; ++step) {
          const int wq = u >> 6;
          const uint64_t bit = 1ull << (u & 63);
#pragma unroll
          for (int q = 0; q < kMaxW; ++q) m[q] |= (q == wq) ? bit : 0ull;
          if (u == 0) break;
          u = sm.opar[u - 1];
        }
      }
      uint64_t* dst = p.mask + ((size_t)b * (B + 1) + i) * W;
#pragma unroll
      for (int q = 0; q < kMaxW; ++q)
        if (q < W) dst[q] = m[q];
    }
  }
}

}  // namespace ddt
