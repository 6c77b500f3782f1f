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
// workgroup per request (four waves per SIMD: a lone wave issues only about
// a quarter of the SIMD's vector rate, and every step here is short):
//  1. Threshold. tau = the B-th best score among the L*K prefixes that
//     deviate from the all-rank-0 spine only in their last position, exact:
//     a histogram of those scores above a lower bound, one scan for the bin
//     holding the B-th, exact ranking inside that bin.
//     These are B valid prefixes, so every one of the true top B scores at
//     least tau.
//  2. Enumerate E = {prefixes with score >= tau} by "chains": a chain is an
//     anchor prefix whose last rank is >= 1 followed by its rank-0
//     extensions. Generation g holds the chains with g nonzero ranks; a
//     generation's deviating children are counted by binary search over the
//     sorted row, allocated by a block scan (DPP inside waves), each new
//     anchor finds its parent by binary search over the parents' offsets,
//     the chain lengths are summed by a second block scan, and every chain
//     entry is then written by its own thread. The generations stop as soon
//     as no new entry has a deviating child reaching tau. Drafter trees
//     have <= 3 deviations per path in practice, so this needs a few
//     block-synchronous steps instead of one per tree level.
//     Fast path (decided per request): when every nonzero row value's binary
//     exponent lies within 11 of the first row's top value's, every sum of
//     <= 32 row values is exact in float64 (a 22-binade span, 24-bit
//     mantissas and 5 bits of carries fit in 53 bits), so a rank-0
//     extension's score is (S + P0[e] - P0[d]) - Z[e-1] whatever the order
//     of summation; when in
//     addition every row's top log-probability is clearly negative no score
//     clamps, so a chain's scores strictly decrease and its length is one
//     binary search. Otherwise chains are walked step by step with the
//     clamp, in the same arithmetic as the canonical score.
//  3. Histogram E's scores into bins over [tau, best]; the first bins that
//     hold >= B entries form E2, which contains the output. Place each entry
//     of E2 in the order (score, then 128-bit lexicographic rank key) by
//     counting the entries before it. Emit the first B, mapping parents to
//     output node numbers (a parent is in the output and precedes it).
//  4. Write the bit-packed ancestor mask rows from the parents in LDS.
// If E would exceed kECap entries, the B-th best of the entries found so far
// is a valid, tighter threshold and the enumeration restarts from it (at most
// kSelRetries times); only if that does not help (massive exact ties, V < B)
// does the block run the pages' best-first heap in one thread, in LDS:
// exact, slower, and only for such inputs.
#pragma once

#include "common.hpp"

namespace ddt {

constexpr int kSelThreads = 1024;  // conditioned-row selection's workgroup
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelNT = 1024;  // independent-row selection's workgroup
constexpr int kSelBins = 1024;  // histogram bins of the threshold and the ordering
constexpr int kECap = 2048;
static_assert(kECap / kSelNT >= 2, "two entries per thread at least");
constexpr int kSelRetries = 3;  // threshold raises after an enumeration overflow
constexpr int kMaxLK = 8192;
constexpr int kMaxL = 32;
constexpr int kMaxB = 512;
constexpr int kMaxW = (kMaxB + 1 + 63) / 64;
constexpr int kHeapCap = 2 * kMaxB + 2;
// capacity of one merge-tree level: ceil(L / 2) * min(2K, B) entries
constexpr int kMergeCap = 4096;

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
  // derived on the host (select_derived): i / K = (i * kmag) >> 32 and
  // t / W = (t * wmag) >> 32 for i, t < 2^13 (exact while i * K < 2^32),
  // and q1 = min(ceil(B / L), K)
  uint64_t kmag, wmag;
  int32_t q1;
  // conditioned rows (SparklingTree; null for independent rows)
  const float* sp_lp;      // [batch][L-1][K][K] child row d, parent candidate, child candidate
  const uint8_t* sp_best;  // [batch][L-1][K] each row's best child
  const float* sp_blp;     // [batch][L-1][K] its log-prob
};

struct SelEnum {
  double eS[kECap];
  double eSc[kECap];
  uint64_t eLh[kECap];
  uint64_t eLl[kECap];
  int16_t ePar[kECap];
  uint16_t eRank[kECap];
  uint8_t eDep[kECap];
  int cnt[kECap + 1];  // output rank of each entry
  uint32_t own[kECap];  // enumeration: a generation's new anchor -> (parent << 16) | rank
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
  uint8_t cand[kHeapCap];   // conditioned rows: the entry's candidate index
  uint8_t pcand[kHeapCap];  // and its parent's (the row its siblings come from)
  // emitted nodes
  int16_t out_e[kMaxB];
};

struct SelectSmem {
  float v[kMaxLK];
  double lse[kMaxL];
  double Z[kMaxL];
  double P0[kMaxL + 1];
  double sig[kMaxL + 1];
  union {
    SelEnum en;
    SelHeap hp;
    struct {  // merge tree of the threshold (before the enumeration)
      double a[kMergeCap];
      double b[kMergeCap];
    } mt;
  } u;
  int opar[kMaxB];  // parent node number of output node j+1
  alignas(16) int wsum[kSelWaves];
  int A1;    // the first generation's anchors (counted by wave 0)
  int kexc;  // entries before the threshold's bin
  int n2;
  int kcut;
  alignas(16) int hist[kSelBins];
  alignas(16) int hexc[kSelBins];  // entries in the bins before each bin
  double tau;
  double hscale;  // the threshold histogram's bins per unit score
  double tcut;    // the threshold found by the thread holding the cut bin
  double oscale;  // the ordering histogram's bins per unit score (independent rows)
  int nE;
  int ovf;
  int nsel;
  alignas(16) uint32_t wbad[kSelWaves];  // per wave: some value outside the exact-sum window
  int ncand;                 // entries of this generation with a deviating child
  int np1;                   // parents listed for a generation counted by wave 0
  int cand[kWave];           // the first kWave of them
  int pcand[kWave];          // the listed parents of the current generation
  int f2;                    // every row's top log-probability is clearly negative
};

__device__ __forceinline__ void lex_set_digit(uint64_t& hi, uint64_t& lo, int d, uint32_t r,
                                              int bpd) {
  const int s = 128 - d * bpd;  // bit position of the digit's LSB (>= 6)
  const uint64_t v = r;
  // the digit lies in the high word, the low word, or straddles them
  const uint64_t h = s >= 64 ? v << (s - 64) : (s + bpd > 64 ? v >> (64 - s) : 0ull);
  const uint64_t l = s >= 64 ? 0ull : v << s;
  hi |= h;
  lo |= l;
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
// Exact B-th best one-deviation score (requires L * K >= B). Row d's scores
// s_d(r) = min(sig_d, P0_d + v_d[r] - Z_d) do not increase with r. Lower
// bound mn: the q-th score of every row, q = min(ceil(B / L), K), leaves
// >= B scores at or above the smallest of them. The scores in [mn, best]
// fall into kSelBins bins (index monotone in the score, equal scores share
// a bin); one scan finds the bin holding the B-th, whose few members are
// ranked exactly. Members beyond kMergeCap (flat rows) return mn instead, a
// valid lower bound.
// onedev(i) gives the i-th of the LK scores; lane_bound(lane) a per-lane
// value whose minimum over wave 0 is a lower bound with >= B scores at or
// above it. mem (memcap doubles of LDS, not read by onedev) holds the cut
// bin's members.
// With EXACT false the result is instead the lower edge of the bin holding
// the B-th, moved down by a millionth of a bin: at or below every member of
// that bin, so a valid lower bound with the same guarantee, found without
// ranking the bin (a slightly larger E to enumerate).
template <bool EXACT = true, int NT = kSelThreads, class OD, class LB>
__device__ double sel_tau_hist(SelectSmem& sm, int LK, int B, OD onedev, LB lane_bound,
                               double* mem = nullptr, int memcap = kMergeCap) {
  constexpr int NW = NT / kWave, BPT = kSelBins / NT;  // bins per thread in the scan
  static_assert(BPT * NT == kSelBins, "whole bins per thread");
  if (mem == nullptr) mem = sm.u.mt.a;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int j = tid; j < kSelBins; j += NT) sm.hist[j] = 0;
  if (w == 0) {
    double x = lane_bound(lane);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double y = __shfl_xor(x, o);
      x = y < x ? y : x;
    }
    if (lane == 0) {
      sm.tau = x;
      sm.n2 = 0;
      const double span = sm.sig[1] - x;
      sm.hscale = span > 0.0 ? (double)kSelBins / span : 0.0;
    }
  }
  __syncthreads();
  // one thread divided: scale = kSelBins / (top - mn), or 0 for an empty span
  const double mn = sm.tau, top = sm.sig[1], scale = sm.hscale;
  auto bin_of = [&](double sc) -> int {
    const double t = (top - sc) * scale;
    return t >= (double)(kSelBins - 1) ? kSelBins - 1 : (t > 0.0 ? (int)t : 0);
  };
  for (int i = tid; i < LK; i += NT) {
    const double sc = onedev(i);
    if (sc >= mn) atomicAdd(&sm.hist[bin_of(sc)], 1);
  }
  __syncthreads();
  // scan: this thread's BPT consecutive bins, then the waves' totals
  int h[BPT], hs = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    h[j] = sm.hist[tid * BPT + j];
    hs += h[j];
  }
  const int x = wave_incl_scan(hs);
  if (lane == kWave - 1) sm.wsum[w] = x;
  __syncthreads();
  int tot;
  int run = waves_before<NW>(sm.wsum, w, tot) + x - hs;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int exc = run;
    run += h[j];
    if (run >= B && exc < B) {
      const int kc = tid * BPT + j;
      sm.kcut = kc;
      sm.kexc = exc;
      if (!EXACT) {
        double e = mn;
        if (scale > 0.0 && kc < kSelBins - 1) {
          const double edge = top - ((double)kc + 1.000001) / scale;
          e = edge > mn ? edge : mn;
        }
        sm.tcut = e;
      }
    }
  }
  __syncthreads();
  if constexpr (!EXACT) return sm.tcut;
  const int kb = sm.kcut, t = B - 1 - sm.kexc;  // the B-th is member t of bin kb
  for (int i = tid; i < LK; i += NT) {
    const double sc = onedev(i);
    if (sc >= mn && bin_of(sc) == kb) {
      const int k = atomicAdd(&sm.n2, 1);
      if (k < memcap) mem[k] = sc;
    }
  }
  __syncthreads();
  const int m = sm.n2;
  if (m > memcap) return mn;
  for (int k = tid; k < m; k += NT) {
    const double v = mem[k];
    int gt = 0, ge = 0;
    for (int j = 0; j < m; ++j) {
      const double u = mem[j];
      gt += u > v ? 1 : 0;
      ge += u >= v ? 1 : 0;
    }
    if (gt <= t && t < ge) sm.tau = v;  // every such member holds the same value
  }
  __syncthreads();
  return sm.tau;
}

// ---------------------------------------------------------------------------
// Phase 3 (after an enumeration without overflow): order E, emit the
// first B (tokens, parents, log-probs, depths, node count). en.eRank holds
// each entry's index into its row's candidate table.
// With PRE_SCALE the caller has stored kSelBins / (best - tau) (0 for an
// empty span) in sm.oscale before a barrier.
template <bool ZERO_HIST = true, int NT = kSelThreads, bool PRE_SCALE = false>
__device__ __forceinline__ void sel_order_emit(const SelectParams& p, SelectSmem& sm, int64_t b,
                                               double tau) {
  constexpr int NPT = kECap / NT, NW = NT / kWave, BPT = kSelBins / NT;
  static_assert(NPT * NT == kECap && BPT * NT == kSelBins, "whole entries and bins per thread");
  SelEnum& en = sm.u.en;
  const int tid = threadIdx.x;
  const int L = p.L, K = p.K, B = p.B, LK = L * K;
  (void)L;
  // ---- 3. order E, emit the first B ----------------------------------------
  // E's scores fall into kSelBins bins over [tau, best] (bin index
  // monotone in the score, so equal scores share a bin and a lower bin
  // holds only better scores). E2 = the entries of the first bins that
  // hold >= B of them (all of E when nE <= B); it is closed upwards in the
  // order, so it holds the output. E2 is placed in bin order, and an
  // entry's position is its bin's offset plus the members of its own bin
  // before it (score, then the 128-bit lexicographic rank key).
  const int nE = sm.nE;
  // token ids of this thread's entries, loaded now so that the ordering's
  // barriers cover the global-load latency
  int etok[NPT];
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int i = tid + k * NT;
    etok[k] = i < nE ? p.ids[(size_t)b * LK + (size_t)(en.eDep[i] - 1) * K + en.eRank[i]] : -1;
  }
  const double top = sm.sig[1];  // the best prefix: depth 1, rank 0
  const double span = top - tau;
  const double scale = PRE_SCALE ? sm.oscale : (span > 0.0 ? (double)kSelBins / span : 0.0);
  auto bin_of = [&](double sc) -> int {
    const double t = (top - sc) * scale;
    return t >= (double)(kSelBins - 1) ? kSelBins - 1 : (t > 0.0 ? (int)t : 0);
  };
  if constexpr (ZERO_HIST) {
    for (int j = tid; j < kSelBins; j += NT) sm.hist[j] = 0;
    __syncthreads();
  }
  int ebin[NPT];
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int i = tid + k * NT;
    ebin[k] = i < nE ? bin_of(en.eSc[i]) : kSelBins;
    if (i < nE) atomicAdd(&sm.hist[ebin[k]], 1);
  }
  __syncthreads();
  {
    // scan: this thread's BPT consecutive bins, then the waves' totals
    int h[BPT], hs = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      h[j] = sm.hist[tid * BPT + j];
      hs += h[j];
    }
    const int x = wave_incl_scan(hs);
    const int lane = tid & 63, w = tid >> 6;
    if (lane == kWave - 1) sm.wsum[w] = x;
    __syncthreads();
    int tot;
    int run = waves_before<NW>(sm.wsum, w, tot) + x - hs;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int bin = tid * BPT + j, exc = run;
      run += h[j];
      // the first bin reaching B is the cut (the last bin when nE <= B)
      if (nE > B ? (run >= B && exc < B) : bin == kSelBins - 1) sm.kcut = bin;
      sm.hexc[bin] = exc;
      sm.hist[bin] = 0;  // now the bins' fill counters (only this thread read it)
    }
  }
  __syncthreads();
  const int kcut = sm.kcut;
  // E2 in bin order, with compact copies of the order keys: scores in eS,
  // rank keys in the (dead) table of row values
  double* s2 = en.eS;
  uint64_t* h2 = (uint64_t*)sm.v;
  uint64_t* l2 = h2 + kECap;
  static_assert(2 * kECap * sizeof(uint64_t) <= sizeof(sm.v), "rank keys fit the row table");
  int epos[NPT];
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int i = tid + k * NT;
    epos[k] = -1;
    if (i < nE && ebin[k] <= kcut) {
      const int q = sm.hexc[ebin[k]] + atomicAdd(&sm.hist[ebin[k]], 1);
      epos[k] = q;
      s2[q] = en.eSc[i];
      h2[q] = en.eLh[i];
      l2[q] = en.eLl[i];
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int i = tid + k * NT;
    if (epos[k] >= 0) {
      const int bb = ebin[k], me = epos[k];
      const int lo = sm.hexc[bb], hi = bb + 1 < kSelBins ? sm.hexc[bb + 1] : nE;
      const double si = s2[me];
      const uint64_t hi_i = h2[me], lo_i = l2[me];
      int rank = lo;
      // the bin's members four at a time, their loads issued together (an
      // index past the bin reads this entry itself, which never precedes it)
      for (int q = lo; q < hi; q += 4) {
        double sq[4];
        uint64_t hq[4], lq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int qq = q + j < hi ? q + j : me;
          sq[j] = s2[qq];
          hq[j] = h2[qq];
          lq[j] = l2[qq];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          rank += (sq[j] > si || (sq[j] == si && (hq[j] < hi_i || (hq[j] == hi_i && lq[j] < lo_i))))
                      ? 1
                      : 0;
      }
      en.cnt[i] = rank;
    }
  }
  __syncthreads();
  const int nsel = nE < B ? nE : B;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int i = tid + k * NT;
    if (epos[k] >= 0) {
      const int j = en.cnt[i];
      if (j < nsel) {
        // a parent of an output node is an earlier output node
        const size_t o = (size_t)b * B + j;
        const int pe = en.ePar[i];
        const int par = pe < 0 ? 0 : en.cnt[pe] + 1;
        p.tree_tokens[o] = etok[k];
        p.parents[o] = par;
        p.logq[o] = (float)en.eSc[i];
        if (p.depths) p.depths[o] = en.eDep[i];
        sm.opar[j] = par;
      }
    }
  }
  for (int j = nsel + tid; j < B; j += NT) {
    const size_t o = (size_t)b * B + j;
    p.tree_tokens[o] = -1;
    p.parents[o] = -1;
    p.logq[o] = -INFINITY;
    if (p.depths) p.depths[o] = 0;
  }
  if (tid == 0) {
    p.num_nodes[b] = nsel;
    sm.nsel = nsel;
  }
  __syncthreads();
}

// Phase 4: the bit-packed ancestor mask from the emitted parents (opar[j] =
// parent node number of node j+1, in LDS; nodes past nsel get zero rows).
// One thread per (row, 64-bit word): it walks the row's ancestor chain and
// keeps the bits that fall in its word, so consecutive threads write
// consecutive words.
template <int NT = kSelThreads>
__device__ __forceinline__ void sel_mask_rows(const SelectParams& p, const int* opar, int nsel,
                                              int64_t b) {
  if (!p.mask) return;
  const int B = p.B, W = p.W;
  uint64_t* dst = p.mask + (size_t)b * (B + 1) * W;
  for (int t = threadIdx.x; t < (B + 1) * W; t += NT) {
    const int i = (int)(((uint64_t)(uint32_t)t * p.wmag) >> 32), q = t - i * W;  // t / W
    uint64_t m = 0;
    if (i <= nsel) {
      int u = i;
      for (int step = 0; step <= kMaxL + 1; ++step) {
        m |= (u >> 6) == q ? 1ull << (u & 63) : 0ull;
        if (u == 0) break;
        u = opar[u - 1];
      }
    }
    dst[t] = m;
  }
}

template <int NT = kSelThreads>
__device__ __forceinline__ void sel_mask(const SelectParams& p, SelectSmem& sm, int64_t b) {
  sel_mask_rows<NT>(p, sm.opar, sm.nsel, b);
}

// Inclusive scan over the wave of op(a, b) = (b > a ? a : b), a from the
// earlier lanes: the running minimum in which a later equal value replaces
// an earlier one. By DPP, in the order of the integer scan above (shifts by
// 1, 2, 4, 8 inside rows, then row broadcasts); a lane without a partner
// sees +inf. For non-NaN values op is associative, so every lane gets the
// left-to-right fold's value bit for bit.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64_or_inf(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWS, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)0x7FF00000, (int)(uint32_t)(u >> 32),
                                                            CTRL, ROWS, 0xf, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double wave_runmin_scan(double x) {
  auto op = [](double a, double b) { return b > a ? a : b; };
  x = op(dpp_f64_or_inf<0x111, 0xf>(x), x);  // row_shr:1
  x = op(dpp_f64_or_inf<0x112, 0xf>(x), x);  // row_shr:2
  x = op(dpp_f64_or_inf<0x114, 0xf>(x), x);  // row_shr:4
  x = op(dpp_f64_or_inf<0x118, 0xf>(x), x);  // row_shr:8
  x = op(dpp_f64_or_inf<0x142, 0xa>(x), x);  // row_bcast:15
  x = op(dpp_f64_or_inf<0x143, 0xc>(x), x);  // row_bcast:31
  return x;
}

__global__ __launch_bounds__(kSelNT) void select_kernel(SelectParams p) {
  constexpr int NT = kSelNT, NW = NT / kWave, NPT = kECap / NT;
  static_assert(NPT * NT == kECap, "whole entries per thread");
  __shared__ SelectSmem sm;
  SelEnum& en = sm.u.en;
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int L = p.L, K = p.K, B = p.B, LK = L * K, bpd = p.bpd;
  const float* vals = p.vals + (size_t)b * LK;
  // the threshold's lower-bound rank: the q1-th one-deviation score of every
  // row, q1 = min(ceil(B / L), K) in [1, K], leaves >= B scores at or above
  // the smallest
  const int q1 = p.q1;

  if (tid < kWave) {
    // Z_d and the spine (all ranks 0), float64, in wave 0's registers while
    // the other waves stage the table. Lane d sums rows 0..d-1 itself, left
    // to right, so every lane gets its own prefix with the additions of the
    // serial definition; the chain is unrolled over the first rows, whose
    // values every lane loads (same addresses across the wave), and the
    // lanes past their own row sit out the additions.
    const int lane = tid;
    // lane d holds row d's normaliser, top value, last value and rank-q1
    // value (four loads issued together: clamped addresses, no branches)
    const int lc = lane < L ? lane : 0;
    const double zl0 = p.lse[(size_t)b * L + lc];
    const float* vrow = vals + (size_t)lc * K;
    const float vl0 = vrow[0], vk0 = vrow[K - 1], vq0 = vrow[q1 - 1];
    const double zl = lane < L ? zl0 : 0.0;
    const float vl = lane < L ? vl0 : 0.0f, vk = lane < L ? vk0 : 0.0f;
    const float vq = lane < L ? vq0 : 0.0f;
    constexpr int kPre = 15;  // rows whose values every lane holds
    double zr[kPre];
    float vr[kPre];
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      const int jj = j < L ? j : 0;  // rows past L only reach lanes past L
      zr[j] = p.lse[(size_t)b * L + jj];
      vr[j] = vals[(size_t)jj * K];
    }
    double Zx = 0.0, Sx = 0.0;  // rows < d
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      if (j < lane) {
        Zx += zr[j];
        Sx += (double)vr[j];
      }
    }
    for (int j = kPre; j < L - 1; ++j) {  // deeper trees: broadcast by readlane
      const double zj = lane_value(zl, j);
      const double vj = (double)lane_value(vl, j);
      if (j < lane) {
        Zx += zj;
        Sx += vj;
      }
    }
    const double Zi = Zx + zl, Si = Sx + (double)vl;  // rows <= d: Z_d, P0[d+1]
    const double raw = lane < L ? Si - Zi : INFINITY;
    // spine scores sig[d+1] = the running minimum of 0, raw_0 .. raw_d (a
    // later equal value replaces an earlier one): a DPP scan when no score
    // is NaN (the operation is then associative), else serially
    double sg;
    if (__ballot(raw != raw) == 0) {
      sg = wave_runmin_scan(raw);
      sg = sg > 0.0 ? 0.0 : sg;
    } else {
      double sc = 0.0;
      sg = 0.0;
      for (int j = 0; j < L; ++j) {
        const double r = lane_value(raw, j);
        sc = r > sc ? sc : r;
        if (lane == j) sg = sc;
      }
    }
    // every row's top log-probability below -M, M far above the rounding of
    // any score (a difference of sums of magnitude <= the sum of every |Z_d|
    // and every row's largest |value|)
    const double mag = wave_sum(lane < L ? fabs(Zi) + (double)fmaxf(fabsf(vl), fabsf(vk)) : 0.0);
    const double M = 1e-12 * (1.0 + mag);
    const uint64_t ok = __ballot(lane >= L || (double)vl - zl < -M);
    if (LK >= B) {
      // the threshold's lower bound: the smallest rank-q one-deviation score
      // over the rows (the same arithmetic as the histogram's)
      double sgx = __shfl_up(sg, 1);  // sig[d]
      sgx = lane == 0 ? 0.0 : sgx;
      const double r1 = (Sx + (double)vq) - Zi;
      const double od = lane < L ? (r1 > sgx ? sgx : r1) : INFINITY;
      const double mn = wave_min(od);
      if (lane == 0) {  // lane 0's sg is sig[1], the best score
        sm.tau = mn;
        sm.n2 = 0;
        const double span = sg - mn;
        sm.hscale = span > 0.0 ? (double)kSelBins / span : 0.0;
      }
    }
    if (lane < L) {
      sm.Z[lane] = Zi;
      sm.P0[lane + 1] = Si;
      sm.sig[lane + 1] = sg;
    }
    if (lane == 0) {
      sm.P0[0] = 0.0;
      sm.sig[0] = 0.0;
      sm.nE = 0;
      sm.ovf = 0;
      sm.f2 = ok == ~0ull ? 1 : 0;
      sm.wbad[0] = 0;
    }
  } else {
    // waves 1..: stage the table, clear the threshold's histogram, and check
    // the exact-sum window: every nonzero value's exponent within 11 of the
    // first row's top value's (denormals count as exponent 1)
    constexpr int NS = NT - kWave;  // staging threads
    const int eref = (int)((__float_as_uint(vals[0]) >> 23) & 0xFFu);
    bool bad = false;
    auto check = [&](float v) {
      int e = (int)((__float_as_uint(v) >> 23) & 0xFFu);
      e = e == 0 ? 1 : e;
      bad |= v != 0.0f && (e == 255 || e < eref - 11 || e > eref + 11);
    };
    // two values per thread per step, both loads in flight together
    for (int i = tid - kWave; i < LK; i += 2 * NS) {
      const bool two = i + NS < LK;
      const float v0 = vals[i], v1 = vals[two ? i + NS : i];
      __builtin_amdgcn_sched_barrier(0);  // both loads issued before the first store
      sm.v[i] = v0;
      if (two) sm.v[i + NS] = v1;
      check(v0);
      check(v1);
    }
    for (int j = tid - kWave; j < kSelBins; j += NT - kWave) sm.hist[j] = 0;
    const uint64_t wb = __ballot(bad);
    if ((tid & 63) == 0) sm.wbad[tid >> 6] = wb != 0 ? 1u : 0u;
  }
  __syncthreads();


  // ---- 1. threshold from the one-deviation prefixes -------------------------
  // The rows' one-deviation scores fall into kSelBins bins over [mn, best]
  // (mn, the lower bound, and the bins' scale are in place, the histogram
  // cleared); wave 0 then finds the bin holding the B-th and sets tau to its
  // lower edge moved down by a millionth of a bin (at or below every member
  // of that bin, so >= B scores reach it), and without a barrier goes on to
  // the spine entries reaching tau and the first generation's child counts.
  if (LK >= B) {
    const uint64_t kmag = p.kmag;  // row d = i / K by a multiply
    const double mn = sm.tau, top = sm.sig[1], scale = sm.hscale;
    for (int i = tid; i < LK; i += NT) {
      const int d = (int)(((uint64_t)(uint32_t)i * kmag) >> 32);
      const double raw = (sm.P0[d] + (double)sm.v[i]) - sm.Z[d];
      const double sc = raw > sm.sig[d] ? sm.sig[d] : raw;
      if (sc >= mn) {
        const double t = (top - sc) * scale;
        atomicAdd(&sm.hist[t >= (double)(kSelBins - 1) ? kSelBins - 1 : (t > 0.0 ? (int)t : 0)], 1);
      }
    }
    __syncthreads();
  }
  if (tid < kWave) {
    const int lane = tid;
    double t = -INFINITY;
    if (LK >= B) {
      // lane l sums bins [16 l, 16 l + 16); a wave scan; the lane whose
      // range reaches B walks its bins to the cut
      constexpr int BPL = kSelBins / kWave;
      int h[BPL], hs = 0;
#pragma unroll
      for (int j = 0; j < BPL; j += 4) {
        const int4 q = *(const int4*)&sm.hist[lane * BPL + j];
        h[j] = q.x;
        h[j + 1] = q.y;
        h[j + 2] = q.z;
        h[j + 3] = q.w;
        hs += q.x + q.y + q.z + q.w;
      }
      const int inc = wave_incl_scan(hs);
      int run = inc - hs, kc = kSelBins;
#pragma unroll
      for (int j = 0; j < BPL; ++j) {
        const int exc = run;
        run += h[j];
        if (run >= B && exc < B) kc = lane * BPL + j;
      }
      kc = wave_min(kc);  // the one lane that holds the cut
      const double mn = sm.tau, top = sm.sig[1], scale = sm.hscale;
      t = mn;
      if (scale > 0.0 && kc < kSelBins - 1) {
        const double edge = top - ((double)kc + 1.000001) / scale;
        t = edge > mn ? edge : mn;
      }
    }
    // spine prefixes reaching t (the spine's scores do not increase)
    const int D0 = __popcll(__ballot(lane < L && sm.sig[lane + 1] >= t));
    if (lane < D0) {
      en.eS[lane] = sm.P0[lane + 1];
      en.eSc[lane] = sm.sig[lane + 1];
      en.ePar[lane] = (int16_t)(lane - 1);
      en.eRank[lane] = 0;
      en.eDep[lane] = (uint8_t)(lane + 1);
      en.eLh[lane] = 0;
      en.eLl[lane] = (uint64_t)(lane + 1);
    }
    // the first generation's parents: the root (lane 0, depth 0) and spine
    // entry u - 1 (lane u, depth u, sum P0[u]); deviating children reaching
    // t counted by binary search in the sorted row, the count search's test
    int c = 0;
    if (lane <= D0 && lane < L) {
      const double S = lane == 0 ? 0.0 : sm.P0[lane];
      const float* row = sm.v + lane * K;
      const double Zd = sm.Z[lane];
      int lo = 1, hi = K;  // first failing rank lies in [lo, hi]
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((S + (double)row[mid]) - Zd >= t) lo = mid + 1;
        else hi = mid;
      }
      c = lo - 1;
    }
    const int cinc = wave_incl_scan(c);
    if (lane <= D0) en.own[lane] = (uint32_t)(cinc - c);  // parents' first anchor slots
    if (lane == kWave - 1) sm.A1 = cinc;
    if (lane == 0) {
      sm.tau = t;
      sm.nE = D0;
      sm.ncand = 0;
      const double span = sm.sig[1] - t;  // the ordering's scale for this tau
      sm.oscale = span > 0.0 ? (double)kSelBins / span : 0.0;
    }
  }
  __syncthreads();
  double tau = sm.tau;

  // Fast path: sums of row values are exact (their exponents span <= 22, so
  // every S is the same whatever the summation order) and no score clamps
  // (every step along a path lowers the score by more than any rounding).
  // Then a rank-0 extension to depth e scores (S + (P0[e] - P0[d])) - Z[e-1]
  // directly, strictly decreasing in e: chains are found by binary search.
  uint32_t anybad = 0;  // the waves' flags, four per 16-byte read
#pragma unroll
  for (int i = 0; i < NW; i += 4) {
    const uint4 t = *(const uint4*)&sm.wbad[i];
    anybad |= t.x | t.y | t.z | t.w;
  }
  const bool fast = sm.f2 != 0 && anybad == 0;
  // ---- 2. enumerate E = {score >= tau} by chains ----------------------------
  // If E outgrows its capacity, every entry found so far is a valid prefix
  // scoring >= tau: the B-th best of them is a valid, usually much tighter,
  // threshold, and the enumeration restarts from it (kSelRetries times at
  // most, then the heap).
  for (int attempt = 0;; ++attempt) {
    int D0;
    if (attempt == 0) {
      D0 = sm.nE;  // wave 0's spine entries, counts and offsets are in place
    } else {
      // spine prefixes reaching tau (the spine's scores do not increase):
      // one ballot over L <= 32 lanes
      D0 = __popcll(__ballot((tid & 63) < L && sm.sig[(tid & 63) + 1] >= tau));
      for (int d = tid; d < D0; d += NT) {
        en.eS[d] = sm.P0[d + 1];
        en.eSc[d] = sm.sig[d + 1];
        en.ePar[d] = (int16_t)(d - 1);
        en.eRank[d] = 0;
        en.eDep[d] = (uint8_t)(d + 1);
        en.eLh[d] = 0;
        en.eLl[d] = (uint64_t)(d + 1);
      }
      if (tid == 0) {
        sm.nE = D0;
        const double span = sm.sig[1] - tau;  // the ordering's scale for this tau
        sm.oscale = span > 0.0 ? (double)kSelBins / span : 0.0;
      }
      for (int j = tid; j < kSelBins; j += NT) sm.hist[j] = 0;  // the ordering's histogram
      __syncthreads();
    }
    int g0 = 0, g1 = D0, root = 1;
    // A generation's parents are either all entries of the previous one
    // ([g0, g1), after the root for the first), counted by the whole block,
    // or, when at most kWave of them have deviating children, just those
    // (listed while they were written), counted by wave 0 alone.
    bool counted = attempt == 0;  // the first generation counted by wave 0
    bool listed = false;          // parents are pcand[0 .. np)
    for (;;) {
      int np = root + (g1 - g0);
      uint32_t* poff = en.own;  // parents' first anchor slots
      int A;
      if (counted) {
        counted = false;
        A = sm.A1;
        if (listed) np = sm.np1;
        if (tid == 0) sm.ncand = 0;  // every wave read it before the last barrier
        // the ordering's histogram (the threshold's scan read it before the
        // last barrier)
        if (root) for (int j = tid; j < kSelBins; j += NT) sm.hist[j] = 0;
        if (A == 0 || A > kECap) {
          if (tid == 0 && A > kECap) sm.ovf = 1;  // more new anchors than entries fit
          __syncthreads();
          break;
        }
      } else {
      if (np > kECap) {  // parents must fit the count array
        if (tid == 0) sm.ovf = 1;
        __syncthreads();
        break;
      }
      // deviating children (rank >= 1) of each parent that reach tau, counted
      // by binary search in the sorted row; ceil(np / NT) <= NPT parents per
      // thread, consecutive, so the offsets follow parent order
      const int ppt = (np + NT - 1) / NT;
      int cpar[NPT], csum = 0;
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        cpar[k] = 0;
        const int i = tid * ppt + k;
        if (k < ppt && i < np) {
          double S = 0.0;
          int d = 0;
          if (!(root && i == 0)) {
            const int e = g0 + i - root;
            S = en.eS[e];
            d = en.eDep[e];
          }
          if (d < L) {
            const float* row = sm.v + d * K;
            const double Zd = sm.Z[d];
            int lo = 1, hi = K;  // first failing rank lies in [lo, hi]
            while (lo < hi) {
              const int mid = (lo + hi) >> 1;
              if ((S + (double)row[mid]) - Zd >= tau) lo = mid + 1;
              else hi = mid;
            }
            cpar[k] = lo - 1;
          }
        }
        csum += cpar[k];
      }
      const int off = block_excl_scan_reg<NT>(csum, sm.wsum, A);
      if (A == 0) break;
      if (A > kECap) {  // more new anchors than entries fit
        if (tid == 0) sm.ovf = 1;
        __syncthreads();
        break;
      }
      // parents' first anchor slots (their exclusive offsets, which do not
      // decrease with the parent index): each anchor finds its parent by
      // binary search, so no thread writes a long run of labels
      {
        int run = off;
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
          const int i = tid * ppt + k;
          if (k < ppt && i < np) poff[i] = (uint32_t)run;
          run += cpar[k];
        }
      }
      __syncthreads();
      if (tid == 0) sm.ncand = 0;  // set below, read after this generation's last barrier
      }
      const int nE0 = sm.nE;
      // does an entry at depth dd with sum S have a deviating child (rank 1
      // of the next row) reaching tau? the count search's own test
      auto has_child = [&](int dd, double S) {
        return dd < L && K > 1 && (S + (double)sm.v[dd * K + 1]) - sm.Z[dd] >= tau;
      };
      auto note_child = [&](int e) {  // entry e has a deviating child
        const int ci = atomicAdd(&sm.ncand, 1);
        if (ci < kWave) sm.cand[ci] = e;
      };
      // anchors, consecutive per thread (ceil(A / NT) <= NPT of them): the
      // parent, S and score, and the chain length -- the anchor, then its
      // rank-0 extensions while they reach tau (S summed left to right, the
      // next four depths' spine values read per step)
      const int apt = (A + NT - 1) / NT;
      double aS[NPT], aSc[NPT];
      uint64_t aLh[NPT], aLl[NPT];
      int aD[NPT], aPe[NPT], aR[NPT], aEll[NPT], esum = 0;
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        aEll[k] = 0;  // 0: no anchor in this slot
        const int a = tid * apt + k;
        if (k < apt && a < A) {
          int lo = 0, hi = np - 1;  // the last parent whose first slot is <= a
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((int)poff[mid] <= a) lo = mid;
            else hi = mid - 1;
          }
          const int u = lo;
          const int r = a - (int)poff[u] + 1;
          double Su = 0.0, scu = 0.0;
          int du = 0, pe = -1;
          uint64_t lh = 0, ll = 0;
          if (!(root && u == 0)) {
            pe = listed ? sm.pcand[u] : g0 + u - root;
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
          bool alive = !fast;
          double S2 = S, sc2 = sc;
          if (fast) {
            // the deepest e in [d, L] with (S + (P0[e] - P0[d])) - Z[e-1] >= tau
            const double pd = sm.P0[d];
            int lo2 = d, hi2 = L;
            while (lo2 < hi2) {
              const int mid = (lo2 + hi2 + 1) >> 1;
              if ((S + (sm.P0[mid] - pd)) - sm.Z[mid - 1] >= tau) lo2 = mid;
              else hi2 = mid - 1;
            }
            ell = lo2 - d + 1;
          }
          for (int dd0 = d + 1; dd0 <= L && alive; dd0 += 4) {
            float v4[4];
            double z4[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int row = (dd0 + q <= L ? dd0 + q : L) - 1;
              v4[q] = sm.v[row * K];
              z4[q] = sm.Z[row];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const bool valid = alive && dd0 + q <= L;
              const double S3 = S2 + (double)v4[q];
              const double raw2 = S3 - z4[q];
              const double sc3 = raw2 > sc2 ? sc2 : raw2;
              alive = valid && sc3 >= tau;
              S2 = alive ? S3 : S2;
              sc2 = alive ? sc3 : sc2;
              ell += alive ? 1 : 0;
            }
          }
          aS[k] = S;
          aSc[k] = sc;
          aLh[k] = lh;
          aLl[k] = ll;
          aD[k] = d;
          aPe[k] = pe;
          aR[k] = r;
          aEll[k] = ell;
        }
        esum += aEll[k];
      }
      // slots in anchor order: a block scan of the chain lengths; the
      // anchor entries first, and every slot of a chain labelled with its
      // anchor's slot (the parents' offsets are dead after the scan)
      int T;
      const int aoff = block_excl_scan_reg<NT>(esum, sm.wsum, T);
      uint32_t* aslot = en.own;
      int arun = nE0 + aoff;
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        const int a = tid * apt + k;
        const int pos = arun;
        arun += aEll[k];
        if (k < apt && a < A) {
          const int pend = pos + aEll[k] < kECap ? pos + aEll[k] : kECap;
          for (int q = pos; q < pend; q += 4) {  // four labels per step
            aslot[q] = (uint32_t)pos;
            if (q + 1 < pend) aslot[q + 1] = (uint32_t)pos;
            if (q + 2 < pend) aslot[q + 2] = (uint32_t)pos;
            if (q + 3 < pend) aslot[q + 3] = (uint32_t)pos;
          }
          if (pos < kECap) {
            if (has_child(aD[k], aS[k])) note_child(pos);
            en.eS[pos] = aS[k];
            en.eSc[pos] = aSc[k];
            en.ePar[pos] = (int16_t)aPe[k];
            en.eRank[pos] = (uint16_t)aR[k];
            en.eDep[pos] = (uint8_t)aD[k];
            en.eLh[pos] = aLh[k];
            en.eLl[pos] = aLl[k] | (uint64_t)aD[k];
          }
        }
      }
      const int nEnd = nE0 + T < kECap ? nE0 + T : kECap;
      __syncthreads();
      if (tid == 0) {
        sm.nE = nE0 + T;
        // entries [0, kECap) stay valid prefixes scoring >= tau
        if (nE0 + T > kECap) sm.ovf = 1;
      }
      // chain entries, one thread per slot: its anchor's slot from the
      // label, then S summed left to right from the anchor's and the
      // score's running minimum along the chain
      for (int q = nE0 + tid; q < nEnd; q += NT) {
        const int pa = (int)aslot[q], j = q - pa;
        if (j == 0) continue;
        const int d = en.eDep[pa];
        double S2 = en.eS[pa], sc2 = en.eSc[pa];
        if (fast) {
          S2 += sm.P0[d + j] - sm.P0[d];
          sc2 = S2 - sm.Z[d + j - 1];
        } else {
          for (int i = 1; i <= j; ++i) {
            const int row = d + i - 1;  // depth d + i
            S2 += (double)sm.v[row * K];
            const double raw2 = S2 - sm.Z[row];
            sc2 = raw2 > sc2 ? sc2 : raw2;
          }
        }
        if (has_child(d + j, S2)) note_child(q);
        en.eS[q] = S2;
        en.eSc[q] = sc2;
        en.ePar[q] = (int16_t)(q - 1);
        en.eRank[q] = 0;
        en.eDep[q] = (uint8_t)(d + j);
        en.eLh[q] = en.eLh[pa];
        en.eLl[q] = (en.eLl[pa] & ~63ull) | (uint64_t)(d + j);
      }
      __syncthreads();
      // no entry of this generation has a deviating child: the next
      // generation would find no anchors
      const int nc = sm.ncand;
      if (sm.ovf || nc == 0) break;
      g0 = g1;
      g1 = sm.nE;
      root = 0;
      listed = nc <= kWave;
      if (listed) {
        // wave 0 counts the listed parents' deviating children reaching tau
        // (the count search's test) and lays out their first anchor slots
        if (tid < kWave) {
          const int lane = tid;
          int c = 0, e = 0;
          if (lane < nc) {
            e = sm.cand[lane];
            const double S = en.eS[e];
            const int d = en.eDep[e];
            if (d < L) {
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
          }
          const int cinc = wave_incl_scan(c);
          if (lane < nc) {
            poff[lane] = (uint32_t)(cinc - c);
            sm.pcand[lane] = e;
          }
          if (lane == kWave - 1) sm.A1 = cinc;
          if (lane == 0) sm.np1 = nc;
        }
        __syncthreads();
        counted = true;
      }
    }
    if (!sm.ovf) break;
    // overflow: entries [0, n) are prefixes scoring >= tau
    const int n = sm.nE < kECap ? sm.nE : kECap;
    if (attempt == kSelRetries || n < B) break;
    const double t1 = sel_tau_hist<true, NT>(
        sm, n, B, [&](int i) { return en.eSc[i]; }, [&](int) { return tau; },
        reinterpret_cast<double*>(en.eLh), kECap);
    if (!(t1 > tau)) break;
    tau = t1;
    if (tid == 0) sm.ovf = 0;
    __syncthreads();
  }

  if (sm.ovf) {
    __syncthreads();
    if (tid == 0) heap_fallback(p, sm, b);
    __syncthreads();
  } else {
    sel_order_emit<false, NT, true>(p, sm, b, tau);
  }
  sel_mask<NT>(p, sm, b);
}

}  // namespace ddt
