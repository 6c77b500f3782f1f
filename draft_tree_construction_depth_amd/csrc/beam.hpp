// Fixed-branching beam tree on SparklingTree's conditioned rows
// (SparklingTree post, "Future Ideas", item 4: a beam with a fixed branching
// budget instead of the best-first heap, branches spread evenly over the
// depths).
//
// Rows as for sparkling_build: row 1 = the first drafter row over its top C
// candidates; the children of a node holding candidate c at depth d are row
// d+1 conditioned on c (the table `lp` of sp_table_kernel). Depth by depth,
// the beam keeps the w_d best children of the previous depth's beam: score
// (sum of lp along the path, float64) desc, then rank tuple lexicographic asc
// (a child's rank = its position in its row by lp desc, token asc). The tree
// is every beam node, emitted depth by depth in beam order.
//
// MI355X design: one 256-thread workgroup per request (a depth is a chain of
// short block-synchronous steps: small workgroups synchronise faster),
// widths <= 64, so a depth has at most 64 x 128 candidates. Their scores and
// log-probs go to LDS; the w-th best is found by a histogram over [min, max]
// (256 bins, monotone in the score)
// and one scan; the bins above the cut are taken whole, the cut bin is
// resolved exactly with full keys (each member's rank in its row by counting,
// then counting among the members), or, when it holds more than kBmCut
// members (flat rows, exact ties), by extracting its best member w times.
// The new beam is ordered by full key (counting among <= 64 entries).
#pragma once

#include "common.hpp"
#include "select.hpp"
#include "sparkling.hpp"

namespace ddt {

constexpr int kBmThreads = 256;
constexpr int kBmWaves = kBmThreads / kWave;
constexpr int kBmMaxW = 64;
constexpr int kBmMaxM = kBmMaxW * kSpC;  // candidates of one depth, at most
constexpr int kBmBins = kBmThreads;
constexpr int kBmCut = 512;  // cut-bin members ranked by counting, at most

struct BeamParams {
  SelectParams sp;         // vals, ids, L, K = C, B, bpd, outputs, mask, W, sp_lp
  int32_t widths[kMaxL];   // beam width per depth (<= kBmMaxW)
};

struct BeamSmem {
  double cs[kBmMaxM];         // candidate scores of the current depth
  float clp[kBmMaxM];         // their log-probs (the beam's rows, in LDS for ranking)
  float lp0[kSpC];            // row 1 over its candidates
  int32_t tok[kSpMaxLC];      // [L][C] candidate tokens
  // the beam of the previous depth (entry u: candidate c, score, rank key, node)
  int32_t bc[kBmMaxW];
  double bS[kBmMaxW];
  uint64_t bh[kBmMaxW], bl[kBmMaxW];
  int32_t bnode[kBmMaxW];
  // the selection of the current depth
  int32_t sel[kBmMaxW];       // candidate index m = u * C + j
  int32_t srank[kBmMaxW];     // child rank of each selected candidate
  double sS[kBmMaxW];         // and its key: score, parent rank key
  uint64_t sH[kBmMaxW], sL[kBmMaxW];
  int32_t cut[kBmCut];        // members of the cut bin
  int32_t crank[kBmCut];      // their child ranks
  double cS[kBmCut];          // and their keys
  uint64_t cH[kBmCut], cL[kBmCut];
  int hist[kBmBins];
  alignas(16) int wsum[kBmWaves];
  double rmin[kBmWaves], rmax[kBmWaves];
  int opar[kMaxB];            // the tree, written out at the end
  int otok[kMaxB];
  float oq[kMaxB];
  uint8_t odep[kMaxB];
  int nsel, ncut, kcut, kexc, nprev, nout;
  int pick;
  uint64_t taken[kBmMaxM / 64];  // cut members already extracted (fallback)
};

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global memory operations (which
// __syncthreads() drains as well).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// the child rank of candidate j in row `r` of tokens `t`: entries before it
// by (lp desc, token asc)
__device__ __forceinline__ int bm_rank(const float* r, const int32_t* t, int C, int j) {
  const float v = r[j];
  const int tj = t[j];
  int n = 0;
  for (int q = 0; q < C; ++q) n += (r[q] > v || (r[q] == v && t[q] < tj)) ? 1 : 0;
  return n;
}

// the same, one wavefront for one candidate: two compares a lane, ballots
__device__ __forceinline__ int bm_rank_wave(const float* r, const int32_t* t, int C, int j) {
  const int lane = threadIdx.x & (kWave - 1);
  const float v = r[j];
  const int tj = t[j];
  int n = 0;
  for (int q0 = 0; q0 < C; q0 += kWave) {
    const int q = q0 + lane;
    const bool bt = q < C && (r[q] > v || (r[q] == v && t[q] < tj));
    n += __popcll(__ballot(bt));
  }
  return n;
}

// full key order of two candidates: score desc, then parent key asc, then
// child rank asc (parent keys differ for different parents)
__device__ __forceinline__ bool bm_before(double sa, uint64_t ha, uint64_t la, int ra, double sb,
                                          uint64_t hb, uint64_t lb, int rb) {
  if (sa != sb) return sa > sb;
  if (ha != hb) return ha < hb;
  if (la != lb) return la < lb;
  return ra < rb;
}

__global__ __launch_bounds__(kBmThreads) void beam_kernel(BeamParams bp) {
  __shared__ BeamSmem sm;
  const SelectParams& p = bp.sp;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t b = blockIdx.x;
  const int L = p.L, C = p.K, B = p.B, LC = L * C, bpd = p.bpd;
  // m / C by a multiply with the host's ceil(2^32 / C) (exact for m C < 2^32)
  const uint64_t cmag = p.kmag;
  auto divC = [&](int m) { return (int)(((uint64_t)(uint32_t)m * cmag) >> 32); };
  const float* lpb = p.sp_lp + (size_t)b * (L - 1) * C * C;
  for (int i = tid; i < LC; i += kBmThreads) sm.tok[i] = p.ids[(size_t)b * LC + i];
  if (wv == 0) {
    // row 1 over its candidates (as the SparklingTree selection)
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
#pragma unroll
    for (int q = 0; q < kSpC / kWave; ++q) {
      const int j = lane + q * kWave;
      if (j < C) sm.lp0[j] = x[q] - lse;
    }
  }
  if (tid == 0) {
    sm.nprev = 1;  // the root
    sm.bc[0] = 0;
    sm.bS[0] = 0.0;
    sm.bh[0] = 0;
    sm.bl[0] = 0;
    sm.bnode[0] = 0;
    sm.nout = 0;
  }
  __syncthreads();
  for (int d = 0; d < L; ++d) {
    const int np = sm.nprev;
    const int w = bp.widths[d];
    if (np == 0 || w == 0) break;
    const int M = np * C;
    const int32_t* tk = sm.tok + d * C;
    auto row = [&](int u) -> const float* {
      return d == 0 ? sm.lp0 : lpb + ((size_t)(d - 1) * C + sm.bc[u]) * C;
    };
    // ---- candidate scores, their range --------------------------------------
    double mn = INFINITY, mxs = -INFINITY;
    for (int m = tid; m < M; m += kBmThreads) {
      const int u = divC(m), j = m - u * C;
      const float v = row(u)[j];
      const double s = sm.bS[u] + (double)v;
      sm.cs[m] = s;
      sm.clp[m] = v;
      mn = s < mn ? s : mn;
      mxs = s > mxs ? s : mxs;
    }
    int nsel = 0;  // candidates taken before the cut bin's
    if (w >= M) {
      for (int m = tid; m < M; m += kBmThreads) {
        const int u = divC(m);
        sm.sel[m] = m;
        sm.sS[m] = sm.cs[m];
        sm.sH[m] = sm.bh[u];
        sm.sL[m] = sm.bl[u];
      }
      nsel = M;
      lds_barrier();
    } else {
      mn = wave_min(mn);
      mxs = wave_max(mxs);
      if (lane == 0) {
        sm.rmin[wv] = mn;
        sm.rmax[wv] = mxs;
      }
      sm.hist[tid] = 0;
      if (tid == 0) {
        sm.ncut = 0;
        sm.nsel = 0;
      }
      lds_barrier();
      mn = sm.rmin[0];
      mxs = sm.rmax[0];
      for (int q = 1; q < kBmWaves; ++q) {
        mn = sm.rmin[q] < mn ? sm.rmin[q] : mn;
        mxs = sm.rmax[q] > mxs ? sm.rmax[q] : mxs;
      }
      const double span = mxs - mn;
      const double scale = span > 0.0 ? (double)kBmBins / span : 0.0;
      auto bin_of = [&](double s) -> int {
        const double t = (mxs - s) * scale;
        return t >= (double)(kBmBins - 1) ? kBmBins - 1 : (t > 0.0 ? (int)t : 0);
      };
      for (int m = tid; m < M; m += kBmThreads) atomicAdd(&sm.hist[bin_of(sm.cs[m])], 1);
      lds_barrier();
      {
        const int h = sm.hist[tid];
        const int x = wave_incl_scan(h);
        if (lane == kWave - 1) sm.wsum[wv] = x;
        lds_barrier();
        int pre = 0;
        for (int q = 0; q < wv; ++q) pre += sm.wsum[q];
        const int inc = pre + x, exc = inc - h;
        if (inc >= w && exc < w) {
          sm.kcut = tid;
          sm.kexc = exc;
        }
      }
      lds_barrier();
      const int kc = sm.kcut;
      nsel = sm.kexc;  // taken whole: the bins before the cut
      for (int m = tid; m < M; m += kBmThreads) {
        const double sc = sm.cs[m];
        const int bn = bin_of(sc);
        const int u = divC(m);
        if (bn < kc) {
          const int k = atomicAdd(&sm.nsel, 1);
          sm.sel[k] = m;
          sm.sS[k] = sc;
          sm.sH[k] = sm.bh[u];
          sm.sL[k] = sm.bl[u];
        } else if (bn == kc) {
          const int k = atomicAdd(&sm.ncut, 1);
          if (k < kBmCut) {
            sm.cut[k] = m;
            sm.cS[k] = sc;
            sm.cH[k] = sm.bh[u];
            sm.cL[k] = sm.bl[u];
          }
        }
      }
      lds_barrier();
      const int nc = sm.ncut, need = w - nsel;
      if (nc <= kBmCut) {
        // members' child ranks, then their order by full key
        for (int k = wv; k < nc; k += kBmWaves) {
          const int m = sm.cut[k], u = divC(m);
          const int r = bm_rank_wave(sm.clp + u * C, tk, C, m - u * C);
          if (lane == 0) sm.crank[k] = r;
        }
        lds_barrier();
        for (int k = tid; k < nc; k += kBmThreads) {
          const double s = sm.cS[k];
          const uint64_t h = sm.cH[k], l = sm.cL[k];
          const int r = sm.crank[k];
          int pos = 0;
          for (int q = 0; q < nc; ++q)
            pos += bm_before(sm.cS[q], sm.cH[q], sm.cL[q], sm.crank[q], s, h, l, r) ? 1 : 0;
          if (pos < need) {
            const int o = nsel + pos;
            sm.sel[o] = sm.cut[k];
            sm.srank[o] = r;
            sm.sS[o] = s;
            sm.sH[o] = h;
            sm.sL[o] = l;
          }
        }
        lds_barrier();
      } else {
        // many exact ties: take the best remaining cut-bin candidate `need`
        // times (child ranks computed once)
        for (int q = tid; q < kBmMaxM / 64; q += kBmThreads) sm.taken[q] = 0;
        lds_barrier();
        for (int t = 0; t < need; ++t) {
          double bs = -INFINITY;
          uint64_t bh = ~0ull, bl = ~0ull;
          int br = 0x7FFFFFFF, bm = -1;
          for (int m = tid; m < M; m += kBmThreads) {
            if (bin_of(sm.cs[m]) != kc || ((sm.taken[m >> 6] >> (m & 63)) & 1)) continue;
            const int u = divC(m);
            const int r = bm_rank(sm.clp + u * C, tk, C, m - u * C);
            if (bm < 0 || bm_before(sm.cs[m], sm.bh[u], sm.bl[u], r, bs, bh, bl, br)) {
              bs = sm.cs[m];
              bh = sm.bh[u];
              bl = sm.bl[u];
              br = r;
              bm = m;
            }
          }
#pragma unroll
          for (int o = 1; o < kWave; o <<= 1) {
            const double os = __shfl_xor(bs, o);
            const uint64_t oh = __shfl_xor(bh, o), ol = __shfl_xor(bl, o);
            const int orr = __shfl_xor(br, o), om = __shfl_xor(bm, o);
            if (om >= 0 && (bm < 0 || bm_before(os, oh, ol, orr, bs, bh, bl, br))) {
              bs = os;
              bh = oh;
              bl = ol;
              br = orr;
              bm = om;
            }
          }
          if (lane == 0) {
            sm.cut[wv] = bm;
            sm.crank[wv] = br;
          }
          lds_barrier();
          if (tid == 0) {
            int best = -1;
            for (int q = 0; q < kBmWaves; ++q) {
              const int mq = sm.cut[q];
              if (mq < 0) continue;
              if (best < 0) {
                best = q;
                continue;
              }
              const int mb = sm.cut[best], ub = divC(mb), uq = divC(mq);
              if (bm_before(sm.cs[mq], sm.bh[uq], sm.bl[uq], sm.crank[q], sm.cs[mb], sm.bh[ub],
                            sm.bl[ub], sm.crank[best]))
                best = q;
            }
            const int mb = sm.cut[best], ub = divC(mb);
            sm.sel[nsel + t] = mb;
            sm.srank[nsel + t] = sm.crank[best];
            sm.sS[nsel + t] = sm.cs[mb];
            sm.sH[nsel + t] = sm.bh[ub];
            sm.sL[nsel + t] = sm.bl[ub];
            sm.taken[mb >> 6] |= 1ull << (mb & 63);
          }
          lds_barrier();
        }
      }
      nsel = w;
    }
    // ---- the new beam: child ranks of the whole-bin entries, keys, order ----
    const int cutfrom = w >= M ? M : sm.kexc;  // entries before it need their rank
    for (int k = wv; k < cutfrom; k += kBmWaves) {
      const int m = sm.sel[k], u = divC(m);
      const int r = bm_rank_wave(sm.clp + u * C, tk, C, m - u * C);
      if (lane == 0) sm.srank[k] = r;
    }
    lds_barrier();
    // entry k: candidate m, score, key = parent key + digit; its position by
    // counting; written straight into the next beam (staged in registers)
    int nb_c = 0, nb_node = 0, nb_pos = -1;
    double nb_S = 0.0;
    uint64_t nb_h = 0, nb_l = 0;
    if (tid < nsel) {
      const int m = sm.sel[tid], u = divC(m), j = m - u * C;
      const double s = sm.sS[tid];
      uint64_t h = sm.sH[tid], l = sm.sL[tid];
      const int r = sm.srank[tid];
      int pos = 0;
      for (int q = 0; q < nsel; ++q)
        pos += bm_before(sm.sS[q], sm.sH[q], sm.sL[q], sm.srank[q], s, h, l, r) ? 1 : 0;
      lex_set_digit(h, l, d + 1, (uint32_t)r, bpd);
      const int node = sm.nout + pos + 1;
      sm.otok[node - 1] = tk[j];
      sm.oq[node - 1] = (float)s;
      sm.odep[node - 1] = (uint8_t)(d + 1);
      sm.opar[node - 1] = sm.bnode[u];
      nb_c = j;
      nb_S = s;
      nb_h = h;
      nb_l = l;
      nb_node = node;
      nb_pos = pos;
    }
    lds_barrier();  // every read of the old beam is done
    if (nb_pos >= 0) {
      sm.bc[nb_pos] = nb_c;
      sm.bS[nb_pos] = nb_S;
      sm.bh[nb_pos] = nb_h;
      sm.bl[nb_pos] = nb_l;
      sm.bnode[nb_pos] = nb_node;
    }
    if (tid == 0) {
      sm.nprev = nsel;
      sm.nout += nsel;
    }
    lds_barrier();
  }
  const int nout = sm.nout;
  for (int j = tid; j < B; j += kBmThreads) {
    const size_t o = (size_t)b * B + j;
    const bool in = j < nout;
    p.tree_tokens[o] = in ? sm.otok[j] : -1;
    p.parents[o] = in ? sm.opar[j] : -1;
    p.logq[o] = in ? sm.oq[j] : -INFINITY;
    if (p.depths) p.depths[o] = in ? (int)sm.odep[j] : 0;
  }
  if (tid == 0) p.num_nodes[b] = nout;
  sel_mask_rows<kBmThreads>(p, sm.opar, nout, b);
}

}  // namespace ddt
