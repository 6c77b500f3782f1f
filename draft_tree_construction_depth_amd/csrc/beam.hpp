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
// MI355X design: one 1024-thread workgroup per request, widths <= 64, so a
// depth has at most 64 x 128 candidates. Their scores go to LDS; the w-th best
// is found by a histogram over [min, max] (1024 bins, monotone in the score)
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

constexpr int kBmMaxW = 64;
constexpr int kBmMaxM = kBmMaxW * kSpC;  // candidates of one depth, at most
constexpr int kBmBins = kSelThreads;
constexpr int kBmCut = 512;  // cut-bin members ranked by counting, at most

struct BeamParams {
  SelectParams sp;         // vals, ids, L, K = C, B, bpd, outputs, mask, W, sp_lp
  int32_t widths[kMaxL];   // beam width per depth (<= kBmMaxW)
};

struct BeamSmem {
  double cs[kBmMaxM];         // candidate scores of the current depth
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
  int32_t cut[kBmCut];        // members of the cut bin
  int32_t crank[kBmCut];      // their child ranks
  int16_t mrank[kBmMaxM];     // child ranks of the cut bin's members (tie fallback)
  int hist[kBmBins];
  alignas(16) int wsum[kSelWaves];
  double rmin[kSelWaves], rmax[kSelWaves];
  int opar[kMaxB];
  int nsel, ncut, kcut, kexc, nprev, nout;
  int pick;
  uint64_t taken[kBmMaxM / 64];  // cut members already extracted (fallback)
};

// the child rank of candidate j in row `r` of tokens `t`: entries before it
// by (lp desc, token asc)
__device__ __forceinline__ int bm_rank(const float* r, const int32_t* t, int C, int j) {
  const float v = r[j];
  const int tj = t[j];
  int n = 0;
  for (int q = 0; q < C; ++q) n += (r[q] > v || (r[q] == v && t[q] < tj)) ? 1 : 0;
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

__global__ __launch_bounds__(kSelThreads) void beam_kernel(BeamParams bp) {
  __shared__ BeamSmem sm;
  const SelectParams& p = bp.sp;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t b = blockIdx.x;
  const int L = p.L, C = p.K, B = p.B, LC = L * C, bpd = p.bpd;
  const float* lpb = p.sp_lp + (size_t)b * (L - 1) * C * C;
  for (int i = tid; i < LC; i += kSelThreads) sm.tok[i] = p.ids[(size_t)b * LC + i];
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
    for (int m = tid; m < M; m += kSelThreads) {
      const int u = m / C, j = m - u * C;
      const double s = sm.bS[u] + (double)row(u)[j];
      sm.cs[m] = s;
      mn = s < mn ? s : mn;
      mxs = s > mxs ? s : mxs;
    }
    int nsel = 0;  // candidates taken before the cut bin's
    if (w >= M) {
      for (int m = tid; m < M; m += kSelThreads) sm.sel[m] = m;
      nsel = M;
      __syncthreads();
    } else {
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const double a = __shfl_xor(mn, o), c = __shfl_xor(mxs, o);
        mn = a < mn ? a : mn;
        mxs = c > mxs ? c : mxs;
      }
      if (lane == 0) {
        sm.rmin[wv] = mn;
        sm.rmax[wv] = mxs;
      }
      sm.hist[tid] = 0;
      if (tid == 0) {
        sm.ncut = 0;
        sm.nsel = 0;
      }
      __syncthreads();
      mn = sm.rmin[0];
      mxs = sm.rmax[0];
      for (int q = 1; q < kSelWaves; ++q) {
        mn = sm.rmin[q] < mn ? sm.rmin[q] : mn;
        mxs = sm.rmax[q] > mxs ? sm.rmax[q] : mxs;
      }
      const double span = mxs - mn;
      const double scale = span > 0.0 ? (double)kBmBins / span : 0.0;
      auto bin_of = [&](double s) -> int {
        const double t = (mxs - s) * scale;
        return t >= (double)(kBmBins - 1) ? kBmBins - 1 : (t > 0.0 ? (int)t : 0);
      };
      for (int m = tid; m < M; m += kSelThreads) atomicAdd(&sm.hist[bin_of(sm.cs[m])], 1);
      __syncthreads();
      {
        const int h = sm.hist[tid];
        const int x = wave_incl_scan(h);
        if (lane == kWave - 1) sm.wsum[wv] = x;
        __syncthreads();
        int pre = 0;
        for (int q = 0; q < wv; ++q) pre += sm.wsum[q];
        const int inc = pre + x, exc = inc - h;
        if (inc >= w && exc < w) {
          sm.kcut = tid;
          sm.kexc = exc;
        }
      }
      __syncthreads();
      const int kc = sm.kcut;
      nsel = sm.kexc;  // taken whole: the bins before the cut
      for (int m = tid; m < M; m += kSelThreads) {
        const int bn = bin_of(sm.cs[m]);
        if (bn < kc) sm.sel[atomicAdd(&sm.nsel, 1)] = m;
        else if (bn == kc) {
          const int k = atomicAdd(&sm.ncut, 1);
          if (k < kBmCut) sm.cut[k] = m;
        }
      }
      __syncthreads();
      const int nc = sm.ncut, need = w - nsel;
      if (nc <= kBmCut) {
        // members' child ranks, then their order by full key
        for (int k = tid; k < nc; k += kSelThreads) {
          const int m = sm.cut[k], u = m / C;
          sm.crank[k] = bm_rank(row(u), tk, C, m - u * C);
        }
        __syncthreads();
        for (int k = tid; k < nc; k += kSelThreads) {
          const int m = sm.cut[k], u = m / C;
          const double s = sm.cs[m];
          const uint64_t h = sm.bh[u], l = sm.bl[u];
          const int r = sm.crank[k];
          int pos = 0;
          for (int q = 0; q < nc; ++q) {
            const int mq = sm.cut[q], uq = mq / C;
            pos += bm_before(sm.cs[mq], sm.bh[uq], sm.bl[uq], sm.crank[q], s, h, l, r) ? 1 : 0;
          }
          if (pos < need) {
            sm.sel[nsel + pos] = m;
            sm.srank[nsel + pos] = r;
          }
        }
        __syncthreads();
      } else {
        // many exact ties: take the best remaining cut-bin candidate `need`
        // times (child ranks computed once)
        for (int q = tid; q < kBmMaxM / 64; q += kSelThreads) sm.taken[q] = 0;
        for (int m = tid; m < M; m += kSelThreads)
          if (bin_of(sm.cs[m]) == kc) {
            const int u = m / C;
            sm.mrank[m] = (int16_t)bm_rank(row(u), tk, C, m - u * C);
          }
        __syncthreads();
        for (int t = 0; t < need; ++t) {
          double bs = -INFINITY;
          uint64_t bh = ~0ull, bl = ~0ull;
          int br = 0x7FFFFFFF, bm = -1;
          for (int m = tid; m < M; m += kSelThreads) {
            if (bin_of(sm.cs[m]) != kc || ((sm.taken[m >> 6] >> (m & 63)) & 1)) continue;
            const int u = m / C;
            const int r = sm.mrank[m];
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
          __syncthreads();
          if (tid == 0) {
            int best = -1;
            for (int q = 0; q < kSelWaves; ++q) {
              const int mq = sm.cut[q];
              if (mq < 0) continue;
              if (best < 0) {
                best = q;
                continue;
              }
              const int mb = sm.cut[best], ub = mb / C, uq = mq / C;
              if (bm_before(sm.cs[mq], sm.bh[uq], sm.bl[uq], sm.crank[q], sm.cs[mb], sm.bh[ub],
                            sm.bl[ub], sm.crank[best]))
                best = q;
            }
            const int mb = sm.cut[best];
            sm.sel[nsel + t] = mb;
            sm.srank[nsel + t] = sm.crank[best];
            sm.taken[mb >> 6] |= 1ull << (mb & 63);
          }
          __syncthreads();
        }
      }
      nsel = w;
    }
    // ---- the new beam: child ranks of the whole-bin entries, keys, order ----
    const int cutfrom = w >= M ? M : sm.kexc;  // entries before it need their rank
    for (int k = tid; k < cutfrom; k += kSelThreads) {
      const int m = sm.sel[k], u = m / C;
      sm.srank[k] = bm_rank(row(u), tk, C, m - u * C);
    }
    __syncthreads();
    // entry k: candidate m, score, key = parent key + digit; its position by
    // counting; written straight into the next beam (staged in registers)
    int nb_c = 0, nb_node = 0, nb_pos = -1;
    double nb_S = 0.0;
    uint64_t nb_h = 0, nb_l = 0;
    if (tid < nsel) {
      const int m = sm.sel[tid], u = m / C, j = m - u * C;
      const double s = sm.cs[m];
      uint64_t h = sm.bh[u], l = sm.bl[u];
      const int r = sm.srank[tid];
      int pos = 0;
      for (int q = 0; q < nsel; ++q) {
        const int mq = sm.sel[q], uq = mq / C;
        pos += bm_before(sm.cs[mq], sm.bh[uq], sm.bl[uq], sm.srank[q], s, h, l, r) ? 1 : 0;
      }
      lex_set_digit(h, l, d + 1, (uint32_t)r, bpd);
      const int node = sm.nout + pos + 1;
      const size_t o = (size_t)b * B + node - 1;
      p.tree_tokens[o] = tk[j];
      p.parents[o] = sm.bnode[u];
      p.logq[o] = (float)s;
      if (p.depths) p.depths[o] = d + 1;
      sm.opar[node - 1] = sm.bnode[u];
      nb_c = j;
      nb_S = s;
      nb_h = h;
      nb_l = l;
      nb_node = node;
      nb_pos = pos;
    }
    __syncthreads();  // every read of the old beam is done
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
    __syncthreads();
  }
  const int nout = sm.nout;
  for (int j = nout + tid; j < B; j += kSelThreads) {
    const size_t o = (size_t)b * B + j;
    p.tree_tokens[o] = -1;
    p.parents[o] = -1;
    p.logq[o] = -INFINITY;
    if (p.depths) p.depths[o] = 0;
  }
  if (tid == 0) p.num_nodes[b] = nout;
  sel_mask_rows(p, sm.opar, nout, b);
}

}  // namespace ddt
