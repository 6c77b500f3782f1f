// DSpark's survival-ranked verification budget (DSpark explainer, "Hardware
// aware prefix scheduler"; DSpark guide, "Survival probability" and
// "Picking the budget").
//
// Per request b and block position p a confidence head gives c[b][p], the
// chance that guess p survives if every earlier guess did. A slot's survival
// is the product of the confidences up to it (float64, left to right, each
// confidence clamped into [0, 1], NaN as 0). All R*P slots of the batch rank
// by survival (ties: lower request, then lower position); keeping the first
// n costs one target step over T = R + n tokens and is expected to yield R +
// (sum of the kept survivals) tokens; the budget is the n maximising
// expected tokens per millisecond over a measured cost table cost[T] (the
// smallest n among equal maxima; counts the table does not cover are not
// candidates). Each request keeps the prefix of its block that lies in the
// first n.
//
// MI355X design: the whole batch is one ranking problem of at most 4096
// slots, so one 1024-thread workgroup does it in LDS. A request's survivals
// never increase along its block, so the R blocks are already sorted runs:
// the ranking is a merge tree of at most 12 levels (merge path: one co-rank
// search per thread and level, then a short sequential merge; no full sort).
// Then a float64 block scan gives every count's expected tokens, a block
// reduction the best count, and LDS counters the per-request lengths.
#pragma once

#include "common.hpp"

namespace ddt {

constexpr int kDsThreads = 1024;
constexpr int kDsWaves = kDsThreads / kWave;
constexpr int kDsMaxN = 4096;  // slots (requests x block positions), at most
constexpr int kDsPerThread = kDsMaxN / kDsThreads;

struct DsParams {
  const float* conf;  // [R][P] per-position confidences
  int32_t R, P;
  const float* cost;  // [n_cost] step cost in ms by token count T
  int32_t n_cost;     // > R
  int32_t* keep;      // [R] guesses kept per request
  double* survival;   // [R][P] (may be null)
  int32_t* n_keep;    // [1] the budget n
  double* expected;   // [1] expected tokens R + sum of kept survivals (may be null)
  double* objective;  // [1] expected tokens per ms (may be null)
};

struct DsSmem {
  double key[2][kDsMaxN];
  uint16_t idx[2][kDsMaxN];
  int cnt[kDsMaxN];
  double wsum[kDsWaves];
  double bf[kDsWaves];
  int bn[kDsWaves];
};

__device__ __forceinline__ double ds_wave_incl_scan(double x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// the better of two candidate counts: larger objective, then smaller n
__device__ __forceinline__ bool ds_better(double f, int n, double g, int m) {
  return f > g || (f == g && n < m);
}

__global__ __launch_bounds__(kDsThreads) void dspark_budget_kernel(DsParams p) {
  __shared__ DsSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int R = p.R, P = p.P, N = R * P;
  // ---- survival products: confidences staged in LDS by coalesced loads,
  // then one thread per request multiplies along its block
  float* cf = reinterpret_cast<float*>(sm.key[1]);
  for (int i = tid; i < N; i += kDsThreads) {
    const float c = p.conf[i];
    cf[i] = c != c ? 0.0f : fminf(fmaxf(c, 0.0f), 1.0f);
  }
  for (int b = tid; b < R; b += kDsThreads) sm.cnt[b] = 0;
  __syncthreads();
  for (int b = tid; b < R; b += kDsThreads) {
    double acc = 1.0;
    for (int q0 = 0; q0 < P; q0 += 8) {  // eight reads in flight, then the chain
      float c8[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) c8[q] = q0 + q < P ? cf[b * P + q0 + q] : 1.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q0 + q < P) {
          acc = acc * (double)c8[q];
          sm.key[0][b * P + q0 + q] = acc;
          sm.idx[0][b * P + q0 + q] = (uint16_t)(b * P + q0 + q);
        }
    }
  }
  __syncthreads();
  if (p.survival)
    for (int i = tid; i < N; i += kDsThreads) p.survival[i] = sm.key[0][i];
  // ---- merge tree over the R sorted runs -----------------------------------
  // Merge path: at each level every thread writes kDsPerThread consecutive
  // outputs of one merged pair of runs (A first on equal survival: A holds
  // the lower requests). One co-rank search finds how many of its first
  // outputs come from A, then the outputs merge sequentially (a thread's
  // outputs may run into the next pair, which starts from its beginning).
  int src = 0;
  for (int r = P; r < N; r *= 2) {
    const double* ks = sm.key[src];
    const uint16_t* is = sm.idx[src];
    double* kd = sm.key[src ^ 1];
    uint16_t* id = sm.idx[src ^ 1];
    const int o0 = tid * kDsPerThread;
    if (o0 < N) {
      int ps = (o0 / (2 * r)) * (2 * r);
      int a0 = ps, na = min(r, N - a0), b0 = a0 + r, nb = max(0, min(r, N - b0));
      const int dg = o0 - ps;
      int lo = max(0, dg - nb), hi = min(dg, na);
      while (lo < hi) {  // largest i with A[i-1] >= B[dg-i]
        const int mid = (lo + hi + 1) >> 1;
        if (ks[a0 + mid - 1] >= ks[b0 + dg - mid]) lo = mid;
        else hi = mid - 1;
      }
      int i = lo, j = dg - lo;
#pragma unroll
      for (int k = 0; k < kDsPerThread; ++k) {
        const int pos = o0 + k;
        if (pos < N) {
          if (pos - ps == 2 * r) {
            ps = pos;
            a0 = ps;
            na = min(r, N - a0);
            b0 = a0 + r;
            nb = max(0, min(r, N - b0));
            i = 0;
            j = 0;
          }
          const bool ta = j >= nb || (i < na && ks[a0 + i] >= ks[b0 + j]);
          const int from = ta ? a0 + i : b0 + j;
          i += ta ? 1 : 0;
          j += ta ? 0 : 1;
          kd[pos] = ks[from];
          id[pos] = is[from];
        }
      }
    }
    src ^= 1;
    __syncthreads();
  }
  const double* key = sm.key[src];
  const uint16_t* idx = sm.idx[src];
  // ---- expected tokens of every count: float64 scan, kDsPerThread slots a thread
  double loc[kDsPerThread];
  double run = 0.0;
#pragma unroll
  for (int k = 0; k < kDsPerThread; ++k) {
    const int i = tid * kDsPerThread + k;
    run += i < N ? key[i] : 0.0;
    loc[k] = run;
  }
  const double inc = ds_wave_incl_scan(run);
  if (lane == kWave - 1) sm.wsum[wv] = inc;
  __syncthreads();
  double pre = inc - run;
  for (int w = 0; w < wv; ++w) pre += sm.wsum[w];
  // counts n = tid * kDsPerThread + k + 1 (and n = 0 on thread 0)
  double bf = -INFINITY;
  int bn = 0x7FFFFFFF;
  const double Rd = (double)R;
  if (tid == 0) {
    bf = Rd / (double)p.cost[R];
    bn = 0;
  }
#pragma unroll
  for (int k = 0; k < kDsPerThread; ++k) {
    const int n = tid * kDsPerThread + k + 1;
    if (n <= N && R + n < p.n_cost) {
      const double f = (Rd + (pre + loc[k])) / (double)p.cost[R + n];
      if (ds_better(f, n, bf, bn)) {
        bf = f;
        bn = n;
      }
    }
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double of = __shfl_xor(bf, o);
    const int on = __shfl_xor(bn, o);
    if (ds_better(of, on, bf, bn)) {
      bf = of;
      bn = on;
    }
  }
  if (lane == 0) {
    sm.bf[wv] = bf;
    sm.bn[wv] = bn;
  }
  __syncthreads();
  bf = sm.bf[0];
  bn = sm.bn[0];
  for (int w = 1; w < kDsWaves; ++w)
    if (ds_better(sm.bf[w], sm.bn[w], bf, bn)) {
      bf = sm.bf[w];
      bn = sm.bn[w];
    }
  // ---- per-request lengths: the first bn ranked slots ----------------------
  for (int i = tid; i < bn; i += kDsThreads) atomicAdd(&sm.cnt[idx[i] / P], 1);
  // the expected tokens of the chosen count: the thread whose slots end at bn
  if (bn == 0 && tid == 0) {
    p.n_keep[0] = 0;
    if (p.expected) p.expected[0] = Rd;
    if (p.objective) p.objective[0] = bf;
  }
#pragma unroll
  for (int k = 0; k < kDsPerThread; ++k)
    if (tid * kDsPerThread + k + 1 == bn) {
      p.n_keep[0] = bn;
      if (p.expected) p.expected[0] = Rd + (pre + loc[k]);
      if (p.objective) p.objective[0] = bf;
    }
  __syncthreads();
  for (int b = tid; b < R; b += kDsThreads) p.keep[b] = sm.cnt[b];
}

}  // namespace ddt
