// Stage 1: per-row log-sum-exp and exact sorted top-K over the vocabulary.
//
// SparklingTree post, section "Step 1: Sorting the DFlash marginals": each
// drafter row is upcast to float32, its top K = min(budget, V) logits are
// kept in sorted order with their token ids, and the row's log-sum-exp is
// taken. Equal logits rank by lower token id; -0 equals +0.
//
// MI355X design. A row (V ~ 152k bf16 = 297 KiB) is split into S chunks of
// 256 threads x NV x 16 B; every chunk is one workgroup that loads its whole
// chunk into registers with coalesced 16-byte loads, so HBM is read exactly
// once. From registers the block computes (a) its max and sum of exp in
// float32 (per element: one subtract, one multiply, one v_exp_f32, one add),
// and (b) its exact top-K: each wave picks a threshold from the maxima of
// 32-element groups (a 16/32-step ballot search), the block keeps the
// smallest of the four wave thresholds, which provably leaves at least K
// elements above it, collects the ~1.1-1.3 K survivors into LDS and bitonic-
// sorts them. The last block of a row to finish (agent-scope release/acquire
// around an atomic ticket) merges the S sorted lists and the S (max, sum)
// pairs into the row's table and normaliser.
#pragma once

#include "common.hpp"

namespace ddt {

constexpr int kS1Threads = 256;
constexpr int kCandCap = 2048;

struct Stage1Params {
  const void* logits;  // [rows][V] bf16 or f32
  int64_t rows;
  int64_t V;
  int64_t chunk;  // elements per chunk
  int32_t S;      // chunks per row
  int32_t K;
  uint64_t* part_keys;  // [rows][S][K]  (S > 1)
  double* part_ms;      // [rows][S][2]  (max, sum exp(x - max))  (S > 1)
  uint32_t* row_ctr;    // [rows], zero on entry, zero on exit
  int32_t* out_ids;     // [rows][K]
  float* out_vals;      // [rows][K]
  double* out_lse;      // [rows]
};

struct Stage1Smem {
  uint64_t cand[kCandCap];
  uint64_t red_u64[kS1Threads / kWave];
  double red_f64[kS1Threads / kWave];
  float red_f32[kS1Threads / kWave];
  uint32_t red_u32[kS1Threads / kWave];
  uint32_t n;
  int flag;
};

template <int DT>
__device__ __forceinline__ uint32_t elem_bits(const uint4& v, int e) {
  if (DT == 0) {
    const int q = e >> 1;
    const uint32_t w = q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
    return (e & 1) ? (w & 0xFFFF0000u) : (w << 16);
  } else {
    return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
  }
}

// Hide the register contents from the optimiser so that the cheap bf16->f32
// conversions are recomputed in each pass instead of keeping 128 converted
// floats live (which would halve occupancy).
template <int NV>
__device__ __forceinline__ void launder(uint4 (&raw)[NV]) {
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    asm volatile("" : "+v"(raw[j].x), "+v"(raw[j].y), "+v"(raw[j].z), "+v"(raw[j].w));
  }
}

// Block-wide reductions for kS1Threads threads. Each ends with a barrier so
// the scratch slot can be reused by the next call.
__device__ __forceinline__ float s1_block_max_f32(float v, Stage1Smem& sm) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) sm.red_f32[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sm.red_f32[0];
#pragma unroll
  for (int i = 1; i < kS1Threads / kWave; ++i) r = fmaxf(r, sm.red_f32[i]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ double s1_block_sum_f64(double v, Stage1Smem& sm) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sm.red_f64[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int i = 0; i < kS1Threads / kWave; ++i) r += sm.red_f64[i];
  __syncthreads();
  return r;
}
__device__ __forceinline__ uint64_t s1_block_max_u64(uint64_t v, Stage1Smem& sm) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) sm.red_u64[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t r = sm.red_u64[0];
#pragma unroll
  for (int i = 1; i < kS1Threads / kWave; ++i) r = r > sm.red_u64[i] ? r : sm.red_u64[i];
  __syncthreads();
  return r;
}
__device__ __forceinline__ uint32_t s1_block_sum_u32(uint32_t v, Stage1Smem& sm) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sm.red_u32[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < kS1Threads / kWave; ++i) r += sm.red_u32[i];
  __syncthreads();
  return r;
}

__device__ __forceinline__ void push_cand(Stage1Smem& sm, uint64_t key) {
  const uint32_t pos = atomicAdd(&sm.n, 1u);
  if (pos < (uint32_t)kCandCap) sm.cand[pos] = key;
}

// Sort the first n candidates (n <= kCandCap) largest first; entries past n
// up to the next power of two are padded with 0.
__device__ __forceinline__ void sort_cands(Stage1Smem& sm, int n) {
  const int np = next_pow2(n < 1 ? 1 : n);
  for (int i = n + threadIdx.x; i < np; i += kS1Threads) sm.cand[i] = 0;
  __syncthreads();
  bitonic_desc_u64<kS1Threads>(sm.cand, np);
}

__device__ __forceinline__ void write_row_table(const Stage1Params& p, int64_t row, Stage1Smem& sm,
                                                double lse) {
  const int K = p.K;
  for (int i = threadIdx.x; i < K; i += kS1Threads) {
    const uint64_t k = sm.cand[i];
    p.out_ids[row * K + i] = (int32_t)cand_id(k);
    p.out_vals[row * K + i] = key_value(cand_vkey(k));
  }
  if (threadIdx.x == 0) p.out_lse[row] = lse;
}

// Merge the S partial (sorted top-K, max, sum) records of `row` into the
// row's table. Runs in the last block of the row to finish.
__device__ void merge_row(const Stage1Params& p, int64_t row, Stage1Smem& sm) {
  const int S = p.S, K = p.K, tid = threadIdx.x;
  const uint64_t* pk = p.part_keys + (size_t)row * S * K;
  const double* pm = p.part_ms + (size_t)row * S * 2;

  // Normaliser: z = M + log(sum_s sum_s * exp(max_s - M)), float64.
  float mloc = -INFINITY;
  for (int s = tid; s < S; s += kS1Threads) mloc = fmaxf(mloc, (float)pm[2 * s]);
  const float M = s1_block_max_f32(mloc, sm);
  double acc = 0.0;
  for (int s = tid; s < S; s += kS1Threads) acc += pm[2 * s + 1] * exp(pm[2 * s] - (double)M);
  const double tot = s1_block_sum_f64(acc, sm);
  const double lse = (double)M + log(tot);

  // Every list's K-th key bounds the row's K-th key from below.
  uint64_t tl = 0;
  for (int s = tid; s < S; s += kS1Threads) {
    const uint64_t k = pk[(size_t)s * K + K - 1];
    tl = tl > k ? tl : k;
  }
  if (tid == 0) sm.n = 0;
  uint64_t tau = s1_block_max_u64(tl, sm);
  if (tau == 0) tau = 1;
  for (int i = tid; i < S * K; i += kS1Threads) {
    const uint64_t k = pk[i];
    if (k >= tau) push_cand(sm, k);
  }
  __syncthreads();
  int n = (int)sm.n;
  if (n > kCandCap) {
    // Exact K-th key by bisection over the 64-bit key (rare: needs more than
    // kCandCap entries above every list's K-th).
    uint64_t T = 0;
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t c = T | (1ull << bit);
      uint32_t cnt = 0;
      for (int i = tid; i < S * K; i += kS1Threads) cnt += pk[i] >= c ? 1u : 0u;
      if (s1_block_sum_u32(cnt, sm) >= (uint32_t)K) T = c;
    }
    if (tid == 0) sm.n = 0;
    __syncthreads();
    for (int i = tid; i < S * K; i += kS1Threads) {
      const uint64_t k = pk[i];
      if (k != 0 && k >= T) push_cand(sm, k);
    }
    __syncthreads();
    n = (int)sm.n;
  }
  sort_cands(sm, n);
  write_row_table(p, row, sm, lse);
  if (tid == 0) p.row_ctr[row] = 0;
}

// Exact top-K of a chunk when more than kCandCap elements tie above the
// group threshold: bisection for the K-th largest 64-bit key, re-reading the
// chunk from memory (L2-resident) on every step. Rare (massively tied rows);
// kept out of line so the common path keeps its registers. Returns the
// number of candidates left in sm.cand (exactly min(K, valid elements)).
template <int DT>
__device__ __noinline__ int exact_chunk_select(const Stage1Params& p, const char* rowp,
                                               int64_t c0, int64_t c1, Stage1Smem& sm) {
  auto key_at = [&](int64_t idx) -> uint64_t {
    const uint32_t bits = DT == 0 ? ((uint32_t)((const uint16_t*)rowp)[idx] << 16)
                                  : ((const uint32_t*)rowp)[idx];
    return cand_key(order_key(bits), (uint32_t)idx);
  };
  uint64_t T = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t c = T | (1ull << bit);
    uint32_t cnt = 0;
    for (int64_t i = c0 + threadIdx.x; i < c1; i += kS1Threads) cnt += key_at(i) >= c ? 1u : 0u;
    if (s1_block_sum_u32(cnt, sm) >= (uint32_t)p.K) T = c;
  }
  if (threadIdx.x == 0) sm.n = 0;
  __syncthreads();
  for (int64_t i = c0 + threadIdx.x; i < c1; i += kS1Threads) {
    const uint64_t k = key_at(i);
    if (k >= T) push_cand(sm, k);
  }
  __syncthreads();
  return (int)sm.n;
}

template <int DT, int NV, int GS, bool ALIGNED>
__global__ __launch_bounds__(kS1Threads) void stage1_kernel(Stage1Params p) {
  constexpr int EPV = DT == 0 ? 8 : 4;  // elements per 16-byte vector
  constexpr int G = NV / GS;            // threshold groups per thread
  constexpr uint32_t NEG_INF_DW = DT == 0 ? 0xFF80FF80u : 0xFF800000u;
  __shared__ Stage1Smem sm;

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / p.S;
  const int chunk = (int)(blockIdx.x % p.S);
  const int64_t c0 = (int64_t)chunk * p.chunk;
  const int64_t c1 = (c0 + p.chunk < p.V) ? c0 + p.chunk : p.V;
  const int K = p.K;
  const char* rowp = (const char*)p.logits + (size_t)row * (size_t)p.V * (DT == 0 ? 2 : 4);

  // ---- load the chunk into registers (invalid slots hold -inf) -------------
  uint4 raw[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t e0 = c0 + ((int64_t)j * kS1Threads + tid) * EPV;
    if (ALIGNED) {
      if (e0 < c1) {
        raw[j] = *(const uint4*)(rowp + e0 * (DT == 0 ? 2 : 4));
      } else {
        raw[j] = make_uint4(NEG_INF_DW, NEG_INF_DW, NEG_INF_DW, NEG_INF_DW);
      }
    } else {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = NEG_INF_DW;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const int64_t idx = e0 + e;
        if (idx < c1) {
          if (DT == 0) {
            const uint32_t b = ((const uint16_t*)rowp)[idx];
            const int q = e >> 1;
            w[q] = (e & 1) ? ((w[q] & 0x0000FFFFu) | (b << 16)) : ((w[q] & 0xFFFF0000u) | b);
          } else {
            w[e] = ((const uint32_t*)rowp)[idx];
          }
        }
      }
      raw[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }

  // ---- per-vector and per-group maxima -------------------------------------
  float vm[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < EPV; ++e) m = fmaxf(m, __uint_as_float(elem_bits<DT>(raw[j], e)));
    vm[j] = m;
  }
  uint32_t gk[G];
  float tmax = -INFINITY;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = vm[g * GS];
#pragma unroll
    for (int q = 1; q < GS; ++q) m = fmaxf(m, vm[g * GS + q]);
    tmax = fmaxf(tmax, m);
    gk[g] = (m == -INFINITY) ? 0u : order_key(__float_as_uint(m));
  }

  // ---- sum of exp relative to the thread max -------------------------------
  launder<NV>(raw);
  float ssum = 0.0f;
  if (tmax != -INFINITY) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float x = __uint_as_float(elem_bits<DT>(raw[j], e));
        ssum += __builtin_amdgcn_exp2f((x - tmax) * kLog2e);
      }
    }
  }

  // ---- wave threshold: largest T with >= ceil(K/4) group maxima >= T -------
  const int need = (K + 3) >> 2;
  uint32_t T = 0;
  for (int bit = 31; bit >= (DT == 0 ? 16 : 0); --bit) {
    const uint32_t c = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) cnt += __popcll(__ballot(gk[g] >= c));
    if (cnt >= need) T = c;
  }
  if ((tid & 63) == 0) sm.red_u32[tid >> 6] = T;
  if (tid == 0) sm.n = 0;
  __syncthreads();
  uint32_t t0 = sm.red_u32[0];
#pragma unroll
  for (int i = 1; i < kS1Threads / kWave; ++i) t0 = min(t0, sm.red_u32[i]);

  // ---- collect every element with key >= t0 --------------------------------
  launder<NV>(raw);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (gk[g] != 0 && gk[g] >= t0) {
#pragma unroll
      for (int q = 0; q < GS; ++q) {
        const int j = g * GS + q;
        const int64_t e0 = c0 + ((int64_t)j * kS1Threads + tid) * EPV;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const uint32_t k = order_key(elem_bits<DT>(raw[j], e));
          if (e0 + e < c1 && k >= t0) push_cand(sm, cand_key(k, (uint32_t)(e0 + e)));
        }
      }
    }
  }
  __syncthreads();
  int n = (int)sm.n;
  if (n > kCandCap) n = exact_chunk_select<DT>(p, rowp, c0, c1, sm);
  sort_cands(sm, n);

  // ---- chunk normaliser -----------------------------------------------------
  const float M = s1_block_max_f32(tmax, sm);
  double part = 0.0;
  if (tmax != -INFINITY) part = (double)(ssum * __builtin_amdgcn_exp2f((tmax - M) * kLog2e));
  const double ssum_blk = s1_block_sum_f64(part, sm);

  if (p.S == 1) {
    write_row_table(p, row, sm, (double)M + log(ssum_blk));
    return;
  }

  // ---- publish the chunk's partial record ----------------------------------
  uint64_t* pk = p.part_keys + ((size_t)row * p.S + chunk) * K;
  for (int i = tid; i < K; i += kS1Threads) pk[i] = i < n ? sm.cand[i] : 0ull;
  if (tid == 0) {
    p.part_ms[((size_t)row * p.S + chunk) * 2] = (double)M;
    p.part_ms[((size_t)row * p.S + chunk) * 2 + 1] = ssum_blk;
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = atomicAdd(&p.row_ctr[row], 1u);
    sm.flag = (old == (uint32_t)(p.S - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!sm.flag) return;
  __threadfence();
  merge_row(p, row, sm);
}

}  // namespace ddt
