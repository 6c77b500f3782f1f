// Stage 1: per-row log-sum-exp and exact sorted top-K over the vocabulary.
//
// SparklingTree post, section "Step 1: Sorting the DFlash marginals": each
// drafter row is upcast to float32, its top K = min(budget, V) logits are
// kept in sorted order with their token ids, and the row's log-sum-exp is
// taken. Equal logits rank by lower token id; -0 equals +0.
//
// MI355X design (no synchronisation between workgroups):
//
// A row (V ~ 152k bf16 = 297 KiB) is cut into chunks of 256 threads x NV x
// 16 B held in registers after one round of 16-byte global loads, so HBM is
// read exactly once. Per chunk:
//  1. max pass: per-thread maxima of G groups of 32 elements (v_max3);
//  2. threshold: each wave finds, by a 16-step (bf16) ballot bisection, the
//     largest value with >= K/4 of its group maxima at or above it; the
//     smallest of the four wave thresholds leaves >= K chunk elements at or
//     above it (one element per qualifying group);
//  3. fused pass: per element one shift/mask (bf16->f32), one fma and one
//     v_exp_f32 of x*c - m*c (c = log2 e rounded to float, the rounding is
//     folded back in float64 per thread), one add, and one compare against
//     the threshold whose wave ballot also places the rare survivors into the
//     wave's LDS region (mbcnt offsets, no atomics).
// Two shapes:
//  stage1_chunk_kernel + stage1_merge_kernel (few rows): one workgroup per
//    chunk writes a record (survivors, threshold, normaliser partial); one
//    wavefront per row then keeps the survivors at or above the largest
//    chunk threshold, finds the exact K-th (value, id) key by a ballot
//    bisection over registers, ranks the K winners by counting and writes
//    the row's table and log-sum-exp (float64).
//  stage1_row_kernel (many rows): one workgroup walks all chunks of its row
//    with double-buffered register loads (chunk i+1 in flight while chunk i
//    is processed), raises the row threshold chunk by chunk and finishes the
//    row itself in the same way: no records, no second launch.
#pragma once

#include "common.hpp"

namespace ddt {

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) v4u32* gvec_ptr;
typedef const __attribute__((address_space(1))) uint16_t* gu16_ptr;
typedef const __attribute__((address_space(1))) uint32_t* gu32_ptr;

constexpr int kS1Threads = 256;
constexpr int kS1Waves = kS1Threads / kWave;
constexpr int kCandCap = 2048;                // LDS survivors of one workgroup
constexpr int kWaveCap = kCandCap / kS1Waves;  // per-wave region
constexpr int kMergeSlots = 40;                // record slots per lane in the merge
constexpr float kLog2eF = 1.44269504088896340736f;
constexpr double kLog2eErr = 1.4426950408889634074 - (double)kLog2eF;  // log2(e) - c
constexpr double kLn2 = 0.69314718055994530942;

struct Stage1Params {
  const void* logits;  // [rows][V] bf16 or f32, 16-byte aligned base
  int64_t rows;
  int64_t V;
  int64_t chunk;  // elements per chunk
  int32_t S;      // chunks per row
  int32_t K;
  int32_t capp;     // survivor slots per chunk record (>= K; S * capp <= 64 * kMergeSlots)
  int32_t idbits;   // ids are < 2^idbits
  int32_t* cnt;     // [rows][S] survivors in each record
  uint32_t* thr;    // [rows][S] the chunk's value-key threshold
  double* meta;     // [rows][S][2] (log2 offset, sum): chunk sum exp = sum * 2^offset
  uint64_t* cands;  // [rows][S][capp] survivor keys (value key << 32 | ~id)
  int32_t* out_ids;   // [rows][K]
  float* out_vals;    // [rows][K]
  double* out_lse;    // [rows]
};

template <int DT>
__device__ __forceinline__ uint32_t elem_bits(const v4u32& v, int e) {
  if (DT == 0) {
    const int q = e >> 1;
    const uint32_t w = q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
    return (e & 1) ? (w & 0xFFFF0000u) : (w << 16);
  } else {
    return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
  }
}

// Hide register contents from the optimiser so that the cheap bf16->f32
// conversions are recomputed in each pass instead of keeping every converted
// float live (which would halve occupancy).
template <int NV>
__device__ __forceinline__ void launder(v4u32 (&raw)[NV]) {
#pragma unroll
  for (int j = 0; j < NV; ++j) asm volatile("" : "+v"(raw[j]));
}

// Number of set bits of m at lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Float threshold equivalent to "order key >= t": t = 0 admits every finite
// value (and no -inf, which marks masked slots).
__device__ __forceinline__ float key_threshold(uint32_t t) {
  return t == 0 ? -3.402823466e38f : key_value(t);
}

template <int DT, int NV, int GS>
__device__ __forceinline__ void group_maxima(const v4u32 (&raw)[NV], float (&gmax)[NV / GS],
                                             uint32_t (&gk)[NV / GS]) {
  constexpr int EPV = DT == 0 ? 8 : 4;
#pragma unroll
  for (int g = 0; g < NV / GS; ++g) {
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < GS; ++q) {
#pragma unroll
      for (int e = 0; e < EPV; ++e)
        m = fmaxf(m, __uint_as_float(elem_bits<DT>(raw[g * GS + q], e)));
    }
    gmax[g] = m;
    gk[g] = m == -INFINITY ? 0u : order_key(__float_as_uint(m));
  }
}

// Largest T (value key) with >= need of this wave's group maxima >= T, or 0.
template <int DT, int G>
__device__ __forceinline__ uint32_t wave_threshold(const uint32_t (&gk)[G], int need) {
  uint32_t T = 0;
  for (int bit = 31; bit >= (DT == 0 ? 16 : 0); --bit) {
    const uint32_t c = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) cnt += __popcll(__ballot(gk[g] >= c));
    if (cnt >= need) T = c;
  }
  return T;
}

// Fused pass over a register-resident chunk: returns the thread's sum of
// 2^(x*c - mc) (8-term sums per vector, then pairwise), and appends every
// element >= tf to this wave's LDS region (wn = survivors so far, uniform).
template <int DT, int NV>
__device__ __forceinline__ float exp_collect(v4u32 (&raw)[NV], float mc, float tf, int64_t c0,
                                             uint64_t* region, int& wn) {
  constexpr int EPV = DT == 0 ? 8 : 4;
  static_assert(NV <= 16 && (NV & (NV - 1)) == 0, "pairwise levels");
  const uint32_t id_base = (uint32_t)c0 + threadIdx.x * EPV;
  float lvl[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // pairwise partial sums (binary carry)
  float total = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const uint32_t id0 = id_base + (uint32_t)(j * kS1Threads * EPV);
    // keep the vectors in order: convert, exponentiate and test vector j
    // before vector j+1 (otherwise every converted float stays live)
    asm volatile("" : "+v"(raw[j]));
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const uint32_t bits = elem_bits<DT>(raw[j], e);
      const float x = __uint_as_float(bits);
      a += __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2eF, -mc));
      const bool pass = x >= tf;
      const uint64_t M = __ballot(pass);
      if (M) {
        const int pos = wn + lanes_below(M);
        if (pass && pos < kWaveCap) region[pos] = cand_key(order_key(bits), id0 + e);
        wn += __popcll(M);
      }
    }
    asm volatile("" : "+v"(a));
    // a joins the pairwise tree ((v0+v1)+(v2+v3))+...: vector j closes the
    // levels given by the trailing one bits of j
    int L = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (L == b && ((j >> b) & 1)) {
        a += lvl[b];
        L = b + 1;
      }
    }
    if (L < 4) lvl[L] = a;
    if (j == NV - 1) total = a;
  }
  return total;
}

// ---------------------------------------------------------------------------
// Exact top-K by one wavefront from up to 64 * kMergeSlots keys held in
// registers (0 = empty slot): ballot bisection for the K-th largest key, then
// each winner's rank by counting. Writes the table row. `stage` is a
// wave-private LDS area of >= K keys. Requires >= K nonzero keys.
template <int NS>
__device__ __forceinline__ void wave_topk_finish(uint64_t (&v)[NS], int R, int K,
                                                 int idbits, bool bf16, uint64_t* stage,
                                                 int32_t* out_ids, float* out_vals) {
  const int lane = threadIdx.x & 63;
  auto count_ge = [&](uint64_t x) -> int {
    int c = 0;
#pragma unroll
    for (int r = 0; r < NS; ++r)
      if (r < R) c += __popcll(__ballot(v[r] >= x));
    return c;
  };
  uint64_t T = 0;
  for (int bit = 63; bit >= 32; --bit) {
    if (bf16 && bit < 48) {
      // bf16 value keys have a constant low half: 0x0000 (>= 0) or 0xFFFF
      T |= (T >> 63) ? 0ull : 0x0000FFFF00000000ull;
      break;
    }
    const uint64_t x = T | (1ull << bit);
    if (count_ge(x) >= K) T = x;
  }
  // ids are < 2^idbits: the inverted id's higher bits are all ones
  T |= 0xFFFFFFFFull & ~((1ull << idbits) - 1ull);
  for (int bit = idbits - 1; bit >= 0; --bit) {
    const uint64_t x = T | (1ull << bit);
    if (count_ge(x) >= K) T = x;
  }
  // the K winners (keys are unique) into the wave's staging area
  int nw = 0;
#pragma unroll
  for (int r = 0; r < NS; ++r) {
    if (r < R) {
      const bool win = v[r] >= T && v[r] != 0;
      const uint64_t M = __ballot(win);
      if (win) stage[nw + lanes_below(M)] = v[r];
      nw += __popcll(M);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // rank of winner i = number of larger winners
  for (int i0 = 0; i0 < K; i0 += kWave) {
    const int i = i0 + lane;
    const uint64_t mine = i < K ? stage[i] : 0ull;
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < K; ++j) rank += stage[j] > mine ? 1 : 0;
    if (i < K) {
      out_ids[rank] = (int32_t)cand_id(mine);
      out_vals[rank] = key_value(cand_vkey(mine));
    }
  }
}

// ---------------------------------------------------------------------------
// Chunk kernel (one workgroup per chunk).

struct ChunkSmem {
  uint64_t cand[kCandCap];
  double red_d[kS1Waves];
  uint32_t red_u[kS1Waves];
  int wn[kS1Waves];
};

// Exact top-K of a chunk from memory when survivors overflow the LDS regions
// (massively tied rows): bisection for the K-th largest key, re-reading the
// chunk (L2-resident) each step; leaves exactly min(K, elements) keys at the
// front of sm.cand and returns that count. Kept out of line.
template <int DT>
__device__ __noinline__ int exact_chunk_select(const char* rowp, int64_t c0, int64_t c1, int K,
                                               ChunkSmem& sm) {
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
    cnt = wave_sum(cnt);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sm.red_u[threadIdx.x >> 6] = cnt;
    __syncthreads();
    uint32_t tot = 0;
#pragma unroll
    for (int w = 0; w < kS1Waves; ++w) tot += sm.red_u[w];
    if (tot >= (uint32_t)K) T = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) sm.wn[0] = 0;
  __syncthreads();
  for (int64_t i = c0 + threadIdx.x; i < c1; i += kS1Threads) {
    const uint64_t k = key_at(i);
    if (k >= T) sm.cand[atomicAdd(&sm.wn[0], 1)] = k;
  }
  __syncthreads();
  return sm.wn[0];
}

// MODE 0: every 16-byte vector of the chunk lies in the row.
// MODE 1: vectors past the row's end are masked to -inf (a row's last chunk).
// MODE 2: element loads (rows whose byte length is not a multiple of 16).
template <int DT, int NV, int GS, int MODE>
__device__ __forceinline__ void chunk_body(const Stage1Params& p, ChunkSmem& sm, int64_t row,
                                           int chunk, int64_t c0, int64_t c1) {
  constexpr int EPV = DT == 0 ? 8 : 4;
  constexpr int G = NV / GS;
  constexpr uint32_t NEG_INF_DW = DT == 0 ? 0xFF80FF80u : 0xFF800000u;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int K = p.K;
  const size_t esz = DT == 0 ? 2 : 4;
  const char* rowp = (const char*)p.logits + (size_t)row * (size_t)p.V * esz;
  const int64_t nvec = (c1 - c0 + EPV - 1) / EPV;

  v4u32 raw[NV];
  if (MODE == 0 || MODE == 1) {
    const gvec_ptr base = (gvec_ptr)(rowp + c0 * esz);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int vi = j * kS1Threads + tid;
      raw[j] = base[(MODE == 0 || vi < nvec) ? vi : 0];
    }
    if (MODE == 1) {
#pragma unroll
      for (int j = 0; j < NV; ++j)
        if (j * kS1Threads + tid >= nvec) raw[j] = v4u32{NEG_INF_DW, NEG_INF_DW, NEG_INF_DW, NEG_INF_DW};
    }
  } else {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const int64_t idx = c0 + ((int64_t)j * kS1Threads + tid) * EPV + e;
        const int64_t cl = idx < c1 ? idx : c0;
        const uint32_t b = DT == 0 ? (uint32_t)((gu16_ptr)rowp)[cl] : ((gu32_ptr)rowp)[cl];
        if (DT == 0) {
          const uint32_t h = idx < c1 ? b : 0xFF80u;
          wd[e >> 1] |= (e & 1) ? (h << 16) : h;
        } else {
          wd[e] = idx < c1 ? b : NEG_INF_DW;
        }
      }
      raw[j] = v4u32{wd[0], wd[1], wd[2], wd[3]};
    }
  }

  float gmax[G];
  uint32_t gk[G];
  group_maxima<DT, NV, GS>(raw, gmax, gk);
  float tmax = gmax[0];
#pragma unroll
  for (int g = 1; g < G; ++g) tmax = fmaxf(tmax, gmax[g]);
  const uint32_t Tw = wave_threshold<DT, G>(gk, (K + 3) >> 2);
  // thread log2 offset: m*c as rounded, plus m*(log2 e - c)
  const float mc = tmax * kLog2eF;
  const double off = tmax == -INFINITY ? -INFINITY : (double)mc + (double)tmax * kLog2eErr;
  const double off_w = wave_max(off);
  if (lane == 0) {
    sm.red_u[w] = Tw;
    sm.red_d[w] = off_w;
  }
  __syncthreads();
  uint32_t t0 = sm.red_u[0];
  double OFF = sm.red_d[0];
#pragma unroll
  for (int i = 1; i < kS1Waves; ++i) {
    t0 = min(t0, sm.red_u[i]);
    OFF = OFF > sm.red_d[i] ? OFF : sm.red_d[i];
  }

  launder<NV>(raw);
  int wn = 0;
  const float ssum = exp_collect<DT, NV>(raw, tmax == -INFINITY ? 0.0f : mc, key_threshold(t0), c0,
                                         sm.cand + w * kWaveCap, wn);
  const double part = tmax == -INFINITY ? 0.0 : (double)ssum * exp2(off - OFF);
  const double part_w = wave_sum(part);
  __syncthreads();  // the reads of red_d / red_u above are done
  if (lane == 0) {
    sm.red_d[w] = part_w;
    sm.wn[w] = wn;
  }
  __syncthreads();
  double tot = 0.0;
  int n = 0, ovf = 0;
  int base[kS1Waves];
#pragma unroll
  for (int i = 0; i < kS1Waves; ++i) {
    tot += sm.red_d[i];
    base[i] = n;
    n += sm.wn[i];
    ovf |= sm.wn[i] > kWaveCap;
  }

  const size_t rec = (size_t)row * p.S + chunk;
  uint64_t* dst = p.cands + rec * p.capp;
  if (!ovf && n <= p.capp) {
    for (int i = tid; i < n; i += kS1Threads) {
      int ww = 0;
#pragma unroll
      for (int q = 1; q < kS1Waves; ++q) ww += i >= base[q] ? 1 : 0;
      dst[i] = sm.cand[ww * kWaveCap + (i - base[ww])];
    }
  } else {
    // More survivors than the record holds (heavy ties): keep the exact top K.
    __syncthreads();
    if (ovf) {
      n = exact_chunk_select<DT>(rowp, c0, c1, K, sm);
    } else {
      // gather the wave regions to the front, then sort
      uint64_t r[kCandCap / kS1Threads];
#pragma unroll
      for (int k = 0; k < kCandCap / kS1Threads; ++k) {
        const int i = tid + k * kS1Threads;
        int ww = 0;
#pragma unroll
        for (int q = 1; q < kS1Waves; ++q) ww += i >= base[q] ? 1 : 0;
        r[k] = i < n ? sm.cand[ww * kWaveCap + (i - base[ww])] : 0ull;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kCandCap / kS1Threads; ++k) sm.cand[tid + k * kS1Threads] = r[k];
      __syncthreads();
    }
    const int np = next_pow2(n < 1 ? 1 : n);
    for (int i = n + tid; i < np; i += kS1Threads) sm.cand[i] = 0;
    __syncthreads();
    bitonic_desc_u64<kS1Threads>(sm.cand, np);
    n = n < K ? n : K;
    for (int i = tid; i < n; i += kS1Threads) dst[i] = sm.cand[i];
  }
  if (tid == 0) {
    p.cnt[rec] = n;
    p.thr[rec] = t0;
    p.meta[2 * rec] = OFF;
    p.meta[2 * rec + 1] = tot;
  }
}

template <int DT, int NV, int GS, bool ALIGNED>
__global__ __launch_bounds__(kS1Threads) void stage1_chunk_kernel(Stage1Params p) {
  __shared__ ChunkSmem sm;
  const int64_t row = blockIdx.x / p.S;
  const int chunk = (int)(blockIdx.x % p.S);
  const int64_t c0 = (int64_t)chunk * p.chunk;
  const int64_t c1 = (c0 + p.chunk < p.V) ? c0 + p.chunk : p.V;
  if constexpr (!ALIGNED) {
    chunk_body<DT, NV, GS, 2>(p, sm, row, chunk, c0, c1);
  } else {
    if (c1 - c0 == p.chunk) chunk_body<DT, NV, GS, 0>(p, sm, row, chunk, c0, c1);
    else chunk_body<DT, NV, GS, 1>(p, sm, row, chunk, c0, c1);
  }
}

// ---------------------------------------------------------------------------
// Row merge: one wavefront per row.
constexpr int kMergeWaves = 4;

struct MergeSmem {
  uint64_t stage[kMergeWaves][512];
};

template <int DT>
__global__ __launch_bounds__(kWave* kMergeWaves) void stage1_merge_kernel(Stage1Params p) {
  __shared__ MergeSmem sm;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kMergeWaves + w;
  if (row >= p.rows) return;
  const int S = p.S, K = p.K, capp = p.capp;

  int ni = 0;
  uint32_t ti = 0;
  double oi = -INFINITY, si = 0.0;
  if (lane < S) {
    const size_t rec = (size_t)row * S + lane;
    ni = p.cnt[rec];
    ti = p.thr[rec];
    oi = p.meta[2 * rec];
    si = p.meta[2 * rec + 1];
  }
  // normaliser: z = ln2 * (OFF + log2(sum_s sum_s * 2^(off_s - OFF))), float64
  const double OFF = wave_max(oi);
  const double s = wave_sum(oi == -INFINITY ? 0.0 : si * exp2(oi - OFF));
  if (lane == 0) p.out_lse[row] = kLn2 * (OFF + log2(s));

  // Each chunk holds >= K elements at or above its threshold, so the row's
  // K-th key is at or above the largest threshold; every record holds all of
  // its chunk's elements at or above the chunk threshold (or its exact top K).
  const uint64_t lo = (uint64_t)wave_max(ti) << 32;
  const int span = S * capp;
  const int R = (span + kWave - 1) / kWave;  // <= kMergeSlots (checked on the host)
  const uint64_t* src = p.cands + (size_t)row * span;
  uint64_t v[kMergeSlots];
#pragma unroll
  for (int r = 0; r < kMergeSlots; ++r) {
    v[r] = 0;
    if (r < R) {
      const int i = r * kWave + lane;
      const int ch = i / capp;
      const int n_ch = __shfl(ni, ch < S ? ch : 0);
      const uint64_t k = (i < span && i - ch * capp < n_ch) ? src[i] : 0ull;
      v[r] = k >= lo ? k : 0ull;
    }
  }
  wave_topk_finish(v, R, K, p.idbits, DT == 0, sm.stage[w], p.out_ids + row * K,
                   p.out_vals + row * K);
}

// ---------------------------------------------------------------------------
// Row-persistent kernel (one workgroup per row).

struct RowSmem {
  uint64_t cand[kCandCap];
  double red_d[kS1Waves];
  uint32_t red_u[2][kS1Waves];
  int wn[kS1Waves];
};

// Loads are issued unconditionally so that the wait counts stay static: a
// chunk past the row's end (nvec == 0) loads one vector of the row's start in
// every lane, which costs one cache line per wave.
template <int NV>
__device__ __forceinline__ void load_chunk_vec(v4u32 (&buf)[NV], const char* rowp, int64_t c0,
                                               int64_t nvec, size_t esz) {
  const gvec_ptr base = (gvec_ptr)(rowp + (nvec > 0 ? c0 * esz : 0));
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = j * kS1Threads + threadIdx.x;
    buf[j] = base[vi < nvec ? vi : 0];
  }
}

// One register-resident chunk of the row: fold it into the thread's running
// (max, offset, sum), raise the row threshold `rthr` with this chunk's
// threshold and append the chunk's elements at or above it.
template <int DT, int NV, int GS>
__device__ __forceinline__ void row_process(v4u32 (&raw)[NV], RowSmem& sm, int par, int64_t c0,
                                            int64_t nvec, int K, float& m_run, float& mc_run,
                                            double& s_run, uint32_t& rthr, int& wn) {
  constexpr int G = NV / GS;
  constexpr uint32_t NEG_INF_DW = DT == 0 ? 0xFF80FF80u : 0xFF800000u;
  const int tid = threadIdx.x, w = tid >> 6;
  launder<NV>(raw);
  if (nvec < (int64_t)NV * kS1Threads) {
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (j * kS1Threads + tid >= nvec) raw[j] = v4u32{NEG_INF_DW, NEG_INF_DW, NEG_INF_DW, NEG_INF_DW};
  }
  float gmax[G];
  uint32_t gk[G];
  group_maxima<DT, NV, GS>(raw, gmax, gk);
  float cmax = gmax[0];
#pragma unroll
  for (int g = 1; g < G; ++g) cmax = fmaxf(cmax, gmax[g]);
  const uint32_t Tw = wave_threshold<DT, G>(gk, (K + 3) >> 2);
  if ((tid & 63) == 0) sm.red_u[par][w] = Tw;
  __syncthreads();
  uint32_t t0 = sm.red_u[par][0];
#pragma unroll
  for (int i = 1; i < kS1Waves; ++i) t0 = min(t0, sm.red_u[par][i]);
  rthr = rthr > t0 ? rthr : t0;

  // The previous terms were taken relative to the rounded offset mc_run, so
  // they are rescaled by exactly 2^(mc_run - mc).
  const float m_new = fmaxf(m_run, cmax);
  const float mc = m_new == m_run ? mc_run : m_new * kLog2eF;
  launder<NV>(raw);
  const float acc = exp_collect<DT, NV>(raw, m_new == -INFINITY ? 0.0f : mc, key_threshold(rthr),
                                        c0, sm.cand + w * kWaveCap, wn);
  if (m_new != -INFINITY) {
    const double scale = s_run == 0.0 ? 0.0 : exp2((double)mc_run - (double)mc);
    s_run = s_run * scale + (double)acc;
    m_run = m_new;
    mc_run = mc;
  }
}

// Exact top-K of a whole row from memory (survivors overflow: massive ties).
template <int DT>
__device__ __noinline__ int exact_row_select(const char* rowp, int64_t V, int K, RowSmem& sm) {
  auto key_at = [&](int64_t idx) -> uint64_t {
    const uint32_t bits = DT == 0 ? ((uint32_t)((const uint16_t*)rowp)[idx] << 16)
                                  : ((const uint32_t*)rowp)[idx];
    return cand_key(order_key(bits), (uint32_t)idx);
  };
  uint64_t T = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t c = T | (1ull << bit);
    uint32_t cnt = 0;
    for (int64_t i = threadIdx.x; i < V; i += kS1Threads) cnt += key_at(i) >= c ? 1u : 0u;
    cnt = wave_sum(cnt);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sm.red_u[0][threadIdx.x >> 6] = cnt;
    __syncthreads();
    uint32_t tot = 0;
#pragma unroll
    for (int w = 0; w < kS1Waves; ++w) tot += sm.red_u[0][w];
    if (tot >= (uint32_t)K) T = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) sm.wn[0] = 0;
  __syncthreads();
  for (int64_t i = threadIdx.x; i < V; i += kS1Threads) {
    const uint64_t k = key_at(i);
    if (k >= T) sm.cand[atomicAdd(&sm.wn[0], 1)] = k;
  }
  __syncthreads();
  return sm.wn[0];
}

template <int DT, int NV, int GS>
__global__ __launch_bounds__(kS1Threads) void stage1_row_kernel(Stage1Params p) {
  constexpr int EPV = DT == 0 ? 8 : 4;
  __shared__ RowSmem sm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int64_t row = blockIdx.x;
  const int K = p.K, S = p.S;
  const size_t esz = DT == 0 ? 2 : 4;
  const char* rowp = (const char*)p.logits + (size_t)row * (size_t)p.V * esz;
  const int64_t CH = p.chunk;
  auto nvec_of = [&](int c) -> int64_t {  // 0 past the row's end
    const int64_t c0 = (int64_t)c * CH;
    const int64_t c1 = c0 + CH < p.V ? c0 + CH : p.V;
    return c1 > c0 ? (c1 - c0) / EPV : 0;
  };
  float m_run = -INFINITY, mc_run = -INFINITY;
  double s_run = 0.0;
  uint32_t rthr = 0;
  int wn = 0;
  v4u32 A[NV], Bf[NV];
  load_chunk_vec<NV>(A, rowp, 0, nvec_of(0), esz);
  for (int c = 0; c < S; c += 2) {
    load_chunk_vec<NV>(Bf, rowp, (int64_t)(c + 1) * CH, nvec_of(c + 1), esz);
    row_process<DT, NV, GS>(A, sm, 0, (int64_t)c * CH, nvec_of(c), K, m_run, mc_run, s_run, rthr,
                            wn);
    load_chunk_vec<NV>(A, rowp, (int64_t)(c + 2) * CH, nvec_of(c + 2), esz);
    if (c + 1 < S)
      row_process<DT, NV, GS>(Bf, sm, 1, (int64_t)(c + 1) * CH, nvec_of(c + 1), K, m_run, mc_run,
                              s_run, rthr, wn);
  }

  // row normaliser: per thread s * 2^(mc + m*(log2 e - c)), float64
  const double off = m_run == -INFINITY ? -INFINITY : (double)mc_run + (double)m_run * kLog2eErr;
  const double off_w = wave_max(off);
  __syncthreads();  // every survivor is in; the red_u reads are done
  if (lane == 0) {
    sm.red_d[w] = off_w;
    sm.wn[w] = wn;
  }
  __syncthreads();
  double OFF = sm.red_d[0];
#pragma unroll
  for (int i = 1; i < kS1Waves; ++i) OFF = OFF > sm.red_d[i] ? OFF : sm.red_d[i];
  const double part_w = wave_sum(m_run == -INFINITY ? 0.0 : s_run * exp2(off - OFF));
  int wcnt[kS1Waves], ovf = 0;
#pragma unroll
  for (int i = 0; i < kS1Waves; ++i) {
    wcnt[i] = sm.wn[i];
    ovf |= wcnt[i] > kWaveCap;
  }
  __syncthreads();
  if (lane == 0) sm.red_d[w] = part_w;
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
#pragma unroll
    for (int i = 0; i < kS1Waves; ++i) tot += sm.red_d[i];
    p.out_lse[row] = kLn2 * (OFF + log2(tot));
  }
  if (ovf) {
    // survivors overflowed a wave region: exact selection from memory
    const int n = exact_row_select<DT>(rowp, p.V, K, sm);
    const int np = next_pow2(n < 1 ? 1 : n);
    for (int i = n + tid; i < np; i += kS1Threads) sm.cand[i] = 0;
    __syncthreads();
    bitonic_desc_u64<kS1Threads>(sm.cand, np);
    for (int i = tid; i < K; i += kS1Threads) {
      const uint64_t k = sm.cand[i];
      p.out_ids[row * K + i] = (int32_t)cand_id(k);
      p.out_vals[row * K + i] = key_value(cand_vkey(k));
    }
    return;
  }
  // wave 0 finishes the row from the four regions (<= kCandCap survivors)
  if (w != 0) return;
  const uint64_t lo = (uint64_t)rthr << 32;
  constexpr int R = kCandCap / kWave;
  uint64_t v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    {
      const int i = r * kWave + lane;  // slot i of region i / kWaveCap
      const int ww = i / kWaveCap, k = i - ww * kWaveCap;
      const uint64_t key = k < wcnt[ww] ? sm.cand[i] : 0ull;
      v[r] = key >= lo ? key : 0ull;
    }
  }
  // the survivors are in registers now: sm.cand serves as the staging area
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  wave_topk_finish(v, R, K, p.idbits, DT == 0, sm.cand, p.out_ids + row * K, p.out_vals + row * K);
}

}  // namespace ddt
