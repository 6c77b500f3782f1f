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
//    workgroup per row then keeps the survivors at or above the largest
//    chunk threshold and ranks them: bf16 rows by a histogram over their
//    value codes (one scan; equal values ordered by id), otherwise through
//    the exact K-th (value, id) key from a ballot bisection over registers
//    (four waves' counts summed in LDS) and counting; then writes the row's
//    table and log-sum-exp (float64).
//  stage1_row_kernel (many rows): one workgroup walks all chunks of its row
//    with double-buffered register loads (chunk i+1 in flight while chunk i
//    is processed), raises the row threshold on a schedule of chunks, keeps
//    whole 16-byte vectors that reach it in LDS (compacting a wave's region
//    against the current threshold when it would overflow) and finishes the
//    row itself: the kept vectors' elements at or above the final threshold
//    become candidates, ranked for bf16 rows by a histogram over their value
//    codes (ties by id inside a code), else by counting larger keys. No
//    records, no second launch.
#pragma once

#include "common.hpp"

namespace ddt {

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
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
// Row merge: one workgroup per row.
constexpr int kMergeWaves = 4;  // one workgroup of four waves per row
constexpr int kMergeWSlots = (kMergeSlots + kMergeWaves - 1) / kMergeWaves;

// Value-code bins of the bf16 merge (codes between the largest chunk
// threshold and the row maximum).
constexpr int kMergeBins = 1024;

struct MergeSmem {
  union alignas(16) {
    uint64_t win[512];                     // the row's K winners (K <= 512)
    uint64_t sorted[kMergeSlots * kWave];  // bf16: candidates in code order
  };
  int hist[kMergeBins];  // bf16: candidates per code, then those in higher codes
  uint64_t ranked[512];  // bf16: the K winners by rank
  uint32_t range[kMergeSlots * kWave];  // bf16: each placed candidate's code range
  int nrel;
  int scan[kMergeWaves];
  int cnt[2][kMergeWaves];  // per-wave counts of a bisection step, double buffered
  int nw[kMergeWaves];
  uint64_t hi[kMergeWaves];
};

// One workgroup per row; wave w holds record slots w, w+4, ... (slot r = 64
// keys). Each chunk holds >= K elements at or above its threshold, so the
// row's K-th key is at or above the largest threshold; every record holds all
// of its chunk's elements at or above the chunk threshold (or its exact top
// K). The K-th largest key comes from a bisection over the key bits whose
// counts are one ballot per slot, summed over the four waves; the K winners
// are then ranked by counting.
template <int DT>
__global__ __launch_bounds__(kWave* kMergeWaves) void stage1_merge_kernel(Stage1Params p) {
  __shared__ MergeSmem sm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int64_t row = blockIdx.x;
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
  if (w == 0) {
    // normaliser: z = ln2 * (OFF + log2(sum_s sum_s * 2^(off_s - OFF))), float64
    const double OFF = wave_max(oi);
    const double s = wave_sum(oi == -INFINITY ? 0.0 : si * exp2(oi - OFF));
    if (lane == 0) p.out_lse[row] = kLn2 * (OFF + log2(s));
  }
  const uint64_t lo = (uint64_t)wave_max(ti) << 32;
  const int span = S * capp;
  const int R = (span + kWave - 1) / kWave;  // <= kMergeSlots (checked on the host)
  const uint64_t* src = p.cands + (size_t)row * span;
  // every slot's load in flight at once (clamped in-bounds reads, masked
  // afterwards: a load under a per-lane condition would wait for the one
  // before it)
  uint64_t v[kMergeWSlots];
#pragma unroll
  for (int q = 0; q < kMergeWSlots; ++q) {
    const int r = w + kMergeWaves * q;
    const int i = r * kWave + lane;
    v[q] = r < R ? src[i < span ? i : span - 1] : 0ull;
  }
#pragma unroll
  for (int q = 0; q < kMergeWSlots; ++q) {
    const int r = w + kMergeWaves * q;
    const int i = r * kWave + lane;
    const int ch = i / capp;
    const int n_ch = __shfl(ni, ch < S ? ch : 0);
    v[q] = (r < R && i < span && i - ch * capp < n_ch && v[q] >= lo) ? v[q] : 0ull;
  }
  int par = 0;
  auto count_ge = [&](uint64_t x) -> int {
    int c = 0;
#pragma unroll
    for (int q = 0; q < kMergeWSlots; ++q)
      if (w + kMergeWaves * q < R) c += __popcll(__ballot(v[q] >= x));
    if (lane == 0) sm.cnt[par][w] = c;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int i = 0; i < kMergeWaves; ++i) t += sm.cnt[par][i];
    par ^= 1;
    return t;
  };
  // every candidate lies in [lo, hi]: the bits above the highest one where
  // lo and hi differ are common to all of them, so the bisection starts there
  uint64_t hi = 0;
#pragma unroll
  for (int q = 0; q < kMergeWSlots; ++q) hi = v[q] > hi ? v[q] : hi;
  hi = wave_max(hi);
  if (lane == 0) sm.hi[w] = hi;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kMergeWaves; ++i) hi = sm.hi[i] > hi ? sm.hi[i] : hi;
  int32_t* oid = p.out_ids + row * K;
  float* oval = p.out_vals + row * K;
  // bf16 rows: every candidate's rank from a histogram over its value code
  // (candidates in higher codes, by an exclusive scan) plus the larger keys
  // of its own code (equal values, ordered by id); no bisection
  const int lo_code = (int)(lo >> 48), hi_code = (int)(hi >> 48);
  const int nbins = hi_code - lo_code + 1;
  if (DT == 0 && lo != 0 && nbins <= kMergeBins) {
    for (int i = tid; i < nbins; i += kWave * kMergeWaves) sm.hist[i] = 0;
    __syncthreads();
    int bin[kMergeWSlots], slot[kMergeWSlots];
#pragma unroll
    for (int q = 0; q < kMergeWSlots; ++q) {
      bin[q] = hi_code - (int)(v[q] >> 48);
      slot[q] = v[q] != 0 ? atomicAdd(&sm.hist[bin[q]], 1) : 0;
    }
    __syncthreads();
    const int total = block_excl_scan<kWave * kMergeWaves>(sm.hist, nbins, sm.scan);  // + barrier
    // candidates of the codes that start below rank K, in code order, each
    // with its code's range [b0, b1) (packed b0 << 16 | b1); they fill
    // positions [0, nrel)
    if (tid == 0) sm.nrel = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kMergeWSlots; ++q) {
      if (v[q] == 0) continue;
      const int b0 = sm.hist[bin[q]];
      if (b0 >= K) continue;
      const int b1 = bin[q] + 1 < nbins ? sm.hist[bin[q] + 1] : total;
      sm.sorted[b0 + slot[q]] = v[q];
      sm.range[b0 + slot[q]] = ((uint32_t)b0 << 16) | (uint32_t)b1;
      if (b0 + slot[q] == b1 - 1) atomicMax(&sm.nrel, b1);
    }
    __syncthreads();
    // one candidate per thread: its rank is its code's start plus the larger
    // keys of its code (16-byte LDS reads, eight keys a batch)
    const int nrel = sm.nrel;
    const u64x2* s2 = (const u64x2*)&sm.sorted[0];
    for (int t = tid; t < nrel; t += kWave * kMergeWaves) {
      const uint64_t me = sm.sorted[t];
      const uint32_t rg = sm.range[t];
      const int b0 = (int)(rg >> 16), b1 = (int)(rg & 0xFFFFu);
      int rank = b0, j = b0;
      if ((j & 1) && j < b1) rank += sm.sorted[j++] > me ? 1 : 0;
      for (; j + 8 <= b1; j += 8) {
        const u64x2 a0 = s2[j >> 1], a1 = s2[(j >> 1) + 1], a2 = s2[(j >> 1) + 2],
                    a3 = s2[(j >> 1) + 3];
        rank += (a0.x > me) + (a0.y > me) + (a1.x > me) + (a1.y > me) + (a2.x > me) + (a2.y > me) +
                (a3.x > me) + (a3.y > me);
      }
      for (; j + 2 <= b1; j += 2) {
        const u64x2 a0 = s2[j >> 1];
        rank += (a0.x > me) + (a0.y > me);
      }
      if (j < b1) rank += sm.sorted[j] > me ? 1 : 0;
      if (rank < K) sm.ranked[rank] = me;
    }
    __syncthreads();
    // the K winners in order, written by consecutive threads
    for (int i = tid; i < K; i += kWave * kMergeWaves) {
      const uint64_t k = sm.ranked[i];
      oid[i] = (int32_t)cand_id(k);
      oval[i] = key_value(cand_vkey(k));
    }
    return;
  }
  const int top = (lo ^ hi) == 0 ? 31 : 63 - __clzll(lo ^ hi);
  uint64_t T = top >= 63 ? 0ull : lo & ~((2ull << top) - 1ull);
  for (int bit = top < 63 ? top : 63; bit >= 32; --bit) {
    if (DT == 0 && bit < 48) break;
    const uint64_t x = T | (1ull << bit);
    if (count_ge(x) >= K) T = x;
  }
  // bf16 value keys have a constant low half: 0x0000 (>= 0) or 0xFFFF
  if (DT == 0) T = (T & 0xFFFF000000000000ull) | ((T >> 63) ? 0ull : 0x0000FFFF00000000ull);
  // ids are < 2^idbits: the inverted id's higher bits are all ones. If
  // exactly K keys reach the K-th value, no id bisection is needed.
  T |= 0xFFFFFFFFull & ~((1ull << p.idbits) - 1ull);
  if (count_ge(T) > K) {
    for (int bit = p.idbits - 1; bit >= 0; --bit) {
      const uint64_t x = T | (1ull << bit);
      if (count_ge(x) >= K) T = x;
    }
  }
  // the K winners (keys are unique) into LDS, waves in order
  int nw = 0;
#pragma unroll
  for (int q = 0; q < kMergeWSlots; ++q)
    if (w + kMergeWaves * q < R) nw += __popcll(__ballot(v[q] >= T && v[q] != 0));
  if (lane == 0) sm.nw[w] = nw;
  __syncthreads();
  int pos = 0;
  for (int i = 0; i < w; ++i) pos += sm.nw[i];
#pragma unroll
  for (int q = 0; q < kMergeWSlots; ++q) {
    if (w + kMergeWaves * q < R) {
      const bool win = v[q] >= T && v[q] != 0;
      const uint64_t M = __ballot(win);
      if (win) sm.win[pos + lanes_below(M)] = v[q];
      pos += __popcll(M);
    }
  }
  __syncthreads();
  // rank of winner i = number of larger winners
  for (int i = tid; i < K; i += kWave * kMergeWaves) {
    const uint64_t mine = sm.win[i];
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < K; ++j) rank += sm.win[j] > mine ? 1 : 0;
    oid[rank] = (int32_t)cand_id(mine);
    oval[rank] = key_value(cand_vkey(mine));
  }
}

// ---------------------------------------------------------------------------
// Row-persistent kernel (one workgroup per row, no barrier inside the loop).
//
// Claims. Each wave keeps in registers the largest 32-element group maxima it
// has seen in its part of the row (at most 64 * kListRegs of them) and
// publishes in LDS the largest value key T with >= ceil(K/4) of them at or
// above T. A claim certifies ceil(K/4) distinct row elements >= T in that
// wave's part, so the smallest of the four claims certifies >= K elements:
// the row's K-th largest value is at or above it. Claims only grow, so a
// wave may read the others' claims without a barrier (a stale claim is a
// smaller, still valid, one); only the first chunk waits for all four.
// Keeping. A 16-byte vector whose maximum reaches the running threshold is
// copied, with its position, into the wave's LDS region (one ballot per
// vector, no per-element work). After the last chunk the kept vectors are
// filtered against the final threshold and the exact top K is selected.
// Normaliser. Per thread, terms 2^(x*c - mc) with an integer offset mc =
// ceil(m*c) of the running maximum m: every exponent argument is <= ~0 and
// raising the offset rescales the float64 sum exactly (ldexp). Each chunk
// takes a max pass (vector maxima, which also feed the claims and the keep
// test) and an exponent pass.
// Loads. Every 16-byte load is a buffer load whose resource covers the
// chunk's bytes inside the row (clamped): vectors past the row's end read as
// zero without touching memory and are then set to -inf.

constexpr int kVecCap = 448;          // kept vectors per wave
constexpr int kKeyCap = 2 * kVecCap;  // candidate keys per wave (in the wave's vector region)
constexpr int kListRegs = 2;          // list of 64 * kListRegs group maxima per wave (>= ceil(K/4))
// Claim schedule: chunks 0 .. kClaimDense-1 update the wave's claim, later
// chunks only every kClaimEvery-th; in between, each lane folds its group
// maxima into a pending maximum per group slot (the maximum of several groups
// is still one element, so the certificate stays valid, only looser). The
// looser threshold keeps more vectors; a wave whose region would overflow
// first compacts it against its current threshold (compact_kept).
constexpr int kClaimDense = 5;
constexpr int kClaimEvery = 3;

// 37.1 KiB: four workgroups fit in one CU's 160 KiB.
struct RowSmem {
  union {
    v4u32 vec[kS1Waves][kVecCap];      // kept vectors
    uint64_t keys[kS1Waves][kKeyCap];  // after the loop: final candidates
  };
  uint32_t vpos[kS1Waves][kVecCap];  // index of each kept vector's first element
  uint32_t lst[kS1Waves][kWave * kListRegs];  // list compaction
  uint32_t claim[kS1Waves];
  uint32_t red_u[kS1Waves];
  uint32_t red_k[kS1Waves];
  int scan[kS1Waves];
  double red_d[kS1Waves];
  int wn[kS1Waves];
};

// Bins of the bf16 rank histogram (one per bf16 value between the row's
// threshold and its maximum) and candidates per thread it handles.
constexpr int kHistBins = 1024;
constexpr int kHistCPT = 4;
static_assert(kHistBins <= kS1Waves * kVecCap, "the histogram lives in vpos");

__device__ __forceinline__ float fmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

template <int DT>
__device__ __forceinline__ float vec_max(const float (&x)[DT == 0 ? 8 : 4]) {
  if constexpr (DT == 0) {
    const float a = fmax3(x[0], x[1], x[2]);
    const float b = fmax3(x[3], x[4], x[5]);
    return fmax3(fmax3(a, x[6], x[7]), b, b);
  } else {
    return fmax3(fmax3(x[0], x[1], x[2]), x[3], x[3]);
  }
}

// Chunk loads: slab j of the chunk (256 threads x 16 B) at vector offset
// 16 t + 4096 j through one buffer resource over the chunk's bytes inside the
// row, so vectors past the row's end read as zero without touching memory.
// (One resource per slab cost about 17 scalar instructions per load; one per
// chunk, 2.8 us less per batch-64 launch.) The logits are read once, so the
// loads carry the nontemporal hint.
constexpr int kLoadNT = 2;  // cache-policy bit "nt" of buffer loads
template <int NV>
__device__ __forceinline__ void load_chunk_buf(v4u32 (&buf)[NV], const char* rowp,
                                               int64_t cbyte, int64_t rowbytes) {
  // one resource over the chunk's bytes that lie inside the row; slab j at
  // vector offset j x 4 KiB (the bounds check covers the vector offset)
  const int64_t left = rowbytes - cbyte;
  constexpr int kCB = NV * kS1Threads * 16;
  const int nrec = left <= 0 ? 0 : (left >= kCB ? kCB : (int)left);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(rowp + (left > 0 ? cbyte : 0)), (short)0, nrec, 0x00020000);
  // (the slab offsets are formed at each load, not held in registers)
  int voff = (int)threadIdx.x * 16;
  asm volatile("" : "+v"(voff));
#pragma unroll
  for (int j = 0; j < NV; ++j)
    buf[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + j * kS1Threads * 16, 0, kLoadNT);
}

// Vector maxima of a register-resident chunk.
template <int DT, int NV>
__device__ __forceinline__ void max_pass(v4u32 (&raw)[NV], float (&vmax)[NV]) {
  constexpr int EPV = DT == 0 ? 8 : 4;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    asm volatile("" : "+v"(raw[j]));  // convert, use and drop vector j before j+1
    float x[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) x[e] = __uint_as_float(elem_bits<DT>(raw[j], e));
    vmax[j] = vec_max<DT>(x);
  }
}

// The thread's sum of 2^(x*c - mc) over the chunk: 8-term sums per vector,
// then pairwise over vectors.
template <int DT, int NV>
__device__ __forceinline__ float exp_pass(v4u32 (&raw)[NV], float mc) {
  constexpr int EPV = DT == 0 ? 8 : 4;
  static_assert(NV <= 16 && (NV & (NV - 1)) == 0, "pairwise levels");
  float lvl[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float total = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    asm volatile("" : "+v"(raw[j]));
    float a = __builtin_amdgcn_exp2f(__builtin_fmaf(__uint_as_float(elem_bits<DT>(raw[j], 0)),
                                                    kLog2eF, -mc));
#pragma unroll
    for (int e = 1; e < EPV; ++e)
      a += __builtin_amdgcn_exp2f(__builtin_fmaf(__uint_as_float(elem_bits<DT>(raw[j], e)),
                                                 kLog2eF, -mc));
    asm volatile("" : "+v"(a));
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

// Raise this wave's claim with G new group-maximum keys per lane (0 = a group
// of padding only). lst holds the list (0 = empty slot); stage is wave-private
// LDS for 64 * kListRegs keys. Returns the claim (0 = none yet).
template <int DT, int G>
__device__ __forceinline__ uint32_t claim_update(uint32_t (&lst)[kListRegs],
                                                 const uint32_t (&gk)[G], int need,
                                                 int lregs, uint32_t* stage) {
  uint32_t T = 0;
  for (int bit = 31; bit >= (DT == 0 ? 16 : 0); --bit) {
    const uint32_t c = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < kListRegs; ++r)
      if (r < lregs) cnt += __popcll(__ballot(lst[r] >= c));
#pragma unroll
    for (int g = 0; g < G; ++g) cnt += __popcll(__ballot(gk[g] >= c));
    if (cnt >= need) T = c;
  }
  // keep the entries at or above T (all nonzero entries while T = 0)
  const uint32_t lo = T ? T : 1u;
  const int cap = kWave * lregs;
  const int lane = threadIdx.x & 63;
  int n = 0;
  auto put = [&](uint32_t v) {
    const bool keep = v >= lo;
    const uint64_t M = __ballot(keep);
    const int pos = n + lanes_below(M);
    if (keep && pos < cap) stage[pos] = v;
    n += __popcll(M);
  };
#pragma unroll
  for (int r = 0; r < kListRegs; ++r)
    if (r < lregs) put(lst[r]);
#pragma unroll
  for (int g = 0; g < G; ++g) put(gk[g]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int r = 0; r < kListRegs; ++r) {
    const int i = r * kWave + lane;
    lst[r] = (r < lregs && i < n && i < cap) ? stage[i] : 0u;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return T;
}

// Keep, in order, only the wave's kept vectors whose maximum reaches tf
// (wave-local; a write never passes the vectors still to be read). Returns
// the new count.
template <int DT>
__device__ __forceinline__ int compact_kept(RowSmem& sm, int w, int n, float tf) {
  constexpr int EPV = DT == 0 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  int kept = 0;
  for (int b = 0; b < n; b += kWave) {
    const int i = b + lane;
    const bool valid = i < n;
    const v4u32 v = valid ? sm.vec[w][i] : v4u32{0u, 0u, 0u, 0u};
    const uint32_t ps = valid ? sm.vpos[w][i] : 0u;
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < EPV; ++e) m = fmaxf(m, __uint_as_float(elem_bits<DT>(v, e)));
    const bool keep = valid && m >= tf;
    const uint64_t M = __ballot(keep);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (keep) {
      const int pos = kept + lanes_below(M);
      sm.vec[w][pos] = v;
      sm.vpos[w][pos] = ps;
    }
    kept += __popcll(M);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return kept;
}

struct RowRun {
  float m;       // running maximum of the thread's elements
  float mc;      // integer offset ceil(m * c) of s (-inf while m = -inf)
  double s;      // sum of 2^(x*c - mc) over the thread's elements so far
  uint32_t thr;  // running threshold (value key; 0 = none yet)
  int wn;        // vectors kept by this wave (uniform)
  uint32_t lst[kListRegs];
  uint32_t pend[4];  // group maxima not yet in the list (0 = none)
};

__device__ __forceinline__ bool claim_due(int c) {
  return c < kClaimDense || (c - kClaimDense) % kClaimEvery == kClaimEvery - 1;
}

template <int DT, int NV, int GS, bool FIRST>
__device__ __forceinline__ void row_chunk(v4u32 (&raw)[NV], RowSmem& sm, int64_t c0, int64_t nvec,
                                          int need, int lregs, RowRun& st, bool upd) {
  constexpr int EPV = DT == 0 ? 8 : 4;
  constexpr int G = NV / GS;
  static_assert(G <= 4, "pending slots");
  constexpr uint32_t NEG_INF_DW = DT == 0 ? 0xFF80FF80u : 0xFF800000u;
  static_assert(GS == 4, "group = 4 vectors");
  const int tid = threadIdx.x, w = tid >> 6;
  if (nvec < (int64_t)NV * kS1Threads) {
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (j * kS1Threads + tid >= nvec) raw[j] = v4u32{NEG_INF_DW, NEG_INF_DW, NEG_INF_DW, NEG_INF_DW};
  }
  float vmax[NV];
  max_pass<DT, NV>(raw, vmax);
  uint32_t gk[G];
  float cm = -INFINITY;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float m = fmax3(fmax3(vmax[4 * g], vmax[4 * g + 1], vmax[4 * g + 2]), vmax[4 * g + 3],
                          vmax[4 * g + 3]);
    gk[g] = m == -INFINITY ? 0u : order_key(__float_as_uint(m));
    cm = fmax3(cm, m, m);
  }
  if (cm > st.m) {
    const float mcn = ceilf(cm * kLog2eF);
    if (mcn != st.mc) {
      const double d = (double)st.mc - (double)mcn;  // exact: both are integers; -inf at first
      st.s = d < -1100.0 ? 0.0 : ldexp(st.s, (int)d);
      st.mc = mcn;
    }
    st.m = cm;
  }

  // claims
  if (FIRST || upd) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      gk[g] = gk[g] > st.pend[g] ? gk[g] : st.pend[g];
      st.pend[g] = 0;
    }
    const uint32_t Tw = claim_update<DT, G>(st.lst, gk, need, lregs, &sm.lst[w][0]);
    if ((tid & 63) == 0)
      __hip_atomic_store(&sm.claim[w], Tw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) st.pend[g] = st.pend[g] > gk[g] ? st.pend[g] : gk[g];
  }
  if (FIRST) __syncthreads();
  uint32_t t0 = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < kS1Waves; ++i)
    t0 = min(t0, __hip_atomic_load(&sm.claim[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
  st.thr = st.thr > t0 ? st.thr : t0;
  const float tf = key_threshold(st.thr);

  // normaliser terms
  st.s += (double)exp_pass<DT, NV>(raw, st.m == -INFINITY ? 0.0f : st.mc);

  // keep the vectors that reach the threshold; if they would not fit, first
  // drop the kept vectors that the (since raised) threshold excludes
  uint64_t KM[NV];
  int add = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    KM[j] = __ballot(vmax[j] >= tf);
    add += __popcll(KM[j]);
  }
  if (add) {
    if (st.wn + add > kVecCap && st.wn <= kVecCap) st.wn = compact_kept<DT>(sm, w, st.wn, tf);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const uint64_t M = KM[j];
      if (M) {
        const int pos = st.wn + lanes_below(M);
        if (((M >> (tid & 63)) & 1) && pos < kVecCap) {
          sm.vec[w][pos] = raw[j];
          sm.vpos[w][pos] = (uint32_t)c0 + (uint32_t)((j * kS1Threads + tid) * EPV);
        }
        st.wn += __popcll(M);
      }
    }
  }
}

// Exact top-K of a whole row from memory (kept vectors overflowed: massive
// ties). Leaves the K keys in keys (flat) and returns K.
template <int DT>
__device__ __noinline__ int exact_row_select(const char* rowp, int64_t V, int K, RowSmem& sm) {
  uint64_t* out = &sm.keys[0][0];
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
  for (int64_t i = threadIdx.x; i < V; i += kS1Threads) {
    const uint64_t k = key_at(i);
    if (k >= T) out[atomicAdd(&sm.wn[0], 1)] = k;
  }
  __syncthreads();
  return sm.wn[0];
}

// Start of wave 1, 2, 3's candidates in the flat candidate order.
__device__ __forceinline__ int b1_of(const int (&k)[kS1Waves]) { return k[0]; }
__device__ __forceinline__ int b2_of(const int (&k)[kS1Waves]) { return k[0] + k[1]; }
__device__ __forceinline__ int b3_of(const int (&k)[kS1Waves]) { return k[0] + k[1] + k[2]; }

// Wave priority by progress through the row. A CU holds up to four rows
// whose waves share each SIMD, and the SIMD's arbiter otherwise favours the
// oldest wave: the first row dispatched runs far ahead and the last one ends
// nearly alone, with little to hide its latency. Lowering a wave's priority
// as it advances (four levels over the row) keeps the rows of a CU closer
// together (batch 64: rows end 45-54 us into the launch instead of 35-61).
// Only when every row is resident at once (PRIO): while more rows wait for a
// slot, staggered ends keep the CUs' slots refilling evenly (batch 256: 2%
// slower with the schedule on every row, 3% with it on the last generation).
__device__ __forceinline__ void progress_priority(int c, int S) {
  const int q = (4 * c) / S;
  if (q <= 0)
    __builtin_amdgcn_s_setprio(3);
  else if (q == 1)
    __builtin_amdgcn_s_setprio(2);
  else if (q == 2)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

template <int DT, int NV, int GS, bool PRIO>
__global__ __launch_bounds__(kS1Threads, 4) void stage1_row_kernel(Stage1Params p) {
  constexpr int EPV = DT == 0 ? 8 : 4;
  __shared__ RowSmem sm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int64_t row = blockIdx.x;
  const int K = p.K, S = p.S;
  const int need = (K + 3) >> 2, lregs = (need + kWave - 1) / kWave;
  const size_t esz = DT == 0 ? 2 : 4;
  const char* rowp = (const char*)p.logits + (size_t)row * (size_t)p.V * esz;
  const int64_t CH = p.chunk;
  const int64_t rowbytes = p.V * (int64_t)esz, CB = CH * (int64_t)esz;
  auto nvec_of = [&](int c) -> int64_t {  // 0 past the row's end
    const int64_t c0 = (int64_t)c * CH;
    const int64_t c1 = c0 + CH < p.V ? c0 + CH : p.V;
    return c1 > c0 ? (c1 - c0) / EPV : 0;
  };
  RowRun st;
  st.m = -INFINITY;
  st.mc = -INFINITY;
  st.s = 0.0;
  st.thr = 0;
  st.wn = 0;
#pragma unroll
  for (int r = 0; r < kListRegs; ++r) st.lst[r] = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) st.pend[g] = 0;

  v4u32 A[NV], Bf[NV];
  load_chunk_buf<NV>(A, rowp, 0, rowbytes);
  load_chunk_buf<NV>(Bf, rowp, CB, rowbytes);
  // the priority changes only at the first chunk of each quarter of the row:
  // pnext is the next such chunk (one compare per chunk instead of the
  // division and the level switch)
  int pnext = 0;
  auto prio = [&](int c) {
    if (PRIO && c >= pnext) {
      progress_priority(c, S);
      const int q = (4 * c) / S;
      pnext = ((q + 1) * S + 3) / 4;
    }
  };
  prio(0);
  row_chunk<DT, NV, GS, true>(A, sm, 0, nvec_of(0), need, lregs, st, true);
  load_chunk_buf<NV>(A, rowp, 2 * CB, rowbytes);
  for (int c = 1; c < S; c += 2) {
    prio(c);
    row_chunk<DT, NV, GS, false>(Bf, sm, (int64_t)c * CH, nvec_of(c), need, lregs, st,
                                 claim_due(c));
    load_chunk_buf<NV>(Bf, rowp, (int64_t)(c + 2) * CB, rowbytes);
    prio(c + 1);
    if (c + 1 < S)
      row_chunk<DT, NV, GS, false>(A, sm, (int64_t)(c + 1) * CH, nvec_of(c + 1), need, lregs, st,
                                   claim_due(c + 1));
    load_chunk_buf<NV>(A, rowp, (int64_t)(c + 3) * CB, rowbytes);
  }

  // row normaliser: per thread s * 2^(mc + m*(log2 e - c)), float64
  const double off = st.m == -INFINITY ? -INFINITY : (double)st.mc + (double)st.m * kLog2eErr;
  const double off_w = wave_max(off);
  const uint32_t top_w = wave_max(st.m == -INFINITY ? 0u : order_key(__float_as_uint(st.m)));
  if (lane == 0) {
    sm.red_d[w] = off_w;
    sm.red_k[w] = top_w;
    sm.wn[w] = st.wn;
  }
  __syncthreads();  // claims, kept vectors and counts are final
  double OFF = sm.red_d[0];
#pragma unroll
  for (int i = 1; i < kS1Waves; ++i) OFF = OFF > sm.red_d[i] ? OFF : sm.red_d[i];
  const double part_w = wave_sum(st.m == -INFINITY ? 0.0 : st.s * exp2(off - OFF));
  uint32_t T = 0xFFFFFFFFu, TOP = 0;
  int ovf = 0;
#pragma unroll
  for (int i = 0; i < kS1Waves; ++i) {
    T = min(T, sm.claim[i]);
    TOP = max(TOP, sm.red_k[i]);
    ovf |= sm.wn[i] > kVecCap;
  }
  __syncthreads();
  if (lane == 0) sm.red_d[w] = part_w;

  // filter this wave's kept vectors against the final threshold; the keys
  // go to the same region once the vectors are in registers
  constexpr int VR = (kVecCap + kWave - 1) / kWave;
  int kn = 0;
  if (!ovf) {
    const float tf = key_threshold(T);
    const int nvk = st.wn;
    v4u32 kv[VR];
    uint32_t kp[VR];
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      const int i = r * kWave + lane;
      const bool valid = i < nvk;
      kv[r] = valid ? sm.vec[w][i] : v4u32{0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
      kp[r] = valid ? sm.vpos[w][i] : 0u;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // per lane: which elements of its vectors reach the threshold; then one
    // wave prefix of the counts places them
    uint32_t km[VR];
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      uint32_t m = 0;
      if (r * kWave < nvk) {
#pragma unroll
        for (int e = 0; e < EPV; ++e)
          m |= (__uint_as_float(elem_bits<DT>(kv[r], e)) >= tf ? 1u : 0u) << e;
        m = (r * kWave + lane) < nvk ? m : 0u;
      }
      km[r] = m;
      cnt += __popc(m);
    }
    int pos = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {  // cnt <= 7 * 8 < 64
      const uint64_t M = __ballot((cnt >> bit) & 1);
      pos += lanes_below(M) << bit;
      tot += __popcll(M) << bit;
    }
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      uint32_t m = km[r];
      while (m) {
        const int e = __builtin_ctz(m);
        m &= m - 1;
        if (pos < kKeyCap)
          sm.keys[w][pos] = cand_key(order_key(elem_bits<DT>(kv[r], e)), kp[r] + e);
        ++pos;
      }
    }
    kn = tot;
  }
  if (lane == 0) sm.wn[w] = kn;
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
#pragma unroll
    for (int i = 0; i < kS1Waves; ++i) tot += sm.red_d[i];
    p.out_lse[row] = kLn2 * (OFF + log2(tot));
  }
  int kcnt[kS1Waves], ntot = 0;
#pragma unroll
  for (int i = 0; i < kS1Waves; ++i) {
    kcnt[i] = sm.wn[i];
    ovf |= kcnt[i] > kKeyCap;
    ntot += kcnt[i];
  }
  int32_t* oid = p.out_ids + row * K;
  float* oval = p.out_vals + row * K;
  if (ovf) {
    // exact selection from memory
    __syncthreads();
    const int n = exact_row_select<DT>(rowp, p.V, K, sm);
    uint64_t* a = &sm.keys[0][0];
    const int np = next_pow2(n < 1 ? 1 : n);
    for (int i = n + tid; i < np; i += kS1Threads) a[i] = 0;
    __syncthreads();
    bitonic_desc_u64<kS1Threads>(a, np);
    for (int i = tid; i < K; i += kS1Threads) {
      const uint64_t k = a[i];
      oid[i] = (int32_t)cand_id(k);
      oval[i] = key_value(cand_vkey(k));
    }
    return;
  }
  // >= K distinct candidates. bf16 rows: a histogram over the value codes
  // between the threshold and the row maximum gives each candidate the number
  // of larger values (an exclusive scan), and only equal values are compared
  // one by one (by id). Otherwise each rank is the number of larger keys.
  const int R = (T != 0 && TOP >= T) ? (int)((TOP - T) >> 16) + 1 : kHistBins + 1;
  if (DT == 0 && ntot <= kHistCPT * kS1Threads && R <= kHistBins) {
    int* hist = (int*)&sm.vpos[0][0];  // the kept vectors' positions are dead
    for (int i = tid; i < R; i += kS1Threads) hist[i] = 0;
    uint64_t mk[kHistCPT];
    int bin[kHistCPT], slot[kHistCPT];
#pragma unroll
    for (int c = 0; c < kHistCPT; ++c) {
      const int i = tid + c * kS1Threads;
      const int ww = (i >= b1_of(kcnt)) + (i >= b2_of(kcnt)) + (i >= b3_of(kcnt));
      const int off0 = ww == 0 ? 0 : ww == 1 ? b1_of(kcnt) : ww == 2 ? b2_of(kcnt) : b3_of(kcnt);
      mk[c] = i < ntot ? sm.keys[ww][i - off0] : 0ull;
      bin[c] = (int)((TOP - cand_vkey(mk[c])) >> 16);
    }
    __syncthreads();  // every source key is in registers; the histogram is zero
#pragma unroll
    for (int c = 0; c < kHistCPT; ++c)
      if (tid + c * kS1Threads < ntot) slot[c] = atomicAdd(&hist[bin[c]], 1);
    __syncthreads();
    block_excl_scan<kS1Threads>(hist, R, sm.scan);  // hist[b]: candidates in bins < b
    uint64_t* sorted = &sm.keys[0][0];
#pragma unroll
    for (int c = 0; c < kHistCPT; ++c)
      if (tid + c * kS1Threads < ntot) sorted[hist[bin[c]] + slot[c]] = mk[c];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kHistCPT; ++c) {
      if (tid + c * kS1Threads < ntot) {
        const int lo = hist[bin[c]], hi = bin[c] + 1 < R ? hist[bin[c] + 1] : ntot;
        int rank = lo;
        for (int q = lo; q < hi; ++q) rank += sorted[q] > mk[c] ? 1 : 0;
        if (rank < K) {
          oid[rank] = (int32_t)cand_id(mk[c]);
          oval[rank] = key_value(cand_vkey(mk[c]));
        }
      }
    }
    return;
  }
  // >= K distinct candidates: each one's rank is the number of larger ones
  const int b1 = kcnt[0], b2 = b1 + kcnt[1], b3 = b2 + kcnt[2];
  for (int i = tid; i < ntot; i += kS1Threads) {
    const int ww = (i >= b1) + (i >= b2) + (i >= b3);
    const uint64_t mine = sm.keys[ww][i - (ww == 0 ? 0 : ww == 1 ? b1 : ww == 2 ? b2 : b3)];
    int rank = 0;
#pragma unroll
    for (int q = 0; q < kS1Waves; ++q) {
      // 16-byte LDS reads, eight keys per batch (the region starts 16-byte aligned)
      const u64x2* kq = (const u64x2*)&sm.keys[q][0];
      const int n = kcnt[q], np = n >> 1;
      int j = 0;
      for (; j + 4 <= np; j += 4) {
        const u64x2 a0 = kq[j], a1 = kq[j + 1], a2 = kq[j + 2], a3 = kq[j + 3];
        rank += (a0.x > mine) + (a0.y > mine) + (a1.x > mine) + (a1.y > mine) +
                (a2.x > mine) + (a2.y > mine) + (a3.x > mine) + (a3.y > mine);
      }
      for (; j < np; ++j) {
        const u64x2 a0 = kq[j];
        rank += (a0.x > mine) + (a0.y > mine);
      }
      if (n & 1) rank += sm.keys[q][n - 1] > mine ? 1 : 0;
    }
    if (rank < K) {
      oid[rank] = (int32_t)cand_id(mine);
      oval[rank] = key_value(cand_vkey(mine));
    }
  }
}

}  // namespace ddt
