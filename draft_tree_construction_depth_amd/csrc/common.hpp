// Shared device helpers for the draft-tree kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ddt {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// Total order on float32 bit patterns as unsigned integers: larger key <=>
// larger value, with -0 mapped onto +0. NaN is outside the supported inputs.
__device__ __forceinline__ uint32_t order_key(uint32_t u) {
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// 64-bit candidate key: value key in the high word, inverted id in the low
// word, so that a larger key means a larger value or, on equal values, a
// lower id. Key 0 never occurs for a real element and marks padding.
__device__ __forceinline__ uint64_t cand_key(uint32_t vkey, uint32_t id) {
  return ((uint64_t)vkey << 32) | (uint32_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint32_t cand_id(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }
__device__ __forceinline__ uint32_t cand_vkey(uint64_t k) { return (uint32_t)(k >> 32); }

// Number of set bits of m at lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Wave-wide reductions (every lane of the wave active; every lane gets the
// result). Inside each row of 16 lanes by DPP moves (quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_ror:4, row_ror:8: no LDS round trips), then the
// four row results combined from readlanes.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

template <int CTRL, typename T>
__device__ __forceinline__ T dpp_move(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit lanes");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = dpp_u32<CTRL>((uint32_t)u), hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}

template <typename T>
__device__ __forceinline__ T lane_value(T v, int lane) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(
        T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}

template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, dpp_move<0xB1>(v));
  v = op(v, dpp_move<0x4E>(v));
  v = op(v, dpp_move<0x124>(v));
  v = op(v, dpp_move<0x128>(v));
  return op(op(lane_value(v, 0), lane_value(v, 16)), op(lane_value(v, 32), lane_value(v, 48)));
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
  return wave_reduce(v, [](T a, T b) { return a > b ? a : b; });
}

template <typename T>
__device__ __forceinline__ T wave_min(T v) {
  return wave_reduce(v, [](T a, T b) { return a < b ? a : b; });
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  return wave_reduce(v, [](T a, T b) { return a + b; });
}

// Inclusive scan of one int per lane over the 64 lanes, by DPP: shifts by
// 1, 2, 4, 8 inside each row of 16 lanes, then row 0's last lane added to
// rows 1 and 3 and lane 31 to rows 2 and 3. Every lane of the wave must be
// active.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Sum of the first w of NW <= 16 per-wave totals in LDS (16-byte aligned);
// total gets the sum of all NW. Lane l < NW reads total l, a DPP scan inside
// the first row of 16 lanes forms the prefixes, and two readlanes at the
// wave's own (uniform) index pick them: no per-wave-index selects. Every
// lane of the wave must be active.
template <int NW>
__device__ __forceinline__ int waves_before(const int* wsum, int w, int& total) {
  static_assert(NW % 4 == 0 && NW <= 16, "at most 16 waves, int4-aligned totals");
  const int lane = threadIdx.x & 63;
  int x = lane < NW ? wsum[lane] : 0;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  const int ws = __builtin_amdgcn_readfirstlane(w);
  total = __builtin_amdgcn_readlane(x, NW - 1);
  const int pre = __builtin_amdgcn_readlane(x, ws > 0 ? ws - 1 : 0);
  return ws > 0 ? pre : 0;
}

// Exclusive scan of one int per thread over the block (every thread calls
// it); total gets the block sum. wsum: NT/64 ints of LDS, 16-byte aligned.
// One barrier; a later call reusing wsum needs a barrier in between.
template <int NT>
__device__ __forceinline__ int block_excl_scan_reg(int x, int* wsum, int& total) {
  constexpr int NW = NT / kWave;
  static_assert(NW % 4 == 0, "int4 reads of the wave totals");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_incl_scan(x);
  if (lane == kWave - 1) wsum[w] = inc;
  __syncthreads();
  return waves_before<NW>(wsum, w, total) + inc - x;
}

// In-place exclusive scan of a[0..n) (LDS) by NT threads; returns the total.
// wsum needs NT/64 ints of LDS. Ends with a barrier.
template <int NT>
__device__ int block_excl_scan(int* a, int n, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int NW = NT / kWave;
  const int seg = (n + NT - 1) / NT;
  const int b0 = min(tid * seg, n), b1 = min(b0 + seg, n);
  int s = 0;
  for (int i = b0; i < b1; ++i) s += a[i];
  const int x = wave_incl_scan(s);
  if (lane == kWave - 1) wsum[w] = x;
  __syncthreads();
  int pre = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    int t = wsum[i];
    pre += (i < w) ? t : 0;
    total += t;
  }
  int run = pre + x - s;
  for (int i = b0; i < b1; ++i) {
    int t = a[i];
    a[i] = run;
    run += t;
  }
  __syncthreads();
  return total;
}

// Bitonic sort of n (a power of two) 64-bit keys in LDS, largest first.
template <int NT>
__device__ void bitonic_desc_u64(uint64_t* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += NT) {
        const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int hi = lo + j;
        const uint64_t x = a[lo], y = a[hi];
        const bool big_first = (lo & k) == 0;
        if (big_first ? (x < y) : (x > y)) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

}  // namespace ddt
