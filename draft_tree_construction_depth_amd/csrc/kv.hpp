// KV-cache compaction to the accepted path.
//
// DDTree explainer, section 5 ("KV cache management"): after each round only
// the accepted path's cache is kept. The verification pass wrote the key and
// value rows of the tree's nodes at positions past + j (j = 0 the root, the
// bonus token; j = 1..B the nodes in output order). After the walk accepted
// nodes a_1..a_n, rows past + i (i = 1..n) take the rows of node a_i and the
// cache's length becomes past + n + 1; every other row is left as it was.
//
// MI355X design: the work is a scattered copy of n rows per (layer, request,
// KV head), HBM-bound. One wavefront per such slice moves its K and V rows:
// a row of R bytes (R <= 1024, a multiple of 16) is R/16 lanes of 16-byte
// loads, so a wave moves 64*16/R rows per instruction. In place is safe
// without a barrier: node numbers increase along a path (a_i >= i), so a
// destination row past + i is never the source of a later row, and a wave's
// stores of a batch are issued after that batch's loads and all earlier ones
// have returned.
#pragma once

#include "common.hpp"

namespace ddt {

constexpr int kKvThreads = 256;
constexpr int kKvBatch = 8;  // load groups held in registers per batch

struct KvParams {
  unsigned char* k;  // [layers][batch][heads][cap][row_bytes]
  unsigned char* v;
  int64_t layers, batch, cap;
  int32_t heads;
  int32_t row_bytes;   // multiple of 16, <= 1024
  const int32_t* past_len;    // [batch]
  const int32_t* accepted;    // [batch][L] node numbers, -1 padded
  const int32_t* accept_len;  // [batch]
  int32_t L;
  int32_t* new_len;  // [batch], may be null
};

typedef unsigned int kv_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kKvThreads) void kv_compact_kernel(KvParams p) {
  const int64_t slices = p.layers * p.batch * p.heads;
  const int64_t slice = (int64_t)blockIdx.x * (kKvThreads / kWave) + (threadIdx.x >> 6);
  if (slice >= slices) return;  // whole wave
  const int lane = threadIdx.x & 63;
  const int64_t b = (slice / p.heads) % p.batch;
  const int head = (int)(slice % p.heads);
  const int64_t layer = slice / (p.heads * p.batch);
  const int past = p.past_len[b];
  int n = p.accept_len[b];
  n = n < 0 ? 0 : (n > p.L ? p.L : n);
  if (layer == 0 && head == 0 && lane == 0 && p.new_len) p.new_len[b] = past + n + 1;
  const int lpr = p.row_bytes >> 4;  // lanes per row
  const int rpi = kWave / lpr;       // rows per load instruction
  const int q = lane / lpr, ch = lane - q * lpr;
  const bool lane_on = q < rpi;      // lanes past rpi * lpr idle
  const size_t slice_off = (size_t)slice * (size_t)p.cap * (size_t)p.row_bytes;
  const int32_t* acc = p.accepted + b * p.L;
  for (int i0 = 1; i0 <= n; i0 += kKvBatch * rpi) {  // uniform
    kv_u32x4 kr[kKvBatch], vr[kKvBatch];
    int64_t dst[kKvBatch];
#pragma unroll
    for (int g = 0; g < kKvBatch; ++g) {
      const int i = i0 + g * rpi + q;  // this lane's row: slot past + i
      dst[g] = -1;
      if (lane_on && i <= n) {
        const int node = acc[i - 1];
        const int64_t src = (int64_t)past + node, d = (int64_t)past + i;
        if (node >= 0 && src < p.cap && d < p.cap && past >= 0) {
          const size_t so = slice_off + (size_t)src * p.row_bytes + 16 * ch;
          kr[g] = *(const kv_u32x4*)(p.k + so);
          vr[g] = *(const kv_u32x4*)(p.v + so);
          dst[g] = d;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < kKvBatch; ++g) {
      if (dst[g] >= 0) {
        const size_t dof = slice_off + (size_t)dst[g] * p.row_bytes + 16 * ch;
        *(kv_u32x4*)(p.k + dof) = kr[g];
        *(kv_u32x4*)(p.v + dof) = vr[g];
      }
    }
  }
}

}  // namespace ddt
