// Read-ceiling probe: the stage-1 launch geometry and load path with nothing
// computed on the data.
//
// Stage 1 (SparklingTree post, "Step 1: Sorting the DFlash marginals") reads
// every drafter row once. Its speed of light on this chip is not the HBM
// data-sheet peak but what a kernel that only streams those rows reaches: one
// 256-thread workgroup per row, chunks of 256 threads x NV x 16 bytes loaded
// through per-slab buffer resources with the nontemporal hint, double
// buffered in registers. The loaded words are XOR-folded and one word per
// wave is written, so the loads cannot be dropped; the written bytes (16 per
// row) are negligible. The measured rate is the practical ceiling the stage-1
// kernel's achieved bandwidth is reported against.
#pragma once

#include "stage1.hpp"

namespace ddt {

struct ProbeParams {
  const char* src;
  int64_t row_bytes;  // a multiple of 16
  uint32_t* sink;     // [rows][4]
};

template <int NV>
__device__ __forceinline__ uint32_t fold_chunk(const v4u32 (&a)[NV]) {
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) x ^= a[j][0] ^ a[j][1] ^ a[j][2] ^ a[j][3];
  return x;
}

template <int NV>
__global__ __launch_bounds__(kS1Threads) void read_probe_kernel(ProbeParams p) {
  const char* rowp = p.src + (size_t)blockIdx.x * p.row_bytes;
  constexpr int64_t kChunk = (int64_t)kS1Threads * NV * 16;
  v4u32 a[NV], b[NV];
  uint32_t acc = 0;
  load_chunk_buf<NV>(a, rowp, 0, p.row_bytes);
  for (int64_t c = 0; c < p.row_bytes; c += 2 * kChunk) {
    load_chunk_buf<NV>(b, rowp, c + kChunk, p.row_bytes);  // beyond the row: zeros
    acc ^= fold_chunk<NV>(a);
    load_chunk_buf<NV>(a, rowp, c + 2 * kChunk, p.row_bytes);
    acc ^= fold_chunk<NV>(b);
  }
  acc = wave_reduce(acc, [](uint32_t u, uint32_t v) { return u ^ v; });
  if ((threadIdx.x & 63) == 0) p.sink[(size_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

}  // namespace ddt
