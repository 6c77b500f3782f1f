// Read-ceiling probe: the stage-1 launch geometry and load path with nothing
// computed on the data.
//
// Stage 1 (SparklingTree post, "Step 1: Sorting the DFlash marginals") reads
// every drafter row once. Its speed of light on this chip is not the HBM
// data-sheet peak but what a kernel that only streams those rows reaches: one
// 256-thread workgroup per row, chunks of 256 threads x NV x 16 bytes loaded
// through one buffer resource per chunk with the nontemporal hint, double
// buffered in registers. The loaded words are XOR-folded and one word per
// wave is written, so the loads cannot be dropped; the written bytes (16 per
// row) are negligible. The measured rate is the practical ceiling the stage-1
// kernel's achieved bandwidth is reported against.
#pragma once

#include "stage1.hpp"
#include "treespark.hpp"

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


// TreeSpark load probe: the schedule of ts_gemm_kernel's loads with nothing
// computed (TreeSpark README, item 1: each depth streams the head weight W
// once while every workgroup re-reads its parents' embedding rows). One
// 256-thread workgroup per 128 vocabulary rows, two per CU, a 4-stage W ring
// filled by buffer-to-LDS loads three steps ahead, one barrier per step;
// EPAT selects the embedding loads that go with it (128 parents, two steps
// ahead, into registers): 0 none, 1 the MFMA B layout (16 bytes of each of
// 32 parents' rows per instruction), 2 whole 128-byte lines (8 parents per
// instruction), 3 whole lines of only the first 16 parents of each wave (half
// the embedding traffic). WPOL is W's cache policy (2: nt, 0x12: sc1 nt). The words
// read are XOR-folded; a word is written only on an impossible value, so the
// loads stay live and the written bytes are nil.
struct TsProbeParams {
  const uint16_t* W;
  const uint16_t* E;
  const int32_t* ptok;  // [128] parent tokens
  int64_t V;
  int32_t H;
  uint32_t* sink;       // [256]
};

template <int EPAT, int WPOL>
__global__ __launch_bounds__(kTsThreads, 2) void ts_load_probe_kernel(TsProbeParams p) {
  __shared__ TsGemmSmem sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int ws = __builtin_amdgcn_readfirstlane(w);
  const int64_t V = p.V;
  const int H = p.H, nks = H / kTsKT;
  const int64_t vt0 = (int64_t)blockIdx.x * kTsBV;
  const int64_t wbytes = (V - vt0) * H * 2;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.W + vt0 * H), (short)0, (int)(wbytes < 0x7FFFFFFF ? wbytes : 0x7FFFFFFF), 0x00020000);
  const __amdgpu_buffer_rsrc_t ers = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.E, (short)0, (int)(uint32_t)(V * H * 2), 0x00020000);
  uint32_t woff[4], eoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t v = vt0 + 8 * (4 * i + w) + (l >> 3);
    woff[i] = (uint32_t)(((v < V ? v : V - 1) - vt0) * H * 2 + (((l & 7) ^ (l >> 3)) << 4));
    if (EPAT == 1)
      eoff[i] = (uint32_t)p.ptok[32 * w + (l & 31)] * (uint32_t)H * 2u + 16u * (uint32_t)(l >> 5) +
                32u * (uint32_t)i;
    else
      eoff[i] = (uint32_t)p.ptok[32 * w + 8 * i + (l >> 3)] * (uint32_t)H * 2u +
                (uint32_t)(((l & 7) ^ (l >> 3)) << 4);
  }
  auto load_w = [&](int ks) {
    const int kc = ks < nks ? ks : nks - 1;
    const int st = ks % kTsStages;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (ts_lds_ptr)&sm.w[st][8 * (4 * i + ws)][0], 16,
                                               woff[i], kc * kTsKT * 2, 0, WPOL);
  };
  auto load_e = [&](u32x4 (&d)[4], int ks) {
    if (EPAT == 0) return;
    const int kc = ks < nks ? ks : nks - 1;
#pragma unroll
    for (int i = 0; i < (EPAT == 3 ? 2 : 4); ++i)
      d[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ers, (int)eoff[i], kc * kTsKT * 2, 0));
  };
  // the GEMM's wait: W(ks) and E(ks) arrived, later steps' loads in flight
  constexpr int kWait = EPAT == 0 ? 0x0F78 : EPAT == 3 ? 0x0F7A : 0x0F7C;  // vmcnt(8 / 10 / 12)
  uint32_t acc = 0;
  auto step = [&](int ks, u32x4 (&ec)[4], u32x4 (&en)[4]) {
    __builtin_amdgcn_s_waitcnt(kWait);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    load_e(en, ks + 2);
    load_w(ks + 3);
    const uint32_t a = (uint32_t)(uintptr_t)(ts_lds_ptr)&sm.w[ks % kTsStages][l & 31][0] +
                       16u * (uint32_t)(l >> 5);
    u32x4 x;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(a));
    acc ^= x[0] ^ x[3];
    if (EPAT == 3) acc ^= ec[0][0] ^ ec[1][1];
    else if (EPAT != 0) acc ^= ec[0][0] ^ ec[1][1] ^ ec[2][2] ^ ec[3][3];
  };
  asm volatile("" ::"v"(eoff[0]), "v"(eoff[1]), "v"(eoff[2]), "v"(eoff[3]));
  u32x4 e0[4] = {}, e1[4] = {}, e2[4] = {};
  load_w(0);
  asm volatile("" ::: "memory");
  load_e(e0, 0);
  asm volatile("" ::: "memory");
  load_w(1);
  asm volatile("" ::: "memory");
  load_e(e1, 1);
  asm volatile("" ::: "memory");
  load_w(2);
  int ks = 0;
  for (; ks + 3 <= nks; ks += 3) {
    step(ks, e0, e2);
    step(ks + 1, e1, e0);
    step(ks + 2, e2, e1);
  }
  if (ks < nks) step(ks, e0, e2);
  if (ks + 1 < nks) step(ks + 1, e1, e0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (acc == 0x9E3779B9u) p.sink[tid] = acc;
}

// The same loads for a 256-row vocabulary tile: eight waves (one workgroup
// per CU, a 4-stage 32 KB W ring), waves w and w + 4 sharing parents
// 32 (w % 4) .. + 31, each loading half of their whole-line chunks, so the
// embedding traffic per W byte is half the 128-row tile's.
template <int WPOL>
__global__ __launch_bounds__(2 * kTsThreads, 1) void ts_load_probe256_kernel(TsProbeParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t w256[kTsStages][2 * kTsBV][kTsKT];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int ws = __builtin_amdgcn_readfirstlane(w);
  const int64_t V = p.V;
  const int H = p.H, nks = H / kTsKT;
  const int64_t vt0 = (int64_t)blockIdx.x * 2 * kTsBV;
  const int64_t wbytes = (V - vt0) * H * 2;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.W + vt0 * H), (short)0, (int)(wbytes < 0x7FFFFFFF ? wbytes : 0x7FFFFFFF), 0x00020000);
  const __amdgpu_buffer_rsrc_t ers = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.E, (short)0, (int)(uint32_t)(V * H * 2), 0x00020000);
  uint32_t woff[4], eoff[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t v = vt0 + 8 * (8 * i + w) + (l >> 3);
    woff[i] = (uint32_t)(((v < V ? v : V - 1) - vt0) * H * 2 + (((l & 7) ^ (l >> 3)) << 4));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
    eoff[i] = (uint32_t)p.ptok[32 * (w & 3) + 16 * (w >> 2) + 8 * i + (l >> 3)] * (uint32_t)H * 2u +
              (uint32_t)(((l & 7) ^ (l >> 3)) << 4);
  auto load_w = [&](int ks) {
    const int kc = ks < nks ? ks : nks - 1;
    const int st = ks % kTsStages;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (ts_lds_ptr)&w256[st][8 * (8 * i + ws)][0], 16,
                                               woff[i], kc * kTsKT * 2, 0, WPOL);
  };
  auto load_e = [&](u32x4 (&d)[2], int ks) {
    const int kc = ks < nks ? ks : nks - 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      d[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ers, (int)eoff[i], kc * kTsKT * 2, 0));
  };
  uint32_t acc = 0;
  auto step = [&](int ks, u32x4 (&ec)[2], u32x4 (&en)[2]) {
    __builtin_amdgcn_s_waitcnt(0x0F7A);  // vmcnt(10): W(ks) and E(ks) arrived
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    load_e(en, ks + 2);
    load_w(ks + 3);
    const uint32_t a = (uint32_t)(uintptr_t)(ts_lds_ptr)&w256[ks % kTsStages][l & 31][0] +
                       16u * (uint32_t)(l >> 5);
    u32x4 x;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(a));
    acc ^= x[0] ^ x[3] ^ ec[0][0] ^ ec[1][1];
  };
  asm volatile("" ::"v"(eoff[0]), "v"(eoff[1]));
  u32x4 e0[2] = {}, e1[2] = {}, e2[2] = {};
  load_w(0);
  asm volatile("" ::: "memory");
  load_e(e0, 0);
  asm volatile("" ::: "memory");
  load_w(1);
  asm volatile("" ::: "memory");
  load_e(e1, 1);
  asm volatile("" ::: "memory");
  load_w(2);
  int ks = 0;
  for (; ks + 3 <= nks; ks += 3) {
    step(ks, e0, e2);
    step(ks + 1, e1, e0);
    step(ks + 2, e2, e1);
  }
  if (ks < nks) step(ks, e0, e2);
  if (ks + 1 < nks) step(ks + 1, e1, e0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (acc == 0x9E3779B9u) p.sink[tid & 255] = acc;
}

// The 256-row loads again with persistent workgroups: G workgroups (one per
// CU), workgroup x streams tiles x, x + G, ... as one continuous step
// sequence (no workgroup start between its tiles; the embedding chunk of
// step g is chunk g mod H / 64 of every tile).
template <int WPOL>
__global__ __launch_bounds__(2 * kTsThreads, 1) void ts_load_probe256p_kernel(TsProbeParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t w256[kTsStages][2 * kTsBV][kTsKT];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int ws = __builtin_amdgcn_readfirstlane(w);
  const int64_t V = p.V;
  const int H = p.H, nks = H / kTsKT;
  const int G = gridDim.x;
  const int ntile = (int)((V + 2 * kTsBV - 1) / (2 * kTsBV));
  const int mytiles = ntile > (int)blockIdx.x ? (ntile - 1 - (int)blockIdx.x) / G + 1 : 0;
  const int nsteps = mytiles * nks;
  // one resource over all of W (byte offsets below 2^31); rows past V read zeros
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.W, (short)0, (int)(V * H * 2 < 0x7FFFFFFF ? V * H * 2 : 0x7FFFFFFF), 0x00020000);
  const __amdgpu_buffer_rsrc_t ers = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.E, (short)0, (int)(uint32_t)(V * H * 2), 0x00020000);
  uint32_t woff[4], eoff[2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    woff[i] = (uint32_t)((8 * (8 * i + w) + (l >> 3)) * H * 2 + (((l & 7) ^ (l >> 3)) << 4));
#pragma unroll
  for (int i = 0; i < 2; ++i)
    eoff[i] = (uint32_t)p.ptok[32 * (w & 3) + 16 * (w >> 2) + 8 * i + (l >> 3)] * (uint32_t)H * 2u +
              (uint32_t)(((l & 7) ^ (l >> 3)) << 4);
  // step g of this workgroup: tile blockIdx.x + (g / nks) G, chunk g % nks
  auto load_w = [&](int g) {
    const int gc = g < nsteps ? g : nsteps - 1;
    const int t = gc / nks, kc = gc - t * nks;
    const int64_t row0 = (int64_t)((int)blockIdx.x + t * G) * 2 * kTsBV;
    const int so = (int)(row0 * H * 2) + kc * kTsKT * 2;
    const int st = g % kTsStages;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (ts_lds_ptr)&w256[st][8 * (8 * i + ws)][0], 16,
                                               woff[i], so, 0, WPOL);
  };
  auto load_e = [&](u32x4 (&d)[2], int g) {
    const int gc = g < nsteps ? g : nsteps - 1;
    const int kc = gc % nks;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      d[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ers, (int)eoff[i], kc * kTsKT * 2, 0));
  };
  uint32_t acc = 0;
  auto step = [&](int g, u32x4 (&ec)[2], u32x4 (&en)[2]) {
    __builtin_amdgcn_s_waitcnt(0x0F7A);  // vmcnt(10)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    load_e(en, g + 2);
    load_w(g + 3);
    const uint32_t a = (uint32_t)(uintptr_t)(ts_lds_ptr)&w256[g % kTsStages][l & 31][0] +
                       16u * (uint32_t)(l >> 5);
    u32x4 x;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(a));
    acc ^= x[0] ^ x[3] ^ ec[0][0] ^ ec[1][1];
  };
  if (nsteps == 0) return;
  asm volatile("" ::"v"(eoff[0]), "v"(eoff[1]));
  u32x4 e0[2] = {}, e1[2] = {}, e2[2] = {};
  load_w(0);
  asm volatile("" ::: "memory");
  load_e(e0, 0);
  asm volatile("" ::: "memory");
  load_w(1);
  asm volatile("" ::: "memory");
  load_e(e1, 1);
  asm volatile("" ::: "memory");
  load_w(2);
  int g = 0;
  for (; g + 3 <= nsteps; g += 3) {
    step(g, e0, e2);
    step(g + 1, e1, e0);
    step(g + 2, e2, e1);
  }
  if (g < nsteps) step(g, e0, e2);
  if (g + 1 < nsteps) step(g + 1, e1, e0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (acc == 0x9E3779B9u) p.sink[tid & 255] = acc;
}

}  // namespace ddt
