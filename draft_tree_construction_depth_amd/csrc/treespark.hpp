// TreeSpark parent-conditioned tree expansion.
//
// TreeSpark README, item 1 ("Parent-Conditioned Tree Drafting from One
// Backbone Pass"): one backbone pass gives vocabulary logits l_d for every
// draft depth; a first-order Markov head specialises depth d to a parent
// token t_u, z_d(u) = l_d + W . e(t_u) with e(t) = E[t]; trees expand with
// branching factor k per parent, the frontier is pruned by joint path score
// and a global top-N packing keeps N non-root nodes (item 2 names the policy:
// per-parent top-k expansion, joint path-score frontier pruning, global
// top-N packing).
//
// Per depth d (all requests at once):
//  ts_gemm_kernel   Z[v, m] = sum_h W[v, h] E[t_m, h] for every vocabulary
//                   row v and every frontier parent m, on MFMA (bf16 in,
//                   float32 accumulate), with the epilogue fused: z = Z + l_d,
//                   then per parent column the tile's max, sum of exp and
//                   top-k -> one partial record per (128-row tile, parent).
//                   W (V x H bf16, 778 MB at the README shape) streams from
//                   HBM once per depth through an LDS ring; each wave takes
//                   32 parents' embedding rows straight into registers.
//  ts_merge_kernel  per request: each parent's log-sum-exp (float64) and
//                   top-k from the partials (the k best lie in the k tiles
//                   with the best tile maxima); children scored parent score
//                   + z - lse; the frontier for d+1 = the best F children.
// Then ts_pack_kernel ranks every candidate and keeps the best N.
// Order everywhere: score desc, then rank tuple lexicographic asc, the rank
// tuple held as 4-bit digits (j + 1) from the top of a 64-bit key so that a
// prefix precedes its extensions. Ties of z inside a parent: lower token id.
#pragma once

#include "common.hpp"

namespace ddt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTsThreads = 256;
constexpr int kTsBV = 128;     // W rows per workgroup (4 MFMA tiles of 32)
constexpr int kTsBM = 128;     // parent columns per workgroup (32 per wave)
constexpr int kTsKT = 64;      // reduction elements per step
constexpr int kTsKMax = 8;     // largest branching factor k
constexpr int kTsFMax = 8;     // largest frontier width F
constexpr int kTsDMax = 16;    // largest depth (4-bit digits in a 64-bit key)

struct TsGemmParams {
  const uint16_t* W;       // [V][H] bf16
  const uint16_t* E;       // [V][H] bf16
  const uint16_t* bb;      // [batch][D][V] bf16 backbone logits
  const int32_t* ptok;     // [M] parent tokens
  int64_t V;
  int32_t H, D, d;         // d: 0-based depth
  int32_t M, Fd, k;        // parents, parents per request, branching factor
  int32_t Mtot;            // parent slots of the partial records
  int32_t nvt;             // 128-row vocabulary tiles
  float* pmax;             // [Mtot][nvt] (parent-major: the merge reads a parent's tiles in a row)
  float* psum;             // [Mtot][nvt] sum of exp(z - pmax)
  float* pval;             // [Mtot][nvt][kTsKMax] top-k z, best first
  int32_t* pid;            // [Mtot][nvt][kTsKMax]
};

constexpr int kTsPad = 0x7FFFFFFF;  // id of an empty list slot (value -inf)

// (x, i) before (y, j) in the order value desc, id asc.
__device__ __forceinline__ bool ts_before(float x, int i, float y, int j) {
  return x > y || (x == y && i < j);
}

__device__ __forceinline__ void ts_cas(float& av, int& ai, float& bv, int& bi) {
  const bool sw = ts_before(bv, bi, av, ai);
  const float tv = av;
  const int ti = ai;
  av = sw ? bv : av;
  ai = sw ? bi : ai;
  bv = sw ? tv : bv;
  bi = sw ? ti : bi;
}

// Sort KK entries best first (odd-even transposition, KK rounds).
template <int KK>
__device__ __forceinline__ void ts_sort(float (&v)[KK], int (&id)[KK]) {
#pragma unroll
  for (int r = 0; r < KK; ++r)
#pragma unroll
    for (int i = r & 1; i + 1 < KK; i += 2) ts_cas(v[i], id[i], v[i + 1], id[i + 1]);
}

// Insert into a best-first list a value whose id exceeds every id in it (rows
// visited in increasing order, list already full of real entries): it
// precedes entry i exactly when its value is larger.
template <int KK>
__device__ __forceinline__ void ts_insert_inc(float (&val)[KK], int (&ids)[KK], float x, int id) {
  bool bt[KK];
#pragma unroll
  for (int i = 0; i < KK; ++i) bt[i] = x > val[i];
#pragma unroll
  for (int i = KK - 1; i >= 0; --i) {
    const bool shift = i > 0 && bt[i > 0 ? i - 1 : 0];
    const float pv = i > 0 ? val[i > 0 ? i - 1 : 0] : x;
    const int pi = i > 0 ? ids[i > 0 ? i - 1 : 0] : id;
    val[i] = shift ? pv : (bt[i] ? x : val[i]);
    ids[i] = shift ? pi : (bt[i] ? id : ids[i]);
  }
}

// Best KK of two best-first lists: a[i] vs b[KK-1-i] keeps the best KK as a
// bitonic sequence, then log2(KK) half-cleaner stages sort it.
template <int KK>
__device__ __forceinline__ void ts_merge_sorted(float (&av)[KK], int (&ai)[KK], const float (&bv)[KK],
                                                const int (&bi)[KK]) {
#pragma unroll
  for (int i = 0; i < KK; ++i) {
    const bool t = ts_before(bv[KK - 1 - i], bi[KK - 1 - i], av[i], ai[i]);
    av[i] = t ? bv[KK - 1 - i] : av[i];
    ai[i] = t ? bi[KK - 1 - i] : ai[i];
  }
#pragma unroll
  for (int d = KK / 2; d > 0; d >>= 1)
#pragma unroll
    for (int i = 0; i < KK; ++i)
      if ((i & d) == 0) ts_cas(av[i], ai[i], av[i + d], ai[i + d]);
}

// ---------------------------------------------------------------------------
// GEMM schedule: the head weight W streams into an LDS ring by direct
// buffer-to-LDS loads, each wave instruction reading eight whole 128-byte row
// segments, three k-steps ahead; the parents' embedding chunks come from the
// L2 into registers two steps ahead, also as whole 128-byte segments (eight
// parents per instruction: an instruction in the MFMA B layout would touch 32
// lines for 32 bytes each, which costs the stream about a third of its rate),
// and each wave re-lays its own chunk in MFMA order through a private LDS
// slot at the step that uses it. Wave w owns parent columns [32 w, 32 w + 32)
// against all 128 vocabulary rows of the tile, so each parent's partial
// record comes out of one wave, with no cross-wave combine.
constexpr int kTsStages = 4;  // W ring depth (16 KiB per stage)
// W is read once per launch: its loads carry the nontemporal hint, so that
// they do not push the parents' embedding rows and the partial records (read
// by the merge next) out of the caches
constexpr int kTsLoadNT = 2;

// LDS row r, 16-byte chunk c holds W chunk c ^ (r & 7) of that row's step
// segment, so that a fragment read of 32 consecutive rows spreads over all
// banks; each wave's embedding slot holds its 32 parents' step segments the
// same way (80 KiB in all: two workgroups per CU).
struct alignas(16) TsGemmSmem {
  uint16_t w[kTsStages][kTsBV][kTsKT];
  uint16_t e[kTsThreads / kWave][32][kTsKT];
};

typedef __attribute__((address_space(3))) void* ts_lds_ptr;

template <int KK>
__global__ __launch_bounds__(kTsThreads, 2) void ts_gemm_kernel(TsGemmParams p) {
  __shared__ TsGemmSmem sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int vt = blockIdx.x;
  const int m0 = blockIdx.y * kTsBM;
  const int H = p.H;
  const int64_t V = p.V;
  const int ncols = p.M - m0 < kTsBM ? p.M - m0 : kTsBM;
  const bool active = 32 * w < ncols;  // wave-uniform: this wave has parents
  const int ws = __builtin_amdgcn_readfirstlane(w);  // the wave index in a scalar register
  const int64_t vt0 = (int64_t)vt * kTsBV;
  const int nks = H / kTsKT;

  // W loads: instruction i of wave w covers tile rows 8 g .. 8 g + 7, g = 4 i
  // + w; lane l takes row 8 g + l / 8 and chunk (l % 8) ^ (l / 8) of it, and
  // lands at LDS chunk l % 8 of that row (the instruction writes 64
  // consecutive 16-byte slots). Rows past V read row V - 1 (masked later).
  // (buffer loads over this tile's rows: a fixed per-lane byte offset and the
  // step's offset in a scalar, so no per-step vector address temporaries)
  const int64_t wbytes = (V - vt0) * H * 2;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.W + vt0 * H), (short)0, (int)(wbytes < 0x7FFFFFFF ? wbytes : 0x7FFFFFFF), 0x00020000);
  uint32_t woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t v = vt0 + 8 * (4 * i + w) + (l >> 3);
    woff[i] = (uint32_t)(((v < V ? v : V - 1) - vt0) * H * 2 + (((l & 7) ^ (l >> 3)) << 4));
  }
  // E: instruction i of wave w reads the step segments of its parents
  // 8 i .. 8 i + 7 (column 32 w + j, clamped to the last parent; masked
  // later); lane l takes parent 8 i + l / 8, chunk (l % 8) ^ (l / 8), so that
  // the lane-ordered write of the four registers into the wave's slot lands
  // in the swizzled layout. A buffer resource over the table (byte offsets
  // are unsigned 32-bit: the host rejects tables of 4 GiB or more; a token
  // past the table reads zeros).
  const __amdgpu_buffer_rsrc_t ers = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.E, (short)0, (int)(uint32_t)(V * H * 2), 0x00020000);
  uint32_t eoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int pcol = m0 + 32 * w + 8 * i + (l >> 3);
    pcol = pcol < p.M ? pcol : p.M - 1;
    eoff[i] = (uint32_t)p.ptok[pcol] * (uint32_t)H * 2u + (uint32_t)(((l & 7) ^ (l >> 3)) << 4);
  }

  // W loads always issue, so that the wait counts stay static; past the last
  // step they read the last embedding chunk, which the L2 holds, instead of
  // W lines from HBM again. One code path for both, the source selected by
  // value: a branch here makes the compiler add waits of its own in every
  // step. E past the last step re-reads the last chunk.
  auto load_w = [&](int ks) {
    const int st = ks % kTsStages;
    const bool past = ks >= nks;
    const __amdgpu_buffer_rsrc_t rs = past ? ers : wrs;
    const int so = (past ? nks - 1 : ks) * kTsKT * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (ts_lds_ptr)&sm.w[st][8 * (4 * i + ws)][0], 16,
                                               past ? eoff[i] : woff[i], so, 0, kTsLoadNT);
  };
  auto load_e = [&](u32x4 (&dst)[4], int ks) {
    const int kc = ks < nks ? ks : nks - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             ers, (int)eoff[i], kc * kTsKT * 2, 0));
  };

  // LDS byte address, in stage 0, of this lane's A fragment for MFMA step s
  // of vocabulary tile 0 (tile m adds m * 4096): row l % 32, chunk 2 s + l / 32
  // swizzled by the row's low three bits (row & 7 == l & 7)
  const uint32_t wbase = (uint32_t)(uintptr_t)(ts_lds_ptr)&sm.w[0][0][0];
  uint32_t fa[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    fa[s] = wbase + (uint32_t)((l & 31) * kTsKT * 2) + (uint32_t)(((2 * s + (l >> 5)) ^ (l & 7)) * 16);
  // the wave's embedding slot: lane l writes bytes 16 l (+ 1 KiB per
  // register) and reads its B fragment for MFMA step s, parent column l % 32
  // and chunk 2 s + l / 32, from the same swizzled place as A's
  const uint32_t ebase = (uint32_t)(uintptr_t)(ts_lds_ptr)&sm.e[ws][0][0];
  const uint32_t ewr = ebase + 16u * (uint32_t)l;
  uint32_t erd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) erd[s] = fa[s] - wbase + ebase;

  f32x16 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.0f;

  // Step ks: wait for this thread's loads of W(ks) and E(ks) (the twelve
  // memory instructions issued since, W(ks + 1), E(ks + 1) and W(ks + 2), may
  // stay in flight: E goes out before W in each step, so waiting for E(ks)
  // does not also wait for W(ks + 1)), barrier (every wave's W(ks) is in
  // LDS, and every wave is done with the stage W(ks + 3) will overwrite),
  // issue E(ks + 2) and W(ks + 3),
  // in one asm block that waits for its LDS operations (the compiler would
  // wait for every direct-to-LDS load in flight before an LDS access it can
  // see): write E(ks) into the wave's slot, read the step's 4 B and 16 A
  // fragments (a wave's LDS operations take effect in order), then the 16
  // MFMAs.
  auto step = [&](int ks, u32x4 (&ec)[4], u32x4 (&en)[4]) {
    // the wait as a builtin, so that the compiler knows E(ks) has arrived and
    // adds no wait of its own before the MFMAs
    __builtin_amdgcn_s_waitcnt(0x0F7C);  // vmcnt(12), expcnt and lgkmcnt unrestricted
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no memory access moves across the barrier
    load_e(en, ks + 2);
    load_w(ks + 3);
    if (active) {
      const uint32_t sa = (uint32_t)(ks % kTsStages) * (uint32_t)sizeof(sm.w[0]);
      u32x4 a[4][4], bf[4];
      asm volatile(
          "ds_write_b128 %24, %25\n\t"
          "ds_write_b128 %24, %26 offset:1024\n\t"
          "ds_write_b128 %24, %27 offset:2048\n\t"
          "ds_write_b128 %24, %28 offset:3072\n\t"
          "ds_read_b128 %16, %29\n\t"
          "ds_read_b128 %17, %30\n\t"
          "ds_read_b128 %18, %31\n\t"
          "ds_read_b128 %19, %32\n\t"
          "ds_read_b128 %0, %20\n\t"
          "ds_read_b128 %1, %20 offset:4096\n\t"
          "ds_read_b128 %2, %20 offset:8192\n\t"
          "ds_read_b128 %3, %20 offset:12288\n\t"
          "ds_read_b128 %4, %21\n\t"
          "ds_read_b128 %5, %21 offset:4096\n\t"
          "ds_read_b128 %6, %21 offset:8192\n\t"
          "ds_read_b128 %7, %21 offset:12288\n\t"
          "ds_read_b128 %8, %22\n\t"
          "ds_read_b128 %9, %22 offset:4096\n\t"
          "ds_read_b128 %10, %22 offset:8192\n\t"
          "ds_read_b128 %11, %22 offset:12288\n\t"
          "ds_read_b128 %12, %23\n\t"
          "ds_read_b128 %13, %23 offset:4096\n\t"
          "ds_read_b128 %14, %23 offset:8192\n\t"
          "ds_read_b128 %15, %23 offset:12288\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(a[0][0]), "=&v"(a[1][0]), "=&v"(a[2][0]), "=&v"(a[3][0]),
            "=&v"(a[0][1]), "=&v"(a[1][1]), "=&v"(a[2][1]), "=&v"(a[3][1]),
            "=&v"(a[0][2]), "=&v"(a[1][2]), "=&v"(a[2][2]), "=&v"(a[3][2]),
            "=&v"(a[0][3]), "=&v"(a[1][3]), "=&v"(a[2][3]), "=&v"(a[3][3]),
            "=&v"(bf[0]), "=&v"(bf[1]), "=&v"(bf[2]), "=&v"(bf[3])
          : "v"(fa[0] + sa), "v"(fa[1] + sa), "v"(fa[2] + sa), "v"(fa[3] + sa), "v"(ewr),
            "v"(ec[0]), "v"(ec[1]), "v"(ec[2]), "v"(ec[3]), "v"(erd[0]), "v"(erd[1]), "v"(erd[2]),
            "v"(erd[3]));
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a[m][s]), __builtin_bit_cast(bf16x8, bf[s]), acc[m], 0, 0,
              0);
    } else {
      // consume E(ks) here too, so that on both paths its registers are known
      // to have arrived before the next loads reuse them (else the compiler
      // drains every load in flight at the loop's back edge)
      asm volatile("" ::"v"(ec[0]), "v"(ec[1]), "v"(ec[2]), "v"(ec[3]));
    }
  };

  // The prologue issues W(0), E(0), W(1), E(1), W(2) in that order, with the
  // parents' tokens read first: the step's vmcnt(12) relies on it, and a
  // prologue reordered by the compiler (E after every W, behind a wait for
  // the token loads) makes it add waits of its own inside the loop that
  // drain the W look-ahead.
  asm volatile("" ::"v"(eoff[0]), "v"(eoff[1]), "v"(eoff[2]), "v"(eoff[3]));
  u32x4 e0[4], e1[4], e2[4];
  load_w(0);
  asm volatile("" ::: "memory");
  load_e(e0, 0);
  asm volatile("" ::: "memory");
  load_w(1);
  asm volatile("" ::: "memory");
  load_e(e1, 1);
  asm volatile("" ::: "memory");
  load_w(2);
  // whole rotations in the loop, the one or two remaining steps after it (an
  // exit between the steps of a rotation also makes the compiler add waits
  // that drain the look-ahead)
  int ks = 0;
  for (; ks + 3 <= nks; ks += 3) {
    step(ks, e0, e2);
    step(ks + 1, e1, e0);
    step(ks + 2, e2, e1);
  }
  if (ks < nks) step(ks, e0, e2);
  if (ks + 1 < nks) step(ks + 1, e1, e0);
  // drain the look-ahead loads (they target LDS this workgroup owns)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (!active) return;

  // ---- epilogue: z = Z + l_d; per parent column the tile's max, exp sum and
  // top-k. acc[m][r] holds vocabulary row 32 m + 8 (r / 4) + 4 (l / 32) + r % 4
  // of the tile and parent column 32 w + l % 32; lanes l and l ^ 32 share a
  // column. Rows visited in (m, r) order increase.
  const int col = 32 * w + (l & 31);
  const bool colok = col < ncols;
  const int m = m0 + (colok ? col : 0);
  const int req = m / p.Fd;
  // the backbone row of the parent's request; rows past V read row V - 1,
  // and the logit is added after the mask (-inf plus a finite logit) so that
  // every load is used and all 64 issue unconditionally, back to back
  const uint16_t* lrow = p.bb + ((int64_t)req * p.D + p.d) * V;
  // all 64 logits in flight at once: each group of four consecutive rows
  // (r % 4) is one 8-byte load when the tile lies inside the vocabulary and
  // V is a multiple of 4 (so the row starts 8-byte aligned), else one load
  // per row
  uint32_t lq[16][2];
  if (vt0 + kTsBV <= V && (V & 3) == 0) {
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const int64_t v = vt0 + 32 * (g >> 2) + 8 * (g & 3) + 4 * (l >> 5);
      const uint2 q = *reinterpret_cast<const uint2*>(lrow + v);
      lq[g][0] = q.x;
      lq[g][1] = q.y;
    }
  } else {
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const int64_t v = vt0 + 32 * (g >> 2) + 8 * (g & 3) + 4 * (l >> 5);
      uint32_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = lrow[v + e < V ? v + e : V - 1];
      lq[g][0] = h[0] | (h[1] << 16);
      lq[g][1] = h[2] | (h[3] << 16);
    }
  }
  float z[64];
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t v = vt0 + 32 * t + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
      const uint32_t pr = lq[4 * t + (r >> 2)][(r >> 1) & 1];
      const float lv = __uint_as_float((r & 1) ? (pr & 0xFFFF0000u) : (pr << 16));
      z[16 * t + r] = (v < V ? acc[t][r] : -INFINITY) + lv;
      mx = fmaxf(mx, z[16 * t + r]);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float sacc = 0.0f;
#pragma unroll
  for (int q = 0; q < 64; ++q) sacc += z[q] == -INFINITY ? 0.0f : __expf(z[q] - mx);
  sacc += __shfl_xor(sacc, 32);
  float tv[KK];
  int ti[KK];
#pragma unroll
  for (int q = 0; q < KK; ++q) {
    const int64_t v = vt0 + 32 * (q >> 4) + 8 * ((q & 15) >> 2) + 4 * (l >> 5) + (q & 3);
    tv[q] = z[q];
    ti[q] = v < V ? (int)v : kTsPad;
  }
  ts_sort<KK>(tv, ti);
#pragma unroll
  for (int q = KK; q < 64; ++q) {
    const int64_t v = vt0 + 32 * (q >> 4) + 8 * ((q & 15) >> 2) + 4 * (l >> 5) + (q & 3);
    if (v < V) ts_insert_inc<KK>(tv, ti, z[q], (int)v);
  }
  float ov[KK];
  int oi[KK];
#pragma unroll
  for (int i = 0; i < KK; ++i) {
    ov[i] = __shfl_xor(tv[i], 32);
    oi[i] = __shfl_xor(ti[i], 32);
  }
  ts_merge_sorted<KK>(tv, ti, ov, oi);
  if (l < 32 && colok) {
    const size_t o = (size_t)(m0 + col) * p.nvt + vt;
    p.pmax[o] = mx;
    p.psum[o] = sacc;
#pragma unroll
    for (int i = 0; i < KK; ++i) {
      p.pval[o * kTsKMax + i] = tv[i];
      p.pid[o * kTsKMax + i] = ti[i];
    }
  }
}

// ---------------------------------------------------------------------------
// Candidate store and per-depth parent lists (workspace).
struct TsState {
  int32_t* ctok;    // [batch][cmax] candidate tokens
  double* cscore;   // [batch][cmax] path scores
  uint64_t* ckey;   // [batch][cmax] rank-tuple keys
  int32_t* cpar;    // [batch][cmax] parent candidate (-1: the anchor)
  int32_t* cdep;    // [batch][cmax] depth (1-based)
  int32_t* ccount;  // [batch] (written from depth 0 on; depth 0 reads none)
  int32_t* fcount;  // [batch] parents of the current depth (likewise)
  int32_t* ptok[2];   // [batch * F] parent tokens, by depth parity (depth 0: the anchors)
  int32_t* pcand[2];  // [batch * F] parent candidate index (-1: anchor)
  int32_t cmax;
};

struct TsMergeParams {
  TsState st;
  const float* pmax;
  const float* psum;
  const float* pval;
  const int32_t* pid;
  int32_t nvt, Mtot;
  int32_t d, D;       // 0-based depth, depths
  int32_t Fd, Fn;     // parents per request at this depth / the next
  int32_t k, F;
  int32_t base;       // candidates per request before this depth
};

__device__ __forceinline__ uint64_t ts_zkey(float x, int id) {
  return ((uint64_t)order_key(__float_as_uint(x)) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id);
}

// One 1024-thread workgroup per request; the four waves of group g merge
// parents g, g + 4, ...: one pass over the tiles' maxima, exp sums (float32
// terms, float64 totals, rescaled to the running maximum) and best entries,
// which names the k tiles that hold the parent's k best children; only those
// tiles' lists are then read. Groups combine through LDS.
constexpr int kTsMergeThreads = 1024;
constexpr int kTsMergeGroups = 4;
constexpr int kTsGroupWaves = kTsMergeThreads / kWave / kTsMergeGroups;

template <int KK>
__global__ __launch_bounds__(kTsMergeThreads) void ts_merge_kernel(TsMergeParams p) {
  __shared__ int32_t ch_tok[kTsFMax * kTsKMax];
  __shared__ double ch_score[kTsFMax * kTsKMax];
  __shared__ uint64_t ch_key[kTsFMax * kTsKMax];
  __shared__ int32_t ch_cand[kTsFMax * kTsKMax];
  __shared__ double red_d[kTsMergeGroups][kTsGroupWaves];
  __shared__ float red_m[kTsMergeGroups][kTsGroupWaves];
  __shared__ uint64_t red_k[kTsMergeGroups][kTsGroupWaves][KK];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = w / kTsGroupWaves, gw = w - g * kTsGroupWaves;
  const int gt = gw * kWave + lane;  // thread index within the group
  constexpr int GT = kTsGroupWaves * kWave;
  const int64_t b = blockIdx.x;
  TsState& st = p.st;
  const int par = p.d & 1;
  // parents and earlier candidates per request are the same for every
  // request (each parent has exactly k children): taken from the host, so
  // that the record loads need not wait for a load of them
  const int nf = p.Fd;
  const int K = p.k;
  const int base = p.base;
  const int shift = 4 * (kTsDMax - 1 - p.d);  // this depth's digit
  const int rounds = (nf + kTsMergeGroups - 1) / kTsMergeGroups;
  for (int rd = 0; rd < rounds; ++rd) {  // uniform trip count: every group reaches each barrier
    const int i = rd * kTsMergeGroups + g;
    const bool act = i < nf;
    const int m = (int)b * p.Fd + (act ? i : 0);
    // the parent's candidate index (-1: the anchor), read now so that its
    // score and key can be read while the tiles' records are reduced
    const int pc = (p.d == 0 || !act) ? -1 : st.pcand[par][m];
    // One pass over the parent's tiles: each thread loads, for a batch of its
    // tiles at once (consecutive in memory for consecutive threads), the
    // tile's maximum, exp sum and best entry, and keeps its own maximum, its
    // exp sum relative to that and its KK best tile-best keys. The parent's k
    // best entries all lie in the k tiles with the best tile-best keys (any
    // tile holding one of them has a best key at least the k-th best overall,
    // which is at least the k-th best of those k distinct tile bests), so only
    // those tiles' lists are read afterwards.
    constexpr int TB = 8;  // tiles per thread per batch
    const size_t pb = (size_t)m * p.nvt;
    float mx = -INFINITY;
    double s = 0.0;
    uint64_t tk[KK];  // this thread's best tile keys, best first (0 = none)
#pragma unroll
    for (int j = 0; j < KK; ++j) tk[j] = 0;
    for (int t0 = 0; t0 < p.nvt; t0 += TB * GT) {
      float bx[TB], by[TB], bv[TB];
      int bi[TB];
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const int t = t0 + u * GT + gt;
        const bool ok = t < p.nvt;
        const size_t o = pb + (ok ? t : 0);
        bx[u] = ok ? p.pmax[o] : -INFINITY;
        by[u] = ok ? p.psum[o] : 0.0f;
        bv[u] = ok ? p.pval[o * kTsKMax] : -INFINITY;
        bi[u] = ok ? p.pid[o * kTsKMax] : 0x7FFFFFFF;
      }
      float bm = mx;
#pragma unroll
      for (int u = 0; u < TB; ++u) bm = fmaxf(bm, bx[u]);
      if (bm != -INFINITY) {
        if (mx != -INFINITY && bm != mx) s *= (double)__expf(mx - bm);
#pragma unroll
        for (int u = 0; u < TB; ++u)
          if (bx[u] != -INFINITY) s += (double)(by[u] * __expf(bx[u] - bm));
        mx = bm;
      }
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        // the tile's best key into the sorted list (keys are unique)
        const uint64_t x = bi[u] != 0x7FFFFFFF ? ts_zkey(bv[u], bi[u]) : 0ull;
#pragma unroll
        for (int q = KK - 1; q >= 0; --q) {
          const bool above = q > 0 && x > tk[q > 0 ? q - 1 : 0];
          tk[q] = above ? tk[q > 0 ? q - 1 : 0] : (x > tk[q] ? x : tk[q]);
        }
      }
    }
    const double pscore = pc < 0 ? 0.0 : st.cscore[b * st.cmax + pc];
    const uint64_t pkey = pc < 0 ? 0ull : st.ckey[b * st.cmax + pc];
    // the group's maximum, then every thread's sum rescaled to it
    const float wm = wave_max(mx);
    if (lane == 0) red_m[g][gw] = wm;
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kTsGroupWaves; ++q) M = fmaxf(M, red_m[g][q]);
    if (mx != -INFINITY) s *= (double)__expf(mx - M);
    s = wave_sum(s);
    // the wave's KK best tile keys: KK rounds of a max over each lane's best
    // untaken key
    int head = 0;
    uint64_t wbest[KK];
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      uint64_t mine = 0;
#pragma unroll
      for (int j = 0; j < KK; ++j)
        if (j == head) mine = tk[j];
      const uint64_t best = wave_max(mine);
      if (mine == best && best != 0) ++head;
      wbest[r] = best;
    }
    if (lane == 0) {
      red_d[g][gw] = s;
#pragma unroll
      for (int r = 0; r < KK; ++r) red_k[g][gw][r] = wbest[r];
    }
    __syncthreads();
    if (act && gw == 0) {
      // lane r < K takes the r-th best tile of the group (keys unique)
      uint64_t tile_key = 0;
      if (lane < K) {
        uint64_t all[kTsGroupWaves * KK];
#pragma unroll
        for (int q = 0; q < kTsGroupWaves; ++q)
#pragma unroll
          for (int r = 0; r < KK; ++r) all[q * KK + r] = red_k[g][q][r];
        for (int r = 0; r <= lane; ++r) {
          uint64_t bst = 0;
#pragma unroll
          for (int q = 0; q < kTsGroupWaves * KK; ++q) {
            const uint64_t x = all[q];
            if (x > bst && (r == 0 || x < tile_key)) bst = x;
          }
          tile_key = bst;
        }
      }
      // lane q < K * K reads entry q % K of the (q / K)-th best tile's list;
      // then K rounds of a wave maximum give the parent's k best, lane r
      // keeping the r-th
      uint64_t cand = 0;
      {
        const int r = lane / K, j = lane - r * K;
        const uint64_t tkr = (uint64_t)(uint32_t)__shfl((int)(tile_key >> 32), r) << 32 |
                             (uint32_t)__shfl((int)(uint32_t)tile_key, r);
        if (lane < K * K && tkr != 0) {
          const int tile = (int)((0xFFFFFFFFu - (uint32_t)tkr) / (uint32_t)kTsBV);
          const size_t o = pb + tile;
          const int id = p.pid[o * kTsKMax + j];
          if (id != 0x7FFFFFFF) cand = ts_zkey(p.pval[o * kTsKMax + j], id);
        }
      }
      uint64_t pick = 0;
      for (int r = 0; r < K; ++r) {
        const uint64_t best = wave_max(cand);
        if (cand == best) cand = 0;
        if (lane == r) pick = best;
      }
      double tot = 0.0;
#pragma unroll
      for (int q = 0; q < kTsGroupWaves; ++q) tot += red_d[g][q];
      const double lse = (double)M + log(tot);
      if (lane < K) {
        const int c = i * K + lane;
        ch_tok[c] = (int32_t)(0xFFFFFFFFu - (uint32_t)pick);
        ch_score[c] = pscore + ((double)key_value((uint32_t)(pick >> 32)) - lse);
        ch_key[c] = pkey | ((uint64_t)(lane + 1) << shift);
        ch_cand[c] = pc;
      }
    }
    __syncthreads();
  }
  // append the children; the frontier for the next depth = the best F of them
  const int nch = nf * K;
  if (tid < nch) {
    const size_t o = (size_t)b * st.cmax + base + tid;
    st.ctok[o] = ch_tok[tid];
    st.cscore[o] = ch_score[tid];
    st.ckey[o] = ch_key[tid];
    st.cpar[o] = ch_cand[tid];
    st.cdep[o] = p.d + 1;
    if (p.d + 1 < p.D) {
      int rank = 0;
      for (int j = 0; j < nch; ++j) {
        const bool before = ch_score[j] > ch_score[tid] ||
                            (ch_score[j] == ch_score[tid] && ch_key[j] < ch_key[tid]);
        rank += before ? 1 : 0;
      }
      if (rank < p.F) {
        st.ptok[par ^ 1][(size_t)b * p.Fn + rank] = ch_tok[tid];
        st.pcand[par ^ 1][(size_t)b * p.Fn + rank] = base + tid;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    st.ccount[b] = base + nch;
    st.fcount[b] = nch < p.F ? nch : p.F;
  }
}

struct TsPackParams {
  TsState st;
  int32_t N;
  int32_t* tree_tokens;  // [batch][N]
  int32_t* parents;
  float* logq;
  int32_t* depths;
  int32_t* num_nodes;
};

// Global top-N packing: each candidate's rank is the number of candidates
// before it; the best N take positions 1..N (0 = the anchor).
__global__ __launch_bounds__(kTsThreads) void ts_pack_kernel(TsPackParams p) {
  const int64_t b = blockIdx.x;
  const TsState& st = p.st;
  const int n = st.ccount[b];
  const size_t cb = (size_t)b * st.cmax;
  const int N = p.N;
  const int nsel = n < N ? n : N;
  extern __shared__ int32_t rank_s[];  // [cmax]
  for (int i = threadIdx.x; i < n; i += kTsThreads) {
    const double si = st.cscore[cb + i];
    const uint64_t ki = st.ckey[cb + i];
    int r = 0;
    for (int j = 0; j < n; ++j) {
      const double sj = st.cscore[cb + j];
      r += (sj > si || (sj == si && st.ckey[cb + j] < ki)) ? 1 : 0;
    }
    rank_s[i] = r;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kTsThreads) {
    const int r = rank_s[i];
    if (r < nsel) {
      const size_t o = (size_t)b * N + r;
      const int pc = st.cpar[cb + i];
      p.tree_tokens[o] = st.ctok[cb + i];
      p.parents[o] = pc < 0 ? 0 : rank_s[pc] + 1;
      p.logq[o] = (float)st.cscore[cb + i];
      if (p.depths) p.depths[o] = st.cdep[cb + i];
    }
  }
  for (int j = nsel + threadIdx.x; j < N; j += kTsThreads) {
    const size_t o = (size_t)b * N + j;
    p.tree_tokens[o] = -1;
    p.parents[o] = -1;
    p.logq[o] = -INFINITY;
    if (p.depths) p.depths[o] = 0;
  }
  if (threadIdx.x == 0) p.num_nodes[b] = nsel;
}

}  // namespace ddt
