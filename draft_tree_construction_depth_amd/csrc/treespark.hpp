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
//                   HBM once per depth; the parents' embedding rows are
//                   shared by the four waves through LDS.
//  ts_merge_kernel  per request: each parent's log-sum-exp (float64) and
//                   top-k from the partials; children scored parent score +
//                   z - lse; the frontier for d+1 = the best F children.
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
constexpr int kTsBV = 128;     // W rows per workgroup (4 waves x 32)
constexpr int kTsBM = 128;     // parent columns per workgroup (4 MFMA tiles of 32)
constexpr int kTsKT = 64;      // reduction elements per step
constexpr int kTsGPad = 8;     // LDS row padding (bf16) against bank conflicts
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
  int32_t Mtot;            // column stride of the partial records
  float* pmax;             // [nvt][Mtot]
  float* psum;             // [nvt][Mtot] sum of exp(z - pmax)
  float* pval;             // [nvt][Mtot][kTsKMax] top-k z, best first
  int32_t* pid;            // [nvt][Mtot][kTsKMax]
};

// 16-byte aligned so that the fragment reads and the staging stores are
// single 16-byte LDS instructions.
struct alignas(16) TsGemmSmem {
  union {
    uint16_t g[2][kTsBM][kTsKT + kTsGPad];  // parents' embedding rows, double buffered
    struct {
      float mx[4][kTsBM];
      float sm[4][kTsBM];
      float val[4][kTsBM][kTsKMax];
      int id[4][kTsBM][kTsKMax];
    } red;  // per-wave partials of the epilogue
  };
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

template <int KK>
__global__ __launch_bounds__(kTsThreads) void ts_gemm_kernel(TsGemmParams p) {
  __shared__ TsGemmSmem sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int vt = blockIdx.x;
  const int m0 = blockIdx.y * kTsBM;
  const int H = p.H;
  const int64_t V = p.V;
  const int ncols = p.M - m0 < kTsBM ? p.M - m0 : kTsBM;
  const int nct = (ncols + 31) >> 5;  // MFMA column tiles in use

  // W through a buffer resource over this workgroup's rows: the lane's byte
  // offset is fixed, the k-step's goes in a scalar, so no address arithmetic
  // per step (A operand: row l % 32 of the wave's 32 rows; rows past V read
  // row V-1 and are masked later)
  const int64_t vt0 = (int64_t)vt * kTsBV;
  const int64_t vrow = vt0 + w * 32 + (l & 31);
  const int64_t vload = vrow < V ? vrow : V - 1;
  const int64_t wbytes = (V - vt0) * H * 2;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.W + vt0 * H), (short)0, (int)(wbytes < 0x7FFFFFFF ? wbytes : 0x7FFFFFFF), 0x00020000);
  const uint32_t woff = (uint32_t)((vload - vt0) * H * 2 + 16 * (l >> 5));  // < V * H * 2 < 2^32

  // embedding-row staging: thread t copies 16-byte chunk (t % 8) of rows t/8 + 32 i
  const int gch = tid & 7, grow0 = tid >> 3;
  // E as one buffer resource: byte offsets are unsigned 32-bit (the host
  // rejects tables of 4 GiB or more)
  const uint32_t ebytes = (uint32_t)(V * H * 2);
  const __amdgpu_buffer_rsrc_t ers =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.E, (short)0, (int)ebytes, 0x00020000);
  uint32_t eoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = grow0 + 32 * i;
    const int m = m0 + (r < ncols ? r : 0);
    eoff[i] = (uint32_t)p.ptok[m] * (uint32_t)H * 2u + 16u * (uint32_t)gch;
  }

  const int nks = H / kTsKT;
  u32x4 wx0[4], wx1[4], wx2[4], gy0[4], gy1[4];
  auto load_w = [&](u32x4 (&dst)[4], int ks) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      dst[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             wrs, (int)woff, ks * kTsKT * 2 + 32 * s, 0));
  };
  auto load_g = [&](u32x4 (&dst)[4], int ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dst[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ers, (int)eoff[i], ks * kTsKT * 2, 0));
  };
  auto store_g = [&](const u32x4 (&src)[4], int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)&sm.g[buf][grow0 + 32 * i][8 * gch] = src[i];
  };
  // Workgroup barrier for the LDS double buffer only: waits for this wave's
  // LDS traffic, not for its global loads in flight (a full __syncthreads
  // fence would drain them and undo the prefetch).
  auto lds_barrier = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;

  // Step ks multiplies W(ks) with the parents' chunk in LDS buffer ks & 1,
  // issues the loads of W(ks+2) and of the parents' chunk ks+2, and stores
  // chunk ks+1 (loaded during step ks-1) into the other buffer: two steps of
  // latency hidden for both streams. Three W and two chunk register sets
  // rotate by name (six steps unrolled), so no copy waits on a load.
  auto step = [&](int ks, u32x4 (&wu)[4], u32x4 (&wl)[4], u32x4 (&gs)[4], u32x4 (&gl)[4]) {
    const int buf = ks & 1;
    const int kn = ks + 2 < nks ? ks + 2 : nks - 1;  // always issue, so wait counts stay static
    load_w(wl, kn);
    load_g(gl, kn);
    // every B fragment of the step read before the first MFMA, so that the
    // LDS latency is paid once per step, not once per MFMA
    u32x4 braw[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (c < nct)
          braw[s][c] = *(const u32x4*)&sm.g[buf][c * 32 + (l & 31)][16 * s + 8 * (l >> 5)];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, wu[s]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c < nct)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              a, __builtin_bit_cast(bf16x8, braw[s][c]), acc[c], 0, 0, 0);
      }
    }
    if (ks + 1 < nks) store_g(gs, buf ^ 1);
    lds_barrier();
  };

  load_w(wx0, 0);
  load_w(wx1, nks > 1 ? 1 : 0);
  load_g(gy0, 0);
  load_g(gy1, nks > 1 ? 1 : 0);
  store_g(gy0, 0);
  lds_barrier();
  for (int ks = 0; ks < nks; ks += 6) {
    step(ks, wx0, wx2, gy1, gy0);
    if (ks + 1 >= nks) break;
    step(ks + 1, wx1, wx0, gy0, gy1);
    if (ks + 2 >= nks) break;
    step(ks + 2, wx2, wx1, gy1, gy0);
    if (ks + 3 >= nks) break;
    step(ks + 3, wx0, wx2, gy0, gy1);
    if (ks + 4 >= nks) break;
    step(ks + 4, wx1, wx0, gy1, gy0);
    if (ks + 5 >= nks) break;
    step(ks + 5, wx2, wx1, gy0, gy1);
  }
  __syncthreads();

  // ---- epilogue: z = Z + l_d; per column the wave's max, exp sum and top-k
  // acc[c][r] holds row 8 (r / 4) + 4 (l / 32) + r % 4 of the wave's 32 rows,
  // column c * 32 + l % 32; lanes l and l ^ 32 share a column.
  const int64_t vbase = (int64_t)vt * kTsBV + w * 32;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (c >= nct) continue;
    const int col = c * 32 + (l & 31);
    const bool colok = col < ncols;
    const int m = m0 + (colok ? col : 0);
    const int req = m / p.Fd;
    const uint16_t* lrow = p.bb + ((int64_t)req * p.D + p.d) * V;
    float z[16];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t v = vbase + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
      const bool ok = v < V;
      const float lv = __uint_as_float((uint32_t)lrow[ok ? v : V - 1] << 16);  // in-bounds read
      z[r] = ok ? acc[c][r] + lv : -INFINITY;
      mx = fmaxf(mx, z[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += z[r] == -INFINITY ? 0.0f : __expf(z[r] - mx);
    s += __shfl_xor(s, 32);
    // the lane's best KK of its 16 rows (ids increase with r): the first KK
    // sorted, the rest inserted; rows past V are empty slots
    float tv[KK];
    int ti[KK];
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      const int64_t v = vbase + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
      tv[r] = z[r];
      ti[r] = v < V ? (int)v : kTsPad;
    }
    ts_sort<KK>(tv, ti);
#pragma unroll
    for (int r = KK; r < 16; ++r) {
      const int64_t v = vbase + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
      if (v < V) ts_insert_inc<KK>(tv, ti, z[r], (int)v);
    }
    // merge the partner lane's list
    float ov[KK];
    int oi[KK];
#pragma unroll
    for (int i = 0; i < KK; ++i) {
      ov[i] = __shfl_xor(tv[i], 32);
      oi[i] = __shfl_xor(ti[i], 32);
    }
    ts_merge_sorted<KK>(tv, ti, ov, oi);
    if (l < 32) {
      sm.red.mx[w][col] = mx;
      sm.red.sm[w][col] = s;
#pragma unroll
      for (int i = 0; i < KK; ++i) {
        sm.red.val[w][col][i] = tv[i];
        sm.red.id[w][col][i] = ti[i];
      }
    }
  }
  __syncthreads();
  // combine the four waves: one thread per column
  if (tid < ncols) {
    const int col = tid;
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) mx = fmaxf(mx, sm.red.mx[q][col]);
    float s = 0.0f;
    float tv[KK];
    int ti[KK];
#pragma unroll
    for (int i = 0; i < KK; ++i) {
      tv[i] = sm.red.val[0][col][i];
      ti[i] = sm.red.id[0][col][i];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float mq = sm.red.mx[q][col];
      if (mq != -INFINITY) s += sm.red.sm[q][col] * __expf(mq - mx);
      if (q > 0) {
        float bv[KK];
        int bi[KK];
#pragma unroll
        for (int i = 0; i < KK; ++i) {
          bv[i] = sm.red.val[q][col][i];
          bi[i] = sm.red.id[q][col][i];
        }
        ts_merge_sorted<KK>(tv, ti, bv, bi);
      }
    }
    const size_t o = (size_t)vt * p.Mtot + m0 + col;
    p.pmax[o] = mx;
    p.psum[o] = s;
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
  int32_t* ccount;  // [batch]
  int32_t* fcount;  // [batch] parents of the current depth
  int32_t* ptok[2];   // [batch * F] parent tokens, by depth parity
  int32_t* pcand[2];  // [batch * F] parent candidate index (-1: anchor)
  int32_t cmax;
};

__global__ void ts_init_kernel(TsState st, const int32_t* anchor, int64_t batch) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  st.ccount[b] = 0;
  st.fcount[b] = 1;
  st.ptok[0][b] = anchor[b];
  st.pcand[0][b] = -1;
}

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
};

__device__ __forceinline__ uint64_t ts_zkey(float x, int id) {
  return ((uint64_t)order_key(__float_as_uint(x)) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id);
}

// One 1024-thread workgroup per request; the four waves of group g merge
// parents g, g + 4, ...: a pass over the tiles' maxima, then one over their
// exp sums (float32 terms relative to the parent's maximum, float64 total)
// and their top-KK lists; groups combine through LDS.
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
  __shared__ uint64_t red_k[kTsMergeGroups][kTsGroupWaves][KK];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = w / kTsGroupWaves, gw = w - g * kTsGroupWaves;
  const int gt = gw * kWave + lane;  // thread index within the group
  constexpr int GT = kTsGroupWaves * kWave;
  const int64_t b = blockIdx.x;
  TsState& st = p.st;
  const int par = p.d & 1;
  const int nf = st.fcount[b];
  const int K = p.k;
  const int base = st.ccount[b];
  const int shift = 4 * (kTsDMax - 1 - p.d);  // this depth's digit
  const int rounds = (nf + kTsMergeGroups - 1) / kTsMergeGroups;
  for (int rd = 0; rd < rounds; ++rd) {  // uniform trip count: every group reaches each barrier
    const int i = rd * kTsMergeGroups + g;
    const bool act = i < nf;
    const int m = (int)b * p.Fd + (act ? i : 0);
    // pass 1: the parent's maximum z
    float mx = -INFINITY;
    for (int t = gt; t < p.nvt; t += GT) mx = fmaxf(mx, p.pmax[(size_t)t * p.Mtot + m]);
    mx = wave_max(mx);
    if (lane == 0) red_d[g][gw] = mx;
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kTsGroupWaves; ++q) M = fmaxf(M, (float)red_d[g][q]);
    __syncthreads();
    // pass 2: exp sums and top-KK lists
    double s = 0.0;
    float tv[KK];
    int ti[KK];
#pragma unroll
    for (int j = 0; j < KK; ++j) {
      tv[j] = -INFINITY;
      ti[j] = 0x7FFFFFFF;
    }
    for (int t = gt; t < p.nvt; t += GT) {
      const size_t o = (size_t)t * p.Mtot + m;
      const float x = p.pmax[o];
      const float y = p.psum[o];
      float pv[KK];
      int pi[KK];
#pragma unroll
      for (int j = 0; j < KK; ++j) {
        pv[j] = p.pval[o * kTsKMax + j];
        pi[j] = p.pid[o * kTsKMax + j];
      }
      if (x != -INFINITY) s += (double)(y * __expf(x - M));
#pragma unroll
      for (int j = 0; j < KK; ++j) {
        if (j < K && pi[j] != 0x7FFFFFFF) {
          // (val, id) into the sorted list, branch-free
          const float xv = pv[j];
          const int id = pi[j];
          bool bt[KK];
#pragma unroll
          for (int q = 0; q < KK; ++q) bt[q] = q < K && (xv > tv[q] || (xv == tv[q] && id < ti[q]));
#pragma unroll
          for (int q = KK - 1; q >= 0; --q) {
            const bool sh = q > 0 && bt[q > 0 ? q - 1 : 0];
            const float v1 = q > 0 ? tv[q > 0 ? q - 1 : 0] : xv;
            const int i1 = q > 0 ? ti[q > 0 ? q - 1 : 0] : id;
            tv[q] = sh ? v1 : (bt[q] ? xv : tv[q]);
            ti[q] = sh ? i1 : (bt[q] ? id : ti[q]);
          }
        }
      }
    }
    s = wave_sum(s);
    // the group's top-KK: KK rounds of a max over each lane's best untaken key
    int head = 0;
    uint64_t wbest[KK];
#pragma unroll
    for (int r = 0; r < KK; ++r) {
      uint64_t mine = 0;
#pragma unroll
      for (int j = 0; j < KK; ++j)
        if (j == head && ti[j] != 0x7FFFFFFF) mine = ts_zkey(tv[j], ti[j]);
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
    if (act && gw == 0 && lane < K) {
      // lane r picks the r-th best of the group's waves' lists (keys unique)
      uint64_t all[kTsGroupWaves * KK];
#pragma unroll
      for (int q = 0; q < kTsGroupWaves; ++q)
#pragma unroll
        for (int r = 0; r < KK; ++r) all[q * KK + r] = red_k[g][q][r];
      double tot = 0.0;
#pragma unroll
      for (int q = 0; q < kTsGroupWaves; ++q) tot += red_d[g][q];
      const double lse = (double)M + log(tot);
      uint64_t pick = 0;
      for (int r = 0; r <= lane; ++r) {
        uint64_t bst = 0;
#pragma unroll
        for (int q = 0; q < kTsGroupWaves * KK; ++q) {
          const uint64_t x = all[q];
          if (x > bst && (r == 0 || x < pick)) bst = x;
        }
        pick = bst;
      }
      const int pc = st.pcand[par][m];
      const double pscore = pc < 0 ? 0.0 : st.cscore[b * st.cmax + pc];
      const uint64_t pkey = pc < 0 ? 0ull : st.ckey[b * st.cmax + pc];
      const int c = i * K + lane;
      ch_tok[c] = (int32_t)(0xFFFFFFFFu - (uint32_t)pick);
      ch_score[c] = pscore + ((double)key_value((uint32_t)(pick >> 32)) - lse);
      ch_key[c] = pkey | ((uint64_t)(lane + 1) << shift);
      ch_cand[c] = pc;
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
