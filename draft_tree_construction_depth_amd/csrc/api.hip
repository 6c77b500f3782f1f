// C ABI of libddtree.so (declared in include/ddtree.h): argument checks,
// workspace carving, launch geometry and stream-ordered launches.
#include "ddtree.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "select.hpp"
#include "stage1.hpp"
#include "treespark.hpp"
#include "walk.hpp"
#include "kv.hpp"
#include "sparkling.hpp"
#include "dspark.hpp"
#include "beam.hpp"
#include "probe.hpp"

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

int elems_per_vec(int dtype) { return dtype == DDT_BF16 ? 8 : 4; }
size_t elem_size(int dtype) { return dtype == DDT_BF16 ? 2 : 4; }

struct S1Plan {
  bool row;       // one workgroup per row (double-buffered chunks), no merge
  int nv;         // 16-byte vectors per thread
  int64_t chunk;  // elements per chunk (256 * nv * elements per vector)
  int S;          // chunks per row
  int capp;       // candidate slots per chunk record
  bool ok;        // a supported geometry exists
};

int groups_per_thread(int nv) { return nv == 2 ? 1 : nv / 4; }

// Chunk geometry. Big register-resident chunks (16 vectors per thread) once
// the grid has >= 1024 blocks; smaller chunks for few rows, so that a single
// request still spreads over the 256 CUs. Then grow the chunk until the row
// merge can hold every record
// (S * capp <= 64 * kMergeSlots register slots with capp >= K, S <= 64) and
// each wave has >= K/2 group maxima for its threshold.
S1Plan plan_stage1(int64_t rows, int64_t V, int dtype, int K) {
  const int epv = elems_per_vec(dtype);
  const bool vec_rows = ((size_t)V * elem_size(dtype)) % 16 == 0;
  auto nchunks = [&](int nv) {
    const int64_t cap = (int64_t)ddt::kS1Threads * nv * epv;
    return (V + cap - 1) / cap;
  };
  S1Plan p;
  p.ok = false;
  p.row = false;
  // Many rows: one workgroup per row, 8 vectors per thread per chunk, double
  // buffered (every CU holds >= 2 rows in flight).
  if (vec_rows && rows >= 512) {
    p.row = true;
    p.nv = 8;
    p.chunk = (int64_t)ddt::kS1Threads * 8 * epv;
    p.S = (int)nchunks(8);
    p.capp = 0;
    p.ok = true;
    return p;
  }
  const int max_nv = vec_rows ? 16 : 8;
  int nv = 2;
  if (rows * nchunks(4) >= 256) nv = 4;
  if (rows * nchunks(8) >= 512) nv = 8;
  if (rows * nchunks(16) >= 1024) nv = 16;
  if (nv > max_nv) nv = max_nv;
  for (;; nv *= 2) {
    if (nv > max_nv) return p;
    const int64_t S = nchunks(nv);
    if (S > 64) continue;
    const int64_t slots = (int64_t)ddt::kWave * ddt::kMergeSlots;
    const int64_t capp = 2 * (int64_t)K < slots / S ? 2 * (int64_t)K : slots / S;
    if (capp < K) continue;
    if (64 * groups_per_thread(nv) * 2 < K && nv < max_nv) continue;
    p.nv = nv;
    p.S = (int)S;
    p.chunk = (int64_t)ddt::kS1Threads * nv * epv;
    p.capp = (int)capp;
    p.ok = true;
    return p;
  }
}

struct S1Layout {
  size_t cnt, thr, meta, cands, end;
};

S1Layout s1_layout(int64_t rows, const S1Plan& pl, size_t base) {
  S1Layout l;
  const size_t recs = pl.row ? 0 : (size_t)rows * pl.S;
  l.cnt = base + kAlign;  // a small header keeps every valid size positive
  l.thr = align_up(l.cnt + recs * sizeof(int32_t));
  l.meta = align_up(l.thr + recs * sizeof(uint32_t));
  l.cands = align_up(l.meta + recs * 2 * sizeof(double));
  l.end = align_up(l.cands + recs * pl.capp * sizeof(uint64_t));
  return l;
}

struct BuildLayout {
  S1Layout s1;
  size_t vals, ids, lse, end;
};

BuildLayout build_layout(int64_t batch, int32_t L, int64_t V, int32_t B, int dtype) {
  const int64_t rows = batch * L;
  const int K = (int)(B < V ? B : V);
  BuildLayout l;
  l.s1 = s1_layout(rows, plan_stage1(rows, V, dtype, K), 0);
  size_t off = l.s1.end;
  l.vals = off;
  off = align_up(off + (size_t)rows * K * sizeof(float));
  l.ids = off;
  off = align_up(off + (size_t)rows * K * sizeof(int32_t));
  l.lse = off;
  off = align_up(off + (size_t)rows * sizeof(double));
  l.end = off;
  return l;
}

// Compute units of the current device (cached per device).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int DT, int NV, int GS>
void launch_chunks(bool aligned, dim3 grid, const ddt::Stage1Params& prm, hipStream_t st) {
  if (aligned) {
    hipLaunchKernelGGL((ddt::stage1_chunk_kernel<DT, NV, GS, true>), grid,
                       dim3(ddt::kS1Threads), 0, st, prm);
  } else {
    hipLaunchKernelGGL((ddt::stage1_chunk_kernel<DT, NV, GS, false>), grid,
                       dim3(ddt::kS1Threads), 0, st, prm);
  }
}

template <int DT>
hipError_t launch_stage1_dt(const S1Plan& pl, bool aligned, int64_t rows,
                            const ddt::Stage1Params& prm, hipStream_t st) {
  if (pl.row) {
    // the row kernel holds four workgroups per CU
    if (rows <= 4 * (int64_t)cu_count())
      hipLaunchKernelGGL((ddt::stage1_row_kernel<DT, 8, 4, true>), dim3((unsigned)rows),
                         dim3(ddt::kS1Threads), 0, st, prm);
    else
      hipLaunchKernelGGL((ddt::stage1_row_kernel<DT, 8, 4, false>), dim3((unsigned)rows),
                         dim3(ddt::kS1Threads), 0, st, prm);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(rows * pl.S));
  switch (pl.nv) {
    case 16:
      // plan_stage1 picks 16 vectors per thread only for 16-byte multiple rows
      if (!aligned) return hipErrorInvalidValue;
      hipLaunchKernelGGL((ddt::stage1_chunk_kernel<DT, 16, 4, true>), grid,
                         dim3(ddt::kS1Threads), 0, st, prm);
      break;
    case 8: launch_chunks<DT, 8, 4>(aligned, grid, prm, st); break;
    case 4: launch_chunks<DT, 4, 4>(aligned, grid, prm, st); break;
    default: launch_chunks<DT, 2, 2>(aligned, grid, prm, st); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 mgrid((unsigned)rows);
  hipLaunchKernelGGL((ddt::stage1_merge_kernel<DT>), mgrid, dim3(ddt::kWave * ddt::kMergeWaves),
                     0, st, prm);
  return hipGetLastError();
}

int ceil_log2_64(int64_t x) {
  int b = 0;
  while (((int64_t)1 << b) < x) ++b;
  return b;
}

hipError_t launch_stage1(int dtype, const S1Plan& pl, const void* logits, int64_t rows,
                         int64_t V, int K, const S1Layout& lay, char* ws, int32_t* ids,
                         float* vals, double* lse, hipStream_t st) {
  ddt::Stage1Params prm;
  prm.logits = logits;
  prm.rows = rows;
  prm.V = V;
  prm.chunk = pl.chunk;
  prm.S = pl.S;
  prm.K = K;
  prm.capp = pl.capp;
  prm.idbits = ceil_log2_64(V) < 1 ? 1 : ceil_log2_64(V);
  prm.cnt = (int32_t*)(ws + lay.cnt);
  prm.thr = (uint32_t*)(ws + lay.thr);
  prm.meta = (double*)(ws + lay.meta);
  prm.cands = (uint64_t*)(ws + lay.cands);
  prm.out_ids = ids;
  prm.out_vals = vals;
  prm.out_lse = lse;
  // The base pointer is 16-byte aligned (checked by the callers), so rows can
  // be read with 16-byte vectors iff their byte length is a multiple of 16.
  const bool aligned = ((size_t)V * elem_size(dtype)) % 16 == 0;
  if (dtype == DDT_BF16) return launch_stage1_dt<0>(pl, aligned, rows, prm, st);
  return launch_stage1_dt<1>(pl, aligned, rows, prm, st);
}

int ceil_log2(int x) {
  int b = 0;
  while ((1 << b) < x) ++b;
  return b;
}

bool valid_dtype(int dtype) { return dtype == DDT_BF16 || dtype == DDT_F32; }

// Host-side constants of a selection launch: multipliers for the kernels'
// divisions by K and W (exact for the table and mask indices, < 2^13) and the
// threshold's lower-bound rank.
void select_derived(ddt::SelectParams& sp) {
  const uint64_t k = (uint64_t)(sp.K > 0 ? sp.K : 1), w = (uint64_t)(sp.W > 0 ? sp.W : 1);
  sp.kmag = ((1ull << 32) + k - 1) / k;
  sp.wmag = ((1ull << 32) + w - 1) / w;
  const int c = (sp.B + sp.L - 1) / (sp.L > 0 ? sp.L : 1);
  sp.q1 = c < sp.K ? c : sp.K;
  if (sp.q1 < 1) sp.q1 = 1;
}

int launch_select(const float* vals, const int32_t* ids, const double* lse, int64_t batch,
                  int32_t L, int32_t K, int32_t B, int bpd, int32_t* tree_tokens,
                  int32_t* parents, float* logq, int32_t* depths, int32_t* num_nodes,
                  uint64_t* mask, hipStream_t stream) {
  ddt::SelectParams sp;
  sp.vals = vals;
  sp.ids = ids;
  sp.lse = lse;
  sp.batch = batch;
  sp.L = L;
  sp.K = K;
  sp.B = B;
  sp.bpd = bpd;
  sp.tree_tokens = tree_tokens;
  sp.parents = parents;
  sp.logq = logq;
  sp.depths = depths;
  sp.num_nodes = num_nodes;
  sp.mask = mask;
  sp.W = (B + 1 + 63) / 64;
  sp.sp_lp = nullptr;
  sp.sp_best = nullptr;
  sp.sp_blp = nullptr;
  select_derived(sp);
  hipLaunchKernelGGL(ddt::select_kernel, dim3((unsigned)batch), dim3(ddt::kSelNT), 0, stream,
                     sp);
  return hipGetLastError() == hipSuccess ? DDT_OK : DDT_EHIP;
}

// ---- TreeSpark: per-depth parent counts and the workspace layout ----------
struct TsShape {
  int kk;          // children per parent, min(k, V)
  int Fd[ddt::kTsDMax];  // parents per request at each depth
  int Fmax;        // largest of them
  int cmax;        // candidates per request
  int64_t nvt;     // 128-row tiles of the vocabulary
  int64_t Mtot;    // partial-record parent slots (batch * Fmax); records are [Mtot][nvt]
};

TsShape ts_shape(int64_t batch, int D, int64_t V, int k, int F) {
  TsShape sh;
  sh.kk = (int64_t)k < V ? k : (int)V;
  int fd = 1;
  sh.Fmax = 1;
  sh.cmax = 0;
  for (int d = 0; d < D; ++d) {
    sh.Fd[d] = fd;
    sh.Fmax = fd > sh.Fmax ? fd : sh.Fmax;
    sh.cmax += fd * sh.kk;
    const int nxt = fd * sh.kk;
    fd = nxt < F ? nxt : F;
  }
  sh.nvt = (V + ddt::kTsBV - 1) / ddt::kTsBV;
  sh.Mtot = batch * sh.Fmax;
  return sh;
}

struct TsLayout {
  size_t pmax, psum, pval, pid, ctok, cscore, ckey, cpar, cdep, ccount, fcount, ptok[2], pcand[2];
  size_t total;
};

TsLayout ts_layout(int64_t batch, const TsShape& sh) {
  TsLayout l;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const size_t rec = (size_t)sh.nvt * sh.Mtot;
  l.pmax = take(rec * 4);
  l.psum = take(rec * 4);
  l.pval = take(rec * ddt::kTsKMax * 4);
  l.pid = take(rec * ddt::kTsKMax * 4);
  const size_t nc = (size_t)batch * sh.cmax;
  l.ctok = take(nc * 4);
  l.cscore = take(nc * 8);
  l.ckey = take(nc * 8);
  l.cpar = take(nc * 4);
  l.cdep = take(nc * 4);
  l.ccount = take((size_t)batch * 4);
  l.fcount = take((size_t)batch * 4);
  for (int q = 0; q < 2; ++q) {
    l.ptok[q] = take((size_t)sh.Mtot * 4);
    l.pcand[q] = take((size_t)sh.Mtot * 4);
  }
  l.total = o;
  return l;
}

int ts_check(int64_t batch, int32_t D, int64_t V, int32_t H, int32_t k, int32_t F, int32_t N) {
  if (batch < 0 || D <= 0 || V <= 0 || H <= 0 || k <= 0 || F <= 0 || N <= 0) return DDT_EINVAL;
  if (D > ddt::kTsDMax || k > ddt::kTsKMax || F > ddt::kTsFMax || H % ddt::kTsKT != 0 ||
      V > 0x7FFFFFFFLL || N > 4096 || batch > 0x7FFFFFFFLL / ddt::kTsFMax ||
      V * (int64_t)H * 2 > 0xFFFFFFFFLL)  // byte offsets into E are 32-bit
    return DDT_ENOTSUP;
  return DDT_OK;
}

// ---- SparklingTree: workspace layout ---------------------------------------
struct SpLayout {
  S1Layout s1;
  size_t vals, ids, lse, lp, best, blp, end;
};

SpLayout sp_layout(int64_t batch, int32_t L, int64_t V, int32_t C, int dtype) {
  const int64_t rows = batch * L;
  SpLayout l;
  l.s1 = s1_layout(rows, plan_stage1(rows, V, dtype, C), 0);
  size_t off = l.s1.end;
  l.vals = off;
  off = align_up(off + (size_t)rows * C * sizeof(float));
  l.ids = off;
  off = align_up(off + (size_t)rows * C * sizeof(int32_t));
  l.lse = off;
  off = align_up(off + (size_t)rows * sizeof(double));
  const size_t prow = (size_t)batch * (L - 1) * C;  // conditioned rows
  l.lp = off;
  off = align_up(off + prow * C * sizeof(float));
  l.best = off;
  off = align_up(off + prow * sizeof(uint8_t));
  l.blp = off;
  off = align_up(off + prow * sizeof(float));
  l.end = off;
  return l;
}

// SparklingTree's rows: 1. every drafter row cut to its top C (value desc,
// id asc); 2. the conditioned child rows (Markov deltas on MFMA, log-probs,
// best child) into the workspace
int sp_rows(const void* logits, int dtype, const uint16_t* W1, const uint16_t* W2t, int64_t batch,
            int32_t L, int64_t V, int32_t C, int32_t R, const S1Plan& pl, const SpLayout& lay,
            char* ws, hipStream_t stream) {
  float* tv = (float*)(ws + lay.vals);
  int32_t* ti = (int32_t*)(ws + lay.ids);
  double* tz = (double*)(ws + lay.lse);
  hipError_t e =
      launch_stage1(dtype, pl, logits, batch * L, V, C, lay.s1, ws, ti, tv, tz, stream);
  if (e != hipSuccess) return DDT_EHIP;
  if (L > 1) {
    ddt::SpTableParams tp;
    tp.W1 = W1;
    tp.W2t = W2t;
    tp.ids = ti;
    tp.vals = tv;
    tp.L = L;
    tp.C = C;
    tp.R = R;
    tp.lp = (float*)(ws + lay.lp);
    tp.best = (uint8_t*)(ws + lay.best);
    tp.blp = (float*)(ws + lay.blp);
    hipLaunchKernelGGL(ddt::sp_table_kernel, dim3((unsigned)batch, (unsigned)(L - 1)),
                       dim3(ddt::kSpThreads), 0, stream, tp);
    if (hipGetLastError() != hipSuccess) return DDT_EHIP;
  }
  return DDT_OK;
}

int sp_check(int dtype, int64_t batch, int32_t L, int64_t V, int32_t C, int32_t R, int32_t B) {
  if (!valid_dtype(dtype) || batch < 0 || L <= 0 || V <= 0 || C <= 0 || R <= 0 || B <= 0)
    return DDT_EINVAL;
  if (C > V) return DDT_EINVAL;
  if (C > ddt::kSpC || R % ddt::kSpKT != 0 || R > ddt::kSpRMax) return DDT_ENOTSUP;
  if (B > DDT_MAX_B || L > DDT_MAX_L || V > 0x7FFFFFFFLL || batch > 0x7FFFFFFFLL)
    return DDT_ENOTSUP;
  const int bpd = ceil_log2(C) < 1 ? 1 : ceil_log2(C);
  if (L * bpd > 122 || (int64_t)L * C > ddt::kSpMaxLC) return DDT_ENOTSUP;
  return DDT_OK;
}

// ---- ddtree_build: shared checks and launches -------------------------------
int build_check(const void* logits, int dtype, int64_t batch, int32_t L, int64_t V, int32_t B,
                const int32_t* tree_tokens, const int32_t* parents, const float* logq,
                const int32_t* num_nodes, BuildLayout& lay) {
  if (!valid_dtype(dtype) || batch < 0 || L <= 0 || V <= 0 || B <= 0) return DDT_EINVAL;
  if (batch == 0) return DDT_OK;
  if (!logits || !tree_tokens || !parents || !logq || !num_nodes) return DDT_EINVAL;
  if ((uintptr_t)logits % 16 != 0) return DDT_EINVAL;
  if (B > DDT_MAX_B || L > DDT_MAX_L || V > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  const int K = (int)(B < V ? B : V);
  const int bpd = ceil_log2(K) < 1 ? 1 : ceil_log2(K);
  if ((int64_t)L * K > DDT_MAX_LK || L * bpd > 122) return DDT_ENOTSUP;
  const int64_t rows = batch * L;
  const S1Plan pl = plan_stage1(rows, V, dtype, K);
  if (!pl.ok || rows * pl.S > 0x7FFFFFFFLL || batch > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  lay = build_layout(batch, L, V, B, dtype);
  return DDT_OK;
}

int build_launch(const void* logits, int dtype, int64_t batch, int32_t L, int64_t V, int32_t B,
                 int32_t* tree_tokens, int32_t* parents, float* logq, int32_t* depths,
                 int32_t* num_nodes, uint64_t* mask, const BuildLayout& lay, char* ws,
                 hipStream_t stream) {
  const int K = (int)(B < V ? B : V);
  const int bpd = ceil_log2(K) < 1 ? 1 : ceil_log2(K);
  const int64_t rows = batch * L;
  const S1Plan pl = plan_stage1(rows, V, dtype, K);
  float* tv = (float*)(ws + lay.vals);
  int32_t* ti = (int32_t*)(ws + lay.ids);
  double* tz = (double*)(ws + lay.lse);
  hipError_t e = launch_stage1(dtype, pl, logits, rows, V, K, lay.s1, ws, ti, tv, tz, stream);
  if (e != hipSuccess) return DDT_EHIP;
  return launch_select(tv, ti, tz, batch, L, K, B, bpd, tree_tokens, parents, logq, depths,
                       num_nodes, mask, stream);
}

// ---- the static scratch of ddtree_build_noalloc ------------------------------
// One array per GPU, held until the process ends. In host code `scratch`
// names a host-side stand-in, never the device memory: every use goes
// through the address hipGetSymbolAddress returns for the current device,
// taken once per device and kept.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
constexpr int kNoAllocMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kNoAllocMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
char* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = (char*)ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int ddt_abi_version(void) { return 1; }

const char* ddt_status_string(int status) {
  switch (status) {
    case DDT_OK: return "ok";
    case DDT_EINVAL: return "invalid argument";
    case DDT_ENOTSUP: return "unsupported size";
    case DDT_EWORKSPACE: return "workspace too small";
    case DDT_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t ddtree_row_topk_workspace_size(int64_t rows, int64_t V, int32_t K, int dtype) {
  if (rows <= 0 || V <= 0 || K <= 0 || K > V || !valid_dtype(dtype)) return 0;
  const S1Plan pl = plan_stage1(rows, V, dtype, K);
  return pl.ok ? s1_layout(rows, pl, 0).end : 0;
}

int ddtree_row_topk(const void* logits, int dtype, int64_t rows, int64_t V, int32_t K,
                    int32_t* ids, float* vals, double* lse, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(dtype) || rows < 0 || V <= 0 || K <= 0) return DDT_EINVAL;
  if (K > V) return DDT_EINVAL;
  if (rows == 0) return DDT_OK;
  if (!logits || !ids || !vals || !lse || !workspace) return DDT_EINVAL;
  if ((uintptr_t)logits % 16 != 0) return DDT_EINVAL;
  if (K > DDT_MAX_B || V > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  const S1Plan pl = plan_stage1(rows, V, dtype, K);
  if (!pl.ok || rows * pl.S > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  const S1Layout lay = s1_layout(rows, pl, 0);
  if (workspace_bytes < lay.end) return DDT_EWORKSPACE;
  const hipError_t e = launch_stage1(dtype, pl, logits, rows, V, K, lay, (char*)workspace, ids,
                                     vals, lse, stream);
  return e == hipSuccess ? DDT_OK : DDT_EHIP;
}

size_t ddtree_build_workspace_size(int64_t batch, int32_t L, int64_t V, int32_t B, int dtype) {
  if (batch <= 0 || L <= 0 || V <= 0 || B <= 0 || !valid_dtype(dtype)) return 0;
  const int K = (int)(B < V ? B : V);
  if (!plan_stage1(batch * L, V, dtype, K).ok) return 0;
  return build_layout(batch, L, V, B, dtype).end;
}

int ddtree_build(const void* logits, int dtype, int64_t batch, int32_t L, int64_t V, int32_t B,
                 int32_t* tree_tokens, int32_t* parents, float* logq, int32_t* depths,
                 int32_t* num_nodes, uint64_t* mask, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  BuildLayout lay;
  const int chk = build_check(logits, dtype, batch, L, V, B, tree_tokens, parents, logq,
                              num_nodes, lay);
  if (chk != DDT_OK || batch == 0) return chk;
  if (!workspace) return DDT_EINVAL;
  if (workspace_bytes < lay.end) return DDT_EWORKSPACE;
  return build_launch(logits, dtype, batch, L, V, B, tree_tokens, parents, logq, depths,
                      num_nodes, mask, lay, (char*)workspace, stream);
}

int ddtree_build_noalloc(const void* logits, int dtype, int64_t batch, int32_t L, int64_t V,
                         int32_t B, int32_t* tree_tokens, int32_t* parents, float* logq,
                         int32_t* depths, int32_t* num_nodes, uint64_t* mask,
                         hipStream_t stream) {
  BuildLayout lay;
  const int chk = build_check(logits, dtype, batch, L, V, B, tree_tokens, parents, logq,
                              num_nodes, lay);
  if (chk != DDT_OK || batch == 0) return chk;
  if (lay.end > kNoAllocScratchBytes) return DDT_ENOTSUP;
  char* ws = noalloc_scratch();
  if (!ws) return DDT_EHIP;
  return build_launch(logits, dtype, batch, L, V, B, tree_tokens, parents, logq, depths,
                      num_nodes, mask, lay, ws, stream);
}

int ddtree_select(const float* vals, const int32_t* ids, const double* lse, int64_t batch,
                  int32_t L, int32_t K, int32_t B, int32_t* tree_tokens, int32_t* parents,
                  float* logq, int32_t* depths, int32_t* num_nodes, uint64_t* mask,
                  hipStream_t stream) {
  if (batch < 0 || L <= 0 || K <= 0 || B <= 0) return DDT_EINVAL;
  if (batch == 0) return DDT_OK;
  if (!vals || !ids || !lse || !tree_tokens || !parents || !logq || !num_nodes) return DDT_EINVAL;
  if (B > DDT_MAX_B || L > DDT_MAX_L || K > DDT_MAX_B || batch > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  const int bpd = ceil_log2(K) < 1 ? 1 : ceil_log2(K);
  if ((int64_t)L * K > DDT_MAX_LK || L * bpd > 122) return DDT_ENOTSUP;
  return launch_select(vals, ids, lse, batch, L, K, B, bpd, tree_tokens, parents, logq, depths,
                       num_nodes, mask, stream);
}

int ddtree_mask(const int32_t* parents, const int32_t* num_nodes, int64_t batch, int32_t B,
                uint64_t* mask, hipStream_t stream) {
  if (batch < 0 || B <= 0) return DDT_EINVAL;
  if (batch == 0) return DDT_OK;
  if (!parents || !num_nodes || !mask) return DDT_EINVAL;
  if (B > DDT_MAX_B || batch > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  ddt::MaskParams mp;
  mp.parents = parents;
  mp.num_nodes = num_nodes;
  mp.batch = batch;
  mp.B = B;
  mp.W = (B + 1 + 63) / 64;
  mp.mask = mask;
  hipLaunchKernelGGL(ddt::mask_kernel, dim3((unsigned)batch), dim3(ddt::kMaskThreads), 0, stream,
                     mp);
  return hipGetLastError() == hipSuccess ? DDT_OK : DDT_EHIP;
}

int ddtree_accept(const int32_t* tree_tokens, const int32_t* parents, const int32_t* num_nodes,
                  const int32_t* target_tokens, int64_t batch, int32_t B, int32_t L,
                  int32_t* accepted_nodes, int32_t* accept_len, int32_t* next_token,
                  hipStream_t stream) {
  if (batch < 0 || B <= 0 || L <= 0) return DDT_EINVAL;
  if (batch == 0) return DDT_OK;
  if (!tree_tokens || !parents || !num_nodes || !target_tokens || !accepted_nodes ||
      !accept_len || !next_token)
    return DDT_EINVAL;
  if (B > DDT_MAX_B || L > DDT_MAX_L || batch > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  ddt::WalkParams wp;
  wp.tree_tokens = tree_tokens;
  wp.parents = parents;
  wp.num_nodes = num_nodes;
  wp.target_tokens = target_tokens;
  wp.batch = batch;
  wp.B = B;
  wp.L = L;
  wp.accepted_nodes = accepted_nodes;
  wp.accept_len = accept_len;
  wp.next_token = next_token;
  hipLaunchKernelGGL(ddt::walk_kernel, dim3((unsigned)batch), dim3(ddt::kWave), 0, stream, wp);
  return hipGetLastError() == hipSuccess ? DDT_OK : DDT_EHIP;
}

int ddtree_read_probe(const void* src, int64_t rows, int64_t row_bytes, uint32_t* sink,
                      hipStream_t stream) {
  if (rows < 0 || row_bytes <= 0) return DDT_EINVAL;
  if (rows == 0) return DDT_OK;
  if (!src || !sink || (uintptr_t)src % 16 != 0 || row_bytes % 16 != 0) return DDT_EINVAL;
  if (rows > 0x7FFFFFFFLL || row_bytes > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  ddt::ProbeParams pp;
  pp.src = (const char*)src;
  pp.row_bytes = row_bytes;
  pp.sink = sink;
  hipLaunchKernelGGL(ddt::read_probe_kernel<8>, dim3((unsigned)rows), dim3(ddt::kS1Threads), 0,
                     stream, pp);
  return hipGetLastError() == hipSuccess ? DDT_OK : DDT_EHIP;
}

int ddtree_ts_load_probe(const void* W, const void* E, const int32_t* ptok, int64_t V, int32_t H,
                         int32_t variant, uint32_t* sink, hipStream_t stream) {
  if (!W || !E || !ptok || !sink || V <= 0 || H <= 0 || H % ddt::kTsKT != 0) return DDT_EINVAL;
  if ((uintptr_t)W % 16 != 0 || (uintptr_t)E % 16 != 0) return DDT_EINVAL;
  if (variant < 0 || variant > 7) return DDT_EINVAL;
  if (V * H * 2 >= (int64_t)1 << 32 || V > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  ddt::TsProbeParams tp;
  tp.W = (const uint16_t*)W;
  tp.E = (const uint16_t*)E;
  tp.ptok = ptok;
  tp.V = V;
  tp.H = H;
  tp.sink = sink;
  const dim3 grid((unsigned)((V + ddt::kTsBV - 1) / ddt::kTsBV)), block(ddt::kTsThreads);
  switch (variant) {
    case 0: hipLaunchKernelGGL((ddt::ts_load_probe_kernel<0, 2>), grid, block, 0, stream, tp); break;
    case 1: hipLaunchKernelGGL((ddt::ts_load_probe_kernel<1, 2>), grid, block, 0, stream, tp); break;
    case 2: hipLaunchKernelGGL((ddt::ts_load_probe_kernel<2, 2>), grid, block, 0, stream, tp); break;
    case 3: hipLaunchKernelGGL((ddt::ts_load_probe_kernel<2, 0x12>), grid, block, 0, stream, tp); break;
    case 4: hipLaunchKernelGGL((ddt::ts_load_probe_kernel<0, 0x12>), grid, block, 0, stream, tp); break;
    case 5: hipLaunchKernelGGL((ddt::ts_load_probe_kernel<3, 2>), grid, block, 0, stream, tp); break;
    case 7: {
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          cus <= 0)
        return DDT_EHIP;
      hipLaunchKernelGGL((ddt::ts_load_probe256p_kernel<2>), dim3((unsigned)cus),
                         dim3(2 * ddt::kTsThreads), 0, stream, tp);
      break;
    }
    default:
      hipLaunchKernelGGL((ddt::ts_load_probe256_kernel<2>),
                         dim3((unsigned)((V + 2 * ddt::kTsBV - 1) / (2 * ddt::kTsBV))),
                         dim3(2 * ddt::kTsThreads), 0, stream, tp);
      break;
  }
  return hipGetLastError() == hipSuccess ? DDT_OK : DDT_EHIP;
}

int ddtree_compact_kv(void* k_cache, void* v_cache, int64_t layers, int64_t batch,
                      int32_t heads, int64_t cap, int32_t row_bytes, const int32_t* past_len,
                      const int32_t* accepted_nodes, const int32_t* accept_len, int32_t L,
                      int32_t* new_len, hipStream_t stream) {
  if (layers < 0 || batch < 0 || heads < 0 || cap <= 0 || row_bytes <= 0 || L <= 0)
    return DDT_EINVAL;
  if (layers == 0 || batch == 0 || heads == 0) return DDT_OK;
  if (!k_cache || !v_cache || !past_len || !accepted_nodes || !accept_len) return DDT_EINVAL;
  if (((uintptr_t)k_cache | (uintptr_t)v_cache) & 15) return DDT_EINVAL;
  if (row_bytes % 16 != 0 || row_bytes > 1024 || L > DDT_MAX_L) return DDT_ENOTSUP;
  const int64_t slices = layers * batch * heads;
  const int64_t per_block = ddt::kKvThreads / ddt::kWave;
  const int64_t blocks = (slices + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFFLL || batch > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  ddt::KvParams kp;
  kp.k = (unsigned char*)k_cache;
  kp.v = (unsigned char*)v_cache;
  kp.layers = layers;
  kp.batch = batch;
  kp.cap = cap;
  kp.heads = heads;
  kp.row_bytes = row_bytes;
  kp.past_len = past_len;
  kp.accepted = accepted_nodes;
  kp.accept_len = accept_len;
  kp.L = L;
  kp.new_len = new_len;
  hipLaunchKernelGGL(ddt::kv_compact_kernel, dim3((unsigned)blocks), dim3(ddt::kKvThreads), 0,
                     stream, kp);
  return hipGetLastError() == hipSuccess ? DDT_OK : DDT_EHIP;
}

size_t treespark_workspace_size(int64_t batch, int32_t D, int64_t V, int32_t H, int32_t k,
                                int32_t F, int32_t N) {
  if (ts_check(batch, D, V, H, k, F, N) != DDT_OK || batch == 0) return 0;
  return ts_layout(batch, ts_shape(batch, D, V, k, F)).total;
}

int treespark_expand(const void* backbone, const void* W, const void* E, const int32_t* anchor,
                     int64_t batch, int32_t D, int64_t V, int32_t H, int32_t k, int32_t F,
                     int32_t N, int32_t* tree_tokens, int32_t* parents, float* logq,
                     int32_t* depths, int32_t* num_nodes, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  const int chk = ts_check(batch, D, V, H, k, F, N);
  if (chk != DDT_OK) return chk;
  if (batch == 0) return DDT_OK;
  if (!backbone || !W || !E || !anchor || !tree_tokens || !parents || !logq || !num_nodes ||
      !workspace)
    return DDT_EINVAL;
  if (((uintptr_t)W | (uintptr_t)E) % 16 != 0) return DDT_EINVAL;
  const TsShape sh = ts_shape(batch, D, V, k, F);
  const TsLayout lay = ts_layout(batch, sh);
  if (workspace_bytes < lay.total) return DDT_EWORKSPACE;
  char* ws = (char*)workspace;
  ddt::TsState st;
  st.ctok = (int32_t*)(ws + lay.ctok);
  st.cscore = (double*)(ws + lay.cscore);
  st.ckey = (uint64_t*)(ws + lay.ckey);
  st.cpar = (int32_t*)(ws + lay.cpar);
  st.cdep = (int32_t*)(ws + lay.cdep);
  st.ccount = (int32_t*)(ws + lay.ccount);
  st.fcount = (int32_t*)(ws + lay.fcount);
  for (int q = 0; q < 2; ++q) {
    st.ptok[q] = (int32_t*)(ws + lay.ptok[q]);
    st.pcand[q] = (int32_t*)(ws + lay.pcand[q]);
  }
  st.cmax = sh.cmax;
  float* pmax = (float*)(ws + lay.pmax);
  float* psum = (float*)(ws + lay.psum);
  float* pval = (float*)(ws + lay.pval);
  int32_t* pid = (int32_t*)(ws + lay.pid);

  // depth 0's parents are the anchors themselves (the merge at depth 0 takes
  // one parent, candidate -1, and no candidates before it), so no state is
  // initialised on the device
  int base = 0;  // candidates per request before depth d
  for (int d = 0; d < D; ++d) {
    const int Fd = sh.Fd[d];
    const int64_t M = batch * Fd;
    ddt::TsGemmParams gp;
    gp.W = (const uint16_t*)W;
    gp.E = (const uint16_t*)E;
    gp.bb = (const uint16_t*)backbone;
    gp.ptok = d == 0 ? anchor : st.ptok[d & 1];
    gp.V = V;
    gp.H = H;
    gp.D = D;
    gp.d = d;
    gp.M = (int32_t)M;
    gp.Fd = Fd;
    gp.k = sh.kk;
    gp.Mtot = (int32_t)sh.Mtot;
    gp.nvt = (int32_t)sh.nvt;
    gp.pmax = pmax;
    gp.psum = psum;
    gp.pval = pval;
    gp.pid = pid;
    const dim3 ggrid((unsigned)sh.nvt, (unsigned)((M + ddt::kTsBM - 1) / ddt::kTsBM));
    if (sh.kk <= 4)
      hipLaunchKernelGGL(ddt::ts_gemm_kernel<4>, ggrid, dim3(ddt::kTsThreads), 0, stream, gp);
    else
      hipLaunchKernelGGL(ddt::ts_gemm_kernel<8>, ggrid, dim3(ddt::kTsThreads), 0, stream, gp);
    if (hipGetLastError() != hipSuccess) return DDT_EHIP;
    ddt::TsMergeParams mp;
    mp.st = st;
    mp.pmax = pmax;
    mp.psum = psum;
    mp.pval = pval;
    mp.pid = pid;
    mp.nvt = (int32_t)sh.nvt;
    mp.Mtot = (int32_t)sh.Mtot;
    mp.d = d;
    mp.D = D;
    mp.Fd = Fd;
    mp.Fn = d + 1 < D ? sh.Fd[d + 1] : 1;
    mp.k = sh.kk;
    mp.F = F;
    mp.base = base;
    if (sh.kk <= 4)
      hipLaunchKernelGGL(ddt::ts_merge_kernel<4>, dim3((unsigned)batch),
                         dim3(ddt::kTsMergeThreads), 0, stream, mp);
    else
      hipLaunchKernelGGL(ddt::ts_merge_kernel<8>, dim3((unsigned)batch),
                         dim3(ddt::kTsMergeThreads), 0, stream, mp);
    if (hipGetLastError() != hipSuccess) return DDT_EHIP;
    base += Fd * sh.kk;
  }
  ddt::TsPackParams pp;
  pp.st = st;
  pp.N = N;
  pp.tree_tokens = tree_tokens;
  pp.parents = parents;
  pp.logq = logq;
  pp.depths = depths;
  pp.num_nodes = num_nodes;
  hipLaunchKernelGGL(ddt::ts_pack_kernel, dim3((unsigned)batch), dim3(ddt::kTsThreads),
                     (size_t)sh.cmax * 4, stream, pp);
  return hipGetLastError() == hipSuccess ? DDT_OK : DDT_EHIP;
}

size_t sparkling_build_workspace_size(int64_t batch, int32_t L, int64_t V, int32_t C,
                                      int32_t R, int32_t B, int dtype) {
  if (batch <= 0 || sp_check(dtype, batch, L, V, C, R, B) != DDT_OK) return 0;
  if (!plan_stage1(batch * L, V, dtype, C).ok) return 0;
  return sp_layout(batch, L, V, C, dtype).end;
}

int sparkling_build(const void* logits, int dtype, const uint16_t* W1, const uint16_t* W2t,
                    int64_t batch, int32_t L, int64_t V, int32_t C, int32_t R, int32_t B,
                    int32_t* tree_tokens, int32_t* parents, float* logq, int32_t* depths,
                    int32_t* num_nodes, uint64_t* mask, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  const int chk = sp_check(dtype, batch, L, V, C, R, B);
  if (chk != DDT_OK) return chk;
  if (batch == 0) return DDT_OK;
  if (!logits || !W1 || !W2t || !tree_tokens || !parents || !logq || !num_nodes || !workspace)
    return DDT_EINVAL;
  if ((uintptr_t)logits % 16 != 0 || (uintptr_t)W1 % 16 != 0 || (uintptr_t)W2t % 16 != 0)
    return DDT_EINVAL;
  const int64_t rows = batch * L;
  const S1Plan pl = plan_stage1(rows, V, dtype, C);
  if (!pl.ok || rows * pl.S > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  const SpLayout lay = sp_layout(batch, L, V, C, dtype);
  if (workspace_bytes < lay.end) return DDT_EWORKSPACE;
  char* ws = (char*)workspace;
  float* tv = (float*)(ws + lay.vals);
  int32_t* ti = (int32_t*)(ws + lay.ids);
  double* tz = (double*)(ws + lay.lse);
  float* lp = (float*)(ws + lay.lp);
  uint8_t* best = (uint8_t*)(ws + lay.best);
  float* blp = (float*)(ws + lay.blp);
  if (sp_rows(logits, dtype, W1, W2t, batch, L, V, C, R, pl, lay, ws, stream) != DDT_OK)
    return DDT_EHIP;
  // 3. best-first selection on the conditioned rows, then the mask
  ddt::SelectParams sp;
  sp.vals = tv;
  sp.ids = ti;
  sp.lse = tz;
  sp.batch = batch;
  sp.L = L;
  sp.K = C;
  sp.B = B;
  sp.bpd = ceil_log2(C) < 1 ? 1 : ceil_log2(C);
  sp.tree_tokens = tree_tokens;
  sp.parents = parents;
  sp.logq = logq;
  sp.depths = depths;
  sp.num_nodes = num_nodes;
  sp.mask = mask;
  sp.W = (B + 1 + 63) / 64;
  sp.sp_lp = lp;
  sp.sp_best = best;
  sp.sp_blp = blp;
  select_derived(sp);
  hipLaunchKernelGGL(ddt::sp_select_kernel, dim3((unsigned)batch), dim3(ddt::kSelThreads), 0,
                     stream, sp);
  return hipGetLastError() == hipSuccess ? DDT_OK : DDT_EHIP;
}

int dspark_budget(const float* conf, int64_t batch, int32_t P, const float* cost_ms,
                  int32_t n_cost, int32_t* keep, double* survival, int32_t* n_keep,
                  double* expected_tokens, double* objective, hipStream_t stream) {
  if (batch < 0 || P <= 0) return DDT_EINVAL;
  if (batch == 0) return DDT_OK;
  if (batch * P > ddt::kDsMaxN) return DDT_ENOTSUP;
  if (n_cost <= batch) return DDT_EINVAL;  // the step without guesses must be costed
  if (!conf || !cost_ms || !keep || !n_keep) return DDT_EINVAL;
  ddt::DsParams dp;
  dp.conf = conf;
  dp.R = (int32_t)batch;
  dp.P = P;
  dp.cost = cost_ms;
  dp.n_cost = n_cost;
  dp.keep = keep;
  dp.survival = survival;
  dp.n_keep = n_keep;
  dp.expected = expected_tokens;
  dp.objective = objective;
  hipLaunchKernelGGL(ddt::dspark_budget_kernel, dim3(1), dim3(ddt::kDsThreads), 0, stream, dp);
  return hipGetLastError() == hipSuccess ? DDT_OK : DDT_EHIP;
}

int sparkling_beam(const void* logits, int dtype, const uint16_t* W1, const uint16_t* W2t,
                   int64_t batch, int32_t L, int64_t V, int32_t C, int32_t R,
                   const int32_t* widths, int32_t budget, int32_t* tree_tokens,
                   int32_t* parents, float* logq, int32_t* depths, int32_t* num_nodes,
                   uint64_t* mask, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (L <= 0 || budget < 0) return DDT_EINVAL;
  if (L > DDT_MAX_L) return DDT_ENOTSUP;
  // the schedule: the caller's widths, or the budget spread evenly over the
  // depths with the remainder on the first ones ("evenly spread branches")
  int32_t w[DDT_MAX_L];
  if (!widths && budget > DDT_MAX_B) return DDT_ENOTSUP;
  for (int d = 0; d < L; ++d) w[d] = widths ? widths[d] : budget / L + (d < budget % L ? 1 : 0);
  int32_t B = 0;
  for (int d = 0; d < L; ++d) {
    if (w[d] < 0) return DDT_EINVAL;
    if (w[d] > ddt::kBmMaxW) return DDT_ENOTSUP;
    B += w[d];
  }
  if (B <= 0 || (widths && budget != 0 && budget != B)) return DDT_EINVAL;
  const int chk = sp_check(dtype, batch, L, V, C, R, B);
  if (chk != DDT_OK) return chk;
  if (batch == 0) return DDT_OK;
  if (!logits || !W1 || !W2t || !tree_tokens || !parents || !logq || !num_nodes || !workspace)
    return DDT_EINVAL;
  if ((uintptr_t)logits % 16 != 0 || (uintptr_t)W1 % 16 != 0 || (uintptr_t)W2t % 16 != 0)
    return DDT_EINVAL;
  const int64_t rows = batch * L;
  const S1Plan pl = plan_stage1(rows, V, dtype, C);
  if (!pl.ok || rows * pl.S > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  const SpLayout lay = sp_layout(batch, L, V, C, dtype);
  if (workspace_bytes < lay.end) return DDT_EWORKSPACE;
  char* ws = (char*)workspace;
  if (sp_rows(logits, dtype, W1, W2t, batch, L, V, C, R, pl, lay, ws, stream) != DDT_OK)
    return DDT_EHIP;
  ddt::BeamParams bp;
  ddt::SelectParams& sp = bp.sp;
  sp.vals = (const float*)(ws + lay.vals);
  sp.ids = (const int32_t*)(ws + lay.ids);
  sp.lse = (const double*)(ws + lay.lse);
  sp.batch = batch;
  sp.L = L;
  sp.K = C;
  sp.B = B;
  sp.bpd = ceil_log2(C) < 1 ? 1 : ceil_log2(C);
  sp.tree_tokens = tree_tokens;
  sp.parents = parents;
  sp.logq = logq;
  sp.depths = depths;
  sp.num_nodes = num_nodes;
  sp.mask = mask;
  sp.W = (B + 1 + 63) / 64;
  sp.sp_lp = (const float*)(ws + lay.lp);
  sp.sp_best = (const uint8_t*)(ws + lay.best);
  sp.sp_blp = (const float*)(ws + lay.blp);
  select_derived(sp);
  for (int d = 0; d < ddt::kMaxL; ++d) bp.widths[d] = d < L ? w[d] : 0;
  hipLaunchKernelGGL(ddt::beam_kernel, dim3((unsigned)batch), dim3(ddt::kBmThreads), 0, stream,
                     bp);
  return hipGetLastError() == hipSuccess ? DDT_OK : DDT_EHIP;
}

}  // extern "C"
