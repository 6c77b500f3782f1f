// C ABI of libddtree.so (declared in include/ddtree.h): argument checks,
// workspace carving, launch geometry and stream-ordered launches.
#include "ddtree.h"

#include <hip/hip_runtime.h>

#include "select.hpp"
#include "stage1.hpp"
#include "walk.hpp"

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
    hipLaunchKernelGGL((ddt::stage1_row_kernel<DT, 8, 4>), dim3((unsigned)rows),
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
  const dim3 mgrid((unsigned)((rows + ddt::kMergeWaves - 1) / ddt::kMergeWaves));
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
  hipLaunchKernelGGL(ddt::select_kernel, dim3((unsigned)batch), dim3(ddt::kSelThreads), 0, stream,
                     sp);
  return hipGetLastError() == hipSuccess ? DDT_OK : DDT_EHIP;
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
  if (!valid_dtype(dtype) || batch < 0 || L <= 0 || V <= 0 || B <= 0) return DDT_EINVAL;
  if (batch == 0) return DDT_OK;
  if (!logits || !tree_tokens || !parents || !logq || !num_nodes || !workspace)
    return DDT_EINVAL;
  if ((uintptr_t)logits % 16 != 0) return DDT_EINVAL;
  if (B > DDT_MAX_B || L > DDT_MAX_L || V > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  const int K = (int)(B < V ? B : V);
  const int bpd = ceil_log2(K) < 1 ? 1 : ceil_log2(K);
  if ((int64_t)L * K > DDT_MAX_LK || L * bpd > 122) return DDT_ENOTSUP;
  const int64_t rows = batch * L;
  const S1Plan pl = plan_stage1(rows, V, dtype, K);
  if (!pl.ok || rows * pl.S > 0x7FFFFFFFLL || batch > 0x7FFFFFFFLL) return DDT_ENOTSUP;
  const BuildLayout lay = build_layout(batch, L, V, B, dtype);
  if (workspace_bytes < lay.end) return DDT_EWORKSPACE;
  char* ws = (char*)workspace;
  float* tv = (float*)(ws + lay.vals);
  int32_t* ti = (int32_t*)(ws + lay.ids);
  double* tz = (double*)(ws + lay.lse);
  hipError_t e = launch_stage1(dtype, pl, logits, rows, V, K, lay.s1, ws, ti, tv, tz, stream);
  if (e != hipSuccess) return DDT_EHIP;
  return launch_select(tv, ti, tz, batch, L, K, B, bpd, tree_tokens, parents, logq, depths,
                       num_nodes, mask, stream);
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

}  // extern "C"
