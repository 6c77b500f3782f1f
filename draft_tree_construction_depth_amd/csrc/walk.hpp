// Stage 3 (standalone) and stage 4: ancestor mask and greedy acceptance walk.
//
// Mask: SparklingTree post, "Step 4: Creating the tree mask" -- each node
// sees itself, its ancestors and the root. Bits are packed LSB first into
// 64-bit words; one thread builds one row by walking the parent chain.
//
// Walk: DDTree explainer, section 5 (verifier walk), TreeSpark README item 4
// (argmax-following acceptance walk). One wavefront per request loads the
// request's parent, token and target-token arrays (B <= 512, so <= 8 nodes
// per lane), stages the targets in LDS, and marks in parallel, for every
// node, the child that carries the node's target token (at most one: the
// siblings are distinct tokens of one row). The walk then follows those
// marks from the root, one LDS read per accepted node, at most L steps.
#pragma once

#include "common.hpp"

namespace ddt {

constexpr int kMaskThreads = 256;
constexpr int kWalkMaxPerLane = 8;  // B <= 512

struct MaskParams {
  const int32_t* parents;
  const int32_t* num_nodes;
  int64_t batch;
  int32_t B;
  int32_t W;
  uint64_t* mask;
};

__global__ __launch_bounds__(kMaskThreads) void mask_kernel(MaskParams p) {
  __shared__ int spar[512];
  const int64_t b = blockIdx.x;
  const int B = p.B, W = p.W;
  int n = p.num_nodes[b];
  n = n < 0 ? 0 : (n > B ? B : n);
  const int32_t* par = p.parents + (size_t)b * B;
  // parents in LDS, a malformed one (not an earlier node) ends its chain
  for (int j = threadIdx.x; j < n; j += kMaskThreads) {
    const int pu = par[j];
    spar[j] = pu < 0 || pu > j ? -1 : pu;
  }
  __syncthreads();
  // one thread per (row, 64-bit word): the row's ancestor chain, this word's bits
  uint64_t* dst = p.mask + (size_t)b * (B + 1) * W;
  for (int t = threadIdx.x; t < (B + 1) * W; t += kMaskThreads) {
    const int i = t / W, q = t - i * W;
    uint64_t m = 0;
    if (i <= n) {
      int u = i;
      for (int step = 0; step <= B; ++step) {
        m |= (u >> 6) == q ? 1ull << (u & 63) : 0ull;
        if (u == 0) break;
        const int pu = spar[u - 1];
        if (pu < 0) break;
        u = pu;
      }
    }
    dst[t] = m;
  }
}

struct WalkParams {
  const int32_t* tree_tokens;
  const int32_t* parents;
  const int32_t* num_nodes;
  const int32_t* target_tokens;  // [batch][B+1]
  int64_t batch;
  int32_t B;
  int32_t L;
  int32_t* accepted_nodes;  // [batch][L]
  int32_t* accept_len;
  int32_t* next_token;
};

__global__ __launch_bounds__(kWave) void walk_kernel(WalkParams p) {
  // LDS: every node's target token, and for every node the lowest-numbered
  // child that carries that token (kNone: none)
  constexpr int kNone = 0x7FFFFFFF;
  __shared__ int s_tgt[kWalkMaxPerLane * kWave + 1];
  __shared__ int s_next[kWalkMaxPerLane * kWave + 1];
  const int64_t b = blockIdx.x;
  const int lane = threadIdx.x;
  const int B = p.B, L = p.L;
  const int32_t* tgt = p.target_tokens + (size_t)b * (B + 1);
  // node j+1 lives in lane j % 64, slot j / 64, with its parent, token and
  // target token. Every load (bounded by B, not by the node count) is issued
  // together with the node count's; nodes past the count are masked after.
  int par[kWalkMaxPerLane], tok[kWalkMaxPerLane], tg[kWalkMaxPerLane];
#pragma unroll
  for (int t = 0; t < kWalkMaxPerLane; ++t) {
    const int j = lane + t * kWave;
    const bool in = j < B;
    par[t] = in ? p.parents[(size_t)b * B + j] : -1;
    tok[t] = in ? p.tree_tokens[(size_t)b * B + j] : 0;
    tg[t] = in ? tgt[j + 1] : 0;
  }
  const int root_tgt = tgt[0];
  int n = p.num_nodes[b];
  n = n < 0 ? 0 : (n > B ? B : n);
  if (lane == 0) {
    s_tgt[0] = root_tgt;
    s_next[0] = kNone;
  }
#pragma unroll
  for (int t = 0; t < kWalkMaxPerLane; ++t) {
    const int j = lane + t * kWave;
    if (j < B) {
      s_tgt[j + 1] = tg[t];
      s_next[j + 1] = kNone;
    }
  }
  // (one wavefront: its LDS operations take effect in program order)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // a node whose token is its parent's target token is that parent's next
  // step (siblings carry distinct tokens; with equal ones the lowest node
  // number wins); malformed parents (not an earlier node) never match
#pragma unroll
  for (int t = 0; t < kWalkMaxPerLane; ++t) {
    const int j = lane + t * kWave;
    if (j < n && par[t] >= 0 && par[t] <= j && tok[t] == s_tgt[par[t]])
      atomicMin(&s_next[par[t]], j + 1);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // the walk itself: one LDS read per accepted node
  int cur = 0, len = 0, path = -1;
  while (len < L) {
    const int nx = s_next[cur];
    if (nx == kNone) break;
    if (lane == len) path = nx;
    ++len;
    cur = nx;
  }
  for (int i = lane; i < L; i += kWave) p.accepted_nodes[(size_t)b * L + i] = i == lane ? path : -1;
  if (lane == 0) {
    p.accept_len[b] = len;
    p.next_token[b] = s_tgt[cur];
  }
}

}  // namespace ddt
