// Stage 3 (standalone) and stage 4: ancestor mask and greedy acceptance walk.
//
// Mask: SparklingTree post, "Step 4: Creating the tree mask" -- each node
// sees itself, its ancestors and the root. Bits are packed LSB first into
// 64-bit words; one thread builds one row by walking the parent chain.
//
// Walk: DDTree explainer, section 5 (verifier walk), TreeSpark README item 4
// (argmax-following acceptance walk). One wavefront per request holds the
// request's parent, token and target-token arrays in registers (B <= 512, so
// <= 8 nodes per lane); each step is one compare and one ballot per held
// slot plus one cross-lane read of the next target, and the walk takes at
// most L steps.
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
    par[t] = in ? p.parents[(size_t)b * B + j] : -2;
    tok[t] = in ? p.tree_tokens[(size_t)b * B + j] : 0;
    tg[t] = in ? tgt[j + 1] : 0;
  }
  const int root_tgt = tgt[0];
  int n = p.num_nodes[b];
  n = n < 0 ? 0 : (n > B ? B : n);
  const int slots = (n + kWave - 1) / kWave;  // uniform
#pragma unroll
  for (int t = 0; t < kWalkMaxPerLane; ++t)
    if (lane + t * kWave >= n) par[t] = -2;  // never a child
  int cur = 0, len = 0, want = root_tgt;
  while (len < L) {
    // the child of cur carrying the wanted token (lowest node number if
    // several); its target token is read from its lane
    int found = 0, next = 0;
#pragma unroll
    for (int t = 0; t < kWalkMaxPerLane; ++t) {
      if (t < slots && found == 0) {
        const uint64_t M = __ballot(par[t] == cur && tok[t] == want);
        if (M) {
          const int src = __builtin_ctzll(M);
          found = t * kWave + src + 1;
          next = __builtin_amdgcn_readlane(tg[t], src);
        }
      }
    }
    if (found == 0) break;
    if (lane == 0) p.accepted_nodes[(size_t)b * L + len] = found;
    ++len;
    cur = found;
    want = next;
  }
  for (int i = len + lane; i < L; i += kWave) p.accepted_nodes[(size_t)b * L + i] = -1;
  if (lane == 0) {
    p.accept_len[b] = len;
    p.next_token[b] = want;
  }
}

}  // namespace ddt
