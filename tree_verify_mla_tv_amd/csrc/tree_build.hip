// Best-first draft-tree builder: the step before verify.
//
// [Verify page = "The Precision Imperative: Validating Numerical Accuracy in a
//  Custom CUDA Attention Kernel", "The Context: What Led to This Moment" (a GPU
//  best-first tree builder in place of a per-request CPU heap); RoPE page =
//  "Precision as Correctness: The Float64 RoPE Decision in a Custom CUDA
//  Inference Engine", "The Broader Context: A Full Native Engine from Scratch"
//  (its tests are bit-exact against the reference).]
//
// A node is a path of drafter candidates, one per depth; its score is the
// float32 sum of their log-probs from the root down.  The tree takes, budget
// times, the best node whose parent is already in the tree: higher score, then
// smaller depth, smaller parent index, smaller candidate rank (candidates at a
// depth ranked by log-prob, higher first, equal ones by index; NaN = -inf).
//
// One wave per request.  Instead of all K children of every tree node, the
// frontier holds, per tree node, only its best child not yet taken: a
// sibling never beats the better-ranked sibling before it (its score is no
// higher, fl(s + x) being monotone in x, and on equal scores its rank is
// larger), so popping the best of these gives the same sequence.  Each pop
// replaces the popped entry by its next sibling and adds the new node's first
// child, so the frontier grows by at most one entry per pop: at most
// budget + 1 <= 64 entries, one per lane.
#include "tv_kernels.h"

namespace tv {

namespace {

constexpr int kBuildMaxK = 64;
constexpr int kBuildMaxNodes = 64;                   // root + budget <= 64: one frontier entry per lane
constexpr int kBuildMaxDepth = kBuildMaxNodes - 1;  // depths past the budget are never reached

// Order-preserving key of a float (larger value -> larger key); -0 and +0 share one.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Frontier entry packed so that the larger key is the better node: score key
// in the high word; then 63 - depth, 63 - parent, 63 - rank (6 bits each).
// Keys of distinct nodes differ ((depth, parent, rank) names the node); an
// empty lane holds 0, below every real key (order_key(-inf) > 0).
__device__ __forceinline__ unsigned long long pack_entry(float score, int depth, int par, int rank) {
  const uint32_t lo = (static_cast<uint32_t>(63 - depth) << 12) | (static_cast<uint32_t>(63 - par) << 6) |
                      static_cast<uint32_t>(63 - rank);
  return (static_cast<unsigned long long>(order_key(score)) << 32) | lo;
}

// One step of a wave maximum over 64-bit keys: each lane takes the larger of
// its key and the key DPP control kCtrl brings it (rows outside kRowMask keep
// theirs).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ unsigned long long dpp_max_step(unsigned long long x) {
  const int lo = static_cast<int>(static_cast<uint32_t>(x));
  const int hi = static_cast<int>(static_cast<uint32_t>(x >> 32));
  const uint32_t plo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(lo, lo, kCtrl, kRowMask, 0xf, false));
  const uint32_t phi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(hi, hi, kCtrl, kRowMask, 0xf, false));
  const unsigned long long p = (static_cast<unsigned long long>(phi) << 32) | plo;
  return p > x ? p : x;
}

// Maximum of x over the wave, in every lane: within quads (lane ^ 1, lane ^ 2),
// half rows (mirror of 8), rows (mirror of 16), then row 0 into row 1 and row
// 2 into row 3 (broadcast of lane 15), rows 0-1 into rows 2-3 (lane 31): lane
// 63 ends with the maximum, read back as a scalar.
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) {
  x = dpp_max_step<0xB1, 0xf>(x);   // quad_perm [1, 0, 3, 2]
  x = dpp_max_step<0x4E, 0xf>(x);   // quad_perm [2, 3, 0, 1]
  x = dpp_max_step<0x141, 0xf>(x);  // row_half_mirror
  x = dpp_max_step<0x140, 0xf>(x);  // row_mirror
  x = dpp_max_step<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_max_step<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x)), 63));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x >> 32)), 63));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

__global__ __launch_bounds__(64) void tree_build_kernel(const float* __restrict__ logp,
                                                        const int32_t* __restrict__ cand_tok,
                                                        const int32_t* __restrict__ root_tok, int D, int K, int budget,
                                                        int32_t* __restrict__ parent, int32_t* __restrict__ token,
                                                        int32_t* __restrict__ depth, float* __restrict__ score,
                                                        int32_t* __restrict__ n_nodes) {
  __shared__ float s_raw[kBuildMaxDepth * kBuildMaxK];
  __shared__ float s_lp[kBuildMaxDepth][kBuildMaxK];         // log-probs in rank order
  __shared__ unsigned char s_idx[kBuildMaxDepth][kBuildMaxK];  // rank -> candidate index
  __shared__ int s_par[kBuildMaxNodes];
  __shared__ int s_dep[kBuildMaxNodes];
  __shared__ int s_cand[kBuildMaxNodes];  // node -> offset of its candidate in cand_tok[b]
  __shared__ float s_sc[kBuildMaxNodes];

  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int De = min(D, budget);  // a node at depth d needs d pops
  const float* lp_b = logp + static_cast<int64_t>(b) * D * K;
  const int32_t* tok_b = cand_tok + static_cast<int64_t>(b) * D * K;

  // Rank the candidates of every depth used: rank = number of candidates with
  // a higher log-prob, or an equal one at a smaller index.
  const int n_lp = De * K;
  for (int i = lane; i < n_lp; i += 64) {
    const float v = lp_b[i];
    s_raw[i] = v != v ? -INFINITY : v;
  }
  __syncthreads();
  for (int i = lane; i < n_lp; i += 64) {
    const int d = i / K;
    const int c = i - d * K;
    const float v = s_raw[i];
    int rank = 0;
    for (int j = 0; j < K; ++j) {
      const float u = s_raw[d * K + j];
      rank += (u > v) | ((u == v) & (j < c));
    }
    s_lp[d][rank] = v;
    s_idx[d][rank] = static_cast<unsigned char>(c);
  }
  __syncthreads();

  // Frontier entry of this lane.
  bool valid = false;
  float e_score = 0.f, e_pscore = 0.f;  // entry's score and its parent's score
  int e_depth = 0, e_par = 0, e_rank = 0;
  if (lane == 0 && De >= 1) {
    valid = true;
    e_depth = 1;
    e_par = 0;
    e_rank = 0;
    e_pscore = 0.f;
    e_score = 0.f + s_lp[0][0];
  }
  int n = 0;
  while (n < budget) {
    const unsigned long long mine = valid ? pack_entry(e_score, e_depth, e_par, e_rank) : 0ull;
    const unsigned long long m = wave_max_u64(mine);
    if (m == 0ull) break;  // frontier empty (m is wave-uniform)
    const unsigned long long win_mask = __ballot(valid && mine == m);
    const int w = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(win_mask)) - 1);
    // The winner's entry, to every lane.
    const float sc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e_score), w));
    const int d = __builtin_amdgcn_readlane(e_depth, w);
    const int par = __builtin_amdgcn_readlane(e_par, w);
    const int r = __builtin_amdgcn_readlane(e_rank, w);
    ++n;
    if (lane == 0) {
      s_par[n] = par;
      s_dep[n] = d;
      s_sc[n] = sc;
      s_cand[n] = (d - 1) * K + s_idx[d - 1][r];
    }
    // The winner's lane moves on to the next sibling, if any.
    if (lane == w) {
      if (r + 1 < K) {
        e_rank = r + 1;
        e_score = e_pscore + s_lp[d - 1][r + 1];
      } else {
        valid = false;
      }
    }
    // The new node's first child goes to the lowest empty lane (one exists:
    // at most n entries remain after the pop, n <= 63).
    if (d < De) {
      const unsigned long long empty = __ballot(!valid);
      const int f = __ffsll(static_cast<long long>(empty)) - 1;
      if (lane == f) {
        valid = true;
        e_depth = d + 1;
        e_par = n;
        e_rank = 0;
        e_pscore = sc;
        e_score = sc + s_lp[d][0];
      }
    }
  }
  __syncthreads();
  // Slot i = lane: the root, the n drafted nodes, then empty slots.
  if (lane <= budget) {
    const int64_t o = static_cast<int64_t>(b) * (budget + 1) + lane;
    if (lane == 0) {
      parent[o] = -1;
      depth[o] = 0;
      score[o] = 0.f;
      token[o] = root_tok[b];
    } else if (lane <= n) {
      parent[o] = s_par[lane];
      depth[o] = s_dep[lane];
      score[o] = s_sc[lane];
      token[o] = tok_b[s_cand[lane]];
    } else {
      parent[o] = -1;
      depth[o] = -1;
      score[o] = -INFINITY;
      token[o] = -1;
    }
  }
  if (lane == 0) n_nodes[b] = n;
}

}  // namespace

hipError_t launch_tree_build(const float* logp, const int32_t* cand_tok, const int32_t* root_tok, int B, int D, int K,
                             int budget, int32_t* parent, int32_t* token, int32_t* depth, float* score,
                             int32_t* n_nodes, hipStream_t stream) {
  tree_build_kernel<<<dim3(static_cast<unsigned>(B)), 64, 0, stream>>>(logp, cand_tok, root_tok, D, K, budget, parent,
                                                                        token, depth, score, n_nodes);
  return hipGetLastError();
}

}  // namespace tv
