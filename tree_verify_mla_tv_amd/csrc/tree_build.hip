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
// budget + 1 <= 256 entries, four slots per lane.
#include "tv_kernels.h"

namespace tv {

namespace {

constexpr int kBuildMaxK = 64;
constexpr int kBuildSlots = 4;                          // frontier slots per lane
constexpr int kBuildMaxNodes = 64 * kBuildSlots;        // root + budget
constexpr int kBuildMaxEntries = 8192;                  // ranked candidates held in LDS: min(D, budget) * K

// Order-preserving key of a float (larger value -> larger key); -0 and +0 share one.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Frontier entry packed so that the larger key is the better node: score key
// in the high word; then 255 - depth, 255 - parent (8 bits each) and 63 - rank
// (6 bits).  Keys of distinct nodes differ ((depth, parent, rank) names the
// node); an empty slot holds 0, below every real key (order_key(-inf) > 0).
__device__ __forceinline__ unsigned long long pack_entry(float score, int depth, int par, int rank) {
  const uint32_t lo = (static_cast<uint32_t>(255 - depth) << 14) | (static_cast<uint32_t>(255 - par) << 6) |
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

// kSlots frontier slots per lane: 1 for budgets below 64, 4 up to 255.
template <int kSlots>
__global__ __launch_bounds__(64) void tree_build_kernel(const float* __restrict__ logp,
                                                        const int32_t* __restrict__ cand_tok,
                                                        const int32_t* __restrict__ root_tok, int D, int K, int budget,
                                                        int32_t* __restrict__ parent, int32_t* __restrict__ token,
                                                        int32_t* __restrict__ depth, float* __restrict__ score,
                                                        int32_t* __restrict__ n_nodes) {
  __shared__ float s_raw[kBuildMaxEntries];
  __shared__ float s_lp[kBuildMaxEntries];           // [d * K + rank]: log-probs in rank order
  __shared__ unsigned char s_idx[kBuildMaxEntries];  // [d * K + rank]: candidate index
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
    s_lp[d * K + rank] = v;
    s_idx[d * K + rank] = static_cast<unsigned char>(c);
  }
  __syncthreads();

  // Frontier slots of this lane (static indices only, so they stay in registers).
  bool valid[kSlots];
  float e_score[kSlots], e_pscore[kSlots];  // entry's score and its parent's score
  int e_depth[kSlots], e_par[kSlots], e_rank[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    valid[j] = false;
    e_score[j] = e_pscore[j] = 0.f;
    e_depth[j] = e_par[j] = e_rank[j] = 0;
  }
  if (lane == 0 && De >= 1) {
    valid[0] = true;
    e_depth[0] = 1;
    e_score[0] = 0.f + s_lp[0];
  }
  int n = 0;
  while (n < budget) {
    // This lane's best slot, then the wave's best.
    unsigned long long mine = 0ull;
    int my_slot = 0;
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      const unsigned long long k = valid[j] ? pack_entry(e_score[j], e_depth[j], e_par[j], e_rank[j]) : 0ull;
      if (k > mine) {
        mine = k;
        my_slot = j;
      }
    }
    const unsigned long long m = wave_max_u64(mine);
    if (m == 0ull) break;  // frontier empty (m is wave-uniform)
    const unsigned long long win_mask = __ballot(mine == m);
    const int w = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(win_mask)) - 1);
    const int ws = __builtin_amdgcn_readlane(my_slot, w);
    // The winner's entry, to every lane.
    float sel_score = e_score[0], sel_pscore = e_pscore[0];
    int sel_depth = e_depth[0], sel_par = e_par[0], sel_rank = e_rank[0];
#pragma unroll
    for (int j = 1; j < kSlots; ++j) {
      if (ws == j) {
        sel_score = e_score[j];
        sel_pscore = e_pscore[j];
        sel_depth = e_depth[j];
        sel_par = e_par[j];
        sel_rank = e_rank[j];
      }
    }
    const float sc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_score), w));
    const float psc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_pscore), w));
    const int d = __builtin_amdgcn_readlane(sel_depth, w);
    const int par = __builtin_amdgcn_readlane(sel_par, w);
    const int r = __builtin_amdgcn_readlane(sel_rank, w);
    ++n;
    if (lane == 0) {
      s_par[n] = par;
      s_dep[n] = d;
      s_sc[n] = sc;
      s_cand[n] = (d - 1) * K + s_idx[(d - 1) * K + r];
    }
    // The winning slot moves on to the next sibling, if any.
    const bool has_sibling = r + 1 < K;
    const float sib_score = has_sibling ? psc + s_lp[(d - 1) * K + r + 1] : 0.f;
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      if (lane == w && ws == j) {
        if (has_sibling) {
          e_rank[j] = r + 1;
          e_score[j] = sib_score;
        } else {
          valid[j] = false;
        }
      }
    }
    // The new node's first child goes to an empty slot (one exists: at most
    // n entries remain after the pop, and n < 64 * kSlots).
    if (d < De) {
      const float child_score = sc + s_lp[d * K];
      bool placed = false;
#pragma unroll
      for (int j = 0; j < kSlots; ++j) {
        const unsigned long long empty = __ballot(!valid[j]);
        if (!placed && empty != 0ull) {
          placed = true;
          if (lane == __ffsll(static_cast<long long>(empty)) - 1) {
            valid[j] = true;
            e_depth[j] = d + 1;
            e_par[j] = n;
            e_rank[j] = 0;
            e_pscore[j] = sc;
            e_score[j] = child_score;
          }
        }
      }
    }
  }
  __syncthreads();
  // Slot i (lane + 64 j): the root, the n drafted nodes, then empty slots.
  for (int i = lane; i <= budget; i += 64) {
    const int64_t o = static_cast<int64_t>(b) * (budget + 1) + i;
    if (i == 0) {
      parent[o] = -1;
      depth[o] = 0;
      score[o] = 0.f;
      token[o] = root_tok[b];
    } else if (i <= n) {
      parent[o] = s_par[i];
      depth[o] = s_dep[i];
      score[o] = s_sc[i];
      token[o] = tok_b[s_cand[i]];
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
  if (budget < 64)
    tree_build_kernel<1><<<dim3(static_cast<unsigned>(B)), 64, 0, stream>>>(logp, cand_tok, root_tok, D, K, budget,
                                                                           parent, token, depth, score, n_nodes);
  else
    tree_build_kernel<kBuildSlots><<<dim3(static_cast<unsigned>(B)), 64, 0, stream>>>(
        logp, cand_tok, root_tok, D, K, budget, parent, token, depth, score, n_nodes);
  return hipGetLastError();
}

}  // namespace tv
