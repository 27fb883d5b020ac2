// Internal launch interface between the C ABI (tv_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tv_device.h"

namespace tv {

constexpr int kMaxQ = 256;     // tree nodes per request
constexpr int kAncWords = kMaxQ / 64;  // 64-bit ancestor words per node
constexpr int kMaxHalf = 64;  // d_r <= 128

// inv_freq[k] = 1 / theta^(2k/d_r), computed on the host in float64 and passed
// by value so every thread of a launch uses the same table.
struct RopeFreq {
  double inv_freq[kMaxHalf];
};

hipError_t launch_rope_neox(void* x, bool bf16, const int32_t* pos, int n_seq, int n_tok, int n_head, int d_r,
                            int64_t seq_stride, int64_t tok_stride, int64_t pos_seq_stride, const RopeFreq& f,
                            hipStream_t stream);
hipError_t launch_tree_positions(const int32_t* parent, int B, int q_len, int prefix_len, int32_t* pos,
                                 hipStream_t stream);
hipError_t launch_tree_rope(float* q_rope, void* k_rope, bool bf16, const int32_t* parent, int B, int q_len, int H,
                            int d_r, int prefix_len, const RopeFreq& f, hipStream_t stream);
// The same for a ragged batch, from the request records the prep kernel wrote
// (launch_ragged_prep).
hipError_t launch_tree_rope_ragged(float* q_rope, void* k_rope, bool bf16, const int32_t* parent, const int32_t* req,
                                   int B, int max_q, int H, int d_r, int kv_stride, const RopeFreq& f,
                                   hipStream_t stream);

// ---------------------------------------------------------------------------
// Attention
// ---------------------------------------------------------------------------
enum class AttnKernel : int { kValu = 0, kMfmaBf16 = 1 };

// Workgroup geometry of the two kernel families.
constexpr int kValuRows = 16;     // query rows per workgroup
constexpr int kValuKeys = 32;     // kv rows per LDS tile
constexpr int kValuThreads = 256;
constexpr int kMfmaRows = 128;    // 4 waves x 32 query rows
constexpr int kMfmaKeys = 32;
constexpr int kMfmaThreads = 256;
// Tiles of a unit that hold tree keys or the unit's range end: at most
// q_len / 32 + 2.
constexpr int kMaxBoundaryTiles = kMaxQ / kMfmaKeys + 2;

// How one tv_verify_attn call is cut into workgroups ("units").  A pure
// function of the shapes (never of the device), so the workspace size can be
// asked for ahead.
//
// The R = q_len * H query rows of a tree are cut into row blocks of
// rows_per_block; every row block but possibly the last is full.  Full blocks
// are cut into split_full kv ranges of chunk_full rows, the partial last block
// into split_tail ranges of chunk_tail rows (a short last round of the grid is
// then filled by short units).  Units of full blocks come first in launch
// order, ordered by tree, then kv range, then row block.  A row block cut into
// more than one range writes partial results to the workspace ("slots",
// numbered by tree, row block, range), combined afterwards by the merge pass.
struct AttnPlan {
  AttnKernel kernel;
  int rows_per_block;
  int keys_per_tile;
  int n_rb;        // row blocks per tree
  int full_rb;     // full row blocks per tree (n_rb or n_rb - 1)
  int split_full, chunk_full;
  int split_tail, chunk_tail;  // meaningful when full_rb < n_rb
  long long units;
  long long target;            // workgroups that run at once (ragged plans)
  bool tail_pieces;            // ragged: cut the partial last row blocks into pieces on the device
  long long n_slots;           // partial-result slots in the workspace
  long long merge_blocks;      // row blocks that need merging
  size_t ws_bytes;
  size_t ws_o_off, ws_m_off, ws_l_off;
};

struct AttnShape {
  int B, H, q_len, prefix_len, kv_len, d_c, d_r;
  bool kv_bf16;
};

AttnPlan plan_attention(const AttnShape& s);
// Ragged batch: s.q_len is the bound max_q_len and s.kv_len the cache stride.
AttnPlan plan_attention_ragged(const AttnShape& s);

struct AttnArgs {
  const float* q_lat;
  const float* q_rope;
  const void* c_kv;
  const void* k_rope;
  const int32_t* parent;
  float* out;
  float* lse;
  float* ws_o;  // [n_slots][rows_per_block][d_c]  (normalised partial outputs)
  float* ws_m;  // [n_slots][rows_per_block]       (row max, natural-log units)
  float* ws_l;  // [n_slots][rows_per_block]       (sum of exp(s - m))
  int B, H, q_len, prefix_len, kv_len, R;
  int rows_per_block, n_rb, full_rb, split_full, chunk_full, split_tail, chunk_tail;
  float sm_scale;
  // Ragged batches (per-request lengths, on the device): req points at the
  // request records the prep kernel wrote (null for a uniform batch).
  const int32_t* req;
  int kv_stride;  // cache rows per request
  int chunk;      // keys per kv piece
};

// Request record of a ragged batch: [B][kReqFields] int32, then kReqTotals
// totals (units of full row blocks, all units, merged blocks).  Units of full
// row blocks come first in launch order, request by request; the pieces of
// the partial last row blocks after them.
enum ReqField : int {
  kReqQStart = 0,  // first node of the request in the packed node arrays
  kReqQLen,        // nodes (0 .. max_q_len)
  kReqPrefix,      // prefix rows
  kReqNFull,       // full row blocks
  kReqSplit,       // kv pieces per full row block
  kReqTSplit,      // kv pieces of the partial last row block (0: no such block)
  kReqTChunk,      // keys per piece of the partial block
  kReqFull0,       // first unit of the full blocks
  kReqTail0,       // first unit of the partial block, counted from the end of all full-block units
  kReqSlot0,       // first partial-result slot
  kReqMerge0,      // first merged row block
  kReqFields
};
constexpr int kReqTotals = 3;
// Most pieces the partial last row block of a request is cut into (to fill
// the last round of workgroups).
constexpr int kMaxTailSplit = 16;

// The work of one unit (one workgroup), with the shape of its request.
struct Unit {
  int b, rb, split;
  int k_begin, k_end;
  long long slot;  // partial-result slot, or -1 when the row block is not split
  int q_len, P, R, kv_len;
  long long row0;     // packed (node, head) row of the request's node 0
  long long par0;     // offset of the request's parent array
  long long kv_row0;  // first cache row of the request
};

__device__ __forceinline__ Unit decode_unit(const AttnArgs& a, long long u) {
  Unit w;
  const long long units_full = static_cast<long long>(a.B) * a.full_rb * a.split_full;
  int chunk;
  if (u < units_full) {
    // Tree, then kv range, then row block: the row blocks reading one kv range
    // are neighbours in launch order (and so mostly share an XCD's L2).
    w.rb = static_cast<int>(u % a.full_rb);
    const long long t = u / a.full_rb;
    w.split = static_cast<int>(t % a.split_full);
    w.b = static_cast<int>(t / a.split_full);
    chunk = a.chunk_full;
    w.slot = a.split_full > 1 ? (static_cast<long long>(w.b) * a.full_rb + w.rb) * a.split_full + w.split : -1;
  } else {
    const long long u2 = u - units_full;
    w.split = static_cast<int>(u2 % a.split_tail);
    w.b = static_cast<int>(u2 / a.split_tail);
    w.rb = a.n_rb - 1;
    chunk = a.chunk_tail;
    const long long base = a.split_full > 1 ? units_full : 0;
    w.slot = a.split_tail > 1 ? base + static_cast<long long>(w.b) * a.split_tail + w.split : -1;
  }
  w.k_begin = w.split * chunk;
  w.k_end = min(a.kv_len, w.k_begin + chunk);
  w.q_len = a.q_len;
  w.P = a.prefix_len;
  w.R = a.R;
  w.kv_len = a.kv_len;
  w.row0 = static_cast<long long>(w.b) * a.R;
  w.par0 = static_cast<long long>(w.b) * a.q_len;
  w.kv_row0 = static_cast<long long>(w.b) * a.kv_len;
  return w;
}

// Workgroup x of a launch runs on XCD x % 8 (the hardware deals workgroups to
// the 8 XCDs in turn), and each XCD has its own L2.  Units are numbered tree by
// tree, full row blocks first, then the pieces of the split tail blocks; this
// order gives each XCD a contiguous run of full-block units and then a
// contiguous run of pieces, so the workgroups sharing a tree's latent rows
// mostly share one L2.  It is a bijection on [0, units): within each of the
// two ranges the first multiple of 8 is dealt XCD by XCD, the rest in order.
//
// When every XCD has at least two rounds of full-block units and half a round
// of pieces, half of its CUs start with pieces instead (an XCD's j-th
// workgroup: full units 0..15, then pieces 0..15, then the other full units,
// then the other pieces).  The two halves then reach their unit boundaries at
// different times, so the bursts of query loads and output stores at those
// boundaries do not all hit HBM at once; the last workgroup still ends at the
// same time.
__device__ __forceinline__ long long unit_of_block(const AttnArgs& a, long long x) {
  constexpr int kXcds = 8;
  constexpr int kHalfXcd = 16;  // half of one XCD's 32 CUs
  const long long units_full = static_cast<long long>(a.B) * a.full_rb * a.split_full;
  const long long units = units_full + (a.full_rb < a.n_rb ? static_cast<long long>(a.B) * a.split_tail : 0);
  const long long n_f = units_full / kXcds;           // full-block units per XCD
  const long long n_p = (units - units_full) / kXcds;  // pieces per XCD
  if (units_full % kXcds == 0 && (units - units_full) % kXcds == 0 && n_f >= 2 * kHalfXcd && n_p >= kHalfXcd) {
    const long long k = x % kXcds;
    const long long j = x / kXcds;
    if (j < kHalfXcd) return k * n_f + j;
    if (j < 2 * kHalfXcd) return units_full + k * n_p + (j - kHalfXcd);
    if (j < n_f + kHalfXcd) return k * n_f + (j - kHalfXcd);
    return units_full + k * n_p + (j - n_f);
  }
  const long long f8 = units_full / kXcds * kXcds;
  if (x < f8) return (x % kXcds) * (f8 / kXcds) + x / kXcds;
  const long long p = x - f8;
  const long long r8 = (units - f8) / kXcds * kXcds;
  if (p < r8) return f8 + (p % kXcds) * (r8 / kXcds) + p / kXcds;
  return x;
}

// Last request whose first entry in column `field` is <= v (requests with
// nothing to do share that entry with the next one, so the search lands on the
// request that owns v).
__device__ __forceinline__ int find_request(const int32_t* rq, int B, int field, long long v) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (rq[mid * kReqFields + field] <= v) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Ragged batch: block x of the launch (an upper bound of units) -> its unit,
// or false past the batch's real total.  The real units are dealt to the XCDs
// as unit_of_block deals a uniform batch's (full-block units, then pieces).
__device__ __forceinline__ bool decode_unit_ragged(const AttnArgs& a, long long x, Unit& w) {
  const int32_t* rq = a.req;
  const long long u_full = rq[a.B * kReqFields];
  const long long total = rq[a.B * kReqFields + 1];
  if (x >= total) return false;
  constexpr int kXcds = 8;
  const long long f8 = u_full / kXcds * kXcds;
  long long u = x;
  if (x < f8) {
    u = (x % kXcds) * (f8 / kXcds) + x / kXcds;
  } else {
    const long long p = x - f8;
    const long long r8 = (total - f8) / kXcds * kXcds;
    if (p < r8) u = f8 + (p % kXcds) * (r8 / kXcds) + p / kXcds;
  }
  int b, chunk;
  const int32_t* r;
  if (u < u_full) {
    b = find_request(rq, a.B, kReqFull0, u);
    r = rq + b * kReqFields;
    const int local = static_cast<int>(u - r[kReqFull0]);
    const int n_full = r[kReqNFull];
    const int n_split = r[kReqSplit];
    w.rb = local % n_full;
    w.split = local / n_full;
    chunk = a.chunk;
    w.slot = n_split > 1 ? static_cast<long long>(r[kReqSlot0]) + static_cast<long long>(w.rb) * n_split + w.split
                         : -1;
  } else {
    b = find_request(rq, a.B, kReqTail0, u - u_full);
    r = rq + b * kReqFields;
    const int piece = static_cast<int>(u - u_full - r[kReqTail0]);
    const int n_split = r[kReqSplit];
    const long long full_slots = n_split > 1 ? static_cast<long long>(r[kReqNFull]) * n_split : 0;
    w.rb = r[kReqNFull];
    w.split = piece;
    chunk = r[kReqTChunk];
    w.slot = r[kReqTSplit] > 1 ? r[kReqSlot0] + full_slots + piece : -1;
  }
  w.b = b;
  w.q_len = r[kReqQLen];
  w.P = r[kReqPrefix];
  w.R = w.q_len * a.H;
  w.kv_len = w.P + w.q_len;
  w.k_begin = w.split * chunk;
  w.k_end = min(w.kv_len, w.k_begin + chunk);
  w.row0 = static_cast<long long>(r[kReqQStart]) * a.H;
  w.par0 = r[kReqQStart];
  w.kv_row0 = static_cast<long long>(b) * a.kv_stride;
  return true;
}

hipError_t launch_attention(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream);
// Request records of a ragged batch (lengths prefix_len[B], q_len[B] in device
// memory) into a.req; then launch_attention runs the batch.
hipError_t launch_ragged_prep(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, const int32_t* prefix_len,
                              const int32_t* q_len, hipStream_t stream);

// The steps after verify (accept.hip).
hipError_t launch_argmax_rows(const void* logits, bool bf16, bool vec, int64_t n_rows, int vocab, int32_t* out,
                              hipStream_t stream);
hipError_t launch_tree_accept(const int32_t* parent, const int32_t* draft, const int32_t* target, int B, int q_len,
                              int32_t* path, int32_t* accept_len, int32_t* bonus, hipStream_t stream);
hipError_t launch_kv_compact(void* c_kv, void* k_rope, int elem_bytes, const int32_t* path, const int32_t* accept_len,
                             int prefix_len, int B, int kv_len, int q_len, int d_c, int d_r, hipStream_t stream);
// The step before verify (tree_build.hip).
hipError_t launch_tree_build(const float* logp, const int32_t* cand_tok, const int32_t* root_tok, int B, int D, int K,
                             int budget, int32_t* parent, int32_t* token, int32_t* depth, float* score,
                             int32_t* n_nodes, hipStream_t stream);

// Kernel launchers (one per kernel family).
hipError_t launch_attn_valu(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_mfma_bf16(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream);

// Ancestor bit masks of one tree: bit m % 64 of word s_anc[i * kAncWords +
// m / 64] is set iff node m is node i or one of its ancestors (words past the
// tree's nodes stay 0).  Thread i walks its own path (<= q_len steps: a parent
// outside [0, i) ends it).  Ends with a barrier.
__device__ __forceinline__ void build_ancestors(const int32_t* __restrict__ parent_b, int q_len, int* s_par,
                                                unsigned long long* s_anc) {
  for (int i = threadIdx.x; i < q_len; i += blockDim.x) s_par[i] = clamp_parent(parent_b[i], i);
  __syncthreads();
  for (int i = threadIdx.x; i < q_len; i += blockDim.x) {
    unsigned long long w[kAncWords] = {};
    for (int n = i; n >= 0; n = s_par[n]) {
      const unsigned long long bit = 1ull << (n & 63);
#pragma unroll
      for (int k = 0; k < kAncWords; ++k) w[k] |= (n >> 6) == k ? bit : 0ull;  // static indices: no scratch
    }
#pragma unroll
    for (int k = 0; k < kAncWords; ++k) s_anc[i * kAncWords + k] = w[k];
  }
  __syncthreads();
}

// Whether tree key rel (0 <= rel < q_len) is visible from node `node`.
__device__ __forceinline__ bool anc_bit(const unsigned long long* s_anc, int node, int rel) {
  return ((s_anc[node * kAncWords + (rel >> 6)] >> (rel & 63)) & 1ull) != 0ull;
}

}  // namespace tv
