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

hipError_t launch_rope_neox(void* x, bool bf16, const int32_t* pos, int n_seq, int64_t n_tok, int n_head, int d_r,
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
enum class AttnKernel : int { kValu = 0, kMfmaBf16 = 1, kMfmaF32 = 2, kMfmaBf16Q2 = 3, kMfmaF32Narrow = 4 };

// Workgroup geometry of the kernels: the bf16-cache matrix-core kernels (d_c
// 512, d_r 64; queries as two bf16 terms by default, or rounded to one on
// request), the fp32-cache matrix-core kernel (the same dims) and the
// vector-ALU kernel (every other supported shape).
constexpr int kValuRows = 16;     // query rows per workgroup
constexpr int kValuKeys = 32;     // kv rows per LDS tile
constexpr int kValuThreads = 256;
constexpr int kMfmaRows = 128;    // 4 waves x 32 query rows (bf16 queries)
constexpr int kQ2Rows = 64;       // 4 waves x 16 query rows (queries as hi + lo bf16 terms)
constexpr int kMfmaKeys = 32;
constexpr int kMfmaThreads = 256;
constexpr int kF32Rows = 64;      // 4 waves x 16 query rows
constexpr int kF32Keys = 32;
constexpr int kF32Threads = 256;
// The fp32 kernel's narrow form (uniform batches with few 64-row blocks): 32
// query rows, the unit's keys cut in two halves of 16-key tiles, one pair of
// waves per half.  Its plans count tiles of 32 keys, one 16-key tile per half.
constexpr int kF32NarrowRows = 32;
constexpr int kF32NarrowKeys = 16;
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
  long long n_slots;           // partial-result slots in the workspace
  long long merge_blocks;      // row blocks that need merging
  size_t ws_bytes;
  size_t ws_o_off, ws_m_off, ws_l_off;
};

struct AttnShape {
  int B, H, q_len, prefix_len, kv_len, d_c, d_r;
  bool kv_bf16;
  bool bf16_queries;  // bf16 cache at (512, 64): round the scaled queries to one bf16 term
  bool f32_wide;      // fp32 cache at (512, 64): the 64-row form at every size (no narrow form)
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
  const int4* merge_tab;  // the merge table after the records (MergeField order)
  int kv_stride;          // cache rows per request
  int n_nodes;            // rows of the caller's packed node arrays (the prep clamps the lengths to them)
  int* queue;             // kXcdQueues unit counters in the workspace (ragged batches; the prep kernel zeroes them)
};

// Records of a ragged batch, written by the prep kernel into the workspace
// (int32): [B][kReqFields] per request, then the request's two classes of
// units in launch order -- first unit cls_u0[2B] and class id cls_id[2B]
// (2b: the row blocks before the last, 2b + 1: the last row block) -- then
// kReqTotals totals.  A class is every (row block, kv piece) unit of those
// blocks; its pieces are equal but the last.  Classes run longest piece
// first.
enum ReqField : int {
  kReqQStart = 0,  // first node of the request in the packed node arrays
  kReqQLen,        // nodes (0 .. max_q_len)
  kReqPrefix,      // prefix rows
  kReqNBlk,        // row blocks (the last may be partial); 0 when q_len is 0
  kReqBSplit,      // kv pieces per row block before the last
  kReqBChunk,      // keys per such piece
  kReqTSplit,      // kv pieces of the last row block
  kReqTChunk,      // keys per such piece
  kReqSlot0,       // first partial-result slot
  kReqMerge0,      // first merged row block
  kReqFields
};
enum ReqTotal : int { kTotUnits = 0, kTotMerge, kTotChoice, kReqTotals };

__host__ __device__ inline const int32_t* req_cls_u0(const int32_t* rq, int B) { return rq + B * kReqFields; }
__host__ __device__ inline const int32_t* req_cls_id(const int32_t* rq, int B) { return rq + B * kReqFields + 2 * B; }
__host__ __device__ inline const int32_t* req_totals(const int32_t* rq, int B) {
  return rq + B * kReqFields + 4 * B;
}
__host__ __device__ inline size_t req_words(int B) { return static_cast<size_t>(B) * (kReqFields + 4) + kReqTotals; }
// After the records, at the next 16-byte boundary, the merge table: one entry
// per merged row block (a row block whose kv range was cut into pieces), in
// merged-block order.
enum MergeField : int {
  kMtSlot0 = 0,  // first slot of the block's pieces
  kMtSplit,      // pieces
  kMtRow0,       // first output row (packed node * H + head)
  kMtRows,       // rows of the block that exist
  kMtFields
};
__host__ __device__ inline size_t merge_table_word0(int B) { return (req_words(B) + 3) & ~static_cast<size_t>(3); }

// Planning of a ragged batch, in tiles of 32 keys (every kernel's tile).  A
// unit costs its tiles plus a set-up (tree masks, queries, first tile,
// output) of PlanCost::setup tiles.  Candidate plans cap the pieces of the
// row blocks before the last at cap_body tiles and those of the last block at
// cap_tail (at most kMaxTailSplit pieces, but never fewer than the other
// blocks get): the last blocks' shorter pieces fill the gaps the longer units
// leave.  Candidate 0 cuts nothing; the others take cap_body = T0 x {2/3, 1,
// 1/2, 1/4} and cap_tail = cap_body / {1, 2, 4, 8, 16} (at least
// PlanCost::min_piece tiles), T0 = the whole batch's cost per concurrent
// workgroup.
constexpr int kPlanTile = 32;
constexpr int kMaxTailSplit = 16;
struct PlanCost {
  int setup;            // tiles
  int min_piece;        // tiles
  int pieces_per_step;  // split pieces the merge pass combines per tile-step of the whole GPU
};
// The bf16 matrix-core and the VALU kernels: a unit's set-up is ~10 of their
// tile-steps; the fp32 matrix-core kernel's (its 32-row form: one 16-key tile
// per half per 32-key plan tile) is several times longer, and its set-up
// about one.
constexpr PlanCost kPlanCostDefault{10, 8, 16};
constexpr PlanCost kPlanCostF32{1, 1, 80};
constexpr int kPlanBody = 4, kPlanTail = 5;
constexpr int kPlanCands = 1 + kPlanBody * kPlanTail;

// Caps of candidate c given T0 (tiles); at most kPlanNoCut, which no request
// reaches (tiles < 2^26), so larger caps cut nothing either.
constexpr int kPlanNoCut = 1 << 30;
__host__ __device__ inline void plan_caps(long long T0, int c, int min_piece, int& cap_body, int& cap_tail) {
  if (c == 0) {
    cap_body = cap_tail = kPlanNoCut;
    return;
  }
  const int i = (c - 1) / kPlanTail, j = (c - 1) % kPlanTail;
  const long long num = i == 0 ? 2 : 1;
  const long long den = i == 0 ? 3 : (1 << (i - 1));
  long long body = (T0 < kPlanNoCut ? T0 : kPlanNoCut) * num / den;
  long long tail = body >> j;
  body = body < min_piece ? min_piece : (body > kPlanNoCut ? kPlanNoCut : body);
  tail = tail < min_piece ? min_piece : tail;
  cap_body = static_cast<int>(body);
  cap_tail = static_cast<int>(tail);
}

// One request's cut under caps (cap_body, cap_tail): pieces and tiles per
// piece for the row blocks before the last (n_body, c_body) and for the last
// (n_tail, c_tail).  1 <= tiles < 2^26.
struct ReqCut {
  int n_body, c_body, n_tail, c_tail;
};
__host__ __device__ inline ReqCut cut_request(int tiles, int cap_body, int cap_tail) {
  const unsigned t = static_cast<unsigned>(tiles);
  ReqCut r;
  unsigned n = (t + cap_body - 1u) / static_cast<unsigned>(cap_body);
  r.c_body = static_cast<int>((t + n - 1u) / n);
  r.n_body = static_cast<int>((t + r.c_body - 1u) / static_cast<unsigned>(r.c_body));
  n = (t + cap_tail - 1u) / static_cast<unsigned>(cap_tail);
  n = n < kMaxTailSplit ? n : kMaxTailSplit;
  n = n > static_cast<unsigned>(r.n_body) ? n : static_cast<unsigned>(r.n_body);
  r.c_tail = static_cast<int>((t + n - 1u) / n);
  r.n_tail = static_cast<int>((t + r.c_tail - 1u) / static_cast<unsigned>(r.c_tail));
  return r;
}

// Histogram bucket of a unit's cost (>= 1 tile): 4 buckets per octave.
__host__ __device__ inline int plan_bucket(int t) {
  const int e = 31 - __builtin_clz(static_cast<unsigned>(t));
  const int k = 4 * e + ((static_cast<unsigned>(t) << 2 >> e) & 3);
  return k < 63 ? k : 63;
}
__host__ __device__ inline long long plan_bucket_lo(int k) { return (static_cast<long long>(4 + (k & 3)) << (k >> 2)) >> 2; }

// Estimated span of a candidate, in tile-steps: the work per workgroup plus
// half the shortest unit (the last units fill gaps), at least the longest
// unit, and with more units than workgroups at least the longest unit plus the
// (M+1)-th longest (some workgroup runs two); plus the merge pass, one
// tile-step of the whole GPU per pieces_per_step pieces.
// k2 is the bucket of the (M+1)-th longest unit (the longest bucket k whose
// units and all longer ones number at least M + 1), or -1 when there are at
// most M units.
__host__ __device__ inline double plan_estimate(long long work, long long d_min, long long d_max, long long pieces,
                                                int pieces_per_step, int k2, long long M) {
  double e = static_cast<double>(work) / M + 0.5 * d_min;
  e = e > d_max ? e : static_cast<double>(d_max);
  if (k2 >= 0) {
    const double two = static_cast<double>(d_max + plan_bucket_lo(k2));
    e = e > two ? e : two;
  }
  return e + static_cast<double>(pieces) / pieces_per_step;
}

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
__host__ __device__ inline int find_request(const int32_t* rq, int B, int field, long long v) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (rq[mid * kReqFields + field] <= v) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Ragged batch: block x of the launch (an upper bound of units) -> its unit,
// or false past the batch's real total.  Units are numbered class by class in
// launch order (longest pieces first), so the longest units start first and
// the short ones fill in at the end.  Within the class of the blocks before
// the last, unit = piece * (blocks) + block: the row blocks reading one kv
// piece are neighbours.  Runs of kDealGroup consecutive units go to one XCD
// (workgroup x runs on XCD x % 8), so neighbours share that XCD's L2.
constexpr int kDealGroup = 8;
__host__ __device__ inline bool decode_unit_ragged(const AttnArgs& a, long long x, Unit& w) {
  const int32_t* rq = a.req;
  const int32_t* u0 = req_cls_u0(rq, a.B);
  const long long total = req_totals(rq, a.B)[kTotUnits];
  if (x >= total) return false;
  {
    constexpr int kXcds = 8, kGroup = kDealGroup;
    const long long whole = total / (kXcds * kGroup) * (kXcds * kGroup);
    if (x < whole) {
      const long long k = x % kXcds, j = x / kXcds;
      x = (j / kGroup) * (kXcds * kGroup) + k * kGroup + j % kGroup;
    }
  }
  int lo = 0, hi = 2 * a.B - 1;  // last class whose first unit is <= x (empty classes come last)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (u0[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  const int id = req_cls_id(rq, a.B)[lo];
  const int local = static_cast<int>(x - u0[lo]);
  const int b = id >> 1;
  const int32_t* r = rq + b * kReqFields;
  const int n_before = r[kReqNBlk] - 1;
  const int bsplit = r[kReqBSplit];
  int chunk;
  if ((id & 1) == 0) {
    w.rb = local % n_before;
    w.split = local / n_before;
    chunk = r[kReqBChunk];
    w.slot = bsplit > 1 ? static_cast<long long>(r[kReqSlot0]) + static_cast<long long>(w.rb) * bsplit + w.split : -1;
  } else {
    w.rb = n_before;
    w.split = local;
    chunk = r[kReqTChunk];
    const long long before = bsplit > 1 ? static_cast<long long>(n_before) * bsplit : 0;
    w.slot = r[kReqTSplit] > 1 ? r[kReqSlot0] + before + local : -1;
  }
  w.b = b;
  w.q_len = r[kReqQLen];
  w.P = r[kReqPrefix];
  w.R = w.q_len * a.H;
  w.kv_len = w.P + w.q_len;
  w.k_begin = w.split * chunk;
  w.k_end = w.kv_len < w.k_begin + chunk ? w.kv_len : w.k_begin + chunk;
  w.row0 = static_cast<long long>(r[kReqQStart]) * a.H;
  w.par0 = r[kReqQStart];
  w.kv_row0 = static_cast<long long>(b) * a.kv_stride;
  return true;
}

// Ragged batches run a persistent grid: one workgroup per CU (two for the
// vector kernel) takes launch slots from its XCD's counter, slot x = xcd + 8 j
// for the j-th take on that XCD, so the units reaching each XCD are the ones a
// grid of one workgroup per unit would deal it (runs of kDealGroup
// neighbours sharing its L2), handed out as its CUs free up.  The counters sit
// after the merge table in the workspace and the prep kernel zeroes them.
// The grid (at least 256 workgroups) gives every counter workgroups.
constexpr int kXcdQueues = 8;
__host__ __device__ inline size_t queue_word0(int B, long long max_merges) {
  return merge_table_word0(B) + static_cast<size_t>(max_merges) * kMtFields;
}

// Next unit of this workgroup in a ragged batch, or false when its XCD's
// slots are used up (uniform across the workgroup).  The leading barrier
// keeps the previous unit's LDS reads ahead of the next unit's writes; the
// slot goes through readfirstlane so the unit's fields stay scalar.
__device__ __forceinline__ bool next_unit_ragged(const AttnArgs& a, Unit& w) {
  __shared__ int s_slot;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int k = static_cast<int>(blockIdx.x % kXcdQueues);
    s_slot = k + kXcdQueues * atomicAdd(a.queue + k, 1);
  }
  __syncthreads();
  return decode_unit_ragged(a, __builtin_amdgcn_readfirstlane(s_slot), w);
}

// The loop of a persistent ragged workgroup: body(a, w) for each unit it
// takes.  The kernels using it take one argument, an AttnArgs by value, which
// therefore starts the kernel-argument segment; the segment pointer passes
// through an empty asm statement at each unit, so the compiler reloads the
// arguments a unit needs where it needs them instead of holding every one in
// registers across the whole loop (which spills).
template <typename Body>
__device__ __forceinline__ void for_each_ragged_unit(Body body) {
  using KernArgs = const __attribute__((address_space(4))) AttnArgs*;
  KernArgs pa = (KernArgs)__builtin_amdgcn_kernarg_segment_ptr();
  Unit w;
  for (;;) {
    asm volatile("" : "+s"(pa));
    const AttnArgs& a = *(const AttnArgs*)pa;
    if (!next_unit_ragged(a, w)) return;
    body(a, w);
  }
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
hipError_t launch_attn_mfma_q2(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_mfma_f32(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream);

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

// build_ancestors for a workgroup of at least q_len threads whose thread t
// already holds parent[t] (any value for t >= q_len): the parent loads can be
// issued early, ahead of other loads, and waited for here.  Ends with a barrier.
__device__ __forceinline__ void build_ancestors_loaded(int par_t, int q_len, int* s_par,
                                                       unsigned long long* s_anc) {
  if (static_cast<int>(threadIdx.x) < q_len) s_par[threadIdx.x] = clamp_parent(par_t, threadIdx.x);
  __syncthreads();
  for (int i = threadIdx.x; i < q_len; i += blockDim.x) {
    unsigned long long w[kAncWords] = {};
    for (int n = i; n >= 0; n = s_par[n]) {
      const unsigned long long bit = 1ull << (n & 63);
#pragma unroll
      for (int k = 0; k < kAncWords; ++k) w[k] |= (n >> 6) == k ? bit : 0ull;
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

// 1 if kv key `key` is visible from tree node `node` (0 <= node < kMaxQ): the
// key lies below the unit's range end k_end and is a prefix key (key < P) or
// the node or one of its ancestors.  Written straight-line on purpose: every
// lane reads an ancestor word at a clamped index and the answer is built with
// integer and/or, with no short-circuit test.  (With the form
// `key < k_end && (key < P || anc_bit(...))` the device compiler once emitted
// code that dropped a visible tree key.)
__device__ __forceinline__ unsigned key_visible(const unsigned long long* s_anc, int node, int key, int P,
                                                int k_end) {
  const int rel = min(max(key - P, 0), kMaxQ - 1);
  const unsigned long long word = s_anc[node * kAncWords + (rel >> 6)];
  const unsigned in_range = key < k_end ? 1u : 0u;
  const unsigned in_prefix = key < P ? 1u : 0u;
  const unsigned anc = static_cast<unsigned>((word >> (rel & 63)) & 1ull);
  return in_range & (in_prefix | anc);
}

}  // namespace tv
