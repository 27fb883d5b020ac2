// Launch planning for tree-verify attention, the split-kv merge pass, and the
// choice of kernel.
//
// Planning: the R = q_len * H rows of a tree form row blocks; each (tree, row
// block, kv range) is one workgroup.  When there are too few row blocks to
// fill the GPU, every block's kv range is cut into splits; when only the last,
// partial row block of each tree would spill into an extra, mostly idle round
// of workgroups, only those blocks are cut, so their pieces fill that round.
// Split pieces write (normalised partial output, row max, row sum) to the
// caller's workspace and the merge pass combines them by log-sum-exp weights.
#include "tv_kernels.h"

namespace tv {

namespace {
constexpr int kNumCU = 256;          // MI355X; fixed so plans depend on shapes only
constexpr int kMinKeysPerSplit = 256;
// The fp32 matrix-core kernel's tile-step is ~6x the bf16 kernel's (the same
// flops at a sixteenth of the rate, over half the rows), so its set-up is worth
// about one tile and pieces may be as short as one tile.
constexpr int kF32SetupTiles = 1;
constexpr int kF32MinKeysPerSplit = kF32Keys / 2;  // pieces still round up to whole tiles

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int ceil_div(long long a, long long b) { return static_cast<int>((a + b - 1) / b); }

// Cut kv_len rows into at most `want` ranges of a whole number of tiles.
void cut(int kv_len, int want, int tile, int& n, int& chunk, int min_keys = kMinKeysPerSplit) {
  const int max_split = kv_len / min_keys > 1 ? kv_len / min_keys : 1;
  n = want < 1 ? 1 : (want > max_split ? max_split : want);
  chunk = ceil_div(kv_len, n);
  chunk = ceil_div(chunk, tile) * tile;
  n = ceil_div(kv_len, chunk);
}

// Splits for `blocks` row blocks over kv_len keys when they alone cannot fill
// `slots` concurrent workgroups: the count that minimises the launch's time,
// modelled as rounds of workgroups x (tiles per piece + a unit's fixed set-up
// in tile-steps); ties go to fewer splits (less merging).  Rounding the count
// up instead (blocks x splits just above slots) would add a nearly empty
// second round.
void cut_for_blocks(int kv_len, long long blocks, long long slots, int tile, int setup_tiles, int& n, int& chunk,
                    int min_keys = kMinKeysPerSplit) {
  const int max_split = kv_len / min_keys > 1 ? kv_len / min_keys : 1;
  long long best_cost = -1;
  int best = 1;
  for (int want = 1; want <= max_split; ++want) {
    int sn, sc;
    cut(kv_len, want, tile, sn, sc, min_keys);
    if (sn != want) continue;  // an equivalent cut was already counted
    const long long rounds = (blocks * sn + slots - 1) / slots;
    const long long cost = rounds * (sc / tile + setup_tiles);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = sn;
    }
  }
  cut(kv_len, best, tile, n, chunk, min_keys);
}
}  // namespace

// Kernel of a shape: the bf16-cache matrix-core kernels at (512, 64) -- the
// queries as two bf16 terms unless bf16_queries asks for one -- the fp32-cache
// matrix-core kernel at (512, 64), the vector-ALU kernel otherwise.
void choose_kernel(const AttnShape& s, AttnPlan& p) {
  const bool mfma = s.kv_bf16 && s.d_c == 512 && s.d_r == 64;
  const bool f32 = !s.kv_bf16 && s.d_c == 512 && s.d_r == 64;
  p.kernel = mfma ? (s.bf16_queries ? AttnKernel::kMfmaBf16 : AttnKernel::kMfmaBf16Q2)
                  : f32 ? AttnKernel::kMfmaF32 : AttnKernel::kValu;
  p.rows_per_block = p.kernel == AttnKernel::kMfmaBf16   ? kMfmaRows
                     : p.kernel == AttnKernel::kMfmaBf16Q2 ? kQ2Rows
                     : f32                                 ? kF32Rows
                                                           : kValuRows;
  p.keys_per_tile = mfma ? kMfmaKeys : kValuKeys;
}

AttnPlan plan_attention(const AttnShape& s) {
  AttnPlan p{};
  choose_kernel(s, p);
  const bool mfma = p.kernel == AttnKernel::kMfmaBf16 || p.kernel == AttnKernel::kMfmaBf16Q2;
  const int R = s.q_len * s.H;
  if (p.kernel == AttnKernel::kMfmaF32 && !s.f32_wide &&
      static_cast<long long>(s.B) * ceil_div(R, kF32Rows) <= kNumCU / 2) {
    // At most half a round of 64-row blocks: the narrow form (32-row blocks,
    // each unit's keys in two halves) gives every kv piece twice the
    // workgroups, pads fewer rows, and its pieces' partial results are half
    // the wide form's for the same work per workgroup.  With more blocks the
    // wide form reads each key tile for twice the rows.
    p.kernel = AttnKernel::kMfmaF32Narrow;
    p.rows_per_block = kF32NarrowRows;
  }
  const bool f32 = p.kernel == AttnKernel::kMfmaF32 || p.kernel == AttnKernel::kMfmaF32Narrow;
  p.n_rb = ceil_div(R, p.rows_per_block);
  bool has_tail = (R % p.rows_per_block) != 0;
  // Workgroups resident per CU: a matrix-core kernel takes a whole CU; the VALU
  // one about one, so aim at two rounds for it.
  const long long target = mfma || f32 ? kNumCU : 2 * kNumCU;

  const long long blocks = static_cast<long long>(s.B) * p.n_rb;
  if (!has_tail && p.n_rb > 1 && blocks > target && blocks % target != 0) {
    // Whole blocks only, but the last round of workgroups would be partly
    // idle: treat each tree's last block as the tail to cut into pieces when
    // that shortens the launch (in rounds of whole-block units; pieces that
    // fit beside the last round's full units cost nothing, an extra round of
    // pieces 1 / split; plus a tenth of a round for the merge).
    const long long full_units = static_cast<long long>(s.B) * (p.n_rb - 1);
    const long long rem = full_units % target;
    long long free_slots = target - rem;
    if (free_slots < s.B) free_slots += target;
    int n, chunk;
    cut(s.kv_len, static_cast<int>(free_slots / s.B), p.keys_per_tile, n, chunk,
        f32 ? kF32MinKeysPerSplit : kMinKeysPerSplit);
    const bool fits = rem != 0 && static_cast<long long>(s.B) * n <= target - rem;
    const double t_cut = static_cast<double>((full_units + target - 1) / target) + (fits ? 0.0 : 1.0 / n) + 0.1;
    const double t_whole = static_cast<double>((blocks + target - 1) / target);
    if (n > 1 && t_cut < t_whole) has_tail = true;
  }
  p.full_rb = has_tail ? p.n_rb - 1 : p.n_rb;
  if (blocks < target) {
    // Too few row blocks: cut every block's kv range.  A unit's set-up (tree
    // masks, queries, first tile, output) costs about ten tile-steps.
    cut_for_blocks(s.kv_len, blocks, target, p.keys_per_tile, f32 ? kF32SetupTiles : 10, p.split_full, p.chunk_full,
                   f32 ? kF32MinKeysPerSplit : kMinKeysPerSplit);
    p.split_tail = p.split_full;
    p.chunk_tail = p.chunk_full;
  } else {
    cut(s.kv_len, 1, p.keys_per_tile, p.split_full, p.chunk_full);
    p.split_tail = p.split_full;
    p.chunk_tail = p.chunk_full;
    if (has_tail) {
      // Fill the last round with pieces of the partial blocks.
      const long long full_units = static_cast<long long>(s.B) * p.full_rb;
      long long free_slots = target - full_units % target;
      const long long tails = s.B;
      if (free_slots < tails) free_slots += target;
      cut(s.kv_len, static_cast<int>(free_slots / tails), p.keys_per_tile, p.split_tail, p.chunk_tail,
          f32 ? kF32MinKeysPerSplit : kMinKeysPerSplit);
    }
  }
  if (p.full_rb == 0) {  // only a partial block per tree
    p.split_full = 1;
    p.chunk_full = s.kv_len;
  }
  const long long units_full = static_cast<long long>(s.B) * p.full_rb * p.split_full;
  const long long units_tail = has_tail ? static_cast<long long>(s.B) * p.split_tail : 0;
  p.units = units_full + units_tail;
  p.n_slots = (p.split_full > 1 ? units_full : 0) + (p.split_tail > 1 ? units_tail : 0);
  p.merge_blocks = (p.split_full > 1 ? static_cast<long long>(s.B) * p.full_rb : 0) +
                   (has_tail && p.split_tail > 1 ? s.B : 0);
  p.ws_bytes = 0;
  if (p.n_slots > 0) {
    const size_t rows = static_cast<size_t>(p.n_slots) * p.rows_per_block;
    p.ws_o_off = 0;
    p.ws_m_off = align256(rows * s.d_c * sizeof(float));
    p.ws_l_off = p.ws_m_off + align256(rows * sizeof(float));
    p.ws_bytes = p.ws_l_off + align256(rows * sizeof(float));
  }
  return p;
}

// Ragged batch: launch sizes from the bounds (B requests of at most max_q_len
// nodes over at most kv_stride keys); the prep kernel makes the plan from the
// device lengths.  Partial-result slots are capped at max(2 target,
// min(kMaxTailSplit B, 4 target)) (a candidate plan needing more is not
// taken; cutting nothing needs none; more than four rounds of pieces never
// pays).  Every unit is a row block whole or a split piece, so units <= B n_rb
// + slots; merged blocks <= min(B n_rb, slots / 2).
AttnPlan plan_attention_ragged(const AttnShape& s) {
  AttnPlan p{};
  choose_kernel(s, p);
  if (p.kernel == AttnKernel::kMfmaF32 &&
      static_cast<long long>(s.B) * ceil_div(static_cast<long long>(s.q_len) * s.H, kF32Rows) <= kNumCU / 2) {
    // The uniform batches' rule, on the bounds: at most half a round of
    // 64-row blocks runs on the 32-row form.  (Measured on ragged fp32
    // batches: 64 requests x 8 heads x <= 8 nodes, 1.07 -> 0.87 ms; with 16
    // or 8 requests x 64 heads x <= 33 nodes the 64-row form is 20-30 %
    // faster, its tiles serving twice the rows.)
    p.kernel = AttnKernel::kMfmaF32Narrow;
    p.rows_per_block = kF32NarrowRows;
  }
  const bool mfma = p.kernel == AttnKernel::kMfmaBf16 || p.kernel == AttnKernel::kMfmaBf16Q2;
  const bool f32 = p.kernel == AttnKernel::kMfmaF32 || p.kernel == AttnKernel::kMfmaF32Narrow;
  p.n_rb = ceil_div(static_cast<long long>(s.q_len) * s.H, p.rows_per_block);
  p.full_rb = p.n_rb;
  p.split_full = p.split_tail = 1;
  p.chunk_full = p.chunk_tail = s.kv_len;
  p.target = mfma || f32 ? kNumCU : 2 * kNumCU;
  const long long blocks = static_cast<long long>(s.B) * p.n_rb;
  long long cap = static_cast<long long>(s.B) * kMaxTailSplit;
  cap = cap < 4 * p.target ? cap : 4 * p.target;
  p.n_slots = 2 * p.target > cap ? 2 * p.target : cap;
  p.units = blocks + p.n_slots;
  p.merge_blocks = blocks < p.n_slots / 2 ? blocks : p.n_slots / 2;
  const size_t rec = align256((queue_word0(s.B, p.merge_blocks) + kXcdQueues) * sizeof(int32_t));
  p.ws_o_off = rec;
  p.ws_m_off = rec + align256(static_cast<size_t>(p.n_slots) * p.rows_per_block * s.d_c * sizeof(float));
  p.ws_l_off = p.ws_m_off + align256(static_cast<size_t>(p.n_slots) * p.rows_per_block * sizeof(float));
  p.ws_bytes = p.ws_l_off + align256(static_cast<size_t>(p.n_slots) * p.rows_per_block * sizeof(float));
  return p;
}

namespace {

static_assert(kMfmaKeys == kPlanTile && kValuKeys == kPlanTile && kF32Keys == kPlanTile &&
                  2 * kF32NarrowKeys == kPlanTile,
              "plans count tiles of 32 keys for every kernel");

// Lengths of request b as the prep kernel clamped them (into the bounds and
// the caller's packed node rows) and wrote them into its record; its row
// blocks and tiles.
struct ReqLen {
  int q, P, nblk, tiles;
};
__device__ __forceinline__ ReqLen req_len(const int32_t* rq, int b, int H, int rpb) {
  ReqLen r;
  r.q = rq[b * kReqFields + kReqQLen];
  r.P = rq[b * kReqFields + kReqPrefix];
  r.nblk = (r.q * H + rpb - 1) / rpb;
  r.tiles = (r.P + r.q + kPlanTile - 1) / kPlanTile;
  return r;
}

// The same from the clamped lengths (q, P) of the request.
__device__ __forceinline__ ReqLen req_len_of(int q, int P, int H, int rpb) {
  ReqLen r;
  r.q = q;
  r.P = P;
  r.nblk = (q * H + rpb - 1) / rpb;
  r.tiles = (P + q + kPlanTile - 1) / kPlanTile;
  return r;
}

constexpr int kPrepThreads = 1024;
constexpr int kPrepLdsReqs = 2048;  // requests whose clamped lengths the prep kernel keeps in LDS
constexpr int kSortMax = 4096;  // classes sorted in LDS (B <= 2048); larger batches keep request order
constexpr int kRankSortMax = 256;  // up to this many classes by rank (two barriers), more by a bitonic network

// Sum over the workgroup (ends with every thread holding the total).
__device__ long long block_sum(long long v, long long* s_part) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_part[wave] = v;
  __syncthreads();
  long long t = 0;
  for (int i = 0; i < kPrepThreads / 64; ++i) t += s_part[i];
  return t;
}

// Exclusive scan over the workgroup of one value per thread (wave scans by
// shuffles, then the 16 wave totals); returns this thread's offset; *total
// gets the sum.
__device__ int block_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  __syncthreads();
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < kPrepThreads / 64; ++w) {
    const int sw = s_wave[w];
    before += w < wave ? sw : 0;
    tot += sw;
  }
  *total = tot;
  return before + x - v;
}

// The records of a ragged batch (one workgroup of 1024 threads):
//  1. T0 = sum over requests of row blocks x (tiles + set-up) / target;
//  2. for every candidate cut (plan_caps): units, pieces, shortest and
//     longest unit and a histogram of unit costs; the candidate with the
//     least plan_estimate among those within the slot budget is taken;
//  3. the requests' two classes are sorted by piece length, longest first
//     (ties by class id), and numbered in that order; nodes, slots and merged
//     blocks are numbered request by request.
__global__ __launch_bounds__(kPrepThreads) void ragged_prep_kernel(const int32_t* __restrict__ prefix_len,
                                                                   const int32_t* __restrict__ q_len, int n_nodes,
                                                                   int B, int H, int max_q, int kv_stride, int rpb,
                                                                   int target,
                                                                   int max_slots, int max_merges, PlanCost cost,
                                                                   int32_t* __restrict__ rq) {
  __shared__ long long s_part[kPrepThreads / 64];
  __shared__ unsigned long long s_units[kPlanCands], s_pieces[kPlanCands];
  __shared__ int s_dmin[kPlanCands], s_dmax[kPlanCands];
  __shared__ int s_hist[kPlanCands][64];
  __shared__ double s_est[kPlanCands];
  __shared__ int s_capb[kPlanCands], s_capt[kPlanCands];
  __shared__ int s_choice;
  __shared__ int s_scan[kPrepThreads / 64];
  __shared__ unsigned long long s_sort[kSortMax];
  __shared__ int s_len[kPrepLdsReqs][2];  // clamped (q_len, prefix) per request, for B <= kPrepLdsReqs
  const int t = threadIdx.x;
  // Every phase after the first reads the clamped lengths: from LDS when the
  // batch fits (one global round trip fewer per phase), else from the records.
  const bool in_lds = B <= kPrepLdsReqs;
  auto lengths = [&](int b) {
    return in_lds ? req_len_of(s_len[b][0], s_len[b][1], H, rpb) : req_len(rq, b, H, rpb);
  };
  const int per = (B + kPrepThreads - 1) / kPrepThreads;
  const int b0 = min(B, t * per), b1 = min(B, b0 + per);

  // 0. Lengths: q_len into [0, max_q], then the packed nodes into the caller's
  //    n_nodes rows (the request that crosses n_nodes keeps the nodes below it,
  //    later requests none), prefix into [0, kv_stride - q].  Every later
  //    phase reads these from the records.
  {
    int n_raw = 0;
    for (int b = b0; b < b1; ++b) n_raw += min(max(q_len[b], 0), max_q);
    int tot_raw;
    int o_raw = block_scan(n_raw, s_scan, &tot_raw);
    for (int b = b0; b < b1; ++b) {
      const int q = min(max(q_len[b], 0), max_q);
      const int qc = min(q, max(0, n_nodes - o_raw));
      o_raw += q;
      const int pc = min(max(prefix_len[b], 0), kv_stride - qc);
      rq[b * kReqFields + kReqQLen] = qc;
      rq[b * kReqFields + kReqPrefix] = pc;
      if (in_lds) {
        s_len[b][0] = qc;
        s_len[b][1] = pc;
      }
    }
    __syncthreads();
  }

  long long w0 = 0, wt = 0;
  for (int b = b0; b < b1; ++b) {
    const ReqLen r = lengths(b);
    w0 += static_cast<long long>(r.nblk) * (r.tiles + cost.setup);
    wt += static_cast<long long>(r.nblk) * r.tiles;
  }
  const long long T0 = max(1ll, block_sum(w0, s_part) / target);
  const long long Wt = block_sum(wt, s_part);

  for (int i = t; i < kPlanCands * 64; i += kPrepThreads) (&s_hist[0][0])[i] = 0;
  if (t < kPlanCands) {
    s_units[t] = s_pieces[t] = 0;
    s_dmin[t] = INT_MAX;
    s_dmax[t] = 0;
    plan_caps(T0, t, cost.min_piece, s_capb[t], s_capt[t]);
  }
  __syncthreads();
  // One (request, candidate) pair per thread at a time.
  for (int i = t; i < B * kPlanCands; i += kPrepThreads) {
    const int b = i / kPlanCands, c = i - b * kPlanCands;
    const ReqLen r = lengths(b);
    if (r.nblk == 0) continue;
    const ReqCut k = cut_request(r.tiles, s_capb[c], s_capt[c]);
    const int last_b = r.tiles - (k.n_body - 1) * k.c_body, last_t = r.tiles - (k.n_tail - 1) * k.c_tail;
    const int nb = r.nblk - 1;
    const unsigned long long units = static_cast<unsigned long long>(nb) * k.n_body + k.n_tail;
    const unsigned long long pieces =
        (k.n_body > 1 ? static_cast<unsigned long long>(nb) * k.n_body : 0ull) + (k.n_tail > 1 ? k.n_tail : 0);
    atomicAdd(&s_units[c], units);
    if (pieces) atomicAdd(&s_pieces[c], pieces);
    atomicMin(&s_dmin[c], min(nb ? last_b : INT_MAX, last_t) + cost.setup);
    atomicMax(&s_dmax[c], max(nb ? k.c_body : 0, k.c_tail) + cost.setup);
    // (counts of candidates past the slot budget may wrap; those are never read)
    if (nb) {
      if (k.n_body > 1) atomicAdd(&s_hist[c][plan_bucket(k.c_body + cost.setup)], nb * (k.n_body - 1));
      atomicAdd(&s_hist[c][plan_bucket(last_b + cost.setup)], nb);
    }
    if (k.n_tail > 1) atomicAdd(&s_hist[c][plan_bucket(k.c_tail + cost.setup)], k.n_tail - 1);
    atomicAdd(&s_hist[c][plan_bucket(last_t + cost.setup)], 1);
  }
  __syncthreads();
  // One wave per candidate.  Lane i holds bucket 63 - i; an inclusive scan
  // over the lanes gives each bucket's count of units that long or longer,
  // and the lowest lane where it reaches target + 1 names the bucket of the
  // (target+1)-th longest unit.
  {
    const int wave = t >> 6, lane = t & 63;
    for (int c = wave; c < kPlanCands; c += kPrepThreads / 64) {
      long long cum = s_hist[c][63 - lane];
      for (int d = 1; d < 64; d <<= 1) {
        const long long o = __shfl_up(cum, d);
        if (lane >= d) cum += o;
      }
      const unsigned long long hit = __ballot(cum >= static_cast<long long>(target) + 1);
      if (lane == 0) {
        const long long units = static_cast<long long>(s_units[c]);
        const long long pieces = static_cast<long long>(s_pieces[c]);
        const int k2 = units > target && hit ? 63 - (__ffsll(static_cast<long long>(hit)) - 1) : -1;
        s_est[c] = pieces > max_slots || units == 0
                       ? (c == 0 ? 0.0 : -1.0)
                       : plan_estimate(Wt + cost.setup * units, s_dmin[c], s_dmax[c], pieces, cost.pieces_per_step,
                                       k2, target);
      }
    }
  }
  __syncthreads();
  // The least estimate among the candidates within the slot budget (negative
  // marks the others; the uncut candidate 0 always qualifies), the lowest
  // index among equals: a reduction across wave 0.
  if (t < 64) {
    double v = t < kPlanCands && s_est[t] >= 0.0 ? s_est[t] : INFINITY;
    int c = t;
    for (int d = 32; d >= 1; d >>= 1) {
      const double ov = __shfl_xor(v, d);
      const int oc = __shfl_xor(c, d);
      if (ov < v || (ov == v && oc < c)) {
        v = ov;
        c = oc;
      }
    }
    if (t == 0) s_choice = c;
  }
  __syncthreads();
  const int cap_b = s_capb[s_choice], cap_t = s_capt[s_choice];

  // Per request: nodes, slots, merged blocks (request order).
  int n_q = 0, n_slot = 0, n_merge = 0;
  for (int b = b0; b < b1; ++b) {
    const ReqLen r = lengths(b);
    if (r.nblk == 0) continue;
    const ReqCut k = cut_request(r.tiles, cap_b, cap_t);
    n_q += r.q;
    n_slot += (k.n_body > 1 ? (r.nblk - 1) * k.n_body : 0) + (k.n_tail > 1 ? k.n_tail : 0);
    n_merge += (k.n_body > 1 ? r.nblk - 1 : 0) + (k.n_tail > 1 ? 1 : 0);
  }
  int tot_q, tot_slot, tot_merge;
  int o_q = block_scan(n_q, s_scan, &tot_q);
  int o_slot = block_scan(n_slot, s_scan, &tot_slot);
  int o_merge = block_scan(n_merge, s_scan, &tot_merge);
  for (int b = b0; b < b1; ++b) {
    const ReqLen r = lengths(b);
    ReqCut k{1, r.tiles, 1, r.tiles};
    if (r.nblk > 0) k = cut_request(r.tiles, cap_b, cap_t);
    int32_t* o = rq + b * kReqFields;
    o[kReqQStart] = o_q;
    o[kReqQLen] = r.q;
    o[kReqPrefix] = r.P;
    o[kReqNBlk] = r.nblk;
    o[kReqBSplit] = k.n_body;
    o[kReqBChunk] = k.c_body * kPlanTile;
    o[kReqTSplit] = k.n_tail;
    o[kReqTChunk] = k.c_tail * kPlanTile;
    o[kReqSlot0] = o_slot;
    o[kReqMerge0] = o_merge;
    // Merge table: the blocks before the last (if cut), then the last (if cut).
    int4* mt = reinterpret_cast<int4*>(rq + merge_table_word0(B));
    const int body = k.n_body > 1 && r.nblk > 1 ? r.nblk - 1 : 0;
    for (int m = 0; m < body && o_merge + m < max_merges; ++m)
      mt[o_merge + m] = make_int4(o_slot + m * k.n_body, k.n_body, o_q * H + m * rpb, rpb);
    if (r.nblk > 0 && k.n_tail > 1 && o_merge + body < max_merges)
      mt[o_merge + body] = make_int4(o_slot + body * k.n_body, k.n_tail, o_q * H + (r.nblk - 1) * rpb,
                                     r.q * H - (r.nblk - 1) * rpb);
    if (r.nblk > 0) {
      o_q += r.q;
      o_slot += (k.n_body > 1 ? (r.nblk - 1) * k.n_body : 0) + (k.n_tail > 1 ? k.n_tail : 0);
      o_merge += (k.n_body > 1 ? r.nblk - 1 : 0) + (k.n_tail > 1 ? 1 : 0);
    }
  }

  // Classes in launch order: longest piece first, ties by id; classes with no
  // units last.  Without the sort (very large batches) request order.
  const int n_cls = 2 * B;
  const bool sorted = n_cls <= kSortMax;
  auto cls_of = [&](int id, int& units, int& len) {
    const ReqLen r = lengths(id >> 1);
    units = 0;
    len = 0;
    if (r.nblk == 0) return;
    const ReqCut k = cut_request(r.tiles, cap_b, cap_t);
    if (id & 1) {
      units = k.n_tail;
      len = k.c_tail;
    } else if (r.nblk > 1) {
      units = (r.nblk - 1) * k.n_body;
      len = k.c_body;
    }
  };
  int n_sort = 1;
  if (sorted && n_cls <= kRankSortMax) {
    // Keys are distinct (the id is in the low bits): each class's position is
    // the number of smaller keys.
    unsigned long long key = 0;
    if (t < n_cls) {
      int units, len;
      cls_of(t, units, len);
      key = (static_cast<unsigned long long>(0xffffffffu - static_cast<unsigned>(units ? len : 0)) << 32) |
            static_cast<unsigned>(t);
      s_sort[t] = key;
    }
    __syncthreads();
    int rank = 0;
    if (t < n_cls)
      for (int j = 0; j < n_cls; ++j) rank += s_sort[j] < key ? 1 : 0;
    __syncthreads();
    if (t < n_cls) s_sort[rank] = key;
    __syncthreads();
  } else if (sorted) {
    while (n_sort < n_cls) n_sort <<= 1;
    for (int i = t; i < n_sort; i += kPrepThreads) {
      unsigned long long key = ~0ull;
      if (i < n_cls) {
        int units, len;
        cls_of(i, units, len);
        key = (static_cast<unsigned long long>(0xffffffffu - static_cast<unsigned>(units ? len : 0)) << 32) |
              static_cast<unsigned>(i);
      }
      s_sort[i] = key;
    }
    __syncthreads();
    for (int k = 2; k <= n_sort; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = t; i < n_sort; i += kPrepThreads) {
          const int l = i ^ j;
          if (l > i) {
            const unsigned long long x = s_sort[i], y = s_sort[l];
            const bool up = (i & k) == 0;
            if ((x > y) == up) {
              s_sort[i] = y;
              s_sort[l] = x;
            }
          }
        }
        __syncthreads();
      }
    }
  }
  // Number the units class by class in launch order: thread t takes a
  // contiguous run of positions.
  const int cper = (n_cls + kPrepThreads - 1) / kPrepThreads;
  const int p0 = min(n_cls, t * cper), p1 = min(n_cls, p0 + cper);
  int n_u = 0;
  for (int p = p0; p < p1; ++p) {
    const int id = sorted ? static_cast<int>(s_sort[p] & 0xffffffffu) : p;
    int units, len;
    cls_of(id, units, len);
    n_u += units;
  }
  int tot_units;
  int o_u = block_scan(n_u, s_scan, &tot_units);
  int32_t* cu0 = rq + B * kReqFields;
  int32_t* cid = cu0 + 2 * B;
  for (int p = p0; p < p1; ++p) {
    const int id = sorted ? static_cast<int>(s_sort[p] & 0xffffffffu) : p;
    int units, len;
    cls_of(id, units, len);
    cu0[p] = o_u;
    cid[p] = id;
    o_u += units;
  }
  if (t == 0) {
    int32_t* tot = cid + 2 * B;
    tot[kTotUnits] = tot_units;
    tot[kTotMerge] = tot_merge;
    tot[kTotChoice] = s_choice;
  }
  // The persistent attention grid's per-XCD unit counters start at zero.
  if (t < kXcdQueues) rq[queue_word0(B, max_merges) + t] = 0;
}

}  // namespace

// Combine the pieces of split row blocks: w_s = l_s * exp(m_s - max m),
// out = sum w_s o_s / sum w_s, lse = max m + log(sum w_s).  One thread per
// (merged row block, row r within it, float4 column).  The pieces are read in
// batches, all loads of a batch issued together, and the running max is
// carried across batches by rescaling (one memory round trip per batch).
//
// A merged block: where its pieces' slots start, how many there are, and
// which rows of the output they belong to.
struct MergeBlock {
  long long slot0;  // first slot of the block's pieces
  long long row0;   // output row that the block's row base counts from
  int n_split;      // pieces
  int row_base;     // the block's first row, counted from row0
  int R;            // rows below this bound (counted from row0) exist
};

// Merged block mb of a uniform batch: the full row blocks of every tree
// (when they are cut), then the partial last blocks.
__device__ __forceinline__ MergeBlock merge_block(const AttnArgs& a, long long mb) {
  const long long full_blocks = a.split_full > 1 ? static_cast<long long>(a.B) * a.full_rb : 0;
  MergeBlock k;
  int b, rb;
  if (mb < full_blocks) {
    b = static_cast<int>(mb / a.full_rb);
    rb = static_cast<int>(mb % a.full_rb);
    k.n_split = a.split_full;
    k.slot0 = mb * a.split_full;
  } else {
    b = static_cast<int>(mb - full_blocks);
    rb = a.n_rb - 1;
    k.n_split = a.split_tail;
    k.slot0 = (a.split_full > 1 ? full_blocks * a.split_full : 0) + static_cast<long long>(b) * a.split_tail;
  }
  k.R = a.R;
  k.row0 = static_cast<long long>(b) * a.R;
  k.row_base = rb * a.rows_per_block;
  return k;
}

// Row r of merged block k, float4 column col4: the pieces' partial outputs
// combined by log-sum-exp (online rescaled, eight pieces' loads at a time).
__device__ __forceinline__ void merge_row(const AttnArgs& a, int d_c, const MergeBlock& k, int r, int col4) {
  const int rpb = a.rows_per_block;
  const int row = k.row_base + r;
  if (row >= k.R) return;
  constexpr int kBatch = 8;
  float M = -INFINITY, W = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < k.n_split; s0 += kBatch) {
    float l[kBatch], m[kBatch];
    float4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const long long sr = (k.slot0 + s0 + j) * rpb + r;
      const bool in = s0 + j < k.n_split;
      l[j] = in ? a.ws_l[sr] : 0.f;
      m[j] = in ? a.ws_m[sr] : 0.f;
      v[j] = in ? *reinterpret_cast<const float4*>(a.ws_o + sr * d_c + col4 * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // pieces with no visible key (row sum 0) add nothing
    float mb_max = -INFINITY;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) mb_max = l[j] > 0.f ? fmaxf(mb_max, m[j]) : mb_max;
    if (mb_max == -INFINITY) continue;
    const float Mn = fmaxf(M, mb_max);
    const float sc = expf(M - Mn);  // 0 on the first batch with a visible key
    W *= sc;
    acc.x *= sc;
    acc.y *= sc;
    acc.z *= sc;
    acc.w *= sc;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float w = l[j] > 0.f ? l[j] * expf(m[j] - Mn) : 0.f;
      W += w;
      acc.x = fmaf(w, v[j].x, acc.x);
      acc.y = fmaf(w, v[j].y, acc.y);
      acc.z = fmaf(w, v[j].z, acc.z);
      acc.w = fmaf(w, v[j].w, acc.w);
    }
    M = Mn;
  }
  const float inv = 1.f / W;
  const long long grow = k.row0 + row;
  *reinterpret_cast<float4*>(a.out + grow * d_c + col4 * 4) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (col4 == 0 && a.lse) a.lse[grow] = M + logf(W);
}

// Uniform batch: threads cover the rows that exist, the merged full row
// blocks (rows_per_block rows each) and then the merged partial last blocks
// (R - (n_rb - 1) rows_per_block rows each); the grid strides over them.  The
// block of an element follows from its index by division.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int d_c, long long n_blocks) {
  const int cpt = d_c / 4;
  const int rpb = a.rows_per_block;
  const long long full_blocks = a.split_full > 1 ? static_cast<long long>(a.B) * a.full_rb : 0;
  const long long tail_rows = a.R - static_cast<long long>(a.n_rb - 1) * rpb;
  const long long full_rows = full_blocks * rpb;
  const long long total = (full_rows + (n_blocks - full_blocks) * tail_rows) * cpt;
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int col4 = static_cast<int>(idx % cpt);
    const long long row_i = idx / cpt;
    if (row_i < full_rows) {
      merge_row(a, d_c, merge_block(a, row_i / rpb), static_cast<int>(row_i % rpb), col4);
    } else {
      const long long t = row_i - full_rows;
      merge_row(a, d_c, merge_block(a, full_blocks + t / tail_rows), static_cast<int>(t % tail_rows), col4);
    }
  }
}

// Ragged batch: a workgroup takes tasks of 256 / (d_c / 4) rows of one merged
// block.  The prep kernel wrote each merged block's slots and rows into the
// merge table, so a task needs one 16-byte load before its pieces' loads.
// Tasks are numbered block after block up to the real number of merged blocks
// (from the records); the grid strides over them.
__global__ __launch_bounds__(256) void attn_merge_ragged_kernel(AttnArgs a, int d_c) {
  const int cpt = d_c / 4;
  const int task_rows = blockDim.x / cpt;
  const int tasks_per_block = (a.rows_per_block + task_rows - 1) / task_rows;
  const long long n_tasks = static_cast<long long>(req_totals(a.req, a.B)[kTotMerge]) * tasks_per_block;
  const int r_in = static_cast<int>(threadIdx.x) / cpt;
  const int col4 = static_cast<int>(threadIdx.x) % cpt;
  if (r_in >= task_rows) return;  // only when d_c / 4 does not divide 256 (no barrier below)
  for (long long t = blockIdx.x; t < n_tasks; t += gridDim.x) {
    const int r = static_cast<int>(t % tasks_per_block) * task_rows + r_in;
    const int4 e = a.merge_tab[t / tasks_per_block];
    MergeBlock k;
    k.slot0 = e.x;
    k.n_split = e.y;
    k.row0 = e.z;
    k.row_base = 0;
    k.R = e.w;
    if (r < a.rows_per_block) merge_row(a, d_c, k, r, col4);
  }
}

hipError_t launch_attention(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  // A ragged batch runs a persistent grid (next_unit_ragged): as many
  // workgroups as run at once, at most the bound of units.
  AttnPlan lp = plan;
  if (a.req) lp.units = plan.units < plan.target ? plan.units : plan.target;
  hipError_t e = lp.kernel == AttnKernel::kMfmaBf16Q2 ? launch_attn_mfma_q2(s, lp, a, stream)
                 : lp.kernel == AttnKernel::kMfmaBf16 ? launch_attn_mfma_bf16(s, lp, a, stream)
                 : lp.kernel == AttnKernel::kMfmaF32 || lp.kernel == AttnKernel::kMfmaF32Narrow
                     ? launch_attn_mfma_f32(s, lp, a, stream)
                                                      : launch_attn_valu(s, lp, a, stream);
  if (e != hipSuccess || plan.merge_blocks == 0) return e;
  if (a.req) {
    // The tasks of the bound (merged blocks x tasks per block), at most 8
    // workgroups per CU: the bound can far exceed the real count, and every
    // workgroup past it still reads the count before it leaves (measured:
    // 16384 workgroups cost ~7 us more than 2048 at 32 real merged blocks).
    // The kernel strides over the real count.
    const int task_rows = 256 / (s.d_c / 4);
    long long grid = plan.merge_blocks * ((plan.rows_per_block + task_rows - 1) / task_rows);
    if (grid > 8 * kNumCU) grid = 8 * kNumCU;
    attn_merge_ragged_kernel<<<dim3(static_cast<unsigned>(grid)), 256, 0, stream>>>(a, s.d_c);
    return hipGetLastError();
  }
  const long long full_blocks = plan.split_full > 1 ? static_cast<long long>(s.B) * plan.full_rb : 0;
  const long long tail_rows =
      static_cast<long long>(s.q_len) * s.H - static_cast<long long>(plan.n_rb - 1) * plan.rows_per_block;
  const long long rows = full_blocks * plan.rows_per_block + (plan.merge_blocks - full_blocks) * tail_rows;
  const long long grid = (rows * (s.d_c / 4) + 255) / 256;
  attn_merge_kernel<<<dim3(static_cast<unsigned>(grid)), 256, 0, stream>>>(a, s.d_c, plan.merge_blocks);
  return hipGetLastError();
}

hipError_t launch_ragged_prep(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, const int32_t* prefix_len,
                              const int32_t* q_len, hipStream_t stream) {
  const bool f32 = plan.kernel == AttnKernel::kMfmaF32 || plan.kernel == AttnKernel::kMfmaF32Narrow;
  ragged_prep_kernel<<<dim3(1), kPrepThreads, 0, stream>>>(prefix_len, q_len, a.n_nodes, s.B, s.H, s.q_len, s.kv_len,
                                                           plan.rows_per_block, static_cast<int>(plan.target),
                                                           static_cast<int>(plan.n_slots),
                                                           static_cast<int>(plan.merge_blocks),
                                                           f32 ? kPlanCostF32 : kPlanCostDefault,
                                                           const_cast<int32_t*>(a.req));
  return hipGetLastError();
}

}  // namespace tv
