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
constexpr int kMinKeysPerTailPiece = 1024;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int ceil_div(long long a, long long b) { return static_cast<int>((a + b - 1) / b); }

// Cut kv_len rows into at most `want` ranges of a whole number of tiles.
void cut(int kv_len, int want, int tile, int& n, int& chunk) {
  const int max_split = kv_len / kMinKeysPerSplit > 1 ? kv_len / kMinKeysPerSplit : 1;
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
void cut_for_blocks(int kv_len, long long blocks, long long slots, int tile, int setup_tiles, int& n, int& chunk) {
  const int max_split = kv_len / kMinKeysPerSplit > 1 ? kv_len / kMinKeysPerSplit : 1;
  long long best_cost = -1;
  int best = 1;
  for (int want = 1; want <= max_split; ++want) {
    int sn, sc;
    cut(kv_len, want, tile, sn, sc);
    if (sn != want) continue;  // an equivalent cut was already counted
    const long long rounds = (blocks * sn + slots - 1) / slots;
    const long long cost = rounds * (sc / tile + setup_tiles);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = sn;
    }
  }
  cut(kv_len, best, tile, n, chunk);
}
}  // namespace

AttnPlan plan_attention(const AttnShape& s) {
  AttnPlan p{};
  const bool mfma = s.kv_bf16 && s.d_c == 512 && s.d_r == 64;
  p.kernel = mfma ? AttnKernel::kMfmaBf16 : AttnKernel::kValu;
  p.rows_per_block = mfma ? kMfmaRows : kValuRows;
  p.keys_per_tile = mfma ? kMfmaKeys : kValuKeys;
  const int R = s.q_len * s.H;
  p.n_rb = ceil_div(R, p.rows_per_block);
  const bool has_tail = (R % p.rows_per_block) != 0;
  p.full_rb = has_tail ? p.n_rb - 1 : p.n_rb;
  // Workgroups resident per CU: the MFMA kernel takes a whole CU; the VALU one
  // about one (its LDS is ~114 KB at d_c = 512), so aim at two rounds for it.
  const long long target = mfma ? kNumCU : 2 * kNumCU;

  const long long blocks = static_cast<long long>(s.B) * p.n_rb;
  if (blocks < target) {
    // Too few row blocks: cut every block's kv range.  A unit's set-up (tree
    // masks, queries, first tile, output) costs about ten tile-steps.
    cut_for_blocks(s.kv_len, blocks, target, p.keys_per_tile, 10, p.split_full, p.chunk_full);
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
      cut(s.kv_len, static_cast<int>(free_slots / tails), p.keys_per_tile, p.split_tail, p.chunk_tail);
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

// Ragged batch: the same choices as plan_attention, made from upper bounds (B
// requests of at most max_q_len nodes over at most kv_stride keys).  With too
// few row blocks to fill the GPU, every row block's kv range is cut into
// pieces of chunk_full keys (shorter requests get fewer pieces).  Otherwise
// full row blocks stay whole and the prep kernel cuts each request's partial
// last row block into as many pieces (at most kMaxTailSplit) as fill the last
// round of workgroups.  units, n_slots and merge_blocks are upper bounds (the
// launch sizes); the workspace starts with the request records.
AttnPlan plan_attention_ragged(const AttnShape& s) {
  AttnPlan p{};
  const bool mfma = s.kv_bf16 && s.d_c == 512 && s.d_r == 64;
  p.kernel = mfma ? AttnKernel::kMfmaBf16 : AttnKernel::kValu;
  p.rows_per_block = mfma ? kMfmaRows : kValuRows;
  p.keys_per_tile = mfma ? kMfmaKeys : kValuKeys;
  p.n_rb = ceil_div(static_cast<long long>(s.q_len) * s.H, p.rows_per_block);
  p.full_rb = p.n_rb;
  p.target = mfma ? kNumCU : 2 * kNumCU;
  const long long blocks = static_cast<long long>(s.B) * p.n_rb;
  if (blocks < p.target) {
    cut_for_blocks(s.kv_len, blocks, p.target, p.keys_per_tile, 10, p.split_full, p.chunk_full);
    p.tail_pieces = false;
    p.units = blocks * p.split_full;
    p.n_slots = p.split_full > 1 ? p.units : 0;
    p.merge_blocks = p.split_full > 1 ? blocks : 0;
  } else {
    p.split_full = 1;
    p.chunk_full = ceil_div(s.kv_len, p.keys_per_tile) * p.keys_per_tile;
    p.tail_pieces = true;
    p.units = static_cast<long long>(s.B) * (p.n_rb + kMaxTailSplit);
    p.n_slots = static_cast<long long>(s.B) * kMaxTailSplit;
    p.merge_blocks = s.B;
  }
  p.split_tail = p.split_full;
  p.chunk_tail = p.chunk_full;
  const size_t rec = align256((static_cast<size_t>(s.B) * kReqFields + kReqTotals) * sizeof(int32_t));
  p.ws_bytes = rec;
  p.ws_o_off = p.ws_m_off = p.ws_l_off = rec;
  if (p.n_slots > 0) {
    const size_t rows = static_cast<size_t>(p.n_slots) * p.rows_per_block;
    p.ws_m_off = rec + align256(rows * s.d_c * sizeof(float));
    p.ws_l_off = p.ws_m_off + align256(rows * sizeof(float));
    p.ws_bytes = p.ws_l_off + align256(rows * sizeof(float));
  }
  return p;
}

namespace {

static_assert(kMfmaKeys == kValuKeys, "piece sizes of the partial blocks are whole tiles of either kernel");

// Request records of a ragged batch (one workgroup of 1024 threads).  Lengths
// are clamped into the bounds (q_len to [0, max_q], prefix to [0, kv_stride -
// q_len]).  Per request: full row blocks and their pieces, the pieces of the
// partial last block, and (exclusive scans over the batch) its first node,
// full-block unit, partial-block unit, slot and merged block; then the totals.
struct ReqShape {
  int q, P, n_full, split, tsplit, tchunk;
};

__device__ __forceinline__ ReqShape req_shape(const int32_t* prefix_len, const int32_t* q_len, int b, int H, int max_q,
                                              int kv_stride, int rpb, int chunk, bool tail_pieces, int g_tsplit) {
  ReqShape r;
  r.q = min(max(q_len[b], 0), max_q);
  r.P = min(max(prefix_len[b], 0), kv_stride - r.q);
  const int R = r.q * H;
  const int kv = r.P + r.q;
  r.n_full = R / rpb;
  r.split = tail_pieces ? 1 : max((kv + chunk - 1) / chunk, 1);
  r.tsplit = 0;
  r.tchunk = 0;
  if (R % rpb != 0) {
    if (!tail_pieces) {
      r.tsplit = r.split;
      r.tchunk = chunk;
    } else {
      // Pieces of at least kMinKeysPerTailPiece keys: a unit's set-up (~10
      // tile-steps) should stay small next to its sweep.
      const int want = min(g_tsplit, max(1, kv / kMinKeysPerTailPiece));
      r.tchunk = (((kv + want - 1) / want + kMfmaKeys - 1) / kMfmaKeys) * kMfmaKeys;  // whole tiles (both kernels: 32 keys)
      r.tsplit = (kv + r.tchunk - 1) / r.tchunk;
    }
  }
  return r;
}

__global__ __launch_bounds__(1024) void ragged_prep_kernel(const int32_t* __restrict__ prefix_len,
                                                           const int32_t* __restrict__ q_len, int B, int H,
                                                           int max_q, int kv_stride, int rpb, int chunk,
                                                           int tail_pieces, int target, int32_t* __restrict__ rq) {
  constexpr int kN = 5;  // nodes, full-block units, partial-block units, slots, merged blocks
  __shared__ int s_scan[kN][1024];
  __shared__ int s_tsplit;
  const int t = threadIdx.x;
  const int per = (B + 1023) / 1024;
  const int b0 = min(B, t * per);
  const int b1 = min(B, b0 + per);
  // Pieces of the partial blocks: fill what the full blocks leave of their
  // last round (a round more if that is less than one piece per block).
  int g_tsplit = 1;
  if (tail_pieces) {
    int full = 0, part = 0;
    for (int b = b0; b < b1; ++b) {
      const ReqShape r = req_shape(prefix_len, q_len, b, H, max_q, kv_stride, rpb, chunk, false, 1);
      full += r.n_full;
      part += r.tsplit > 0;
    }
    s_scan[0][t] = full;
    s_scan[1][t] = part;
    __syncthreads();
    for (int off = 512; off > 0; off >>= 1) {
      if (t < off) {
        s_scan[0][t] += s_scan[0][t + off];
        s_scan[1][t] += s_scan[1][t + off];
      }
      __syncthreads();
    }
    if (t == 0) {
      const int n_part = s_scan[1][0];
      int free_slots = target - s_scan[0][0] % target;
      if (free_slots < n_part) free_slots += target;
      s_tsplit = min(max(free_slots / max(n_part, 1), 1), kMaxTailSplit);
    }
    __syncthreads();
    g_tsplit = s_tsplit;
    __syncthreads();
  }
  int sum[kN] = {0, 0, 0, 0, 0};
  for (int b = b0; b < b1; ++b) {
    const ReqShape r = req_shape(prefix_len, q_len, b, H, max_q, kv_stride, rpb, chunk, tail_pieces, g_tsplit);
    sum[0] += r.q;
    sum[1] += r.n_full * r.split;
    sum[2] += r.tsplit;
    sum[3] += (r.split > 1 ? r.n_full * r.split : 0) + (r.tsplit > 1 ? r.tsplit : 0);
    sum[4] += (r.split > 1 ? r.n_full : 0) + (r.tsplit > 1 ? 1 : 0);
  }
#pragma unroll
  for (int k = 0; k < kN; ++k) s_scan[k][t] = sum[k];
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int v[kN];
#pragma unroll
    for (int k = 0; k < kN; ++k) v[k] = t >= off ? s_scan[k][t - off] : 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kN; ++k) s_scan[k][t] += v[k];
    __syncthreads();
  }
  int run[kN];
#pragma unroll
  for (int k = 0; k < kN; ++k) run[k] = s_scan[k][t] - sum[k];
  for (int b = b0; b < b1; ++b) {
    const ReqShape r = req_shape(prefix_len, q_len, b, H, max_q, kv_stride, rpb, chunk, tail_pieces, g_tsplit);
    int32_t* o = rq + b * kReqFields;
    o[kReqQStart] = run[0];
    o[kReqQLen] = r.q;
    o[kReqPrefix] = r.P;
    o[kReqNFull] = r.n_full;
    o[kReqSplit] = r.split;
    o[kReqTSplit] = r.tsplit;
    o[kReqTChunk] = r.tchunk;
    o[kReqFull0] = run[1];
    o[kReqTail0] = run[2];
    o[kReqSlot0] = run[3];
    o[kReqMerge0] = run[4];
    run[0] += r.q;
    run[1] += r.n_full * r.split;
    run[2] += r.tsplit;
    run[3] += (r.split > 1 ? r.n_full * r.split : 0) + (r.tsplit > 1 ? r.tsplit : 0);
    run[4] += (r.split > 1 ? r.n_full : 0) + (r.tsplit > 1 ? 1 : 0);
  }
  if (t == 1023) {
    rq[B * kReqFields] = s_scan[1][1023];
    rq[B * kReqFields + 1] = s_scan[1][1023] + s_scan[2][1023];
    rq[B * kReqFields + 2] = s_scan[4][1023];
  }
}

}  // namespace

// Combine the pieces of split row blocks: w_s = l_s * exp(m_s - max m),
// out = sum w_s o_s / sum w_s, lse = max m + log(sum w_s).
// One thread per (merged row block, row, float4 column).
// n_blocks: merged row blocks launched (for a ragged batch an upper bound;
// blocks past the batch's total return at once).
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int d_c, long long n_blocks) {
  const int cpt = d_c / 4;
  const int rpb = a.rows_per_block;
  const long long full_blocks = a.split_full > 1 ? static_cast<long long>(a.B) * a.full_rb : 0;
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n_blocks * rpb * cpt) return;
  const int col4 = static_cast<int>(idx % cpt);
  const int r = static_cast<int>((idx / cpt) % rpb);
  const long long mb = idx / (static_cast<long long>(cpt) * rpb);
  int rb, n_split, R;
  long long slot0, row0;
  if (a.req) {
    if (mb >= a.req[a.B * kReqFields + 2]) return;
    const int bq = find_request(a.req, a.B, kReqMerge0, mb);
    const int32_t* rec = a.req + bq * kReqFields;
    const int m = static_cast<int>(mb - rec[kReqMerge0]);
    const int split = rec[kReqSplit];
    const int full_merges = split > 1 ? rec[kReqNFull] : 0;
    if (m < full_merges) {  // a full row block
      rb = m;
      n_split = split;
      slot0 = static_cast<long long>(rec[kReqSlot0]) + static_cast<long long>(m) * split;
    } else {  // the partial last row block
      rb = rec[kReqNFull];
      n_split = rec[kReqTSplit];
      slot0 = static_cast<long long>(rec[kReqSlot0]) + static_cast<long long>(full_merges) * split;
    }
    R = rec[kReqQLen] * a.H;
    row0 = static_cast<long long>(rec[kReqQStart]) * a.H;
  } else if (mb < full_blocks) {
    const int b = static_cast<int>(mb / a.full_rb);
    rb = static_cast<int>(mb % a.full_rb);
    n_split = a.split_full;
    slot0 = mb * a.split_full;
    R = a.R;
    row0 = static_cast<long long>(b) * a.R;
  } else {
    const int b = static_cast<int>(mb - full_blocks);
    rb = a.n_rb - 1;
    n_split = a.split_tail;
    slot0 = (a.split_full > 1 ? full_blocks * a.split_full : 0) + static_cast<long long>(b) * a.split_tail;
    R = a.R;
    row0 = static_cast<long long>(b) * a.R;
  }
  const int row = rb * rpb + r;
  if (row >= R) return;
  // The pieces' loads are issued in batches with no branch between them, so a
  // thread waits for one memory round trip per batch rather than per piece.
  constexpr int kBatch = 8;
  float M = -INFINITY;
  for (int s0 = 0; s0 < n_split; s0 += kBatch) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (s0 + k < n_split) M = fmaxf(M, a.ws_m[(slot0 + s0 + k) * rpb + r]);
  }
  float W = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < n_split; s0 += kBatch) {
    float l[kBatch], m[kBatch];
    float4 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const long long sr = (slot0 + s0 + k) * rpb + r;
      const bool in = s0 + k < n_split;
      l[k] = in ? a.ws_l[sr] : 0.f;
      m[k] = in ? a.ws_m[sr] : 0.f;
      v[k] = in ? *reinterpret_cast<const float4*>(a.ws_o + sr * d_c + col4 * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      // a piece with no visible key (row sum 0) adds nothing
      const float w = l[k] > 0.f ? l[k] * expf(m[k] - M) : 0.f;
      W += w;
      acc.x = fmaf(w, v[k].x, acc.x);
      acc.y = fmaf(w, v[k].y, acc.y);
      acc.z = fmaf(w, v[k].z, acc.z);
      acc.w = fmaf(w, v[k].w, acc.w);
    }
  }
  const float inv = 1.f / W;
  const long long grow = row0 + row;
  *reinterpret_cast<float4*>(a.out + grow * d_c + col4 * 4) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (col4 == 0 && a.lse) a.lse[grow] = M + logf(W);
}

hipError_t launch_attention(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  hipError_t e = plan.kernel == AttnKernel::kMfmaBf16 ? launch_attn_mfma_bf16(s, plan, a, stream)
                                                       : launch_attn_valu(s, plan, a, stream);
  if (e != hipSuccess || plan.merge_blocks == 0) return e;
  const long long total = plan.merge_blocks * plan.rows_per_block * (s.d_c / 4);
  attn_merge_kernel<<<dim3(static_cast<unsigned>((total + 255) / 256)), 256, 0, stream>>>(a, s.d_c,
                                                                                           plan.merge_blocks);
  return hipGetLastError();
}

hipError_t launch_ragged_prep(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, const int32_t* prefix_len,
                              const int32_t* q_len, hipStream_t stream) {
  ragged_prep_kernel<<<dim3(1), 1024, 0, stream>>>(prefix_len, q_len, s.B, s.H, s.q_len, s.kv_len,
                                                   plan.rows_per_block, plan.chunk_full, plan.tail_pieces ? 1 : 0,
                                                   static_cast<int>(plan.target), const_cast<int32_t*>(a.req));
  return hipGetLastError();
}

}  // namespace tv
