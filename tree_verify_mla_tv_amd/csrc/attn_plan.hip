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

// Ragged batch: the same choice of kernel and split count, made from upper
// bounds (B requests of at most max_q_len nodes over at most kv_stride keys);
// each request then cuts its own kv range into pieces of the same size, so
// shorter requests get fewer pieces.  units, n_slots and merge_blocks are
// upper bounds (the launch sizes); the workspace starts with the request
// records.
AttnPlan plan_attention_ragged(const AttnShape& s) {
  AttnPlan p{};
  const bool mfma = s.kv_bf16 && s.d_c == 512 && s.d_r == 64;
  p.kernel = mfma ? AttnKernel::kMfmaBf16 : AttnKernel::kValu;
  p.rows_per_block = mfma ? kMfmaRows : kValuRows;
  p.keys_per_tile = mfma ? kMfmaKeys : kValuKeys;
  p.n_rb = ceil_div(static_cast<long long>(s.q_len) * s.H, p.rows_per_block);
  p.full_rb = p.n_rb;
  const long long target = mfma ? kNumCU : 2 * kNumCU;
  const long long blocks = static_cast<long long>(s.B) * p.n_rb;
  if (blocks < target)
    cut_for_blocks(s.kv_len, blocks, target, p.keys_per_tile, 10, p.split_full, p.chunk_full);
  else
    cut(s.kv_len, 1, p.keys_per_tile, p.split_full, p.chunk_full);
  p.split_tail = p.split_full;
  p.chunk_tail = p.chunk_full;
  p.units = blocks * p.split_full;
  p.n_slots = p.split_full > 1 ? p.units : 0;
  p.merge_blocks = p.split_full > 1 ? blocks : 0;
  const size_t rec = align256((static_cast<size_t>(s.B) * kReqFields + 2) * sizeof(int32_t));
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

// Request records of a ragged batch (one workgroup of 1024 threads): lengths
// clamped into the bounds (q_len to [0, max_q], prefix to [0, kv_stride -
// q_len]), row blocks, kv pieces, and the first unit, slot and merged block of
// each request (exclusive scans over the batch), then the totals.
__global__ __launch_bounds__(1024) void ragged_prep_kernel(const int32_t* __restrict__ prefix_len,
                                                           const int32_t* __restrict__ q_len, int B, int H,
                                                           int max_q, int kv_stride, int rpb, int chunk,
                                                           int32_t* __restrict__ rq) {
  __shared__ int s_scan[4][1024];
  const int t = threadIdx.x;
  const int per = (B + 1023) / 1024;
  const int b0 = min(B, t * per);
  const int b1 = min(B, b0 + per);
  // Per request: nodes, units, slots, merged blocks.
  auto shape = [&](int b, int& q, int& P, int& n_rb, int& n_split) {
    q = min(max(q_len[b], 0), max_q);
    P = min(max(prefix_len[b], 0), kv_stride - q);
    n_rb = (q * H + rpb - 1) / rpb;
    n_split = max((P + q + chunk - 1) / chunk, 1);
  };
  int sum[4] = {0, 0, 0, 0};
  for (int b = b0; b < b1; ++b) {
    int q, P, n_rb, n_split;
    shape(b, q, P, n_rb, n_split);
    sum[0] += q;
    sum[1] += n_rb * n_split;
    sum[2] += n_split > 1 ? n_rb * n_split : 0;
    sum[3] += n_split > 1 ? n_rb : 0;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) s_scan[k][t] = sum[k];
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = t >= off ? s_scan[k][t - off] : 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) s_scan[k][t] += v[k];
    __syncthreads();
  }
  int run[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) run[k] = s_scan[k][t] - sum[k];
  for (int b = b0; b < b1; ++b) {
    int q, P, n_rb, n_split;
    shape(b, q, P, n_rb, n_split);
    int32_t* r = rq + b * kReqFields;
    r[kReqQStart] = run[0];
    r[kReqQLen] = q;
    r[kReqPrefix] = P;
    r[kReqNRb] = n_rb;
    r[kReqSplit] = n_split;
    r[kReqUnit0] = run[1];
    r[kReqSlot0] = run[2];
    r[kReqMerge0] = run[3];
    run[0] += q;
    run[1] += n_rb * n_split;
    run[2] += n_split > 1 ? n_rb * n_split : 0;
    run[3] += n_split > 1 ? n_rb : 0;
  }
  if (t == 1023) {
    rq[B * kReqFields] = s_scan[1][1023];
    rq[B * kReqFields + 1] = s_scan[3][1023];
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
    if (mb >= a.req[a.B * kReqFields + 1]) return;
    const int bq = find_request(a.req, a.B, kReqMerge0, mb);
    const int32_t* rec = a.req + bq * kReqFields;
    rb = static_cast<int>(mb - rec[kReqMerge0]);
    n_split = rec[kReqSplit];
    slot0 = static_cast<long long>(rec[kReqSlot0]) + static_cast<long long>(rb) * n_split;
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
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, a.ws_m[(slot0 + s) * rpb + r]);
  float W = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < n_split; ++s) {
    const long long sr = (slot0 + s) * rpb + r;
    const float l = a.ws_l[sr];
    if (!(l > 0.f)) continue;
    const float w = l * expf(a.ws_m[sr] - M);
    const float4 v = *reinterpret_cast<const float4*>(a.ws_o + sr * d_c + col4 * 4);
    W += w;
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
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
                                                   plan.rows_per_block, plan.chunk_full, const_cast<int32_t*>(a.req));
  return hipGetLastError();
}

}  // namespace tv
