// NeoX RoPE with float64 angles, and tree-node positions.
//
// [RoPE page = "Precision as Correctness: The Float64 RoPE Decision in a Custom
//  CUDA Inference Engine", sections "The Message", "The Float64 Decision" and
//  "What Input Knowledge Is Required" item 1]: the rope slice is split into two
// halves, pair k = (x[k], x[k + d/2]) turns by pos * inv_freq[k], and the angle,
// cos, sin and the rotation are evaluated in float64 with a single rounding
// back to the storage type at the end.
//
// The work is element-wise and memory-bound (the same page, "Assumptions and
// Potential Pitfalls" item 2): each thread owns one pair of one row, so a wave
// touches 64 consecutive elements of each half of a row.  MI355X runs FP64 at
// half the FP32 rate, so the float64 sin/cos cost is hidden behind HBM traffic.
#include "tv_kernels.h"

namespace tv {

// The rotation itself.  Contraction into FMA is disabled so that each product
// and each sum is rounded in float64 exactly as written.
__device__ __forceinline__ void rotate_cs_f64(double x1, double x2, double c, double s, double& y1, double& y2) {
#pragma clang fp contract(off)
  y1 = x1 * c - x2 * s;
  y2 = x2 * c + x1 * s;
}

__device__ __forceinline__ void rotate_pair_f64(double x1, double x2, double ang, double& y1, double& y2) {
  double s, c;
  sincos(ang, &s, &c);
  rotate_cs_f64(x1, x2, c, s, y1, y2);
}

template <typename T>
__global__ __launch_bounds__(256) void rope_neox_kernel(typename T::storage* __restrict__ x,
                                                        const int32_t* __restrict__ pos, int64_t n_tok, int n_head,
                                                        int half, int64_t seq_stride, int64_t tok_stride,
                                                        int64_t pos_seq_stride, int64_t total, RopeFreq f) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int k = static_cast<int>(idx % half);
    int64_t rest = idx / half;
    const int h = static_cast<int>(rest % n_head);
    rest /= n_head;
    const int64_t t = rest % n_tok;
    const int64_t s = rest / n_tok;
    const int64_t p = pos ? pos[s * pos_seq_stride + t] : t;
    typename T::storage* row = x + s * seq_stride + t * tok_stride + static_cast<int64_t>(h) * 2 * half;
    const double x1 = load_f64<T>(row + k);
    const double x2 = load_f64<T>(row + k + half);
    double y1, y2;
    rotate_pair_f64(x1, x2, static_cast<double>(p) * f.inv_freq[k], y1, y2);
    store_from_f64<T>(row + k, y1);
    store_from_f64<T>(row + k + half, y2);
  }
}

// Depth of every node of one tree, into LDS: thread i walks i -> parent -> ...
// -> root.  Parents are clamped (clamp_parent), so every walk strictly
// descends in node index and ends within q_len steps.
__device__ __forceinline__ void tree_depths_lds(const int32_t* __restrict__ parent_b, int q_len, int* s_parent,
                                                int* s_depth) {
  for (int i = threadIdx.x; i < q_len; i += blockDim.x) s_parent[i] = clamp_parent(parent_b[i], i);
  __syncthreads();
  for (int i = threadIdx.x; i < q_len; i += blockDim.x) {
    int d = 0;
    for (int n = s_parent[i]; n >= 0; n = s_parent[n]) ++d;
    s_depth[i] = d;
  }
  __syncthreads();
}

// One block per tree.
__global__ __launch_bounds__(64) void tree_positions_kernel(const int32_t* __restrict__ parent, int q_len,
                                                            int prefix_len, int32_t* __restrict__ pos) {
  __shared__ int s_parent[kMaxQ];
  __shared__ int s_depth[kMaxQ];
  const int b = blockIdx.x;
  tree_depths_lds(parent + static_cast<int64_t>(b) * q_len, q_len, s_parent, s_depth);
  for (int i = threadIdx.x; i < q_len; i += blockDim.x) pos[static_cast<int64_t>(b) * q_len + i] = prefix_len + s_depth[i];
}

// The step's rotation: for tree b (blockIdx.y) and node i (blockIdx.x), the
// node's H query rows q_rope[b,i,h,:] and the tree's own key row
// k_rope[b, prefix+i, :] turn at prefix + depth(i).  Every row of a node shares
// its angles, so the block evaluates the float64 cos/sin of each pair once (in
// LDS) and rotates the H + 1 rows with them: the same values, rounded the same
// way, as evaluating them per row.  A ragged batch (req non-null) takes each
// request's node range, node count and prefix from its record; its query rows
// are packed request after request and its key rows start at b * kv_len
// (kv_len = the cache stride).
template <typename KV>
__global__ __launch_bounds__(256) void tree_rope_kernel(float* __restrict__ q_rope,
                                                        typename KV::storage* __restrict__ k_rope,
                                                        const int32_t* __restrict__ parent, int q_len, int H,
                                                        int half, int prefix_len, int kv_len, RopeFreq f,
                                                        const int32_t* __restrict__ req) {
  __shared__ int s_parent[kMaxQ];
  __shared__ double s_cos[kMaxHalf];
  __shared__ double s_sin[kMaxHalf];
  __shared__ int s_depth;
  const int b = blockIdx.y;
  const int i = blockIdx.x;
  int64_t node0 = static_cast<int64_t>(b) * q_len;
  if (req) {
    const int32_t* r = req + b * kReqFields;
    node0 = r[kReqQStart];
    q_len = r[kReqQLen];
    prefix_len = r[kReqPrefix];
  }
  if (i >= q_len) return;  // the whole block
  // Node i's ancestors all have indices below i (parents are clamped).
  for (int j = threadIdx.x; j <= i; j += blockDim.x) s_parent[j] = clamp_parent(parent[node0 + j], j);
  __syncthreads();
  if (threadIdx.x == 0) {
    int d = 0;
    for (int n = s_parent[i]; n >= 0; n = s_parent[n]) ++d;
    s_depth = d;
  }
  __syncthreads();
  const double pos = static_cast<double>(prefix_len + s_depth);
  for (int k = threadIdx.x; k < half; k += blockDim.x) {
    double sn, cs;
    sincos(pos * f.inv_freq[k], &sn, &cs);
    s_sin[k] = sn;
    s_cos[k] = cs;
  }
  __syncthreads();
  const int per_node = (H + 1) * half;
  for (int idx = threadIdx.x; idx < per_node; idx += blockDim.x) {
    const int h = idx / half;
    const int k = idx - h * half;
    const double c = s_cos[k];
    const double sn = s_sin[k];
    double y1, y2;
    if (h < H) {
      float* row = q_rope + ((node0 + i) * H + h) * 2 * half;
      rotate_cs_f64(static_cast<double>(row[k]), static_cast<double>(row[k + half]), c, sn, y1, y2);
      row[k] = static_cast<float>(y1);
      row[k + half] = static_cast<float>(y2);
    } else {
      typename KV::storage* row = k_rope + (static_cast<int64_t>(b) * kv_len + prefix_len + i) * 2 * half;
      rotate_cs_f64(load_f64<KV>(row + k), load_f64<KV>(row + k + half), c, sn, y1, y2);
      store_from_f64<KV>(row + k, y1);
      store_from_f64<KV>(row + k + half, y2);
    }
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
hipError_t launch_rope_neox(void* x, bool bf16, const int32_t* pos, int n_seq, int64_t n_tok, int n_head, int d_r,
                            int64_t seq_stride, int64_t tok_stride, int64_t pos_seq_stride, const RopeFreq& f,
                            hipStream_t stream) {
  const int half = d_r / 2;
  const int64_t total = static_cast<int64_t>(n_seq) * n_tok * n_head * half;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  // One pair per thread up to 2^20 workgroups; the grid strides past that.
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > (int64_t{1} << 20)) blocks = int64_t{1} << 20;
  if (bf16)
    rope_neox_kernel<BF16><<<dim3(static_cast<unsigned>(blocks)), threads, 0, stream>>>(
        static_cast<uint16_t*>(x), pos, n_tok, n_head, half, seq_stride, tok_stride, pos_seq_stride, total, f);
  else
    rope_neox_kernel<F32><<<dim3(static_cast<unsigned>(blocks)), threads, 0, stream>>>(
        static_cast<float*>(x), pos, n_tok, n_head, half, seq_stride, tok_stride, pos_seq_stride, total, f);
  return hipGetLastError();
}

hipError_t launch_tree_positions(const int32_t* parent, int B, int q_len, int prefix_len, int32_t* pos,
                                 hipStream_t stream) {
  tree_positions_kernel<<<dim3(B), 64, 0, stream>>>(parent, q_len, prefix_len, pos);
  return hipGetLastError();
}

hipError_t launch_tree_rope(float* q_rope, void* k_rope, bool bf16, const int32_t* parent, int B, int q_len, int H,
                            int d_r, int prefix_len, const RopeFreq& f, hipStream_t stream) {
  const int half = d_r / 2;
  const int kv_len = prefix_len + q_len;
  const dim3 grid(static_cast<unsigned>(q_len), static_cast<unsigned>(B));
  if (bf16)
    tree_rope_kernel<BF16><<<grid, 256, 0, stream>>>(q_rope, static_cast<uint16_t*>(k_rope), parent, q_len, H, half,
                                                     prefix_len, kv_len, f, nullptr);
  else
    tree_rope_kernel<F32><<<grid, 256, 0, stream>>>(q_rope, static_cast<float*>(k_rope), parent, q_len, H, half,
                                                    prefix_len, kv_len, f, nullptr);
  return hipGetLastError();
}

hipError_t launch_tree_rope_ragged(float* q_rope, void* k_rope, bool bf16, const int32_t* parent, const int32_t* req,
                                   int B, int max_q, int H, int d_r, int kv_stride, const RopeFreq& f,
                                   hipStream_t stream) {
  const int half = d_r / 2;
  const dim3 grid(static_cast<unsigned>(max_q), static_cast<unsigned>(B));
  if (bf16)
    tree_rope_kernel<BF16><<<grid, 256, 0, stream>>>(q_rope, static_cast<uint16_t*>(k_rope), parent, max_q, H, half,
                                                     0, kv_stride, f, req);
  else
    tree_rope_kernel<F32><<<grid, 256, 0, stream>>>(q_rope, static_cast<float*>(k_rope), parent, max_q, H, half, 0,
                                                    kv_stride, f, req);
  return hipGetLastError();
}

}  // namespace tv
