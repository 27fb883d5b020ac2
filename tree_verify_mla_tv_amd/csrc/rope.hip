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

// The step's rotation: for tree b (blockIdx.y) and the nodes i0 .. i0 + npb - 1
// of group blockIdx.x (i0 = npb * blockIdx.x), each node's H query rows
// q_rope[b,i,h,:] and the tree's own key row k_rope[b, prefix+i, :] turn at
// prefix + depth(i).  Every row of a node shares its angles, so the block
// evaluates each node's float64 cos/sin once (in LDS) and rotates its H + 1
// rows with them: the same values, rounded the same way, as evaluating them
// per row.  The query rows are the traffic (H rows per node against one key
// row): each thread first issues the loads of up to kRopePrefetch items (an
// item = 4 consecutive pairs of one row, 16 bytes of each half) into
// registers, then the block walks the parent chains and evaluates the angles
// while those loads are in flight, then rotates and stores.  Items past the
// prefetch (only when npb * H * half / 4 exceeds 256 kRopePrefetch) and rows
// whose half is not a multiple of 4 take a plain loop.  A ragged batch (req
// non-null) takes each request's node range, node count and prefix from its
// record; its query rows are packed request after request and its key rows
// start at b * kv_len (kv_len = the cache stride).
constexpr int kRopeThreads = 256;
constexpr int kRopePrefetch = 1;  // measured: 2-3 % faster than 2 or 4 at 64 heads x 64 dims
constexpr int kRopeMaxNodes = 8;
static_assert(kMaxQ <= kRopeThreads && kRopeMaxNodes * kMaxHalf <= 2 * kRopeThreads,
              "one parent and at most two angles per thread");

template <typename KV, bool VEC>
__global__ __launch_bounds__(kRopeThreads) void tree_rope_kernel(float* __restrict__ q_rope,
                                                                 typename KV::storage* __restrict__ k_rope,
                                                                 const int32_t* __restrict__ parent, int q_len,
                                                                 int H, int half, int prefix_len, int kv_len,
                                                                 int npb, RopeFreq f,
                                                                 const int32_t* __restrict__ req) {
  __shared__ int s_parent[kMaxQ];
  __shared__ double s_cs[kRopeMaxNodes][kMaxHalf][2];
  const int b = blockIdx.y;
  const int i0 = blockIdx.x * npb;
  int64_t node0 = static_cast<int64_t>(b) * q_len;
  if (req) {
    const int32_t* r = req + b * kReqFields;
    node0 = r[kReqQStart];
    q_len = r[kReqQLen];
    prefix_len = r[kReqPrefix];
  }
  if (i0 >= q_len) return;  // the whole block
  const int nn = min(npb, q_len - i0);
  const int t = threadIdx.x;
  const int i_end = i0 + nn;   // <= q_len <= kMaxQ = 256 = kRopeThreads: one parent per thread
  const int n_ang = nn * half;  // angles of the block: at most 2 per thread

  // What the angle phase reads is loaded first: memory waits count loads in
  // issue order, so waiting for these does not wait for the row loads below.
  const int par = parent[node0 + min(t, i_end - 1)];
  const double fr0 = f.inv_freq[min(t, n_ang - 1) % half];
  const double fr1 = f.inv_freq[min(t + kRopeThreads, n_ang - 1) % half];

  // Query rows of the block's nodes: contiguous, nn * H rows of 2 * half floats.
  float* const q0 = q_rope + (node0 + i0) * H * 2 * half;
  // VEC: half is a multiple of 4 (the host's choice), items of 16 bytes.
  const int qpr = half >> 2;                          // items per row
  const int items = VEC ? nn * H * qpr : 0;
  // The loads are unconditional (items past the end re-read the last item, and
  // only in-range items are stored), so they all issue before any wait.
  float4 x1[kRopePrefetch], x2[kRopePrefetch];
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < kRopePrefetch; ++k) {
      const int it = min(t + k * kRopeThreads, items - 1);
      const int row = it / qpr, c = it - row * qpr;
      const float* rp = q0 + static_cast<int64_t>(row) * 2 * half + 4 * c;
      x1[k] = *reinterpret_cast<const float4*>(rp);
      x2[k] = *reinterpret_cast<const float4*>(rp + half);
    }
  }


  // Depths (ancestors have lower indices: parents are clamped) and angles:
  // each angle's thread walks its node's chain itself (the chain is short and
  // in LDS; one barrier fewer than a shared depth table).
  s_parent[t] = t < i_end ? clamp_parent(par, t) : -1;  // unconditional: the load stays where it is
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int j = t + r * kRopeThreads;
    if (j < n_ang) {
      const int n = j / half, k = j - n * half;
      int d = 0;
      for (int m = s_parent[i0 + n]; m >= 0; m = s_parent[m]) ++d;
      double sn, cs;
      sincos(static_cast<double>(prefix_len + d) * (r == 0 ? fr0 : fr1), &sn, &cs);
      s_cs[n][k][0] = cs;
      s_cs[n][k][1] = sn;
    }
  }
  __syncthreads();
  // The loaded values are first used here.  The empty asm hands them over
  // as if redefined at this point, so the compiler cannot move their float64
  // conversions up next to the loads (where the waits for the data would
  // serialise the loads behind each other).
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < kRopePrefetch; ++k) {
      asm volatile("" : "+v"(x1[k].x), "+v"(x1[k].y), "+v"(x1[k].z), "+v"(x1[k].w));
      asm volatile("" : "+v"(x2[k].x), "+v"(x2[k].y), "+v"(x2[k].z), "+v"(x2[k].w));
    }
  }

  auto rot = [&](float a1, float a2, int n, int k, float& y1, float& y2) {
    double r1, r2;
    rotate_cs_f64(static_cast<double>(a1), static_cast<double>(a2), s_cs[n][k][0], s_cs[n][k][1], r1, r2);
    y1 = static_cast<float>(r1);
    y2 = static_cast<float>(r2);
  };
#pragma unroll
  for (int k = 0; k < kRopePrefetch; ++k) {
    const int it = t + k * kRopeThreads;
    if (it < items) {
      const int row = it / qpr, c = it - row * qpr;
      const int n = row / H, kk = 4 * c;
      float4 y1, y2;
      rot(x1[k].x, x2[k].x, n, kk + 0, y1.x, y2.x);
      rot(x1[k].y, x2[k].y, n, kk + 1, y1.y, y2.y);
      rot(x1[k].z, x2[k].z, n, kk + 2, y1.z, y2.z);
      rot(x1[k].w, x2[k].w, n, kk + 3, y1.w, y2.w);
      float* rp = q0 + static_cast<int64_t>(row) * 2 * half + kk;
      *reinterpret_cast<float4*>(rp) = y1;
      *reinterpret_cast<float4*>(rp + half) = y2;
    }
  }
  // The rest of the query rows: items past the prefetch, or one pair at a
  // time when half is not a multiple of 4.
  if constexpr (VEC) {
    for (int it = t + kRopePrefetch * kRopeThreads; it < items; it += kRopeThreads) {
      const int row = it / qpr, c = it - row * qpr;
      const int n = row / H, kk = 4 * c;
      float* rp = q0 + static_cast<int64_t>(row) * 2 * half + kk;
      const float4 a1 = *reinterpret_cast<const float4*>(rp);
      const float4 a2 = *reinterpret_cast<const float4*>(rp + half);
      float4 y1, y2;
      rot(a1.x, a2.x, n, kk + 0, y1.x, y2.x);
      rot(a1.y, a2.y, n, kk + 1, y1.y, y2.y);
      rot(a1.z, a2.z, n, kk + 2, y1.z, y2.z);
      rot(a1.w, a2.w, n, kk + 3, y1.w, y2.w);
      *reinterpret_cast<float4*>(rp) = y1;
      *reinterpret_cast<float4*>(rp + half) = y2;
    }
  } else {
    for (int it = t; it < nn * H * half; it += kRopeThreads) {
      const int row = it / half, k = it - row * half;
      float* rp = q0 + static_cast<int64_t>(row) * 2 * half;
      float y1, y2;
      rot(rp[k], rp[k + half], row / H, k, y1, y2);
      rp[k] = y1;
      rp[k + half] = y2;
    }
  }
  // The tree's own key rows.
  for (int j = t; j < nn * half; j += kRopeThreads) {
    const int n = j / half, k = j - n * half;
    typename KV::storage* row = k_rope + (static_cast<int64_t>(b) * kv_len + prefix_len + i0 + n) * 2 * half;
    double y1, y2;
    rotate_cs_f64(load_f64<KV>(row + k), load_f64<KV>(row + k + half), s_cs[n][k][0], s_cs[n][k][1], y1, y2);
    store_from_f64<KV>(row + k, y1);
    store_from_f64<KV>(row + k + half, y2);
  }
}

// Nodes per workgroup: as many as keep the block's query items within the
// prefetch (at most kRopeMaxNodes, at least one).
inline int rope_nodes_per_block(int H, int half) {
  const int qpr = (half & 3) == 0 ? half / 4 : half;
  const long long per_node = static_cast<long long>(H) * qpr;
  long long n = static_cast<long long>(kRopeThreads) * kRopePrefetch / (per_node > 0 ? per_node : 1);
  return static_cast<int>(n < 1 ? 1 : (n > kRopeMaxNodes ? kRopeMaxNodes : n));
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

template <typename KV>
void tree_rope_launch(const dim3& grid, float* q_rope, typename KV::storage* k_rope, const int32_t* parent, int q_len,
                      int H, int half, int prefix_len, int kv_len, int npb, const RopeFreq& f, const int32_t* req,
                      hipStream_t stream) {
  if ((half & 3) == 0)
    tree_rope_kernel<KV, true><<<grid, kRopeThreads, 0, stream>>>(q_rope, k_rope, parent, q_len, H, half, prefix_len,
                                                                  kv_len, npb, f, req);
  else
    tree_rope_kernel<KV, false><<<grid, kRopeThreads, 0, stream>>>(q_rope, k_rope, parent, q_len, H, half, prefix_len,
                                                                   kv_len, npb, f, req);
}

hipError_t launch_tree_rope(float* q_rope, void* k_rope, bool bf16, const int32_t* parent, int B, int q_len, int H,
                            int d_r, int prefix_len, const RopeFreq& f, hipStream_t stream) {
  const int half = d_r / 2;
  const int kv_len = prefix_len + q_len;
  const int npb = rope_nodes_per_block(H, half);
  const dim3 grid(static_cast<unsigned>((q_len + npb - 1) / npb), static_cast<unsigned>(B));
  if (bf16)
    tree_rope_launch<BF16>(grid, q_rope, static_cast<uint16_t*>(k_rope), parent, q_len, H, half, prefix_len, kv_len,
                           npb, f, nullptr, stream);
  else
    tree_rope_launch<F32>(grid, q_rope, static_cast<float*>(k_rope), parent, q_len, H, half, prefix_len, kv_len, npb,
                          f, nullptr, stream);
  return hipGetLastError();
}

hipError_t launch_tree_rope_ragged(float* q_rope, void* k_rope, bool bf16, const int32_t* parent, const int32_t* req,
                                   int B, int max_q, int H, int d_r, int kv_stride, const RopeFreq& f,
                                   hipStream_t stream) {
  const int half = d_r / 2;
  const int npb = rope_nodes_per_block(H, half);
  const dim3 grid(static_cast<unsigned>((max_q + npb - 1) / npb), static_cast<unsigned>(B));
  if (bf16)
    tree_rope_launch<BF16>(grid, q_rope, static_cast<uint16_t*>(k_rope), parent, max_q, H, half, 0, kv_stride, npb,
                           f, req, stream);
  else
    tree_rope_launch<F32>(grid, q_rope, static_cast<float*>(k_rope), parent, max_q, H, half, 0, kv_stride, npb, f,
                          req, stream);
  return hipGetLastError();
}

}  // namespace tv
