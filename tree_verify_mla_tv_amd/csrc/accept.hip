// The steps right after verify: the target's greedy token per tree node
// (argmax over the vocabulary), the greedy walk that accepts a path of draft
// nodes, and the post-verify compaction of the accepted nodes' cache rows.
//
// [RoPE page = "Precision as Correctness: The Float64 RoPE Decision in a Custom
//  CUDA Inference Engine", "The Broader Context: A Full Native Engine from
//  Scratch" (a greedy tree-accept kernel; KV cache with post-verify compaction;
//  the loop's greedy output must equal autoregressive greedy output); Golden
//  page = "The Golden Reference: A Pivotal Moment in Building a Native DDTree
//  Inference Engine", "Recursive Refinement of the Decode Loop Design" (root,
//  draft and bonus tokens).]
#include "tv_kernels.h"

namespace tv {

namespace {

// Order-preserving 32-bit key of a float: larger value -> larger key; every NaN
// maps to the largest key and -0.0 to the key of +0.0.
__device__ __forceinline__ uint32_t float_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (x != x) return 0xffffffffu;
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// (key, index) packed so that the max of the packed values is the largest key
// at its lowest index.
__device__ __forceinline__ unsigned long long pack(uint32_t key, uint32_t idx) {
  return (static_cast<unsigned long long>(key) << 32) | static_cast<unsigned long long>(~idx);
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }

template <bool BF16>
__device__ __forceinline__ float load_logit(const void* row, int64_t i) {
  if (BF16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(row)[i]) << 16);
  return static_cast<const float*>(row)[i];
}

// Running maximum of one thread, which sees its indices in increasing order:
// a value replaces the best if it is larger, or if it is the first NaN, so the
// first index wins ties (-0.0 == +0.0 under '>') and the first NaN wins.
struct Best {
  float v = -INFINITY;
  int i = -1;  // -1: nothing seen yet
  __device__ __forceinline__ void see(float x, int idx) {
    const bool take = (i < 0) | (x > v) | ((x != x) & (v == v));
    v = take ? x : v;
    i = take ? idx : i;
  }
  __device__ __forceinline__ unsigned long long packed() const {
    return i < 0 ? 0ull : pack(float_key(v), static_cast<uint32_t>(i));
  }
};

// One workgroup (256 threads) per row.  VEC: the row is 16-byte aligned and a
// whole number of 16-byte chunks (4 floats or 8 bf16), read with 16-byte loads.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void argmax_rows_kernel(const void* __restrict__ logits, int64_t n_rows, int vocab,
                                                          int32_t* __restrict__ out) {
  constexpr int kElem = BF16 ? 2 : 4;
  constexpr int kPerChunk = 16 / kElem;
  const int64_t row = blockIdx.x;
  if (row >= n_rows) return;
  const unsigned char* base = static_cast<const unsigned char*>(logits) + row * static_cast<int64_t>(vocab) * kElem;
  Best best;
  if (VEC) {
    const int chunks = vocab / kPerChunk;
    const uint4* p = reinterpret_cast<const uint4*>(base);
    int c = threadIdx.x;
    // Eight 16-byte chunks in flight per thread.
    for (; c + 7 * 256 < chunks; c += 8 * 256) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p[c + u * 256];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        const int i0 = (c + u * 256) * kPerChunk;
#pragma unroll
        for (int e = 0; e < kPerChunk; ++e)
          best.see(BF16 ? __uint_as_float((w[e / 2] >> (16 * (e & 1))) << 16) : __uint_as_float(w[e]), i0 + e);
      }
    }
    for (; c < chunks; c += 256) {
      const uint4 v = p[c];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      const int i0 = c * kPerChunk;
#pragma unroll
      for (int e = 0; e < kPerChunk; ++e)
        best.see(BF16 ? __uint_as_float((w[e / 2] >> (16 * (e & 1))) << 16) : __uint_as_float(w[e]), i0 + e);
    }
  } else {
    for (int i = threadIdx.x; i < vocab; i += 256) best.see(load_logit<BF16>(base, i), i);
  }
  // Across threads: (key, inverted index) maximum, wave then workgroup.
  unsigned long long m = best.packed();
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = umax64(m, __shfl_xor(m, off));
  __shared__ unsigned long long s_best[4];
  if ((threadIdx.x & 63) == 0) s_best[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long r = umax64(umax64(s_best[0], s_best[1]), umax64(s_best[2], s_best[3]));
    out[row] = static_cast<int32_t>(~static_cast<uint32_t>(r & 0xffffffffu));
  }
}

// One wave per tree: lane l holds nodes l + 64 j (j < kMaxQ / 64), with their
// parents and draft tokens.  From the current node cur, the wanted token is
// target[cur]; the lowest node that is a child of cur carrying that token is
// accepted (one ballot per group of 64 nodes, the lowest group first), until
// none is.  A node whose parent lies outside [0, i) is never a candidate, so
// such a node is simply never accepted (and the walk takes at most q_len - 1
// steps).
__global__ __launch_bounds__(64) void tree_accept_kernel(const int32_t* __restrict__ parent,
                                                         const int32_t* __restrict__ draft,
                                                         const int32_t* __restrict__ target, int q_len,
                                                         int32_t* __restrict__ path, int32_t* __restrict__ accept_len,
                                                         int32_t* __restrict__ bonus) {
  constexpr int kPer = kMaxQ / 64;
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t o = static_cast<int64_t>(b) * q_len;
  __shared__ int32_t s_target[kMaxQ];
  int32_t par[kPer], tok[kPer], my_step[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int node = lane + 64 * j;
    const bool in = node < q_len;
    par[j] = in ? parent[o + node] : -2;
    tok[j] = in ? draft[o + node] : 0;
    my_step[j] = node == 0 ? 0 : -1;  // position of the node on the accepted path
    if (in) s_target[node] = target[o + node];
  }
  __syncthreads();
  int cur = 0;
  int n = 0;
  for (int depth = 1; depth < q_len; ++depth) {
    const int32_t want = s_target[cur];
    int c = -1;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int node = lane + 64 * j;
      const bool cand = node < q_len && node > 0 && par[j] == cur && par[j] < node && tok[j] == want;
      const unsigned long long m = __ballot(cand);
      if (c < 0 && m != 0ull) c = 64 * j + __ffsll(static_cast<long long>(m)) - 1;
    }
    if (c < 0) break;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (lane + 64 * j == c) my_step[j] = depth;
    cur = c;
    n = depth;
  }
  // path[k] = the node whose step is k; -1 past the accepted length.
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (lane + 64 * j < q_len) path[o + lane + 64 * j] = -1;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (my_step[j] >= 0) path[o + my_step[j]] = lane + 64 * j;
  if (lane == 0) {
    accept_len[b] = n;
    bonus[b] = s_target[cur];
  }
}

// Compaction: row prefix_len + k of tree b takes row prefix_len + path[b][k],
// k = 1 .. accept_len[b].  Each thread owns fixed 16-byte chunks of a row and
// walks k upward.  Since path[k] >= k (nodes precede their children on the
// path), a row is read before any write to it: the write to row P + k2 can hit
// the source of an earlier k1 < k2 only, which the same thread has already
// read (same thread, same address, program order); and a read for k never
// hits a row already written (P + path[k] >= P + k).  So no barrier is needed.
// Reads run up to eight rows ahead of the writes for the same reason.
__global__ __launch_bounds__(256) void kv_compact_kernel(unsigned char* __restrict__ c_kv,
                                                         unsigned char* __restrict__ k_rope,
                                                         const int32_t* __restrict__ path,
                                                         const int32_t* __restrict__ accept_len, int prefix_len,
                                                         int kv_len, int q_len, int lat_chunks, int rope_chunks) {
  const int b = blockIdx.y;
  const int chunk = blockIdx.x * blockDim.x + threadIdx.x;
  if (chunk >= lat_chunks + rope_chunks) return;
  const bool lat = chunk < lat_chunks;
  const int row_chunks = lat ? lat_chunks : rope_chunks;
  const int col = lat ? chunk : chunk - lat_chunks;
  uint4* base = reinterpret_cast<uint4*>(lat ? c_kv : k_rope) + static_cast<int64_t>(b) * kv_len * row_chunks + col;
  const int32_t* pb = path + static_cast<int64_t>(b) * q_len;
  const int n = min(max(accept_len[b], 0), q_len - 1);
  for (int k0 = 1; k0 <= n; k0 += 8) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + u;
      if (k <= n) {
        const int m = min(max(pb[k], 0), q_len - 1);
        v[u] = base[static_cast<int64_t>(prefix_len + m) * row_chunks];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + u;
      if (k <= n) base[static_cast<int64_t>(prefix_len + k) * row_chunks] = v[u];
    }
  }
}

}  // namespace

hipError_t launch_argmax_rows(const void* logits, bool bf16, bool vec, int64_t n_rows, int vocab, int32_t* out,
                              hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(n_rows));
  if (bf16) {
    if (vec) argmax_rows_kernel<true, true><<<grid, 256, 0, stream>>>(logits, n_rows, vocab, out);
    else argmax_rows_kernel<true, false><<<grid, 256, 0, stream>>>(logits, n_rows, vocab, out);
  } else {
    if (vec) argmax_rows_kernel<false, true><<<grid, 256, 0, stream>>>(logits, n_rows, vocab, out);
    else argmax_rows_kernel<false, false><<<grid, 256, 0, stream>>>(logits, n_rows, vocab, out);
  }
  return hipGetLastError();
}

hipError_t launch_tree_accept(const int32_t* parent, const int32_t* draft, const int32_t* target, int B, int q_len,
                              int32_t* path, int32_t* accept_len, int32_t* bonus, hipStream_t stream) {
  tree_accept_kernel<<<dim3(static_cast<unsigned>(B)), 64, 0, stream>>>(parent, draft, target, q_len, path,
                                                                         accept_len, bonus);
  return hipGetLastError();
}

hipError_t launch_kv_compact(void* c_kv, void* k_rope, int elem_bytes, const int32_t* path, const int32_t* accept_len,
                             int prefix_len, int B, int kv_len, int q_len, int d_c, int d_r, hipStream_t stream) {
  const int lat_chunks = d_c * elem_bytes / 16;
  const int rope_chunks = d_r * elem_bytes / 16;
  const dim3 grid(static_cast<unsigned>((lat_chunks + rope_chunks + 255) / 256), static_cast<unsigned>(B));
  kv_compact_kernel<<<grid, 256, 0, stream>>>(static_cast<unsigned char*>(c_kv), static_cast<unsigned char*>(k_rope),
                                              path, accept_len, prefix_len, kv_len, q_len, lat_chunks, rope_chunks);
  return hipGetLastError();
}

}  // namespace tv
