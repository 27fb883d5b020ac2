// Tree-verify MLA-absorb attention: the FP32 vector-ALU kernel, the split-kv
// merge, the launch planner and the kernel dispatch.
//
// [Verify page = "The Precision Imperative: Validating Numerical Accuracy in a
//  Custom CUDA Attention Kernel", "The Context: What Led to This Moment": masked
//  absorb attention in three parts (scores, softmax normalisation, weighted
//  accumulation).  Golden page = "The Golden Reference: A Pivotal Moment in
//  Building a Native DDTree Inference Engine", "The Absorb Form of MLA": the
//  score lives in the latent space and one latent row per key serves all heads.]
//
// Unlike the pages' one-block-per-(batch, head, query) design, a workgroup here
// owns a block of query rows (node, head) of one tree and streams the shared
// latent rows through LDS once for all of them; softmax is online (running max
// and sum per row), so scores never leave registers/LDS.  The kv range of a row
// block may be cut into splits that a second pass merges by log-sum-exp weights.
#include "tv_kernels.h"

namespace tv {

constexpr int kValuRows = 16;   // query rows per workgroup
constexpr int kValuKeys = 32;   // kv rows per LDS tile
constexpr int kValuThreads = 256;

template <typename KV>
__device__ __forceinline__ float4 load4(const void* base, int64_t elem_off);
template <>
__device__ __forceinline__ float4 load4<F32>(const void* base, int64_t elem_off) {
  return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem_off);
}
template <>
__device__ __forceinline__ float4 load4<BF16>(const void* base, int64_t elem_off) {
  const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + elem_off);
  return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
}

__device__ __forceinline__ float dot4(float4 a, float4 b, float acc) {
  acc = fmaf(a.x, b.x, acc);
  acc = fmaf(a.y, b.y, acc);
  acc = fmaf(a.z, b.z, acc);
  return fmaf(a.w, b.w, acc);
}

// Ancestor bit masks of one tree: bit m of s_anc[i] is set iff node m is node i
// or one of its ancestors.  Thread i walks its own path (<= q_len steps).
__device__ __forceinline__ void build_ancestors(const int32_t* __restrict__ parent_b, int q_len, int* s_par,
                                                unsigned long long* s_anc) {
  for (int i = threadIdx.x; i < q_len; i += blockDim.x) s_par[i] = clamp_parent(parent_b[i], i);
  __syncthreads();
  for (int i = threadIdx.x; i < q_len; i += blockDim.x) {
    unsigned long long anc = 1ull << i;
    for (int n = s_par[i]; n >= 0; n = s_par[n]) anc |= 1ull << n;
    s_anc[i] = anc;
  }
}

template <typename KV, int DC, int DR>
__global__ __launch_bounds__(kValuThreads) void attn_valu_kernel(AttnArgs a) {
  constexpr int D = DC + DR;
  constexpr int S = D + 4;          // LDS row stride (floats): 16-byte rows, banks shift by 4 per row
  constexpr int C4 = D / 4;         // float4 chunks per row
  constexpr int CPT = DC / 4;       // output float4 columns
  constexpr int RPT = kValuRows * CPT / kValuThreads;  // output rows per thread in the PV phase
  static_assert(RPT >= 1 && kValuRows % RPT == 0, "bad PV split");

  __shared__ __align__(16) float sQ[kValuRows * S];
  __shared__ __align__(16) float sK[kValuKeys * S];
  __shared__ __align__(16) float sP[kValuKeys * kValuRows];  // P transposed: [key][row]
  __shared__ float sAlpha[kValuRows];
  __shared__ float sM[kValuRows];
  __shared__ float sL[kValuRows];
  __shared__ int s_par[kMaxQ];
  __shared__ unsigned long long s_anc[kMaxQ];

  const int tid = threadIdx.x;
  const int split = blockIdx.x % a.n_split;
  const int rest = blockIdx.x / a.n_split;
  const int rb = rest % a.n_rb;
  const int b = rest / a.n_rb;
  const int r0 = rb * kValuRows;
  const int k_begin = split * a.chunk;
  const int k_end = min(a.kv_len, k_begin + a.chunk);
  const int P = a.prefix_len;

  build_ancestors(a.parent + static_cast<int64_t>(b) * a.q_len, a.q_len, s_par, s_anc);

  // Query rows: [q_lat | q_rope], zero past the last row.
  for (int idx = tid; idx < kValuRows * C4; idx += kValuThreads) {
    const int r = idx / C4;
    const int c4 = idx - r * C4;
    const int row = r0 + r;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < a.R) {
      const int64_t grow = static_cast<int64_t>(b) * a.R + row;
      if (c4 < DC / 4)
        v = *reinterpret_cast<const float4*>(a.q_lat + grow * DC + c4 * 4);
      else
        v = *reinterpret_cast<const float4*>(a.q_rope + grow * DR + (c4 - DC / 4) * 4);
    }
    *reinterpret_cast<float4*>(sQ + r * S + c4 * 4) = v;
  }
  __syncthreads();

  // Score-phase role: 16 lanes per row, each lane two keys (sl, sl + 16).
  const int sr = tid / 16;
  const int sl = tid % 16;
  const int node = min((r0 + sr) / a.H, a.q_len - 1);
  const unsigned long long anc = s_anc[node];
  float m_run = -INFINITY;
  float l_run = 0.f;

  // PV-phase role: one float4 column of RPT rows.
  const int col4 = tid % CPT;
  const int rg = tid / CPT;
  float4 o[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) o[i] = make_float4(0.f, 0.f, 0.f, 0.f);

  for (int kt = k_begin; kt < k_end; kt += kValuKeys) {
    __syncthreads();  // previous tile fully consumed
    for (int idx = tid; idx < kValuKeys * C4; idx += kValuThreads) {
      const int j = idx / C4;
      const int c4 = idx - j * C4;
      const int key = kt + j;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (key < k_end) {
        const int64_t krow = static_cast<int64_t>(b) * a.kv_len + key;
        if (c4 < DC / 4)
          v = load4<KV>(a.c_kv, krow * DC + c4 * 4);
        else
          v = load4<KV>(a.k_rope, krow * DR + (c4 - DC / 4) * 4);
      }
      *reinterpret_cast<float4*>(sK + j * S + c4 * 4) = v;
    }
    __syncthreads();

    // Scores for (row sr, keys sl and sl+16).
    float acc0 = 0.f, acc1 = 0.f;
    const float* qrow = sQ + sr * S;
    const float* k0 = sK + sl * S;
    const float* k1 = sK + (sl + 16) * S;
#pragma unroll 4
    for (int d = 0; d < D; d += 4) {
      const float4 qv = *reinterpret_cast<const float4*>(qrow + d);
      acc0 = dot4(qv, *reinterpret_cast<const float4*>(k0 + d), acc0);
      acc1 = dot4(qv, *reinterpret_cast<const float4*>(k1 + d), acc1);
    }
    const int key0 = kt + sl;
    const int key1 = kt + sl + 16;
    const bool vis0 = key0 < k_end && (key0 < P || ((anc >> (key0 - P)) & 1ull));
    const bool vis1 = key1 < k_end && (key1 < P || ((anc >> (key1 - P)) & 1ull));
    const float s0 = vis0 ? acc0 * a.sm_scale : -INFINITY;
    const float s1 = vis1 ? acc1 * a.sm_scale : -INFINITY;

    float tmax = fmaxf(s0, s1);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off, 16));
    const float m_new = fmaxf(m_run, tmax);
    const float p0 = vis0 ? expf(s0 - m_new) : 0.f;
    const float p1 = vis1 ? expf(s1 - m_new) : 0.f;
    const float alpha = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
    float psum = p0 + p1;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) psum += __shfl_xor(psum, off, 16);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    sP[sl * kValuRows + sr] = p0;
    sP[(sl + 16) * kValuRows + sr] = p1;
    if (sl == 0) sAlpha[sr] = alpha;
    __syncthreads();

    // o = o * alpha + P V for this tile (V = the latent part of the K tile).
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float al = sAlpha[rg * RPT + i];
      o[i].x *= al;
      o[i].y *= al;
      o[i].z *= al;
      o[i].w *= al;
    }
    const int nk = min(kValuKeys, k_end - kt);
    for (int j = 0; j < nk; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(sK + j * S + col4 * 4);
      const float* pj = sP + j * kValuRows + rg * RPT;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float p = pj[i];
        o[i].x = fmaf(p, v.x, o[i].x);
        o[i].y = fmaf(p, v.y, o[i].y);
        o[i].z = fmaf(p, v.z, o[i].z);
        o[i].w = fmaf(p, v.w, o[i].w);
      }
    }
  }

  __syncthreads();
  if (sl == 0) {
    sM[sr] = m_run;
    sL[sr] = l_run;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg * RPT + i;
    const int row = r0 + r;
    if (row >= a.R) continue;
    const float l = sL[r];
    const float m = sM[r];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float4 v = make_float4(o[i].x * inv, o[i].y * inv, o[i].z * inv, o[i].w * inv);
    const int64_t grow = static_cast<int64_t>(b) * a.R + row;
    if (a.n_split == 1) {
      *reinterpret_cast<float4*>(a.out + grow * DC + col4 * 4) = v;
      if (col4 == 0 && a.lse) a.lse[grow] = m + logf(l);
    } else {
      const int64_t srow = static_cast<int64_t>(split) * a.B * a.R + grow;
      *reinterpret_cast<float4*>(a.ws_o + srow * DC + col4 * 4) = v;
      if (col4 == 0) {
        a.ws_m[srow] = m;
        a.ws_l[srow] = l;
      }
    }
  }
}

// Combine split partials: w_s = l_s * exp(m_s - max_s m_s), out = sum w_s o_s / sum w_s,
// lse = max m + log(sum w_s).  One thread per (row, float4 column).
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int d_c) {
  const int cpt = d_c / 4;
  const int64_t total = static_cast<int64_t>(a.B) * a.R * cpt;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int64_t grow = idx / cpt;
  const int col4 = static_cast<int>(idx - grow * cpt);
  const int64_t stride = static_cast<int64_t>(a.B) * a.R;
  float M = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, a.ws_m[s * stride + grow]);
  float W = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < a.n_split; ++s) {
    const float l = a.ws_l[s * stride + grow];
    if (!(l > 0.f)) continue;
    const float w = l * expf(a.ws_m[s * stride + grow] - M);
    const float4 v = *reinterpret_cast<const float4*>(a.ws_o + (s * stride + grow) * d_c + col4 * 4);
    W += w;
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  const float inv = 1.f / W;
  *reinterpret_cast<float4*>(a.out + grow * d_c + col4 * 4) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (col4 == 0 && a.lse) a.lse[grow] = M + logf(W);
}

// ---------------------------------------------------------------------------
// Planning and dispatch
// ---------------------------------------------------------------------------
namespace {
constexpr int kNumCU = 256;  // MI355X; fixed so plans depend on shapes only

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
}  // namespace

AttnPlan plan_attention(const AttnShape& s) {
  AttnPlan p{};
  p.kernel = AttnKernel::kValu;
  p.rows_per_block = kValuRows;
  p.keys_per_tile = kValuKeys;
  const int R = s.q_len * s.H;
  p.n_rb = (R + p.rows_per_block - 1) / p.rows_per_block;
  const long long units = static_cast<long long>(s.B) * p.n_rb;
  int n_split = 1;
  if (units < 2 * kNumCU) {
    const long long want = (2 * kNumCU + units - 1) / units;
    const int max_split = s.kv_len / 128 > 1 ? s.kv_len / 128 : 1;  // >= 128 kv rows per split
    n_split = static_cast<int>(want < max_split ? want : max_split);
  }
  int chunk = (s.kv_len + n_split - 1) / n_split;
  chunk = (chunk + p.keys_per_tile - 1) / p.keys_per_tile * p.keys_per_tile;
  n_split = (s.kv_len + chunk - 1) / chunk;
  p.n_split = n_split;
  p.chunk = chunk;
  p.ws_bytes = 0;
  if (n_split > 1) {
    const size_t rows = static_cast<size_t>(n_split) * s.B * R;
    p.ws_o_off = 0;
    p.ws_m_off = align256(rows * s.d_c * sizeof(float));
    p.ws_l_off = p.ws_m_off + align256(rows * sizeof(float));
    p.ws_bytes = p.ws_l_off + align256(rows * sizeof(float));
  }
  return p;
}

template <typename KV, int DC>
static hipError_t launch_valu_dr(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(s.B) * plan.n_rb * plan.n_split));
  if (s.d_r == 32)
    attn_valu_kernel<KV, DC, 32><<<grid, kValuThreads, 0, stream>>>(a);
  else
    attn_valu_kernel<KV, DC, 64><<<grid, kValuThreads, 0, stream>>>(a);
  return hipGetLastError();
}

template <typename KV>
static hipError_t launch_valu(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  switch (s.d_c) {
    case 64: return launch_valu_dr<KV, 64>(s, plan, a, stream);
    case 128: return launch_valu_dr<KV, 128>(s, plan, a, stream);
    case 256: return launch_valu_dr<KV, 256>(s, plan, a, stream);
    default: return launch_valu_dr<KV, 512>(s, plan, a, stream);
  }
}

hipError_t launch_attention(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  hipError_t e = s.kv_bf16 ? launch_valu<BF16>(s, plan, a, stream) : launch_valu<F32>(s, plan, a, stream);
  if (e != hipSuccess || plan.n_split == 1) return e;
  const int64_t total = static_cast<int64_t>(s.B) * a.R * (s.d_c / 4);
  attn_merge_kernel<<<dim3(static_cast<unsigned>((total + 255) / 256)), 256, 0, stream>>>(a, s.d_c);
  return hipGetLastError();
}

}  // namespace tv
