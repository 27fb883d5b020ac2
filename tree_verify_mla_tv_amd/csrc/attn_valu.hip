// Tree-verify MLA-absorb attention: the FP32 vector-ALU kernel (all supported
// shapes; the fp32-cache path).
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

template <typename KV, int DC, int DR>
__device__ __forceinline__ void attn_valu_unit(const AttnArgs& a, const Unit& w) {
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
  __shared__ unsigned long long s_anc[kMaxQ * kAncWords];

  const int tid = threadIdx.x;
  const int r0 = w.rb * kValuRows;
  const int k_begin = w.k_begin;
  const int k_end = w.k_end;
  const int P = w.P;

  build_ancestors(a.parent + w.par0, w.q_len, s_par, s_anc);

  // Query rows: [q_lat | q_rope], zero past the last row.
  for (int idx = tid; idx < kValuRows * C4; idx += kValuThreads) {
    const int r = idx / C4;
    const int c4 = idx - r * C4;
    const int row = r0 + r;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < w.R) {
      const int64_t grow = w.row0 + row;
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
  const int node = min((r0 + sr) / a.H, w.q_len - 1);
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
        const int64_t krow = w.kv_row0 + key;
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
    const bool vis0 = key_visible(s_anc, node, key0, P, k_end) != 0u;
    const bool vis1 = key_visible(s_anc, node, key1, P, k_end) != 0u;
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
    if (row >= w.R) continue;
    const float l = sL[r];
    const float m = sM[r];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float4 v = make_float4(o[i].x * inv, o[i].y * inv, o[i].z * inv, o[i].w * inv);
    const int64_t grow = w.row0 + row;
    if (w.slot < 0) {
      *reinterpret_cast<float4*>(a.out + grow * DC + col4 * 4) = v;
      if (col4 == 0 && a.lse) a.lse[grow] = m + logf(l);
    } else {
      const int64_t srow = w.slot * kValuRows + r;
      *reinterpret_cast<float4*>(a.ws_o + srow * DC + col4 * 4) = v;
      if (col4 == 0) {
        a.ws_m[srow] = m;
        a.ws_l[srow] = l;
      }
    }
  }
}

// A uniform batch: one unit per workgroup.
template <typename KV, int DC, int DR>
__global__ __launch_bounds__(kValuThreads) void attn_valu_kernel(AttnArgs a) {
  attn_valu_unit<KV, DC, DR>(a, decode_unit(a, unit_of_block(a, blockIdx.x)));
}

// A ragged batch: a persistent grid taking units from its XCD's counter.
template <typename KV, int DC, int DR>
__global__ __launch_bounds__(kValuThreads) void attn_valu_ragged_kernel(AttnArgs) {
  for_each_ragged_unit([](const AttnArgs& a, const Unit& w) { attn_valu_unit<KV, DC, DR>(a, w); });
}

template <typename KV, int DC>
static hipError_t launch_valu_dr(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(plan.units));
  if (a.req) {
    if (s.d_r == 32)
      attn_valu_ragged_kernel<KV, DC, 32><<<grid, kValuThreads, 0, stream>>>(a);
    else
      attn_valu_ragged_kernel<KV, DC, 64><<<grid, kValuThreads, 0, stream>>>(a);
  } else if (s.d_r == 32) {
    attn_valu_kernel<KV, DC, 32><<<grid, kValuThreads, 0, stream>>>(a);
  } else {
    attn_valu_kernel<KV, DC, 64><<<grid, kValuThreads, 0, stream>>>(a);
  }
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

hipError_t launch_attn_valu(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  return s.kv_bf16 ? launch_valu<BF16>(s, plan, a, stream) : launch_valu<F32>(s, plan, a, stream);
}

}  // namespace tv
