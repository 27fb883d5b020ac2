// Tree-verify MLA-absorb attention on the CDNA4 matrix cores (bf16 latent
// cache, d_c = 512, d_r = 64; fp32 accumulation).
//
// [Verify page = "The Precision Imperative: Validating Numerical Accuracy in a
//  Custom CUDA Attention Kernel", "The Context: What Led to This Moment"; Golden
//  page = "The Golden Reference: A Pivotal Moment in Building a Native DDTree
//  Inference Engine", "The Absorb Form of MLA".]  With the key projection
// absorbed into the query, every head of a tree attends to the same latent rows,
// so one tree's H * q_len query rows form a dense [R x 576] x [576 x kv] score
// product and a dense [R x kv] x [kv x 512] output product.  Those two products
// run on v_mfma_f32_32x32x16_bf16; the rest (mask, softmax) is VALU work.
//
// Workgroup = 4 waves, one per SIMD; wave w owns 32 query rows.  Per wave:
//   * its 32 query rows live in registers for the whole kv sweep, pre-scaled by
//     sm_scale * log2(e) and rounded once to bf16 (144 VGPRs, the B operand of
//     S^T = K Q^T);
//   * the 32 x 512 fp32 output block lives in 256 accumulator registers
//     (O^T = V^T P^T, so a lane owns one query row in both products and the
//     softmax state is lane-local);
// Per kv tile of 32 latent rows (shared by all 4 waves through LDS):
//   * the tile is copied HBM/L2 -> LDS with global_load_lds_dwordx4 (no VGPR
//     round trip), double-buffered so tile t+1 streams in while tile t is used;
//   * QK reads the tile row-major (ds_read_b128); PV reads the same bytes
//     transposed with ds_read_b64_tr_b16, so no second, transposed copy exists;
//   * softmax is online in base 2 against a per-row reference max fixed by the
//     first tile the row sees; the accumulators are never rescaled.  Weights
//     exp2(s - m_ref) may exceed 1 (fp32 and bf16 carry them exactly as well);
//     if some later score exceeds m_ref by more than 2^64 the workgroup sweeps
//     its kv range once more, with m_ref = the exact row max for the rows that
//     ran out of headroom, so nothing overflows for any finite input.
// Scores of a tile that holds tree rows are masked by the ancestor bit mask.
#include "tv_kernels.h"

namespace tv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(8))) short i16x8_t;

namespace mf {
constexpr int DC = 512, DR = 64, D = DC + DR;
constexpr int KSTEPS = D / 16;                      // 36 k-steps of the score product
constexpr int KSTEPS_LAT = DC / 16;                 // 32 of them in the latent part
constexpr int kPadBytes = 32;                       // gap between latent rows in LDS
constexpr int kLatRowBytes = DC * 2 + kPadBytes;    // 1056
constexpr int kLatBytes = kMfmaKeys * kLatRowBytes; // 33792
constexpr int kRopeBytes = kMfmaKeys * DR * 2;      // 4096
constexpr int kBufBytes = kLatBytes + kRopeBytes;   // 37888
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kHeadroom = 64.0f;                  // log2 units above m_ref before a re-sweep
}  // namespace mf

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

__shared__ __align__(16) unsigned char g_kv_buf0[mf::kBufBytes];
__shared__ __align__(16) unsigned char g_kv_buf1[mf::kBufBytes];

// Copy kv rows [kt, kt + 32) of one tree into an LDS tile buffer.  Rows past
// k_end repeat row k_end - 1 (finite data; their scores are masked).
//   latent rows:  row k at buf + k * kLatRowBytes, 64 chunks of 16 B; wave w
//                 copies rows 8w .. 8w+7, one wave-wide 1 KB copy per row.
//   rope rows:    wave w copies keys 8w .. 8w+7 into buf + kLatBytes + 1024 w,
//                 chunk-major: 16-byte chunk c of key k at slot c * 8 + (k % 8).
__device__ __forceinline__ void stage_tile(unsigned char* buf, const uint16_t* __restrict__ ckv_b,
                                           const uint16_t* __restrict__ krope_b, int kt, int k_end, int wave,
                                           int lane) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int k = wave * 8 + r;
    const int key = min(kt + k, k_end - 1);
    const uint16_t* src = ckv_b + static_cast<int64_t>(key) * mf::DC + lane * 8;
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src), (lds_ptr_t)(buf + k * mf::kLatRowBytes), 16, 0, 0);
  }
  const int c = lane >> 3;
  const int kl = lane & 7;
  const int key = min(kt + wave * 8 + kl, k_end - 1);
  const uint16_t* src = krope_b + static_cast<int64_t>(key) * mf::DR + c * 8;
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src), (lds_ptr_t)(buf + mf::kLatBytes + wave * 1024), 16, 0, 0);
}

// Everything one wave does with one staged tile.
struct WaveState {
  f32x16_t o[16];   // O^T blocks: o[db][i] = out[row][32 db + 8 (i/4) + 4 g2 + i%4]
  float m_ref;      // reference max (log2 units) the exponentials are taken against
  float m_seen;     // exact running max of the row's visible scores (log2 units)
  float l;          // this lane's share of the row's softmax denominator
  bool over;        // a score exceeded m_ref + kHeadroom
};

__device__ __forceinline__ void tile_compute(const unsigned char* buf, const bf16x8_t* qf,
                                             const unsigned char* qrope, WaveState& st, int lane, int kt, int k_end,
                                             int P, unsigned long long anc) {
  const int g2 = lane >> 5;
  const int key_l = lane & 31;
  // ---- S^T = K Q^T: 36 MFMAs 32x32x16, one accumulator chain.  The latent
  // part of Q is in registers (qf), the rope part in LDS (qrope, chunk-major).
  f32x16_t sacc = {};
  const unsigned char* lat = buf + key_l * mf::kLatRowBytes + g2 * 16;
#pragma unroll
  for (int ks = 0; ks < mf::KSTEPS_LAT; ++ks) {
    const bf16x8_t k0 = *reinterpret_cast<const bf16x8_t*>(lat + ks * 32);
    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[ks], sacc, 0, 0, 0);
  }
  const unsigned char* rope = buf + mf::kLatBytes + (key_l >> 3) * 1024 + (key_l & 7) * 16;
#pragma unroll
  for (int ks = mf::KSTEPS_LAT; ks < mf::KSTEPS; ++ks) {
    const int c = g2 + 2 * (ks - mf::KSTEPS_LAT);
    const bf16x8_t k0 = *reinterpret_cast<const bf16x8_t*>(rope + c * 128);
    const bf16x8_t q0 = *reinterpret_cast<const bf16x8_t*>(qrope + c * (kMfmaRows * 16));
    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, q0, sacc, 0, 0, 0);
  }
  float s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = sacc[i];

  // ---- mask: register i holds key kt + 8 (i/4) + 4 g2 + i%4.
  if (kt + kMfmaKeys > P || kt + kMfmaKeys > k_end) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kt + 8 * (i >> 2) + 4 * g2 + (i & 3);
      const int rel = key - P;  // tree node of a tree row; the bit test is valid for 0 <= rel < 64
      const bool tree_vis = (static_cast<unsigned>(rel) < 64u) & (((anc >> (rel & 63)) & 1ull) != 0ull);
      const bool vis = (key < k_end) & ((key < P) | tree_vis);
      s[i] = vis ? s[i] : -INFINITY;
    }
  }

  // ---- softmax weights (base 2) against the row's reference max.
  float mt = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[i]);
  mt = fmaxf(mt, __shfl_xor(mt, 32));  // lanes l and l ^ 32 hold the same row
  st.m_seen = fmaxf(st.m_seen, mt);
  if (st.m_ref == -INFINITY) st.m_ref = mt;  // first visible tile: o and l are still 0
  st.over = st.over || (mt > st.m_ref + mf::kHeadroom);
  const float mref = st.m_ref == -INFINITY ? 0.f : st.m_ref;
  bf16x8_t p0, p1;
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p0[i] = static_cast<__bf16>(exp2f(s[i] - mref));
    p1[i] = static_cast<__bf16>(exp2f(s[i + 8] - mref));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) lsum += static_cast<float>(p0[i]) + static_cast<float>(p1[i]);
  st.l += lsum;

  // ---- O^T += V^T P^T: 16 d-blocks x 2 key halves.  The A operand (V^T) comes
  // from the row-major tile through ds_read_b64_tr_b16: in each 16-lane group,
  // lane j points at 4 consecutive d of key row kb + j/4, and receives back the
  // 4 keys kb .. kb+3 of d = d0 + j.
  const int grp = lane >> 4;
  const int j = lane & 15;
  const int d0 = 16 * (grp & 1) + 4 * (j & 3);
  const unsigned char* vbase = buf + (4 * g2 + (j >> 2)) * mf::kLatRowBytes + d0 * 2;
#pragma unroll
  for (int db = 0; db < 16; ++db) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const unsigned char* va = vbase + (16 * h) * mf::kLatRowBytes + db * 64;
      const unsigned char* vb = va + 8 * mf::kLatRowBytes;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(va));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(vb));
      const i16x8_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8_t v = __builtin_bit_cast(bf16x8_t, both);
      st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, h ? p1 : p0, st.o[db], 0, 0, 0);
    }
  }
}

__global__ __launch_bounds__(kMfmaThreads, 1) void attn_mfma_bf16_kernel(AttnArgs a) {
  __shared__ int s_par[kMaxQ];
  __shared__ unsigned long long s_anc[kMaxQ];
  __shared__ __align__(16) unsigned char s_qrope[kMfmaRows * mf::DR * 2];  // 16 KB
  __shared__ int s_redo;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g2 = lane >> 5;
  const Unit w = decode_unit(a, blockIdx.x);
  const int b = w.b;
  const int P = a.prefix_len;
  const uint16_t* ckv_b = static_cast<const uint16_t*>(a.c_kv) + static_cast<int64_t>(b) * a.kv_len * mf::DC;
  const uint16_t* krope_b = static_cast<const uint16_t*>(a.k_rope) + static_cast<int64_t>(b) * a.kv_len * mf::DR;

  // First tile in flight while the prologue runs.
  const int n_tiles = (w.k_end - w.k_begin + kMfmaKeys - 1) / kMfmaKeys;
  stage_tile(g_kv_buf0, ckv_b, krope_b, w.k_begin, w.k_end, wave, lane);

  build_ancestors(a.parent + static_cast<int64_t>(b) * a.q_len, a.q_len, s_par, s_anc);

  const int row0 = w.rb * kMfmaRows + wave * 32;
  const bool wave_active = row0 < a.R;
  const int row = row0 + (lane & 31);
  const bool row_valid = row < a.R;
  const int node = min(row / a.H, a.q_len - 1);
  const unsigned long long anc = s_anc[node];

  // Query fragments: q[row][8 g2 + 16 ks .. + 7] * sm_scale * log2(e) as bf16.
  // Latent part (ks < 32) in registers; rope part in LDS, chunk-major:
  // 16-byte chunk c of block row r at s_qrope + (c * 128 + r) * 16.
  bf16x8_t qf[mf::KSTEPS_LAT];
  {
    const float sc = a.sm_scale * mf::kLog2e;
    const int64_t grow = static_cast<int64_t>(b) * a.R + (row_valid ? row : 0);
    const float* ql = a.q_lat + grow * mf::DC + 8 * g2;
    const float* qr = a.q_rope + grow * mf::DR + 8 * g2;
    const float z = row_valid ? sc : 0.f;
#pragma unroll
    for (int ks = 0; ks < mf::KSTEPS; ++ks) {
      const float* src = ks < mf::KSTEPS_LAT ? ql + 16 * ks : qr + 16 * (ks - mf::KSTEPS_LAT);
      const float4 x0 = *reinterpret_cast<const float4*>(src);
      const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
      bf16x8_t v;
      v[0] = static_cast<__bf16>(x0.x * z);
      v[1] = static_cast<__bf16>(x0.y * z);
      v[2] = static_cast<__bf16>(x0.z * z);
      v[3] = static_cast<__bf16>(x0.w * z);
      v[4] = static_cast<__bf16>(x1.x * z);
      v[5] = static_cast<__bf16>(x1.y * z);
      v[6] = static_cast<__bf16>(x1.z * z);
      v[7] = static_cast<__bf16>(x1.w * z);
      if (ks < mf::KSTEPS_LAT) {
        qf[ks] = v;
      } else {
        const int c = g2 + 2 * (ks - mf::KSTEPS_LAT);
        *reinterpret_cast<bf16x8_t*>(s_qrope + (c * kMfmaRows + wave * 32 + (lane & 31)) * 16) = v;
      }
    }
  }
  const unsigned char* qrope = s_qrope + (wave * 32 + (lane & 31)) * 16;

  WaveState st;
  st.m_ref = -INFINITY;
  st.m_seen = -INFINITY;
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < 16; ++db) st.o[db] = f32x16_t{};
    st.l = 0.f;
    st.over = false;
    if (pass > 0) stage_tile(g_kv_buf0, ckv_b, krope_b, w.k_begin, w.k_end, wave, lane);
    for (int t = 0; t < n_tiles; t += 2) {
      // tile t in buf0
      __syncthreads();  // buf0's copy landed (each wave waited for its own), buf1 free
      if (t + 1 < n_tiles)
        stage_tile(g_kv_buf1, ckv_b, krope_b, w.k_begin + (t + 1) * kMfmaKeys, w.k_end, wave, lane);
      if (wave_active) tile_compute(g_kv_buf0, qf, qrope, st, lane, w.k_begin + t * kMfmaKeys, w.k_end, P, anc);
      if (t + 1 >= n_tiles) break;
      // tile t + 1 in buf1
      __syncthreads();
      if (t + 2 < n_tiles)
        stage_tile(g_kv_buf0, ckv_b, krope_b, w.k_begin + (t + 2) * kMfmaKeys, w.k_end, wave, lane);
      if (wave_active)
        tile_compute(g_kv_buf1, qf, qrope, st, lane, w.k_begin + (t + 1) * kMfmaKeys, w.k_end, P, anc);
    }
    // Re-sweep (once, with the exact max as reference) if any row overflowed headroom.
    if (threadIdx.x == 0) s_redo = 0;
    __syncthreads();
    if (wave_active && __any(st.over) && lane == 0) s_redo = 1;
    __syncthreads();
    if (pass > 0 || s_redo == 0) break;
    // Only rows that ran out of headroom move their reference, so every other
    // row repeats its first sweep bit for bit (a row's result never depends on
    // another row's scores).
    st.m_ref = st.over ? st.m_seen : st.m_ref;
  }

  if (!wave_active) return;
  const float l_tot = st.l + __shfl_xor(st.l, 32);
  if (!row_valid) return;
  const int64_t grow = static_cast<int64_t>(b) * a.R + row;
  float* dst;
  if (w.slot < 0) {
    dst = a.out + grow * mf::DC;
    if (g2 == 0 && a.lse) a.lse[grow] = (st.m_ref + log2f(l_tot)) * mf::kLn2;
  } else {
    const int64_t srow = w.slot * kMfmaRows + (row - w.rb * kMfmaRows);
    dst = a.ws_o + srow * mf::DC;
    if (g2 == 0) {
      a.ws_m[srow] = st.m_ref * mf::kLn2;
      a.ws_l[srow] = l_tot;
    }
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int db = 0; db < 16; ++db) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 v = make_float4(st.o[db][4 * q4] * inv, st.o[db][4 * q4 + 1] * inv, st.o[db][4 * q4 + 2] * inv,
                                   st.o[db][4 * q4 + 3] * inv);
      *reinterpret_cast<float4*>(dst + 32 * db + 8 * q4 + 4 * g2) = v;
    }
  }
}

hipError_t launch_attn_mfma_bf16(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  attn_mfma_bf16_kernel<<<dim3(static_cast<unsigned>(plan.units)), kMfmaThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace tv
