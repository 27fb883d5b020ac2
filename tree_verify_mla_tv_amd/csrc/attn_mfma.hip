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
#include "attn_mfma_asm.h"

namespace tv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(8))) short i16x8_t;

namespace mf {
constexpr int DC = 512, DR = 64, D = DC + DR;
constexpr int KSTEPS = D / 16;                      // 36 k-steps of the score product
constexpr int KSTEPS_LAT = DC / 16;                 // 32 of them in the latent part
constexpr int kPadBytes = 16;                       // gap between latent rows in LDS
constexpr int kLatRowBytes = DC * 2 + kPadBytes;    // 1040
constexpr int kLatBytes = kMfmaKeys * kLatRowBytes; // 33280
constexpr int kRopeBytes = kMfmaKeys * DR * 2;      // 4096
constexpr int kBufBytes = kLatBytes + kRopeBytes;   // 37376
constexpr int kVtBytes = DC * 64;                   // 32768: V^T tile, 512 rows of 32 keys
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kHeadroom = 64.0f;                  // log2 units above m_ref before a re-sweep
}  // namespace mf

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;
typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4_ptr_t;

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(p)));
}

// Two kv tiles (row-major, as in HBM) and two transposed latent tiles.
__shared__ __align__(16) unsigned char g_k0[mf::kBufBytes];
__shared__ __align__(16) unsigned char g_k1[mf::kBufBytes];
__shared__ __align__(16) unsigned char g_vt0[mf::kVtBytes];
__shared__ __align__(16) unsigned char g_vt1[mf::kVtBytes];

// Copy kv rows [kt, kt + 32) of one tree into a row-major tile buffer.  Rows
// past k_end repeat row k_end - 1 (finite data; their scores are masked).
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

// Transposed latent tile V^T: 512 rows d of 4 chunks of 16 B.  Chunk 2h + g of
// row d holds the 8 keys 16 h + {4 g .. 4 g + 3, 8 + 4 g .. 8 + 4 g + 3} at d,
// i.e. exactly the A operand lane (d % 32) + 32 g needs for the value MFMA of
// key half h.  Chunks are XOR-swizzled by (d >> 2) & 3 so the 16 lanes of a
// 128-bit access hit 16 different bank groups.
__device__ __forceinline__ int vt_offset(int d, int chunk) { return d * 64 + 16 * (chunk ^ ((d >> 2) & 3)); }

// One wave's quarter of the transpose of a row-major tile (d-blocks 4w..4w+3)
// into V^T, through ds_read_b64_tr_b16: in each 16-lane group, lane j points at
// 4 consecutive d of key row kb + j/4 and receives the 4 keys kb .. kb+3 of
// d = d0 + j.
__device__ __forceinline__ void transpose_quarter(const unsigned char* kbuf, unsigned char* vt, int lane, int wave) {
  const int g2 = lane >> 5;
  const int grp = lane >> 4;
  const int j = lane & 15;
  const int d0 = 16 * (grp & 1) + 4 * (j & 3);
  const unsigned char* vbase = kbuf + (4 * g2 + (j >> 2)) * mf::kLatRowBytes + d0 * 2;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int db = 4 * wave + (u >> 1);
    const int h = u & 1;
    const unsigned char* va = vbase + (16 * h) * mf::kLatRowBytes + db * 64;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(va));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(va + 8 * mf::kLatRowBytes));
    const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    *reinterpret_cast<i16x8_t*>(vt + vt_offset(32 * db + (lane & 31), 2 * h + g2)) = v;
  }
}

// Everything one wave keeps across tiles.
struct WaveState {
  f32x16_t o[16];   // O^T blocks: o[db][i] = out[row][32 db + 8 (i/4) + 4 g2 + i%4]
  float m_ref;      // reference max (log2 units) the exponentials are taken against
  float m_seen;     // exact running max of the row's visible scores (log2 units)
  float l;          // this lane's share of the row's softmax denominator
  bool over;        // a score exceeded m_ref + kHeadroom
};

// S^T = K Q^T for one tile, mask, and the tile's softmax weights (bf16).
__device__ __forceinline__ void qk_softmax(const unsigned char* buf, const bf16x8_t* qf, const unsigned char* qrope,
                                           WaveState& st, int lane, int kt, int k_end, int P,
                                           unsigned long long anc, bf16x8_t& p0, bf16x8_t& p1) {
  const int g2 = lane >> 5;
  const int key_l = lane & 31;
  // 36 MFMAs 32x32x16 in one accumulator chain (TV_QK_ASM, generated): the
  // latent part of Q is in registers (qf), the rope part in LDS (qrope,
  // chunk-major); every K fragment is read 4 MFMAs ahead of its use.
  const uint32_t lat = lds_addr(buf + key_l * mf::kLatRowBytes + g2 * 16);
  const uint32_t rope = lds_addr(buf + mf::kLatBytes + (key_l >> 3) * 1024 + (key_l & 7) * 16 + g2 * 128);
  const uint32_t qr = lds_addr(qrope + g2 * (kMfmaRows * 16));
  f32x16_t sacc;
  bf16x8_t k0, k1, k2, k3, k4, k5, r0, r1, r2, r3;
  asm volatile(TV_QK_ASM
               : [s] "=&v"(sacc), [k0] "=&v"(k0), [k1] "=&v"(k1), [k2] "=&v"(k2), [k3] "=&v"(k3), [k4] "=&v"(k4),
                 [k5] "=&v"(k5), [r0] "=&v"(r0), [r1] "=&v"(r1), [r2] "=&v"(r2), [r3] "=&v"(r3)
               : [lat] "v"(lat), [rope] "v"(rope), [qr] "v"(qr), [q0] "v"(qf[0]), [q1] "v"(qf[1]), [q2] "v"(qf[2]),
                 [q3] "v"(qf[3]), [q4] "v"(qf[4]), [q5] "v"(qf[5]), [q6] "v"(qf[6]), [q7] "v"(qf[7]), [q8] "v"(qf[8]),
                 [q9] "v"(qf[9]), [q10] "v"(qf[10]), [q11] "v"(qf[11]), [q12] "v"(qf[12]), [q13] "v"(qf[13]),
                 [q14] "v"(qf[14]), [q15] "v"(qf[15]), [q16] "v"(qf[16]), [q17] "v"(qf[17]), [q18] "v"(qf[18]),
                 [q19] "v"(qf[19]), [q20] "v"(qf[20]), [q21] "v"(qf[21]), [q22] "v"(qf[22]), [q23] "v"(qf[23]),
                 [q24] "v"(qf[24]), [q25] "v"(qf[25]), [q26] "v"(qf[26]), [q27] "v"(qf[27]), [q28] "v"(qf[28]),
                 [q29] "v"(qf[29]), [q30] "v"(qf[30]), [q31] "v"(qf[31])
               : "memory");
  float s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = sacc[i];

  // Mask: register i holds key kt + 8 (i/4) + 4 g2 + i%4.
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

  // Softmax weights (base 2) against the row's reference max.
  float mt = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[i]);
  mt = fmaxf(mt, __shfl_xor(mt, 32));  // lanes l and l ^ 32 hold the same row
  st.m_seen = fmaxf(st.m_seen, mt);
  if (st.m_ref == -INFINITY) st.m_ref = mt;  // first visible tile: o and l are still 0
  st.over = st.over || (mt > st.m_ref + mf::kHeadroom);
  const float mref = st.m_ref == -INFINITY ? 0.f : st.m_ref;
  // v_exp_f32 directly: arguments are <= 64 (or -inf for masked keys, giving
  // 0); results below the normal range may flush to 0, which only drops keys
  // weighing < 2^-126 of the reference.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p0[i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(s[i] - mref));
    p1[i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(s[i + 8] - mref));
  }
  // The denominator sums the rounded weights the value product uses, two at a
  // time with a bf16 dot product against (1, 1).
  const bf16x2_t one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  float lsum = st.l;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{p0[i], p0[i + 1]}, one2, lsum, false);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{p1[i], p1[i + 1]}, one2, lsum, false);
  }
  st.l = lsum;
}

// O^T += V^T P^T for one tile: 16 d-blocks x 2 key halves, A operand read from
// the transposed tile with ds_read_b128, 4 MFMAs ahead.
__device__ __forceinline__ void pv(const unsigned char* vt, WaveState& st, int lane, const bf16x8_t& p0,
                                   const bf16x8_t& p1) {
  const int g2 = lane >> 5;
  const int dl = lane & 31;
  // 32 MFMAs (TV_PV_ASM, generated); MFMA n = 2 db + h reads V^T at a_h + 2048 db.
  const uint32_t a0 = lds_addr(vt + vt_offset(dl, g2));
  const uint32_t a1 = lds_addr(vt + vt_offset(dl, 2 + g2));
  bf16x8_t v0, v1, v2, v3, v4, v5;
  asm volatile(TV_PV_ASM
               : [o0] "+a"(st.o[0]), [o1] "+a"(st.o[1]), [o2] "+a"(st.o[2]), [o3] "+a"(st.o[3]), [o4] "+a"(st.o[4]),
                 [o5] "+a"(st.o[5]), [o6] "+a"(st.o[6]), [o7] "+a"(st.o[7]), [o8] "+a"(st.o[8]), [o9] "+a"(st.o[9]),
                 [o10] "+a"(st.o[10]), [o11] "+a"(st.o[11]), [o12] "+a"(st.o[12]), [o13] "+a"(st.o[13]),
                 [o14] "+a"(st.o[14]), [o15] "+a"(st.o[15]), [v0] "=&v"(v0), [v1] "=&v"(v1), [v2] "=&v"(v2),
                 [v3] "=&v"(v3), [v4] "=&v"(v4), [v5] "=&v"(v5)
               : [a0] "v"(a0), [a1] "v"(a1), [p0] "v"(p0), [p1] "v"(p1)
               : "memory");
}

// The value product of this tile with this wave's quarter of the next tile's
// transpose (kn -> vn, as transpose_quarter) woven into the MFMA chain.
__device__ __forceinline__ void pv_transpose(const unsigned char* vt, const unsigned char* kn, unsigned char* vn,
                                             WaveState& st, int lane, int wave, const bf16x8_t& p0,
                                             const bf16x8_t& p1) {
  const int g2 = lane >> 5;
  const int dl = lane & 31;
  const int grp = lane >> 4;
  const int j = lane & 15;
  const uint32_t a0 = lds_addr(vt + vt_offset(dl, g2));
  const uint32_t a1 = lds_addr(vt + vt_offset(dl, 2 + g2));
  const int d0 = 16 * (grp & 1) + 4 * (j & 3);
  const uint32_t tb = lds_addr(kn + (4 * g2 + (j >> 2)) * mf::kLatRowBytes + d0 * 2 + 256 * wave);
  const uint32_t wb0 = lds_addr(vn + vt_offset(dl, g2) + 8192 * wave);
  const uint32_t wb1 = lds_addr(vn + vt_offset(dl, 2 + g2) + 8192 * wave);
  bf16x8_t v0, v1, v2, v3, v4, v5;
  i16x4_t t0lo, t0hi, t1lo, t1hi, t2lo, t2hi, t3lo, t3hi, t4lo, t4hi, t5lo, t5hi, t6lo, t6hi, t7lo, t7hi;
  asm volatile(TV_PV_TRANSPOSE_ASM
               : [o0] "+a"(st.o[0]), [o1] "+a"(st.o[1]), [o2] "+a"(st.o[2]), [o3] "+a"(st.o[3]), [o4] "+a"(st.o[4]),
                 [o5] "+a"(st.o[5]), [o6] "+a"(st.o[6]), [o7] "+a"(st.o[7]), [o8] "+a"(st.o[8]), [o9] "+a"(st.o[9]),
                 [o10] "+a"(st.o[10]), [o11] "+a"(st.o[11]), [o12] "+a"(st.o[12]), [o13] "+a"(st.o[13]),
                 [o14] "+a"(st.o[14]), [o15] "+a"(st.o[15]), [v0] "=&v"(v0), [v1] "=&v"(v1), [v2] "=&v"(v2),
                 [v3] "=&v"(v3), [v4] "=&v"(v4), [v5] "=&v"(v5), [t0lo] "=&v"(t0lo), [t0hi] "=&v"(t0hi),
                 [t1lo] "=&v"(t1lo), [t1hi] "=&v"(t1hi), [t2lo] "=&v"(t2lo), [t2hi] "=&v"(t2hi),
                 [t3lo] "=&v"(t3lo), [t3hi] "=&v"(t3hi), [t4lo] "=&v"(t4lo), [t4hi] "=&v"(t4hi),
                 [t5lo] "=&v"(t5lo), [t5hi] "=&v"(t5hi), [t6lo] "=&v"(t6lo), [t6hi] "=&v"(t6hi),
                 [t7lo] "=&v"(t7lo), [t7hi] "=&v"(t7hi)
               : [a0] "v"(a0), [a1] "v"(a1), [p0] "v"(p0), [p1] "v"(p1), [tb] "v"(tb), [wb0] "v"(wb0),
                 [wb1] "v"(wb1)
               : "memory");
}

__global__ __launch_bounds__(kMfmaThreads, 1) void attn_mfma_bf16_kernel(AttnArgs a) {
  __shared__ int s_par[kMaxQ];
  __shared__ unsigned long long s_anc[kMaxQ];
  __shared__ __align__(16) unsigned char s_qrope[kMfmaRows * mf::DR * 2];  // 16 KB
  __shared__ int s_redo;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g2 = lane >> 5;
  const Unit w = decode_unit(a, unit_of_block(a, blockIdx.x));
  const int b = w.b;
  const int P = a.prefix_len;
  const uint16_t* ckv_b = static_cast<const uint16_t*>(a.c_kv) + static_cast<int64_t>(b) * a.kv_len * mf::DC;
  const uint16_t* krope_b = static_cast<const uint16_t*>(a.k_rope) + static_cast<int64_t>(b) * a.kv_len * mf::DR;

  const int n_tiles = (w.k_end - w.k_begin + kMfmaKeys - 1) / kMfmaKeys;
  auto stage = [&](unsigned char* buf, int t) {
    stage_tile(buf, ckv_b, krope_b, w.k_begin + t * kMfmaKeys, w.k_end, wave, lane);
  };

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
  // One tile step.  On entry (after the first barrier) tile t is in kc and its
  // transpose in vc; tile t+1 is in flight to kn.  After the second barrier
  // tile t+1 has landed and kc is free, so tile t+2 is sent to kc while the
  // waves run the value product on vc and transpose tile t+1 into vn.
  auto step = [&](int t, unsigned char* kc, unsigned char* kn, unsigned char* vc, unsigned char* vn) {
    // Every wave computes (a wave past the last row works on zero queries and
    // stores nothing), since all four share the transposes.
    bf16x8_t p0, p1;
    __syncthreads();
    qk_softmax(kc, qf, qrope, st, lane, w.k_begin + t * kMfmaKeys, w.k_end, P, anc, p0, p1);
    // Tile t+1 (this wave's share, sent one step ago) must have landed in kn
    // before the barrier: the transpose below reads all of it.  The barrier
    // alone only drains LDS instructions, not the HBM->LDS copies, and the
    // compiler cannot see the LDS reads inside the asm blocks.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 2 < n_tiles) stage(kc, t + 2);
    // On the last tile the transpose of kn into vn is idle work on a buffer
    // nobody reads again; doing it anyway keeps a single code path.
    pv_transpose(vc, kn, vn, st, lane, wave, p0, p1);
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < 16; ++db) st.o[db] = f32x16_t{};
    st.l = 0.f;
    st.over = false;
    stage(g_k0, 0);
    if (n_tiles > 1) stage(g_k1, 1);
    __syncthreads();
    transpose_quarter(g_k0, g_vt0, lane, wave);
    for (int t = 0; t < n_tiles; ++t) {
      const bool odd = t & 1;
      step(t, odd ? g_k1 : g_k0, odd ? g_k0 : g_k1, odd ? g_vt1 : g_vt0, odd ? g_vt0 : g_vt1);
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
