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
// Workgroup = 4 waves, one per SIMD, 128 query rows (row blocks rb = 0..3 of
// 32 rows).  Wave w
//   * computes the scores and softmax weights of row block w: its 32 query rows
//     live in registers for the whole kv sweep, pre-scaled by
//     sm_scale * log2(e) and rounded once to bf16 (the B operand of
//     S^T = K Q^T), and the weights go to LDS for all four waves;
//   * accumulates output columns 128 w .. 128 w + 127 of all 128 rows:
//     O^T[rb][db] = V^T P^T in 16 x 16 fp32 accumulator registers per lane
//     (all 256), with V^T read straight from the row-major tile by
//     ds_read_b64_tr_b16 (no transposed copy).
// So each latent fragment read from LDS feeds four matrix ops, and the
// accumulators are never rescaled: the softmax is online in base 2 against a
// per-row reference max fixed by the first tile the row sees.  Weights
// exp2(s - m_ref) may exceed 1 (fp32 and bf16 carry them exactly as well); if
// some later score exceeds m_ref by more than 2^64 the workgroup sweeps its kv
// range once more, with m_ref = the exact row max for the rows that ran out of
// headroom, so nothing overflows for any finite input.
//
// Step t of the sweep (one barrier): the copy of tile t+1 HBM -> LDS starts
// (global_load_lds_dwordx4, three tile buffers in rotation); scores of tile t
// (TV_QK_ASM); mask and row max; then one asm block (TV_PVS_ASM) runs the
// value product of tile t-1 and, woven between its matrix ops, the
// exponentials, bf16 packing, row sums and LDS stores of tile t's weights.
#include "tv_kernels.h"
#include "attn_mfma_asm.h"

namespace tv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

namespace mf {
constexpr int DC = 512, DR = 64, D = DC + DR;
constexpr int KSTEPS = D / 16;                      // 36 k-steps of the score product
constexpr int KSTEPS_LAT = DC / 16;                 // 32 of them in the latent part
constexpr int kPadBytes = 16;                       // gap between latent rows in LDS
constexpr int kLatRowBytes = DC * 2 + kPadBytes;    // 1040
constexpr int kLatBytes = kMfmaKeys * kLatRowBytes; // 33280
constexpr int kRopeBytes = kMfmaKeys * DR * 2;      // 4096
constexpr int kBufBytes = kLatBytes + kRopeBytes;   // 37376
constexpr int kPBytes = kMfmaRows * kMfmaKeys * 2;  // 8192: one tile's bf16 weights
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kHeadroom = 64.0f;                  // log2 units above m_ref before a re-sweep
}  // namespace mf

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(p)));
}

// Three kv tile buffers (row-major, as in HBM), used in rotation.
__shared__ __align__(16) unsigned char g_k0[mf::kBufBytes];
__shared__ __align__(16) unsigned char g_k1[mf::kBufBytes];
__shared__ __align__(16) unsigned char g_k2[mf::kBufBytes];
// Softmax weights of two consecutive tiles: [rb][key half h][lane][8 x bf16],
// lane l holding row 32 rb + l % 32 and keys 16 h + {4 g .. 4 g + 3,
// 8 + 4 g .. 8 + 4 g + 3} (g = l / 32) -- the B operand of the value MFMA.
__shared__ __align__(16) unsigned char g_p[2][mf::kPBytes];

// Copy kv rows [kt, kt + 32) of one tree into a tile buffer.  Rows past k_end
// repeat row k_end - 1 (finite data; their scores are masked).
//   latent rows:  row k at buf + k * kLatRowBytes, 64 chunks of 16 B; wave w
//                 copies rows 8w .. 8w+7, one wave-wide 1 KB copy per row.
//   rope rows:    wave w copies keys 8w .. 8w+7 into buf + kLatBytes + 1024 w,
//                 chunk-major: 16-byte chunk c of key k at slot c * 8 + (k % 8).
// Buffer loads straight to LDS (buffer_load_dwordx4 ... lds): the tree's base
// is in the scalar resource, the row in a scalar offset, and each lane adds its
// 16-byte chunk (lane16 = 16 * lane), so a copy costs no address registers.
// Nine loads per wave; the caller waits for them (vmcnt) before the barrier
// that publishes the tile.
struct TreeKv {
  __amdgpu_buffer_rsrc_t lat;   // c_kv rows of the tree, 1024 B each
  __amdgpu_buffer_rsrc_t rope;  // k_rope rows of the tree, 128 B each
};

__device__ __forceinline__ void stage_tile(unsigned char* buf, const TreeKv& kv, int kt, int k_end, int wave,
                                           int lane, uint32_t lane16) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int k = wave * 8 + r;
    const int key = min(kt + k, k_end - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kv.lat, (lds_ptr_t)(buf + k * mf::kLatRowBytes), 16, lane16,
                                             key * (mf::DC * 2), 0, 0);
  }
  const int c = lane >> 3;
  const int kl = lane & 7;
  const int key = min(kt + wave * 8 + kl, k_end - 1);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(kv.rope, (lds_ptr_t)(buf + mf::kLatBytes + wave * 1024), 16,
                                           key * (mf::DR * 2) + c * 16, 0, 0, 0);
}

// Per-lane row state of the softmax (rows of the wave's own row block).
struct RowState {
  float m_ref;   // reference max (log2 units) the exponentials are taken against
  float m_seen;  // exact running max of the row's visible scores (log2 units)
  float l;       // this lane's share of the row's softmax denominator
  bool over;     // a score exceeded m_ref + kHeadroom
};

// Lanes l and l + 32 hold the same row: swap the wave's halves and combine.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// S^T = K Q^T for one tile (lane: row lane % 32, keys 8 (i/4) + 4 g + i % 4 in
// register i), masked, and the row's max folded into the state.  Returns the
// reference the exponentials are taken against.
__device__ __forceinline__ float scores(const unsigned char* buf, const bf16x8_t* qf, const unsigned char* qrope,
                                        RowState& st, int lane, int kt, int k_end, int P, unsigned long long anc,
                                        float (&s)[16]) {
  const int g2 = lane >> 5;
  const int key_l = lane & 31;
  // 36 MFMAs 32x32x16 in one accumulator chain: the latent part of Q is in
  // registers (qf), the rope part in LDS (qrope, chunk-major); every K
  // fragment is read 4 MFMAs ahead of its use.
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
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = sacc[i];

  // Mask (only tiles reaching past the prefix or the unit's kv range).
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

  float mt = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[i]);
  mt = max_halves(mt);
  st.m_seen = fmaxf(st.m_seen, mt);
  if (st.m_ref == -INFINITY) st.m_ref = mt;  // first visible tile: nothing accumulated yet
  st.over = st.over || (mt > st.m_ref + mf::kHeadroom);
  return st.m_ref == -INFINITY ? 0.f : st.m_ref;
}

// O^T += V^T P^T for the previous tile (kp, weights pp) with this tile's
// softmax (scores s against mref, weights to pc) woven in.  v_exp_f32 is used
// directly: its arguments are <= 64 or -inf (masked keys, giving 0), and
// results below the normal range may flush to 0, which only drops keys
// weighing < 2^-126 of the reference.
__device__ __forceinline__ void value_and_softmax(const unsigned char* kp, const unsigned char* pp, unsigned char* pc,
                                                  f32x16_t (&o)[16], float (&s)[16], float mref, float& l,
                                                  int lane, int wave) {
  const int g2 = lane >> 5;
  const int grp = lane >> 4;
  const int j = lane & 15;
  // ds_read_b64_tr_b16: in each 16-lane group lane j points at 4 consecutive
  // latent columns of key row 4 g + j / 4 and receives, for column
  // 16 (grp & 1) + j, the 4 keys of those rows.
  const uint32_t tb =
      lds_addr(kp + (4 * g2 + (j >> 2)) * mf::kLatRowBytes + (16 * (grp & 1) + 4 * (j & 3)) * 2 + 256 * wave);
  const uint32_t pb = lds_addr(pp + lane * 16);
  const uint32_t pw0 = lds_addr(pc + wave * 2048 + lane * 16);
  const uint32_t pw1 = pw0 + 1024;
  bf16x8_t pi0, pi1, pi2, pi3, pi4, pi5, pi6, pi7;
  uint32_t pk0, pk1, pk2, pk3, pk4, pk5, pk6, pk7;
  asm volatile(TV_PVS_ASM
               : [o0] "+a"(o[0]), [o1] "+a"(o[1]), [o2] "+a"(o[2]), [o3] "+a"(o[3]), [o4] "+a"(o[4]),
                 [o5] "+a"(o[5]), [o6] "+a"(o[6]), [o7] "+a"(o[7]), [o8] "+a"(o[8]), [o9] "+a"(o[9]),
                 [o10] "+a"(o[10]), [o11] "+a"(o[11]), [o12] "+a"(o[12]), [o13] "+a"(o[13]), [o14] "+a"(o[14]),
                 [o15] "+a"(o[15]), [s0] "+v"(s[0]), [s1] "+v"(s[1]), [s2] "+v"(s[2]), [s3] "+v"(s[3]),
                 [s4] "+v"(s[4]), [s5] "+v"(s[5]), [s6] "+v"(s[6]), [s7] "+v"(s[7]), [s8] "+v"(s[8]),
                 [s9] "+v"(s[9]), [s10] "+v"(s[10]), [s11] "+v"(s[11]), [s12] "+v"(s[12]), [s13] "+v"(s[13]),
                 [s14] "+v"(s[14]), [s15] "+v"(s[15]), [l] "+v"(l), [pi0] "=&v"(pi0), [pi1] "=&v"(pi1),
                 [pi2] "=&v"(pi2), [pi3] "=&v"(pi3), [pi4] "=&v"(pi4), [pi5] "=&v"(pi5), [pi6] "=&v"(pi6),
                 [pi7] "=&v"(pi7), [pk0] "=&v"(pk0), [pk1] "=&v"(pk1), [pk2] "=&v"(pk2), [pk3] "=&v"(pk3),
                 [pk4] "=&v"(pk4), [pk5] "=&v"(pk5), [pk6] "=&v"(pk6), [pk7] "=&v"(pk7)
               : [mref] "v"(mref), [tb] "v"(tb), [pb] "v"(pb), [pw0] "v"(pw0), [pw1] "v"(pw1)
               : "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251",
                 "v252", "v253", "v254", "v255", "memory");
}

__global__ __launch_bounds__(kMfmaThreads, 1) void attn_mfma_bf16_kernel(AttnArgs a) {
  __shared__ int s_par[kMaxQ];
  __shared__ unsigned long long s_anc[kMaxQ];
  __shared__ __align__(16) unsigned char s_qrope[kMfmaRows * mf::DR * 2];  // 16 KB
  __shared__ float s_row_l[kMfmaRows];
  __shared__ int s_redo;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g2 = lane >> 5;
  const Unit w = decode_unit(a, unit_of_block(a, blockIdx.x));
  const int b = w.b;
  const int P = a.prefix_len;
  // Buffer resources over this tree's rows (raw buffers: dword 3 of the
  // descriptor as for any untyped gfx9 buffer; the host keeps kv_len * 1024
  // below 2^31, so every offset fits).
  TreeKv kv;
  {
    const uint16_t* ckv_b = static_cast<const uint16_t*>(a.c_kv) + static_cast<int64_t>(b) * a.kv_len * mf::DC;
    const uint16_t* krope_b = static_cast<const uint16_t*>(a.k_rope) + static_cast<int64_t>(b) * a.kv_len * mf::DR;
    kv.lat = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(ckv_b), 0, a.kv_len * (mf::DC * 2), 0x00020000);
    kv.rope = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(krope_b), 0, a.kv_len * (mf::DR * 2), 0x00020000);
  }
  const uint32_t lane16 = lane * 16;

  const int n_tiles = (w.k_end - w.k_begin + kMfmaKeys - 1) / kMfmaKeys;
  auto stage = [&](unsigned char* buf, int t) {
    stage_tile(buf, kv, w.k_begin + t * kMfmaKeys, w.k_end, wave, lane, lane16);
  };

  build_ancestors(a.parent + static_cast<int64_t>(b) * a.q_len, a.q_len, s_par, s_anc);

  // This wave's own rows (row block rb = wave).
  const int row0 = w.rb * kMfmaRows + wave * 32;
  const int row = row0 + (lane & 31);
  const bool row_valid = row < a.R;
  const int node = min(row / a.H, a.q_len - 1);
  const unsigned long long anc = s_anc[node];

  // Query fragments: q[row][8 g2 + 16 ks .. + 7] * sm_scale * log2(e) as bf16.
  // Latent part (ks < 32) in registers; rope part in LDS, chunk-major:
  // 16-byte chunk c of block row r at s_qrope + (c * 128 + r) * 16.  Rows past
  // R get zero queries (their results are never stored).
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

  f32x16_t o[16];  // o[4 rb + db][i] = O[32 rb + lane % 32][128 wave + 32 db + 8 (i/4) + 4 g2 + i % 4]
  RowState st;
  st.m_ref = -INFINITY;
  st.m_seen = -INFINITY;

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = f32x16_t{};
    st.l = 0.f;
    st.over = false;
    // The weights "before tile 0" are zeros, so step 0's value product adds
    // nothing (it reads tile 0's finite latent rows).
    *reinterpret_cast<uint4*>(g_p[1] + threadIdx.x * 32) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(g_p[1] + threadIdx.x * 32 + 16) = make_uint4(0, 0, 0, 0);
    stage(g_k0, 0);
    unsigned char* kp = g_k2;  // tile t-1
    unsigned char* kc = g_k0;  // tile t
    unsigned char* kn = g_k1;  // tile t+1
    // Step t: scores of tile t, value product of tile t-1.  The extra step
    // t = n_tiles only runs the value product of the last tile.
    for (int t = 0; t <= n_tiles; ++t) {
      // Tile t (this wave's copies) has landed; after the barrier every wave's
      // has, the weights of tile t-1 are in LDS, and tile t-2's buffer (kn) and
      // weights buffer are no longer read.  The barrier alone drains only LDS
      // instructions, not the HBM->LDS copies, and the compiler cannot see the
      // LDS reads inside the asm blocks.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (t + 1 < n_tiles) stage(kn, t + 1);
      float s[16];
      float mref = 0.f;
      if (t < n_tiles) {
        mref = scores(kc, qf, qrope, st, lane, w.k_begin + t * kMfmaKeys, w.k_end, P, anc, s);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = -INFINITY;
      }
      value_and_softmax(t == 0 ? kc : kp, g_p[(t + 1) & 1], g_p[t & 1], o, s, mref, st.l, lane, wave);
      unsigned char* nx = kp;
      kp = kc;
      kc = kn;
      kn = nx;
    }
    // Re-sweep (once, with the exact max as reference) if any row overflowed headroom.
    if (threadIdx.x == 0) s_redo = 0;
    __syncthreads();
    if (__any(st.over) && lane == 0) s_redo = 1;
    __syncthreads();
    if (pass > 0 || s_redo == 0) break;
    // Only rows that ran out of headroom move their reference, so every other
    // row repeats its first sweep bit for bit (a row's result never depends on
    // another row's scores).
    st.m_ref = st.over ? st.m_seen : st.m_ref;
  }

  // Row sums of the wave's own rows, for all four waves.
  const float l_tot = sum_halves(st.l);
  if (g2 == 0) s_row_l[wave * 32 + lane] = l_tot;
  const int64_t tree_row0 = static_cast<int64_t>(b) * a.R;
  if (g2 == 0 && row_valid) {
    if (w.slot < 0) {
      if (a.lse) a.lse[tree_row0 + row] = (st.m_ref + log2f(l_tot)) * mf::kLn2;
    } else {
      const int64_t srow = w.slot * kMfmaRows + wave * 32 + lane;
      a.ws_m[srow] = st.m_ref * mf::kLn2;
      a.ws_l[srow] = l_tot;
    }
  }
  __syncthreads();

#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int r = w.rb * kMfmaRows + rb * 32 + (lane & 31);
    if (r < a.R) {
      const float lr = s_row_l[rb * 32 + (lane & 31)];
      const float inv = lr > 0.f ? 1.f / lr : 0.f;
      float* dst = w.slot < 0 ? a.out + (tree_row0 + r) * mf::DC
                              : a.ws_o + (w.slot * kMfmaRows + rb * 32 + (lane & 31)) * mf::DC;
      dst += 128 * wave + 4 * g2;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const f32x16_t& v = o[4 * rb + db];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          *reinterpret_cast<float4*>(dst + 32 * db + 8 * q4) =
              make_float4(v[4 * q4] * inv, v[4 * q4 + 1] * inv, v[4 * q4 + 2] * inv, v[4 * q4 + 3] * inv);
        }
      }
    }
  }
}

hipError_t launch_attn_mfma_bf16(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  attn_mfma_bf16_kernel<<<dim3(static_cast<unsigned>(plan.units)), kMfmaThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace tv
