// Tree-verify MLA-absorb attention on the CDNA4 matrix cores, bf16 latent
// cache (d_c = 512, d_r = 64), with the queries kept to fp32 precision.
//
// [Verify page = "The Precision Imperative: Validating Numerical Accuracy in a
//  Custom CUDA Attention Kernel", "The Context: What Led to This Moment" and
//  "Assumptions and Their Implications"; Golden page = "The Golden Reference: A
//  Pivotal Moment in Building a Native DDTree Inference Engine", "The Absorb
//  Form of MLA".]  The cache is bf16, so the keys and values are exact bf16
// matrix-core operands; the queries arrive in fp32.  Rounding a query to bf16
// moves each score by up to 2^-9 of its terms, which on inputs with a few
// dominant latent channels (structured activations rather than i.i.d. draws)
// shifts near-one-hot weights far past the bf16-cache tolerance.  This kernel
// carries each scaled query x as hi = bf16(x) plus lo = bf16(x - hi) (x to
// 2^-17), so the scores are those of the fp32 queries up to fp32 accumulation.
// The value product runs in fp16: the softmax weights are rounded to fp16
// (2^-11, where bf16 would give 2^-8), and each bf16 latent row is converted
// to fp16 in registers: bf16 carries 8 significant bits, fp16 11, so the
// conversion is exact for magnitudes from 2^-17 (where fp16's subnormal
// spacing 2^-24 is the bf16 value's last bit) to 65504; smaller values round
// to that spacing, magnitudes of 65520 or more overflow.  fp16 weights bound the reference-max headroom:
// a weight exp2(s - m_ref) must stay below 65504, so a tile whose scores pass
// m_ref by more than kHeadroom triggers the re-sweep.
//
// Workgroup = 4 waves (one per SIMD), 64 query rows of one tree.  Wave w owns
// rows 16 w .. 16 w + 15 for the scores: the B operand of its score product
// S^T = K Q^T has 32 columns, the hi terms of its 16 rows in columns 0..15 and
// the lo terms in 16..31, so one v_mfma_f32_32x32x16_bf16 per k-step gives both
// and a swap of lane rows adds them (the same matrix-op count per key tile as a
// 32-row block with bf16 queries, for half the rows).  Every wave accumulates
// output columns 128 w .. 128 w + 127 of all 64 rows (O^T = V^T P^T, two row
// blocks of 32, 8 x 16 fp32 accumulators per lane).  The sweep, the copy of
// the kv tiles, the softmax against a reference max and the re-sweep are those
// of attn_mfma.hip (the headroom here 2^15, for the fp16 weights); one step is
// one barrier and one generated asm block (TV_Q2_STEP_ASM, gen_mfma_q2_asm.py).
#include "attn_mfma_common.h"
#include "attn_mfma_q2_asm.h"

namespace tv {

namespace q2 {
constexpr int kRows = kQ2Rows;                      // 64 query rows per workgroup
constexpr int kPBytes = kRows * kMfmaKeys * 2;      // 4096: one tile's fp16 weights
constexpr float kHeadroom = 15.0f;                  // log2 units above m_ref: weights below 2^15 fit fp16
}  // namespace q2

// Three kv tile buffers in rotation (layout of attn_mfma_common.h).
__shared__ __align__(16) unsigned char g_q2_k0[mf::kBufBytes];
__shared__ __align__(16) unsigned char g_q2_k1[mf::kBufBytes];
__shared__ __align__(16) unsigned char g_q2_k2[mf::kBufBytes];
// Softmax weights of two consecutive tiles, [rb][key half h][lane][8 x fp16]:
// lane L holds row 32 rb + L % 32 and keys 16 h + {4 G .. 4 G + 3, 8 + 4 G ..
// 8 + 4 G + 3} (G = L / 32) -- the B operand of the value product.
__shared__ __align__(16) unsigned char g_q2_p[2][q2::kPBytes];

// One step (TV_Q2_STEP_ASM): scores of the tile in kc (hi and lo columns,
// combined; lane l keeps row l % 16 and keys 16 (rho & 1) + 8 (i/4) +
// 4 (rho >> 1) + i % 4 in score i, rho = l / 16), masked where bit i of vis is
// clear (if nm), row state, weights summed into st.l and stored to pc; the
// value product of the previous tile; the copy of the next tile into kn.
__device__ __forceinline__ void step_q2(const StepBufs& sb, const TreeKv& kv, const bf16x8_t* qf, f32x16_t (&o)[8],
                                        RowState& st, int lane, int wave, int kt, uint32_t vis, int nm) {
  const int g2 = lane >> 5;
  const int grp = lane >> 4;
  const int j = lane & 15;
  const int key_l = lane & 31;
  const uint32_t lat = lds_addr(sb.kc + key_l * mf::kLatRowBytes + g2 * 16);
  const uint32_t rope = lds_addr(sb.kc + mf::kLatBytes + (key_l >> 3) * 1024 + (key_l & 7) * 16 + g2 * 128);
  // Value fragments: as in attn_mfma.hip (ds_read_b64_tr_b16 over the
  // row-major tile, columns 128 wave + 32 q + 8 db + 4 gp + {0..3}).
  const uint32_t tb = lds_addr(sb.kp + (4 * g2 + (j >> 2)) * mf::kLatRowBytes + 64 * (j & 3) + 8 * (grp & 1) +
                               256 * wave);
  const uint32_t pb = lds_addr(sb.pp + lane * 16);
  // This lane's 8 weights: row 16 wave + j, key half rho & 1, key group
  // rho >> 1 -> B-operand lane 32 (rho >> 1) + 16 (wave & 1) + j of row block
  // wave >> 1, half rho & 1.
  const int rho = lane >> 4;
  const uint32_t pw = lds_addr(sb.pc + ((2 * (wave >> 1) + (rho & 1)) * 64 + 32 * (rho >> 1) + 16 * (wave & 1) + j) * 16);
  const StageArgs sa = stage_args(sb.kn, kv, kt + kMfmaKeys, wave, lane);
  const uint32_t mb = __builtin_amdgcn_readfirstlane(sa.mb);
  const uint32_t mr = __builtin_amdgcn_readfirstlane(sa.mr);
  const int kb = __builtin_amdgcn_readfirstlane(sa.kb);
  const int km = __builtin_amdgcn_readfirstlane(kv.kmax);
  const int nms = __builtin_amdgcn_readfirstlane(nm);
  uint32_t t, ms;
  asm volatile(TV_Q2_STEP_ASM
               : [o0] "+a"(o[0]), [o1] "+a"(o[1]), [o2] "+a"(o[2]), [o3] "+a"(o[3]), [o4] "+a"(o[4]),
                 [o5] "+a"(o[5]), [o6] "+a"(o[6]), [o7] "+a"(o[7]), [l] "+v"(st.l), [mref] "+v"(st.m_ref),
                 [mseen] "+v"(st.m_seen), [exc] "+v"(st.exc), [t] "=&s"(t), [ms] "=&s"(ms)
               : [lat] "v"(lat), [rope] "v"(rope), [tb] "v"(tb), [pb] "v"(pb), [pw] "v"(pw), [mb] "s"(mb),
                 [mr] "s"(mr), [kb] "s"(kb), [km] "s"(km), [l16] "v"(kv.lane16), [ro] "v"(sa.ro), [rl] "s"(kv.lat),
                 [rr] "s"(kv.rope), [mask] "v"(vis), [nm] "s"(nms), [q0] "v"(qf[0]), [q1] "v"(qf[1]),
                 [q2] "v"(qf[2]), [q3] "v"(qf[3]), [q4] "v"(qf[4]), [q5] "v"(qf[5]), [q6] "v"(qf[6]),
                 [q7] "v"(qf[7]), [q8] "v"(qf[8]), [q9] "v"(qf[9]), [q10] "v"(qf[10]), [q11] "v"(qf[11]),
                 [q12] "v"(qf[12]), [q13] "v"(qf[13]), [q14] "v"(qf[14]), [q15] "v"(qf[15]), [q16] "v"(qf[16]),
                 [q17] "v"(qf[17]), [q18] "v"(qf[18]), [q19] "v"(qf[19]), [q20] "v"(qf[20]), [q21] "v"(qf[21]),
                 [q22] "v"(qf[22]), [q23] "v"(qf[23]), [q24] "v"(qf[24]), [q25] "v"(qf[25]), [q26] "v"(qf[26]),
                 [q27] "v"(qf[27]), [q28] "v"(qf[28]), [q29] "v"(qf[29]), [q30] "v"(qf[30]), [q31] "v"(qf[31]),
                 [qr0] "v"(qf[32]), [qr1] "v"(qf[33]), [qr2] "v"(qf[34]), [qr3] "v"(qf[35])
               : TV_Q2_STEP_CLOBBERS, "vcc", "scc", "memory");
}

// Sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one row's lanes).
__device__ __forceinline__ float sum_row_lanes(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ void attn_mfma_q2_unit(const AttnArgs& a, const Unit& w) {
  __shared__ int s_par[kMaxQ];
  __shared__ unsigned long long s_anc[kMaxQ * kAncWords];
  __shared__ float s_row_l[q2::kRows];
  __shared__ int s_redo;
  __shared__ uint8_t s_vis[kMaxBoundaryTiles * kMfmaThreads];  // masks of the boundary tiles, per thread

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g2 = lane >> 5;
  const int rho = lane >> 4;
  const int j = lane & 15;
  const int P = w.P;
  TreeKv kv;
  kv.lat = raw_buffer(static_cast<const uint16_t*>(a.c_kv) + w.kv_row0 * mf::DC,
                      static_cast<uint32_t>(w.kv_len) * (mf::DC * 2));
  kv.rope = raw_buffer(static_cast<const uint16_t*>(a.k_rope) + w.kv_row0 * mf::DR,
                       static_cast<uint32_t>(w.kv_len) * (mf::DR * 2));
  kv.lane16 = lane * 16;
  kv.kmax = w.k_end - 1;

  const int n_tiles = (w.k_end - w.k_begin + kMfmaKeys - 1) / kMfmaKeys;

  build_ancestors(a.parent + w.par0, w.q_len, s_par, s_anc);

  // This lane's row: row 16 wave + j of the block (every lane group rho of
  // the wave covers the same 16 rows).
  const int row = w.rb * q2::kRows + wave * 16 + j;
  const bool row_valid = row < w.R;
  const int node = min(row / a.H, w.q_len - 1);

  // Query operand: lane l supplies column l % 32 of B, k-rows 8 g2 .. 8 g2 + 7
  // of each k-step: dims 16 ks + 8 g2 .. + 7 of its row, the hi term in
  // columns 0..15 (lanes with bit 4 clear) and the lo term in 16..31.  The
  // scale sm_scale * log2(e) is applied in fp32 first (one rounding); rows
  // past R get zero queries (their results are never stored).
  bf16x8_t qf[mf::KSTEPS];
  {
    const float sc = a.sm_scale * mf::kLog2e;
    const int64_t grow = w.row0 + (row_valid ? row : 0);
    const float* ql = a.q_lat + grow * mf::DC + 8 * g2;
    const float* qr = a.q_rope + grow * mf::DR + 8 * g2;
    const float z = row_valid ? sc : 0.f;
    const bool lo_term = (lane & 16) != 0;
#pragma unroll
    for (int ks = 0; ks < mf::KSTEPS; ++ks) {
      const float* src = ks < mf::KSTEPS_LAT ? ql + 16 * ks : qr + 16 * (ks - mf::KSTEPS_LAT);
      const float4 x0 = *reinterpret_cast<const float4*>(src);
      const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
      const float xs[8] = {x0.x * z, x0.y * z, x0.z * z, x0.w * z, x1.x * z, x1.y * z, x1.z * z, x1.w * z};
      bf16x8_t v;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 hi = static_cast<__bf16>(xs[e]);
        const __bf16 lo = static_cast<__bf16>(xs[e] - static_cast<float>(hi));  // x - hi is exact in fp32
        v[e] = lo_term ? lo : hi;
      }
      qf[ks] = v;
    }
  }

  // Visibility of the boundary tiles (those holding tree keys or the range
  // end; at most q_len / 32 + 2 of them): bit i of this lane's mask says
  // whether key kt + 16 (rho & 1) + 8 (i/4) + 4 (rho >> 1) + i % 4 is visible
  // from the row's node.
  const int t_first = max(0, (min(P, w.k_end) - w.k_begin) / kMfmaKeys);
  {
    const int n_bt = min(n_tiles - t_first, kMaxBoundaryTiles);
    for (int bt = 0; bt < n_bt; ++bt) {
      const int kt = w.k_begin + (t_first + bt) * kMfmaKeys;
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = kt + 16 * (rho & 1) + 8 * (i >> 2) + 4 * (rho >> 1) + (i & 3);
        m |= key_visible(s_anc, node, key, P, w.k_end) << i;
      }
      s_vis[bt * kMfmaThreads + threadIdx.x] = static_cast<uint8_t>(m);
    }
  }

  // o[4 rb + db][i] = O[32 rb + lane % 32][col(db, i)], col as in attn_mfma.hip:
  //   col(db, i) = 128 wave + 64 ((i >> 2) & 1) + 32 g2 + 8 db + 4 (i >> 3) + (i & 3).
  f32x16_t o[8];
  RowState st;
  st.m_ref = -INFINITY;
  st.m_seen = -INFINITY;

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = f32x16_t{};
    st.l = 0.f;
    st.exc = -INFINITY;
    // The weights "before tile 0" are zeros, so step 0's value product adds
    // nothing (it reads tile 0's finite latent rows).
    *reinterpret_cast<uint4*>(g_q2_p[1] + threadIdx.x * 16) = make_uint4(0, 0, 0, 0);
    stage_tile(g_q2_k0, kv, w.k_begin, wave, lane);
    unsigned char* kp = g_q2_k2;  // tile t-1
    unsigned char* kc = g_q2_k0;  // tile t
    unsigned char* kn = g_q2_k1;  // tile t+1
    for (int t = 0; t <= n_tiles; ++t) {
      // As in attn_mfma.hip: this wave's copies of tile t have landed, and
      // after the barrier every wave's have, tile t-1's weights are in LDS,
      // and the buffers of tile t-2 are free.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int kt = w.k_begin + t * kMfmaKeys;
      uint32_t vis = 0xffu;
      int nm = 0;
      if (t == n_tiles) {
        vis = 0;
        nm = 1;
      } else if (kt + kMfmaKeys > P || kt + kMfmaKeys > w.k_end) {
        nm = 1;
        vis = s_vis[min(t - t_first, kMaxBoundaryTiles - 1) * kMfmaThreads + threadIdx.x];
      }
      const StepBufs sb{kc, t == 0 ? kc : kp, kn, g_q2_p[(t + 1) & 1], g_q2_p[t & 1]};
      step_q2(sb, kv, qf, o, st, lane, wave, kt, vis, nm);
      unsigned char* nx = kp;
      kp = kc;
      kc = kn;
      kn = nx;
    }
    asm volatile("s_waitcnt vmcnt(0)\n" TV_MFMA_DRAIN_ASM ::: "memory");
    const bool over = st.exc > q2::kHeadroom;
    if (threadIdx.x == 0) s_redo = 0;
    __syncthreads();
    if (__any(over) && lane == 0) s_redo = 1;
    __syncthreads();
    if (pass > 0 || s_redo == 0) break;
    st.m_ref = over ? st.m_seen : st.m_ref;
  }

  // Row sums: each of the row's four lanes holds the sum of its 8 keys per tile.
  const float l_tot = sum_row_lanes(st.l);
  if (rho == 0) s_row_l[wave * 16 + j] = l_tot;
  const int64_t tree_row0 = w.row0;
  if (rho == 0 && row_valid) {
    if (w.slot < 0) {
      if (a.lse) a.lse[tree_row0 + row] = (st.m_ref + log2f(l_tot)) * mf::kLn2;
    } else {
      const int64_t srow = w.slot * q2::kRows + wave * 16 + j;
      a.ws_m[srow] = st.m_ref * mf::kLn2;
      a.ws_l[srow] = l_tot;
    }
  }
  __syncthreads();

  // Output, one row block (32 rows x 512 columns, fp32) at a time, through
  // LDS as in attn_mfma.hip: rows 0-15 staged in g_q2_k0, 16-31 in g_q2_k1.
  constexpr int kOutPitch = mf::DC * 4 + 16;
  const int rl = lane & 31;
  unsigned char* const stage_row = (rl < 16 ? g_q2_k0 : g_q2_k1) + (rl & 15) * kOutPitch;
  const int c16 = threadIdx.x & 127;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float lr = s_row_l[rb * 32 + rl];
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const f32x16_t& v = o[4 * rb + db];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int col = 128 * wave + 32 * g2 + 64 * (q4 & 1) + 8 * db + 4 * (q4 >> 1);
        *reinterpret_cast<float4*>(stage_row + col * 4) =
            make_float4(v[4 * q4] * inv, v[4 * q4 + 1] * inv, v[4 * q4 + 2] * inv, v[4 * q4 + 3] * inv);
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int pass = 0; pass < 16; ++pass) {
      const int rr = 2 * pass + (threadIdx.x >> 7);  // row within the block
      const int r = w.rb * q2::kRows + rb * 32 + rr;
      if (r < w.R) {
        const float4 v = *reinterpret_cast<const float4*>((rr < 16 ? g_q2_k0 : g_q2_k1) + (rr & 15) * kOutPitch +
                                                          c16 * 16);
        float* dst = w.slot < 0 ? a.out + (tree_row0 + r) * mf::DC
                                : a.ws_o + (w.slot * q2::kRows + rb * 32 + rr) * mf::DC;
        reinterpret_cast<float4*>(dst)[c16] = v;
      }
    }
    __syncthreads();
  }
}

// A uniform batch: one unit per workgroup.
__global__ __launch_bounds__(kMfmaThreads, 1) void attn_mfma_q2_kernel(AttnArgs a) {
  attn_mfma_q2_unit(a, decode_unit(a, unit_of_block(a, blockIdx.x)));
}

// A ragged batch: a persistent grid taking units from its XCD's counter.
__global__ __launch_bounds__(kMfmaThreads, 1) void attn_mfma_q2_ragged_kernel(AttnArgs) {
  for_each_ragged_unit([](const AttnArgs& a, const Unit& w) { attn_mfma_q2_unit(a, w); });
}

hipError_t launch_attn_mfma_q2(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(plan.units));
  if (a.req)
    attn_mfma_q2_ragged_kernel<<<grid, kMfmaThreads, 0, stream>>>(a);
  else
    attn_mfma_q2_kernel<<<grid, kMfmaThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace tv
