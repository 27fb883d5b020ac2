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
// Step t of the sweep is one barrier and one asm block (TV_STEP_ASM): the
// scores of tile t with the copy of tile t+1 HBM -> LDS woven in (three tile
// buffers in rotation), then the value product of tile t-1 with the mask, row
// max, exponentials, bf16 packing, row sums and LDS stores of tile t's weights
// woven in.
#include "attn_mfma_common.h"

namespace tv {

// Three kv tile buffers (row-major, as in HBM), used in rotation.
__shared__ __align__(16) unsigned char g_k0[mf::kBufBytes];
__shared__ __align__(16) unsigned char g_k1[mf::kBufBytes];
__shared__ __align__(16) unsigned char g_k2[mf::kBufBytes];
// Softmax weights of two consecutive tiles: [rb][key half h][lane][8 x bf16],
// lane l holding row 32 rb + l % 32 and keys 16 h + {4 g .. 4 g + 3,
// 8 + 4 g .. 8 + 4 g + 3} (g = l / 32) -- the B operand of the value MFMA.
__shared__ __align__(16) unsigned char g_p[2][mf::kPBytes];

// One step (TV_STEP_ASM): S^T = K Q^T for the tile in kc (lane: row
// lane % 32, keys 8 (i/4) + 4 g + i % 4 in score i), masked where bit i of
// vis is clear (if nm), row max folded into the state, weights exp2(s - ref)
// summed into st.l and stored to pc; O^T += V^T P^T for the previous tile; the
// copy of the next tile into kn.
__device__ __forceinline__ void step(const StepBufs& sb, const TreeKv& kv, const bf16x8_t* qf,
                                     const unsigned char* qrope, f32x16_t (&o)[16], RowState& st, int lane,
                                     int wave, int kt, uint32_t vis, int nm) {
  const int g2 = lane >> 5;
  const int grp = lane >> 4;
  const int j = lane & 15;
  const int key_l = lane & 31;
  // Score fragments: K row key_l, 16 bytes at 32 ks (latent) or chunk-major
  // rope; query rope fragments chunk-major in qrope.
  const uint32_t lat = lds_addr(sb.kc + key_l * mf::kLatRowBytes + g2 * 16);
  const uint32_t rope = lds_addr(sb.kc + mf::kLatBytes + (key_l >> 3) * 1024 + (key_l & 7) * 16 + g2 * 128);
  const uint32_t qr = lds_addr(qrope + g2 * (kMfmaRows * 16));
  // Value fragments by ds_read_b64_tr_b16: in each 16-lane group, lane
  // j = 4 m + q reads 8 bytes (4 consecutive latent columns) of key row
  // 4 g2 + m, and output lane 4 q + e receives element e of lane 4 m + q's
  // piece as its key m.  Lane (m, q) of group parity gp = grp & 1 reads the
  // columns 128 wave + 32 q + 8 db + 4 gp + {0..3} (column set db = 0..3), so
  // the 32 lanes served together (4 rows, row pitch 1040 B) fall on 32
  // distinct 8-byte bank slots; the accumulators' columns are permuted the
  // same way and put back in order when the output is stored.
  const uint32_t tb = lds_addr(sb.kp + (4 * g2 + (j >> 2)) * mf::kLatRowBytes + 64 * (j & 3) + 8 * (grp & 1) +
                               256 * wave);
  const uint32_t pb = lds_addr(sb.pp + lane * 16);
  const uint32_t pw = lds_addr(sb.pc + wave * 2048 + lane * 16);
  const StageArgs sa = stage_args(sb.kn, kv, kt + kMfmaKeys, wave, lane);
  // Scalar operands are wave-uniform by construction; readfirstlane makes
  // that visible to the compiler, which must place them in SGPRs.
  const uint32_t mb = __builtin_amdgcn_readfirstlane(sa.mb);
  const uint32_t mr = __builtin_amdgcn_readfirstlane(sa.mr);
  const int kb = __builtin_amdgcn_readfirstlane(sa.kb);
  const int km = __builtin_amdgcn_readfirstlane(kv.kmax);
  const int nms = __builtin_amdgcn_readfirstlane(nm);
  uint32_t t, ms;
  asm volatile(TV_STEP_ASM
               : [o0] "+a"(o[0]), [o1] "+a"(o[1]), [o2] "+a"(o[2]), [o3] "+a"(o[3]), [o4] "+a"(o[4]),
                 [o5] "+a"(o[5]), [o6] "+a"(o[6]), [o7] "+a"(o[7]), [o8] "+a"(o[8]), [o9] "+a"(o[9]),
                 [o10] "+a"(o[10]), [o11] "+a"(o[11]), [o12] "+a"(o[12]), [o13] "+a"(o[13]), [o14] "+a"(o[14]),
                 [o15] "+a"(o[15]), [l] "+v"(st.l), [mref] "+v"(st.m_ref), [mseen] "+v"(st.m_seen),
                 [exc] "+v"(st.exc), [t] "=&s"(t), [ms] "=&s"(ms)
               : [lat] "v"(lat), [rope] "v"(rope), [qr] "v"(qr), [tb] "v"(tb), [pb] "v"(pb), [pw] "v"(pw),
                 [mb] "s"(mb), [mr] "s"(mr), [kb] "s"(kb), [km] "s"(km), [l16] "v"(kv.lane16),
                 [ro] "v"(sa.ro), [rl] "s"(kv.lat), [rr] "s"(kv.rope), [mask] "v"(vis), [nm] "s"(nms),
                 [q0] "v"(qf[0]), [q1] "v"(qf[1]), [q2] "v"(qf[2]), [q3] "v"(qf[3]), [q4] "v"(qf[4]),
                 [q5] "v"(qf[5]), [q6] "v"(qf[6]), [q7] "v"(qf[7]), [q8] "v"(qf[8]), [q9] "v"(qf[9]),
                 [q10] "v"(qf[10]), [q11] "v"(qf[11]), [q12] "v"(qf[12]), [q13] "v"(qf[13]), [q14] "v"(qf[14]),
                 [q15] "v"(qf[15]), [q16] "v"(qf[16]), [q17] "v"(qf[17]), [q18] "v"(qf[18]), [q19] "v"(qf[19]),
                 [q20] "v"(qf[20]), [q21] "v"(qf[21]), [q22] "v"(qf[22]), [q23] "v"(qf[23]), [q24] "v"(qf[24]),
                 [q25] "v"(qf[25]), [q26] "v"(qf[26]), [q27] "v"(qf[27]), [q28] "v"(qf[28]), [q29] "v"(qf[29]),
                 [q30] "v"(qf[30]), [q31] "v"(qf[31])
               : TV_STEP_CLOBBERS, "vcc", "scc", "memory");
}

__device__ __forceinline__ void attn_mfma_bf16_unit(const AttnArgs& a, const Unit& w) {
  __shared__ int s_par[kMaxQ];
  __shared__ unsigned long long s_anc[kMaxQ * kAncWords];
  __shared__ __align__(16) unsigned char s_qrope[kMfmaRows * mf::DR * 2];  // 16 KB
  __shared__ float s_row_l[kMfmaRows];
  __shared__ int s_redo;
  __shared__ uint16_t s_vis[kMaxBoundaryTiles * kMfmaThreads];  // masks of the boundary tiles, per thread

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g2 = lane >> 5;
  const int P = w.P;
  // Raw buffers over this tree's rows (the host keeps kv_len * 1024 below
  // 2^31, so every offset fits in 32 bits).
  TreeKv kv;
  kv.lat = raw_buffer(static_cast<const uint16_t*>(a.c_kv) + w.kv_row0 * mf::DC,
                      static_cast<uint32_t>(w.kv_len) * (mf::DC * 2));
  kv.rope = raw_buffer(static_cast<const uint16_t*>(a.k_rope) + w.kv_row0 * mf::DR,
                       static_cast<uint32_t>(w.kv_len) * (mf::DR * 2));
  kv.lane16 = lane * 16;
  kv.kmax = w.k_end - 1;

  const int n_tiles = (w.k_end - w.k_begin + kMfmaKeys - 1) / kMfmaKeys;

  build_ancestors(a.parent + w.par0, w.q_len, s_par, s_anc);

  // This wave's own rows (row block rb = wave).
  const int row0 = w.rb * kMfmaRows + wave * 32;
  const int row = row0 + (lane & 31);
  const bool row_valid = row < w.R;
  const int node = min(row / a.H, w.q_len - 1);

  // Query fragments: q[row][8 g2 + 16 ks .. + 7] * sm_scale * log2(e) as bf16.
  // Latent part (ks < 32) in registers; rope part in LDS, chunk-major:
  // 16-byte chunk c of block row r at s_qrope + (c * 128 + r) * 16.  Rows past
  // R get zero queries (their results are never stored).
  bf16x8_t qf[mf::KSTEPS_LAT];
  {
    const float sc = a.sm_scale * mf::kLog2e;
    const int64_t grow = w.row0 + (row_valid ? row : 0);
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

  // Visibility of the boundary tiles: the tiles from t_first on hold tree keys
  // or the range end (kt + 32 > min(P, k_end)); at most q_len / 32 + 2 of
  // them.  Score i of this thread holds key kt + 8 (i/4) + 4 g2 + i % 4;
  // bit i of its mask says whether that key is visible from the row's node.
  const int t_first = max(0, (min(P, w.k_end) - w.k_begin) / kMfmaKeys);
  {
    const int n_bt = min(n_tiles - t_first, kMaxBoundaryTiles);
    for (int j = 0; j < n_bt; ++j) {
      const int kt = w.k_begin + (t_first + j) * kMfmaKeys;
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt + 8 * (i >> 2) + 4 * g2 + (i & 3);
        m |= key_visible(s_anc, node, key, P, w.k_end) << i;
      }
      s_vis[j * kMfmaThreads + threadIdx.x] = static_cast<uint16_t>(m);
    }
  }

  // o[4 rb + db][i] = O[32 rb + lane % 32][col(db, i)] with (value-operand row
  // 8 (i/4) + 4 g2 + i % 4 = 16 gp + 4 q + e, see step)
  //   col(db, i) = 128 wave + 32 q + 8 db + 4 gp + e
  //              = 128 wave + 64 ((i >> 2) & 1) + 32 g2 + 8 db + 4 (i >> 3) + (i & 3).
  f32x16_t o[16];
  RowState st;
  st.m_ref = -INFINITY;
  st.m_seen = -INFINITY;

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = f32x16_t{};
    st.l = 0.f;
    st.exc = -INFINITY;
    // The weights "before tile 0" are zeros, so step 0's value product adds
    // nothing (it reads tile 0's finite latent rows).
    *reinterpret_cast<uint4*>(g_p[1] + threadIdx.x * 32) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(g_p[1] + threadIdx.x * 32 + 16) = make_uint4(0, 0, 0, 0);
    stage_tile(g_k0, kv, w.k_begin, wave, lane);
    unsigned char* kp = g_k2;  // tile t-1
    unsigned char* kc = g_k0;  // tile t
    unsigned char* kn = g_k1;  // tile t+1
    // Step t: scores of tile t, value product of tile t-1, copy of tile t+1.
    // The extra step t = n_tiles has nothing to score (every key masked; its
    // tile buffer holds the clamped copy made at the step before) and runs
    // the value product of the last tile.  Copies past the unit's range are
    // clamped to its last row and land in buffers nobody reads again.
    for (int t = 0; t <= n_tiles; ++t) {
      // Tile t (this wave's copies) has landed; after the barrier every wave's
      // has, the weights of tile t-1 are in LDS, and tile t-2's buffer (kn) and
      // weights buffer are no longer read.  The barrier alone drains only LDS
      // instructions, not the HBM->LDS copies, and the compiler cannot see the
      // LDS accesses inside the asm blocks.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int kt = w.k_begin + t * kMfmaKeys;
      uint32_t vis = 0xffffu;
      int nm = 0;
      if (t == n_tiles) {
        vis = 0;
        nm = 1;
      } else if (kt + kMfmaKeys > P || kt + kMfmaKeys > w.k_end) {
        nm = 1;
        vis = s_vis[min(t - t_first, kMaxBoundaryTiles - 1) * kMfmaThreads + threadIdx.x];
      }
      const StepBufs sb{kc, t == 0 ? kc : kp, kn, g_p[(t + 1) & 1], g_p[t & 1]};
      step(sb, kv, qf, qrope, o, st, lane, wave, kt, vis, nm);
      unsigned char* nx = kp;
      kp = kc;
      kc = kn;
      kn = nx;
    }
    asm volatile("s_waitcnt vmcnt(0)\n" TV_MFMA_DRAIN_ASM ::: "memory");
    // Re-sweep (once, with the exact max as reference) if any row overflowed headroom.
    const bool over = st.exc > mf::kHeadroom;
    if (threadIdx.x == 0) s_redo = 0;
    __syncthreads();
    if (__any(over) && lane == 0) s_redo = 1;
    __syncthreads();
    if (pass > 0 || s_redo == 0) break;
    // Only rows that ran out of headroom move their reference, so every other
    // row repeats its first sweep bit for bit (a row's result never depends on
    // another row's scores).
    st.m_ref = over ? st.m_seen : st.m_ref;
  }

  // Row sums of the wave's own rows, for all four waves.
  const float l_tot = sum_halves(st.l);
  if (g2 == 0) s_row_l[wave * 32 + lane] = l_tot;
  const int64_t tree_row0 = w.row0;
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

  // Output, one row block (32 rows x 512 columns, fp32) at a time, through LDS
  // so that every store instruction writes whole rows: each wave drops its 128
  // columns of the 32 rows (normalised by the row sum) into the idle tile
  // buffers, rows 0-15 in g_k0 and 16-31 in g_k1 at a 2064-byte pitch (16 rows
  // of 128-bit writes hit 16 different bank groups); then all 256 threads copy
  // two 2 KB rows per pass, 16 bytes each, to HBM.
  constexpr int kOutPitch = mf::DC * 4 + 16;
  const int rl = lane & 31;
  unsigned char* const stage_row = (rl < 16 ? g_k0 : g_k1) + (rl & 15) * kOutPitch;
  const int c16 = threadIdx.x & 127;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
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
      const int r = w.rb * kMfmaRows + rb * 32 + rr;
      if (r < w.R) {
        const float4 v = *reinterpret_cast<const float4*>((rr < 16 ? g_k0 : g_k1) + (rr & 15) * kOutPitch + c16 * 16);
        float* dst = w.slot < 0 ? a.out + (tree_row0 + r) * mf::DC
                                : a.ws_o + (w.slot * kMfmaRows + rb * 32 + rr) * mf::DC;
        reinterpret_cast<float4*>(dst)[c16] = v;
      }
    }
    __syncthreads();
  }
}

// A uniform batch: one unit per workgroup.
__global__ __launch_bounds__(kMfmaThreads, 1) void attn_mfma_bf16_kernel(AttnArgs a) {
  attn_mfma_bf16_unit(a, decode_unit(a, unit_of_block(a, blockIdx.x)));
}

hipError_t launch_attn_mfma_bf16(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  // Ragged batches always run the two-term kernel (their entry points take no
  // query-precision option).
  if (a.req) return hipErrorNotSupported;
  attn_mfma_bf16_kernel<<<dim3(static_cast<unsigned>(plan.units)), kMfmaThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace tv
