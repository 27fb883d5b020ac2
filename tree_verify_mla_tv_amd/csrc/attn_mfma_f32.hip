// Tree-verify MLA-absorb attention for an fp32 cache with d_c = 512, d_r = 64:
// the fp32 matrix-core kernel (v_mfma_f32_16x16x4_f32).
//
// [Verify page = "The Precision Imperative: Validating Numerical Accuracy in a
//  Custom CUDA Attention Kernel", "The Context: What Led to This Moment": masked
//  absorb attention in three parts (scores, softmax normalisation, weighted
//  accumulation).  Golden page = "The Golden Reference: A Pivotal Moment in
//  Building a Native DDTree Inference Engine", "The Absorb Form of MLA": one
//  latent row per key serves every head, and it is both the key (with its rope
//  part) and the value.]
//
// One workgroup = 4 waves = 64 query rows (node, head) of one tree; wave w owns
// rows 16 w .. 16 w + 15 of the block.  Keys stream through LDS 32 at a time as
// fp32 rows [c_kv | k_rope] (576 floats, padded to 580 so the 16 rows a
// 16-byte read touches fall in distinct banks), in two tile buffers: the next
// tile is loaded into registers half at a time while the current one is in
// use (its second half is stored before the value product, whose operand
// reads need the registers).
//
// Scores S^T (32 keys x 16 rows per wave) = K Q^T as two 16 x 16 blocks.  In
// v_mfma_f32_16x16x4_f32 lane l supplies A[l % 16][l / 16] and B[l / 16][l %
// 16], and holds D[4 (l / 16) + v][l % 16] in register v.  The 576-term dot
// product is taken in a different order than d = 0 .. 575: step s of lane
// group g = l / 16 contracts d = 144 g + s, so each lane reads four steps of its
// key row with one 16-byte LDS load and keeps its query row's 144 values of
// quarter g in registers (scaled by sm_scale * log2(e), so scores come out in
// log2 units).
//
// Softmax: a per-row reference maximum m_ref, set by the first tile with a
// visible key, is kept for the whole sweep (weights exp2(s - m_ref) are not
// rescaled); scores more than 64 above it (where a weight could leave the range
// fp32 carries safely) send the workgroup through the sweep once more with
// m_ref = the row's maximum over the sweep.  Weights stay fp32.
//
// Value product O^T (512 x 16 rows per wave) = V^T P^T: the contraction over
// keys runs in the order in which the score blocks already hold them (lane
// group g, register v of block b = key 16 b + 4 g + v), so the weights feed the
// matrix core straight from the score registers.  O^T lives in 32 blocks of 16
// x 16 (128 registers per lane); block 4 m + r holds the d = 64 m + 4 x + r
// (x = 0 .. 15), so each 16-byte read of a value row feeds four blocks.
#include "tv_kernels.h"

namespace tv {

namespace {

constexpr int DC = 512, DR = 64, D = DC + DR;
constexpr int kQuarter = D / 4;                        // 144 contraction steps per lane group
constexpr int kStride = D + 4;                         // LDS row stride in floats
constexpr int kTileChunks = kF32Keys * (D / 4);        // float4 chunks per key tile
constexpr int kTileFloats = kF32Keys * kStride;
constexpr int kHalfChunks = kTileChunks / 2 / kF32Threads;  // per thread, per half tile
constexpr float kHeadroom = 64.f;                      // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
static_assert(kTileChunks % (2 * kF32Threads) == 0 && kHalfChunks == DC / 64 + 1 && DR == 64 && kF32Threads == 256,
              "a half tile is 16 rows x (8 latent + 1 rope) float4 columns of 16 threads");
static_assert(kF32Rows == 64 && kF32Keys == 32 && kF32Threads == 256, "geometry");

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma16(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// This thread's share of half h of key tile [kt, kt + 32): row 16 h + t / 16
// of the tile, float4 columns t % 16 + 16 i (i < 8: the latent row, 256 bytes
// apart) and the rope row's float4 t % 16, so a thread keeps two base
// addresses.  Rows past the unit's range end read the last row; they are
// stored as 0 (store_half), the select made at the store so that the loads
// do not wait.  Returns whether the row is in range.
__device__ __forceinline__ bool load_half(const AttnArgs& a, const Unit& w, int kt, int h,
                                          float4 (&r)[kHalfChunks]) {
  const int row = 16 * h + (threadIdx.x >> 4);
  const int cg = threadIdx.x & 15;
  const int key = kt + row;
  const int64_t krow = w.kv_row0 + min(key, w.k_end - 1);
  const float* lat = static_cast<const float*>(a.c_kv) + krow * DC + 4 * cg;
  const float* rope = static_cast<const float*>(a.k_rope) + krow * DR + 4 * cg;
#pragma unroll
  for (int i = 0; i < DC / 64; ++i) r[i] = *reinterpret_cast<const float4*>(lat + 64 * i);
  r[DC / 64] = *reinterpret_cast<const float4*>(rope);
  return key < w.k_end;
}

// (component-wise selects: a select of whole float4s was compiled through
// private memory)
__device__ __forceinline__ void store_half(float* buf, int h, const float4 (&r)[kHalfChunks], bool in) {
  float* dst = buf + (16 * h + (threadIdx.x >> 4)) * kStride + 4 * (threadIdx.x & 15);
#pragma unroll
  for (int i = 0; i <= DC / 64; ++i) {
    const float4 v = r[i];
    *reinterpret_cast<float4*>(dst + (i < DC / 64 ? 64 * i : DC)) =
        make_float4(in ? v.x : 0.f, in ? v.y : 0.f, in ? v.z : 0.f, in ? v.w : 0.f);
  }
}

}  // namespace

__device__ __forceinline__ void attn_mfma_f32_unit(const AttnArgs& a, const Unit& w) {
  __shared__ __align__(16) float sK[2 * kTileFloats];  // two key tiles: the one in use and the next
  __shared__ int s_par[kMaxQ];
  __shared__ unsigned long long s_anc[kMaxQ * kAncWords];
  __shared__ int s_redo;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ln = lane & 15;  // query row within the wave's 16; key / d within a 16-block
  const int lg = lane >> 4;  // lane group: contraction quarter (scores), key group (values)
  const int P = w.P;

  const int r_blk = wave * 16 + ln;  // row within the block
  const int row = w.rb * kF32Rows + r_blk;
  const bool row_valid = row < w.R;
  const int node = min(row / a.H, w.q_len - 1);

  const int n_tiles = (w.k_end - w.k_begin + kF32Keys - 1) / kF32Keys;
  // The block's 64 query rows come in coalesced (consecutive threads read
  // consecutive 16-byte pieces of a row; rows past R read row 0 of the tree)
  // and go to the idle tile buffers at the tile's row pitch; each lane then
  // reads its quarter back.  (Read straight from HBM, each lane's quarter made
  // every load instruction touch 64 separate pieces of 16 rows.)  The first
  // key tile's first half is requested with them, and the tree's ancestor
  // masks are built while both are in flight.
  static_assert(kF32Rows * kStride <= 2 * kTileFloats, "the query block fits the tile buffers");
  static_assert(kMaxQ <= kF32Threads, "one parent per thread");
  constexpr int kQChunks = kF32Rows * (D / 4) / kF32Threads;  // 36 float4 per thread
  // Every load of the prologue is issued before the first wait, queries
  // first (waits count loads in issue order): one memory round trip instead
  // of one per batch.
  floatx4 x[kQChunks];
#pragma unroll
  for (int i = 0; i < kQChunks; ++i) {
    const int idx = threadIdx.x + kF32Threads * i;
    const int r = idx / (D / 4), d = 4 * (idx - r * (D / 4));
    const int gr = w.rb * kF32Rows + r;
    const int64_t grow = w.row0 + (gr < w.R ? gr : 0);
    const float* src = d < DC ? a.q_lat + grow * DC + d : a.q_rope + grow * DR + (d - DC);
    x[i] = *reinterpret_cast<const floatx4*>(src);
  }
  float4 pre[kHalfChunks];
  bool pre_in = false;
  if (n_tiles > 0) pre_in = load_half(a, w, w.k_begin, 0, pre);
  const int par_t = a.parent[w.par0 + min(static_cast<int>(threadIdx.x), w.q_len - 1)];
  // Every load above is issued before anything waits: the empty asm (with a
  // memory clobber) keeps the loads above it and the LDS stores below it, and
  // hands over the query values there.  (Left alone, the compiler paired each
  // load with its store and waited for each in turn.)
#pragma unroll
  for (int i = 0; i < kQChunks; i += 4) asm volatile("" : "+v"(x[i]), "+v"(x[i + 1]), "+v"(x[i + 2]), "+v"(x[i + 3])::"memory");
#pragma unroll
  for (int i = 0; i < kQChunks; ++i) {
    const int idx = threadIdx.x + kF32Threads * i;
    const int r = idx / (D / 4), d = 4 * (idx - r * (D / 4));
    *reinterpret_cast<floatx4*>(sK + r * kStride + d) = x[i];
  }
  build_ancestors_loaded(par_t, w.q_len, s_par, s_anc);  // ends with a barrier: the query block is in LDS
  // Query quarter lg of this lane's row: d = 144 lg + s, scaled; zero past R.
  float qf[kQuarter];
  {
    const float sc = row_valid ? a.sm_scale * kLog2e : 0.f;
    const float* qs = sK + r_blk * kStride + lg * kQuarter;
#pragma unroll
    for (int c = 0; c < kQuarter / 4; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(qs + 4 * c);
      qf[4 * c] = x.x * sc;
      qf[4 * c + 1] = x.y * sc;
      qf[4 * c + 2] = x.z * sc;
      qf[4 * c + 3] = x.w * sc;
    }
  }
  __syncthreads();  // the tile buffers are free again

  float m_ref = -INFINITY, m_seen = -INFINITY, exc = -INFINITY, l_run = 0.f;
  floatx4 o[DC / 16];
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int j = 0; j < DC / 16; ++j) o[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    if (n_tiles > 0) {
      if (pass > 0) pre_in = load_half(a, w, w.k_begin, 0, pre);
      store_half(sK, 0, pre, pre_in);
      pre_in = load_half(a, w, w.k_begin, 1, pre);
      store_half(sK, 1, pre, pre_in);
    }
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
      // Tile t is in buffer t % 2; the next tile goes to the other buffer in
      // two halves, loaded before and stored after each phase.  The barrier at
      // the end of a tile separates the reads of a buffer from its next fill.
      const int kt = w.k_begin + t * kF32Keys;
      const float* cur = sK + (t & 1) * kTileFloats;
      float* nxt = sK + ((t + 1) & 1) * kTileFloats;
      const bool more = t + 1 < n_tiles;
      if (more) pre_in = load_half(a, w, kt + kF32Keys, 0, pre);

      // Scores: block b holds keys 16 b + 4 lg + v (register v) of row ln.
      floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      {
        const float* k0 = cur + ln * kStride + lg * kQuarter;
        const float* k1 = k0 + 16 * kStride;
#pragma unroll
        for (int c = 0; c < kQuarter / 4; ++c) {
          const float4 a0 = *reinterpret_cast<const float4*>(k0 + 4 * c);
          const float4 a1 = *reinterpret_cast<const float4*>(k1 + 4 * c);
          s0 = mfma16(a0.x, qf[4 * c], s0);
          s1 = mfma16(a1.x, qf[4 * c], s1);
          s0 = mfma16(a0.y, qf[4 * c + 1], s0);
          s1 = mfma16(a1.y, qf[4 * c + 1], s1);
          s0 = mfma16(a0.z, qf[4 * c + 2], s0);
          s1 = mfma16(a1.z, qf[4 * c + 2], s1);
          s0 = mfma16(a0.w, qf[4 * c + 3], s0);
          s1 = mfma16(a1.w, qf[4 * c + 3], s1);
        }
      }
      if (more) {
        store_half(nxt, 0, pre, pre_in);
        pre_in = load_half(a, w, kt + kF32Keys, 1, pre);
      }
      float p[8];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[v] = s0[v];
        p[4 + v] = s1[v];
      }
      // Mask: keys past the range end, and tree keys that are not ancestors of
      // the row's node (only tiles reaching the tree keys or the range end).
      // key_visible is straight-line; one select per score.
      if (kt + kF32Keys > min(P, w.k_end)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int key = kt + 16 * (i >> 2) + 4 * lg + (i & 3);
          p[i] = key_visible(s_anc, node, key, P, w.k_end) != 0u ? p[i] : -INFINITY;
        }
      }
      float tmax = p[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, p[i]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      m_seen = fmaxf(m_seen, tmax);
      if (pass == 0) {
        m_ref = m_ref == -INFINITY ? tmax : m_ref;
        exc = fmaxf(exc, tmax - m_ref);  // NaN (nothing visible yet) leaves exc as it is
      }
      const float mr = m_ref == -INFINITY ? 0.f : m_ref;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = exp2f(p[i] - mr);  // -inf (masked) -> 0
        l_run += p[i];
      }

      // The next tile's second half goes to LDS before the value product, so
      // its registers are free for the value operands.
      if (more) store_half(nxt, 1, pre, pre_in);

      // Values: contraction step (b, v) takes key 16 b + 4 lg + v of lane group
      // lg.  Output block 4 m + r holds d = 64 m + 4 x + r in its row x, so a
      // lane's operands for blocks 4 m .. 4 m + 3 are the four consecutive
      // floats at d = 64 m + 4 ln: one 16-byte LDS read feeds four products.
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float* vrow = cur + (16 * (i >> 2) + 4 * lg + (i & 3)) * kStride + 4 * ln;
#pragma unroll
        for (int m = 0; m < DC / 64; ++m) {
          const float4 va = *reinterpret_cast<const float4*>(vrow + 64 * m);
          o[4 * m] = mfma16(va.x, p[i], o[4 * m]);
          o[4 * m + 1] = mfma16(va.y, p[i], o[4 * m + 1]);
          o[4 * m + 2] = mfma16(va.z, p[i], o[4 * m + 2]);
          o[4 * m + 3] = mfma16(va.w, p[i], o[4 * m + 3]);
        }
      }
      __syncthreads();
    }

    if (pass > 0) break;
    if (threadIdx.x == 0) s_redo = 0;
    __syncthreads();
    const bool over = exc > kHeadroom;
    if (over) s_redo = 1;
    __syncthreads();
    if (s_redo == 0) break;
    // Only rows that ran out of headroom move their reference, so every other
    // row repeats its first sweep bit for bit.
    m_ref = over ? m_seen : m_ref;
  }

  // Row sum over the four lane groups that share the row.
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_valid && lg == 0) {
    if (w.slot < 0) {
      if (a.lse) a.lse[w.row0 + row] = (m_ref + log2f(l_tot)) * kLn2;
    } else {
      const int64_t srow = w.slot * kF32Rows + r_blk;
      a.ws_m[srow] = m_ref * kLn2;
      a.ws_l[srow] = l_tot;
    }
  }
  // Output through LDS, so that each store instruction writes 1 KB of
  // consecutive bytes (written straight from the accumulators, a store
  // touched 16 B in each of 64 places).  The tile buffers are free: every wave
  // has passed a barrier since its last read of them.  Register v of block
  // 4 m + r holds d = 64 m + 4 (4 lg + v) + r of row ln; a row's staging
  // pitch of 516 floats puts the 16 rows a store serves in distinct banks.
  constexpr int kOutStride = DC + 4;
  static_assert(kF32Rows * kOutStride <= 2 * kTileFloats, "the output block fits the tile buffers");
  float* const so = sK;
#pragma unroll
  for (int m = 0; m < DC / 64; ++m)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      *reinterpret_cast<float4*>(so + r_blk * kOutStride + 64 * m + 16 * lg + 4 * v) =
          make_float4(o[4 * m][v] * inv, o[4 * m + 1][v] * inv, o[4 * m + 2][v] * inv, o[4 * m + 3][v] * inv);
  __syncthreads();
  const int rows = min(kF32Rows, w.R - w.rb * kF32Rows);  // rows of the block that exist
  float* const dst = w.slot < 0 ? a.out + (w.row0 + static_cast<int64_t>(w.rb) * kF32Rows) * DC
                                : a.ws_o + w.slot * kF32Rows * DC;
  for (int idx = threadIdx.x; idx < rows * (DC / 4); idx += kF32Threads) {
    const int r = idx / (DC / 4);
    const int c4 = idx - r * (DC / 4);
    *reinterpret_cast<float4*>(dst + static_cast<int64_t>(r) * DC + 4 * c4) =
        *reinterpret_cast<const float4*>(so + r * kOutStride + 4 * c4);
  }
}

// A uniform batch: one unit per workgroup.
__global__ __launch_bounds__(kF32Threads, 1) void attn_mfma_f32_kernel(AttnArgs a) {
  attn_mfma_f32_unit(a, decode_unit(a, unit_of_block(a, blockIdx.x)));
}

// A ragged batch: a persistent grid taking units from its XCD's counter.
__global__ __launch_bounds__(kF32Threads, 1) void attn_mfma_f32_ragged_kernel(AttnArgs) {
  for_each_ragged_unit([](const AttnArgs& a, const Unit& w) { attn_mfma_f32_unit(a, w); });
}

hipError_t launch_attn_mfma_f32(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(plan.units));
  if (a.req)
    attn_mfma_f32_ragged_kernel<<<grid, kF32Threads, 0, stream>>>(a);
  else
    attn_mfma_f32_kernel<<<grid, kF32Threads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace tv
