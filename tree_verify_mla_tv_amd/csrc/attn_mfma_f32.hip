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
#include <type_traits>

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

// ---------------------------------------------------------------------------
// The narrow form, for uniform batches whose 64-row blocks are too few to
// fill the GPU: one workgroup = 32 query rows (node, head) of one tree, and the
// unit's keys are cut in two halves of 16-key tiles (the first half takes the
// odd tile when their count is odd).  Waves 0 and 1 take rows 0-15 and 16-31
// over the first half, waves 2 and 3 the same rows over the second.  The two
// halves of a row are combined by log-sum-exp weights through LDS before the
// output leaves, so a kv piece of the plan serves twice the workgroups of the
// wide form with the same partial results per row.
//
// The block's scaled queries stay in LDS (32 rows at the 580-float pitch) and
// each half has one 16-key tile buffer beside them; the matrix core's query
// operands are read from LDS like its key operands, which leaves the registers
// that the wide form spends on its query quarter (144 per lane) free for
// reading operands ahead of their use and for holding the whole next tile
// (18 float4 per thread), loaded at the start of a tile and stored after it.
// Per wave and tile: the scores of 16 keys (144 products as two accumulation
// chains, chunks c and c + 18 of each lane group's quarter), the values of
// those 16 keys (128 products), as in the wide form's one 16-key block.
namespace {

constexpr int kNarrowTileFloats = kF32NarrowKeys * kStride;
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
static_assert(kF32NarrowRows == 32 && kF32NarrowKeys == 16, "two row groups of 16, two halves of 16-key tiles");
static_assert(kF32NarrowRows * kStride + 2 * kNarrowTileFloats == 2 * kTileFloats,
              "queries and two tile buffers take the wide form's LDS");

// Thread th (0 .. 127) of a half's two waves: part p of the half's tile at kt,
// row 8 p + th / 16, float4 columns th % 16 + 16 i and the rope float4 th % 16
// (load_half's pattern over 128 threads).  Rows at or past the half's end he
// read the unit's last row and are stored as 0.
__device__ __forceinline__ bool load_part(const AttnArgs& a, const Unit& w, int th, int kt, int he, int p,
                                          float4 (&r)[kHalfChunks]) {
  const int row = 8 * p + (th >> 4);
  const int cg = th & 15;
  const int key = kt + row;
  const int64_t krow = w.kv_row0 + min(key, w.k_end - 1);
  const float* lat = static_cast<const float*>(a.c_kv) + krow * DC + 4 * cg;
  const float* rope = static_cast<const float*>(a.k_rope) + krow * DR + 4 * cg;
#pragma unroll
  for (int i = 0; i < DC / 64; ++i) r[i] = *reinterpret_cast<const float4*>(lat + 64 * i);
  r[DC / 64] = *reinterpret_cast<const float4*>(rope);
  return key < he;
}

__device__ __forceinline__ void store_part(float* buf, int th, int p, const float4 (&r)[kHalfChunks], bool in) {
  float* dst = buf + (8 * p + (th >> 4)) * kStride + 4 * (th & 15);
#pragma unroll
  for (int i = 0; i <= DC / 64; ++i) {
    const float4 v = r[i];
    *reinterpret_cast<float4*>(dst + (i < DC / 64 ? 64 * i : DC)) =
        make_float4(in ? v.x : 0.f, in ? v.y : 0.f, in ? v.z : 0.f, in ? v.w : 0.f);
  }
}

}  // namespace

__device__ __forceinline__ void attn_mfma_f32_narrow_unit(const AttnArgs& a, const Unit& w) {
  __shared__ __align__(16) float sQ[kF32NarrowRows * kStride];   // the block's scaled queries
  __shared__ __align__(16) float sK[2 * kNarrowTileFloats];      // one tile per half
  __shared__ int s_par[kMaxQ];
  __shared__ unsigned long long s_anc[kMaxQ * kAncWords];
  __shared__ float s_mh[2][kF32NarrowRows], s_lh[2][kF32NarrowRows];  // each half's row max and sum
  __shared__ int s_redo;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int kh = wave >> 1;               // kv half
  const int th = threadIdx.x & 127;       // thread within the half's two waves
  const int r_blk = 16 * (wave & 1) + ln;  // row within the block
  const int row = w.rb * kF32NarrowRows + r_blk;
  const bool row_valid = row < w.R;
  const int node = min(row / a.H, w.q_len - 1);
  const int P = w.P;

  // Tiles of the half: keys [hb, he).  The second half may hold one tile
  // fewer, or none: its loop still runs the first half's count (masked
  // tiles), so both pairs meet at every barrier.
  const int n16 = (w.k_end - w.k_begin + kF32NarrowKeys - 1) / kF32NarrowKeys;
  const int nt = (n16 + 1) / 2;
  const int hb = w.k_begin + kh * nt * kF32NarrowKeys;
  const int he = kh == 0 ? min(w.k_end, hb + nt * kF32NarrowKeys) : w.k_end;

  // Prologue: the block's 32 query rows coalesced (rows past R read row 0 of
  // the tree and are stored as 0), the half's first tile and the parents,
  // all requested before anything waits.
  constexpr int kQChunks = kF32NarrowRows * (D / 4) / kF32Threads;  // 18 float4 per thread
  floatx4 x[kQChunks];
#pragma unroll
  for (int i = 0; i < kQChunks; ++i) {
    const int idx = threadIdx.x + kF32Threads * i;
    const int r = idx / (D / 4), d = 4 * (idx - r * (D / 4));
    const int gr = w.rb * kF32NarrowRows + r;
    const int64_t grow = w.row0 + (gr < w.R ? gr : 0);
    const float* src = d < DC ? a.q_lat + grow * DC + d : a.q_rope + grow * DR + (d - DC);
    x[i] = *reinterpret_cast<const floatx4*>(src);
  }
  float4 st0[kHalfChunks], st1[kHalfChunks];  // the next tile of the half, parts 0 and 1
  bool in0 = false, in1 = false;
  if (nt > 0) {
    in0 = load_part(a, w, th, hb, he, 0, st0);
    in1 = load_part(a, w, th, hb, he, 1, st1);
  }
  const int par_t = a.parent[w.par0 + min(static_cast<int>(threadIdx.x), w.q_len - 1)];
#pragma unroll
  for (int i = 0; i < kQChunks; i += 2) asm volatile("" : "+v"(x[i]), "+v"(x[i + 1])::"memory");
  {
    const float sc = a.sm_scale * kLog2e;  // scores in log2 units
#pragma unroll
    for (int i = 0; i < kQChunks; ++i) {
      const int idx = threadIdx.x + kF32Threads * i;
      const int r = idx / (D / 4), d = 4 * (idx - r * (D / 4));
      const float s = w.rb * kF32NarrowRows + r < w.R ? sc : 0.f;
      *reinterpret_cast<floatx4*>(sQ + r * kStride + d) = x[i] * s;
    }
  }
  build_ancestors_loaded(par_t, w.q_len, s_par, s_anc);  // ends with a barrier

  float* const mine = sK + kh * kNarrowTileFloats;  // this half's tile buffer
  const float* const kq = mine + ln * kStride + lg * kQuarter;  // key ln's quarter lg
  const float* const qq = sQ + r_blk * kStride + lg * kQuarter;  // row r_blk's quarter lg
  float m_ref = -INFINITY, m_seen = -INFINITY, exc = -INFINITY, l_run = 0.f;
  floatx4 o[DC / 16];
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int j = 0; j < DC / 16; ++j) o[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    if (nt > 0) {
      if (pass > 0) {
        in0 = load_part(a, w, th, hb, he, 0, st0);
        in1 = load_part(a, w, th, hb, he, 1, st1);
      }
      store_part(mine, th, 0, st0, in0);
      store_part(mine, th, 1, st1, in1);
    }
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
      const int kt = hb + t * kF32NarrowKeys;
      const bool more = t + 1 < nt;
      if (more) {
        in0 = load_part(a, w, th, kt + kF32NarrowKeys, he, 0, st0);
        in1 = load_part(a, w, th, kt + kF32NarrowKeys, he, 1, st1);
      }

      // Scores: register v holds key 4 lg + v of row ln; each chunk's key and
      // query values are read one chunk ahead of their use.
      floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      {
        constexpr int kHalfQ = kQuarter / 8;  // 18 chunks per chain
        float4 ka[2], kb[2], qa[2], qb[2];
        ka[0] = *reinterpret_cast<const float4*>(kq);
        kb[0] = *reinterpret_cast<const float4*>(kq + 4 * kHalfQ);
        qa[0] = *reinterpret_cast<const float4*>(qq);
        qb[0] = *reinterpret_cast<const float4*>(qq + 4 * kHalfQ);
#pragma unroll
        for (int c = 0; c < kHalfQ; ++c) {
          const int u = c & 1;
          if (c + 1 < kHalfQ) {
            ka[u ^ 1] = *reinterpret_cast<const float4*>(kq + 4 * (c + 1));
            kb[u ^ 1] = *reinterpret_cast<const float4*>(kq + 4 * (c + 1 + kHalfQ));
            qa[u ^ 1] = *reinterpret_cast<const float4*>(qq + 4 * (c + 1));
            qb[u ^ 1] = *reinterpret_cast<const float4*>(qq + 4 * (c + 1 + kHalfQ));
          }
          s0 = mfma16(ka[u].x, qa[u].x, s0);
          s1 = mfma16(kb[u].x, qb[u].x, s1);
          s0 = mfma16(ka[u].y, qa[u].y, s0);
          s1 = mfma16(kb[u].y, qb[u].y, s1);
          s0 = mfma16(ka[u].z, qa[u].z, s0);
          s1 = mfma16(kb[u].z, qb[u].z, s1);
          s0 = mfma16(ka[u].w, qa[u].w, s0);
          s1 = mfma16(kb[u].w, qb[u].w, s1);
        }
        // Schedule: the first chunk's four reads, then per chunk the next
        // chunk's four reads ahead of its eight products.
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
        for (int c = 0; c < kHalfQ; ++c) {
          if (c + 1 < kHalfQ) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 0);
        }
      }
      float p[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) p[v] = s0[v] + s1[v];
      if (kt + kF32NarrowKeys > min(P, he)) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          p[v] = key_visible(s_anc, node, kt + 4 * lg + v, P, he) != 0u ? p[v] : -INFINITY;
      }
      float tmax = fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3]));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      m_seen = fmaxf(m_seen, tmax);
      if (pass == 0) {
        m_ref = m_ref == -INFINITY ? tmax : m_ref;
        exc = fmaxf(exc, tmax - m_ref);  // NaN (nothing visible yet) leaves exc as it is
      }
      const float mr = m_ref == -INFINITY ? 0.f : m_ref;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[v] = exp2f(p[v] - mr);  // -inf (masked) -> 0
        l_run += p[v];
      }

      // Values: step v takes key 4 lg + v; block 4 m + r holds d = 64 m + 4 x
      // + r.  A step's eight value reads are issued one step ahead.
      {
        const float* vrow = mine + (4 * lg) * kStride + 4 * ln;
        float4 vb[2][DC / 64];
#pragma unroll
        for (int m = 0; m < DC / 64; ++m) vb[0][m] = *reinterpret_cast<const float4*>(vrow + 64 * m);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (v + 1 < 4) {
#pragma unroll
            for (int m = 0; m < DC / 64; ++m)
              vb[(v + 1) & 1][m] = *reinterpret_cast<const float4*>(vrow + (v + 1) * kStride + 64 * m);
          }
#pragma unroll
          for (int m = 0; m < DC / 64; ++m) {
            const float4 va = vb[v & 1][m];
            o[4 * m] = mfma16(va.x, p[v], o[4 * m]);
            o[4 * m + 1] = mfma16(va.y, p[v], o[4 * m + 1]);
            o[4 * m + 2] = mfma16(va.z, p[v], o[4 * m + 2]);
            o[4 * m + 3] = mfma16(va.w, p[v], o[4 * m + 3]);
          }
        }
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, DC / 64, 1);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (v + 1 < 4) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, DC / 64, 1);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, DC / 16, 1);
        }
      }
      // Every wave is done with the tile before the next one replaces it.
      __syncthreads();
      if (more) {
        store_part(mine, th, 0, st0, in0);
        store_part(mine, th, 1, st1, in1);
        __syncthreads();
      }
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

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);

  // The two halves of a row are combined through LDS, each half's waves
  // finishing half the columns: the first half d < 256 (m < 4), the second
  // d >= 256.  Each wave writes its unnormalised accumulators of the columns
  // the other half finishes, and its row max and sum; both halves then take
  // the same weights (the same operations on the same four numbers) and leave
  // the normalised values of their columns at the same places.  Register v of
  // block 4 m + r holds d = 64 m + 4 (4 lg + v) + r of row ln (the wide form's
  // staging layout, pitch 516 floats, here in the query buffer).  Every wave
  // has passed a barrier since its last read of the queries.
  constexpr int kOutStride = DC + 4;
  constexpr int kHalfM = DC / 128;  // column groups of 64 per half
  static_assert(kF32NarrowRows * kOutStride <= kF32NarrowRows * kStride, "the output block fits the query buffer");
  float* const so = sQ;
  // (m runs over compile-time ranges in both branches: the accumulators stay
  // in registers)
  const auto give = [&](auto m0c) {
    constexpr int m0 = decltype(m0c)::value;
#pragma unroll
    for (int m = m0; m < m0 + kHalfM; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        *reinterpret_cast<float4*>(so + r_blk * kOutStride + 64 * m + 16 * lg + 4 * v) =
            make_float4(o[4 * m][v], o[4 * m + 1][v], o[4 * m + 2][v], o[4 * m + 3][v]);
  };
  if (kh == 0)
    give(std::integral_constant<int, kHalfM>{});  // the other half's columns
  else
    give(std::integral_constant<int, 0>{});
  if (lg == 0) {
    s_mh[kh][r_blk] = m_ref;
    s_lh[kh][r_blk] = l_tot;
  }
  __syncthreads();
  {
    // A half with no weight (no visible key, or every weight below fp32's
    // range against its reference) takes none.
    const float m0 = s_mh[0][r_blk], l0 = s_lh[0][r_blk], m1 = s_mh[1][r_blk], l1 = s_lh[1][r_blk];
    const bool has0 = l0 > 0.f, has1 = l1 > 0.f;
    const float M = has0 && has1 ? fmaxf(m0, m1) : (has1 ? m1 : m0);
    const float w0 = has0 ? exp2f(m0 - M) : 0.f;
    const float w1 = has1 ? exp2f(m1 - M) : 0.f;
    const float L = l0 * w0 + l1 * w1;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const float c0 = w0 * inv, c1 = w1 * inv;
    const float c_own = kh == 0 ? c0 : c1, c_oth = kh == 0 ? c1 : c0;
    // o0 c0 + o1 c1 (the first half's term first in both halves)
    const auto keep = [&](auto m0c, bool first) {
      constexpr int m0 = decltype(m0c)::value;
#pragma unroll
      for (int m = m0; m < m0 + kHalfM; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float4* at = reinterpret_cast<float4*>(so + r_blk * kOutStride + 64 * m + 16 * lg + 4 * v);
          const float4 h = *at;
          const float4 mine = make_float4(o[4 * m][v] * c_own, o[4 * m + 1][v] * c_own, o[4 * m + 2][v] * c_own,
                                          o[4 * m + 3][v] * c_own);
          const float4 oth = make_float4(h.x * c_oth, h.y * c_oth, h.z * c_oth, h.w * c_oth);
          *at = first ? make_float4(mine.x + oth.x, mine.y + oth.y, mine.z + oth.z, mine.w + oth.w)
                      : make_float4(oth.x + mine.x, oth.y + mine.y, oth.z + mine.z, oth.w + mine.w);
        }
    };
    if (kh == 0)
      keep(std::integral_constant<int, 0>{}, true);  // this half's columns
    else
      keep(std::integral_constant<int, kHalfM>{}, false);
    if (kh == 0 && row_valid && lg == 0) {
      if (w.slot < 0) {
        if (a.lse) a.lse[w.row0 + row] = (M + log2f(L)) * kLn2;
      } else {
        const int64_t srow = w.slot * kF32NarrowRows + r_blk;
        a.ws_m[srow] = M * kLn2;
        a.ws_l[srow] = L;
      }
    }
  }
  __syncthreads();
  const int rows = min(kF32NarrowRows, w.R - w.rb * kF32NarrowRows);
  float* const dst = w.slot < 0 ? a.out + (w.row0 + static_cast<int64_t>(w.rb) * kF32NarrowRows) * DC
                                : a.ws_o + w.slot * kF32NarrowRows * DC;
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

// The narrow form: a uniform batch, one unit per workgroup; a ragged batch, a
// persistent grid.
__global__ __launch_bounds__(kF32Threads, 1) void attn_mfma_f32_narrow_kernel(AttnArgs a) {
  attn_mfma_f32_narrow_unit(a, decode_unit(a, unit_of_block(a, blockIdx.x)));
}
__global__ __launch_bounds__(kF32Threads, 1) void attn_mfma_f32_narrow_ragged_kernel(AttnArgs) {
  for_each_ragged_unit([](const AttnArgs& a, const Unit& w) { attn_mfma_f32_narrow_unit(a, w); });
}

hipError_t launch_attn_mfma_f32(const AttnShape& s, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(plan.units));
  if (plan.kernel == AttnKernel::kMfmaF32Narrow) {
    if (a.req)
      attn_mfma_f32_narrow_ragged_kernel<<<grid, kF32Threads, 0, stream>>>(a);
    else
      attn_mfma_f32_narrow_kernel<<<grid, kF32Threads, 0, stream>>>(a);
  } else if (a.req)
    attn_mfma_f32_ragged_kernel<<<grid, kF32Threads, 0, stream>>>(a);
  else
    attn_mfma_f32_kernel<<<grid, kF32Threads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace tv
