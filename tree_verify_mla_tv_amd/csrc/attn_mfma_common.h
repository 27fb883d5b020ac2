// Pieces shared by the two bf16-cache matrix-core kernels (attn_mfma.hip:
// bf16 queries, 128 rows per workgroup; attn_mfma_q2.hip: queries as two bf16
// terms, 64 rows per workgroup): tile geometry in LDS, the HBM -> LDS copy of
// a kv tile, and the softmax row state.
#pragma once

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

// Copy kv rows [kt, kt + 32) of one tree into a tile buffer.  Rows past k_end
// repeat row k_end - 1 (finite data; their scores are masked).
//   latent rows:  row k at buf + k * kLatRowBytes, 64 chunks of 16 B; wave w
//                 copies rows 8w .. 8w+7, one wave-wide 1 KB copy per row.
//   rope rows:    wave w copies keys 8w .. 8w+7 into buf + kLatBytes + 1024 w,
//                 chunk-major: 16-byte chunk c of key k at slot c * 8 + (k % 8).
// Buffer loads straight to LDS (buffer_load_dwordx4 ... lds, TV_STAGE_ASM): the
// tree's base is in a raw buffer descriptor, the row in a scalar offset, and
// each lane adds its 16-byte chunk.  Nine loads per wave; the caller waits for
// them (vmcnt) before the barrier that publishes the tile.  Inside the sweep
// the same loads are woven into the score chain (TV_STEP_ASM).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

struct TreeKv {
  u32x4_t lat;      // raw buffer over the tree's c_kv rows (1024 B each)
  u32x4_t rope;     // raw buffer over the tree's k_rope rows (128 B each)
  uint32_t lane16;  // 16 * lane: the lane's chunk of a latent row
  int kmax;         // last key of the unit's kv range
};

// Raw (untyped) buffer descriptor: base address, stride 0, size in bytes, and
// dword 3 as for any untyped gfx9 buffer.
__device__ __forceinline__ u32x4_t raw_buffer(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return u32x4_t{static_cast<uint32_t>(p), static_cast<uint32_t>(p >> 32) & 0xffffu, bytes, 0x00020000u};
}

// Per-tile arguments of a copy into buf of the tile starting at key kt.
struct StageArgs {
  uint32_t mb;  // LDS address of the wave's first latent row
  uint32_t mr;  // LDS address of the wave's rope rows
  int kb;       // first key of the wave's rows
  uint32_t ro;  // the lane's rope byte offset in the buffer
};

__device__ __forceinline__ StageArgs stage_args(const unsigned char* buf, const TreeKv& kv, int kt, int wave,
                                                int lane) {
  StageArgs sa;
  sa.mb = lds_addr(buf) + wave * 8 * mf::kLatRowBytes;
  sa.mr = lds_addr(buf) + mf::kLatBytes + wave * 1024;
  sa.kb = kt + wave * 8;
  sa.ro = static_cast<uint32_t>(min(sa.kb + (lane & 7), kv.kmax)) * (mf::DR * 2) + (lane >> 3) * 16;
  return sa;
}

__device__ __forceinline__ void stage_tile(const unsigned char* buf, const TreeKv& kv, int kt, int wave, int lane) {
  const StageArgs sa = stage_args(buf, kv, kt, wave, lane);
  const uint32_t mb = __builtin_amdgcn_readfirstlane(sa.mb);
  const uint32_t mr = __builtin_amdgcn_readfirstlane(sa.mr);
  const int kb = __builtin_amdgcn_readfirstlane(sa.kb);
  const int km = __builtin_amdgcn_readfirstlane(kv.kmax);
  uint32_t t, ms;
  asm volatile(TV_STAGE_ASM
               : [t] "=&s"(t), [ms] "=&s"(ms)
               : [mb] "s"(mb), [mr] "s"(mr), [kb] "s"(kb), [km] "s"(km), [l16] "v"(kv.lane16),
                 [ro] "v"(sa.ro), [rl] "s"(kv.lat), [rr] "s"(kv.rope)
               : "memory");
}

// Per-lane row state of the softmax (rows of the wave's own row block).
struct RowState {
  float m_ref;   // reference max (log2 units) the exponentials are taken against
  float m_seen;  // exact running max of the row's visible scores (log2 units)
  float l;       // this lane's share of the row's softmax denominator
  float exc;     // largest (tile max - m_ref) seen; above kHeadroom means overflow risk
};

// Lanes l and l + 32 hold the same row: swap the wave's halves and add.
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffers of one step: scores of the tile in kc (keys from kt), values of the
// tile in kp with the weights pp, this tile's weights to pc, and the copy of
// the tile after kc into kn.
struct StepBufs {
  const unsigned char* kc;
  const unsigned char* kp;
  const unsigned char* kn;
  const unsigned char* pp;
  unsigned char* pc;
};

}  // namespace tv
