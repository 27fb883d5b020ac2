// Device-side helpers shared by the libtv kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tv {

constexpr int kWave = 64;  // CDNA wavefront width

// ---------------------------------------------------------------------------
// Storage types.  bf16 is carried as raw uint16 bit patterns.
// ---------------------------------------------------------------------------
struct F32 {
  using storage = float;
  static constexpr int bytes = 4;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Low / high bf16 of a packed pair, widened to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Round-to-nearest-even from float64 straight to bf16 (one rounding; finite,
// normal-range inputs).  The rounding is done on the double's 52-bit mantissa
// (keep 7 bits, ties to even); the rounded double is then exact in fp32 and its
// top 16 bits are the bf16 pattern.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint64_t lsb = (u >> 45) & 1ull;
  u += 0x00000FFFFFFFFFFFull + lsb;  // (1 << 44) - 1 + lsb
  u &= ~0x00001FFFFFFFFFFFull;       // clear the 45 dropped bits
  const float f = static_cast<float>(__longlong_as_double(static_cast<long long>(u)));
  return static_cast<uint16_t>(__float_as_uint(f) >> 16);
}

template <typename T>
__device__ __forceinline__ double load_f64(const typename T::storage* p);
template <>
__device__ __forceinline__ double load_f64<F32>(const float* p) {
  return static_cast<double>(*p);
}
template <>
__device__ __forceinline__ double load_f64<BF16>(const uint16_t* p) {
  return static_cast<double>(bf16_bits_to_f32(*p));
}

template <typename T>
__device__ __forceinline__ void store_from_f64(typename T::storage* p, double v);
template <>
__device__ __forceinline__ void store_from_f64<F32>(float* p, double v) {
  *p = static_cast<float>(v);  // one RNE rounding
}
template <>
__device__ __forceinline__ void store_from_f64<BF16>(uint16_t* p, double v) {
  *p = f64_to_bf16_rne(v);
}

// ---------------------------------------------------------------------------
// Tree helpers
// ---------------------------------------------------------------------------
// A parent outside [0, i) (or any parent of the root) is read as "no parent".
__device__ __forceinline__ int clamp_parent(int p, int i) { return (p >= 0 && p < i) ? p : -1; }

}  // namespace tv
