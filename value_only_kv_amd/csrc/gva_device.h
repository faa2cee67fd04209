// gva_device.h - device helpers shared by the GVA kernels (gfx950, wave64).
#ifndef GVA_DEVICE_H_
#define GVA_DEVICE_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gva_internal.h"

namespace gvad {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One round-to-nearest-even from float64 to a binary format with float32's exponent range
// (8 exponent bits, bias 127) and M stored mantissa bits: M = 7 gives bfloat16, M = 23 gives
// float32. Done on the float64 bit pattern with integer arithmetic, so the result does not
// depend on the hardware's rounding or denormal modes. Subnormal results are produced
// exactly; float64 subnormals round to a signed zero.
template <int M>
__device__ __forceinline__ uint32_t round_f64_rne(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t sign = static_cast<uint32_t>(u >> 63) << (M + 8);
  const uint64_t mag = u & 0x7fffffffffffffffull;
  const uint32_t inf = 0xFFu << M;
  if (mag >= 0x7ff0000000000000ull)
    return mag == 0x7ff0000000000000ull ? (sign | inf) : (sign | inf | (1u << (M - 1)));
  const int ebits = static_cast<int>(mag >> 52);
  if (ebits == 0) return sign;
  const int e = ebits - 1023;                                   // |x| in [2^e, 2^(e+1))
  const uint64_t sig = (mag & 0xfffffffffffffull) | (1ull << 52);  // x = sig * 2^(e - 52)
  const int sh = (e >= -126) ? (52 - M) : (52 - M + (-126 - e));  // bits dropped from sig
  if (sh > 53) return sign;                                     // below half the least quantum
  uint64_t r = sig >> sh;
  const uint64_t rem = sig & ((1ull << sh) - 1);
  const uint64_t half = 1ull << (sh - 1);
  if (rem > half || (rem == half && (r & 1ull))) ++r;
  if (e >= -126) {
    // r in [2^M, 2^(M+1)]; a carry to 2^(M+1) lands in the exponent field by the addition.
    const uint64_t out = (static_cast<uint64_t>(e + 127) << M) + (r - (1ull << M));
    if ((out >> M) >= 0xFF) return sign | inf;
    return sign | static_cast<uint32_t>(out);
  }
  return sign | static_cast<uint32_t>(r);  // subnormal; r == 2^M is the least normal
}

__device__ __forceinline__ uint16_t f64_to_bf16_bits(double x) {
  return static_cast<uint16_t>(round_f64_rne<7>(x));
}
__device__ __forceinline__ uint32_t f64_to_f32_bits(double x) { return round_f64_rne<23>(x); }
__device__ __forceinline__ float f64_to_f32(double x) { return __uint_as_float(f64_to_f32_bits(x)); }
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Rotate one interleaved pair by the angle whose (cos, sin) is (c, s), in float64 with each
// product and each sum rounded on its own (no fused multiply-add).
__device__ __forceinline__ void rotate_pair_f64(double x0, double x1, double c, double s,
                                                double *y0, double *y1) {
#pragma clang fp contract(off)
  const double a = x0 * c;
  const double b = x1 * s;
  *y0 = a - b;
  const double e = x0 * s;
  const double f = x1 * c;
  *y1 = e + f;
}

// Exchanges across rows of 16 lanes with the gfx950 row-swap instructions (checked on the
// hardware): v_permlane16_swap returns, in every lane, its own value and that of lane ^ 16 (in
// some order); v_permlane32_swap the same for lane ^ 32. They stay in the vector ALU, where a
// cross-lane shuffle would take a round trip through the LDS unit.
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ void raise_err(int32_t *flag, int32_t bits) {
  if (flag) atomicOr(flag, bits);
}

// Physical block of position p of sequence b, or -1 (with the error bit raised) when the
// table entry is outside the pool.
__device__ __forceinline__ int64_t block_of(const gva::DecodeArgs &a, int b, int p) {
  const int32_t blk = a.block_table[static_cast<int64_t>(b) * a.max_blocks + (p >> a.log2_bs)];
  if (blk < 0 || static_cast<int64_t>(blk) >= a.num_blocks) return -1;
  return blk;
}

}  // namespace gvad

#endif  // GVA_DEVICE_H_
