// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;     // CDNA wavefront width
constexpr int kXcds = 8;      // MI355X: 8 accelerator complex dies, workgroups dealt round-robin
constexpr int kQBlock = 128;  // fp8 scale block along the reduction dimension

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 with round-to-nearest-even (NaN stays a quiet NaN): the compiler's
// __bf16 conversion, which gfx950 executes as one v_cvt_pk_bf16_f32 per pair of values.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// OCP e4m3fn encode of a float32 with round-to-nearest-even and saturation to
// +-448, written from the format definition (1 sign, 4 exponent bits with bias
// 7, 3 mantissa bits; exponent field 0 is subnormal with spacing 2^-9).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |v| >= 448 (and inf): saturate
  int e = static_cast<int>(a >> 23) - 127;    // unbiased float exponent
  if (e < -6) {
    // subnormal result: round |v| / 2^-9 to an integer 0..8 (8 == smallest normal)
    float q = rintf(__uint_as_float(a) * 512.0f);  // exact scaling by a power of two
    return sign | static_cast<uint32_t>(q);
  }
  // normal: keep 3 mantissa bits, round half to even on the dropped 20 bits
  uint32_t mant = a & 0x7fffffu;
  uint32_t keep = mant >> 20;
  uint32_t rest = mant & 0xfffffu;
  uint32_t r = (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ? 1u : 0u;
  uint32_t code = (static_cast<uint32_t>(e + 7) << 3) + keep + r;  // carry rolls into the exponent
  if (code > 0x7eu) code = 0x7eu;
  return sign | code;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xfu;
  uint32_t m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : static_cast<float>(m) * 0.001953125f;
  return __uint_as_float(__float_as_uint(v) | s);
}

// Wave-wide reductions over 64 lanes (butterfly through ds_swizzle-free shuffles).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace moe
