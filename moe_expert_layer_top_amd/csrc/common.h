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

// silu(g) = g / (1 + e^-g) for results rounded to bf16 or fp8 next: the hardware
// exponential and reciprocal (v_exp_f32, v_rcp_f32, about 1 ulp each) instead of the
// correctly rounded division sequence; the error stays far below the 8-bit mantissa.
__device__ __forceinline__ float silu_fast(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// OCP e4m3fn encode (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent
// field 0 subnormal with spacing 2^-9) with round-to-nearest-even and saturation to +-448,
// of four floats packed as bytes 0 .. 3: gfx950's v_cvt_pk_fp8_f32, two values per
// instruction, on the values clamped to +-448 first.  On every non-NaN float32 it gives
// the same code as the encode written out from the format definition (rounding the 20
// dropped mantissa bits half to even, subnormals as round(|v| / 2^-9), |v| >= 448 to
// 0x7e); a NaN input gives +-448.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  const float ca = fminf(fmaxf(a, -448.0f), 448.0f), cb = fminf(fmaxf(b, -448.0f), 448.0f);
  const float cc = fminf(fmaxf(c, -448.0f), 448.0f), cd = fminf(fmaxf(d, -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);   // bytes 0, 1
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cc, cd, w, true);         // bytes 2, 3
  return static_cast<uint32_t>(w);
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
