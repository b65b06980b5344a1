// Device helpers shared by the NVFP4 MoE kernels (gfx950, wave64).
//
// Number formats: E2M1 codes (OCP MX v1.0 FP4), E4M3 block scales (OFP8
// "e4m3fn", max 448, no infinities), binary32 global scales.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// 16-byte load that does not need to stay in the caches (streamed once).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// Materializes v in a register at this point.  Loads that feed it are then
// issued before any later branch instead of being sunk into the branches that
// use them (which serializes one memory round trip per branch).
template <typename T>
__device__ __forceinline__ void keep_issued(T& v) { asm volatile("" : "+v"(v)); }

constexpr int kBlock = 16;            // elements per E4M3 block scale
constexpr float kGlobalNum = 2688.0f;  // 448 (E4M3 max) * 6 (E2M1 max)

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Global scale from an absolute maximum: 2688 / a, 1 for a == 0, +inf
// clamped to FLT_MAX.  IEEE division (correctly rounded by default in HIP).
__device__ __forceinline__ float global_scale(float a) {
  if (!(a > 0.0f)) return 1.0f;
  float g = kGlobalNum / a;
  return __builtin_isinf(g) ? 3.402823466e38f : g;
}

// E4M3 encode, round to nearest even, saturating at 448 (0x7E); s >= 0 finite.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  if (s >= 448.0f) return 0x7Eu;
  if (s < 0.015625f) {                   // below 2^-6: subnormal codes, quantum 2^-9
    return static_cast<uint32_t>(__builtin_rintf(s * 512.0f));  // 0..8 (8 == 2^-6)
  }
  uint32_t u = __float_as_uint(s);
  uint32_t e = (u >> 23) - 120u;         // biased E4M3 exponent: (u>>23) - 127 + 7
  uint32_t m = u & 0x7FFFFFu;
  uint32_t keep = m >> 20, rem = m & 0xFFFFFu;
  uint32_t up = (rem > 0x80000u) | ((rem == 0x80000u) & keep);
  uint32_t code = (e << 3) + keep + up;  // mantissa carry bumps the exponent
  return code > 0x7Eu ? 0x7Eu : code;
}

// E4M3 bits -> binary32 value (exact).
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  if (e == 0) return static_cast<float>(m) * 0.001953125f;   // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Eight binary32 values (already multiplied by the block's r) -> eight E2M1
// codes packed into a dword, element 0 in the low nibble.  The gfx950
// converter with scale 1.0 rounds to nearest even, saturates at +-6 and keeps
// the sign of zero (checked against the CPU encoder on the device).
__device__ __forceinline__ uint32_t e2m1_pack8(const float* v) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[0], v[1], 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], 1.0f, 3);
  return r;
}

// Eight packed E2M1 codes times one E4M3 scale value -> eight fp16 values.
// The products need at most 6 significant bits and lie in [2^-10, 2688], so
// fp16 holds them exactly.  The converter applies only a power-of-two scale,
// so the scale goes through a packed fp16 multiply instead.
__device__ __forceinline__ half8 dequant8_f16(uint32_t codes, half2v scale2) {
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * scale2;
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * scale2;
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * scale2;
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * scale2;
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ half2v e4m3_half2(uint32_t b) {
  _Float16 h = static_cast<_Float16>(e4m3_value(b));  // exact: E4M3 values are fp16 values
  half2v r;
  r[0] = h;
  r[1] = h;
  return r;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Quantize one 16-element block held as binary32 values with global scale g.
// Returns the E4M3 scale byte; writes the 8 code bytes as two dwords.
// The operation order is the recipe's: s = RN(RN(amax*g)/6), r = RN(g/d)
// (saturated to FLT_MAX), code = E2M1(RN(x*r)); no contraction is possible
// (no additions).
__device__ __forceinline__ uint32_t quantize_block16(const float* x, float g, uint32_t& lo,
                                                     uint32_t& hi) {
  float ab = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(x[i]));
  float t = ab * g;
  float s = t / 6.0f;
  uint32_t sb = e4m3_encode(s);
  float d = e4m3_value(sb);
  float r = d > 0.0f ? g / d : 0.0f;
  if (__builtin_isinf(r)) r = 3.402823466e38f;  // g clamped to FLT_MAX: keep r finite
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = x[i] * r;
  lo = e2m1_pack8(v);
  hi = e2m1_pack8(v + 8);
  return sb;
}

}  // namespace nvfp4
