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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// E4M3 encode, round to nearest even, saturating at 448 (0x7E), for s >= 0.
// gfx950's converter produces the OCP E4M3 byte directly; on [0, 464) it
// rounds to nearest even with values in [448, 464) going to 448, the same
// bytes as the software definition (every fp32 value of the interval was
// compared on the device).  Per-row global scales keep the block scales
// below 448 * (1 + 2^-22) (t = RN(amax_b * g) <= 2688 (1 + 2^-24)^2 since
// amax_b <= amax_row); a static global scale can push them anywhere up to
// +inf, which the clamp to 448 saturates (448 encodes as 0x7E either way).
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(fminf(s, 448.0f), 0.0f, 0, false)) & 0xFFu;
}

// E4M3 bits -> binary32 value (exact; b <= 0x7E or its negative).
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(b), 0);
}

// RN(t / 6) for t >= 0.  q0 = RN(t * RN(1/6)) is within an ulp, the residual
// t - 6 q0 is exact with an FMA, and one FMA correction rounds correctly
// (Markstein's theorem for a correctly rounded reciprocal).  Checked against
// the binary64 quotient on every non-negative float: equal for t >= 2^-125;
// below, both results are under 2^-120 and encode to the same E4M3 zero.
__device__ __forceinline__ float div6_rn(float t) {
  const float c = 0.16666667163372039794921875f;  // RN(1/6)
  const float q0 = t * c;
  return __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, t), c, q0);
}

// RN(g / d) for an E4M3 value d > 0 and g >= 2^-117 (every global scale
// 2688 / amax is, for finite amax), +inf saturated to FLT_MAX.  y = RN(1/d)
// comes from the hardware reciprocal plus one Newton step (exact for all 126
// E4M3 values, compared on the device); the quotient then takes the same
// FMA correction as div6_rn.  Compared with the binary64 quotient for every
// E4M3 divisor over the binades of g from 2^-117 up (no mismatch; the
// mismatches below come from subnormal quotients, which cannot occur here).
__device__ __forceinline__ float div_e4m3_rn(float g, float d) {
  float y = __builtin_amdgcn_rcpf(d);
  y = __builtin_fmaf(__builtin_fmaf(-d, y, 1.0f), y, y);
  const float q0 = g * y;
  const float q = __builtin_fmaf(__builtin_fmaf(-q0, d, g), y, q0);
  return __builtin_isinf(q0) ? 3.402823466e38f : __builtin_fminf(q, 3.402823466e38f);
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
  const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * scale2;
  const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * scale2;
  const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * scale2;
  const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * scale2;
  typedef _Float16 half4 __attribute__((ext_vector_type(4)));
  const half4 lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const half4 hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// bf16 operands (W4A16).  E4M3 scale byte -> binary32, exactly: the byte
// shifted to bits 20.. is the binary32 with the same exponent field (bias
// 127 instead of 7) and fraction, i.e. the value times 2^-120; scaling by
// 2^120 is exact (subnormal E4M3 values included).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __uint_as_float((b & 0xffu) << 20) * 0x1p120f;
}
// 8 E2M1 codes times their block scale as bf16: code (exact in binary32)
// times the scale is exact in binary32 (at most 6 significant bits), hence
// also in bf16 (8 significant bits), so the rounding conversion is exact.
__device__ __forceinline__ bf16x8 dequant8_bf16(uint32_t codes, float scale) {
  const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  bf16x8 r;
  r[0] = static_cast<__bf16>(v0[0] * scale);
  r[1] = static_cast<__bf16>(v0[1] * scale);
  r[2] = static_cast<__bf16>(v1[0] * scale);
  r[3] = static_cast<__bf16>(v1[1] * scale);
  r[4] = static_cast<__bf16>(v2[0] * scale);
  r[5] = static_cast<__bf16>(v2[1] * scale);
  r[6] = static_cast<__bf16>(v3[0] * scale);
  r[7] = static_cast<__bf16>(v3[1] * scale);
  return r;
}

__device__ __forceinline__ half2v e4m3_half2(uint32_t b) {
  _Float16 h = static_cast<_Float16>(e4m3_value(b));  // exact: E4M3 values are fp16 values
  half2v r;
  r[0] = h;
  r[1] = h;
  return r;
}

// Cross-lane exchanges of a wave in the vector ALU (no LDS round trip):
// DPP within each row of 16 lanes, then v_permlane16_swap (rows 0 <-> 1,
// 2 <-> 3) and v_permlane32_swap (lower <-> upper half).  DPP controls:
// quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror (lane i <-> 7 - i of
// each 8), row_mirror (lane i <-> 15 - i), row_ror 4 and 8.  Callers run
// them with every lane of the wave active.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140,
              kDppRor4 = 0x124, kDppRor8 = 0x128;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, CTRL, 0xF, 0xF, false);
}
// A value swapped with itself across a row pair (PAIR = 16) or the two
// halves (PAIR = 32): each lane gets its own value in one result and its
// partner's (lane ^ PAIR) in the other, so a commutative combination of the
// two reduces over the pair whichever way round they come.
template <int PAIR>
__device__ __forceinline__ void lane_pair(uint32_t v, uint32_t& a, uint32_t& b) {
  if constexpr (PAIR == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  } else {
    static_assert(PAIR == 32, "row pairs or halves");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  }
}

// Maximum over the wave (exact, the same in every lane).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(v))));
  uint32_t a, b;
  lane_pair<16>(__float_as_uint(v), a, b);
  v = fmaxf(__uint_as_float(a), __uint_as_float(b));
  lane_pair<32>(__float_as_uint(v), a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}

// Quantize one 16-element block held as binary32 values with global scale g,
// given the block's amax.  Returns the E4M3 scale byte; writes the 8 code
// bytes as two dwords.  The operation order is the recipe's: s =
// RN(RN(amax*g)/6), r = RN(g/d) (saturated to FLT_MAX), code = E2M1(RN(x*r));
// the divisions use the correctly rounded forms above.
__device__ __forceinline__ uint32_t quantize_block16_amax(const float* x, float ab, float g,
                                                          uint32_t& lo, uint32_t& hi) {
  const float t = ab * g;
  const uint32_t sb = e4m3_encode(div6_rn(t));
  const float d = e4m3_value(sb);
  const float r = d > 0.0f ? div_e4m3_rn(g, d) : 0.0f;
  // |x r| <= 6.375 with a per-row global scale; with a static one the
  // product can be anything up to +-inf, so it is clamped to the E2M1 range
  // first (the saturating encoder maps every |v| >= 5 to 6, so the clamp
  // changes no code)
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_fmed3f(x[i] * r, -6.0f, 6.0f);
  lo = e2m1_pack8(v);
  hi = e2m1_pack8(v + 8);
  return sb;
}

__device__ __forceinline__ uint32_t quantize_block16(const float* x, float g, uint32_t& lo,
                                                     uint32_t& hi) {
  float ab = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(x[i]));
  return quantize_block16_amax(x, ab, g, lo, hi);
}

}  // namespace nvfp4
