// Per-row NVFP4 quantization by one wave (shared by the standalone quantize
// kernel and the MoE forward's prologue).
#pragma once

#include "common.hpp"

namespace nvfp4 {

__device__ __forceinline__ void unpack16(const uint4& a, const uint4& b, float* f) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}

__device__ __forceinline__ float amax16_bf16(const uint4& a, const uint4& b) {
  // |x| of finite bf16 values orders like the integer (bits & 0x7FFF)
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m = max(m, w[i] & 0x7FFFu);
    m = max(m, (w[i] >> 16) & 0x7FFFu);
  }
  return __uint_as_float(m << 16);
}

// A row held in registers: lane l owns blocks l, l + 64, ... (NB of them).
template <int NB>
struct RowRegs {
  uint4 v[NB][2];
};

// Unconditional loads (block index clamped) so that they are all in flight
// together; blocks past the row end are masked out by the quantize step.
template <int NB>
__device__ __forceinline__ void load_row(RowRegs<NB>& rr, const uint16_t* __restrict__ xrow, int nblk,
                                         int lane) {
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int b = lane + kWave * i;
    const uint4* p = reinterpret_cast<const uint4*>(xrow + 16 * (b < nblk ? b : nblk - 1));
    rr.v[i][0] = load_stream16(p);
    rr.v[i][1] = load_stream16(p + 1);
  }
}

// The dequantized values of one quantized block (code x block scale; exact
// in fp16) as two 16-byte stores.
__device__ __forceinline__ void store_block_f16(_Float16* dst, uint32_t lo, uint32_t hi, uint32_t sb) {
  const half2v sc = e4m3_half2(sb);
  half8* d = reinterpret_cast<half8*>(dst);
  d[0] = dequant8_f16(lo, sc);
  d[1] = dequant8_f16(hi, sc);
}

// The fp16 copy of a row handed over already quantized: blocks b0, b0 + step,
// ... of codes crow / scales srow.
__device__ __forceinline__ void dequant_row_f16(const uint8_t* __restrict__ crow,
                                                const uint8_t* __restrict__ srow, int nblk,
                                                _Float16* __restrict__ x16row, int b0, int step) {
  for (int b = b0; b < nblk; b += step) {
    const uint2 c = *reinterpret_cast<const uint2*>(crow + 8 * b);
    store_block_f16(x16row + 16 * b, c.x, c.y, srow[b]);
  }
}

// Row amax -> g, then every block of the row; the block amaxes of the first
// pass are reused by the second.  gfix: NULL for the row's own global scale
// 2688 / amax, else a given one.
template <int NB>
__device__ __forceinline__ void quantize_row_regs(const RowRegs<NB>& rr, int nblk, uint8_t* __restrict__ crow,
                                                  uint8_t* __restrict__ srow, float* __restrict__ gout,
                                                  int lane, _Float16* __restrict__ x16row = nullptr,
                                                  const float* gfix = nullptr) {
  float bam[NB];
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    bam[i] = amax16_bf16(rr.v[i][0], rr.v[i][1]);
    if (lane + kWave * i < nblk) am = fmaxf(am, bam[i]);
  }
  const float g = gfix ? *gfix : global_scale(wave_max(am));
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int b = lane + kWave * i;
    if (b < nblk) {
      float f[16];
      unpack16(rr.v[i][0], rr.v[i][1], f);
      uint32_t lo, hi;
      const uint32_t sb = quantize_block16_amax(f, bam[i], g, lo, hi);
      *reinterpret_cast<uint2*>(crow + 8 * b) = make_uint2(lo, hi);
      srow[b] = static_cast<uint8_t>(sb);
      if (x16row) store_block_f16(x16row + 16 * b, lo, hi, sb);
    }
  }
  if (lane == 0) *gout = g;
}

template <int NB>
__device__ __forceinline__ void quantize_row_wave(const uint16_t* __restrict__ xrow, int nblk,
                                  uint8_t* __restrict__ crow, uint8_t* __restrict__ srow,
                                  float* __restrict__ gout, int lane, _Float16* __restrict__ x16row = nullptr,
                                  const float* gfix = nullptr) {
  if constexpr (NB > 0) {
    RowRegs<NB> rr;
    load_row<NB>(rr, xrow, nblk, lane);
    quantize_row_regs<NB>(rr, nblk, crow, srow, gout, lane, x16row, gfix);
  } else {
    // Rows too long for the register cache: amax pass, then quantize pass.
    float am = 0.0f;
    for (int b = lane; b < nblk; b += kWave) {
      const uint4* p = reinterpret_cast<const uint4*>(xrow + 16 * b);
      am = fmaxf(am, amax16_bf16(p[0], p[1]));
    }
    const float g = gfix ? *gfix : global_scale(wave_max(am));
    for (int b = lane; b < nblk; b += kWave) {
      const uint4* p = reinterpret_cast<const uint4*>(xrow + 16 * b);
      float f[16];
      unpack16(p[0], p[1], f);
      uint32_t lo, hi;
      const uint32_t sb = quantize_block16(f, g, lo, hi);
      *reinterpret_cast<uint2*>(crow + 8 * b) = make_uint2(lo, hi);
      srow[b] = static_cast<uint8_t>(sb);
      if (x16row) store_block_f16(x16row + 16 * b, lo, hi, sb);
    }
    if (lane == 0) *gout = g;
  }
}

}  // namespace nvfp4
