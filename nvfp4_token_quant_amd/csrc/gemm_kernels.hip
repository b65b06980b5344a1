// Grouped expert GEMMs of the NVFP4 MoE layer on gfx950.
//
// GEMM1 (gate+up) with the SwiGLU activation and, once every column band of a
// tile is done, the per-row re-quantization of the activation; GEMM2 (down)
// on the re-quantized rows.  [P3] (sglang PR #36624 summary), "Feature and
// motivation": the expert GEMM with activation and finalize around it; [P1]
// (sglang PR #28354 summary), "Implementation breakdown" items 2-3: NVFP4
// w13 / w2 weights with block scales and per-expert alphas.
//
// MFMA operand choice.  NVFP4 scales are E4M3 per 16 elements; gfx950's
// scaled FP4 MFMA takes power-of-two (E8M0) scales per 32 elements, so it
// cannot carry them.  Each E2M1 code times its E4M3 block scale is formed
// exactly in fp16 (<= 6 significant bits, magnitudes in [2^-10, 2688]) and fed
// to v_mfma_f32_16x16x32_f16 with fp32 accumulation; the binary32 global
// scales (per token / per expanded row, per expert) are applied once in the
// epilogue.
//
// Operand roles: weight rows are MFMA operand A (16 output columns x 32 k per
// fragment), token rows operand B (32 k x 16 rows).  Per 128-wide K step a
// lane holds 16 bytes (32 codes) of one weight row; the four MFMAs of the step
// use its 8-code pieces q = 0..3, and the token operand uses the same k
// assignment (lane group g holds k = 32g + 8q + i), so every k is summed once.
#include "common.hpp"
#include "kernels.hpp"

namespace nvfp4 {

// E4M3 byte -> the same value as two packed fp16.  The E4M3 bit pattern
// shifted left by 7 is an fp16 pattern worth value * 2^-8 (exponent bias 15
// instead of 7, also for E4M3 subnormals, which land on fp16 subnormals), so
// one packed multiply by 256 restores the value exactly.
__device__ __forceinline__ half2v e4m3_to_half2(uint32_t b) {
  const uint32_t bits = (b & 0xFFu) * 0x00800080u;  // (b << 7) | (b << 23)
  half2v h;
  __builtin_memcpy(&h, &bits, 4);
  const half2v k256 = {256.0f16, 256.0f16};
  return h * k256;
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// Epilogues.
// ---------------------------------------------------------------------------

// GEMM1: per lane, fragment pair (gate fh, up fh) holds h[n = c0 + 16 fh + 4g + i]
// for row m = 16 fm + r16.  act = silu(h_gate) * h_up in fp32, stored with the
// band's per-row amax.
template <int FM, int FNH>
__device__ __forceinline__ void g1_epilogue(const FwdParams& p, const f32x4 (&acc)[2 * FNH][FM],
                                            int e, int row0, int nrows, int c0,
                                            const float* s_ginv, float (*s_amax)[16 * FM], int wave,
                                            int g, int r16) {
  const float wginv = 1.0f / p.w13g[e];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = fm * 16 + r16;
    const float alpha = s_ginv[m] * wginv;
    float am = 0.0f;
#pragma unroll
    for (int fh = 0; fh < FNH; ++fh) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float hg = acc[fh][fm][i] * alpha;
        const float hu = acc[FNH + fh][fm][i] * alpha;
        a[i] = hg / (1.0f + __expf(-hg)) * hu;
        am = fmaxf(am, fabsf(a[i]));
      }
      if (m < nrows) {
        const int n = c0 + fh * 16 + 4 * g;
        *reinterpret_cast<float4*>(p.act + static_cast<int64_t>(row0 + m) * p.I + n) =
            make_float4(a[0], a[1], a[2], a[3]);
      }
    }
    am = fmaxf(am, __shfl_xor(am, 16, kWave));
    am = fmaxf(am, __shfl_xor(am, 32, kWave));
    if (g == 0) s_amax[wave][m] = am;
  }
}

// The band's per-row amax of act (one partial per GEMM1 column band; GEMM2's
// staging or the re-quantization kernel reduces them).
template <int MT>
__device__ __forceinline__ void g1_store_band_amax(const FwdParams& p, float (*s_amax)[MT], int row0,
                                                   int nrows) {
  __syncthreads();
  if (threadIdx.x < MT && static_cast<int>(threadIdx.x) < nrows) {
    const int m = threadIdx.x;
    const float v = fmaxf(fmaxf(s_amax[0][m], s_amax[1][m]), fmaxf(s_amax[2][m], s_amax[3][m]));
    p.act_amax[static_cast<int64_t>(row0 + m) * gridDim.y + blockIdx.y] = v;
  }
}

// Re-quantize 16 consecutive act values of one expanded row with its g2 (same
// recipe as the token quantizer, on binary32 input).
__device__ __forceinline__ uint32_t requant_block(const float* __restrict__ src, float g2,
                                                  uint32_t& lo, uint32_t& hi) {
  const float4* s4 = reinterpret_cast<const float4*>(src);
  float f[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = s4[q];
    f[4 * q] = v.x; f[4 * q + 1] = v.y; f[4 * q + 2] = v.z; f[4 * q + 3] = v.w;
  }
  return quantize_block16(f, g2, lo, hi);
}

// GEMM2: per lane, fragment f holds y[n = n0 + 16 f + 4g + i] of row m.
template <int FM, int FN>
__device__ __forceinline__ void g2_epilogue(const FwdParams& p, const f32x4 (&acc)[FN][FM], int e,
                                            int row0, int nrows, int n0, const float* s_ginv,
                                            const int* s_slot, int g, int r16) {
  const float wginv = 1.0f / p.w2g[e];
  const int H = p.H;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = fm * 16 + r16;
    if (m >= nrows) continue;
    const float alpha = s_ginv[m] * wginv;
    const int64_t row = row0 + m;
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int n = n0 + f * 16 + 4 * g;
      const float y0 = acc[f][fm][0] * alpha, y1 = acc[f][fm][1] * alpha;
      const float y2 = acc[f][fm][2] * alpha, y3 = acc[f][fm][3] * alpha;
      if (p.deterministic) {
        *reinterpret_cast<float4*>(p.y + row * H + n) = make_float4(y0, y1, y2, y3);
      } else {
        const int slot = s_slot[m];
        const float w = p.topk_w[slot];
        float* dst = p.out_acc + static_cast<int64_t>(slot / p.k) * H + n;
        atomicAdd(dst + 0, w * y0);
        atomicAdd(dst + 1, w * y1);
        atomicAdd(dst + 2, w * y2);
        atomicAdd(dst + 3, w * y3);
      }
    }
  }
}

// Rows of the token operand for local row m of a tile: GEMM1 reads the
// per-token quantized activations of token perm[row] / k, GEMM2 the
// re-quantized activation of the expanded row itself.
template <int MODE>
__device__ __forceinline__ void tile_rows(const FwdParams& p, int row0, int nrows, int mt,
                                          int* s_src, float* s_ginv, int* s_slot) {
  if (static_cast<int>(threadIdx.x) < mt) {
    const int m = threadIdx.x;
    int src = -1, slot = -1;
    float gi = 0.0f;
    if (m < nrows) {
      slot = p.perm[row0 + m];
      src = MODE == 0 ? slot / p.k : row0 + m;
      gi = 1.0f / (MODE == 0 ? p.xq_g[src] : p.a2_g[src]);
    }
    s_src[m] = src;
    s_ginv[m] = gi;
    if (s_slot) s_slot[m] = slot;
  }
}

// ---------------------------------------------------------------------------
// Stream kernel (few rows per expert: decode).  One block = one tile of up to
// 16*FM rows x a band of 64*FN weight rows (4 waves x FN fragments of 16).
// The tile's token operand is staged once in LDS as FP4 codes + E4M3 scales
// (dynamic LDS: MT rows x (K/2 + 16) code bytes and (K/16 + 4) scale bytes);
// each wave then walks K in 128-wide steps with the code pieces of the next
// kStreamDepth steps in flight, and fetches the weight scales of 8 steps with
// one 16-byte load (the GEMM scale layout keeps them contiguous).  Every load
// of the loop is unconditional (steps past the end re-read the last one) and
// issued in consumption order, so the waits only cover the oldest step.
// MODE 0: GEMM1 (weights W13, FN/2 gate + FN/2 up fragments, SwiGLU);
// MODE 1: GEMM2 (weights W2, FN output fragments).
// ---------------------------------------------------------------------------
constexpr int kStreamDepth = 8;

// Copy `bytes` bytes from global memory to LDS with global_load_lds: one wave
// instruction moves 64 x W bytes (lane l moves bytes [W l, W l + W) of the
// chunk) to consecutive LDS addresses.  bytes % W == 0; dst 16-byte aligned.
template <int W>
__device__ __forceinline__ void copy_rows_to_lds(const uint8_t* src, uint8_t* dst, int bytes,
                                                 int lane) {
  for (int c = 0; c < bytes; c += 64 * W) {
    if (c + W * lane < bytes) {
      auto* d = (__attribute__((address_space(3))) void*)(dst + c);
      if constexpr (W == 16)
        __builtin_amdgcn_global_load_lds(src + c + W * lane, d, 16, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(src + c + W * lane, d, 4, 0, 0);
    }
  }
}

template <int FM, int FN, int MODE>
__global__ __launch_bounds__(256) void moe_stream_kernel(FwdParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int MT = 16 * FM;
  constexpr int FNH = FN / 2;
  __shared__ int s_src[MT];
  __shared__ int s_slot[MT];
  __shared__ float s_ginv[MT];
  __shared__ float s_aux[4][MT];
  if (static_cast<int>(blockIdx.x) >= *p.n_tiles) return;
  const int4 td = p.tiles[blockIdx.x];
  const int e = td.x, row0 = td.y, nrows = td.z;
  const int K = MODE == 0 ? p.H : p.I;
  const int cpitch = K / 2 + 16, spitch = K / 16 + 4;
  uint8_t* lc = smem;
  uint8_t* ls = smem + MT * cpitch;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4, r16 = lane & 15;

  // this wave's weight rows
  // fragment f = 16 weight rows = one 16-row group of the fragment-major copy
  const int S = ksteps(K), Q = sgroups(K);
  const uint8_t* cptr[FN];
  const uint8_t* sptr[FN];
  int cbase;
  if (MODE == 0) {
    cbase = blockIdx.y * (64 * FNH) + wave * 16 * FNH;
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int64_t n = f < FNH ? cbase + f * 16 : p.I + cbase + (f - FNH) * 16;
      const int64_t grp = (static_cast<int64_t>(e) * 2 * p.I + n) / 16;
      cptr[f] = p.w13c + grp * S * 1024 + 16 * lane;
      sptr[f] = p.w13s + grp * Q * 1024 + 16 * lane;
    }
  } else {
    cbase = blockIdx.y * (64 * FN) + wave * 16 * FN;
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int64_t grp = (static_cast<int64_t>(e) * p.H + cbase + f * 16) / 16;
      cptr[f] = p.w2c + grp * S * 1024 + 16 * lane;
      sptr[f] = p.w2s + grp * Q * 1024 + 16 * lane;
    }
  }
  const int nsteps = S;
  const int last = nsteps - 1;
  // Loads past the last step go to a 1 KB always-cached dummy block instead
  // (keeps every load unconditional without re-reading weights).
  const uint8_t* dummy = p.dummy + 16 * lane;
  // weights first, so that they are in flight while the token operand stages
  uint4 wsc_cur[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) wsc_cur[f] = *reinterpret_cast<const uint4*>(sptr[f]);
  uint4 wb[kStreamDepth][FN];
#pragma unroll
  for (int d = 0; d < kStreamDepth; ++d) {
#pragma unroll
    for (int f = 0; f < FN; ++f) wb[d][f] = load_stream16(d <= last ? cptr[f] + 1024 * d : dummy);
  }

  // Stage the token operand with direct global->LDS copies (no registers):
  // each wave copies whole rows, 1 KB of codes / 256 B of scales per
  // instruction, and waits for its copies before the barrier.  Rows past
  // nrows are zero-filled.
  tile_rows<MODE>(p, row0, nrows, MT, s_src, s_ginv, MODE == 1 ? s_slot : nullptr);
  __syncthreads();
  {
    const uint8_t* a_codes = MODE == 0 ? p.xq_codes : p.a2_codes;
    const uint8_t* a_scales = MODE == 0 ? p.xq_scales : p.a2_scales;
    const int cbytes = K / 2, sbytes = K / 16;
    for (int m = wave; m < nrows; m += 4) {
      const int64_t src = s_src[m];
      copy_rows_to_lds<16>(a_codes + src * cbytes, lc + m * cpitch, cbytes, lane);
      copy_rows_to_lds<4>(a_scales + src * sbytes, ls + m * spitch, sbytes, lane);
    }
    for (int it = threadIdx.x; it < (MT - nrows) * (cbytes / 16); it += 256) {
      const int m = nrows + it / (cbytes / 16), j = it % (cbytes / 16);
      *reinterpret_cast<uint4*>(lc + m * cpitch + 16 * j) = make_uint4(0, 0, 0, 0);
    }
    for (int it = threadIdx.x; it < (MT - nrows) * (sbytes / 4); it += 256) {
      const int m = nrows + it / (sbytes / 4), j = it % (sbytes / 4);
      *reinterpret_cast<uint32_t*>(ls + m * spitch + 4 * j) = 0u;
    }
    __builtin_amdgcn_s_waitcnt(0);
  }

  f32x4 acc[FN][FM];
#pragma unroll
  for (int f = 0; f < FN; ++f)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) acc[f][fm] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // token operand staged

  for (int s8 = 0; s8 < nsteps; s8 += 8) {
    // scales of the next 8 steps (one 16-byte load per fragment row)
    uint4 wsc_nxt[FN];
    const bool more = s8 + 8 <= last;
#pragma unroll
    for (int f = 0; f < FN; ++f)
      wsc_nxt[f] = *reinterpret_cast<const uint4*>(more ? sptr[f] + 1024 * ((s8 + 8) / 8) : dummy);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int s = s8 + d;
      constexpr int kSlots = kStreamDepth;
      const int slot = d % kSlots;
      if (s < nsteps) {
        uint4 bc[FM];
        half2v bsc[FM][2];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          const int r = fm * 16 + r16;
          bc[fm] = *reinterpret_cast<const uint4*>(lc + r * cpitch + 64 * s + 16 * g);
          const uint32_t sw = *reinterpret_cast<const uint16_t*>(ls + r * spitch + 8 * s + 2 * g);
          bsc[fm][0] = e4m3_to_half2(sw);
          bsc[fm][1] = e4m3_to_half2(sw >> 8);
        }
        half2v wsc[FN][2];
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const uint32_t w16 = word_of(wsc_cur[f], d >> 1) >> (16 * (d & 1));
          wsc[f][0] = e4m3_to_half2(w16);
          wsc[f][1] = e4m3_to_half2(w16 >> 8);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          half8 bq[FM];
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) bq[fm] = dequant8_f16(word_of(bc[fm], q), bsc[fm][q >> 1]);
#pragma unroll
          for (int f = 0; f < FN; ++f) {
            const half8 aq = dequant8_f16(word_of(wb[slot][f], q), wsc[f][q >> 1]);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
              acc[f][fm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, bq[fm], acc[f][fm], 0, 0, 0);
          }
        }
      }
      const int sn = s + kStreamDepth;
#pragma unroll
      for (int f = 0; f < FN; ++f) wb[slot][f] = load_stream16(sn <= last ? cptr[f] + 1024 * sn : dummy);
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) wsc_cur[f] = wsc_nxt[f];
  }

  if (MODE == 0) {
    g1_epilogue<FM, FNH>(p, reinterpret_cast<const f32x4(&)[2 * FNH][FM]>(acc), e, row0, nrows,
                         cbase, s_ginv, s_aux, wave, g, r16);
    g1_store_band_amax<MT>(p, s_aux, row0, nrows);
  } else {
    g2_epilogue<FM, FN>(p, acc, e, row0, nrows, cbase, s_ginv, s_slot, g, r16);
  }
}

// ---------------------------------------------------------------------------
// Tiled kernel (many rows per expert: prefill).  64-row tiles; the token
// operand is staged in LDS as fp16 in K chunks of 256; each wave streams FN
// weight fragments of 16 rows per chunk.
// ---------------------------------------------------------------------------
constexpr int kTiledKC = 256;
constexpr int kTiledPitch = kTiledKC + 8;  // fp16 elements per LDS row (16-byte pad)

template <int FM, int FN, int MODE>
__global__ __launch_bounds__(256) void moe_tiled_kernel(FwdParams p) {
  constexpr int MT = 16 * FM;
  constexpr int FNH = FN / 2;
  __shared__ _Float16 lds[MT][kTiledPitch];
  __shared__ int s_src[MT];
  __shared__ int s_slot[MT];
  __shared__ float s_ginv[MT];
  __shared__ float s_amax[4][MT];
  if (static_cast<int>(blockIdx.x) >= *p.n_tiles) return;
  const int4 td = p.tiles[blockIdx.x];
  const int e = td.x, row0 = td.y, nrows = td.z;
  const int K = MODE == 0 ? p.H : p.I;
  const uint8_t* a_codes = MODE == 0 ? p.xq_codes : p.a2_codes;
  const uint8_t* a_scales = MODE == 0 ? p.xq_scales : p.a2_scales;
  tile_rows<MODE>(p, row0, nrows, MT, s_src, s_ginv, MODE == 1 ? s_slot : nullptr);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4, r16 = lane & 15;
  // fragment f = 16 weight rows = one 16-row group of the fragment-major copy
  const int S = ksteps(K), Q = sgroups(K);
  const uint8_t* cptr[FN];
  const uint8_t* sptr[FN];
  int cbase;
  if (MODE == 0) {
    cbase = blockIdx.y * (64 * FNH) + wave * 16 * FNH;
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int64_t n = f < FNH ? cbase + f * 16 : p.I + cbase + (f - FNH) * 16;
      const int64_t grp = (static_cast<int64_t>(e) * 2 * p.I + n) / 16;
      cptr[f] = p.w13c + grp * S * 1024 + 16 * lane;
      sptr[f] = p.w13s + grp * Q * 1024 + 16 * lane;
    }
  } else {
    cbase = blockIdx.y * (64 * FN) + wave * 16 * FN;
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int64_t grp = (static_cast<int64_t>(e) * p.H + cbase + f * 16) / 16;
      cptr[f] = p.w2c + grp * S * 1024 + 16 * lane;
      sptr[f] = p.w2s + grp * Q * 1024 + 16 * lane;
    }
  }
  f32x4 acc[FN][FM];
#pragma unroll
  for (int f = 0; f < FN; ++f)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) acc[f][fm] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kc = 0; kc < K; kc += kTiledKC) {
    const int nsteps = min(kTiledKC, K - kc) / 128;
    uint4 wb[2][FN];
    uint32_t wsb[2][FN];
    const int s0 = kc / 128;  // even: both steps of the chunk are in one scale group
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const uint4 sg = *reinterpret_cast<const uint4*>(sptr[f] + 1024 * (s0 / 8));
      const uint32_t w = word_of(sg, (s0 % 8) / 2);
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        wb[d][f] = load_stream16(cptr[f] + 1024 * min(s0 + d, S - 1));
        wsb[d][f] = w >> (16 * d);
      }
    }
    __syncthreads();  // previous chunk consumed; row table ready
    const int items = MT * nsteps * 4;
    for (int it = threadIdx.x; it < items; it += 256) {
      const int m = it / (nsteps * 4);
      const int kk = (it - m * nsteps * 4) * 32;
      const int src = s_src[m];
      half8* dst = reinterpret_cast<half8*>(&lds[m][kk]);
      if (src >= 0) {
        const uint4 cw = *reinterpret_cast<const uint4*>(a_codes + static_cast<int64_t>(src) * (K / 2) + (kc + kk) / 2);
        const uint32_t sw = *reinterpret_cast<const uint16_t*>(a_scales + static_cast<int64_t>(src) * (K / 16) + (kc + kk) / 16);
        const half2v s0 = e4m3_to_half2(sw), s1 = e4m3_to_half2(sw >> 8);
        dst[0] = dequant8_f16(cw.x, s0);
        dst[1] = dequant8_f16(cw.y, s0);
        dst[2] = dequant8_f16(cw.z, s1);
        dst[3] = dequant8_f16(cw.w, s1);
      } else {
        const half8 z = {0, 0, 0, 0, 0, 0, 0, 0};
        dst[0] = z; dst[1] = z; dst[2] = z; dst[3] = z;
      }
    }
    __syncthreads();
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      if (d < nsteps) {
        half2v wsc[FN][2];
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          wsc[f][0] = e4m3_to_half2(wsb[d][f]);
          wsc[f][1] = e4m3_to_half2(wsb[d][f] >> 8);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          half8 bq[FM];
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
            bq[fm] = *reinterpret_cast<const half8*>(&lds[fm * 16 + r16][d * 128 + 32 * g + 8 * q]);
#pragma unroll
          for (int f = 0; f < FN; ++f) {
            const half8 aq = dequant8_f16(word_of(wb[d][f], q), wsc[f][q >> 1]);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
              acc[f][fm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, bq[fm], acc[f][fm], 0, 0, 0);
          }
        }
      }
    }
  }

  if (MODE == 0) {
    g1_epilogue<FM, FNH>(p, reinterpret_cast<const f32x4(&)[2 * FNH][FM]>(acc), e, row0, nrows,
                         cbase, s_ginv, s_amax, wave, g, r16);
    g1_store_band_amax<MT>(p, s_amax, row0, nrows);
  } else {
    g2_epilogue<FM, FN>(p, acc, e, row0, nrows, cbase, s_ginv, s_slot, g, r16);
  }
}

// ---------------------------------------------------------------------------
// Re-quantization of every expanded row for the tiled path: one wave per row
// reads its act row (I binary32 values), takes the row amax over the GEMM1
// band partials, and quantizes 16-element blocks (lane b handles blocks b,
// b + 64, ...).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void moe_requant_kernel(FwdParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (row >= p.R) return;
  const int I = p.I;
  float a = 0.0f;
  for (int j = lane; j < p.g1_bands; j += kWave) a = fmaxf(a, p.act_amax[row * p.g1_bands + j]);
  const float g2 = global_scale(wave_max(a));
  if (lane == 0) p.a2_g[row] = g2;
  for (int b = lane; b < I / 16; b += kWave) {
    uint32_t lo, hi;
    const uint32_t sb = requant_block(p.act + row * I + 16 * b, g2, lo, hi);
    *reinterpret_cast<uint2*>(p.a2_codes + row * (I / 2) + 8 * b) = make_uint2(lo, hi);
    p.a2_scales[row * (I / 16) + b] = static_cast<uint8_t>(sb);
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
constexpr int kTiledFN = 2;

int stream_lds_bytes(int fm, int K) { return 16 * fm * ((K / 2 + 16) + (K / 16 + 4)); }

// Kernel family, rows per tile and fragments per wave for a forward of T
// tokens.  Stream kernels use 4 fragments per wave (the token operand's
// dequantization is shared by more weight rows) when that still gives at
// least two blocks per CU, else 2 (more, smaller blocks for tiny batches).
void choose_gemm(int64_t T, FwdParams* p) {
  const int H = p->H, I = p->I, E = p->E;
  const int64_t R = T * p->k;
  const int64_t active = R < E ? R : E;
  const int64_t avg = (R + active - 1) / (active > 0 ? active : 1);
  const int Kmax = H > I ? H : I;
  const bool bands_fit = H % 128 == 0 && I % 64 == 0;
  if (bands_fit && avg <= 16 && stream_lds_bytes(1, Kmax) <= 65536) {
    p->mt = 16;
    p->gemm_kind = kGemmStream;
  } else if (bands_fit && avg <= 32 && stream_lds_bytes(2, Kmax) <= 65536) {
    p->mt = 32;
    p->gemm_kind = kGemmStream;
  } else {
    p->mt = 64;
    p->gemm_kind = kGemmTiled;
  }
  if (p->gemm_kind == kGemmStream) {
    const int64_t tiles = (R + p->mt - 1) / p->mt > active ? (R + p->mt - 1) / p->mt : active;
    const int64_t want = 2 * 256;
    p->g1_fn = (I % 128 == 0 && tiles * (I / 128) >= want) ? 4 : 2;
    p->g2_fn = (H % 256 == 0 && tiles * (H / 256) >= want) ? 4 : 2;
    p->g1_bands = I / (32 * p->g1_fn);
  } else {
    p->g1_fn = p->g2_fn = kTiledFN;
    p->g1_bands = I / (64 * (kTiledFN / 2));
  }
}

template <int FM, int FN1, int FN2>
static void launch_stream(const FwdParams& p, int max_tiles, hipStream_t s, hipEvent_t const* ev) {
  const int nb1 = p.I / (32 * FN1);
  moe_stream_kernel<FM, FN1, 0><<<dim3(max_tiles, nb1), 256, stream_lds_bytes(FM, p.H), s>>>(p);
  if (ev) (void)hipEventRecord(ev[2], s);
  moe_requant_kernel<<<(p.R + 3) / 4, 256, 0, s>>>(p);
  const int nb2 = p.H / (64 * FN2);
  moe_stream_kernel<FM, FN2, 1><<<dim3(max_tiles, nb2), 256, stream_lds_bytes(FM, p.I), s>>>(p);
  if (ev) (void)hipEventRecord(ev[3], s);
}

template <int FM>
static void launch_stream_fm(const FwdParams& p, int max_tiles, hipStream_t s, hipEvent_t const* ev) {
  if (p.g1_fn == 4 && p.g2_fn == 4) launch_stream<FM, 4, 4>(p, max_tiles, s, ev);
  else if (p.g1_fn == 4) launch_stream<FM, 4, 2>(p, max_tiles, s, ev);
  else if (p.g2_fn == 4) launch_stream<FM, 2, 4>(p, max_tiles, s, ev);
  else launch_stream<FM, 2, 2>(p, max_tiles, s, ev);
}

hipError_t launch_grouped_gemms(const FwdParams& p, int max_tiles, hipStream_t s,
                                hipEvent_t const* ev) {
  if (p.gemm_kind == kGemmStream) {
    if (p.mt == 16)
      launch_stream_fm<1>(p, max_tiles, s, ev);
    else
      launch_stream_fm<2>(p, max_tiles, s, ev);
  } else {
    const int nb1 = p.I / (64 * (kTiledFN / 2));
    moe_tiled_kernel<4, kTiledFN, 0><<<dim3(max_tiles, nb1), 256, 0, s>>>(p);
    if (ev) (void)hipEventRecord(ev[2], s);
    moe_requant_kernel<<<(p.R + 3) / 4, 256, 0, s>>>(p);
    const int nb2 = p.H / (64 * kTiledFN);
    moe_tiled_kernel<4, kTiledFN, 1><<<dim3(max_tiles, nb2), 256, 0, s>>>(p);
    if (ev) (void)hipEventRecord(ev[3], s);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
