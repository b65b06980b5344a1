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
#include <algorithm>
#include <atomic>

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

// Workgroup barrier for LDS data only.  A full __syncthreads also waits for
// every outstanding global load and store (the global->LDS copies count as
// loads), which would drain the weight prefetch or wait for output stores;
// here the caller has already waited for the copies it needs, this wave's
// LDS accesses are complete (lgkmcnt 0), and the memory clobber keeps the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------
// Epilogues.
// ---------------------------------------------------------------------------

// GEMM1: per lane, fragment pair (gate fh, up fh) holds h[n = c0 + 16 fh + 4g + i]
// for row m = 16 fm + r16; ginv[fm] = 1 / (that row's token global scale),
// wginv = 1 / (the expert's W13 global scale).
// act = silu(h_gate) * h_up in fp32, stored with the row's amax over these
// columns in s_amax[wave][m].  BF16: W4A16's GEMM2 input, act rounded to
// bf16 (nearest even), is stored as well (a2q16, the same index).
template <int FM, int FNH, int SM = 16 * FM, bool BF16 = false>
__device__ __forceinline__ void g1_epilogue(const FwdParams& p, const f32x4 (&acc)[2 * FNH][FM],
                                            int e, int row0, int nrows, int c0, const float (&ginv)[FM],
                                            float (*s_amax)[SM], int wave, int g, int r16, float wginv) {
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = fm * 16 + r16;
    const float alpha = ginv[fm] * wginv;
    float am = 0.0f;
#pragma unroll
    for (int fh = 0; fh < FNH; ++fh) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float hg = acc[fh][fm][i] * alpha;
        const float hu = acc[FNH + fh][fm][i] * alpha;
        // silu(hg) = hg / (1 + e^-hg) with the hardware exp and reciprocal
        // (about 1 ulp each; e^-hg overflowing to inf gives silu = -0)
        a[i] = hg * __builtin_amdgcn_rcpf(1.0f + __expf(-hg)) * hu;
        am = fmaxf(am, fabsf(a[i]));
      }
      if (m < nrows) {
        const int n = c0 + fh * 16 + 4 * g;
        const int64_t idx = static_cast<int64_t>(row0 + m) * p.I + n;
        *reinterpret_cast<float4*>(p.act + idx) = make_float4(a[0], a[1], a[2], a[3]);
        if constexpr (BF16) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 r;
          r[0] = static_cast<__bf16>(a[0]);
          r[1] = static_cast<__bf16>(a[1]);
          r[2] = static_cast<__bf16>(a[2]);
          r[3] = static_cast<__bf16>(a[3]);
          *reinterpret_cast<bf16x4*>(p.a2q16 + idx) = r;
        }
      }
    }
    am = fmaxf(am, __shfl_xor(am, 16, kWave));
    am = fmaxf(am, __shfl_xor(am, 32, kWave));
    if (g == 0) s_amax[wave][m] = am;
  }
}

// The block's per-row amax of act over its columns (one partial per GEMM1
// column band; the re-quantization kernel reduces them).
template <int MT>
__device__ __forceinline__ void g1_store_band_amax(const FwdParams& p, float (*s_amax)[MT], int row0,
                                                   int nrows, int band, int nbands) {
  lds_barrier();  // s_amax complete (the act stores need not be)
  if (threadIdx.x < MT && static_cast<int>(threadIdx.x) < nrows) {
    const int m = threadIdx.x;
    const float v = fmaxf(fmaxf(s_amax[0][m], s_amax[1][m]), fmaxf(s_amax[2][m], s_amax[3][m]));
    p.act_amax[static_cast<int64_t>(row0 + m) * nbands + band] = v;
  }
}

// Atomic finalize: GEMM2 results are staged in LDS, 64 columns per row at
// this pitch (64 + 4 floats: consecutive rows start on different banks), and
// added into out_acc a row at a time (256 contiguous bytes per atomic
// instruction).
constexpr int kAtomicPitch = 68;

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

// Four binary32 values -> four bf16 (nearest even), element 0 in the low half.
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2(f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16),
                    f32_to_bf16_rne(c) | (f32_to_bf16_rne(d) << 16));
}

// GEMM2: per lane, fragment f holds y[n = n0 + 16 f + 4g + i] of row m =
// 16 fm + r16; ginv[fm] = 1 / (that row's a2 global scale), slot[fm] = its
// t*k+j, wginv = 1 / (the expert's W2 global scale).  y is stored by slot
// (row t*k+j of y is token t's j-th expert output), so the finalize reads
// each token's k rows contiguously, without the inverse permutation.  Like
// the layer's input and output, the expanded rows' outputs are held in bf16
// (rounded to nearest even); the finalize sums them in binary32.
template <int FM, int FN>
__device__ __forceinline__ void g2_epilogue(const FwdParams& p, const f32x4 (&acc)[FN][FM], int e,
                                            int row0, int nrows, int n0, const float (&ginv)[FM],
                                            const int (&slot)[FM], int g, int r16, float wginv) {
  const int H = p.H;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = fm * 16 + r16;
    if (m >= nrows) continue;
    const float alpha = ginv[fm] * wginv;
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int n = n0 + f * 16 + 4 * g;
      const float y0 = acc[f][fm][0] * alpha, y1 = acc[f][fm][1] * alpha;
      const float y2 = acc[f][fm][2] * alpha, y3 = acc[f][fm][3] * alpha;
      if (p.deterministic) {
        *reinterpret_cast<uint2*>(p.y + static_cast<int64_t>(slot[fm]) * H + n) = pack_bf16x4(y0, y1, y2, y3);
      } else {
        const float w = slot_weight(p, slot[fm]);
        float* dst = p.out_acc + static_cast<int64_t>(slot_token(p, slot[fm])) * H + n;
        atomicAdd(dst + 0, w * y0);
        atomicAdd(dst + 1, w * y1);
        atomicAdd(dst + 2, w * y2);
        atomicAdd(dst + 3, w * y3);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Stream kernel (few rows per expert: decode).  One block = one tile of up to
// 16*FM rows x 4/KS weight units; wave w takes unit w / KS and the K range
// w % KS of it (KS waves split one unit's K and add their partial sums in LDS
// at the end).  The tile's token operand is staged once in LDS as FP4 codes +
// E4M3 scales (dynamic LDS: MT rows x (K/2 + 16) code bytes and (K/16 + 4)
// scale bytes); each wave then walks its K range in 128-wide steps, one
// 4.5 KB unit record per step, with the next few records in flight.
//
// Issue order.  Vector loads complete in issue order, so a wait for the
// staging copies also waits for every weight load issued before them.  The
// kernel therefore issues two weight steps, then the staging copies, waits,
// and only then fills the rest of the prefetch window: the wave starts
// computing as soon as its first records land instead of after all of them.
// Every later load is unconditional (past the wave's range it reads a zero
// dummy record), so each wait covers exactly the oldest step.
// MODE 0: GEMM1 (W13 units: 2 gate + 2 up fragments, SwiGLU epilogue); the
//   token operand is the per-token quantized x, copied to LDS with direct
//   global->LDS loads.
// MODE 1: GEMM2 (W2 units: 4 output fragments); the token operand is the
//   re-quantization of the tile's act rows, done here: the block reads the
//   rows' GEMM1 amax partials and the act values into registers ahead of the
//   weight stream, then quantizes into LDS (band-0 blocks also store the
//   result, for inspection).  The bands of a tile run on different XCDs
//   (see launch_stream): spreading each expert's weight stream over the
//   XCDs matters more than keeping the repeated act reads in one L2.
// ---------------------------------------------------------------------------
// Weight records each wave keeps in flight.  GEMM2 with a short K range
// (SHORT: at most kStreamShortSteps K steps, e.g. I = 768) keeps 2: measured
// on the decode-shaped layer at T=64 (6 steps per unit), GEMM2 26.2-26.5 ->
// 25.3-25.7 us against 3 (W4A16: 28.3-28.7 -> 27.4-27.6 us), while with 16
// steps (the large layer, I = 2048) 2 records were slower (T=1 17.9 -> 19.9
// us, T=7 52 -> 57 us).
template <int MODE, bool SHORT = false>
struct StreamDepth {
  static constexpr int value = MODE == 0 ? 5 : (SHORT ? 2 : 3);
};
constexpr int kStreamShortSteps = 8;
constexpr int kStreamEarly = 2;  // steps issued before the staging copies

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

// One step's weight operand of a wave: 4 code pieces + the lane's 8 scale bytes.
struct UnitStep {
  uint4 c[kUnitFrags];
  uint2 sc;
};
// NT: non-temporal code loads, for kernels that read each record once (the
// stream kernels; the tiled kernel's 16-row variant).  The 128-row tiled
// kernels read an expert's records again for each of its tiles and load them
// cached (measured: prefill-shaped layer 465-467 -> 440-441 us, GEMM1
// 236-242 -> 218-223 us, GEMM2 187-189 -> 174-177 us; large layer at
// T=2048 2.195 -> 2.078 ms; the decode-shaped layer's stream GEMMs were
// 4-5 us slower with cached loads, W4A16 decode's 16-row tiled GEMM1 3 us).
template <bool NT = true>
__device__ __forceinline__ void load_unit_step(UnitStep& u, const uint8_t* rec, int lane) {
#pragma unroll
  for (int f = 0; f < kUnitFrags; ++f)
    u.c[f] = NT ? load_stream16(rec + 1024 * f + 16 * lane)
                : *reinterpret_cast<const uint4*>(rec + 1024 * f + 16 * lane);
  u.sc = *reinterpret_cast<const uint2*>(rec + kRecCodeBytes + 8 * lane);
}

// acc[f][fm] += W_f (16 x 128 slice of step `step`) * token rows (fm) on the
// token operand staged in LDS.
template <int FM>
__device__ __forceinline__ void unit_step_mfma(f32x4 (&acc)[kUnitFrags][FM], const UnitStep& w,
                                               const uint8_t* lc, const uint8_t* ls, int cpitch,
                                               int spitch, int step, int g, int r16) {
  uint4 bc[FM];
  half2v bsc[FM][2];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int r = fm * 16 + r16;
    bc[fm] = *reinterpret_cast<const uint4*>(lc + r * cpitch + 64 * step + 16 * g);
    const uint32_t sw = *reinterpret_cast<const uint16_t*>(ls + r * spitch + 8 * step + 2 * g);
    bsc[fm][0] = e4m3_to_half2(sw);
    bsc[fm][1] = e4m3_to_half2(sw >> 8);
  }
  half2v wsc[kUnitFrags][2];
#pragma unroll
  for (int f = 0; f < kUnitFrags; ++f) {
    const uint32_t w16 = (f < 2 ? w.sc.x : w.sc.y) >> (16 * (f & 1));
    wsc[f][0] = e4m3_to_half2(w16);
    wsc[f][1] = e4m3_to_half2(w16 >> 8);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    half8 bq[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) bq[fm] = dequant8_f16(word_of(bc[fm], q), bsc[fm][q >> 1]);
#pragma unroll
    for (int f = 0; f < kUnitFrags; ++f) {
      const half8 aq = dequant8_f16(word_of(w.c[f], q), wsc[f][q >> 1]);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        acc[f][fm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, bq[fm], acc[f][fm], 0, 0, 0);
    }
  }
}

// The same step for W4A16: the token rows are staged as bf16 (row pitch
// cpitch bytes; lane group g reads k = 128 step + 32 g + 8 q .. + 7 of row
// 16 fm + r16), the weight fragments are dequantized exactly to bf16.
template <int FM>
__device__ __forceinline__ void unit_step_mfma_a16(f32x4 (&acc)[kUnitFrags][FM], const UnitStep& w,
                                                   const uint8_t* lc, int cpitch, int step, int g, int r16) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    bf16x8 bq[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      bq[fm] = *reinterpret_cast<const bf16x8*>(lc + (fm * 16 + r16) * cpitch + 2 * (128 * step + 32 * g + 8 * q));
#pragma unroll
    for (int f = 0; f < kUnitFrags; ++f) {
      // scale of this q's 16-element block (q 0-1: first byte, q 2-3: second)
      const uint32_t w16 = (f < 2 ? w.sc.x : w.sc.y) >> (16 * (f & 1) + 8 * (q >> 1));
      const bf16x8 aq = dequant8_bf16(word_of(w.c[f], q), e4m3_to_f32(w16));
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        acc[f][fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bq[fm], acc[f][fm], 0, 0, 0);
    }
  }
}

// Act values of one 16-element block of an expanded row.
struct ActBlock {
  float4 v[4];
};

template <int FM, int KS, int MODE, bool A16, bool SHORT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FM == 1 ? 3 + MODE : 2))) void moe_stream_kernel(FwdParams p) {
  // (W4A16 streams GEMM2 only: its GEMM1 runs on the tiled kernel, which
  // measured faster there)
  static_assert(!A16 || MODE == 1, "bf16 staging is GEMM2's");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int MT = 16 * FM;
  constexpr int UB = 4 / KS;  // units per block
  static_assert(!SHORT || MODE == 1, "the short window is GEMM2's");
  constexpr int D = StreamDepth<MODE, SHORT>::value;
  constexpr int kRq = 2;  // re-quantization items per thread loaded ahead of the weights
  __shared__ float s_amax[4][MT];
  __shared__ float s_g2[MT];
  if (static_cast<int>(blockIdx.x) >= *p.n_tiles) return;
  const int4 td = p.tiles[blockIdx.x];
  const int e = td.x, row0 = td.y, nrows = td.z;
  const int K = MODE == 0 ? p.H : p.I;
  const int S = ksteps(K);
  // staged row pitch: FP4 codes (+ a separate scale area), or bf16 values
  // (W4A16); the 16-byte pad puts the 16 rows one MFMA operand read touches
  // on different LDS banks
  const int cpitch = A16 ? 2 * K + 16 : K / 2 + 16, spitch = K / 16 + 4;
  uint8_t* lc = smem;
  uint8_t* ls = smem + MT * cpitch;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4, r16 = lane & 15;

  // this wave's unit and K range
  const int ui = wave / KS, kp = wave % KS;
  const int upe = MODE == 0 ? p.I / 32 : p.H / 64;
  const int j = blockIdx.y * UB + ui;
  const int per = (S + KS - 1) / KS;
  const int sb = min(S, kp * per);
  const int ns = min(S, sb + per) - sb;
  const uint8_t* rec = (MODE == 0 ? p.w13 : p.w2) +
                       (static_cast<int64_t>(e) * upe * S + static_cast<int64_t>(j) * S + sb) * kRecBytes;

  // Rows past nrows in the LDS operand are left as they are: they only feed
  // output columns that are never stored.
  UnitStep wb[D];
  int slot = 0;
  float grow = 1.0f;  // GEMM1: the row's token global scale (lane m < nrows holds row m's)
  if constexpr (MODE == 0) {
    // Source rows of the tile.  The row table load goes first, so that
    // waiting for it does not wait for weights.
    // (lanes past nrows take the last row: the table load and the wait for
    // it are then on every path, ahead of the copies)
    slot = row_slot(p, row0 + min(lane, nrows - 1));
#pragma unroll
    for (int d = 0; d < kStreamEarly; ++d) load_unit_step(wb[d], d < ns ? rec + d * kRecBytes : p.dummy, lane);
    const int src = slot_token(p, slot);
    const int cbytes = K / 2, sbytes = K / 16;
    for (int m = wave; m < nrows; m += 4) {
      const int64_t sm = __builtin_amdgcn_readlane(src, m);
      copy_rows_to_lds<16>(p.xq_codes + sm * cbytes, lc + m * cpitch, cbytes, lane);
      copy_rows_to_lds<4>(p.xq_scales + sm * sbytes, ls + m * spitch, sbytes, lane);
    }
    // The rest of the prefetch window goes out behind the copies; vector
    // memory counts complete in issue order, so waiting until only those
    // records are outstanding covers the copies (and the first records)
    // without draining the window.  Each load_unit_step is kUnitFrags + 1
    // instructions; the records are used on a run-time condition, so none
    // is dropped, and the scheduling barriers keep the issue order.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = kStreamEarly; d < D; ++d) load_unit_step(wb[d], d < ns ? rec + d * kRecBytes : p.dummy, lane);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(D - kStreamEarly) * (kUnitFrags + 1)>();
    __builtin_amdgcn_sched_barrier(0);
    // the epilogue's row scales (used after the loop)
    if (lane < nrows) grow = p.xq_g[src];
  } else if constexpr (A16) {
    // W4A16: GEMM2's input is act rounded to bf16 (nearest even).  The first
    // pieces of the tile's act rows are loaded ahead of the weight window
    // (vector loads complete in issue order), converted into the LDS
    // operand; band-0 blocks also store them (the 16-bit GEMM2 input).
    constexpr int kA = 4;  // 8-value pieces per thread loaded ahead
    const int n8 = K / 8, items = nrows * n8;
    float4 pa[kA][2];
#pragma unroll
    for (int i = 0; i < kA; ++i) {
      const int it = min(static_cast<int>(threadIdx.x) + 256 * i, items - 1);
      const int m = it / n8, c = it - m * n8;
      const float4* src4 = reinterpret_cast<const float4*>(p.act + static_cast<int64_t>(row0 + m) * K + 8 * c);
      pa[i][0] = src4[0];
      pa[i][1] = src4[1];
    }
#pragma unroll
    for (int d = 0; d < D; ++d) load_unit_step(wb[d], d < ns ? rec + d * kRecBytes : p.dummy, lane);
    if (lane < nrows) slot = row_slot(p, row0 + lane);
    auto stage = [&](const float4& a, const float4& b, int it) {
      const int m = it / n8, c = it - m * n8;
      bf16x8 r;
      r[0] = static_cast<__bf16>(a.x); r[1] = static_cast<__bf16>(a.y);
      r[2] = static_cast<__bf16>(a.z); r[3] = static_cast<__bf16>(a.w);
      r[4] = static_cast<__bf16>(b.x); r[5] = static_cast<__bf16>(b.y);
      r[6] = static_cast<__bf16>(b.z); r[7] = static_cast<__bf16>(b.w);
      *reinterpret_cast<bf16x8*>(lc + m * cpitch + 16 * c) = r;
      if (blockIdx.y == 0) *reinterpret_cast<bf16x8*>(p.a2q16 + static_cast<int64_t>(row0 + m) * K + 8 * c) = r;
    };
#pragma unroll
    for (int i = 0; i < kA; ++i) {
      const int it = static_cast<int>(threadIdx.x) + 256 * i;
      if (it < items) stage(pa[i][0], pa[i][1], it);
    }
    for (int it = static_cast<int>(threadIdx.x) + 256 * kA; it < items; it += 256) {
      const int m = it / n8, c = it - m * n8;
      const float4* src4 = reinterpret_cast<const float4*>(p.act + static_cast<int64_t>(row0 + m) * K + 8 * c);
      stage(src4[0], src4[1], it);
    }
  } else {
    // Fused re-quantization.  Loads in issue order: GEMM1 amax partials of
    // the wave's rows, the first kRq act blocks of this thread, the first
    // weight record; the rest of the prefetch window goes out once the
    // operand is staged (with the whole window issued first, GEMM2 took
    // 0.8-0.9 us longer at T=64 on the decode-shaped layer and at T=1 on the
    // large layer).  Each wait below covers only the loads it
    // needs.
    const int nbl = K / 16, nb = p.g1_bands;
    const int items = nrows * nbl;
    constexpr int RPW = MT / 4;  // rows per wave
    float pa[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int m = wave + 4 * i;
      const int64_t row = row0 + min(m, nrows - 1);
      pa[i] = p.act_amax[row * nb + min(lane, nb - 1)];
    }
    ActBlock ab[kRq];
#pragma unroll
    for (int i = 0; i < kRq; ++i) {
      const int it = min(static_cast<int>(threadIdx.x) + 256 * i, items - 1);
      const int m = it / nbl, b = it - m * nbl;
      const float4* src4 = reinterpret_cast<const float4*>(p.act + static_cast<int64_t>(row0 + m) * K + 16 * b);
#pragma unroll
      for (int q = 0; q < 4; ++q) ab[i].v[q] = src4[q];
    }
    load_unit_step(wb[0], 0 < ns ? rec : p.dummy, lane);
    if (lane < nrows) slot = row_slot(p, row0 + lane);
    // row global scales g2 = 2688 / amax(act row)
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int m = wave + 4 * i;
      float a = lane < nb ? pa[i] : 0.0f;
      for (int c = lane + kWave; c < nb; c += kWave)
        a = fmaxf(a, p.act_amax[static_cast<int64_t>(row0 + min(m, nrows - 1)) * nb + c]);
      a = wave_max(a);
      if (lane == 0 && m < nrows) {
        const float g2 = p.static_g ? p.static_g[1] : global_scale(a);
        s_g2[m] = g2;
        if (blockIdx.y == 0) p.a2_g[row0 + m] = g2;
      }
    }
    __syncthreads();
    auto quant_item = [&](const ActBlock& a, int it) {
      const int m = it / nbl, b = it - m * nbl;
      float f[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[4 * q] = a.v[q].x; f[4 * q + 1] = a.v[q].y; f[4 * q + 2] = a.v[q].z; f[4 * q + 3] = a.v[q].w;
      }
      uint32_t lo, hi;
      const uint32_t sb = quantize_block16(f, s_g2[m], lo, hi);
      *reinterpret_cast<uint2*>(lc + m * cpitch + 8 * b) = make_uint2(lo, hi);
      ls[m * spitch + b] = static_cast<uint8_t>(sb);
      if (blockIdx.y == 0) {
        const int64_t row = row0 + m;
        *reinterpret_cast<uint2*>(p.a2_codes + row * (K / 2) + 8 * b) = make_uint2(lo, hi);
        p.a2_scales[row * (K / 16) + b] = static_cast<uint8_t>(sb);
      }
    };
#pragma unroll
    for (int i = 0; i < kRq; ++i) {
      const int it = static_cast<int>(threadIdx.x) + 256 * i;
      if (it < items) quant_item(ab[i], it);
    }
    // tiles with more items than kRq per thread: the rest, batch by batch
    for (int base = 256 * kRq; base < items; base += 256) {
      const int it = base + static_cast<int>(threadIdx.x);
      if (it < items) {
        const int m = it / nbl, b = it - m * nbl;
        const float4* src4 = reinterpret_cast<const float4*>(p.act + static_cast<int64_t>(row0 + m) * K + 16 * b);
        ActBlock a;
#pragma unroll
        for (int q = 0; q < 4; ++q) a.v[q] = src4[q];
        quant_item(a, it);
      }
    }
#pragma unroll
    for (int d = 1; d < D; ++d) load_unit_step(wb[d], d < ns ? rec + d * kRecBytes : p.dummy, lane);
  }

  f32x4 acc[kUnitFrags][FM];
#pragma unroll
  for (int f = 0; f < kUnitFrags; ++f)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) acc[f][fm] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // token operand staged

  for (int s0 = 0; s0 < ns; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int s = s0 + d;
      if (s < ns) {
        if constexpr (A16)
          unit_step_mfma_a16<FM>(acc, wb[d], lc, cpitch, sb + s, g, r16);
        else
          unit_step_mfma<FM>(acc, wb[d], lc, ls, cpitch, spitch, sb + s, g, r16);
      }
      // keep the refill of this slot after its use (no extra register set)
      __builtin_amdgcn_sched_barrier(0);
      const int sn = s + D;
      load_unit_step(wb[d], sn < ns ? rec + static_cast<int64_t>(sn) * kRecBytes : p.dummy, lane);
    }
  }

  if constexpr (KS > 1) {
    // add the K-range partials of the waves that share a unit
    float* red = reinterpret_cast<float*>(smem);
    __syncthreads();  // staged operand no longer read
    if (kp > 0) {
#pragma unroll
      for (int f = 0; f < kUnitFrags; ++f)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[(((wave * kUnitFrags + f) * FM + fm) * 4 + i) * kWave + lane] = acc[f][fm][i];
    }
    __syncthreads();
    if (kp == 0) {
#pragma unroll
      for (int o = 1; o < KS; ++o)
#pragma unroll
        for (int f = 0; f < kUnitFrags; ++f)
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[f][fm][i] += red[((((wave + o) * kUnitFrags + f) * FM + fm) * 4 + i) * kWave + lane];
    }
  }

  float ginv[FM];
  int slots[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    ginv[fm] = A16 ? 1.0f : 1.0f / (MODE == 0 ? __shfl(grow, fm * 16 + r16, kWave) : s_g2[fm * 16 + r16]);
    slots[fm] = __shfl(slot, fm * 16 + r16, kWave);
  }
  if (MODE == 0) {
    if (kp == 0) {
      g1_epilogue<FM, 2>(p, acc, e, row0, nrows, 32 * j, ginv, s_amax, wave, g, r16, 1.0f / p.w13g[e]);
    } else {
      if (g == 0)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) s_amax[wave][fm * 16 + r16] = 0.0f;
    }
    g1_store_band_amax<MT>(p, s_amax, row0, nrows, blockIdx.y, gridDim.y);
  } else if (p.deterministic) {
    if (kp == 0)
      g2_epilogue<FM, kUnitFrags>(p, acc, e, row0, nrows, 64 * j, ginv, slots, g, r16, 1.0f / p.w2g[e]);
  } else {
    // atomic finalize: stage the unit's rows in the (now free) LDS operand
    // area, then one atomic instruction per row (see kAtomicPitch)
    __syncthreads();
    if (kp == 0) {
      float* st = reinterpret_cast<float*>(smem) + ui * MT * kAtomicPitch;
      const float wginv = 1.0f / p.w2g[e];
      int tok = 0;
      float wt = 0.0f;
      if (lane < nrows) {
        tok = slot_token(p, slot);
        wt = slot_weight(p, slot);
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const float alpha = ginv[fm] * wginv;
#pragma unroll
        for (int f = 0; f < kUnitFrags; ++f) {
          const f32x4 v = acc[f][fm];
          *reinterpret_cast<float4*>(st + (fm * 16 + r16) * kAtomicPitch + 16 * f + 4 * g) =
              make_float4(v[0] * alpha, v[1] * alpha, v[2] * alpha, v[3] * alpha);
        }
      }
      const int H = p.H;
      for (int m = 0; m < nrows; ++m) {
        const float v = st[m * kAtomicPitch + lane];
        const int tm = __shfl(tok, m, kWave);
        const float wm = __shfl(wt, m, kWave);
        atomicAdd(p.out_acc + static_cast<int64_t>(tm) * H + 64 * j + lane, wm * v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tiled kernel (many rows per expert: prefill).  One block = a tile of up to
// 16*FM token rows x 4 weight units (4 waves, one unit of 64 weight rows
// each); every wave multiplies its unit with all the tile's token rows, so a
// weight fragment dequantized in registers feeds FM MFMAs.  The token operand
// is the exact fp16 copy of the quantized rows, brought into LDS one 128-wide
// K step ahead by direct global->LDS copies (no registers, no VALU) into two
// alternating buffers.  Layout of a buffer: 1 KB chunk (fm, g) (fm = 16-row
// group of the tile, g = 64-byte quarter of the step's 256-byte row segment)
// holds, at 256 q + 16 r, the 16 bytes (k = 32 g + 8 q .. + 7) of tile row
// 16 fm + r.  One copy instruction fills one chunk (16 rows x 64 contiguous
// bytes each); one MFMA operand read (fm, q) takes 256 contiguous bytes from
// each of the four chunks (fm, g): on gfx950 that reads at the full LDS rate
// of 256 B/clk, whereas 16 lanes reading 16 different 256-byte-strided rows
// (even XOR-swizzled) take twice as long.  Two blocks share a CU (two waves
// per SIMD), which keeps the matrix cores fed while the other block waits at
// its barrier.
//
// Ordering of the copies.  Vector loads complete in issue order.  In step s
// each wave issues its copies of step s + 1 among its MFMAs (after the
// barrier that frees that buffer) and the weight refill of step s + 2 after
// them, so at the start of step s + 1 exactly one refill (kRefillOps
// instructions) was issued after that step's copies: waiting until at most
// kRefillOps loads are outstanding covers the copies and nothing newer.
// Scheduling barriers keep the compiler from moving loads across these
// points.  Before the first step the block waits for all of its loads.
// ---------------------------------------------------------------------------
constexpr int kTiledWaves = 4;
constexpr int kTiledThreads = kTiledWaves * kWave;
constexpr int kTiledRows = 128;  // rows of a tile (8 groups of 16)
constexpr int kRefillOps = kUnitFrags + 1;  // vector memory instructions of load_unit_step

// Rows of the token operand for local row m of a tile: GEMM1 reads the
// per-token quantized activations of the row's token (slot_token), GEMM2
// the re-quantized activation of the expanded row itself.
template <int MODE>
__device__ __forceinline__ void tile_rows(const FwdParams& p, int row0, int nrows, int mt,
                                          int* s_src, float* s_ginv, int* s_slot) {
  if (static_cast<int>(threadIdx.x) < mt) {
    const int m = threadIdx.x;
    int src = -1, slot = -1;
    float gi = 0.0f;
    if (m < nrows) {
      slot = row_slot(p, row0 + m);
      src = MODE == 0 ? slot_token(p, slot) : row0 + m;
      gi = 1.0f / (MODE == 0 ? p.xq_g[src] : p.a2_g[src]);
    }
    s_src[m] = src;
    s_ginv[m] = gi;
    s_slot[m] = slot;
  }
}

// The global->LDS copies of one K step of the tile's fp16 token rows (this
// wave's share; see the kernel comment for the piece placement).  They are
// buffer loads with the LDS bit: unlike global_load_lds (a FLAT instruction
// that the compiler treats as touching both global memory and LDS), they
// leave the LDS counter in order, so each wait for a token fragment waits
// for that fragment's read only, not for every read issued after it.  The
// resource's size also bounds every copy: a read past it returns zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tiled_rsrc(const _Float16* base, int64_t elems) {
  // dword 3 = 0x00020000: 32-bit data format, no swizzle (raw buffer)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(base), static_cast<short>(0),
                                           static_cast<int>(2 * elems), 0x00020000);
}

// One copy instruction: 16 bytes per lane from byte offset `off` of the
// resource into 1 KB chunk `chunk` of the LDS buffer.
__device__ __forceinline__ void tiled_copy_one(__amdgpu_buffer_rsrc_t rs, int off, uint8_t* buf, int chunk) {
  auto* d = (__attribute__((address_space(3))) void*)(buf + 1024 * chunk);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, off, 0, 0, 0);
}

template <int NCP>
__device__ __forceinline__ void tiled_copy_step(__amdgpu_buffer_rsrc_t rs, const int* coff, uint8_t* buf,
                                                int s, int wave) {
  // coff: this lane's source byte offsets of the NCP copies (registers)
#pragma unroll
  for (int u = 0; u < NCP; ++u) tiled_copy_one(rs, coff[u] + 256 * s, buf, wave + kTiledWaves * u);
}

// One K step: wait for this step's copies, start the next step's, MFMAs on
// the LDS operand `cur` and the weight record in `w`, then refill `w` with
// the record two steps ahead.
// NT: the weight records are loaded non-temporally (see load_unit_step).
template <int FM, int NCP, bool A16, bool NT>
__device__ __forceinline__ void tiled_step(f32x4 (&acc)[kUnitFrags][FM], int s, int S, const uint8_t* cur,
                                           uint8_t* nxt, UnitStep& w, const uint8_t* rec, __amdgpu_buffer_rsrc_t a16,
                                           const int (&coff)[NCP], bool has_unit, int wave, int lane) {
  const int g = lane >> 4, r16 = lane & 15;
  wait_vmcnt<kRefillOps>();  // this step's copies have landed (see the kernel comment)
  lds_barrier();             // ... in every wave; the other buffer is free
  const int sn = min(s + 1, S - 1);  // the next step's copies (the last step's are unused)
  if (has_unit) {
    // The step's 4*FM (q, fm) token fragments are read from LDS two ahead of
    // their MFMAs (a rolling three-fragment window), so the read latency
    // hides behind the previous fragments' MFMAs.  The next step's copies
    // go out one per token fragment, between its MFMAs: issued together
    // right after the barrier, as every wave of the CU does at once, they
    // queue behind each other and hold the wave's MFMAs back.
    constexpr int NI = 4 * FM;
    static_assert(NCP <= NI, "one copy per token fragment at most");
    auto ldb = [&](int i) {
      const int q = i / FM, fm = i % FM;
      return *reinterpret_cast<const half8*>(cur + 1024 * (4 * fm + g) + 256 * q + 16 * r16);
    };
    half8 bb[3];
    bb[0] = ldb(0);
    bb[1] = ldb(1);
    half8 aq[kUnitFrags];    // fp16 weight fragments (NVFP4 activations)
    bf16x8 aqb[kUnitFrags];  // bf16 weight fragments (W4A16)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = i / FM, fm = i % FM;
      if (i + 2 < NI) bb[(i + 2) % 3] = ldb(i + 2);
      if (fm == 0) {
#pragma unroll
        for (int f = 0; f < kUnitFrags; ++f) {
          // scale of this q's 16-element block (q 0-1: first byte, q 2-3: second)
          const uint32_t w16 = (f < 2 ? w.sc.x : w.sc.y) >> (16 * (f & 1) + 8 * (q >> 1));
          if constexpr (A16)
            aqb[f] = dequant8_bf16(word_of(w.c[f], q), e4m3_to_f32(w16));
          else
            aq[f] = dequant8_f16(word_of(w.c[f], q), e4m3_to_half2(w16));
        }
      }
#pragma unroll
      for (int f = 0; f < kUnitFrags; ++f) {
        if constexpr (A16)
          acc[f][fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aqb[f], __builtin_bit_cast(bf16x8, bb[i % 3]),
                                                               acc[f][fm], 0, 0, 0);
        else
          acc[f][fm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[f], bb[i % 3], acc[f][fm], 0, 0, 0);
      }
      if (i < NCP) tiled_copy_one(a16, coff[i] + 256 * sn, nxt, wave + kTiledWaves * i);
    }
    // Pin the order for the scheduler: the two first reads, then per
    // fragment one read two ahead and its four MFMAs with one copy in the
    // middle (dequantization VALU is placed freely between them).
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i + 2 < NI) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i < NCP) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM (copy)
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
    }
  } else {
    tiled_copy_step<NCP>(a16, coff, nxt, sn, wave);
  }
  __builtin_amdgcn_sched_barrier(0);
  load_unit_step<NT>(w, rec + static_cast<int64_t>(min(s + 2, S - 1)) * kRecBytes, lane);
  __builtin_amdgcn_sched_barrier(0);
}

// Shared memory of one tiled block, sized for tiles of up to TR rows.
template <int TR>
struct TiledShared {
  uint8_t lds[2][TR * 256] __attribute__((aligned(16)));
  int src[TR];
  int slot[TR];
  float ginv[TR];
  float wginv;  // 1 / (the expert's weight global scale)
  float amax[kTiledWaves][TR];
};
static_assert(sizeof(TiledShared<kTiledRows>) <= 80 * 1024, "two tiled blocks must share a CU's LDS");
// Tiles of at most 16 rows (16-row tiles of decode-sized W4A16 batches): the
// block's LDS and registers are small enough for four blocks per CU.
constexpr int kTiledSmallRows = 16;

// What a tiled block works on.
struct TiledBlock {
  int e, row0, nrows, band, nb;
  int K, S;            // reduction length and its K steps
  int j;               // this wave's unit within the expert
  bool has_unit;       // the last band of units may be partial
  const uint8_t* rec;  // this wave's unit records
};

// GEMM2 epilogue, tiled path.  The accumulator layout gives each lane 4
// columns of 16 rows, so a direct store or atomic would touch 16 rows x 4
// column groups per instruction.  Instead each wave stages 32 rows of its 64
// columns in LDS (the token buffers, free after the K loop) and reads them
// back row-major: a (bf16) y store then writes 8 whole 128-byte row
// segments per instruction, an atomic (w * y into out_acc) one whole 256-byte
// row segment.
// Called by every wave of the block (barriers).
template <int FMV>
__device__ __forceinline__ void tiled_g2_staged(const FwdParams& p, TiledShared<kTiledRows>& sh,
                                                const f32x4 (&acc)[kUnitFrags][FMV], int row0, int nrows,
                                                int n0, const float (&ginv)[FMV], float wginv, bool has_unit,
                                                int wave, int lane) {
  static_assert(kTiledWaves * 32 * kAtomicPitch * 4 <= sizeof(TiledShared<kTiledRows>::lds),
                "staging fits the token buffers");
  const int t = threadIdx.x, g = lane >> 4, r16 = lane & 15;
  wait_vmcnt<0>();  // this wave's last copies have landed
  // every wave is done with the token buffers; for the atomics each row's
  // token and weight replace the copy sources and the (unused) amax partials
  lds_barrier();
  if (!p.deterministic) {
    if (t < kTiledRows) {
      const int sl = t < nrows ? sh.slot[t] : 0;
      sh.src[t] = t < nrows ? slot_token(p, sl) : 0;
      sh.amax[0][t] = t < nrows ? slot_weight(p, sl) : 0.0f;
    }
    lds_barrier();
  }
  if (!has_unit) return;
  float* st = reinterpret_cast<float*>(&sh.lds[0][0]) + wave * 32 * kAtomicPitch;
  const int H = p.H;
#pragma unroll
  for (int r = 0; r < FMV; r += 2) {
    // rows 16 r .. 16 r + 31 of the tile, scaled by their alphas
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (r + h < FMV) {
        const float alpha = ginv[r + h] * wginv;
#pragma unroll
        for (int f = 0; f < kUnitFrags; ++f) {
          const f32x4 v = acc[f][r + h];
          *reinterpret_cast<float4*>(st + (16 * h + r16) * kAtomicPitch + 16 * f + 4 * g) =
              make_float4(v[0] * alpha, v[1] * alpha, v[2] * alpha, v[3] * alpha);
        }
      }
    }
    const int nr = min(32, nrows - 16 * r);
    if (p.deterministic) {
      // lane l: row 8 i + l / 8, columns 8 (l % 8) .. + 7 (one 16-byte bf16
      // store; eight 128-byte row segments per instruction)
      for (int i = 0; 8 * i < nr; ++i) {
        const int m = 8 * i + (lane >> 3);
        if (m < nr) {
          const float* src = st + m * kAtomicPitch + 8 * (lane & 7);
          const float4 a = *reinterpret_cast<const float4*>(src);
          const float4 c = *reinterpret_cast<const float4*>(src + 4);
          const uint2 lo = pack_bf16x4(a.x, a.y, a.z, a.w), hi = pack_bf16x4(c.x, c.y, c.z, c.w);
          // y by slot (see g2_epilogue)
          *reinterpret_cast<uint4*>(p.y + static_cast<int64_t>(sh.slot[16 * r + m]) * H + n0 + 8 * (lane & 7)) =
              make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
      }
    } else {
      for (int m = 0; m < nr; ++m) {
        const int lm = 16 * r + m;
        const float v = st[m * kAtomicPitch + lane];
        atomicAdd(p.out_acc + static_cast<int64_t>(sh.src[lm]) * H + n0 + lane, sh.amax[0][lm] * v);
      }
    }
  }
}

// One tile whose rows fit in FMV 16-row groups: the copies, MFMAs and
// epilogue cover only those groups, so a tile of few rows costs in
// proportion to its rows (FMV is the smallest of 1, 2, 3, 4, 6, 8 groups
// that holds them).
template <int FMV, int MODE, bool A16, int TR>
__device__ __forceinline__ void tiled_tile(const FwdParams& p, TiledShared<TR>& sh, const TiledBlock& b,
                                           UnitStep (&wb)[2], float my_g, int my_slot, float wg) {
  static_assert(16 * FMV <= TR, "the tile's groups fit the block's buffers");
  static_assert(MODE == 0 || TR == kTiledRows, "GEMM2's epilogue stages through the 128-row buffers");
  constexpr bool kNT = TR == kTiledSmallRows;  // 16-row tiles: one tile per expert, records read once
  constexpr int NCP = FMV * 16 * 16 / kWave / kTiledWaves;  // copy instructions per wave and step
  const int row0 = b.row0, nrows = b.nrows, K = b.K, S = b.S, j = b.j;
  const bool has_unit = b.has_unit;
  const uint8_t* rec = b.rec;
  // token operand: GEMM1 gathers rows of xq16 [T, K] (W4A16: of x itself);
  // GEMM2 reads the tile's own rows of a2q16 [Rt, K] (offsets relative to
  // the tile's first row)
  const _Float16* x16 = A16 ? reinterpret_cast<const _Float16*>(p.x) : p.xq16;
  const __amdgpu_buffer_rsrc_t a16 =
      MODE == 0 ? tiled_rsrc(x16, static_cast<int64_t>(p.T) * K)
                : tiled_rsrc(p.a2q16 + static_cast<int64_t>(row0) * K, static_cast<int64_t>(nrows) * K);
  const int t = threadIdx.x;
  const int wave = t / kWave, lane = t & (kWave - 1);
  const int g = lane >> 4, r16 = lane & 15;
  uint8_t* lds0 = sh.lds[0];
  uint8_t* lds1 = sh.lds[1];

  // this wave's copies: instruction u fills chunk c = wave + 4 u, i.e.
  // (fm, g) = (c / 4, c % 4); lane l brings bytes 64 g + 16 (l / 16) .. + 15
  // of the step's segment of tile row 16 fm + l % 16
  int coff[NCP];
#pragma unroll
  for (int u = 0; u < NCP; ++u) {
    const int c = wave + kTiledWaves * u;
    const int r = 16 * (c >> 2) + (lane & 15);
    // byte offset; rows past nrows read the first row (never stored)
    const int src = MODE == 0 ? max(sh.src[r], 0) : (r < nrows ? r : 0);
    coff[u] = 2 * src * K + 64 * (c & 3) + 16 * (lane >> 4);
  }
  tiled_copy_step<NCP>(a16, coff, lds0, 0, wave);
  __builtin_amdgcn_sched_barrier(0);
  // Publish the rows' scales and slots and the expert's weight scale, loaded
  // at the block's start, for the epilogue (the K loop's barriers make the
  // stores visible).  The weight records of the first two steps were issued
  // before everything else; the K loop's waits count one refill newer than
  // the step's copies, so wait here for all of it, the first copies included.
  if (t < TR) {
    sh.ginv[t] = t < nrows ? 1.0f / my_g : 0.0f;
    sh.slot[t] = my_slot;
  }
  if (t == 0) sh.wginv = 1.0f / wg;
  wait_vmcnt<0>();
  __builtin_amdgcn_sched_barrier(0);

  f32x4 acc[kUnitFrags][FMV];
#pragma unroll
  for (int f = 0; f < kUnitFrags; ++f)
#pragma unroll
    for (int fm = 0; fm < FMV; ++fm) acc[f][fm] = f32x4{0.f, 0.f, 0.f, 0.f};

  // straight-line pairs of steps (buffer and register slot fixed per half),
  // so that every wait above counts the same loads on every path
  int s = 0;
  for (; s + 1 < S; s += 2) {
    tiled_step<FMV, NCP, A16, kNT>(acc, s, S, lds0, lds1, wb[0], rec, a16, coff, has_unit, wave, lane);
    tiled_step<FMV, NCP, A16, kNT>(acc, s + 1, S, lds1, lds0, wb[1], rec, a16, coff, has_unit, wave, lane);
  }
  if (s < S) tiled_step<FMV, NCP, A16, kNT>(acc, s, S, lds0, lds1, wb[0], rec, a16, coff, has_unit, wave, lane);

  float ginv[FMV];
  int slots[FMV];
  const float wginv = sh.wginv;
#pragma unroll
  for (int fm = 0; fm < FMV; ++fm) {
    ginv[fm] = sh.ginv[fm * 16 + r16];
    slots[fm] = sh.slot[fm * 16 + r16];
  }
  if constexpr (MODE == 0) {
    if (has_unit) {
      // (W4A16 with 128-row tiles: the tiled GEMM2 reads the bf16 copy)
      g1_epilogue<FMV, 2, TR, A16 && TR == kTiledRows>(p, acc, b.e, row0, nrows, 32 * j, ginv, sh.amax, wave, g,
                                                      r16, wginv);
    } else if (g == 0) {
#pragma unroll
      for (int fm = 0; fm < FMV; ++fm) sh.amax[wave][fm * 16 + r16] = 0.0f;
    }
    g1_store_band_amax<TR>(p, sh.amax, row0, nrows, b.band, b.nb);
  } else {
    tiled_g2_staged<FMV>(p, sh, acc, row0, nrows, 64 * j, ginv, wginv, has_unit, wave, lane);
  }
}

// TR: the most rows a tile of this launch has (kTiledRows, or kTiledSmallRows
// when the tile list was built with 16-row tiles: two blocks per CU, or four).
template <int MODE, bool A16, int TR = kTiledRows>
__global__ __launch_bounds__(kTiledThreads)
__attribute__((amdgpu_waves_per_eu(TR == kTiledSmallRows ? 4 : 2, TR == kTiledSmallRows ? 4 : 2)))
void moe_tiled_kernel(FwdParams p) {
  __shared__ TiledShared<TR> sh;
  // XCD-aware order: consecutive blocks go to the 8 XCDs in turn, so block L
  // runs on XCD L % 8 as that XCD's (L / 8)-th block.  Tiles are dealt to
  // the XCDs in turn (tile t to XCD t % 8) and each XCD runs a tile's bands
  // in a row: the bands share the tile's token rows in that XCD's L2, while
  // the tiles of one hot expert spread over every XCD's path to HBM
  // (measured on the large layer at 2048 tokens: 2.33 -> 2.11 ms against
  // giving each XCD a contiguous eighth of the tile list; prefill unchanged).
  const int nb = gridDim.x / p.tiled_gx;  // bands per tile
  const int L = blockIdx.x, slot = L >> 3;
  const int ntiles = *p.n_tiles;
  const int band = slot % nb, local = slot / nb;
  const int tile = local * 8 + (L & 7);
  if (tile >= ntiles) return;
  const int4 td = p.tiles[tile];
  TiledBlock b;
  b.e = td.x;
  b.row0 = td.y;
  b.nrows = td.z;
  b.band = band;
  b.nb = nb;
  b.K = MODE == 0 ? p.H : p.I;
  b.S = ksteps(b.K);
  const int t = threadIdx.x, wave = t / kWave, lane = t & (kWave - 1);
  const int upe = MODE == 0 ? p.I / 32 : p.H / 64;
  b.j = band * kTiledWaves + wave;
  b.has_unit = b.j < upe;
  b.rec = (MODE == 0 ? p.w13 : p.w2) +
          (static_cast<int64_t>(b.e) * upe + (b.has_unit ? b.j : 0)) * b.S * kRecBytes;

  // Start-up, shortest dependency chains first: the first two steps' weight
  // records need only the tile; GEMM1's token copies need the permutation
  // (the rows' source tokens go to LDS for the copy offsets), GEMM2's need
  // nothing more.  The rows' global scales and slots are loaded here and
  // published by tiled_tile.
  UnitStep wb[2];
  constexpr bool kNT = TR == kTiledSmallRows;  // (as in tiled_tile)
  load_unit_step<kNT>(wb[0], b.rec, lane);
  load_unit_step<kNT>(wb[1], b.rec + static_cast<int64_t>(min(1, b.S - 1)) * kRecBytes, lane);
  float my_g = 1.0f;
  int my_slot = -1;
  // (W4A16: the activations carry no global scale)
  if (MODE == 0) {
    int src = -1;
    if (t < b.nrows) {
      my_slot = row_slot(p, b.row0 + t);
      src = slot_token(p, my_slot);
      if (!A16) my_g = p.xq_g[src];
    }
    if (t < TR) sh.src[t] = src;
    lds_barrier();
  } else if (t < b.nrows) {
    if (!A16) my_g = p.a2_g[b.row0 + t];
    my_slot = row_slot(p, b.row0 + t);
  }
  const float wg = MODE == 0 ? p.w13g[b.e] : p.w2g[b.e];
  if constexpr (TR == kTiledSmallRows) {
    tiled_tile<1, MODE, A16, TR>(p, sh, b, wb, my_g, my_slot, wg);
  } else {
    const int groups = (b.nrows + 15) >> 4;
    if (groups > 6)
      tiled_tile<8, MODE, A16, TR>(p, sh, b, wb, my_g, my_slot, wg);
    else if (groups > 4)
      tiled_tile<6, MODE, A16, TR>(p, sh, b, wb, my_g, my_slot, wg);
    else if (groups > 3)
      tiled_tile<4, MODE, A16, TR>(p, sh, b, wb, my_g, my_slot, wg);
    else if (groups > 2)
      tiled_tile<3, MODE, A16, TR>(p, sh, b, wb, my_g, my_slot, wg);
    else if (groups > 1)
      tiled_tile<2, MODE, A16, TR>(p, sh, b, wb, my_g, my_slot, wg);
    else
      tiled_tile<1, MODE, A16, TR>(p, sh, b, wb, my_g, my_slot, wg);
  }
}

// ---------------------------------------------------------------------------
// Re-quantization of every expanded row for the tiled path: one wave per row
// reads its act row (I binary32 values), takes the row amax over the GEMM1
// band partials, and quantizes 16-element blocks (lane b handles blocks b,
// b + 64, ...); it also writes the dequantized fp16 copy GEMM2 reads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void moe_requant_kernel(FwdParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (row >= p.Rt) return;
  const int I = p.I;
  float a = 0.0f;
  for (int j = lane; j < p.g1_bands; j += kWave) a = fmaxf(a, p.act_amax[row * p.g1_bands + j]);
  const float g2 = p.static_g ? p.static_g[1] : global_scale(wave_max(a));
  if (lane == 0) p.a2_g[row] = g2;
  for (int b = lane; b < I / 16; b += kWave) {
    uint32_t lo, hi;
    const uint32_t sb = requant_block(p.act + row * I + 16 * b, g2, lo, hi);
    *reinterpret_cast<uint2*>(p.a2_codes + row * (I / 2) + 8 * b) = make_uint2(lo, hi);
    p.a2_scales[row * (I / 16) + b] = static_cast<uint8_t>(sb);
    if (p.a2q16) {
      const half2v sc = e4m3_to_half2(sb);
      half8* d = reinterpret_cast<half8*>(p.a2q16 + row * I + 16 * b);
      d[0] = dequant8_f16(lo, sc);
      d[1] = dequant8_f16(hi, sc);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

int stream_lds_bytes(int fm, int K) { return 16 * fm * ((K / 2 + 16) + (K / 16 + 4)); }

// W4A16 stream kernels stage bf16 rows; up to this much dynamic LDS per block
// (two blocks per CU on gfx950).
constexpr int kStreamA16MaxLds = 80 * 1024;

static int stream_lds_total(int fm, int ks, int K, bool atomic = false, bool a16 = false) {
  const int staged = a16 ? 16 * fm * (2 * K + 16) : stream_lds_bytes(fm, K);
  const int red = ks > 1 ? 4 * kUnitFrags * fm * 4 * kWave * 4 : 0;
  // atomic GEMM2 epilogue: each unit's rows at kAtomicPitch floats
  const int stage = atomic ? (4 / ks) * 16 * fm * kAtomicPitch * 4 : 0;
  return std::max(staged, std::max(red, stage));
}

// Waves that split one unit's K range: the smallest of 1, 2, 4 that gives the
// launch at least 8 waves per CU (two per SIMD) over the units that can be
// active, while the block's units still divide the expert's.
static int choose_ks(int64_t units, int upe, int S) {
  const int64_t want = 8 * 256;
  for (int ks : {1, 2}) {
    if ((upe % (4 / ks)) == 0 && units * ks >= want && S >= 2 * ks) return ks;
  }
  return 4;
}

// Kernel family, rows per tile and the K split for a forward of T tokens.
void choose_gemm(int64_t T, FwdParams* p) {
  const int H = p->H, I = p->I, E = p->E;
  const int64_t R = T * p->k;
  const int64_t active = R < E ? R : E;
  const int64_t avg = (R + active - 1) / (active > 0 ? active : 1);
  const int Kmax = H > I ? H : I;
  if (p->a16) {
    // W4A16 with few rows per expert: 16-row tiles, GEMM1 on the tiled
    // kernel and GEMM2 streamed with its rows staged as bf16 (16 rows of
    // 2 I bytes must fit); otherwise the tiled GEMMs with 128-row tiles
    if (avg <= 16 && stream_lds_total(1, 4, I, true, true) <= kStreamA16MaxLds) {
      p->mt = 16;
      p->gemm_kind = kGemmStream;
    } else {
      p->mt = kTiledRows;
      p->gemm_kind = kGemmTiled;
    }
  } else if (avg <= 16 && stream_lds_total(1, 4, Kmax) <= 65536) {
    p->mt = 16;
    p->gemm_kind = kGemmStream;
  } else if (avg <= 32 && stream_lds_total(2, 4, Kmax) <= 65536) {
    p->mt = 32;
    p->gemm_kind = kGemmStream;
  } else {
    // prefill: 128-row tiles; a tile of fewer rows computes only the 16-row
    // groups it needs
    p->mt = kTiledRows;
    p->gemm_kind = kGemmTiled;
  }
  if (p->gemm_kind == kGemmStream) {
    const int64_t tiles = (R + p->mt - 1) / p->mt > active ? (R + p->mt - 1) / p->mt : active;
    p->g1_ks = p->a16 ? 1 : choose_ks(tiles * (I / 32), I / 32, ksteps(H));  // (W4A16: GEMM1 tiled)
    // GEMM2 re-quantizes its tile's rows in every block, so splitting K
    // (more blocks per tile) costs more than the extra parallelism gains
    p->g2_ks = (H / 64) % 4 == 0 ? 1 : (H / 64) % 2 == 0 ? 2 : 4;
    p->g1_bands = (I / 32) / (4 / p->g1_ks);
  } else {
    p->g1_ks = p->g2_ks = 1;
    p->g1_bands = (I / 32 + kTiledWaves - 1) / kTiledWaves;
  }
}

template <int FM, int KS1, int KS2, bool A16>
static void launch_stream(const FwdParams& p, int max_tiles, hipStream_t s, hipEvent_t const* ev) {
  if constexpr (A16) {
    // W4A16: GEMM1 on the tiled kernel (16-row tiles: its 1-group variant,
    // sized for them, four blocks per CU; measured faster than bf16 staging
    // in the stream kernel, whose bf16 weight dequantization costs about
    // twice the fp16 one's VALU)
    static_assert(FM * 16 <= kTiledSmallRows, "the stream path's tiles fit the small tiled blocks");
    const int nbt = (p.I / 32 + kTiledWaves - 1) / kTiledWaves;
    moe_tiled_kernel<0, true, kTiledSmallRows><<<p.tiled_gx * nbt, kTiledThreads, 0, s>>>(p);
    // GEMM2's bf16 staging may take more than the default 64 KB of dynamic
    // LDS.  The attribute belongs to the current device: set once per device
    // (devices past the mask's 64 set it on every call).
    static std::atomic<uint64_t> lds_set{0};
    int dev = 0;
    (void)hipGetDevice(&dev);
    const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t{1} << dev : 0;
    if (bit == 0 || (lds_set.load(std::memory_order_relaxed) & bit) == 0) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_stream_kernel<FM, KS2, 1, A16>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kStreamA16MaxLds);
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_stream_kernel<FM, KS2, 1, A16, true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kStreamA16MaxLds);
      lds_set.fetch_or(bit, std::memory_order_relaxed);
    }
  } else {
    // GEMM1's grid takes the tightest bound on the batch's tiles: at most
    // n = min(E, R) experts have rows, and an expert with c rows has
    // ceil(c / mt) <= 1 + (c - 1) / mt tiles, so at most n + (R - n) / mt
    // (plus the shared expert's).  Blocks past the last tile exit at once but
    // still take a slot when dispatched: at one token on the large layer the
    // looser bound (9 tile columns for 8 tiles) left 8 GEMM1 blocks per XCD
    // waiting for the first ones to end.
    const int64_t nact = std::min<int64_t>(p.E, p.R);
    const int64_t tight = nact + (p.R - nact) / p.mt + (p.shared ? (p.T + p.mt - 1) / p.mt : 0);
    const int gx1 = static_cast<int>(std::min<int64_t>(tight, max_tiles));
    const int nb1 = (p.I / 32) / (4 / KS1);
    moe_stream_kernel<FM, KS1, 0, false><<<dim3(gx1, nb1), 256, stream_lds_total(FM, KS1, p.H), s>>>(p);
  }
  if (ev) (void)hipEventRecord(ev[2], s);
  const int nb2 = (p.H / 64) / (4 / KS2);
  // Consecutive blocks go to the 8 XCDs in turn; with max_tiles columns (not
  // a multiple of 8) the bands of one tile land on different XCDs, so each
  // expert's W2 stream is spread over all XCDs (measured on the large layer
  // at one token: GEMM2 25.0 -> 18.4 us against all bands of a tile on one
  // XCD); the tile's act rows, re-read by every band, come from the last
  // level cache.
  const int lds2 = stream_lds_total(FM, KS2, p.I, !p.deterministic, A16);
  if (KS2 == 1 && ksteps(p.I) <= kStreamShortSteps)
    moe_stream_kernel<FM, KS2, 1, A16, true><<<dim3(max_tiles, nb2), 256, lds2, s>>>(p);
  else
    moe_stream_kernel<FM, KS2, 1, A16><<<dim3(max_tiles, nb2), 256, lds2, s>>>(p);
  if (ev) (void)hipEventRecord(ev[3], s);
}

template <int FM, int KS1, bool A16>
static void launch_stream_ks2(const FwdParams& p, int max_tiles, hipStream_t s, hipEvent_t const* ev) {
  if (p.g2_ks == 1) launch_stream<FM, KS1, 1, A16>(p, max_tiles, s, ev);
  else if (p.g2_ks == 2) launch_stream<FM, KS1, 2, A16>(p, max_tiles, s, ev);
  else launch_stream<FM, KS1, 4, A16>(p, max_tiles, s, ev);
}

template <int FM, bool A16>
static void launch_stream_fm(const FwdParams& p, int max_tiles, hipStream_t s, hipEvent_t const* ev) {
  if (p.g1_ks == 1) launch_stream_ks2<FM, 1, A16>(p, max_tiles, s, ev);
  else if (p.g1_ks == 2) launch_stream_ks2<FM, 2, A16>(p, max_tiles, s, ev);
  else launch_stream_ks2<FM, 4, A16>(p, max_tiles, s, ev);
}

hipError_t launch_grouped_gemms(const FwdParams& p, int max_tiles, hipStream_t s,
                                hipEvent_t const* ev) {
  if (p.gemm_kind == kGemmStream) {
    if (p.a16)
      launch_stream_fm<1, true>(p, max_tiles, s, ev);
    else if (p.mt == 16)
      launch_stream_fm<1, false>(p, max_tiles, s, ev);
    else
      launch_stream_fm<2, false>(p, max_tiles, s, ev);
  } else {
    const int nb1 = (p.I / 32 + kTiledWaves - 1) / kTiledWaves;
    const int nb2 = (p.H / 64 + kTiledWaves - 1) / kTiledWaves;
    // a multiple of 8 tiles keeps every band of a tile on the same XCD (its
    // token rows are then fetched into one L2)
    const int gx = (max_tiles + 7) / 8 * 8;  // == p.tiled_gx
    if (p.a16) {
      // (GEMM1's epilogue also writes GEMM2's bf16 input)
      moe_tiled_kernel<0, true><<<gx * nb1, kTiledThreads, 0, s>>>(p);
      if (ev) (void)hipEventRecord(ev[2], s);
      moe_tiled_kernel<1, true><<<gx * nb2, kTiledThreads, 0, s>>>(p);
    } else {
      moe_tiled_kernel<0, false><<<gx * nb1, kTiledThreads, 0, s>>>(p);
      if (ev) (void)hipEventRecord(ev[2], s);
      moe_requant_kernel<<<(p.Rt + 3) / 4, 256, 0, s>>>(p);
      moe_tiled_kernel<1, false><<<gx * nb2, kTiledThreads, 0, s>>>(p);
    }
    if (ev) (void)hipEventRecord(ev[3], s);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
