// Per-token NVFP4 quantization of bf16 activations and per-expert NVFP4
// quantization of weights (gfx950).
//
// [P1] (sglang PR #28354 summary), "Feature and motivation": a dynamic,
// per-token binary32 global scale; "Implementation breakdown" item 2: the
// activations are quantized to FP4 codes plus block scales before the expert
// GEMMs; "Review highlights": 16 elements per scale.
//
// Layout of the work: one wave per row.  Lane l owns the 16-element blocks
// l, l+64, l+128, ...: each block is two 16-byte loads of bf16, so one wave
// instruction reads 2 KB of contiguous row, and each lane writes its block's
// 8 code bytes with one 8-byte store.  The block amax is lane-local (a lane
// holds whole blocks); the row amax is one wave reduction (plus one LDS
// exchange when a block of four waves shares a row).  With the row's blocks
// cached in registers it is read from HBM once.
#include "common.hpp"
#include "kernels.hpp"
#include "quant_row.hpp"

namespace nvfp4 {


// Rows of up to 2048 blocks (cols <= 32768): one block of 256 threads per
// row, thread t owning blocks t, t + 256, ... (NBL of them) in registers.
// Small per-thread register caches keep eight waves per SIMD resident, so
// many rows' loads are in flight while others quantize; the row amax takes
// one LDS exchange between the block's four waves.
template <int NBL>
__global__ __launch_bounds__(256) void quantize_rows_block_kernel(const uint16_t* __restrict__ x,
                                                                  int64_t rows, int cols, int64_t ld,
                                                                  uint8_t* __restrict__ codes,
                                                                  uint8_t* __restrict__ scales,
                                                                  float* __restrict__ gs) {
  __shared__ float s_am[4];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int nblk = cols / 16;
  const uint16_t* xrow = x + row * ld;
  uint4 v[NBL][2];
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    const uint4* p = reinterpret_cast<const uint4*>(xrow + 16 * min(t + 256 * i, nblk - 1));
    v[i][0] = load_stream16(p);
    v[i][1] = load_stream16(p + 1);
  }
  float bam[NBL];
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    bam[i] = amax16_bf16(v[i][0], v[i][1]);
    if (t + 256 * i < nblk) am = fmaxf(am, bam[i]);
  }
  am = wave_max(am);
  if (lane == 0) s_am[wave] = am;
  __syncthreads();
  const float g = global_scale(fmaxf(fmaxf(s_am[0], s_am[1]), fmaxf(s_am[2], s_am[3])));
  uint8_t* crow = codes + row * (cols / 2);
  uint8_t* srow = scales + row * (cols / 16);
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    const int b = t + 256 * i;
    if (b < nblk) {
      float f[16];
      unpack16(v[i][0], v[i][1], f);
      uint32_t lo, hi;
      const uint32_t sb = quantize_block16_amax(f, bam[i], g, lo, hi);
      // streaming stores: the outputs are not re-read by this kernel
      const u32x2 cv = {lo, hi};
      __builtin_nontemporal_store(cv, reinterpret_cast<u32x2*>(crow + 8 * b));
      __builtin_nontemporal_store(static_cast<uint8_t>(sb), srow + b);
    }
  }
  if (t == 0) gs[row] = g;
}

// Rows of up to 2048 half-blocks (cols <= 16384): one block of 256 threads per
// row, thread t owning the 8-element halves t, t + 256, ... (NH of them) of
// the row's 16-element blocks.  Each wave instruction then reads 1 KB of
// contiguous row and writes 256 contiguous code bytes; a block's two halves
// sit in lanes 2i and 2i + 1, which exchange their half amaxes (one lane
// swap) and both derive the same block scale.  The even lane writes it.
template <int NH>
__global__ __launch_bounds__(256) void quantize_rows_pair_kernel(const uint16_t* __restrict__ x,
                                                                 int64_t rows, int cols, int64_t ld,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales,
                                                                 float* __restrict__ gs) {
  __shared__ float s_am[4];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int nhalf = cols / 8;
  const uint16_t* xrow = x + row * ld;
  uint4 v[NH];
#pragma unroll
  for (int i = 0; i < NH; ++i) v[i] = load_stream16(xrow + 8 * min(t + 256 * i, nhalf - 1));
  // half amaxes (|x| of finite bf16 orders like its low 15 bits), block
  // amaxes from the partner lane, row amax over the valid halves
  float bam[NH];
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < NH; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    const float ha = __uint_as_float(m << 16);
    bam[i] = fmaxf(ha, __shfl_xor(ha, 1, kWave));
    if (t + 256 * i < nhalf) am = fmaxf(am, ha);
  }
  am = wave_max(am);
  if (lane == 0) s_am[wave] = am;
  __syncthreads();
  const float g = global_scale(fmaxf(fmaxf(s_am[0], s_am[1]), fmaxf(s_am[2], s_am[3])));
  uint8_t* crow = codes + row * (cols / 2);
  uint8_t* srow = scales + row * (cols / 16);
#pragma unroll
  for (int i = 0; i < NH; ++i) {
    const int h = t + 256 * i;
    if (h < nhalf) {
      const float sg = div6_rn(bam[i] * g);
      const uint32_t sb = e4m3_encode(sg);
      const float d = e4m3_value(sb);
      const float r = d > 0.0f ? div_e4m3_rn(g, d) : 0.0f;
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      float f[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[2 * j] = __builtin_amdgcn_fmed3f(bf16_lo(w[j]) * r, -6.0f, 6.0f);
        f[2 * j + 1] = __builtin_amdgcn_fmed3f(bf16_hi(w[j]) * r, -6.0f, 6.0f);
      }
      // streaming stores: the outputs are not re-read by this kernel
      __builtin_nontemporal_store(e2m1_pack8(f), reinterpret_cast<uint32_t*>(crow + 4 * h));
      if (!(h & 1)) __builtin_nontemporal_store(static_cast<uint8_t>(sb), srow + h / 2);
    }
  }
  if (t == 0) gs[row] = g;
}

// Longer rows: one wave per row, two passes over the row.
__global__ __launch_bounds__(256) void quantize_rows_long_kernel(const uint16_t* __restrict__ x,
                                                                 int64_t rows, int cols, int64_t ld,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales,
                                                                 float* __restrict__ gs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (row >= rows) return;
  quantize_row_wave<0>(x + row * ld, cols / 16, codes + row * (cols / 2), scales + row * (cols / 16),
                       gs + row, lane);
}

int quant_nb_for_cols(int64_t cols) {
  const int64_t nblk = cols / 16;
  if (nblk <= 64) return 1;
  if (nblk <= 128) return 2;
  if (nblk <= 256) return 4;
  if (nblk <= 512) return 8;
  return 0;
}

hipError_t launch_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                uint8_t* codes, uint8_t* scales, float* gs, hipStream_t s) {
  const int64_t nbl = (cols / 16 + 255) / 256;
  const unsigned grid = static_cast<unsigned>(rows);
  const int c = static_cast<int>(cols);
  switch ((cols / 8 + 255) / 256) {
    case 1: quantize_rows_pair_kernel<1><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); return hipGetLastError();
    case 2: quantize_rows_pair_kernel<2><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); return hipGetLastError();
    case 3: quantize_rows_pair_kernel<3><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); return hipGetLastError();
    case 4: quantize_rows_pair_kernel<4><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); return hipGetLastError();
    case 5: quantize_rows_pair_kernel<5><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); return hipGetLastError();
    case 6: quantize_rows_pair_kernel<6><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); return hipGetLastError();
    case 7: quantize_rows_pair_kernel<7><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); return hipGetLastError();
    case 8: quantize_rows_pair_kernel<8><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); return hipGetLastError();
    default: break;
  }
  switch (nbl) {
    case 1: quantize_rows_block_kernel<1><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); break;
    case 2: quantize_rows_block_kernel<2><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); break;
    case 3: quantize_rows_block_kernel<3><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); break;
    case 4: quantize_rows_block_kernel<4><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); break;
    case 5: quantize_rows_block_kernel<5><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); break;
    case 6: quantize_rows_block_kernel<6><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); break;
    case 7: quantize_rows_block_kernel<7><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); break;
    case 8: quantize_rows_block_kernel<8><<<grid, 256, 0, s>>>(x, rows, c, ld, codes, scales, gs); break;
    default:
      quantize_rows_long_kernel<<<static_cast<unsigned>((rows + 3) / 4), 256, 0, s>>>(x, rows, c, ld, codes,
                                                                                     scales, gs);
      break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weights: one global scale per expert from the amax of the whole expert
// tensor (the per-expert factors w1_alpha / w2_alpha of [P1] "Source
// snippets" undo it), blocks along the last dimension.
// ---------------------------------------------------------------------------

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// grid (chunks, experts): each block reduces a chunk of one expert's values.
__global__ __launch_bounds__(256) void expert_amax_kernel(const float* __restrict__ w,
                                                          int64_t per_expert,
                                                          uint32_t* __restrict__ amax_bits) {
  const int e = blockIdx.y;
  const float4* base = reinterpret_cast<const float4*>(w + static_cast<int64_t>(e) * per_expert);
  const int64_t n4 = per_expert / 4;
  float m = 0.0f;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float4 v = base[i];
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  m = wave_max(m);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    atomicMax(amax_bits + e, __float_as_uint(b));  // non-negative floats order like their bits
  }
}

// One wave per row of one expert; the global scale comes from the expert amax.
__global__ __launch_bounds__(256) void quantize_expert_rows_kernel(
    const float* __restrict__ w, int64_t experts, int64_t rows, int cols,
    const uint32_t* __restrict__ amax_bits, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ gs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t grow = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (grow >= experts * rows) return;
  const int64_t e = grow / rows;
  const float g = global_scale(__uint_as_float(amax_bits[e]));
  if (grow % rows == 0 && lane == 0) gs[e] = g;
  const float* xr = w + grow * cols;
  uint8_t* crow = codes + grow * (cols / 2);
  uint8_t* srow = scales + grow * (cols / 16);
  for (int b = lane; b < cols / 16; b += kWave) {
    const float4* p = reinterpret_cast<const float4*>(xr + 16 * b);
    float f[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 v = p[q];
      f[4 * q] = v.x; f[4 * q + 1] = v.y; f[4 * q + 2] = v.z; f[4 * q + 3] = v.w;
    }
    uint32_t lo, hi;
    const uint32_t sb = quantize_block16(f, g, lo, hi);
    *reinterpret_cast<uint2*>(crow + 8 * b) = make_uint2(lo, hi);
    srow[b] = static_cast<uint8_t>(sb);
  }
}

hipError_t launch_quantize_experts(const float* w, int64_t experts, int64_t rows, int64_t cols,
                                   uint8_t* codes, uint8_t* scales, float* gs, uint32_t* amax_bits,
                                   hipStream_t s) {
  fill_u32_kernel<<<static_cast<unsigned>((experts + 255) / 256), 256, 0, s>>>(amax_bits, experts, 0u);
  const int64_t per_expert = rows * cols;
  int64_t chunks = (per_expert / 4 + 256 * 16 - 1) / (256 * 16);
  if (chunks > 1024) chunks = 1024;
  if (chunks < 1) chunks = 1;
  expert_amax_kernel<<<dim3(static_cast<unsigned>(chunks), static_cast<unsigned>(experts)), 256, 0, s>>>(
      w, per_expert, amax_bits);
  const int64_t total_rows = experts * rows;
  quantize_expert_rows_kernel<<<static_cast<unsigned>((total_rows + 3) / 4), 256, 0, s>>>(
      w, experts, rows, static_cast<int>(cols), amax_bits, codes, scales, gs);
  return hipGetLastError();
}

}  // namespace nvfp4

namespace nvfp4 {

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  fill_u32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace nvfp4
