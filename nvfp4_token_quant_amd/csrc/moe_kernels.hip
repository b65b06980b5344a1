// NVFP4 fused-MoE forward on gfx950: prologue (quantize + route + permute),
// grouped GEMM1 with SwiGLU, grouped GEMM2 with the re-quantization fused into
// its operand staging, and the weighted finalize.
//
// Steps follow the MoE runner of [P3] (sglang PR #36624 summary), "Feature and
// motivation": routing, expandInputRows and activation / finalize around the
// expert GEMMs; the per-token activation quantization and the per-token scale
// handed to the expert GEMMs follow [P1] (sglang PR #28354 summary),
// "Implementation breakdown" item 2.
//
// MFMA operand choice.  NVFP4 scales are E4M3 per 16 elements; gfx950's
// scaled FP4 MFMA takes power-of-two (E8M0) scales per 32 elements, so it
// cannot carry them.  Instead each E2M1 code times its E4M3 block scale is
// formed exactly in fp16 (<= 6 significant bits, magnitudes in [2^-10, 2688])
// and fed to v_mfma_f32_16x16x32_f16 with fp32 accumulation; the binary32
// global scales are applied once in the epilogue.
//
// Operand roles: the weight rows are MFMA operand A (16 output columns n x 32
// k per fragment), the token rows are operand B (32 k x 16 rows m).  Each lane
// loads 16 bytes (32 codes) of one weight row per 128-wide K step; the four
// MFMAs of that step use the lane's 8-code pieces q = 0..3, and the token
// operand is read from LDS with the same k assignment (lane group g holds
// k = 32g + 8q + i), so the reduction covers every k once.
#include "common.hpp"
#include "kernels.hpp"
#include "quant_row.hpp"

namespace nvfp4 {

// ---------------------------------------------------------------------------
// Router: the k largest logits of one token, ties to the smaller expert
// index, slots in descending order; weights = exp(l_j - l_0) normalized over
// the k slots (the softmax over all experts restricted to the chosen k).
// One wave per token; lane l holds experts l, l+64, ...
// ---------------------------------------------------------------------------
__device__ void route_token_wave(const float* __restrict__ lrow, int E, int k,
                                 int32_t* __restrict__ ids_out, float* __restrict__ w_out,
                                 int32_t* __restrict__ lds_ids, int lane) {
  constexpr int kPerLane = kMaxExperts / kWave;
  float v[kPerLane];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = lane + kWave * i;
    v[i] = 0.0f;
    if (e < E) {
      v[i] = lrow[e];
      avail |= 1u << i;
    }
  }
  int my_id = 0;
  float my_v = 0.0f, top = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      if ((avail >> i) & 1u) {
        if (bi == 0x7FFFFFFF || v[i] > bv) {  // ascending index: ties keep the smaller one
          bv = v[i];
          bi = lane + kWave * i;
        }
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      const bool take = (oi != 0x7FFFFFFF) &&
                        (bi == 0x7FFFFFFF || ov > bv || (ov == bv && oi < bi));
      bv = take ? ov : bv;
      bi = take ? oi : bi;
    }
    if ((bi & (kWave - 1)) == lane) avail &= ~(1u << (bi / kWave));
    if (lane == j) {
      my_id = bi;
      my_v = bv;
    }
    if (j == 0) top = bv;
  }
  const float ex = lane < k ? expf(my_v - top) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids_out[lane] = my_id;
    w_out[lane] = ex / sum;
    lds_ids[lane] = my_id;
  }
}

// ---------------------------------------------------------------------------
// Prologue.  Each block takes `tpb` consecutive tokens; each wave quantizes
// and routes tokens of the block, then the block computes, for every (t, j),
// its rank among equal experts inside the block and the block's per-expert
// counts.  The last block to finish (ticket counter; no waiting) turns the
// per-block counts into the stable expandInputRows permutation: rows of one
// expert in ascending (t, j) order, the per-expert offsets and the M-tile list
// of the grouped GEMMs.
// ---------------------------------------------------------------------------
constexpr int kMaxTokensPerBlock = 128;

__device__ void build_schedule_last_block(const FwdParams& p, int nblocks, int tpb) {
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_off[kMaxExperts];
  __shared__ int32_t s_tbase[kMaxExperts];
  __shared__ int32_t s_part[256][2];
  const int tid = threadIdx.x;
  const int E = p.E;
  // 1. per expert: exclusive scan of the per-block counts down the blocks
  for (int e = tid; e < E; e += 256) {
    int run = 0;
    int b = 0;
    for (; b + 8 <= nblocks; b += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = p.blk_counts[(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        p.blk_counts[(b + u) * E + e] = run;
        run += c[u];
      }
    }
    for (; b < nblocks; ++b) {
      const int c = p.blk_counts[b * E + e];
      p.blk_counts[b * E + e] = run;
      run += c;
    }
    s_cnt[e] = run;
    p.counts[e] = run;
  }
  __syncthreads();
  // 2. exclusive scans over experts: row offsets and tile bases
  const int per = (E + 255) / 256;
  int rsum = 0, tsum = 0;
  for (int u = 0; u < per; ++u) {
    const int e = tid * per + u;
    if (e < E) {
      rsum += s_cnt[e];
      tsum += (s_cnt[e] + p.mt - 1) / p.mt;
    }
  }
  s_part[tid][0] = rsum;
  s_part[tid][1] = tsum;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    int a0 = 0, a1 = 0;
    if (tid >= o) {
      a0 = s_part[tid - o][0];
      a1 = s_part[tid - o][1];
    }
    __syncthreads();
    s_part[tid][0] += a0;
    s_part[tid][1] += a1;
    __syncthreads();
  }
  int rbase = s_part[tid][0] - rsum, tbase = s_part[tid][1] - tsum;
  for (int u = 0; u < per; ++u) {
    const int e = tid * per + u;
    if (e < E) {
      s_off[e] = rbase;
      s_tbase[e] = tbase;
      p.offsets[e] = rbase;
      rbase += s_cnt[e];
      tbase += (s_cnt[e] + p.mt - 1) / p.mt;
    }
  }
  if (tid == 255) {
    p.offsets[E] = s_part[255][0];
    *p.n_tiles = s_part[255][1];
  }
  __syncthreads();
  // 3. M-tiles: (expert, first row, rows)
  for (int e = tid; e < E; e += 256) {
    const int c = s_cnt[e];
    const int nt = (c + p.mt - 1) / p.mt;
    for (int i = 0; i < nt; ++i)
      p.tiles[s_tbase[e] + i] = make_int4(e, s_off[e] + i * p.mt, min(p.mt, c - i * p.mt), 0);
  }
  // 4. placement
  for (int i = tid; i < p.R; i += 256) {
    const int t = i / p.k;
    const int b = t / tpb;
    const int e = p.topk_ids[i];
    const int row = s_off[e] + p.blk_counts[b * E + e] + p.loc_rank[i];
    p.perm[row] = i;
    p.inv[i] = row;
  }
  if (tid == 0) *p.ticket = 0u;
}

template <int NB>
__global__ __launch_bounds__(256) void moe_route_kernel(FwdParams p, int tpb) {
  __shared__ int32_t s_ids[kMaxTokensPerBlock * kMaxTopK];
  __shared__ int s_last;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int t0 = blockIdx.x * tpb;
  const int ntok = min(tpb, p.T - t0);
  const int H = p.H, k = p.k;
  for (int lt = wave; lt < ntok; lt += 4) {
    const int64_t t = t0 + lt;
    quantize_row_wave<NB>(p.x + t * H, H / 16, p.xq_codes + t * (H / 2), p.xq_scales + t * (H / 16),
                          p.xq_g + t, lane);
    route_token_wave(p.logits + t * p.E, p.E, k, p.topk_ids + t * k, p.topk_w + t * k,
                     s_ids + lt * k, lane);
    if (!p.deterministic) {
      float4* row = reinterpret_cast<float4*>(p.out_acc + t * H);
      for (int c = lane; c < H / 4; c += kWave) row[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __syncthreads();
  const int nent = ntok * k;
  for (int i = threadIdx.x; i < nent; i += 256) {
    const int e = s_ids[i];
    int r = 0;
    for (int j = 0; j < i; ++j) r += (s_ids[j] == e);
    p.loc_rank[t0 * k + i] = r;
  }
  for (int e = threadIdx.x; e < p.E; e += 256) {
    int c = 0;
    for (int j = 0; j < nent; ++j) c += (s_ids[j] == e);
    p.blk_counts[blockIdx.x * p.E + e] = c;
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(p.ticket, 1u) == gridDim.x - 1) ? 1 : 0;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  build_schedule_last_block(p, gridDim.x, tpb);
}

// ---------------------------------------------------------------------------
// Grouped GEMMs.  One block = one M-tile (up to 16*FM rows of one expert)
// times a band of weight rows; 4 waves, each owning FN fragments of 16 weight
// rows.  The token operand is staged through LDS as exact fp16 in K chunks of
// up to kKC elements; the weight operand streams from HBM straight into
// registers (each weight byte is used by exactly one block per M-tile).
// ---------------------------------------------------------------------------
// K chunk staged per LDS pass: 512 elements for tiles of up to 32 rows, 256
// for 64-row tiles (keeps the staging buffer near 33 KB).
template <int FM>
struct Chunk {
  static constexpr int KC = FM >= 4 ? 256 : 512;
  static constexpr int pitch = KC + 8;  // fp16 elements per LDS row (16-byte pad)
};

// Load the 16-byte code piece and the two block-scale bytes of one weight
// fragment row for one 128-wide K step.  Scales are in the swizzled layout
// [row][g][step][2] (see swizzle_scales_kernel).
__device__ __forceinline__ void load_weight_piece(const uint8_t* __restrict__ wc,
                                                  const uint8_t* __restrict__ ws, int64_t row,
                                                  int K, int step, int g, uint4& codes,
                                                  uint32_t& sc) {
  codes = load_stream16(wc + row * (K / 2) + step * 64 + g * 16);
  sc = *reinterpret_cast<const uint16_t*>(ws + row * (K / 16) + g * (K / 64) + step * 2);
}

template <int FM, int FN>
__device__ __forceinline__ void mma_chunk(const _Float16 (*lds)[Chunk<FM>::pitch], int nsteps,
                                          const uint4 (&wc)[FN][4], const uint32_t (&wsc)[FN][4],
                                          f32x4 (&acc)[FN][FM], int g, int r16) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s >= nsteps) break;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      half8 bfrag[FM];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        bfrag[fm] = *reinterpret_cast<const half8*>(&lds[fm * 16 + r16][s * 128 + 32 * g + 8 * q]);
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const uint32_t word = q == 0 ? wc[f][s].x : q == 1 ? wc[f][s].y : q == 2 ? wc[f][s].z : wc[f][s].w;
        const half2v sc2 = e4m3_half2((wsc[f][s] >> (8 * (q >> 1))) & 0xFFu);
        const half8 afrag = dequant8_f16(word, sc2);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          acc[f][fm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afrag, bfrag[fm], acc[f][fm], 0, 0, 0);
      }
    }
  }
}

// GEMM1: h = x^ . W13[e]^T for act columns [c0, c0 + 64*FNH) of this block
// (gate rows c and up rows I + c), then act = silu(h_gate) * h_up per
// expanded row, stored in fp32 with the block's partial row amax.
template <int FM, int FNH>
__global__ __launch_bounds__(256) void moe_gemm1_kernel(FwdParams p) {
  constexpr int MT = 16 * FM;
  constexpr int FN = 2 * FNH;
  constexpr int kKC = Chunk<FM>::KC;
  __shared__ _Float16 lds[MT][Chunk<FM>::pitch];
  __shared__ int s_tok[MT];
  __shared__ float s_ginv[MT];
  __shared__ float s_amax[4][MT];
  if (static_cast<int>(blockIdx.x) >= *p.n_tiles) return;
  const int4 td = p.tiles[blockIdx.x];
  const int e = td.x, row0 = td.y, nrows = td.z;
  const int H = p.H, I = p.I;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4, r16 = lane & 15;
  if (threadIdx.x < MT) {
    const int m = threadIdx.x;
    int tok = -1;
    float gi = 0.0f;
    if (m < nrows) {
      tok = p.perm[row0 + m] / p.k;
      gi = 1.0f / p.xq_g[tok];
    }
    s_tok[m] = tok;
    s_ginv[m] = gi;
  }
  const int c0 = blockIdx.y * (4 * 16 * FNH) + wave * 16 * FNH;  // first act column of the wave
  const uint8_t* wc = p.w13c + static_cast<int64_t>(e) * 2 * I * (H / 2);
  const uint8_t* ws = p.w13s + static_cast<int64_t>(e) * 2 * I * (H / 16);
  f32x4 acc[FN][FM];
#pragma unroll
  for (int f = 0; f < FN; ++f)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) acc[f][fm] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kc = 0; kc < H; kc += kKC) {
    const int nsteps = min(kKC, H - kc) / 128;
    uint4 wcodes[FN][4];
    uint32_t wsc[FN][4];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int64_t n = (f < FNH) ? (c0 + f * 16 + r16) : (I + c0 + (f - FNH) * 16 + r16);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (s < nsteps) load_weight_piece(wc, ws, n, H, kc / 128 + s, g, wcodes[f][s], wsc[f][s]);
    }
    __syncthreads();
    // stage the token operand: rows x (nsteps*128) fp16, 32 elements per item
    const int items = MT * nsteps * 4;
    for (int it = threadIdx.x; it < items; it += 256) {
      const int m = it / (nsteps * 4);
      const int kk = (it % (nsteps * 4)) * 32;
      const int tok = s_tok[m];
      half8* dst = reinterpret_cast<half8*>(&lds[m][kk]);
      if (tok >= 0) {
        const uint4 cw = *reinterpret_cast<const uint4*>(p.xq_codes + static_cast<int64_t>(tok) * (H / 2) + (kc + kk) / 2);
        const uint16_t sw = *reinterpret_cast<const uint16_t*>(p.xq_scales + static_cast<int64_t>(tok) * (H / 16) + (kc + kk) / 16);
        const half2v s0 = e4m3_half2(sw & 0xFFu), s1 = e4m3_half2(sw >> 8);
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
    mma_chunk<FM, FN>(lds, nsteps, wcodes, wsc, acc, g, r16);
  }

  // epilogue: lane holds D[n = 4g + i][m = r16] of each fragment
  const float wginv = 1.0f / p.w13g[e];
  float am[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    am[fm] = 0.0f;
    const int m = fm * 16 + r16;
    const float alpha = s_ginv[m] * wginv;
#pragma unroll
    for (int fh = 0; fh < FNH; ++fh) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float hg = acc[fh][fm][i] * alpha;
        const float hu = acc[FNH + fh][fm][i] * alpha;
        a[i] = hg / (1.0f + __expf(-hg)) * hu;
        am[fm] = fmaxf(am[fm], fabsf(a[i]));
      }
      if (m < nrows) {
        const int n = c0 + fh * 16 + 4 * g;
        *reinterpret_cast<float4*>(p.act + static_cast<int64_t>(row0 + m) * I + n) =
            make_float4(a[0], a[1], a[2], a[3]);
      }
    }
    am[fm] = fmaxf(am[fm], __shfl_xor(am[fm], 16, kWave));
    am[fm] = fmaxf(am[fm], __shfl_xor(am[fm], 32, kWave));
    if (g == 0) s_amax[wave][m] = am[fm];
  }
  __syncthreads();
  if (threadIdx.x < MT && static_cast<int>(threadIdx.x) < nrows) {
    const int m = threadIdx.x;
    const float v = fmaxf(fmaxf(s_amax[0][m], s_amax[1][m]), fmaxf(s_amax[2][m], s_amax[3][m]));
    p.act_amax[static_cast<int64_t>(row0 + m) * gridDim.y + blockIdx.y] = v;
  }
}

// GEMM2: y = a^2 . W2[e]^T for output columns [n0, n0 + 64*FN).  The token
// operand is the per-row re-quantization of act (same recipe as the token
// quantizer, on fp32 input, with g2 from the row amax), done while staging;
// the blocks of the first column band also store it (codes, scales, g2).
template <int FM, int FN>
__global__ __launch_bounds__(256) void moe_gemm2_kernel(FwdParams p, int n_amax) {
  constexpr int MT = 16 * FM;
  constexpr int kKC = Chunk<FM>::KC;
  __shared__ _Float16 lds[MT][Chunk<FM>::pitch];
  __shared__ float s_g2[MT];
  __shared__ int s_slot[MT];
  if (static_cast<int>(blockIdx.x) >= *p.n_tiles) return;
  const int4 td = p.tiles[blockIdx.x];
  const int e = td.x, row0 = td.y, nrows = td.z;
  const int H = p.H, I = p.I;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4, r16 = lane & 15;
  const bool write_a2 = blockIdx.y == 0;
  if (threadIdx.x < MT) {
    const int m = threadIdx.x;
    float g2 = 1.0f;
    int slot = -1;
    if (m < nrows) {
      float a = 0.0f;
      for (int j = 0; j < n_amax; ++j) a = fmaxf(a, p.act_amax[static_cast<int64_t>(row0 + m) * n_amax + j]);
      g2 = global_scale(a);
      slot = p.perm[row0 + m];
      if (write_a2) p.a2_g[row0 + m] = g2;
    }
    s_g2[m] = g2;
    s_slot[m] = slot;
  }
  __syncthreads();
  const int nb0 = blockIdx.y * (4 * 16 * FN) + wave * 16 * FN;
  const uint8_t* wc = p.w2c + static_cast<int64_t>(e) * H * (I / 2);
  const uint8_t* ws = p.w2s + static_cast<int64_t>(e) * H * (I / 16);
  f32x4 acc[FN][FM];
#pragma unroll
  for (int f = 0; f < FN; ++f)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) acc[f][fm] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kc = 0; kc < I; kc += kKC) {
    const int nsteps = min(kKC, I - kc) / 128;
    uint4 wcodes[FN][4];
    uint32_t wsc[FN][4];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int64_t n = nb0 + f * 16 + r16;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (s < nsteps) load_weight_piece(wc, ws, n, I, kc / 128 + s, g, wcodes[f][s], wsc[f][s]);
    }
    __syncthreads();
    // stage: re-quantize 16-element blocks of act, dequantize to fp16
    const int blocks_per_row = nsteps * 8;
    const int items = MT * blocks_per_row;
    for (int it = threadIdx.x; it < items; it += 256) {
      const int m = it / blocks_per_row;
      const int kb = (it % blocks_per_row) * 16;
      half8* dst = reinterpret_cast<half8*>(&lds[m][kb]);
      if (m < nrows) {
        const int64_t row = row0 + m;
        const float4* src = reinterpret_cast<const float4*>(p.act + row * I + kc + kb);
        float f[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = src[q];
          f[4 * q] = v.x; f[4 * q + 1] = v.y; f[4 * q + 2] = v.z; f[4 * q + 3] = v.w;
        }
        uint32_t lo, hi;
        const uint32_t sb = quantize_block16(f, s_g2[m], lo, hi);
        const half2v sc = e4m3_half2(sb);
        dst[0] = dequant8_f16(lo, sc);
        dst[1] = dequant8_f16(hi, sc);
        if (write_a2) {
          *reinterpret_cast<uint2*>(p.a2_codes + row * (I / 2) + (kc + kb) / 2) = make_uint2(lo, hi);
          p.a2_scales[row * (I / 16) + (kc + kb) / 16] = static_cast<uint8_t>(sb);
        }
      } else {
        const half8 z = {0, 0, 0, 0, 0, 0, 0, 0};
        dst[0] = z; dst[1] = z;
      }
    }
    __syncthreads();
    mma_chunk<FM, FN>(lds, nsteps, wcodes, wsc, acc, g, r16);
  }

  const float wginv = 1.0f / p.w2g[e];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = fm * 16 + r16;
    if (m >= nrows) continue;
    const float alpha = (1.0f / s_g2[m]) * wginv;
    const int64_t row = row0 + m;
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int n = nb0 + f * 16 + 4 * g;
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

// Finalize: out[t, n] = bf16_rne(sum_j w[t, j] * y[inv[t, j], n]) in slot
// order (deterministic), or bf16_rne(out_acc[t, n]) after the atomic epilogue.
// One thread per 8 output columns.
__global__ __launch_bounds__(256) void moe_finalize_kernel(FwdParams p) {
  const int H = p.H, k = p.k;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int per_row = H / 8;
  if (idx >= static_cast<int64_t>(p.T) * per_row) return;
  const int64_t t = idx / per_row;
  const int n = static_cast<int>(idx % per_row) * 8;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (p.deterministic) {
    for (int j = 0; j < k; ++j) {
      const float w = p.topk_w[t * k + j];
      const float4* yr = reinterpret_cast<const float4*>(p.y + static_cast<int64_t>(p.inv[t * k + j]) * H + n);
      const float4 a = yr[0], b = yr[1];
      s[0] += w * a.x; s[1] += w * a.y; s[2] += w * a.z; s[3] += w * a.w;
      s[4] += w * b.x; s[5] += w * b.y; s[6] += w * b.z; s[7] += w * b.w;
    }
  } else {
    const float4* r = reinterpret_cast<const float4*>(p.out_acc + t * H + n);
    const float4 a = r[0], b = r[1];
    s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w; s[4] = b.x; s[5] = b.y; s[6] = b.z; s[7] = b.w;
  }
  uint4 o;
  o.x = f32_to_bf16_rne(s[0]) | (f32_to_bf16_rne(s[1]) << 16);
  o.y = f32_to_bf16_rne(s[2]) | (f32_to_bf16_rne(s[3]) << 16);
  o.z = f32_to_bf16_rne(s[4]) | (f32_to_bf16_rne(s[5]) << 16);
  o.w = f32_to_bf16_rne(s[6]) | (f32_to_bf16_rne(s[7]) << 16);
  *reinterpret_cast<uint4*>(p.out + t * H + n) = o;
}

// ---------------------------------------------------------------------------
// Scale layout for the GEMMs: row-major [rows, K/16] -> [rows][g][step][2]
// with block b = 8*step + 2*g + h, so that lane group g finds the two scales
// of its 32-code piece of K step `step` as one 16-bit word.
// ---------------------------------------------------------------------------
__global__ void swizzle_scales_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                      int64_t rows, int K) {
  const int nb = K / 16;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * nb) return;
  const int64_t row = i / nb;
  const int b = static_cast<int>(i % nb);
  const int step = b / 8, gg = (b % 8) / 2, h = b % 2;
  dst[row * nb + gg * (K / 64) + step * 2 + h] = src[i];
}

__global__ void copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

hipError_t launch_swizzle_scales(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t K,
                                 hipStream_t s) {
  const int64_t n = rows * (K / 16);
  swizzle_scales_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(src, dst, rows, static_cast<int>(K));
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s) {
  copy_f32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

constexpr int kG1FNH = 1;  // gate (and up) fragments per wave in GEMM1
constexpr int kG2FN = 2;   // fragments per wave in GEMM2

int gemm1_cols_per_block() { return 4 * 16 * kG1FNH; }

template <int FM>
static void launch_gemms(const FwdParams& p, int max_tiles, hipStream_t s, hipEvent_t const* ev) {
  const int n1 = p.I / (4 * 16 * kG1FNH);
  moe_gemm1_kernel<FM, kG1FNH><<<dim3(max_tiles, n1), 256, 0, s>>>(p);
  if (ev) (void)hipEventRecord(ev[2], s);
  const int n2 = p.H / (4 * 16 * kG2FN);
  moe_gemm2_kernel<FM, kG2FN><<<dim3(max_tiles, n2), 256, 0, s>>>(p, n1);
  if (ev) (void)hipEventRecord(ev[3], s);
}

hipError_t launch_moe_forward(const FwdParams& p, int max_tiles, hipStream_t s,
                              hipEvent_t const* ev) {
  if (ev) (void)hipEventRecord(ev[0], s);
  int tpb = (p.T + 255) / 256;
  tpb = ((tpb + 3) / 4) * 4;
  if (tpb < 16) tpb = 16;
  if (tpb > kMaxTokensPerBlock) tpb = kMaxTokensPerBlock;
  const int nblocks = (p.T + tpb - 1) / tpb;
  switch (quant_nb_for_cols(p.H)) {
    case 1: moe_route_kernel<1><<<nblocks, 256, 0, s>>>(p, tpb); break;
    case 2: moe_route_kernel<2><<<nblocks, 256, 0, s>>>(p, tpb); break;
    case 4: moe_route_kernel<4><<<nblocks, 256, 0, s>>>(p, tpb); break;
    case 8: moe_route_kernel<8><<<nblocks, 256, 0, s>>>(p, tpb); break;
    default: moe_route_kernel<0><<<nblocks, 256, 0, s>>>(p, tpb); break;
  }
  if (ev) (void)hipEventRecord(ev[1], s);
  switch (p.mt) {
    case 16: launch_gemms<1>(p, max_tiles, s, ev); break;
    case 32: launch_gemms<2>(p, max_tiles, s, ev); break;
    default: launch_gemms<4>(p, max_tiles, s, ev); break;
  }
  const int64_t nthreads = static_cast<int64_t>(p.T) * (p.H / 8);
  moe_finalize_kernel<<<static_cast<unsigned>((nthreads + 255) / 256), 256, 0, s>>>(p);
  if (ev) (void)hipEventRecord(ev[4], s);
  return hipGetLastError();
}

}  // namespace nvfp4
