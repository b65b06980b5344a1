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
// Router reductions.  A candidate is the 64-bit key (order-preserving bits of
// the logit) << 32 | ~expert, so the larger key is the larger logit and, on
// equal logits, the smaller expert index.  -0.0 is keyed as +0.0: a binary32
// comparison finds the two equal, so their tie also goes to the smaller
// index.  Reductions over a 16-lane DPP row use quad permutes (xor 1, xor 2)
// and row rotates (4, 8), one instruction each.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  const uint32_t u = __float_as_uint(v) == 0x80000000u ? 0u : __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(o) << 32) | static_cast<uint32_t>(~e);
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t o = static_cast<uint32_t>(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int key_expert(uint64_t k) { return static_cast<int>(~static_cast<uint32_t>(k)); }

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

// The largest key over a 16-lane DPP row, or over the wave, as two 32-bit
// maxima: of the high words (the ordered logits), then of the low words
// (~expert) of the lanes whose high word is that maximum.  The pair is the
// lexicographic, i.e. 64-bit, maximum; each DPP step is a single max with a
// DPP operand (the 64-bit form takes two moves, a compare and two selects).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppXor1>(v));
  v = max(v, dpp_u32<kDppXor2>(v));
  v = max(v, dpp_u32<kDppRor4>(v));
  v = max(v, dpp_u32<kDppRor8>(v));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row16_max_u32(v);
  uint32_t a, b;
  lane_pair<16>(v, a, b);
  v = max(a, b);
  lane_pair<32>(v, a, b);
  return max(a, b);
}
template <bool WAVE>
__device__ __forceinline__ uint64_t key_max(uint64_t k) {
  const uint32_t h = static_cast<uint32_t>(k >> 32), l = static_cast<uint32_t>(k);
  const uint32_t mh = WAVE ? wave_max_u32(h) : row16_max_u32(h);
  const uint32_t tl = h == mh ? l : 0u;
  const uint32_t ml = WAVE ? wave_max_u32(tl) : row16_max_u32(tl);
  return (static_cast<uint64_t>(mh) << 32) | ml;
}
// (the association, and so the rounding, depends on the lane: a slot's weight
// is normalized by the sum its own lane forms)
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppRor4>(v);
  v += dpp_f32<kDppRor8>(v);
  return v;
}

// Inclusive prefix sum over the wave's lanes (every lane active): steps of
// 1, 2, 4, 8 lanes within each 16-lane row (DPP row_shr; a lane shifted in
// from outside the row adds 0), then every row adds the totals of the rows
// below it (lanes 15, 31, 47).
__device__ __forceinline__ int wave_scan_incl(int v, int lane) {
  v += static_cast<int>(dpp_u32<0x111>(static_cast<uint32_t>(v)));
  v += static_cast<int>(dpp_u32<0x112>(static_cast<uint32_t>(v)));
  v += static_cast<int>(dpp_u32<0x114>(static_cast<uint32_t>(v)));
  v += static_cast<int>(dpp_u32<0x118>(static_cast<uint32_t>(v)));
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

// Inclusive prefix sums of two values over threads 0..255 of a block (its
// first four waves): a wave scan each, then every wave adds the totals of
// the waves below it, exchanged through s_tot (one barrier).  Every thread
// of the block calls it; threads past 255 keep their values.  Returns the
// two totals over the 256 threads.
__device__ __forceinline__ int2 scan256_pair(int& a, int& b, int tid, int (&s_tot)[2][4]) {
  const int wave = tid / kWave, lane = tid & (kWave - 1);
  if (wave < 4) {
    a = wave_scan_incl(a, lane);
    b = wave_scan_incl(b, lane);
    if (lane == kWave - 1) {
      s_tot[0][wave] = a;
      s_tot[1][wave] = b;
    }
  }
  __syncthreads();
  int2 tot = make_int2(0, 0);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave && wave < 4) {
      a += s_tot[0][w];
      b += s_tot[1][w];
    }
    tot.x += s_tot[0][w];
    tot.y += s_tot[1][w];
  }
  return tot;
}

// ---------------------------------------------------------------------------
// Router: the k largest logits of one token, ties to the smaller expert
// index, slots in descending order; weights = exp(l_j - l_0) normalized over
// the k slots (the softmax over all experts restricted to the chosen k).
// Keys order the logits as binary32 compares do (-0 as +0) and, on equal
// values, put the smaller expert first.
//
// Both routers below first sort each lane's keys (largest first) with
// Batcher's odd-even merge sorting network (K. E. Batcher, "Sorting networks
// and their applications", AFIPS 1968), so that each of the k selection
// rounds only takes the maximum of the lanes' heads and pops the winning
// lane's list.  Keys are unique (the expert index is part of them).  Slot j
// ends in lane j of the token's lanes, and its weight is normalized by the
// row-16 sum over the first 16 of them, so both routers give the same ids
// and the same weights.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void key_cx(uint64_t& a, uint64_t& b) {
  const bool sw = b > a;
  const uint64_t hi = sw ? b : a, lo = sw ? a : b;
  a = hi;
  b = lo;
}

template <int N>
__device__ __forceinline__ void sort_keys_desc(uint64_t (&c)[N]) {
#pragma unroll
  for (int p = 1; p < N; p <<= 1)
#pragma unroll
    for (int d = p; d >= 1; d >>= 1)
#pragma unroll
      for (int j = d % p; j + d < N; j += 2 * d)
#pragma unroll
        for (int i = 0; i < d; ++i)
          if (i + j + d < N && (i + j) / (2 * p) == (i + j + d) / (2 * p)) key_cx(c[i + j], c[i + j + d]);
}

// The k selection rounds over the lanes' sorted lists (KMAX >= k rounds at
// most): each round takes the largest head over the 16-lane row (or the
// wave) and pops it from the lane that held it; lane j keeps round j's key.
// After round j at most KMAX - 1 - j more pops follow, so only that many
// leading entries of a list can still become its head and only those are
// shifted.
template <int N, int KMAX, bool WAVE>
__device__ __forceinline__ void select_rounds(uint64_t (&cand)[N], int k, int lane, uint64_t& mine,
                                              uint64_t& top) {
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      const uint64_t best = key_max<WAVE>(cand[0]);
      if (j == 0) top = best;
      mine = lane == j ? best : mine;
      const bool pop = cand[0] == best;  // this lane held the winner
#pragma unroll
      for (int i = 0; i < N && i + 1 < KMAX - j; ++i) cand[i] = pop ? (i + 1 < N ? cand[i + 1] : 0ull) : cand[i];
    }
  }
}

// One wave per token (few tokens: the shortest dependency chain); lane l
// holds experts l, l + 64, ...; lane j < k returns slot j.
template <int KPW>
__device__ void route_token_wave(const float* __restrict__ lrow, int E, int k, int lane, int& my_id,
                                 float& my_w) {
  // unconditional loads (index clamped; invalid candidates get key 0), all
  // in flight at once
  float v[KPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) v[i] = lrow[min(lane + kWave * i, E - 1)];
#pragma unroll
  for (int i = 0; i < KPW; ++i) keep_issued(v[i]);
  uint64_t cand[KPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int e = lane + kWave * i;
    cand[i] = e < E ? route_key(v[i], e) : 0ull;
  }
  sort_keys_desc<KPW>(cand);
  uint64_t mine = 0, top = 0;
  if (k <= 8)
    select_rounds<KPW, 8, true>(cand, k, lane, mine, top);
  else
    select_rounds<KPW, kMaxTopK, true>(cand, k, lane, mine, top);
  const float ex = lane < k ? expf(key_value(mine) - key_value(top)) : 0.0f;
  const float sum = row16_sum(ex);
  my_id = key_expert(mine);
  my_w = ex / sum;
}

// ---------------------------------------------------------------------------
// Prologue for large batches past the two-kernel one below (more than 256
// experts or 8192 tokens), three kernels.
//  1. route: each block takes `tpb` consecutive tokens; each wave quantizes
//     and routes tokens of the block, then the block computes, for every
//     (t, j), its rank among equal experts inside the block and the block's
//     per-expert counts.
//  2. schedule: per expert, exclusive scan of the per-block counts down the
//     blocks, and the expert's total.
//  3. place (one thread per (t, j)): scans over experts for the row offsets
//     (and, in block 0, the M-tile list), then row = offset[e] + block
//     base[b][e] + rank, giving the stable expandInputRows permutation (rows
//     of one expert in ascending (t, j) order) and its inverse.
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 256;

template <int NB, int KPL>
__global__ __launch_bounds__(256) void moe_route_kernel(FwdParams p, int tpb) {
  __shared__ int32_t s_ids[kMaxTokensPerRouteBlock * kMaxTopK];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int t0 = blockIdx.x * tpb;
  const int ntok = min(tpb, p.T - t0);
  const int H = p.H, k = p.k;
  for (int lt = wave; lt < ntok; lt += 4) {
    const int64_t t = t0 + lt;
    if (p.preq) {  // codes handed over: only the tiled GEMMs' fp16 copy is written
      if (p.xq16) dequant_row_f16(p.xq_codes + t * (H / 2), p.xq_scales + t * (H / 16), H / 16, p.xq16 + t * H,
                                  lane, kWave);
    } else if (!p.a16) {  // (W4A16 uses x as it is)
      quantize_row_wave<NB>(p.x + t * H, H / 16, p.xq_codes + t * (H / 2), p.xq_scales + t * (H / 16),
                            p.xq_g + t, lane, p.xq16 ? p.xq16 + t * H : nullptr, p.static_g);
    }
    int id;
    float w;
    route_token_wave<KPL>(p.logits + t * p.E, p.E, k, lane, id, w);
    if (lane < k) {
      p.topk_ids[t * k + lane] = id;
      p.topk_w[t * k + lane] = w;
      s_ids[lt * k + lane] = id;
    }
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
}

// 2. One block per kSchedExperts experts, kSchedThreads / kSchedExperts
//    threads (two waves) per expert; each thread owns a chunk of consecutive
//    route blocks: chunk sums -> inclusive scan over the chunks (a shuffle
//    scan per wave, one LDS exchange between the two waves) -> each thread
//    writes the exclusive per-block bases of its chunk; the expert's total
//    goes to counts[e].  Chunks of up to kU blocks stay in registers between
//    the two passes.
constexpr int kSchedExperts = 2;
constexpr int kSchedPerExpert = kSchedThreads / kSchedExperts;
static_assert(kSchedPerExpert == 2 * kWave, "two waves per expert");

__global__ __launch_bounds__(kSchedThreads) void moe_schedule_kernel(FwdParams p, int nblocks) {
  __shared__ int32_t s_wave[kSchedExperts];
  const int E = p.E;
  const int le = threadIdx.x / kSchedPerExpert, c = threadIdx.x % kSchedPerExpert;
  const int lane = threadIdx.x & (kWave - 1);
  const int e = blockIdx.x * kSchedExperts + le;
  const bool valid = e < E;
  const int cs = (nblocks + kSchedPerExpert - 1) / kSchedPerExpert;
  const int b0 = min(c * cs, nblocks), b1 = min(b0 + cs, nblocks);
  constexpr int kU = 16;  // loads in batches of 16, all in flight together
  int v[kU];
  int sum = 0;
  if (valid) {
    for (int b = b0; b < b1; b += kU) {
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = p.blk_counts[min(b + u, b1 - 1) * E + e];
#pragma unroll
      for (int u = 0; u < kU; ++u) sum += b + u < b1 ? v[u] : 0;
    }
  }
  // inclusive scan over the expert's chunks
  int inc = wave_scan_incl(sum, lane);
  const bool second = c >= kWave;
  if (!second && lane == kWave - 1) s_wave[le] = inc;
  __syncthreads();
  if (second) inc += s_wave[le];
  if (!valid) return;
  if (c == kSchedPerExpert - 1) p.counts[e] = inc;
  int run = inc - sum;
  if (cs <= kU) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (b0 + u < b1) {
        p.blk_counts[(b0 + u) * E + e] = run;
        run += v[u];
      }
    }
    return;
  }
  for (int b = b0; b < b1; b += kU) {
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = p.blk_counts[min(b + u, b1 - 1) * E + e];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (b + u < b1) {
        p.blk_counts[(b + u) * E + e] = run;
        run += v[u];
      }
    }
  }
}

// 3. Every block scans the per-expert totals in LDS for the row offsets (E is
//    at most kMaxExperts), then places its entries; block 0 also publishes the
//    offsets, the tile count and the M-tile list.
__global__ __launch_bounds__(256) void moe_place_kernel(FwdParams p, int tpb) {
  __shared__ int32_t s_off[kMaxExperts];
  __shared__ int32_t s_tb[kMaxExperts];
  __shared__ int s_tot[2][4];
  const int tid = threadIdx.x;
  const int E = p.E, mt = p.mt;
  const int per = (E + 255) / 256;
  int rsum = 0, tsum = 0;
  for (int u = 0; u < per; ++u) {
    const int e = tid * per + u;
    if (e < E) {
      const int cnt = p.counts[e];
      rsum += cnt;
      tsum += (cnt + mt - 1) / mt;
    }
  }
  int rb = rsum, tb = tsum;
  const int2 total = scan256_pair(rb, tb, tid, s_tot);
  rb -= rsum;
  tb -= tsum;
  for (int u = 0; u < per; ++u) {
    const int e = tid * per + u;
    if (e < E) {
      const int cnt = p.counts[e];
      s_off[e] = rb;
      s_tb[e] = tb;
      rb += cnt;
      tb += (cnt + mt - 1) / mt;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = tid; e < E; e += 256) {
      p.offsets[e] = s_off[e];
      const int cnt = p.counts[e];
      const int nt = (cnt + mt - 1) / mt;
      for (int i = 0; i < nt; ++i) p.tiles[s_tb[e] + i] = make_int4(e, s_off[e] + i * mt, min(mt, cnt - i * mt), 0);
    }
    if (tid == 255) {
      p.offsets[E] = total.x;
      *p.n_tiles = append_shared_tiles(p, total.y);
    }
  }
  const int i = blockIdx.x * 256 + tid;
  if (i >= p.R) return;
  const int t = i / p.k;
  const int b = t / tpb;
  const int e = p.topk_ids[i];
  const int row = s_off[e] + p.blk_counts[b * E + e] + p.loc_rank[i];
  p.perm[row] = i;
  p.inv[i] = row;
}

// ---------------------------------------------------------------------------
// Prologue for small batches (T <= 256, E <= 256, T*k <= 2048): block 0
// routes every token and builds the whole schedule in LDS (no cross-block
// communication); blocks 1.. quantize 8 token rows each, one per wave, at the
// same time.
//
// Routing uses 16 lanes per token (4 tokens per wave at once): lane j of a
// group holds experts j, j + 16, ...  Stable ranks come from 64-entry chunks:
// a lane's rank among equal experts in its chunk is the popcount of the lanes
// below it whose expert id matches bit for bit (one ballot per id bit); the
// per-chunk counts are then scanned down the chunks per expert.
// ---------------------------------------------------------------------------
constexpr int kSmallMaxT = 256, kSmallMaxE = 256, kSmallMaxR = 2048;
constexpr int kSmallThreads = 1024;  // 16 waves: 64 tokens routed per pass
constexpr int kSmallWaves = kSmallThreads / 64;

// Router for one token by a 16-lane group (4 tokens per wave; lane gl of
// the group holds experts gl, gl + 16, ...): lane j < k of the group ends
// with slot j (the sorted-list selection of the router section above).
template <int KPL>
__device__ void route_token_group16(const float* __restrict__ lrow, int E, int k, int gl,
                                    int& my_id, float& my_w) {
  float v[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) v[i] = lrow[min(gl + 16 * i, E - 1)];
#pragma unroll
  for (int i = 0; i < KPL; ++i) keep_issued(v[i]);
  uint64_t cand[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = gl + 16 * i;
    cand[i] = e < E ? route_key(v[i], e) : 0ull;
  }
  sort_keys_desc<KPL>(cand);
  uint64_t mine = 0, top = 0;
  if (k <= 8)
    select_rounds<KPL, 8, false>(cand, k, gl, mine, top);
  else
    select_rounds<KPL, kMaxTopK, false>(cand, k, gl, mine, top);
  const float ex = gl < k ? expf(key_value(mine) - key_value(top)) : 0.0f;
  const float sum = row16_sum(ex);
  my_id = key_expert(mine);
  my_w = ex / sum;
}


template <int NB, int KPL>
__global__ __launch_bounds__(kSmallThreads) void moe_prologue_small_kernel(FwdParams p) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int H = p.H, k = p.k, E = p.E, T = p.T, R = p.R;
  if (blockIdx.x > 0) {
    const int64_t t = static_cast<int64_t>(blockIdx.x - 1) * kSmallWaves + wave;
    if (t < T) {
      if (p.preq) {  // codes handed over: only the tiled GEMMs' fp16 copy is written
        if (p.xq16)
          dequant_row_f16(p.xq_codes + t * (H / 2), p.xq_scales + t * (H / 16), H / 16, p.xq16 + t * H, lane,
                          kWave);
      } else if (!p.a16) {  // (W4A16 uses x as it is)
        quantize_row_wave<NB>(p.x + t * H, H / 16, p.xq_codes + t * (H / 2), p.xq_scales + t * (H / 16),
                              p.xq_g + t, lane, p.xq16 ? p.xq16 + t * H : nullptr, p.static_g);
      }
      if (!p.deterministic) {
        float4* row = reinterpret_cast<float4*>(p.out_acc + t * H);
        for (int c = lane; c < H / 4; c += kWave) row[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }
  __shared__ int32_t s_ids[kSmallMaxR];
  __shared__ int32_t s_rank[kSmallMaxR];
  __shared__ int32_t s_cnt[kSmallMaxR / 64][kSmallMaxE];
  __shared__ int32_t s_off[kSmallMaxE];
  __shared__ int32_t s_tbase[kSmallMaxE];
  __shared__ int s_tot[2][4];
  const int tid = threadIdx.x;
  // 1. routing, 4 tokens per wave at a time
  const int grp = lane >> 4, gl = lane & 15;
  for (int t0 = wave * 4; t0 < T; t0 += kSmallWaves * 4) {
    const int t = t0 + grp;
    const int tc = t < T ? t : T - 1;
    int id;
    float w;
    route_token_group16<KPL>(p.logits + static_cast<int64_t>(tc) * E, E, k, gl, id, w);
    if (t < T && gl < k) {
      p.topk_ids[t * k + gl] = id;
      p.topk_w[t * k + gl] = w;
      s_ids[t * k + gl] = id;
    }
  }
  for (int i = tid; i < (kSmallMaxR / 64) * kSmallMaxE; i += kSmallThreads) (&s_cnt[0][0])[i] = 0;
  __syncthreads();
  // 2. ranks inside 64-entry chunks
  const int nch = (R + 63) / 64;
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  for (int c = wave; c < nch; c += kSmallWaves) {
    const int i = 64 * c + lane;
    const bool valid = i < R;
    const int e = valid ? s_ids[i] : 0;
    uint64_t mask = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t bm = __ballot((e >> b) & 1);
      mask &= ((e >> b) & 1) ? bm : ~bm;
    }
    const int rank = __popcll(mask & ((1ull << lane) - 1ull));
    if (valid) {
      s_rank[i] = rank;
      if (rank == 0) s_cnt[c][e] = __popcll(mask);
    }
  }
  __syncthreads();
  // 3. per expert: exclusive scan down the chunks
  int tot = 0, ntile = 0;
  if (tid < E) {
    for (int c = 0; c < nch; ++c) {
      const int v = s_cnt[c][tid];
      s_cnt[c][tid] = tot;
      tot += v;
    }
    ntile = (tot + p.mt - 1) / p.mt;
    p.counts[tid] = tot;
  }
  // 4. exclusive scans over experts (rows and tiles)
  static_assert(kSmallMaxE == 256, "one scan over the first four waves");
  int incr = tot, inct = ntile;
  const int2 total = scan256_pair(incr, inct, tid, s_tot);
  if (tid < E) {
    const int off = incr - tot, tb = inct - ntile;
    s_off[tid] = off;
    s_tbase[tid] = tb;
    p.offsets[tid] = off;
    for (int i = 0; i < ntile; ++i)
      p.tiles[tb + i] = make_int4(tid, off + i * p.mt, min(p.mt, tot - i * p.mt), 0);
  }
  if (tid == kSmallMaxE - 1) {
    p.offsets[E] = total.x;
    *p.n_tiles = append_shared_tiles(p, total.y);
  }
  __syncthreads();
  // 5. placement
  for (int i = tid; i < R; i += kSmallThreads) {
    const int e = s_ids[i];
    const int row = s_off[e] + s_cnt[i / 64][e] + s_rank[i];
    p.perm[row] = i;
    p.inv[i] = row;
  }
}

// Per-token quantization of one row per 256 threads of a 1024-thread block
// (row t; thread qt = tid % 256 owns 16-element blocks qt, qt + 256, ...; the
// row amax is one LDS exchange between the quarter's four waves).  Every
// thread of the block calls it (one barrier); a quarter with t >= T only
// joins the barrier.  Also clears the row's atomic accumulator, or (codes
// handed over) writes only the tiled GEMMs' fp16 copy.
template <int NBL>
__device__ __forceinline__ void prologue_quantize_quarter(const FwdParams& p, int64_t t, int tid) {
  __shared__ float s_am[kSmallWaves];
  const int wave = tid / kWave, lane = tid & (kWave - 1);
  const int qt = tid & 255, q = tid >> 8;
  const int H = p.H, T = p.T;
  if (p.a16 || p.preq) {  // W4A16 uses x as it is; handed-over codes only need the fp16
                          // copy of the tiled GEMMs (if any) and the atomic accumulator cleared
    if (t < T && p.preq && p.xq16)
      dequant_row_f16(p.xq_codes + t * (H / 2), p.xq_scales + t * (H / 16), H / 16, p.xq16 + t * H, qt, 256);
    if (t < T && !p.deterministic) {
      float4* row = reinterpret_cast<float4*>(p.out_acc + t * H);
      for (int c = qt; c < H / 4; c += 256) row[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  const int nblk = H / 16;
  const uint16_t* xrow = p.x + min(t, static_cast<int64_t>(T - 1)) * H;
  uint4 v[NBL][2];
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    const uint4* src = reinterpret_cast<const uint4*>(xrow + 16 * min(qt + 256 * i, nblk - 1));
    v[i][0] = src[0];
    v[i][1] = src[1];
  }
  float bam[NBL];
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    bam[i] = amax16_bf16(v[i][0], v[i][1]);
    if (qt + 256 * i < nblk) am = fmaxf(am, bam[i]);
  }
  am = wave_max(am);
  if (lane == 0) s_am[wave] = am;
  __syncthreads();
  if (t >= T) return;
  const float* sq = s_am + 4 * q;
  const float g = p.static_g ? p.static_g[0] : global_scale(fmaxf(fmaxf(sq[0], sq[1]), fmaxf(sq[2], sq[3])));
  uint8_t* crow = p.xq_codes + t * (H / 2);
  uint8_t* srow = p.xq_scales + t * (H / 16);
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    const int b = qt + 256 * i;
    if (b < nblk) {
      float f[16];
      unpack16(v[i][0], v[i][1], f);
      uint32_t lo, hi;
      const uint32_t sb = quantize_block16_amax(f, bam[i], g, lo, hi);
      *reinterpret_cast<uint2*>(crow + 8 * b) = make_uint2(lo, hi);
      srow[b] = static_cast<uint8_t>(sb);
      if (p.xq16) store_block_f16(p.xq16 + t * H + 16 * b, lo, hi, sb);
    }
  }
  if (qt == 0) p.xq_g[t] = g;
  if (!p.deterministic) {
    float4* row = reinterpret_cast<float4*>(p.out_acc + t * H);
    for (int c = qt; c < H / 4; c += 256) row[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// ---------------------------------------------------------------------------
// Prologue for large batches with E <= 256 and T <= 8192, two kernels.
//  1. route64: blocks 0 .. nr-1 route 64 tokens each (16 lanes per token, the
//     small-batch router, four tokens per wave in one pass) and rank every
//     (t, j) among the block's equal experts (ballots over 64-entry chunks,
//     then a scan of the chunk counts per expert), writing the block's
//     per-expert counts; blocks nr.. quantize token rows at the same time:
//     16 per block, one per wave, or (rows of more than 4096 elements, QB >
//     0) 4 per block, one per 256 threads.
//  2. place64 (one block per routing block, one thread per (t, j)): every
//     block sums the count matrix per expert, over all routing blocks (the
//     totals, scanned over the experts for the row offsets) and over the
//     blocks before its own (its base), then row = offset[e] + base[e] +
//     rank; block 0 also publishes counts, offsets, the tile count and the
//     M-tile list.  Same stable order as the other prologues.
// ---------------------------------------------------------------------------
constexpr int kRoute64Tokens = 64;
constexpr int kRoute64MaxE = 256;
constexpr int kRoute64MaxT = 8192;
static_assert(kRoute64Tokens * kMaxTopK <= kSmallThreads, "one thread per (t, j) of a routing block");

bool use_route64_prologue(const FwdParams& p) { return p.E <= kRoute64MaxE && p.T <= kRoute64MaxT; }

template <int NB, int KPL, int QB>
__global__ __launch_bounds__(kSmallThreads) void moe_route64_kernel(FwdParams p, int nr) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int H = p.H, k = p.k, E = p.E, T = p.T;
  if (QB > 0 && static_cast<int>(blockIdx.x) >= nr) {
    prologue_quantize_quarter<(QB > 0 ? QB : 1)>(p, static_cast<int64_t>(blockIdx.x - nr) * 4 + (threadIdx.x >> 8),
                                                  threadIdx.x);
    return;
  }
  if (static_cast<int>(blockIdx.x) >= nr) {
    const int64_t t = static_cast<int64_t>(blockIdx.x - nr) * kSmallWaves + wave;
    if (t < T) {
      if (p.preq) {  // codes handed over: only the tiled GEMMs' fp16 copy is written
        if (p.xq16)
          dequant_row_f16(p.xq_codes + t * (H / 2), p.xq_scales + t * (H / 16), H / 16, p.xq16 + t * H, lane,
                          kWave);
      } else if (!p.a16) {  // (W4A16 uses x as it is)
        quantize_row_wave<NB>(p.x + t * H, H / 16, p.xq_codes + t * (H / 2), p.xq_scales + t * (H / 16),
                              p.xq_g + t, lane, p.xq16 ? p.xq16 + t * H : nullptr, p.static_g);
      }
      if (!p.deterministic) {
        float4* row = reinterpret_cast<float4*>(p.out_acc + t * H);
        for (int c = lane; c < H / 4; c += kWave) row[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }
  constexpr int kN = kRoute64Tokens * kMaxTopK;
  __shared__ int32_t s_ids[kN];
  __shared__ int32_t s_rank[kN];
  __shared__ int32_t s_cnt[kN / 64][kRoute64MaxE];
  const int tid = threadIdx.x;
  const int b = blockIdx.x, t0 = b * kRoute64Tokens;
  const int ntok = min(kRoute64Tokens, T - t0), n = ntok * k;
  // 1. routing: wave w, group g routes token t0 + 4 w + g
  const int grp = lane >> 4, gl = lane & 15;
  {
    const int lt = 4 * wave + grp;
    const int tc = t0 + min(lt, ntok - 1);
    int id;
    float w;
    route_token_group16<KPL>(p.logits + static_cast<int64_t>(tc) * E, E, k, gl, id, w);
    if (lt < ntok && gl < k) {
      const int64_t i = static_cast<int64_t>(t0 + lt) * k + gl;
      p.topk_ids[i] = id;
      p.topk_w[i] = w;
      s_ids[lt * k + gl] = id;
    }
  }
  for (int i = tid; i < (kN / 64) * kRoute64MaxE; i += kSmallThreads) (&s_cnt[0][0])[i] = 0;
  __syncthreads();
  // 2. ranks inside 64-entry chunks
  const int nch = (n + 63) / 64;
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  if (wave < nch) {
    const int i = 64 * wave + lane;
    const bool valid = i < n;
    const int e = valid ? s_ids[i] : 0;
    uint64_t mask = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t bm = __ballot((e >> bit) & 1);
      mask &= ((e >> bit) & 1) ? bm : ~bm;
    }
    const int rank = __popcll(mask & ((1ull << lane) - 1ull));
    if (valid) {
      s_rank[i] = rank;
      if (rank == 0) s_cnt[wave][e] = __popcll(mask);
    }
  }
  __syncthreads();
  // 3. per expert: exclusive scan down the chunks; the block's count
  if (tid < E) {
    int tot = 0;
    for (int c = 0; c < nch; ++c) {
      const int v = s_cnt[c][tid];
      s_cnt[c][tid] = tot;
      tot += v;
    }
    p.blk_counts[static_cast<int64_t>(b) * E + tid] = tot;
  }
  __syncthreads();
  // 4. rank among the block's equal experts, in (t, j) order
  if (tid < n) p.loc_rank[static_cast<int64_t>(t0) * k + tid] = s_cnt[tid / 64][s_ids[tid]] + s_rank[tid];
}

__global__ __launch_bounds__(kSmallThreads) void moe_place64_kernel(FwdParams p, int nr) {
  constexpr int kParts = kSmallThreads / kRoute64MaxE;  // threads per expert summing the counts
  __shared__ int32_t s_pre[kParts][kRoute64MaxE];
  __shared__ int32_t s_all[kParts][kRoute64MaxE];
  __shared__ int32_t s_base[kRoute64MaxE];
  __shared__ int s_tot[2][4];
  const int tid = threadIdx.x, E = p.E, k = p.k, mt = p.mt;
  const int b = blockIdx.x;
  const int e = tid % kRoute64MaxE, q = tid / kRoute64MaxE;
  int pre = 0, all = 0;
  if (e < E) {
    // rows q, q + kParts, ... in batches of kU loads issued together
    constexpr int kU = 16;
    for (int r0 = q; r0 < nr; r0 += kParts * kU) {
      int c[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) c[u] = p.blk_counts[static_cast<int64_t>(min(r0 + kParts * u, nr - 1)) * E + e];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int r = r0 + kParts * u;
        all += r < nr ? c[u] : 0;
        pre += r < b ? c[u] : 0;
      }
    }
  }
  s_pre[q][e] = pre;
  s_all[q][e] = all;
  __syncthreads();
  // threads 0..255: expert tid's total and base, then the scans over experts
  int cnt = 0, base = 0;
  if (tid < kRoute64MaxE && tid < E) {
#pragma unroll
    for (int i = 0; i < kParts; ++i) {
      cnt += s_all[i][tid];
      base += s_pre[i][tid];
    }
  }
  const int ntile = (cnt + mt - 1) / mt;
  int rb = cnt, tb = ntile;
  const int2 total = scan256_pair(rb, tb, tid, s_tot);
  if (tid < kRoute64MaxE && tid < E) {
    const int off = rb - cnt;
    s_base[tid] = off + base;
    if (b == 0) {
      p.counts[tid] = cnt;
      p.offsets[tid] = off;
      const int t0 = tb - ntile;
      for (int i = 0; i < ntile; ++i) p.tiles[t0 + i] = make_int4(tid, off + i * mt, min(mt, cnt - i * mt), 0);
    }
  }
  if (b == 0 && tid == kRoute64MaxE - 1) {
    p.offsets[E] = total.x;
    *p.n_tiles = append_shared_tiles(p, total.y);
  }
  __syncthreads();
  const int t0 = b * kRoute64Tokens;
  const int n = min(kRoute64Tokens, p.T - t0) * k;
  if (tid < n) {
    const int64_t i = static_cast<int64_t>(t0) * k + tid;
    const int row = s_base[p.topk_ids[i]] + p.loc_rank[i];
    p.perm[row] = static_cast<int32_t>(i);
    p.inv[i] = row;
  }
}

// ---------------------------------------------------------------------------
// Prologue for decode-sized batches (T <= 64, E <= 256): block 0 routes every
// token (a whole wave per token up to kTinyWaveRouteT tokens, else 16 lanes
// per token, all tokens in one pass) and keeps, per expert,
// the 64-bit mask of the tokens routed to it.  A row's place in the stable
// expandInputRows order is then the expert's offset plus the popcount of the
// mask below its token, and the counts come from the masks as well, so the
// whole schedule takes three block barriers.  Blocks 1.. quantize four token
// rows each, one row per 256 threads (thread t owns 16-element blocks t,
// t + 256, ...; the row amax is one LDS exchange between four waves).
// ---------------------------------------------------------------------------
constexpr int kTinyMaxT = 64, kTinyMaxE = 256;
constexpr int kTinyWaveRouteT = 8;  // tokens routed one per wave (see step 1)

template <int NBL, int KPL>
__global__ __launch_bounds__(kSmallThreads) void moe_prologue_tiny_kernel(FwdParams p) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int H = p.H, k = p.k, E = p.E, T = p.T;
  if (blockIdx.x > 0) {
    prologue_quantize_quarter<NBL>(p, static_cast<int64_t>(blockIdx.x - 1) * 4 + (tid >> 8), tid);
    return;
  }
  __shared__ uint64_t s_mask[kTinyMaxE];
  __shared__ int32_t s_ids[kTinyMaxT * kMaxTopK];
  __shared__ int32_t s_off[kTinyMaxE];
  __shared__ int32_t s_wsum[2][4];
  if (tid < kTinyMaxE) s_mask[tid] = 0ull;
  __syncthreads();
  // 1. top-k of every token.  Up to kTinyWaveRouteT tokens: wave w routes
  // token w with all its lanes (the shortest chain: the block's routing is
  // the prologue's critical path); more: wave w, group g routes token
  // 4 w + g.  Waves past the last token skip it.
  if (T <= kTinyWaveRouteT) {
    if (wave < T) {
      int id;
      float w;
      route_token_wave<(KPL >= 4 ? KPL / 4 : 1)>(p.logits + static_cast<int64_t>(wave) * E, E, k, lane, id, w);
      if (lane < k) {
        p.topk_ids[wave * k + lane] = id;
        p.topk_w[wave * k + lane] = w;
        s_ids[wave * k + lane] = id;
        atomicOr(reinterpret_cast<unsigned long long*>(&s_mask[id]), 1ull << wave);
      }
    }
  } else if (4 * wave < T) {
    const int grp = lane >> 4, gl = lane & 15;
    const int tk = 4 * wave + grp;
    int id;
    float w;
    route_token_group16<KPL>(p.logits + static_cast<int64_t>(min(tk, T - 1)) * E, E, k, gl, id, w);
    if (tk < T && gl < k) {
      p.topk_ids[tk * k + gl] = id;
      p.topk_w[tk * k + gl] = w;
      s_ids[tk * k + gl] = id;
      atomicOr(reinterpret_cast<unsigned long long*>(&s_mask[id]), 1ull << tk);
    }
  }
  __syncthreads();
  // 2. rows and tiles per expert, exclusive scans over the experts (waves 0-3)
  int cnt = 0, nt = 0, ic = 0, it = 0;
  if (tid < kTinyMaxE) {
    cnt = tid < E ? __popcll(s_mask[tid]) : 0;
    nt = (cnt + p.mt - 1) / p.mt;
    ic = wave_scan_incl(cnt, lane);
    it = wave_scan_incl(nt, lane);
    if (lane == kWave - 1) {
      s_wsum[0][wave] = ic;
      s_wsum[1][wave] = it;
    }
  }
  __syncthreads();
  if (tid < kTinyMaxE) {
    int rows_total = 0, tiles_total = 0;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      if (w2 < wave) {
        ic += s_wsum[0][w2];
        it += s_wsum[1][w2];
      }
      rows_total += s_wsum[0][w2];
      tiles_total += s_wsum[1][w2];
    }
    const int off = ic - cnt, tb = it - nt;
    s_off[tid] = off;
    if (tid < E) {
      p.counts[tid] = cnt;
      p.offsets[tid] = off;
      for (int i = 0; i < nt; ++i) p.tiles[tb + i] = make_int4(tid, off + i * p.mt, min(p.mt, cnt - i * p.mt), 0);
    }
    if (tid == 0) {
      p.offsets[E] = rows_total;
      *p.n_tiles = append_shared_tiles(p, tiles_total);
    }
  }
  __syncthreads();
  // 3. placement: row = offset of the expert + tokens routed to it before t
  if (tid < T * k) {
    const int tok = tid / k, e = s_ids[tid];
    const int row = s_off[e] + __popcll(s_mask[e] & ((1ull << tok) - 1ull));
    p.perm[row] = tid;
    p.inv[tid] = row;
  }
}

bool use_tiny_prologue(const FwdParams& p) {
  return p.T <= kTinyMaxT && p.E <= kTinyMaxE && p.H / 16 <= 256 * 8 && p.T * p.k <= kSmallThreads;
}

template <int NBL>
static void launch_prologue_tiny(const FwdParams& p, hipStream_t s) {
  const int blocks = 1 + (p.T + 3) / 4;
  if (p.E <= 16) moe_prologue_tiny_kernel<NBL, 1><<<blocks, kSmallThreads, 0, s>>>(p);
  else if (p.E <= 32) moe_prologue_tiny_kernel<NBL, 2><<<blocks, kSmallThreads, 0, s>>>(p);
  else if (p.E <= 64) moe_prologue_tiny_kernel<NBL, 4><<<blocks, kSmallThreads, 0, s>>>(p);
  else if (p.E <= 128) moe_prologue_tiny_kernel<NBL, 8><<<blocks, kSmallThreads, 0, s>>>(p);
  else moe_prologue_tiny_kernel<NBL, 16><<<blocks, kSmallThreads, 0, s>>>(p);
}

bool use_small_prologue(const FwdParams& p) {
  return p.T <= kSmallMaxT && p.E <= kSmallMaxE && p.R <= kSmallMaxR;
}

template <int NB>
static void launch_prologue_small(const FwdParams& p, hipStream_t s) {
  const int blocks = 1 + (p.T + kSmallWaves - 1) / kSmallWaves;
  if (p.E <= 16) moe_prologue_small_kernel<NB, 1><<<blocks, kSmallThreads, 0, s>>>(p);
  else if (p.E <= 32) moe_prologue_small_kernel<NB, 2><<<blocks, kSmallThreads, 0, s>>>(p);
  else if (p.E <= 64) moe_prologue_small_kernel<NB, 4><<<blocks, kSmallThreads, 0, s>>>(p);
  else if (p.E <= 128) moe_prologue_small_kernel<NB, 8><<<blocks, kSmallThreads, 0, s>>>(p);
  else moe_prologue_small_kernel<NB, 16><<<blocks, kSmallThreads, 0, s>>>(p);
}

// Finalize: out[t, n] = bf16_rne(sum_j w[t, j] * y[t * k + j, n]) in slot
// order (deterministic; GEMM2 stores y by slot, in bf16), or
// bf16_rne(out_acc[t, n]) after the atomic epilogue.
// With a shared expert the deterministic sum adds its row R + t last and the
// total is multiplied by the combination scale (1 or 0.5, exact); the atomic
// epilogue applies the scale to each contribution.
// One thread per 8 output columns (16-byte loads of y, one 16-byte store);
// the slots are taken 8 at a time with all their weight and y loads issued
// before the sums.
__device__ __forceinline__ void bf16x8_to_f32(const uint4& v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__global__ __launch_bounds__(256) void moe_finalize_kernel(FwdParams p) {
  const int H = p.H, k = p.k;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int per_row = H / 8;
  if (idx >= static_cast<int64_t>(p.T) * per_row) return;
  const int64_t t = idx / per_row;
  const int n = static_cast<int>(idx % per_row) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (p.deterministic) {
    for (int j0 = 0; j0 < k; j0 += 8) {
      float w[8];
      uint4 y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // GEMM2 stored y by slot: token t's rows are t*k .. t*k + k - 1
        const int64_t sl = t * k + min(j0 + j, k - 1);
        w[j] = j0 + j < k ? p.topk_w[sl] : 0.0f;
        y[j] = *reinterpret_cast<const uint4*>(p.y + sl * H + n);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j0 + j < k) {
          float f[8];
          bf16x8_to_f32(y[j], f);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += w[j] * f[i];
        }
      }
    }
    if (p.shared) {
      float f[8];
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(p.y + (p.R + t) * H + n), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = (acc[i] + f[i]) * p.combine;
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p.out_acc + t * H + n);
    const float4 b = *reinterpret_cast<const float4*>(p.out_acc + t * H + n + 4);
    acc[0] = a.x; acc[1] = a.y; acc[2] = a.z; acc[3] = a.w;
    acc[4] = b.x; acc[5] = b.y; acc[6] = b.z; acc[7] = b.w;
  }
  uint4 o;
  o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
  o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
  o.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
  o.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
  *reinterpret_cast<uint4*>(p.out + t * H + n) = o;
}

// ---------------------------------------------------------------------------
// Weight packing into unit records (layout in kernels.hpp).  One thread per
// 16-byte destination chunk: chunks 0..255 of a record are code pieces, 256..287
// hold the scale bytes of two lanes each.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t unit_fragment_row(int64_t u, int f, int64_t N, int split) {
  const int64_t upe = N / 64;  // units per expert: 32 gate + 32 up rows, or 64 rows
  const int64_t e = u / upe, j = u - e * upe;
  const int64_t r = split ? (f < 2 ? 32 * j + 16 * f : N / 2 + 32 * j + 16 * (f - 2)) : 64 * j + 16 * f;
  return e * N + r;
}

// codes == nullptr: only the scale chunks are written (the records' codes
// stay as they are), one thread per scale chunk.
__global__ void pack_weights_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                    uint8_t* __restrict__ dst, int64_t units, int64_t N, int K,
                                    int split) {
  constexpr int kChunks = kRecBytes / 16;
  constexpr int kCodeChunks = kRecCodeBytes / 16;
  const int S = ksteps(K);
  const int per_rec = codes ? kChunks : kChunks - kCodeChunks;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= units * S * per_rec) return;
  const int64_t rec = c / per_rec;
  const int w = static_cast<int>(c - rec * per_rec) + (codes ? 0 : kCodeChunks);
  const int64_t u = rec / S;
  const int s = static_cast<int>(rec - u * S);
  uint4 v;
  if (w < kCodeChunks) {
    const int f = w / 64, l = w % 64;
    const int64_t row = unit_fragment_row(u, f, N, split) + (l & 15);
    v = *reinterpret_cast<const uint4*>(codes + row * (K / 2) + 64 * s + 16 * (l >> 4));
  } else {
    uint8_t out[16];
    const int l0 = 2 * (w - kCodeChunks);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int l = l0 + h;
#pragma unroll
      for (int f = 0; f < kUnitFrags; ++f) {
        const int64_t row = unit_fragment_row(u, f, N, split) + (l & 15);
        const uint8_t* src = scales + row * (K / 16) + 8 * s + 2 * (l >> 4);
        out[8 * h + 2 * f] = src[0];
        out[8 * h + 2 * f + 1] = src[1];
      }
    }
    __builtin_memcpy(&v, out, 16);
  }
  *reinterpret_cast<uint4*>(dst + (rec * kChunks + w) * 16) = v;
}

__global__ void copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

hipError_t launch_pack_weights(const uint8_t* codes, const uint8_t* scales, uint8_t* dst,
                               int64_t E, int64_t N, int64_t K, int split, hipStream_t s) {
  const int64_t units = E * (N / 64);
  const int per_rec = (codes ? kRecBytes : kRecBytes - kRecCodeBytes) / 16;
  const int64_t n = units * ksteps(static_cast<int>(K)) * per_rec;
  pack_weights_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
      codes, scales, dst, units, N, static_cast<int>(K), split);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s) {
  copy_f32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

template <int NB>
static void launch_route(const FwdParams& p, int nblocks, int tpb, hipStream_t s) {
  if (p.E <= 128)
    moe_route_kernel<NB, 2><<<nblocks, 256, 0, s>>>(p, tpb);
  else if (p.E <= 256)
    moe_route_kernel<NB, 4><<<nblocks, 256, 0, s>>>(p, tpb);
  else
    moe_route_kernel<NB, kMaxExperts / kWave><<<nblocks, 256, 0, s>>>(p, tpb);
  moe_schedule_kernel<<<(p.E + kSchedExperts - 1) / kSchedExperts, kSchedThreads, 0, s>>>(p, nblocks);
  moe_place_kernel<<<(p.R + 255) / 256, 256, 0, s>>>(p, tpb);
}

// NB: row registers of the one-row-per-wave quantizer; QB > 0: rows of more
// than 256 blocks of 16 use the one-row-per-256-threads quantizer with QB
// blocks per thread (more rows in flight per CU).
template <int NB, int QB>
static void launch_route64(const FwdParams& p, hipStream_t s) {
  const int nr = (p.T + kRoute64Tokens - 1) / kRoute64Tokens;
  const int nq = QB > 0 ? (p.T + 3) / 4 : (p.T + kSmallWaves - 1) / kSmallWaves;
  if (p.E <= 16) moe_route64_kernel<NB, 1, QB><<<nr + nq, kSmallThreads, 0, s>>>(p, nr);
  else if (p.E <= 32) moe_route64_kernel<NB, 2, QB><<<nr + nq, kSmallThreads, 0, s>>>(p, nr);
  else if (p.E <= 64) moe_route64_kernel<NB, 4, QB><<<nr + nq, kSmallThreads, 0, s>>>(p, nr);
  else if (p.E <= 128) moe_route64_kernel<NB, 8, QB><<<nr + nq, kSmallThreads, 0, s>>>(p, nr);
  else moe_route64_kernel<NB, 16, QB><<<nr + nq, kSmallThreads, 0, s>>>(p, nr);
  moe_place64_kernel<<<nr, kSmallThreads, 0, s>>>(p, nr);
}

hipError_t launch_moe_forward(const FwdParams& p, int max_tiles, hipStream_t s,
                              hipEvent_t const* ev) {
  if (ev) (void)hipEventRecord(ev[0], s);
  if (use_tiny_prologue(p)) {
    const int nbl = (p.H / 16 + 255) / 256;
    if (nbl <= 1) launch_prologue_tiny<1>(p, s);
    else if (nbl <= 2) launch_prologue_tiny<2>(p, s);
    else if (nbl <= 4) launch_prologue_tiny<4>(p, s);
    else launch_prologue_tiny<8>(p, s);
  } else if (use_small_prologue(p)) {
    switch (quant_nb_for_cols(p.H)) {
      case 1: launch_prologue_small<1>(p, s); break;
      case 2: launch_prologue_small<2>(p, s); break;
      case 4: launch_prologue_small<4>(p, s); break;
      case 8: launch_prologue_small<8>(p, s); break;
      default: launch_prologue_small<0>(p, s); break;
    }
  } else if (use_route64_prologue(p)) {
    const int nblk = p.H / 16;
    if (nblk <= 64) launch_route64<1, 0>(p, s);
    else if (nblk <= 128) launch_route64<2, 0>(p, s);
    else if (nblk <= 256) launch_route64<4, 0>(p, s);
    else if (nblk <= 512) launch_route64<1, 2>(p, s);
    else if (nblk <= 1024) launch_route64<1, 4>(p, s);
    else if (nblk <= 2048) launch_route64<1, 8>(p, s);
    else launch_route64<0, 0>(p, s);
  } else {
    const int tpb = route_tokens_per_block(p.T);
    const int nblocks = (p.T + tpb - 1) / tpb;
    switch (quant_nb_for_cols(p.H)) {
      case 1: launch_route<1>(p, nblocks, tpb, s); break;
      case 2: launch_route<2>(p, nblocks, tpb, s); break;
      case 4: launch_route<4>(p, nblocks, tpb, s); break;
      case 8: launch_route<8>(p, nblocks, tpb, s); break;
      default: launch_route<0>(p, nblocks, tpb, s); break;
    }
  }
  if (ev) (void)hipEventRecord(ev[1], s);
  const hipError_t ge = launch_grouped_gemms(p, max_tiles, s, ev);
  if (ge != hipSuccess) return ge;
  const int64_t nthreads = static_cast<int64_t>(p.T) * (p.H / 8);
  moe_finalize_kernel<<<static_cast<unsigned>((nthreads + 255) / 256), 256, 0, s>>>(p);
  if (ev) (void)hipEventRecord(ev[4], s);
  return hipGetLastError();
}

}  // namespace nvfp4
