// Host-side declarations of the kernel launchers and the forward's parameter
// block.  Shared by the kernel sources and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kMaxRouteBlocks = 1024;      // prologue blocks for T <= 131072
constexpr int kMaxTokensPerRouteBlock = 128;

// Tokens per prologue block: one token per wave up to 4096 tokens, then as
// many as keep the block count at kMaxRouteBlocks.
inline int route_tokens_per_block(int64_t T) {
  if (T <= 4 * kMaxRouteBlocks) return 4;
  int64_t tpb = (T + kMaxRouteBlocks - 1) / kMaxRouteBlocks;
  tpb = (tpb + 3) / 4 * 4;
  return static_cast<int>(tpb > kMaxTokensPerRouteBlock ? kMaxTokensPerRouteBlock : tpb);
}

// Expert weights are re-laid out once at bind time into unit records, so that
// a wave that owns one unit reads one contiguous 4.5 KB piece per K step.
// A unit is four 16-row fragments of one expert's matrix: for W13 [2I, H]
// unit j holds gate rows 32j..32j+31 (fragments 0, 1) and the matching up
// rows I+32j..I+32j+31 (fragments 2, 3); for W2 [H, I] unit j holds rows
// 64j..64j+63.  Record (u, s) for unit u and 128-wide K step s sits at
// (u * ksteps(K) + s) * kRecBytes:
//   bytes [1024 f + 16 l, + 16): lane l of fragment f = row 16 f' + l % 16
//     of the fragment, code bytes [64 s + 16 (l / 16), + 16) of that row
//     (32 codes, k = 128 s + 32 (l / 16) + 0..31);
//   bytes [4096 + 8 l + 2 f, + 2): the two E4M3 scales of that lane's 32
//     codes (blocks 8 s + 2 (l / 16) + {0, 1}).
constexpr int kUnitFrags = 4;
constexpr int kRecCodeBytes = 4096;
constexpr int kRecBytes = kRecCodeBytes + 512;
__host__ __device__ constexpr int ksteps(int K) { return K / 128; }
__host__ __device__ constexpr int64_t w13_units(int64_t E, int64_t I) { return E * (I / 32); }
__host__ __device__ constexpr int64_t w2_units(int64_t E, int64_t H) { return E * (H / 64); }
__host__ __device__ constexpr int64_t packed_bytes(int64_t units, int K) {
  return units * ksteps(K) * kRecBytes;
}

// Grouped-GEMM kernel families.
//   stream: tiles of up to 16*fm rows (fm = 1, 2); the whole token operand of
//           the tile is staged once in LDS as FP4 codes + scales; each wave
//           streams the records of one unit (or a K range of it) with a
//           register prefetch.
//   tiled:  64- or 128-row tiles; the token operand is read as fp16 (the
//           exact dequantized copy the prologue / re-quantization write) and
//           staged in LDS one K step at a time.
enum GemmKind { kGemmStream = 0, kGemmTiled = 1 };

struct FwdParams {
  // R = T*k routed expanded rows [0, R), in expert order.  With a shared
  // expert (shared = 1) the rows [R, R + T) follow: row R + t is token t
  // applied to expert E; Rt is the total.
  int T, H, I, E, k, R, Rt;
  int shared;         // 1: expert E is applied to every token with weight 1
  float combine;      // output scale: 1 (routed + shared), 0.5 ('average')
  int mt;             // rows per M-tile of the grouped GEMMs
  int gemm_kind;      // GemmKind
  int g1_ks, g2_ks;   // stream kernels: waves sharing one unit's K range (1, 2, 4)
  int g1_bands;       // GEMM1 column bands (partial row amaxes per expanded row)
  int tiled_gx;       // tiled kernels: tile slots of the grid (max tiles rounded up to 8)
  int deterministic;  // 1: slot-ordered finalize; 0: fp32 atomics into out_acc
  int a16;            // 1: W4A16 (x and act as bf16 GEMM inputs, no activation quantization)
  int preq;           // 1: x handed over already quantized: xq_codes / xq_scales / xq_g are
                      //    the caller's (read only), x is not read
  const float* static_g;  // NULL, or [2] static global scales of x and of GEMM2's input
  // caller tensors
  const uint16_t* x;
  const float* logits;
  uint16_t* out;
  // per-token quantized activations
  uint8_t* xq_codes;
  uint8_t* xq_scales;
  float* xq_g;
  _Float16* xq16;  // [T, H] the same values dequantized (code x block scale, exact in fp16); tiled path only
  // routing and expandInputRows
  int32_t* topk_ids;
  float* topk_w;
  int32_t* loc_rank;    // [T*k] rank among equal experts inside a prologue block
  int32_t* blk_counts;  // [nblocks, E] per-block counts, then per-block bases
  int32_t* counts;      // [E]
  int32_t* offsets;     // [E+1]
  int32_t* perm;        // [R] routed row -> t*k+j
  int32_t* inv;         // [R] t*k+j -> row
  int4* tiles;          // [max_tiles] (expert, row0, nrows, 0)
  int32_t* n_tiles;     // device scalar
  // intermediates
  float* act;       // [Rt, I]
  float* act_amax;  // [Rt, g1_bands <= I / 32] partial row amax per GEMM1 column band
  uint8_t* a2_codes;
  uint8_t* a2_scales;
  float* a2_g;
  _Float16* a2q16;  // [Rt, I] dequantized re-quantized act (exact in fp16); tiled path only
                    // (W4A16: act rounded to bf16, the same 16-bit slots)
  uint16_t* y;     // [Rt, H] bf16 expert outputs by slot (deterministic finalize)
  float* out_acc;  // [T, H] (atomic finalize)
  // weights: unit records (see kRecBytes) and per-expert global scales
  const uint8_t* w13;
  const float* w13g;
  const uint8_t* w2;
  const float* w2g;
  const uint8_t* dummy;  // kRecBytes of zeros: target of loads past a wave's last K step
};

// Expanded-row helpers.  A routed row's slot is t*k + j (from perm); a
// shared row's slot is the row itself (>= R), so one int names every row's
// token and output weight.
__device__ __forceinline__ int row_slot(const FwdParams& p, int row) { return row < p.R ? p.perm[row] : row; }
__device__ __forceinline__ int slot_token(const FwdParams& p, int slot) {
  return slot < p.R ? slot / p.k : slot - p.R;
}
// weight of a slot in the output sum, the combination scale included
__device__ __forceinline__ float slot_weight(const FwdParams& p, int slot) {
  return slot < p.R ? p.topk_w[slot] * p.combine : p.combine;
}
// Append the shared expert's tiles (rows R .. R + T - 1, expert E) after the
// routed tiles; returns the new tile count.  Called by one thread.
__device__ __forceinline__ int append_shared_tiles(const FwdParams& p, int ntiles) {
  if (!p.shared) return ntiles;
  const int nt = (p.T + p.mt - 1) / p.mt;
  for (int i = 0; i < nt; ++i)
    p.tiles[ntiles + i] = make_int4(p.E, p.R + i * p.mt, min(p.mt, p.T - i * p.mt), 0);
  return ntiles + nt;
}

// quantize.hip
int quant_nb_for_cols(int64_t cols);
hipError_t launch_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                uint8_t* codes, uint8_t* scales, float* gs, hipStream_t s);
hipError_t launch_quantize_experts(const float* w, int64_t experts, int64_t rows, int64_t cols,
                                   uint8_t* codes, uint8_t* scales, float* gs, uint32_t* amax_bits,
                                   hipStream_t s);

// gemm_kernels.hip
// Rows per tile and kernel family for a forward of T tokens.
void choose_gemm(int64_t T, FwdParams* p);
// Dynamic LDS bytes of the stream kernel for reduction length K.
int stream_lds_bytes(int fm, int K);
hipError_t launch_grouped_gemms(const FwdParams& p, int max_tiles, hipStream_t s,
                                hipEvent_t const* events);

// moe_kernels.hip
// events: NULL or 5 events recorded around the four kernels.
hipError_t launch_moe_forward(const FwdParams& p, int max_tiles, hipStream_t s,
                              hipEvent_t const* events);
// Copy row-major codes [E, N, K/2] and scales [E, N, K/16] of one weight
// matrix into unit records.  w13: N = 2I, split = 1 (gate / up halves);
// w2: N = H, split = 0.  N % 64 == 0, K % 128 == 0.  codes == nullptr:
// only the records' scale bytes are written.
hipError_t launch_pack_weights(const uint8_t* codes, const uint8_t* scales, uint8_t* dst,
                               int64_t E, int64_t N, int64_t K, int split, hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);

}  // namespace nvfp4
