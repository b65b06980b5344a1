// Host-side declarations of the kernel launchers and the forward's parameter
// block.  Shared by the kernel sources and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kMaxRouteBlocks = 256;       // prologue blocks for T <= 32768
constexpr int kMaxTokensPerRouteBlock = 128;

// Tokens per prologue block: one token per wave up to 1024 tokens, then as
// many as keep the block count at kMaxRouteBlocks.
inline int route_tokens_per_block(int64_t T) {
  if (T <= 4 * kMaxRouteBlocks) return 4;
  int64_t tpb = (T + kMaxRouteBlocks - 1) / kMaxRouteBlocks;
  tpb = (tpb + 3) / 4 * 4;
  return static_cast<int>(tpb > kMaxTokensPerRouteBlock ? kMaxTokensPerRouteBlock : tpb);
}

// Expert weights are kept in a fragment-major layout so that one wave load
// reads 1 KB of contiguous memory.  A weight matrix [N, K] (N % 16 == 0,
// K % 128 == 0; the experts' matrices stacked along N) is cut into 16-row
// groups i and 128-wide K steps s:
//   codes:  block (i, s) = 1 KB at ((i * steps(K) + s) * 1024); lane l of a
//           wave owns bytes [16 l, 16 l + 16) = row 16 i + l % 16, code bytes
//           [64 s + 16 (l / 16), + 16) of that row (32 codes, k = 128 s +
//           32 (l / 16) + 0..31).
//   scales: block (i, q) = 1 KB at ((i * sgroups(K) + q) * 1024) for steps
//           8 q .. 8 q + 7; lane l owns 16 bytes: for step 8 q + t the two
//           E4M3 bytes of blocks 8 s + 2 (l / 16) + {0, 1} of row 16 i + l % 16
//           at bytes 2 t, 2 t + 1 (zero past the last step).
__host__ __device__ constexpr int ksteps(int K) { return K / 128; }
__host__ __device__ constexpr int sgroups(int K) { return (K / 128 + 7) / 8; }
__host__ __device__ constexpr int64_t packed_scale_bytes(int64_t rows, int K) {
  return rows / 16 * sgroups(K) * 1024;
}

// Grouped-GEMM kernel families.
//   stream: tiles of up to 16*fm rows (fm = 1, 2); the whole token operand of
//           the tile is staged once in LDS as FP4 codes + scales, and each
//           wave streams its weight rows with a 4-step register prefetch.
//   tiled:  64-row tiles; token operand staged in K chunks as fp16.
enum GemmKind { kGemmStream = 0, kGemmTiled = 1 };

struct FwdParams {
  int T, H, I, E, k, R;
  int mt;             // rows per M-tile of the grouped GEMMs
  int gemm_kind;      // GemmKind
  int g1_fn, g2_fn;   // stream kernels: 16-row weight fragments per wave
  int g1_bands;       // GEMM1 column bands (partial row amaxes per expanded row)
  int deterministic;  // 1: slot-ordered finalize; 0: fp32 atomics into out_acc
  // caller tensors
  const uint16_t* x;
  const float* logits;
  uint16_t* out;
  // per-token quantized activations
  uint8_t* xq_codes;
  uint8_t* xq_scales;
  float* xq_g;
  // routing and expandInputRows
  int32_t* topk_ids;
  float* topk_w;
  int32_t* loc_rank;    // [T*k] rank among equal experts inside a prologue block
  int32_t* blk_counts;  // [nblocks, E] per-block counts, then per-block bases
  int32_t* counts;      // [E]
  int32_t* offsets;     // [E+1]
  int32_t* perm;        // [R] row -> t*k+j
  int32_t* inv;         // [R] t*k+j -> row
  int4* tiles;          // [max_tiles] (expert, row0, nrows, 0)
  int32_t* n_tiles;     // device scalar
  uint32_t* ticket;     // device scalar, 0 between launches
  // intermediates
  float* act;       // [R, I]
  float* act_amax;  // [R, I / 64] partial row amax per GEMM1 column band
  uint8_t* a2_codes;
  uint8_t* a2_scales;
  float* a2_g;
  float* y;        // [R, H] (deterministic finalize)
  float* out_acc;  // [T, H] (atomic finalize)
  // weights, fragment-major copies (see ksteps / sgroups)
  const uint8_t* w13c;
  const uint8_t* w13s;
  const float* w13g;
  const uint8_t* w2c;
  const uint8_t* w2s;
  const float* w2g;
  const uint8_t* dummy;  // 1 KB of zeros: target of loads past the last K step
};

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
// Copy row-major codes [rows, K/2] / scales [rows, K/16] into the
// fragment-major layout (rows % 16 == 0, K % 128 == 0).
hipError_t launch_pack_codes(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t K,
                             hipStream_t s);
hipError_t launch_pack_scales(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t K,
                              hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);

}  // namespace nvfp4
