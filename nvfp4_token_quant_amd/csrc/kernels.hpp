// Host-side declarations of the kernel launchers and the forward's parameter
// block.  Shared by the kernel sources and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Tokens handled by one block of the forward's prologue kernel.
constexpr int kRouteTokensPerBlock = 16;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;

struct FwdParams {
  int T, H, I, E, k, R;
  int mt;             // rows per M-tile of the grouped GEMMs
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
  float* act_amax;  // [R, I / g1_cols]
  uint8_t* a2_codes;
  uint8_t* a2_scales;
  float* a2_g;
  float* y;        // [R, H] (deterministic finalize)
  float* out_acc;  // [T, H] (atomic finalize)
  // weights: codes borrowed, scales in the kernels' layout (see swizzle)
  const uint8_t* w13c;
  const uint8_t* w13s;
  const float* w13g;
  const uint8_t* w2c;
  const uint8_t* w2s;
  const float* w2g;
};

// quantize.hip
int quant_nb_for_cols(int64_t cols);
hipError_t launch_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                uint8_t* codes, uint8_t* scales, float* gs, hipStream_t s);
hipError_t launch_quantize_experts(const float* w, int64_t experts, int64_t rows, int64_t cols,
                                   uint8_t* codes, uint8_t* scales, float* gs, uint32_t* amax_bits,
                                   hipStream_t s);

// moe_kernels.hip
// Columns of the gate/up output (act columns) one GEMM1 block covers.
int gemm1_cols_per_block();
// events: NULL or 5 events recorded around the four kernels.
hipError_t launch_moe_forward(const FwdParams& p, int max_tiles, hipStream_t s,
                              hipEvent_t const* events);
// Copy [groups*rows, K/16] row-major E4M3 scales into the GEMM layout.
hipError_t launch_swizzle_scales(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t K,
                                 hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);

}  // namespace nvfp4
