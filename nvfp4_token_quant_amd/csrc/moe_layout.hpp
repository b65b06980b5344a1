// Host-side internals shared by the C-ABI entry points: the byte layout of
// every device buffer a forward uses (carved out of one block of device
// memory), and the forward's launch sequence on those buffers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_moe.h"
#include "kernels.hpp"

namespace nvfp4 {

// Every device buffer of a forward of at most T_cap tokens.  The weights are
// not here: the packed records are the caller's, and the per-expert global
// scales are either the workspace's copies (w13g / w2g below) or the
// caller's arrays.
struct FwdBuffers {
  int64_t T_cap;
  int64_t max_tiles_cap;
  int route_blocks_cap;
  uint8_t* dummy;  // kRecBytes: target of prefetches past a wave's last K step
  // activation quantization
  uint8_t* xq_codes;
  uint8_t* xq_scales;
  float* xq_g;
  _Float16* xq16;
  // routing / permutation
  int32_t* topk_ids;
  float* topk_w;
  int32_t* loc_rank;
  int32_t* blk_counts;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  int4* tiles;
  int32_t* n_tiles;
  float* act_scales;  // [2] static g_x, g_a (MOE_STATIC_ACT_SCALES)
  // intermediates
  float* act;
  float* act_amax;
  uint8_t* a2_codes;
  uint8_t* a2_scales;
  float* a2_g;
  _Float16* a2q16;
  uint16_t* y;  // bf16
  float* out_acc;
  // library copies of the per-expert global scales (own_gscales)
  float* w13g;
  float* w2g;
};

bool cfg_has_shared(const moe_config& c);
int64_t cfg_weight_experts(const moe_config& c);

// Validates a configuration (dims, flags, limits); NVFP4_OK or a status with
// the error message set.
int check_config(const moe_config& c);

// Lays the buffers of a forward of at most T_cap tokens out in one block
// (each piece 256-byte aligned, the dummy record first) and returns the
// block's size.  base == nullptr: sizes only (the pointers are offsets from
// 0).  own_gscales: also room for the copies of the global scales.
int64_t layout_buffers(const moe_config& c, int64_t T_cap, bool own_gscales, uint8_t* base, FwdBuffers* b);

// The weights a forward reads.
struct WeightView {
  const uint8_t* w13;
  const uint8_t* w2;
  const float* w13g;
  const float* w2g;
};

// Activations handed over already quantized (codes [T, H/2], scales
// [T, H/16], global scales [T]); on = false: the forward quantizes x itself.
struct XQ {
  bool on;
  const void* codes;
  const void* scales;
  const float* g;
};

// Host checks, then the forward's kernels on `s` (no allocation, no host
// synchronization).  static_scales_set: the act_scales buffer holds values
// (required with MOE_STATIC_ACT_SCALES).
int run_forward(const moe_config& c, const FwdBuffers& b, const WeightView& w, bool static_scales_set,
                const void* x, const XQ& xq, const float* logits, int64_t T, void* out, hipStream_t s,
                const hipEvent_t* events);

// Checks of a packed-weights descriptor against a configuration.
int check_packed(const moe_config& c, const moe_nvfp4_packed* w);

// The thread-local error message of the C-ABI.
int api_fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int api_ok();
const char* last_error_text();

}  // namespace nvfp4
