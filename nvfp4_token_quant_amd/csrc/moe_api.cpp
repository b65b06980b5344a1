// C-ABI of the NVFP4 fused-MoE layer: argument checks, the workspace (every
// buffer allocated once from the configured token ceiling), weight binding,
// in-place scale refresh and the forward's launch sequence.
//
// [P2] (sglang PR #26696 report), "Feature and motivation" and
// "Implementation breakdown": buffers sized from the first forward's batch
// crashed later batches ("num_tokens (4073) exceeds max_num_tokens (2048)");
// the ceiling now comes from configuration.  [P1] (sglang PR #28354 summary),
// "Implementation breakdown" item 3 and "Source snippets": after a weight
// reload the scales are copied into the existing tensors so that captured
// graphs keep valid addresses, and a metadata change is an error.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "nvfp4_moe.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return NVFP4_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + static_cast<uintptr_t>(nb) && y < x + static_cast<uintptr_t>(na);
}

}  // namespace

struct moe_workspace {
  moe_config cfg;
  int device;
  int64_t max_tiles_cap;
  int route_blocks_cap;
  // activation quantization
  uint8_t* xq_codes;
  uint8_t* xq_scales;
  float* xq_g;
  _Float16* xq16;  // fp16 copies of the quantized token operands (tiled path)
  _Float16* a2q16;
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
  bool act_scales_set;
  // intermediates
  float* act;
  float* act_amax;
  uint8_t* a2_codes;
  uint8_t* a2_scales;
  float* a2_g;
  float* y;
  float* out_acc;
  // weights
  bool bound;
  const void* bound_w13c;  // caller's code pointers at bind time
  const void* bound_w2c;
  uint8_t* w13;  // unit-record copies of codes + scales
  uint8_t* w2;
  float* w13g;
  float* w2g;
  uint8_t* dummy;
  // optional stage-timing events (caller-owned)
  bool timing;
  hipEvent_t events[5];
};

namespace {

bool has_shared(const moe_config& c) { return (c.flags & MOE_SHARED_EXPERT) != 0; }
// expanded rows of the shared expert (one per token of the ceiling)
int64_t shared_rows(const moe_config& c) { return has_shared(c) ? c.max_num_tokens : 0; }
// experts held by the weight buffers (the shared one last)
int64_t weight_experts(const moe_config& c) { return c.num_experts + (has_shared(c) ? 1 : 0); }

// Every buffer the workspace owns, in one list for allocation and release.
template <typename F>
void for_each_buffer(moe_workspace* w, F&& f) {
  const moe_config& c = w->cfg;
  const int64_t T = c.max_num_tokens, H = c.hidden, I = c.inter, E = c.num_experts, k = c.top_k;
  const int64_t R = T * k;               // routed rows
  const int64_t Rt = R + shared_rows(c);  // GEMM rows
  const int64_t Ew = weight_experts(c);
  const int64_t n_amax = I / 32;  // GEMM1 column bands of 32 (the finest band used)
  const bool det = (c.flags & MOE_DETERMINISTIC_FINALIZE) != 0;
  f(reinterpret_cast<void**>(&w->xq_codes), T * H / 2);
  f(reinterpret_cast<void**>(&w->xq_scales), T * H / 16);
  f(reinterpret_cast<void**>(&w->xq_g), T * 4);
  f(reinterpret_cast<void**>(&w->xq16), T * H * 2);
  f(reinterpret_cast<void**>(&w->topk_ids), R * 4);
  f(reinterpret_cast<void**>(&w->topk_w), R * 4);
  f(reinterpret_cast<void**>(&w->loc_rank), R * 4);
  f(reinterpret_cast<void**>(&w->blk_counts), static_cast<int64_t>(w->route_blocks_cap) * E * 4);
  f(reinterpret_cast<void**>(&w->counts), E * 4);
  f(reinterpret_cast<void**>(&w->offsets), (E + 1) * 4);
  f(reinterpret_cast<void**>(&w->perm), R * 4);
  f(reinterpret_cast<void**>(&w->inv), R * 4);
  f(reinterpret_cast<void**>(&w->tiles), w->max_tiles_cap * 16);
  f(reinterpret_cast<void**>(&w->n_tiles), 4);
  f(reinterpret_cast<void**>(&w->act_scales), 2 * 4);
  f(reinterpret_cast<void**>(&w->act), Rt * I * 4);
  f(reinterpret_cast<void**>(&w->act_amax), Rt * n_amax * 4);
  f(reinterpret_cast<void**>(&w->a2_codes), Rt * I / 2);
  f(reinterpret_cast<void**>(&w->a2_scales), Rt * I / 16);
  f(reinterpret_cast<void**>(&w->a2_g), Rt * 4);
  f(reinterpret_cast<void**>(&w->a2q16), Rt * I * 2);
  f(reinterpret_cast<void**>(&w->y), det ? Rt * H * 4 : 0);
  f(reinterpret_cast<void**>(&w->out_acc), det ? 0 : T * H * 4);
  f(reinterpret_cast<void**>(&w->w13), nvfp4::packed_bytes(nvfp4::w13_units(Ew, I), static_cast<int>(H)));
  f(reinterpret_cast<void**>(&w->w2), nvfp4::packed_bytes(nvfp4::w2_units(Ew, H), static_cast<int>(I)));
  f(reinterpret_cast<void**>(&w->w13g), Ew * 4);
  f(reinterpret_cast<void**>(&w->w2g), Ew * 4);
  f(reinterpret_cast<void**>(&w->dummy), nvfp4::kRecBytes);
}

void free_all(moe_workspace* w) {
  for_each_buffer(w, [](void** p, int64_t) {
    if (*p) (void)hipFree(*p);
    *p = nullptr;
  });
}

// Tiles of R routed rows over E experts, plus those of the shared expert's
// T rows (shared_T = 0 without one).
int64_t tiles_bound(int64_t R, int64_t E, int mt, int64_t shared_T) {
  return (R + mt - 1) / mt + std::min(E, R) + (shared_T + mt - 1) / mt;
}

int check_weights_desc(const moe_workspace* ws, const moe_nvfp4_weights* w, bool need_codes) {
  if (!w) return fail(NVFP4_ERR_INVALID_ARG, "weights descriptor is NULL");
  const moe_config& c = ws->cfg;
  if (w->num_experts != weight_experts(c) || w->hidden != c.hidden || w->inter != c.inter)
    return fail(NVFP4_ERR_METADATA_CHANGED,
                "weight dims (E=%lld, H=%lld, I=%lld) differ from the workspace's (E=%lld, H=%lld, "
                "I=%lld); recapture is required",
                (long long)w->num_experts, (long long)w->hidden, (long long)w->inter,
                (long long)weight_experts(c), (long long)c.hidden, (long long)c.inter);
  if (!w->w13_scales || !w->w2_scales || !w->w13_gscale || !w->w2_gscale)
    return fail(NVFP4_ERR_INVALID_ARG, "weight scale pointers must be non-NULL");
  if (!aligned(w->w13_gscale, 4) || !aligned(w->w2_gscale, 4))
    return fail(NVFP4_ERR_INVALID_ARG, "global scale pointers must be 4-byte aligned");
  if (need_codes) {
    if (!w->w13_codes || !w->w2_codes)
      return fail(NVFP4_ERR_INVALID_ARG, "weight code pointers must be non-NULL");
    if (!aligned(w->w13_codes, 16) || !aligned(w->w2_codes, 16))
      return fail(NVFP4_ERR_INVALID_ARG, "weight code pointers must be 16-byte aligned");
  }
  return NVFP4_OK;
}

// Copy codes and scales into the library's unit-record buffers (same
// addresses on every call) and the global scales into their own buffers.
hipError_t copy_weights(moe_workspace* ws, const moe_nvfp4_weights* w, const void* w13c,
                        const void* w2c, hipStream_t s) {
  const moe_config& c = ws->cfg;
  const int64_t E = weight_experts(c), H = c.hidden, I = c.inter;
  hipError_t e = nvfp4::launch_pack_weights(static_cast<const uint8_t*>(w13c),
                                            static_cast<const uint8_t*>(w->w13_scales), ws->w13, E,
                                            2 * I, H, 1, s);
  if (e == hipSuccess)
    e = nvfp4::launch_pack_weights(static_cast<const uint8_t*>(w2c), static_cast<const uint8_t*>(w->w2_scales),
                                   ws->w2, E, H, I, 0, s);
  if (e == hipSuccess) e = nvfp4::launch_copy_f32(w->w13_gscale, ws->w13g, E, s);
  if (e == hipSuccess) e = nvfp4::launch_copy_f32(w->w2_gscale, ws->w2g, E, s);
  return e;
}

}  // namespace

extern "C" {

const char* nvfp4_last_error(void) { return g_last_error.c_str(); }

int nvfp4_quantize_per_token(const void* x_dev, int64_t rows, int64_t cols, int64_t ld_x,
                             void* codes_dev, void* scales_dev, float* gscale_dev, void* stream) {
  if (rows < 0) return fail(NVFP4_ERR_INVALID_ARG, "rows must be >= 0 (got %lld)", (long long)rows);
  if (cols <= 0 || cols % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "cols must be a positive multiple of 16 (got %lld)", (long long)cols);
  if (cols > (int64_t(1) << 30)) return fail(NVFP4_ERR_INVALID_ARG, "cols too large");
  if (ld_x < cols || ld_x % 8 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "ld_x must be >= cols and a multiple of 8 (got %lld)", (long long)ld_x);
  if (rows == 0) return ok();
  if (rows > INT32_MAX) return fail(NVFP4_ERR_INVALID_ARG, "rows must be < 2^31 (got %lld)", (long long)rows);
  if (!x_dev || !codes_dev || !scales_dev || !gscale_dev)
    return fail(NVFP4_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(x_dev, 16) || !aligned(codes_dev, 16) || !aligned(gscale_dev, 4))
    return fail(NVFP4_ERR_INVALID_ARG, "x and codes must be 16-byte aligned, gscale 4-byte aligned");
  const int64_t xbytes = ((rows - 1) * ld_x + cols) * 2;
  if (overlap(x_dev, xbytes, codes_dev, rows * cols / 2) ||
      overlap(x_dev, xbytes, scales_dev, rows * cols / 16) || overlap(x_dev, xbytes, gscale_dev, rows * 4))
    return fail(NVFP4_ERR_ALIAS, "outputs overlap the input x");
  hipError_t e = nvfp4::launch_quantize_rows(static_cast<const uint16_t*>(x_dev), rows, cols, ld_x,
                                             static_cast<uint8_t*>(codes_dev),
                                             static_cast<uint8_t*>(scales_dev), gscale_dev,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "nvfp4_quantize_per_token launch");
  return ok();
}

int nvfp4_quantize_experts(const float* w_dev, int64_t experts, int64_t rows, int64_t cols,
                           void* codes_dev, void* scales_dev, float* gscale_dev, float* scratch_dev,
                           void* stream) {
  if (experts < 1 || experts > 65535 || rows < 1 || cols <= 0 || cols % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARG,
                "need 1 <= experts <= 65535, rows >= 1, cols a positive multiple of 16");
  if (!w_dev || !codes_dev || !scales_dev || !gscale_dev || !scratch_dev)
    return fail(NVFP4_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(w_dev, 16) || !aligned(codes_dev, 16) || !aligned(gscale_dev, 4) || !aligned(scratch_dev, 4))
    return fail(NVFP4_ERR_INVALID_ARG, "w and codes must be 16-byte aligned");
  const int64_t n = experts * rows * cols;
  if (overlap(w_dev, n * 4, codes_dev, n / 2) || overlap(w_dev, n * 4, scales_dev, n / 16))
    return fail(NVFP4_ERR_ALIAS, "outputs overlap the input");
  hipError_t e = nvfp4::launch_quantize_experts(w_dev, experts, rows, cols, static_cast<uint8_t*>(codes_dev),
                                                static_cast<uint8_t*>(scales_dev), gscale_dev,
                                                reinterpret_cast<uint32_t*>(scratch_dev),
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "nvfp4_quantize_experts launch");
  return ok();
}

int moe_workspace_create(const moe_config* cfg, void* stream, moe_workspace** out) {
  if (!cfg || !out) return fail(NVFP4_ERR_INVALID_ARG, "NULL cfg or out");
  *out = nullptr;
  const moe_config c = *cfg;
  if (c.max_num_tokens < 1 || c.max_num_tokens > (int64_t(1) << 24))
    return fail(NVFP4_ERR_INVALID_ARG, "max_num_tokens must be in [1, 2^24] (got %lld)",
                (long long)c.max_num_tokens);
  if (c.hidden < 128 || c.hidden % 128 != 0 || c.hidden > 65536)
    return fail(NVFP4_ERR_INVALID_ARG, "hidden must be a multiple of 128 in [128, 65536] (got %lld)",
                (long long)c.hidden);
  if (c.inter < 128 || c.inter % 128 != 0 || c.inter > 65536)
    return fail(NVFP4_ERR_INVALID_ARG, "inter must be a multiple of 128 in [128, 65536] (got %lld)",
                (long long)c.inter);
  if (c.num_experts < 1 || c.num_experts > nvfp4::kMaxExperts)
    return fail(NVFP4_ERR_INVALID_ARG, "num_experts must be in [1, %d]", nvfp4::kMaxExperts);
  if (c.top_k < 1 || c.top_k > nvfp4::kMaxTopK || c.top_k > c.num_experts)
    return fail(NVFP4_ERR_INVALID_ARG, "top_k must be in [1, min(%d, num_experts)]", nvfp4::kMaxTopK);
  if ((c.flags & ~(MOE_DETERMINISTIC_FINALIZE | MOE_STATIC_ACT_SCALES | MOE_SHARED_EXPERT |
                   MOE_SHARED_AVERAGE | MOE_W4A16)) != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "unknown flags 0x%x", c.flags);
  if ((c.flags & MOE_W4A16) && (c.flags & MOE_STATIC_ACT_SCALES))
    return fail(NVFP4_ERR_INVALID_ARG, "MOE_W4A16 quantizes no activations: MOE_STATIC_ACT_SCALES does not apply");
  if ((c.flags & MOE_SHARED_AVERAGE) && !(c.flags & MOE_SHARED_EXPERT))
    return fail(NVFP4_ERR_INVALID_ARG, "MOE_SHARED_AVERAGE requires MOE_SHARED_EXPERT");
  if (c.num_experts + ((c.flags & MOE_SHARED_EXPERT) ? 1 : 0) > nvfp4::kMaxExperts)
    return fail(NVFP4_ERR_INVALID_ARG, "num_experts plus the shared expert must be <= %d", nvfp4::kMaxExperts);
  if (c.max_num_tokens * (c.top_k + 1) > (int64_t(1) << 30))
    return fail(NVFP4_ERR_INVALID_ARG, "max_num_tokens * (top_k + 1) too large");
  if (c.max_num_tokens * c.hidden >= (int64_t(1) << 30))
    return fail(NVFP4_ERR_INVALID_ARG, "max_num_tokens * hidden must be < 2^30 (got %lld)",
                (long long)(c.max_num_tokens * c.hidden));
  moe_workspace* w = new (std::nothrow) moe_workspace();
  if (!w) return fail(NVFP4_ERR_OOM, "host allocation failed");
  std::memset(static_cast<void*>(w), 0, sizeof(*w));
  w->cfg = c;
  if (hipGetDevice(&w->device) != hipSuccess) {
    delete w;
    return fail(NVFP4_ERR_HIP, "hipGetDevice failed");
  }
  const int64_t Rmax = c.max_num_tokens * c.top_k;
  w->max_tiles_cap = tiles_bound(Rmax, c.num_experts, 16, shared_rows(c));
  w->route_blocks_cap = static_cast<int>(std::max<int64_t>(
      nvfp4::kMaxRouteBlocks,
      (c.max_num_tokens + nvfp4::kMaxTokensPerRouteBlock - 1) / nvfp4::kMaxTokensPerRouteBlock));
  int status = NVFP4_OK;
  for_each_buffer(w, [&](void** p, int64_t bytes) {
    if (status != NVFP4_OK || bytes <= 0) return;
    hipError_t e = hipMalloc(p, static_cast<size_t>(bytes));
    if (e != hipSuccess) {
      *p = nullptr;
      status = fail(NVFP4_ERR_OOM, "hipMalloc of %lld bytes failed: %s", (long long)bytes,
                    hipGetErrorString(e));
    }
  });
  if (status != NVFP4_OK) {
    free_all(w);
    delete w;
    return status;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = nvfp4::launch_fill_u32(reinterpret_cast<uint32_t*>(w->dummy), nvfp4::kRecBytes / 4, 0u, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    free_all(w);
    delete w;
    return hip_fail(e, "workspace initialization");
  }
  *out = w;
  return ok();
}

int moe_workspace_bind_weights(moe_workspace* ws, const moe_nvfp4_weights* w, void* stream) {
  if (!ws) return fail(NVFP4_ERR_INVALID_ARG, "NULL workspace");
  if (ws->bound) return fail(NVFP4_ERR_INVALID_ARG, "weights already bound; use refresh_scales_inplace");
  int st = check_weights_desc(ws, w, true);
  if (st != NVFP4_OK) {
    if (st == NVFP4_ERR_METADATA_CHANGED) g_last_error = "weight dims do not match the workspace";
    return st == NVFP4_ERR_METADATA_CHANGED ? NVFP4_ERR_INVALID_ARG : st;
  }
  hipError_t e = copy_weights(ws, w, w->w13_codes, w->w2_codes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "weight copy");
  ws->bound_w13c = w->w13_codes;
  ws->bound_w2c = w->w2_codes;
  ws->bound = true;
  return ok();
}

int refresh_scales_inplace(moe_workspace* ws, const moe_nvfp4_weights* w, void* stream) {
  if (!ws) return fail(NVFP4_ERR_INVALID_ARG, "NULL workspace");
  if (!ws->bound) return fail(NVFP4_ERR_NO_WEIGHTS, "no weights bound; call moe_workspace_bind_weights");
  int st = check_weights_desc(ws, w, false);
  if (st != NVFP4_OK) return st;
  if ((w->w13_codes && w->w13_codes != ws->bound_w13c) || (w->w2_codes && w->w2_codes != ws->bound_w2c))
    return fail(NVFP4_ERR_METADATA_CHANGED,
                "weight codes moved to a new address; recapture is required (update them in place)");
  hipError_t e = copy_weights(ws, w, ws->bound_w13c, ws->bound_w2c, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "weight refresh");
  return ok();
}

int moe_workspace_set_act_scales(moe_workspace* ws, const float* scales_dev, void* stream) {
  if (!ws) return fail(NVFP4_ERR_INVALID_ARG, "NULL workspace");
  if (!(ws->cfg.flags & MOE_STATIC_ACT_SCALES))
    return fail(NVFP4_ERR_INVALID_ARG, "workspace was created without MOE_STATIC_ACT_SCALES");
  if (!scales_dev || !aligned(scales_dev, 4)) return fail(NVFP4_ERR_INVALID_ARG, "NULL or misaligned scales");
  hipError_t e = nvfp4::launch_copy_f32(scales_dev, ws->act_scales, 2, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "activation scale copy");
  ws->act_scales_set = true;
  return ok();
}

namespace {

// Activations handed over already quantized (codes [T, H/2], scales [T, H/16],
// global scales [T]); on = false: the forward quantizes x itself.
struct XQ {
  bool on;
  const void* codes;
  const void* scales;
  const float* g;
};

int forward_impl(moe_workspace* ws, const void* x_dev, const XQ& xq, const float* logits_dev, int64_t T,
                 void* out_dev, void* stream) {
  if (!ws) return fail(NVFP4_ERR_INVALID_ARG, "NULL workspace");
  const moe_config& c = ws->cfg;
  const bool preq = xq.on;
  if (T < 0) return fail(NVFP4_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
  if (T > c.max_num_tokens)
    return fail(NVFP4_ERR_TOO_MANY_TOKENS, "num_tokens (%lld) exceeds max_num_tokens (%lld)",
                (long long)T, (long long)c.max_num_tokens);
  if (!ws->bound) return fail(NVFP4_ERR_NO_WEIGHTS, "no weights bound; call moe_workspace_bind_weights");
  const bool static_scales = (c.flags & MOE_STATIC_ACT_SCALES) != 0;
  if (static_scales && !ws->act_scales_set)
    return fail(NVFP4_ERR_INVALID_ARG, "static activation scales not set; call moe_workspace_set_act_scales");
  if (preq && (c.flags & MOE_W4A16))
    return fail(NVFP4_ERR_INVALID_ARG, "a MOE_W4A16 workspace takes bf16 activations, not quantized ones");
  if (T == 0) return ok();
  const int64_t H = c.hidden, E = c.num_experts;
  if (!logits_dev || !out_dev) return fail(NVFP4_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(out_dev, 16) || !aligned(logits_dev, 4))
    return fail(NVFP4_ERR_INVALID_ARG, "out must be 16-byte aligned, logits 4-byte aligned");
  if (overlap(out_dev, T * H * 2, logits_dev, T * E * 4))
    return fail(NVFP4_ERR_ALIAS, "out overlaps the router logits (the layer is not in-place)");
  if (preq) {
    if (!xq.codes || !xq.scales || !xq.g) return fail(NVFP4_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(xq.codes, 16) || !aligned(xq.scales, 16) || !aligned(xq.g, 4))
      return fail(NVFP4_ERR_INVALID_ARG, "codes and scales must be 16-byte aligned, global scales 4-byte aligned");
    if (overlap(out_dev, T * H * 2, xq.codes, T * H / 2) || overlap(out_dev, T * H * 2, xq.scales, T * H / 16) ||
        overlap(out_dev, T * H * 2, xq.g, T * 4))
      return fail(NVFP4_ERR_ALIAS, "out overlaps the quantized activations (the layer is not in-place)");
  } else {
    if (!x_dev) return fail(NVFP4_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(x_dev, 16)) return fail(NVFP4_ERR_INVALID_ARG, "x must be 16-byte aligned");
    if (overlap(out_dev, T * H * 2, x_dev, T * H * 2))
      return fail(NVFP4_ERR_ALIAS, "out overlaps x (the layer is not in-place)");
  }

  nvfp4::FwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.T = static_cast<int>(T);
  p.H = static_cast<int>(H);
  p.I = static_cast<int>(c.inter);
  p.E = static_cast<int>(E);
  p.k = c.top_k;
  p.R = static_cast<int>(T * c.top_k);
  p.shared = has_shared(c) ? 1 : 0;
  p.Rt = p.R + (p.shared ? p.T : 0);
  p.combine = (c.flags & MOE_SHARED_AVERAGE) ? 0.5f : 1.0f;
  p.a16 = (c.flags & MOE_W4A16) ? 1 : 0;
  nvfp4::choose_gemm(T, &p);
  p.deterministic = (c.flags & MOE_DETERMINISTIC_FINALIZE) ? 1 : 0;
  p.static_g = static_scales ? ws->act_scales : nullptr;
  p.x = static_cast<const uint16_t*>(x_dev);
  p.logits = logits_dev;
  p.out = static_cast<uint16_t*>(out_dev);
  p.preq = preq ? 1 : 0;
  // handed-over codes are read in place (no kernel writes them when preq)
  p.xq_codes = preq ? static_cast<uint8_t*>(const_cast<void*>(xq.codes)) : ws->xq_codes;
  p.xq_scales = preq ? static_cast<uint8_t*>(const_cast<void*>(xq.scales)) : ws->xq_scales;
  p.xq_g = preq ? const_cast<float*>(xq.g) : ws->xq_g;
  // the fp16 copies are only written and read by the tiled (prefill) kernels
  // (W4A16 reads x itself)
  p.xq16 = p.gemm_kind == nvfp4::kGemmTiled && !p.a16 ? ws->xq16 : nullptr;
  p.a2q16 = p.gemm_kind == nvfp4::kGemmTiled ? ws->a2q16 : nullptr;
  p.topk_ids = ws->topk_ids;
  p.topk_w = ws->topk_w;
  p.loc_rank = ws->loc_rank;
  p.blk_counts = ws->blk_counts;
  p.counts = ws->counts;
  p.offsets = ws->offsets;
  p.perm = ws->perm;
  p.inv = ws->inv;
  p.tiles = ws->tiles;
  p.n_tiles = ws->n_tiles;
  p.act = ws->act;
  p.act_amax = ws->act_amax;
  p.a2_codes = ws->a2_codes;
  p.a2_scales = ws->a2_scales;
  p.a2_g = ws->a2_g;
  p.y = ws->y;
  p.out_acc = ws->out_acc;
  p.w13 = ws->w13;
  p.w13g = ws->w13g;
  p.w2 = ws->w2;
  p.w2g = ws->w2g;
  p.dummy = ws->dummy;
  const int64_t max_tiles = tiles_bound(p.R, E, p.mt, p.shared ? T : 0);
  p.tiled_gx = static_cast<int>((max_tiles + 7) / 8 * 8);
  if (max_tiles > ws->max_tiles_cap) return fail(NVFP4_ERR_INVALID_ARG, "internal: tile bound exceeds capacity");
  hipError_t e = nvfp4::launch_moe_forward(p, static_cast<int>(max_tiles), static_cast<hipStream_t>(stream),
                                           ws->timing ? ws->events : nullptr);
  if (e != hipSuccess) return hip_fail(e, "moe_nvfp4_forward launch");
  return ok();
}

}  // namespace

int moe_nvfp4_forward(moe_workspace* ws, const void* x_dev, const float* logits_dev, int64_t T,
                      void* out_dev, void* stream) {
  return forward_impl(ws, x_dev, XQ{false, nullptr, nullptr, nullptr}, logits_dev, T, out_dev, stream);
}

int moe_nvfp4_forward_quantized(moe_workspace* ws, const void* x_codes_dev, const void* x_scales_dev,
                                const float* x_gscale_dev, const float* logits_dev, int64_t T, void* out_dev,
                                void* stream) {
  return forward_impl(ws, nullptr, XQ{true, x_codes_dev, x_scales_dev, x_gscale_dev}, logits_dev, T, out_dev,
                      stream);
}

int moe_workspace_destroy(moe_workspace* ws) {
  if (!ws) return ok();
  (void)hipDeviceSynchronize();
  free_all(ws);
  delete ws;
  return ok();
}

int moe_token_ceiling(int64_t max_prefill, int64_t piecewise_max, int64_t graph_max_bs,
                      int64_t spec_draft_tokens, int64_t* out) {
  if (!out) return fail(NVFP4_ERR_INVALID_ARG, "NULL out");
  if (max_prefill < 0 || piecewise_max < 0 || graph_max_bs < 0 || spec_draft_tokens < 0)
    return fail(NVFP4_ERR_INVALID_ARG, "limits must be >= 0");
  const int64_t per_bs = spec_draft_tokens > 0 ? spec_draft_tokens : 1;
  int64_t prefill = max_prefill;
  if (piecewise_max > 0) prefill = std::max(prefill, piecewise_max);
  *out = std::max(prefill, graph_max_bs * per_bs);
  return ok();
}

int moe_workspace_set_stage_events(moe_workspace* ws, void* const* events) {
  if (!ws) return fail(NVFP4_ERR_INVALID_ARG, "NULL workspace");
  if (!events) {
    ws->timing = false;
    return ok();
  }
  for (int i = 0; i < 5; ++i) {
    if (!events[i]) return fail(NVFP4_ERR_INVALID_ARG, "event %d is NULL", i);
    ws->events[i] = static_cast<hipEvent_t>(events[i]);
  }
  ws->timing = true;
  return ok();
}

int moe_workspace_buffer(const moe_workspace* ws, int32_t id, void** ptr_out, int64_t* bytes_out) {
  if (!ws || !ptr_out || !bytes_out) return fail(NVFP4_ERR_INVALID_ARG, "NULL argument");
  const moe_config& c = ws->cfg;
  const int64_t T = c.max_num_tokens, H = c.hidden, I = c.inter, E = c.num_experts, R = T * c.top_k;
  const int64_t Rt = R + shared_rows(c);
  void* p = nullptr;
  int64_t n = 0;
  switch (id) {
    case MOE_BUF_XQ_CODES: p = ws->xq_codes; n = T * H / 2; break;
    case MOE_BUF_XQ_SCALES: p = ws->xq_scales; n = T * H / 16; break;
    case MOE_BUF_XQ_GSCALE: p = ws->xq_g; n = T * 4; break;
    case MOE_BUF_TOPK_IDS: p = ws->topk_ids; n = R * 4; break;
    case MOE_BUF_TOPK_W: p = ws->topk_w; n = R * 4; break;
    case MOE_BUF_COUNTS: p = ws->counts; n = E * 4; break;
    case MOE_BUF_OFFSETS: p = ws->offsets; n = (E + 1) * 4; break;
    case MOE_BUF_PERM: p = ws->perm; n = R * 4; break;
    case MOE_BUF_INV: p = ws->inv; n = R * 4; break;
    case MOE_BUF_ACT: p = ws->act; n = Rt * I * 4; break;
    case MOE_BUF_A2_CODES: p = ws->a2_codes; n = Rt * I / 2; break;
    case MOE_BUF_A2_SCALES: p = ws->a2_scales; n = Rt * I / 16; break;
    case MOE_BUF_A2_GSCALE: p = ws->a2_g; n = Rt * 4; break;
    case MOE_BUF_A2_16: p = ws->a2q16; n = Rt * I * 2; break;
    default: return fail(NVFP4_ERR_INVALID_ARG, "unknown buffer id %d", id);
  }
  *ptr_out = p;
  *bytes_out = n;
  return ok();
}

}  // extern "C"
