// C-ABI of the NVFP4 fused-MoE layer: argument checks, the workspace (every
// buffer allocated once from the configured token ceiling), weight packing and
// binding, in-place scale refresh and the forward's launch sequence.
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
#include <type_traits>

#include "nvfp4_moe.h"
#include "kernels.hpp"
#include "moe_layout.hpp"

namespace nvfp4 {

namespace {

thread_local std::string g_last_error;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + static_cast<uintptr_t>(nb) && y < x + static_cast<uintptr_t>(na);
}

int hip_fail(hipError_t e, const char* what) {
  return api_fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Tiles of R routed rows over E experts, plus those of the shared expert's
// T rows (shared_T = 0 without one).
int64_t tiles_bound(int64_t R, int64_t E, int mt, int64_t shared_T) {
  return (R + mt - 1) / mt + std::min(E, R) + (shared_T + mt - 1) / mt;
}

}  // namespace

int api_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int api_ok() {
  g_last_error.clear();
  return NVFP4_OK;
}

const char* last_error_text() { return g_last_error.c_str(); }

bool cfg_has_shared(const moe_config& c) { return (c.flags & MOE_SHARED_EXPERT) != 0; }
int64_t cfg_weight_experts(const moe_config& c) { return c.num_experts + (cfg_has_shared(c) ? 1 : 0); }

int check_config(const moe_config& c) {
  if (c.max_num_tokens < 1 || c.max_num_tokens > (int64_t(1) << 24))
    return api_fail(NVFP4_ERR_INVALID_ARG, "max_num_tokens must be in [1, 2^24] (got %lld)",
                    (long long)c.max_num_tokens);
  if (c.hidden < 128 || c.hidden % 128 != 0 || c.hidden > 65536)
    return api_fail(NVFP4_ERR_INVALID_ARG, "hidden must be a multiple of 128 in [128, 65536] (got %lld)",
                    (long long)c.hidden);
  if (c.inter < 128 || c.inter % 128 != 0 || c.inter > 65536)
    return api_fail(NVFP4_ERR_INVALID_ARG, "inter must be a multiple of 128 in [128, 65536] (got %lld)",
                    (long long)c.inter);
  if (c.num_experts < 1 || c.num_experts > kMaxExperts)
    return api_fail(NVFP4_ERR_INVALID_ARG, "num_experts must be in [1, %d]", kMaxExperts);
  if (c.top_k < 1 || c.top_k > kMaxTopK || c.top_k > c.num_experts)
    return api_fail(NVFP4_ERR_INVALID_ARG, "top_k must be in [1, min(%d, num_experts)]", kMaxTopK);
  if ((c.flags & ~(MOE_DETERMINISTIC_FINALIZE | MOE_STATIC_ACT_SCALES | MOE_SHARED_EXPERT |
                   MOE_SHARED_AVERAGE | MOE_W4A16)) != 0)
    return api_fail(NVFP4_ERR_INVALID_ARG, "unknown flags 0x%x", c.flags);
  if ((c.flags & MOE_W4A16) && (c.flags & MOE_STATIC_ACT_SCALES))
    return api_fail(NVFP4_ERR_INVALID_ARG,
                    "MOE_W4A16 quantizes no activations: MOE_STATIC_ACT_SCALES does not apply");
  if ((c.flags & MOE_SHARED_AVERAGE) && !(c.flags & MOE_SHARED_EXPERT))
    return api_fail(NVFP4_ERR_INVALID_ARG, "MOE_SHARED_AVERAGE requires MOE_SHARED_EXPERT");
  if (cfg_weight_experts(c) > kMaxExperts)
    return api_fail(NVFP4_ERR_INVALID_ARG, "num_experts plus the shared expert must be <= %d", kMaxExperts);
  if (c.max_num_tokens * (c.top_k + 1) > (int64_t(1) << 30))
    return api_fail(NVFP4_ERR_INVALID_ARG, "max_num_tokens * (top_k + 1) too large");
  if (c.max_num_tokens * c.hidden >= (int64_t(1) << 30))
    return api_fail(NVFP4_ERR_INVALID_ARG, "max_num_tokens * hidden must be < 2^30 (got %lld)",
                    (long long)(c.max_num_tokens * c.hidden));
  return NVFP4_OK;
}

int64_t layout_buffers(const moe_config& c, int64_t T_cap, bool own_gscales, uint8_t* base, FwdBuffers* b) {
  const int64_t T = T_cap, H = c.hidden, I = c.inter, E = c.num_experts, k = c.top_k;
  const int64_t R = T * k;                                 // routed rows
  const int64_t Rt = R + (cfg_has_shared(c) ? T : 0);      // GEMM rows
  const int64_t Ew = cfg_weight_experts(c);
  const int64_t n_amax = I / 32;  // GEMM1 column bands of 32 (the finest band used)
  const bool det = (c.flags & MOE_DETERMINISTIC_FINALIZE) != 0;
  b->T_cap = T;
  b->max_tiles_cap = tiles_bound(R, E, 16, cfg_has_shared(c) ? T : 0);
  b->route_blocks_cap = static_cast<int>(
      std::max<int64_t>(kMaxRouteBlocks, (T + kMaxTokensPerRouteBlock - 1) / kMaxTokensPerRouteBlock));
  int64_t off = 0;
  auto take = [&](auto** p, int64_t bytes) {
    using P = std::remove_pointer_t<std::remove_reference_t<decltype(p)>>;
    *p = bytes > 0 ? reinterpret_cast<P>(base + off) : nullptr;
    off += (bytes + 255) / 256 * 256;
  };
  take(&b->dummy, kRecBytes);
  take(&b->xq_codes, T * H / 2);
  take(&b->xq_scales, T * H / 16);
  take(&b->xq_g, T * 4);
  take(&b->xq16, T * H * 2);
  take(&b->topk_ids, R * 4);
  take(&b->topk_w, R * 4);
  take(&b->loc_rank, R * 4);
  take(&b->blk_counts, static_cast<int64_t>(b->route_blocks_cap) * E * 4);
  take(&b->counts, E * 4);
  take(&b->offsets, (E + 1) * 4);
  take(&b->perm, R * 4);
  take(&b->inv, R * 4);
  take(&b->tiles, b->max_tiles_cap * 16);
  take(&b->n_tiles, 4);
  take(&b->act_scales, 2 * 4);
  take(&b->act, Rt * I * 4);
  take(&b->act_amax, Rt * n_amax * 4);
  take(&b->a2_codes, Rt * I / 2);
  take(&b->a2_scales, Rt * I / 16);
  take(&b->a2_g, Rt * 4);
  take(&b->a2q16, Rt * I * 2);
  take(&b->y, det ? Rt * H * 2 : 0);
  take(&b->out_acc, det ? 0 : T * H * 4);
  take(&b->w13g, own_gscales ? Ew * 4 : 0);
  take(&b->w2g, own_gscales ? Ew * 4 : 0);
  return off;
}

int check_packed(const moe_config& c, const moe_nvfp4_packed* w) {
  if (!w) return api_fail(NVFP4_ERR_INVALID_ARG, "packed weights descriptor is NULL");
  if (w->num_experts != cfg_weight_experts(c) || w->hidden != c.hidden || w->inter != c.inter)
    return api_fail(NVFP4_ERR_INVALID_ARG,
                    "weight dims (E=%lld, H=%lld, I=%lld) do not match the layer's (E=%lld, H=%lld, I=%lld)",
                    (long long)w->num_experts, (long long)w->hidden, (long long)w->inter,
                    (long long)cfg_weight_experts(c), (long long)c.hidden, (long long)c.inter);
  if (!w->w13 || !w->w2 || !w->w13_gscale || !w->w2_gscale)
    return api_fail(NVFP4_ERR_INVALID_ARG, "packed weight pointers must be non-NULL");
  if (!aligned(w->w13, 16) || !aligned(w->w2, 16) || !aligned(w->w13_gscale, 4) || !aligned(w->w2_gscale, 4))
    return api_fail(NVFP4_ERR_INVALID_ARG,
                    "packed records must be 16-byte aligned, global scales 4-byte aligned");
  return NVFP4_OK;
}

int run_forward(const moe_config& c, const FwdBuffers& b, const WeightView& wv, bool static_scales_set,
                const void* x_dev, const XQ& xq, const float* logits_dev, int64_t T, void* out_dev,
                hipStream_t stream, const hipEvent_t* events) {
  const bool preq = xq.on;
  if (T < 0) return api_fail(NVFP4_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
  if (T > b.T_cap)
    return api_fail(NVFP4_ERR_TOO_MANY_TOKENS, "num_tokens (%lld) exceeds max_num_tokens (%lld)",
                    (long long)T, (long long)b.T_cap);
  const bool static_scales = (c.flags & MOE_STATIC_ACT_SCALES) != 0;
  if (static_scales && !static_scales_set)
    return api_fail(NVFP4_ERR_INVALID_ARG,
                    "static activation scales not set; call moe_workspace_set_act_scales");
  if (preq && (c.flags & MOE_W4A16))
    return api_fail(NVFP4_ERR_INVALID_ARG, "a MOE_W4A16 workspace takes bf16 activations, not quantized ones");
  if (T == 0) return api_ok();
  const int64_t H = c.hidden, E = c.num_experts;
  if (!logits_dev || !out_dev) return api_fail(NVFP4_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(out_dev, 16) || !aligned(logits_dev, 4))
    return api_fail(NVFP4_ERR_INVALID_ARG, "out must be 16-byte aligned, logits 4-byte aligned");
  if (overlap(out_dev, T * H * 2, logits_dev, T * E * 4))
    return api_fail(NVFP4_ERR_ALIAS, "out overlaps the router logits (the layer is not in-place)");
  if (preq) {
    if (!xq.codes || !xq.scales || !xq.g) return api_fail(NVFP4_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(xq.codes, 16) || !aligned(xq.scales, 16) || !aligned(xq.g, 4))
      return api_fail(NVFP4_ERR_INVALID_ARG,
                      "codes and scales must be 16-byte aligned, global scales 4-byte aligned");
    if (overlap(out_dev, T * H * 2, xq.codes, T * H / 2) || overlap(out_dev, T * H * 2, xq.scales, T * H / 16) ||
        overlap(out_dev, T * H * 2, xq.g, T * 4))
      return api_fail(NVFP4_ERR_ALIAS, "out overlaps the quantized activations (the layer is not in-place)");
  } else {
    if (!x_dev) return api_fail(NVFP4_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(x_dev, 16)) return api_fail(NVFP4_ERR_INVALID_ARG, "x must be 16-byte aligned");
    if (overlap(out_dev, T * H * 2, x_dev, T * H * 2))
      return api_fail(NVFP4_ERR_ALIAS, "out overlaps x (the layer is not in-place)");
  }

  FwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.T = static_cast<int>(T);
  p.H = static_cast<int>(H);
  p.I = static_cast<int>(c.inter);
  p.E = static_cast<int>(E);
  p.k = c.top_k;
  p.R = static_cast<int>(T * c.top_k);
  p.shared = cfg_has_shared(c) ? 1 : 0;
  p.Rt = p.R + (p.shared ? p.T : 0);
  p.combine = (c.flags & MOE_SHARED_AVERAGE) ? 0.5f : 1.0f;
  p.a16 = (c.flags & MOE_W4A16) ? 1 : 0;
  choose_gemm(T, &p);
  p.deterministic = (c.flags & MOE_DETERMINISTIC_FINALIZE) ? 1 : 0;
  p.static_g = static_scales ? b.act_scales : nullptr;
  p.x = static_cast<const uint16_t*>(x_dev);
  p.logits = logits_dev;
  p.out = static_cast<uint16_t*>(out_dev);
  p.preq = preq ? 1 : 0;
  // handed-over codes are read in place (no kernel writes them when preq)
  p.xq_codes = preq ? static_cast<uint8_t*>(const_cast<void*>(xq.codes)) : b.xq_codes;
  p.xq_scales = preq ? static_cast<uint8_t*>(const_cast<void*>(xq.scales)) : b.xq_scales;
  p.xq_g = preq ? const_cast<float*>(xq.g) : b.xq_g;
  // the fp16 copies are only written and read by the tiled (prefill) kernels
  // (W4A16 reads x itself)
  p.xq16 = p.gemm_kind == kGemmTiled && !p.a16 ? b.xq16 : nullptr;
  // (W4A16: GEMM2's bf16 input, also written by the stream kernels)
  p.a2q16 = p.gemm_kind == kGemmTiled || p.a16 ? b.a2q16 : nullptr;
  p.topk_ids = b.topk_ids;
  p.topk_w = b.topk_w;
  p.loc_rank = b.loc_rank;
  p.blk_counts = b.blk_counts;
  p.counts = b.counts;
  p.offsets = b.offsets;
  p.perm = b.perm;
  p.inv = b.inv;
  p.tiles = b.tiles;
  p.n_tiles = b.n_tiles;
  p.act = b.act;
  p.act_amax = b.act_amax;
  p.a2_codes = b.a2_codes;
  p.a2_scales = b.a2_scales;
  p.a2_g = b.a2_g;
  p.y = b.y;
  p.out_acc = b.out_acc;
  p.w13 = wv.w13;
  p.w13g = wv.w13g;
  p.w2 = wv.w2;
  p.w2g = wv.w2g;
  p.dummy = b.dummy;
  const int64_t max_tiles = tiles_bound(p.R, E, p.mt, p.shared ? T : 0);
  p.tiled_gx = static_cast<int>((max_tiles + 7) / 8 * 8);
  if (max_tiles > b.max_tiles_cap) return api_fail(NVFP4_ERR_INVALID_ARG, "internal: tile bound exceeds capacity");
  const int64_t route_blocks = (T + route_tokens_per_block(T) - 1) / route_tokens_per_block(T);
  if (route_blocks > b.route_blocks_cap)
    return api_fail(NVFP4_ERR_INVALID_ARG, "internal: route blocks exceed capacity");
  hipError_t e = launch_moe_forward(p, static_cast<int>(max_tiles), stream, events);
  if (e != hipSuccess) return hip_fail(e, "moe_nvfp4_forward launch");
  return api_ok();
}

}  // namespace nvfp4

using nvfp4::api_fail;
using nvfp4::api_ok;

struct moe_workspace {
  moe_config cfg;
  int device;
  uint8_t* block;  // the one device allocation the buffers are carved from
  nvfp4::FwdBuffers buf;
  bool act_scales_set;
  // weights: the caller's packed records (borrowed); the workspace holds
  // copies of the global scales (buf.w13g / buf.w2g)
  bool bound;
  const uint8_t* w13;
  const uint8_t* w2;
  // optional stage-timing events (caller-owned)
  bool timing;
  hipEvent_t events[5];
};

namespace {

bool is_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + static_cast<uintptr_t>(nb) && y < x + static_cast<uintptr_t>(na);
}

int hip_error(hipError_t e, const char* what) {
  return api_fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dims_ok(int64_t E, int64_t H, int64_t I) {
  return E >= 1 && E <= nvfp4::kMaxExperts && H >= 128 && H % 128 == 0 && H <= 65536 && I >= 128 &&
         I % 128 == 0 && I <= 65536;
}

void packed_sizes(int64_t E, int64_t H, int64_t I, int64_t* b13, int64_t* b2) {
  *b13 = nvfp4::packed_bytes(nvfp4::w13_units(E, I), static_cast<int>(H));
  *b2 = nvfp4::packed_bytes(nvfp4::w2_units(E, H), static_cast<int>(I));
}

// Scales (and, with codes, the codes) of row-major weights into packed
// records.
hipError_t pack(const moe_nvfp4_weights* w, uint8_t* d13, uint8_t* d2, bool with_codes, hipStream_t s) {
  const int64_t E = w->num_experts, H = w->hidden, I = w->inter;
  hipError_t e = nvfp4::launch_pack_weights(with_codes ? static_cast<const uint8_t*>(w->w13_codes) : nullptr,
                                            static_cast<const uint8_t*>(w->w13_scales), d13, E, 2 * I, H, 1, s);
  if (e == hipSuccess)
    e = nvfp4::launch_pack_weights(with_codes ? static_cast<const uint8_t*>(w->w2_codes) : nullptr,
                                   static_cast<const uint8_t*>(w->w2_scales), d2, E, H, I, 0, s);
  return e;
}

}  // namespace

extern "C" {

const char* nvfp4_last_error(void) { return nvfp4::last_error_text(); }

int nvfp4_quantize_per_token(const void* x_dev, int64_t rows, int64_t cols, int64_t ld_x,
                             void* codes_dev, void* scales_dev, float* gscale_dev, void* stream) {
  if (rows < 0) return api_fail(NVFP4_ERR_INVALID_ARG, "rows must be >= 0 (got %lld)", (long long)rows);
  if (cols <= 0 || cols % 16 != 0)
    return api_fail(NVFP4_ERR_INVALID_ARG, "cols must be a positive multiple of 16 (got %lld)", (long long)cols);
  if (cols > (int64_t(1) << 30)) return api_fail(NVFP4_ERR_INVALID_ARG, "cols too large");
  if (ld_x < cols || ld_x % 8 != 0)
    return api_fail(NVFP4_ERR_INVALID_ARG, "ld_x must be >= cols and a multiple of 8 (got %lld)",
                    (long long)ld_x);
  if (rows == 0) return api_ok();
  if (rows > INT32_MAX) return api_fail(NVFP4_ERR_INVALID_ARG, "rows must be < 2^31 (got %lld)", (long long)rows);
  if (!x_dev || !codes_dev || !scales_dev || !gscale_dev)
    return api_fail(NVFP4_ERR_INVALID_ARG, "NULL pointer argument");
  if (!is_aligned(x_dev, 16) || !is_aligned(codes_dev, 16) || !is_aligned(gscale_dev, 4))
    return api_fail(NVFP4_ERR_INVALID_ARG, "x and codes must be 16-byte aligned, gscale 4-byte aligned");
  const int64_t xbytes = ((rows - 1) * ld_x + cols) * 2;
  if (overlaps(x_dev, xbytes, codes_dev, rows * cols / 2) ||
      overlaps(x_dev, xbytes, scales_dev, rows * cols / 16) || overlaps(x_dev, xbytes, gscale_dev, rows * 4))
    return api_fail(NVFP4_ERR_ALIAS, "outputs overlap the input x");
  hipError_t e = nvfp4::launch_quantize_rows(static_cast<const uint16_t*>(x_dev), rows, cols, ld_x,
                                             static_cast<uint8_t*>(codes_dev),
                                             static_cast<uint8_t*>(scales_dev), gscale_dev,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_error(e, "nvfp4_quantize_per_token launch");
  return api_ok();
}

int nvfp4_quantize_experts(const float* w_dev, int64_t experts, int64_t rows, int64_t cols,
                           void* codes_dev, void* scales_dev, float* gscale_dev, float* scratch_dev,
                           void* stream) {
  if (experts < 1 || experts > 65535 || rows < 1 || cols <= 0 || cols % 16 != 0)
    return api_fail(NVFP4_ERR_INVALID_ARG,
                    "need 1 <= experts <= 65535, rows >= 1, cols a positive multiple of 16");
  if (!w_dev || !codes_dev || !scales_dev || !gscale_dev || !scratch_dev)
    return api_fail(NVFP4_ERR_INVALID_ARG, "NULL pointer argument");
  if (!is_aligned(w_dev, 16) || !is_aligned(codes_dev, 16) || !is_aligned(gscale_dev, 4) ||
      !is_aligned(scratch_dev, 4))
    return api_fail(NVFP4_ERR_INVALID_ARG, "w and codes must be 16-byte aligned");
  const int64_t n = experts * rows * cols;
  if (overlaps(w_dev, n * 4, codes_dev, n / 2) || overlaps(w_dev, n * 4, scales_dev, n / 16))
    return api_fail(NVFP4_ERR_ALIAS, "outputs overlap the input");
  hipError_t e = nvfp4::launch_quantize_experts(w_dev, experts, rows, cols, static_cast<uint8_t*>(codes_dev),
                                                static_cast<uint8_t*>(scales_dev), gscale_dev,
                                                reinterpret_cast<uint32_t*>(scratch_dev),
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_error(e, "nvfp4_quantize_experts launch");
  return api_ok();
}

int moe_packed_bytes(int64_t num_experts, int64_t hidden, int64_t inter, int64_t* w13_bytes,
                     int64_t* w2_bytes) {
  if (!w13_bytes || !w2_bytes) return api_fail(NVFP4_ERR_INVALID_ARG, "NULL output");
  if (!dims_ok(num_experts, hidden, inter))
    return api_fail(NVFP4_ERR_INVALID_ARG,
                    "need 1 <= num_experts <= %d and hidden, inter multiples of 128 in [128, 65536]",
                    nvfp4::kMaxExperts);
  packed_sizes(num_experts, hidden, inter, w13_bytes, w2_bytes);
  return api_ok();
}

int moe_pack_weights(const moe_nvfp4_weights* w, void* w13_packed_dev, void* w2_packed_dev, void* stream) {
  if (!w) return api_fail(NVFP4_ERR_INVALID_ARG, "weights descriptor is NULL");
  const int64_t E = w->num_experts, H = w->hidden, I = w->inter;
  if (!dims_ok(E, H, I))
    return api_fail(NVFP4_ERR_INVALID_ARG,
                    "need 1 <= num_experts <= %d and hidden, inter multiples of 128 in [128, 65536]",
                    nvfp4::kMaxExperts);
  if (!w13_packed_dev || !w2_packed_dev || !w->w13_scales || !w->w2_scales)
    return api_fail(NVFP4_ERR_INVALID_ARG, "NULL pointer argument");
  const bool with_codes = w->w13_codes != nullptr;
  if (with_codes != (w->w2_codes != nullptr))
    return api_fail(NVFP4_ERR_INVALID_ARG, "give both code pointers or neither");
  if (!is_aligned(w13_packed_dev, 16) || !is_aligned(w2_packed_dev, 16) ||
      (with_codes && (!is_aligned(w->w13_codes, 16) || !is_aligned(w->w2_codes, 16))))
    return api_fail(NVFP4_ERR_INVALID_ARG, "packed buffers and codes must be 16-byte aligned");
  int64_t b13, b2;
  packed_sizes(E, H, I, &b13, &b2);
  const void* ins[4] = {w->w13_codes, w->w13_scales, w->w2_codes, w->w2_scales};
  const int64_t in_bytes[4] = {with_codes ? E * 2 * I * H / 2 : 0, E * 2 * I * H / 16,
                               with_codes ? E * H * I / 2 : 0, E * H * I / 16};
  for (int i = 0; i < 4; ++i)
    if (overlaps(w13_packed_dev, b13, ins[i], in_bytes[i]) || overlaps(w2_packed_dev, b2, ins[i], in_bytes[i]))
      return api_fail(NVFP4_ERR_ALIAS, "packed buffers overlap the row-major weights");
  if (overlaps(w13_packed_dev, b13, w2_packed_dev, b2))
    return api_fail(NVFP4_ERR_ALIAS, "the two packed buffers overlap");
  hipError_t e = pack(w, static_cast<uint8_t*>(w13_packed_dev), static_cast<uint8_t*>(w2_packed_dev), with_codes,
                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_error(e, "moe_pack_weights launch");
  return api_ok();
}

int moe_workspace_create(const moe_config* cfg, void* stream, moe_workspace** out) {
  if (!cfg || !out) return api_fail(NVFP4_ERR_INVALID_ARG, "NULL cfg or out");
  *out = nullptr;
  const moe_config c = *cfg;
  int st = nvfp4::check_config(c);
  if (st != NVFP4_OK) return st;
  moe_workspace* w = new (std::nothrow) moe_workspace();
  if (!w) return api_fail(NVFP4_ERR_OOM, "host allocation failed");
  std::memset(static_cast<void*>(w), 0, sizeof(*w));
  w->cfg = c;
  if (hipGetDevice(&w->device) != hipSuccess) {
    delete w;
    return api_fail(NVFP4_ERR_HIP, "hipGetDevice failed");
  }
  const int64_t bytes = nvfp4::layout_buffers(c, c.max_num_tokens, true, nullptr, &w->buf);
  hipError_t e = hipMalloc(reinterpret_cast<void**>(&w->block), static_cast<size_t>(bytes));
  if (e != hipSuccess) {
    delete w;
    return api_fail(NVFP4_ERR_OOM, "hipMalloc of %lld bytes failed: %s", (long long)bytes, hipGetErrorString(e));
  }
  nvfp4::layout_buffers(c, c.max_num_tokens, true, w->block, &w->buf);
  hipStream_t s = static_cast<hipStream_t>(stream);
  e = nvfp4::launch_fill_u32(reinterpret_cast<uint32_t*>(w->buf.dummy), nvfp4::kRecBytes / 4, 0u, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipFree(w->block);
    delete w;
    return hip_error(e, "workspace initialization");
  }
  *out = w;
  return api_ok();
}

int moe_workspace_bind_weights(moe_workspace* ws, const moe_nvfp4_packed* w, void* stream) {
  if (!ws) return api_fail(NVFP4_ERR_INVALID_ARG, "NULL workspace");
  if (ws->bound) return api_fail(NVFP4_ERR_INVALID_ARG, "weights already bound; use refresh_scales_inplace");
  int st = nvfp4::check_packed(ws->cfg, w);
  if (st != NVFP4_OK) return st;
  const int64_t E = nvfp4::cfg_weight_experts(ws->cfg);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = nvfp4::launch_copy_f32(w->w13_gscale, ws->buf.w13g, E, s);
  if (e == hipSuccess) e = nvfp4::launch_copy_f32(w->w2_gscale, ws->buf.w2g, E, s);
  if (e != hipSuccess) return hip_error(e, "global scale copy");
  ws->w13 = static_cast<const uint8_t*>(w->w13);
  ws->w2 = static_cast<const uint8_t*>(w->w2);
  ws->bound = true;
  return api_ok();
}

int refresh_scales_inplace(moe_workspace* ws, const moe_nvfp4_weights* w, void* stream) {
  if (!ws) return api_fail(NVFP4_ERR_INVALID_ARG, "NULL workspace");
  if (!ws->bound) return api_fail(NVFP4_ERR_NO_WEIGHTS, "no weights bound; call moe_workspace_bind_weights");
  if (!w) return api_fail(NVFP4_ERR_INVALID_ARG, "weights descriptor is NULL");
  const moe_config& c = ws->cfg;
  const int64_t E = nvfp4::cfg_weight_experts(c);
  if (w->num_experts != E || w->hidden != c.hidden || w->inter != c.inter)
    return api_fail(NVFP4_ERR_METADATA_CHANGED,
                    "weight dims (E=%lld, H=%lld, I=%lld) differ from the bound ones (E=%lld, H=%lld, "
                    "I=%lld); recapture is required",
                    (long long)w->num_experts, (long long)w->hidden, (long long)w->inter, (long long)E,
                    (long long)c.hidden, (long long)c.inter);
  if (w->w13_codes || w->w2_codes)
    return api_fail(NVFP4_ERR_INVALID_ARG,
                    "refresh copies scales only: pass NULL code pointers (reload codes in place with "
                    "moe_pack_weights)");
  if (!w->w13_scales || !w->w2_scales || !w->w13_gscale || !w->w2_gscale)
    return api_fail(NVFP4_ERR_INVALID_ARG, "scale pointers must be non-NULL");
  if (!is_aligned(w->w13_gscale, 4) || !is_aligned(w->w2_gscale, 4))
    return api_fail(NVFP4_ERR_INVALID_ARG, "global scale pointers must be 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = pack(w, const_cast<uint8_t*>(ws->w13), const_cast<uint8_t*>(ws->w2), false, s);
  if (e == hipSuccess) e = nvfp4::launch_copy_f32(w->w13_gscale, ws->buf.w13g, E, s);
  if (e == hipSuccess) e = nvfp4::launch_copy_f32(w->w2_gscale, ws->buf.w2g, E, s);
  if (e != hipSuccess) return hip_error(e, "scale refresh");
  return api_ok();
}

int moe_workspace_set_act_scales(moe_workspace* ws, const float* scales_dev, void* stream) {
  if (!ws) return api_fail(NVFP4_ERR_INVALID_ARG, "NULL workspace");
  if (!(ws->cfg.flags & MOE_STATIC_ACT_SCALES))
    return api_fail(NVFP4_ERR_INVALID_ARG, "workspace was created without MOE_STATIC_ACT_SCALES");
  if (!scales_dev || !is_aligned(scales_dev, 4))
    return api_fail(NVFP4_ERR_INVALID_ARG, "NULL or misaligned scales");
  hipError_t e = nvfp4::launch_copy_f32(scales_dev, ws->buf.act_scales, 2, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_error(e, "activation scale copy");
  ws->act_scales_set = true;
  return api_ok();
}

static int workspace_forward(moe_workspace* ws, const void* x_dev, const nvfp4::XQ& xq, const float* logits_dev,
                             int64_t T, void* out_dev, void* stream) {
  if (!ws) return api_fail(NVFP4_ERR_INVALID_ARG, "NULL workspace");
  if (!ws->bound) return api_fail(NVFP4_ERR_NO_WEIGHTS, "no weights bound; call moe_workspace_bind_weights");
  const nvfp4::WeightView wv{ws->w13, ws->w2, ws->buf.w13g, ws->buf.w2g};
  return nvfp4::run_forward(ws->cfg, ws->buf, wv, ws->act_scales_set, x_dev, xq, logits_dev, T, out_dev,
                            static_cast<hipStream_t>(stream), ws->timing ? ws->events : nullptr);
}

int moe_nvfp4_forward(moe_workspace* ws, const void* x_dev, const float* logits_dev, int64_t T,
                      void* out_dev, void* stream) {
  return workspace_forward(ws, x_dev, nvfp4::XQ{false, nullptr, nullptr, nullptr}, logits_dev, T, out_dev,
                           stream);
}

int moe_nvfp4_forward_quantized(moe_workspace* ws, const void* x_codes_dev, const void* x_scales_dev,
                                const float* x_gscale_dev, const float* logits_dev, int64_t T, void* out_dev,
                                void* stream) {
  return workspace_forward(ws, nullptr, nvfp4::XQ{true, x_codes_dev, x_scales_dev, x_gscale_dev}, logits_dev,
                           T, out_dev, stream);
}

int moe_workspace_destroy(moe_workspace* ws) {
  if (!ws) return api_ok();
  (void)hipDeviceSynchronize();
  if (ws->block) (void)hipFree(ws->block);
  delete ws;
  return api_ok();
}

int moe_token_ceiling(int64_t max_prefill, int64_t piecewise_max, int64_t graph_max_bs,
                      int64_t spec_draft_tokens, int64_t* out) {
  if (!out) return api_fail(NVFP4_ERR_INVALID_ARG, "NULL out");
  if (max_prefill < 0 || piecewise_max < 0 || graph_max_bs < 0 || spec_draft_tokens < 0)
    return api_fail(NVFP4_ERR_INVALID_ARG, "limits must be >= 0");
  const int64_t per_bs = spec_draft_tokens > 0 ? spec_draft_tokens : 1;
  int64_t prefill = max_prefill;
  if (piecewise_max > 0) prefill = std::max(prefill, piecewise_max);
  *out = std::max(prefill, graph_max_bs * per_bs);
  return api_ok();
}

int moe_workspace_set_stage_events(moe_workspace* ws, void* const* events) {
  if (!ws) return api_fail(NVFP4_ERR_INVALID_ARG, "NULL workspace");
  if (!events) {
    ws->timing = false;
    return api_ok();
  }
  for (int i = 0; i < 5; ++i) {
    if (!events[i]) return api_fail(NVFP4_ERR_INVALID_ARG, "event %d is NULL", i);
    ws->events[i] = static_cast<hipEvent_t>(events[i]);
  }
  ws->timing = true;
  return api_ok();
}

int moe_workspace_buffer(const moe_workspace* ws, int32_t id, void** ptr_out, int64_t* bytes_out) {
  if (!ws || !ptr_out || !bytes_out) return api_fail(NVFP4_ERR_INVALID_ARG, "NULL argument");
  const moe_config& c = ws->cfg;
  const nvfp4::FwdBuffers& b = ws->buf;
  const int64_t T = c.max_num_tokens, H = c.hidden, I = c.inter, E = c.num_experts, R = T * c.top_k;
  const int64_t Rt = R + (nvfp4::cfg_has_shared(c) ? T : 0);
  void* p = nullptr;
  int64_t n = 0;
  switch (id) {
    case MOE_BUF_XQ_CODES: p = b.xq_codes; n = T * H / 2; break;
    case MOE_BUF_XQ_SCALES: p = b.xq_scales; n = T * H / 16; break;
    case MOE_BUF_XQ_GSCALE: p = b.xq_g; n = T * 4; break;
    case MOE_BUF_TOPK_IDS: p = b.topk_ids; n = R * 4; break;
    case MOE_BUF_TOPK_W: p = b.topk_w; n = R * 4; break;
    case MOE_BUF_COUNTS: p = b.counts; n = E * 4; break;
    case MOE_BUF_OFFSETS: p = b.offsets; n = (E + 1) * 4; break;
    case MOE_BUF_PERM: p = b.perm; n = R * 4; break;
    case MOE_BUF_INV: p = b.inv; n = R * 4; break;
    case MOE_BUF_ACT: p = b.act; n = Rt * I * 4; break;
    case MOE_BUF_A2_CODES: p = b.a2_codes; n = Rt * I / 2; break;
    case MOE_BUF_A2_SCALES: p = b.a2_scales; n = Rt * I / 16; break;
    case MOE_BUF_A2_GSCALE: p = b.a2_g; n = Rt * 4; break;
    case MOE_BUF_A2_16: p = b.a2q16; n = Rt * I * 2; break;
    default: return api_fail(NVFP4_ERR_INVALID_ARG, "unknown buffer id %d", id);
  }
  *ptr_out = p;
  *bytes_out = n;
  return api_ok();
}

}  // extern "C"
