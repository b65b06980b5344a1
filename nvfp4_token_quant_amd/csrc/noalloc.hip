// The forward for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// Its intermediates (quantized activations, routing tables, the M-tile list,
// the SwiGLU output and its re-quantization, the GEMM2 rows or the atomic
// accumulator) live in `scratch`, one file-scope device array of
// kScratchBytes that each GPU the library runs on holds until the process
// ends.  In host code the array's name only stands in for the symbol; its
// device address on each device comes from hipGetSymbolAddress, queried once
// per device with that device current, and only that address is handed to
// kernels.  Every call on a GPU shares that GPU's array: calls that overlap on
// one GPU (two streams, two threads) race.  Nothing in the array needs to
// start at zero: each forward writes every intermediate it reads (the atomic
// accumulator is cleared by the forward's first kernel), and the record the
// weight prefetch reads past a wave's last K step is loaded but never used.
#include <hip/hip_runtime.h>

#include <mutex>

#include "nvfp4_moe.h"
#include "kernels.hpp"
#include "moe_layout.hpp"

namespace {

constexpr int64_t kScratchBytes = int64_t(64) << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device

// The current device's address of `scratch` (queried on the first call on
// that device).
int scratch_address(uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return nvfp4::api_fail(NVFP4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return nvfp4::api_fail(NVFP4_ERR_INVALID_ARG, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return nvfp4::api_fail(NVFP4_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_OK;
}

// Largest token count whose buffers fit the array (0 if none does).
int64_t max_tokens_in_scratch(const moe_config& c) {
  nvfp4::FwdBuffers b;
  int64_t lo = 0, hi = c.max_num_tokens;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (nvfp4::layout_buffers(c, mid, false, nullptr, &b) <= kScratchBytes) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

}  // namespace

extern "C" int moe_nvfp4_forward_noalloc(const moe_config* cfg, const moe_nvfp4_packed* w, const void* x_dev,
                                         const float* logits_dev, int64_t T, void* out_dev, void* stream) {
  if (!cfg) return nvfp4::api_fail(NVFP4_ERR_INVALID_ARG, "NULL cfg");
  const moe_config c = *cfg;
  int st = nvfp4::check_config(c);
  if (st != NVFP4_OK) return st;
  if (c.flags & MOE_STATIC_ACT_SCALES)
    return nvfp4::api_fail(NVFP4_ERR_INVALID_ARG,
                           "MOE_STATIC_ACT_SCALES needs a workspace (moe_workspace_set_act_scales)");
  st = nvfp4::check_packed(c, w);
  if (st != NVFP4_OK) return st;
  if (T < 0) return nvfp4::api_fail(NVFP4_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
  if (T > c.max_num_tokens)
    return nvfp4::api_fail(NVFP4_ERR_TOO_MANY_TOKENS, "num_tokens (%lld) exceeds max_num_tokens (%lld)",
                           (long long)T, (long long)c.max_num_tokens);
  if (T == 0) return nvfp4::api_ok();
  nvfp4::FwdBuffers b;
  const int64_t need = nvfp4::layout_buffers(c, T, false, nullptr, &b);
  if (need > kScratchBytes)
    return nvfp4::api_fail(NVFP4_ERR_INVALID_ARG,
                           "the forward of %lld tokens needs %lld bytes of intermediates; the no-allocation "
                           "forward holds %lld (at most %lld tokens of this layer): use a workspace",
                           (long long)T, (long long)need, (long long)kScratchBytes,
                           (long long)max_tokens_in_scratch(c));
  uint8_t* base = nullptr;
  st = scratch_address(&base);
  if (st != NVFP4_OK) return st;
  nvfp4::layout_buffers(c, T, false, base, &b);
  const nvfp4::WeightView wv{static_cast<const uint8_t*>(w->w13), static_cast<const uint8_t*>(w->w2),
                             w->w13_gscale, w->w2_gscale};
  return nvfp4::run_forward(c, b, wv, false, x_dev, nvfp4::XQ{false, nullptr, nullptr, nullptr}, logits_dev, T,
                            out_dev, static_cast<hipStream_t>(stream), nullptr);
}
