// Synthetic expert weights on the device (input generation for tests and
// benchmarks; not part of the layer).  Counter-based so that the CPU side,
// which implements the same published generator separately, produces the
// same bits:
//   Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
//   Easy as 1, 2, 3", SC'11) with key (seed, tag) and counter
//   (i / 4, expert, 0, 0); element i of an expert takes output word i % 4,
//   sums its four 16-bit fields, centres the sum (Irwin-Hall of order 4) and
//   scales it by sigma / sqrt(4 (2^32 - 1) / 12) in binary32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <string>

#include "nvfp4_synth.h"

namespace {

__device__ __forceinline__ void philox_round(uint64_t& x0, uint64_t& x1, uint64_t& x2, uint64_t& x3,
                                             uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t hi0 = __umul64hi(M0, x0), lo0 = M0 * x0;
  const uint64_t hi1 = __umul64hi(M1, x2), lo1 = M1 * x2;
  const uint64_t n0 = hi1 ^ x1 ^ k0, n2 = hi0 ^ x3 ^ k1;
  x0 = n0;
  x1 = lo1;
  x2 = n2;
  x3 = lo0;
}

__global__ void synth_weights_kernel(uint64_t seed, uint64_t tag, int64_t expert0, int64_t n_per_expert,
                                     float c, float* __restrict__ out) {
  const int64_t blocks_per_expert = (n_per_expert + 3) / 4;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blk >= blocks_per_expert) return;
  const int64_t e = expert0 + blockIdx.y;
  uint64_t x0 = static_cast<uint64_t>(blk), x1 = static_cast<uint64_t>(e), x2 = 0, x3 = 0;
  uint64_t k0 = seed, k1 = tag;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B97F4A7C15ull;
      k1 += 0xBB67AE8584CAA73Bull;
    }
    philox_round(x0, x1, x2, x3, k0, k1);
  }
  const uint64_t w[4] = {x0, x1, x2, x3};
  float* dst = out + static_cast<int64_t>(blockIdx.y) * n_per_expert + blk * 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (blk * 4 + q >= n_per_expert) break;
    const uint64_t v = w[q];
    const int32_t n = static_cast<int32_t>((v & 0xFFFF) + ((v >> 16) & 0xFFFF) + ((v >> 32) & 0xFFFF) +
                                           ((v >> 48) & 0xFFFF)) - 131070;
    dst[q] = static_cast<float>(n) * c;
  }
}

thread_local std::string g_err;

}  // namespace

extern "C" {

const char* nvfp4_synth_last_error(void) { return g_err.c_str(); }

float nvfp4_synth_scale(double sigma) {
  return static_cast<float>(sigma / sqrt(4.0 * (65536.0 * 65536.0 - 1.0) / 12.0));
}

int nvfp4_synth_weights(uint64_t seed, uint64_t tag, int64_t expert0, int64_t experts,
                        int64_t n_per_expert, double sigma, float* out_dev, void* stream) {
  if (!out_dev || experts < 1 || experts > 65535 || n_per_expert < 1 || expert0 < 0) {
    g_err = "invalid argument";
    return 1;
  }
  const int64_t blocks = (n_per_expert + 3) / 4;
  const dim3 grid(static_cast<unsigned>((blocks + 255) / 256), static_cast<unsigned>(experts));
  synth_weights_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(
      seed, tag, expert0, n_per_expert, nvfp4_synth_scale(sigma), out_dev);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_err = hipGetErrorString(e);
    return 6;
  }
  g_err.clear();
  return 0;
}

}  // extern "C"
