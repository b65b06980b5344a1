// NVFP4 MoE oracle — TEST INFRASTRUCTURE ONLY.
//
// A plain, slow CPU implementation of what the NVFP4 fused-MoE layer with
// online per-token activation quantization computes.  Only the test suite,
// the package smoke check and the benchmark's CPU-baseline leg may load this
// library; the product path never does.  It shares no code with the HIP
// kernels under nvfp4_token_quant_amd/csrc.
//
// Sources ("the pages"):
//   [P1] prhub summary of sglang PR #28354 (CuTe DSL backend: per-token NVFP4
//        online quantization and in-place scale reload).
//   [P2] prhub report of sglang PR #26696 (size CuteDSL MoE buffers from the
//        configured token ceiling).
//   [P3] prhub summary of sglang PR #36624 (Command-A-Plus on SM10X; the MoE
//        runner's step list: routing, expandInputRows, activation, finalize).
//   Format definitions the pages use but do not write out:
//   [MX]  OCP Microscaling Formats (MX) Specification v1.0, FP4 E2M1 element
//         type (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).
//   [OFP8] OCP 8-bit Floating Point Specification (OFP8), E4M3 ("fn":
//         bias 7, max 448, no infinities, NaN = S.1111.111).
//
// Arithmetic rules: binary32 operations round to nearest even, no FMA
// contraction (built with -ffp-contract=off), denormals kept; dot products
// and dequantized values are binary64.
//
// Every function states the passage or definition it follows.  Readings of
// points the pages leave open are marked READING.

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_API extern "C" __attribute__((visibility("default")))

namespace {

float bits_to_float(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// bf16 -> binary32 is exact: the bf16 pattern is the top half of the float.
float bf16_to_float(uint16_t b) { return bits_to_float(static_cast<uint32_t>(b) << 16); }

// binary32 -> bfloat16 rounded to nearest, ties to even: bf16 keeps the top
// 16 bits of the binary32 pattern (sign, the 8 exponent bits, 7 fraction
// bits); the dropped 16 bits decide the rounding (above half: up; exactly
// half: up only if the kept part is odd).  A carry out of the fraction steps
// the exponent, which is the correctly rounded result (up to infinity).
// NaN stays NaN.
uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  const uint32_t dropped = u & 0xffffu;
  uint32_t kept = u >> 16;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) ++kept;
  return static_cast<uint16_t>(kept);
}

// [MX] E2M1 magnitudes, indexed by the 3 low code bits (e1 e0 m).
const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

// [OFP8] E4M3 decode: e = bits 6..3, m = bits 2..0, bias 7; e == 0 is
// subnormal (m/8 * 2^-6).  Only the 127 finite non-negative codes are used.
double e4m3_decode(uint8_t b) {
  int e = (b >> 3) & 15, m = b & 7;
  if (e == 0) return std::ldexp(m / 8.0, -6);
  return std::ldexp(1.0 + m / 8.0, e - 7);
}

// The decode above for all 256 bytes, computed once (the encoder searches
// and the dequantization look values up instead of calling ldexp each time;
// the values are the same).
struct E4M3Table {
  double v[256];
  E4M3Table() {
    for (int b = 0; b < 256; ++b) v[b] = e4m3_decode(static_cast<uint8_t>(b));
  }
};

double e4m3_value(uint8_t b) {
  static const E4M3Table table;
  return table.v[b];
}

}  // namespace

// ---------------------------------------------------------------------------
// Encoders.  Both are "round to nearest, ties to the code whose least
// significant mantissa bit is 0, saturate to the largest finite magnitude"
// written as a search over the format's values: the nearest value wins, and a
// tie keeps the candidate with an even code.
// ---------------------------------------------------------------------------

// [MX] E2M1 encode of a binary32 value.  The sign bit is the IEEE sign bit of
// v, so a negative value that rounds to zero gives code 0x8.  Values beyond 6
// saturate to 6 (6 is simply the nearest grid value).
ORC_API uint8_t orc_e2m1_encode(float v) {
  const uint8_t sign = std::signbit(v) ? 0x8 : 0x0;
  const double a = std::fabs(static_cast<double>(v));
  if (a >= 6.0) return static_cast<uint8_t>(sign | 7);  // saturation
  int best = 0;
  double best_d = std::fabs(a - kE2M1[0]);
  for (int c = 1; c < 8; ++c) {
    double d = std::fabs(a - kE2M1[c]);
    if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_d = d;
    }
  }
  return static_cast<uint8_t>(sign | best);
}

static double e2m1_value(uint8_t code) {
  double v = kE2M1[code & 7];
  return (code & 8) ? -v : v;
}

ORC_API double orc_e2m1_value(uint8_t code) { return e2m1_value(code); }

// [OFP8] E4M3 encode of a non-negative finite scale with saturation to 448
// (0x7E): the nearest of the 127 finite codes 0x00..0x7E, ties to even code.
ORC_API uint8_t orc_e4m3_encode(float s) {
  const double a = static_cast<double>(s);
  if (a >= 448.0) return 0x7E;  // saturation (satfinite)
  int best = 0;
  double best_d = std::fabs(a - e4m3_value(0));
  for (int c = 1; c <= 0x7E; ++c) {
    double d = std::fabs(a - e4m3_value(static_cast<uint8_t>(c)));
    if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_d = d;
    }
  }
  return static_cast<uint8_t>(best);
}

ORC_API double orc_e4m3_value(uint8_t b) { return e4m3_value(b); }

// ---------------------------------------------------------------------------
// Quantization Q.
//
// [P1] "Feature and motivation": the activation path uses a per-token,
// dynamic FP32 global scale.  [P1] "Implementation breakdown" item 2 and
// "Source snippets" (_make_per_token_global_scale): the global scale comes
// from a shared helper that uses the E4M3 maximum; [P1] "Review highlights":
// scale-factor vectors hold 16 elements.
//
// READING (the pages never print the formula): standard two-level NVFP4
// scaling in the encode direction,
//   a   = max |x|                                   (row, or whole tensor)
//   g   = 448*6 / a  (a > 0; +inf clamps to FLT_MAX), g = 1 for a == 0
//   per 16-block b:  s_b = RN(RN(amax_b * g) / 6),  S_b = E4M3(s_b),
//                    d_b = value(S_b),  r_b = d_b > 0 ? RN(g / d_b) : 0,
//                    +inf saturating to FLT_MAX (READING: with g clamped, g / d_b
//                    can overflow, and inf * 0 would make zeros NaN)
//   per element:     c_k = E2M1(RN(x_k * r_b))
//   packing: byte j holds element 2j in the low nibble, 2j+1 in the high one.
// Dequantization: x^_k = value(c_k) * d_b / g (binary64).
// ---------------------------------------------------------------------------

namespace {

float global_scale_from_amax(float a) {
  if (!(a > 0.0f)) return 1.0f;
  float g = 2688.0f / a;  // 2688 = 448 (E4M3 max) * 6 (E2M1 max)
  if (std::isinf(g)) g = FLT_MAX;
  return g;
}

// Quantize one row of K values (K % 16 == 0) with a given global scale g.
void quantize_with_g(const float* x, int64_t K, float g, uint8_t* codes, uint8_t* S) {
  for (int64_t b = 0; b < K / 16; ++b) {
    const float* xb = x + 16 * b;
    float ab = 0.0f;
    for (int i = 0; i < 16; ++i) ab = std::max(ab, std::fabs(xb[i]));
    float t = ab * g;
    float s = t / 6.0f;
    uint8_t sb = orc_e4m3_encode(s);
    S[b] = sb;
    float d = static_cast<float>(e4m3_value(sb));  // exact: E4M3 values are binary32 values
    float r = d > 0.0f ? g / d : 0.0f;
    if (std::isinf(r)) r = FLT_MAX;
    for (int i = 0; i < 16; i += 2) {
      float v0 = xb[i] * r;
      float v1 = xb[i + 1] * r;
      uint8_t c0 = orc_e2m1_encode(v0), c1 = orc_e2m1_encode(v1);
      codes[(16 * b + i) / 2] = static_cast<uint8_t>(c0 | (c1 << 4));
    }
  }
}

}  // namespace

// Global scale of a row / tensor from its values (exposed for pins).
ORC_API float orc_global_scale(const float* x, int64_t n) {
  float a = 0.0f;
  for (int64_t i = 0; i < n; ++i) a = std::max(a, std::fabs(x[i]));
  return global_scale_from_amax(a);
}

// Per-token quantization: each of `rows` rows of x[rows, K] gets its own g.
ORC_API void orc_quantize_rows(const float* x, int64_t rows, int64_t K, uint8_t* codes,
                               uint8_t* S, float* g) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * K;
    float gr = orc_global_scale(xr, K);
    g[r] = gr;
    quantize_with_g(xr, K, gr, codes + r * (K / 2), S + r * (K / 16));
  }
}

// Same as orc_quantize_rows for bf16 input (converted exactly to binary32).
ORC_API void orc_quantize_rows_bf16(const uint16_t* x, int64_t rows, int64_t K,
                                    uint8_t* codes, uint8_t* S, float* g) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    std::vector<float> xf(K);
    for (int64_t k = 0; k < K; ++k) xf[k] = bf16_to_float(x[r * K + k]);
    float gr = orc_global_scale(xf.data(), K);
    g[r] = gr;
    quantize_with_g(xf.data(), K, gr, codes + r * (K / 2), S + r * (K / 16));
  }
}

// Rows quantized with a caller-given global scale per row (used by the
// group quantizer below and by pins of the static-scale case).
ORC_API void orc_quantize_rows_given_g(const float* x, int64_t rows, int64_t K,
                                       const float* g, uint8_t* codes, uint8_t* S) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    quantize_with_g(x + r * K, K, g[r], codes + r * (K / 2), S + r * (K / 16));
}

// Weight quantization: one global scale per group of `rows` rows (one group
// = one expert's w13 [2I, H] or w2 [H, I]); blocks run along K.
// READING: per-expert FP32 global scale from the amax of the whole expert
// tensor; [P1] "Source snippets" names w1_alpha / w2_alpha, the per-expert
// factors that undo activation and weight global scales.
ORC_API void orc_quantize_groups(const float* x, int64_t groups, int64_t rows, int64_t K,
                                 uint8_t* codes, uint8_t* S, float* g) {
  for (int64_t e = 0; e < groups; ++e) {
    const float* xe = x + e * rows * K;
    float ge = orc_global_scale(xe, rows * K);
    g[e] = ge;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
      quantize_with_g(xe + r * K, K, ge, codes + (e * rows + r) * (K / 2),
                      S + (e * rows + r) * (K / 16));
  }
}

// Dequantize rows: out[r, k] = value(c) * value(S) / g_of_row(r), binary64.
// g_stride_rows: how many consecutive rows share one global scale
// (1 for per-token activations, rows-per-expert for weights).
ORC_API void orc_dequantize(const uint8_t* codes, const uint8_t* S, const float* g,
                            int64_t rows, int64_t K, int64_t g_stride_rows, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double gr = g[r / g_stride_rows];
    for (int64_t k = 0; k < K; ++k) {
      uint8_t byte = codes[r * (K / 2) + k / 2];
      uint8_t c = (k & 1) ? (byte >> 4) : (byte & 15);
      double d = e4m3_value(S[r * (K / 16) + k / 16]);
      out[r * K + k] = e2m1_value(c) * d / gr;
    }
  }
}

// ---------------------------------------------------------------------------
// Router.  [P3] "Source snippets" (Cohere2MoeSparseMoeBlock.forward): the
// gate produces router logits and topk turns them into top-k ids and weights;
// [P3] "Feature and motivation" lists routing as its own step.
// READING: the k largest logits (binary32 compare; equal logits go to the
// smaller expert index; slots in descending logit order); weights are the
// softmax over all experts restricted to the chosen k and renormalized, which
// equals exp(l_j - l_0) / sum_j' exp(l_j' - l_0) over the chosen slots.
// ---------------------------------------------------------------------------
ORC_API void orc_router(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* ids,
                        double* w) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    std::vector<char> taken(E, 0);
    for (int64_t j = 0; j < k; ++j) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;  // strict: ties keep the smaller index
      }
      taken[best] = 1;
      ids[t * k + j] = static_cast<int32_t>(best);
    }
    double l0 = l[ids[t * k]];
    double denom = 0.0;
    for (int64_t j = 0; j < k; ++j) denom += std::exp(static_cast<double>(l[ids[t * k + j]]) - l0);
    for (int64_t j = 0; j < k; ++j)
      w[t * k + j] = std::exp(static_cast<double>(l[ids[t * k + j]]) - l0) / denom;
  }
}

// ---------------------------------------------------------------------------
// expandInputRows permutation.  [P3] "Feature and motivation" names it as one
// of the steps around the expert GEMM.  READING: a stable counting sort of
// the token-major list of (t, j) pairs by expert: counts, exclusive offsets,
// rows of one expert in ascending (t, j) order.
//   perm[row] = t*k + j,  inv[t*k + j] = row.
// ---------------------------------------------------------------------------
ORC_API void orc_permute(const int32_t* ids, int64_t T, int64_t k, int64_t E, int32_t* counts,
                         int32_t* offsets, int32_t* perm, int32_t* inv) {
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < T * k; ++i) counts[ids[i]]++;
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> cursor(offsets, offsets + E);
  for (int64_t i = 0; i < T * k; ++i) {
    int32_t row = cursor[ids[i]]++;
    perm[row] = static_cast<int32_t>(i);
    inv[i] = row;
  }
}

// ---------------------------------------------------------------------------
// The layer.  [P3] "Feature and motivation": routing, expandInputRows,
// activation and finalize around the expert GEMM; [P1] "Implementation
// breakdown" items 2-3: the activations are quantized per token before the
// expert GEMMs, the w13 (gate+up) and w2 weights are NVFP4 with block scales,
// and w1_alpha / w2_alpha undo the global scales.
//
// For each token t and slot j with expert e = ids[t, j]:
//   h    = x^[t] . W^13[e]^T               (binary64, length 2I)
//   act  = silu(h[0:I]) * h[I:2I]          (READING: rows [0, I) of w13 are
//                                           the gate, rows [I, 2I) the up
//                                           projection; silu(z) = z/(1+e^-z))
//   a32  = (float) act                     (READING: act stays binary32)
//   (c2, S2, g2) = Q(a32)                  (READING: dynamic re-quantization
//                                           per expanded row)
// With static activation scales (the per-tensor input-scale contract the
// per-token scheme replaces, [P1] "Feature and motivation"; the static
// fc2_input_scale of "Source snippets"), x is quantized with the given g_x
// and a32 with the given g_a instead of 2688 / amax of the row; the block
// recipe is unchanged, so out-of-range values saturate (E4M3 at 448, E2M1
// at 6).
//   y    = a^2 . W^2[e]^T                  (binary64, length H)
// out[t] = sum_j w[t, j] * y_(t, j)        (binary64)
//
// Weights arrive compact: only the experts listed in `experts` (n_experts of
// them, in that order) are present in the code / scale arrays.
// ---------------------------------------------------------------------------

namespace {

struct LayerArgs {
  int64_t H, I, k;
  const uint8_t *w13c, *w13s, *w2c, *w2s;
  const float *w13g, *w2g;
};

void dequant_rows(const uint8_t* codes, const uint8_t* S, double g, int64_t rows, int64_t K,
                  double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < K / 16; ++b) {
      const double d = e4m3_value(S[r * (K / 16) + b]);  // the block's scale
      for (int64_t k = 16 * b; k < 16 * b + 16; ++k) {
        uint8_t byte = codes[r * (K / 2) + k / 2];
        uint8_t c = (k & 1) ? (byte >> 4) : (byte & 15);
        out[r * K + k] = e2m1_value(c) * d / g;
      }
    }
}

double silu(double z) { return z / (1.0 + std::exp(-z)); }

// One expert applied to one dequantized activation row xh[H] -> y[H]; also
// returns the intermediates for the debug entry point.
// a16: W4A16 (the GEMM2 input is act rounded to bf16 instead of its NVFP4
// re-quantization; c2, S2, g2 are left untouched).
void expert_row(const LayerArgs& a, const double* W13, const double* W2, const double* xh,
                double* h, float* a32, uint8_t* c2, uint8_t* S2, float* g2, double* ah,
                double* y, float static_ga, bool a16) {
  const int64_t H = a.H, I = a.I;
  for (int64_t n = 0; n < 2 * I; ++n) {
    double acc = 0.0;
    for (int64_t kk = 0; kk < H; ++kk) acc += xh[kk] * W13[n * H + kk];
    h[n] = acc;
  }
  for (int64_t i = 0; i < I; ++i) a32[i] = static_cast<float>(silu(h[i]) * h[I + i]);
  if (a16) {
    for (int64_t i = 0; i < I; ++i) ah[i] = bf16_to_float(float_to_bf16_rne(a32[i]));
  } else {
    *g2 = static_ga > 0.0f ? static_ga : orc_global_scale(a32, I);
    quantize_with_g(a32, I, *g2, c2, S2);
    dequant_rows(c2, S2, *g2, 1, I, ah);
  }
  for (int64_t n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int64_t i = 0; i < I; ++i) acc += ah[i] * W2[n * I + i];
    y[n] = acc;
  }
}

}  // namespace

namespace {

// The layer from the dequantized activation rows xh [n_tok, H] (binary64) of
// the listed tokens; the remaining arguments as for orc_moe_layer.
int layer_from_rows(const std::vector<double>& xh, const int32_t* ids, const double* w,
                    const int64_t* tokens, int64_t n_tok, int64_t H, int64_t I, int64_t k,
                    const int32_t* experts, int64_t n_experts, const uint8_t* w13c,
                    const uint8_t* w13s, const float* w13g, const uint8_t* w2c, const uint8_t* w2s,
                    const float* w2g, float static_ga, int a16, double* out, double* y_dbg,
                    float* act_dbg, uint8_t* c2_dbg, uint8_t* S2_dbg, float* g2_dbg) {
  LayerArgs a{H, I, k, w13c, w13s, w2c, w2s, w13g, w2g};
  int32_t max_e = 0;
  for (int64_t i = 0; i < n_experts; ++i) max_e = std::max(max_e, experts[i]);
  std::vector<int64_t> slot_of(static_cast<size_t>(max_e) + 1, -1);
  for (int64_t i = 0; i < n_experts; ++i) slot_of[experts[i]] = i;
  for (int64_t ti = 0; ti < n_tok; ++ti)
    for (int64_t j = 0; j < k; ++j) {
      int32_t e = ids[tokens[ti] * k + j];
      if (e > max_e || slot_of[e] < 0) return -1;
    }

  std::vector<double> ybuf(static_cast<size_t>(n_tok * k * H));
  // Parallel over experts: each thread dequantizes one expert's weights and
  // applies it to every listed (token, slot) routed there.
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ei = 0; ei < n_experts; ++ei) {
    bool used = false;
    for (int64_t ti = 0; ti < n_tok && !used; ++ti)
      for (int64_t j = 0; j < k; ++j)
        if (ids[tokens[ti] * k + j] == experts[ei]) used = true;
    if (!used) continue;
    std::vector<double> W13(static_cast<size_t>(2 * I * H)), W2(static_cast<size_t>(H * I));
    dequant_rows(w13c + ei * 2 * I * (H / 2), w13s + ei * 2 * I * (H / 16), w13g[ei], 2 * I, H,
                 W13.data());
    dequant_rows(w2c + ei * H * (I / 2), w2s + ei * H * (I / 16), w2g[ei], H, I, W2.data());
    std::vector<double> h(2 * I), ah(I);
    std::vector<float> a32(I), g2(1);
    std::vector<uint8_t> c2(I / 2), S2(I / 16);
    for (int64_t ti = 0; ti < n_tok; ++ti)
      for (int64_t j = 0; j < k; ++j) {
        if (ids[tokens[ti] * k + j] != experts[ei]) continue;
        double* y = ybuf.data() + (ti * k + j) * H;
        expert_row(a, W13.data(), W2.data(), xh.data() + ti * H, h.data(), a32.data(), c2.data(),
                   S2.data(), g2.data(), ah.data(), y, static_ga, a16 != 0);
        int64_t slot = ti * k + j;
        if (act_dbg) std::memcpy(act_dbg + slot * I, a32.data(), I * sizeof(float));
        if (c2_dbg) std::memcpy(c2_dbg + slot * (I / 2), c2.data(), I / 2);
        if (S2_dbg) std::memcpy(S2_dbg + slot * (I / 16), S2.data(), I / 16);
        if (g2_dbg) g2_dbg[slot] = g2[0];
      }
  }

  // Finalize: weighted sum over the k slots.  [P1] "Implementation
  // breakdown" item 1 and "Risks": fused atomic finalize is the fast,
  // non-deterministic default and deterministic inference switches it off;
  // mathematically both compute this sum.
  for (int64_t ti = 0; ti < n_tok; ++ti)
    for (int64_t n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int64_t j = 0; j < k; ++j)
        acc += w[tokens[ti] * k + j] * ybuf[(ti * k + j) * H + n];
      out[ti * H + n] = acc;
    }
  if (y_dbg) std::memcpy(y_dbg, ybuf.data(), ybuf.size() * sizeof(double));
  return 0;
}

}  // namespace

// Layer output for the tokens listed in `tokens` (n_tok of them).
//   x_bf16   [T_all, H] activations (bf16 bits); only listed rows are read
//   ids, w   [T_all, k] routing (from orc_router); only listed rows are read
//   experts  [n_experts] expert ids present in the compact weight arrays
//   w13c [n_experts, 2I, H/2], w13s [n_experts, 2I, H/16], w13g [n_experts]
//   w2c  [n_experts, H, I/2],  w2s  [n_experts, H, I/16],  w2g  [n_experts]
//   out      [n_tok, H] binary64
//   static_gx, static_ga  > 0: static global scales of x and of the GEMM2
//                         input; <= 0: per-row scales (the default)
//   a16      1: W4A16 — x (bf16) and act rounded to bf16 are the GEMM
//            inputs, no activation quantization (c2/S2/g2 debug not written)
// Optional debug outputs (may be null), per listed token and slot:
//   y_dbg [n_tok, k, H], act_dbg [n_tok, k, I] (binary32),
//   c2_dbg [n_tok, k, I/2], S2_dbg [n_tok, k, I/16], g2_dbg [n_tok, k]
// Returns 0, or -1 if a routed expert is missing from `experts`.
ORC_API int orc_moe_layer(const uint16_t* x_bf16, const int32_t* ids, const double* w,
                          const int64_t* tokens, int64_t n_tok, int64_t H, int64_t I, int64_t k,
                          const int32_t* experts, int64_t n_experts, const uint8_t* w13c,
                          const uint8_t* w13s, const float* w13g, const uint8_t* w2c,
                          const uint8_t* w2s, const float* w2g, float static_gx, float static_ga,
                          int a16, double* out, double* y_dbg, float* act_dbg, uint8_t* c2_dbg,
                          uint8_t* S2_dbg, float* g2_dbg) {
  // Activation rows: Q then dequantize (binary64); W4A16: the bf16 values.
  std::vector<double> xh(static_cast<size_t>(n_tok * H));
  std::vector<uint8_t> c(H / 2), s(H / 16);
  std::vector<float> xf(H);
  for (int64_t ti = 0; ti < n_tok; ++ti) {
    const uint16_t* xr = x_bf16 + tokens[ti] * H;
    for (int64_t kk = 0; kk < H; ++kk) xf[kk] = bf16_to_float(xr[kk]);
    if (a16) {
      for (int64_t kk = 0; kk < H; ++kk) xh[ti * H + kk] = xf[kk];
      continue;
    }
    float g = static_gx > 0.0f ? static_gx : orc_global_scale(xf.data(), H);
    quantize_with_g(xf.data(), H, g, c.data(), s.data());
    dequant_rows(c.data(), s.data(), g, 1, H, xh.data() + ti * H);
  }
  return layer_from_rows(xh, ids, w, tokens, n_tok, H, I, k, experts, n_experts, w13c, w13s, w13g,
                         w2c, w2s, w2g, static_ga, a16, out, y_dbg, act_dbg, c2_dbg, S2_dbg, g2_dbg);
}

// The same layer for activations handed over already quantized (the runner
// contract of [P1] "Implementation breakdown" item 2: FP4 codes, block scales
// and the per-token global scale go into the expert GEMMs): xq_codes
// [T_all, H/2], xq_scales [T_all, H/16] (E4M3 bits), xq_g [T_all] (the
// encode-direction global scale; a value is code x scale / g).  Step 1 of
// the layer (Q of x) is replaced by these; everything after it is the same.
ORC_API int orc_moe_layer_xq(const uint8_t* xq_codes, const uint8_t* xq_scales, const float* xq_g,
                             const int32_t* ids, const double* w, const int64_t* tokens,
                             int64_t n_tok, int64_t H, int64_t I, int64_t k, const int32_t* experts,
                             int64_t n_experts, const uint8_t* w13c, const uint8_t* w13s,
                             const float* w13g, const uint8_t* w2c, const uint8_t* w2s,
                             const float* w2g, float static_ga, double* out) {
  std::vector<double> xh(static_cast<size_t>(n_tok * H));
  for (int64_t ti = 0; ti < n_tok; ++ti) {
    const int64_t t = tokens[ti];
    dequant_rows(xq_codes + t * (H / 2), xq_scales + t * (H / 16), xq_g[t], 1, H,
                 xh.data() + ti * H);
  }
  return layer_from_rows(xh, ids, w, tokens, n_tok, H, I, k, experts, n_experts, w13c, w13s, w13g,
                         w2c, w2s, w2g, static_ga, 0, out, nullptr, nullptr, nullptr, nullptr,
                         nullptr);
}

// Brute-force dense variant (tiny inputs): every expert is applied to every
// token, and the output keeps the routed ones with their weights:
//   out[t] = sum_e [e in topk(t)] * w[t, e] * y_e(t).
// Weights are given for all E experts (not compact).
ORC_API void orc_moe_layer_dense(const uint16_t* x_bf16, const int32_t* ids, const double* w,
                                 int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                                 const uint8_t* w13c, const uint8_t* w13s, const float* w13g,
                                 const uint8_t* w2c, const uint8_t* w2s, const float* w2g,
                                 float static_gx, float static_ga, int a16, double* out) {
  LayerArgs a{H, I, k, w13c, w13s, w2c, w2s, w13g, w2g};
  std::vector<double> W13(static_cast<size_t>(2 * I * H)), W2(static_cast<size_t>(H * I));
  std::vector<double> xh(H), h(2 * I), ah(I), y(H);
  std::vector<float> xf(H), a32(I), g2(1);
  std::vector<uint8_t> c(H / 2), s(H / 16), c2(I / 2), S2(I / 16);
  for (int64_t i = 0; i < T * H; ++i) out[i] = 0.0;
  for (int64_t e = 0; e < E; ++e) {
    dequant_rows(w13c + e * 2 * I * (H / 2), w13s + e * 2 * I * (H / 16), w13g[e], 2 * I, H,
                 W13.data());
    dequant_rows(w2c + e * H * (I / 2), w2s + e * H * (I / 16), w2g[e], H, I, W2.data());
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t kk = 0; kk < H; ++kk) xf[kk] = bf16_to_float(x_bf16[t * H + kk]);
      if (a16) {
        for (int64_t kk = 0; kk < H; ++kk) xh[kk] = xf[kk];
      } else {
        float g = static_gx > 0.0f ? static_gx : orc_global_scale(xf.data(), H);
        quantize_with_g(xf.data(), H, g, c.data(), s.data());
        dequant_rows(c.data(), s.data(), g, 1, H, xh.data());
      }
      expert_row(a, W13.data(), W2.data(), xh.data(), h.data(), a32.data(), c2.data(),
                 S2.data(), g2.data(), ah.data(), y.data(), static_ga, a16 != 0);
      double wt = 0.0;
      for (int64_t j = 0; j < k; ++j)
        if (ids[t * k + j] == e) wt = w[t * k + j];
      for (int64_t n = 0; n < H; ++n) out[t * H + n] += wt * y[n];
    }
  }
}

// ---------------------------------------------------------------------------
// Synthetic weights (input generation, not the method).  Counter-based so
// that the GPU side, which writes its own generator from the same published
// definition, produces the same bits without moving gigabytes over PCIe.
//
// Philox4x64-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3" (SC'11), Philox-4x64 with 10 rounds.  Round: two 64x64->128
// products with multipliers M0 = 0xD2E7470EE14C6C93, M1 = 0xCA5A826395121157;
// new = (hi(M1*x2) ^ x1 ^ k0, lo(M1*x2), hi(M0*x0) ^ x3 ^ k1, lo(M0*x0));
// the key is bumped by the Weyl constants W0 = 0x9E3779B97F4A7C15,
// W1 = 0xBB67AE8584CAA73B between rounds.
// ---------------------------------------------------------------------------
// binary32 -> bfloat16 bits, round to nearest even, for n values.
ORC_API void orc_f32_to_bf16(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = float_to_bf16_rne(x[i]);
}

ORC_API void orc_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2],
                               uint64_t out[4]) {
  uint64_t x0 = ctr_in[0], x1 = ctr_in[1], x2 = ctr_in[2], x3 = ctr_in[3];
  uint64_t k0 = key_in[0], k1 = key_in[1];
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += W0;
      k1 += W1;
    }
    unsigned __int128 p0 = static_cast<unsigned __int128>(M0) * x0;
    unsigned __int128 p1 = static_cast<unsigned __int128>(M1) * x2;
    uint64_t hi0 = static_cast<uint64_t>(p0 >> 64), lo0 = static_cast<uint64_t>(p0);
    uint64_t hi1 = static_cast<uint64_t>(p1 >> 64), lo1 = static_cast<uint64_t>(p1);
    uint64_t n0 = hi1 ^ x1 ^ k0, n1 = lo1, n2 = hi0 ^ x3 ^ k1, n3 = lo0;
    x0 = n0;
    x1 = n1;
    x2 = n2;
    x3 = n3;
  }
  out[0] = x0;
  out[1] = x1;
  out[2] = x2;
  out[3] = x3;
}

// Scale of the Irwin-Hall(4) sum of 16-bit uniforms: sigma / sqrt(4 * (2^32 - 1) / 12),
// computed in binary64 and rounded once to binary32.
ORC_API float orc_synth_scale(double sigma) {
  return static_cast<float>(sigma / std::sqrt(4.0 * (65536.0 * 65536.0 - 1.0) / 12.0));
}

// Synthetic weight tensor of one expert: element i (row-major over
// [rows, cols]) comes from Philox4x64-10 with key (seed, tag) and counter
// (i / 4, expert, 0, 0), output word i % 4; the word's four 16-bit fields are
// summed and centred (Irwin-Hall of order 4, range +-131070) and multiplied
// by orc_synth_scale(sigma) in binary32.
ORC_API void orc_synth_weights(uint64_t seed, uint64_t tag, int64_t expert, int64_t n_elems,
                               double sigma, float* out) {
  const float c = orc_synth_scale(sigma);
  const uint64_t key[2] = {seed, tag};
#pragma omp parallel for schedule(static)
  for (int64_t blk = 0; blk < (n_elems + 3) / 4; ++blk) {
    uint64_t ctr[4] = {static_cast<uint64_t>(blk), static_cast<uint64_t>(expert), 0, 0};
    uint64_t o[4];
    orc_philox4x64_10(ctr, key, o);
    for (int q = 0; q < 4; ++q) {
      int64_t i = blk * 4 + q;
      if (i >= n_elems) break;
      uint64_t wd = o[q];
      int32_t n = static_cast<int32_t>((wd & 0xFFFF) + ((wd >> 16) & 0xFFFF) +
                                       ((wd >> 32) & 0xFFFF) + ((wd >> 48) & 0xFFFF)) -
                  131070;
      out[i] = static_cast<float>(n) * c;
    }
  }
}

ORC_API int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
