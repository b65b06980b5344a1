/*
 * nvfp4_moe.h — C-ABI of the MI355X (gfx950) NVFP4 fused-MoE layer with
 * online per-token activation quantization.
 *
 * Sources ("the pages"):
 *   [P1] prhub summary of sglang PR #28354: the CuTe DSL MoE backend gains
 *        per-token NVFP4 online quantization and in-place scale reload.
 *   [P2] prhub report of sglang PR #26696: MoE buffers are sized from the
 *        configured token ceiling, not from the first forward.
 *   [P3] prhub summary of sglang PR #36624: the MoE runner's steps (routing,
 *        expandInputRows, activation, finalize) around the expert GEMM.
 * NVFP4 here: E2M1 codes (OCP MX v1.0), one E4M3 scale (OFP8 "e4m3fn") per
 * 16 consecutive elements, and one binary32 global scale per token (per
 * expert for weights).
 *
 * Conventions for every entry point
 *   - Pointers named *_dev are device pointers (HBM) of the current HIP device;
 *     the library never copies them to the host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it asynchronously; no entry point synchronizes the
 *     host except moe_workspace_create / _destroy (allocation).  The library
 *     never creates streams ([P3] "Implementation breakdown" item 1: one pool
 *     per stream is what blew up graph-capture memory).
 *   - Return value: NVFP4_OK (0) or an nvfp4_status code.  All argument checks
 *     run on the host before anything is launched; on error nothing is
 *     enqueued and nvfp4_last_error() describes the failure.
 *   - Layouts are row-major and dense unless a leading dimension is given.
 *     Packed codes: byte j of a row holds element 2j in its low nibble and
 *     element 2j+1 in its high nibble.  Block scales are E4M3 bit patterns,
 *     one byte per 16 elements, row-major [rows, cols/16].
 */
#ifndef NVFP4_MOE_H
#define NVFP4_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARG = 1,      /* null / misaligned pointer, bad dimension */
  NVFP4_ERR_TOO_MANY_TOKENS = 2,  /* T above the workspace's max_num_tokens */
  NVFP4_ERR_ALIAS = 3,            /* output overlaps an input */
  NVFP4_ERR_NO_WEIGHTS = 4,       /* forward before moe_workspace_bind_weights */
  NVFP4_ERR_METADATA_CHANGED = 5, /* refresh with other dims */
  NVFP4_ERR_HIP = 6,              /* HIP runtime or launch error */
  NVFP4_ERR_OOM = 7               /* device allocation failed */
} nvfp4_status;

/* Thread-local description of the last error of this thread ("" if none). */
const char* nvfp4_last_error(void);

/*
 * Per-token NVFP4 quantization of a bf16 activation matrix.
 * [P1] "Feature and motivation" and "Implementation breakdown" item 2: each
 * token gets a dynamic binary32 global scale, the activations become packed
 * FP4 codes plus block-16 scales ("Review highlights": vector size 16).
 * Per row: g = 2688 / max|x| (g = 1 for an all-zero row; +inf clamps to
 * FLT_MAX); per 16-block b: S_b = E4M3_rne_sat(RN(RN(amax_b * g) / 6)),
 * r_b = RN(g / value(S_b)) (0 if S_b == 0; +inf saturates to FLT_MAX);
 * code = E2M1_rne_sat(RN(x * r_b)).
 * Dequantization: x ~= value(code) * value(S_b) / g.
 *
 *   x_dev       bf16 [rows, ld_x], 16-byte aligned, ld_x % 8 == 0, ld_x >= cols;
 *               finite values (an inf or NaN gives unspecified codes for its row)
 *   rows        0 <= rows < 2^31 (0 is a no-op)
 *   cols        > 0, multiple of 16
 *   codes_dev   u8 [rows, cols/2], 16-byte aligned   (written)
 *   scales_dev  u8 [rows, cols/16]                   (written)
 *   gscale_dev  f32 [rows], 4-byte aligned           (written)
 * Outputs must not overlap x.  Results are bit-identical to the CPU reading
 * of the recipe above (round to nearest even, no contraction).
 */
int nvfp4_quantize_per_token(const void* x_dev, int64_t rows, int64_t cols, int64_t ld_x,
                             void* codes_dev, void* scales_dev, float* gscale_dev,
                             void* stream);

/*
 * NVFP4 quantization of expert weights with one global scale per expert
 * (the online weight conversion of [P1] "Feature and motivation"; the
 * per-expert factors w1_alpha / w2_alpha of [P1] "Source snippets" undo it).
 * Same recipe as nvfp4_quantize_per_token, with g = 2688 / max|W[e]| over the
 * whole expert tensor and blocks along the last dimension.
 *
 *   w_dev       f32 [experts, rows, cols], 16-byte aligned
 *   experts, rows >= 1; cols > 0, multiple of 16
 *   codes_dev   u8 [experts, rows, cols/2], 16-byte aligned (written)
 *   scales_dev  u8 [experts, rows, cols/16]                  (written)
 *   gscale_dev  f32 [experts]                                (written)
 *   scratch_dev f32 [experts] caller-provided temporary (per-expert amax)
 */
int nvfp4_quantize_experts(const float* w_dev, int64_t experts, int64_t rows, int64_t cols,
                           void* codes_dev, void* scales_dev, float* gscale_dev,
                           float* scratch_dev, void* stream);

/* ---------------------------------------------------------------------- */
/* MoE layer                                                               */
/* ---------------------------------------------------------------------- */

/* Finalize mode flag.  [P1] "Implementation breakdown" item 1 and "Risks"
 * item 5: the fused atomic finalize is fast but not deterministic, and
 * deterministic inference switches it off.  Without this flag the weighted
 * top-k sum is accumulated with fp32 atomics in arrival order; with it the
 * k slot outputs are summed in slot order j = 0..k-1 (bit-reproducible). */
#define MOE_DETERMINISTIC_FINALIZE 0x1u

/* Static activation scales.  [P1] "Feature and motivation": the per-token
 * global scale replaces a static per-tensor input scale; "Source snippets":
 * the static fc2_input_scale of GEMM2's input.  With this flag the forward
 * quantizes x with one given global scale g_x and the SwiGLU output with one
 * given g_a (set by moe_workspace_set_act_scales) instead of 2688 / amax of
 * each row; the block recipe is the same, so values beyond 6 * 448 / g
 * saturate (E4M3 block scale 448, E2M1 code 6). */
#define MOE_STATIC_ACT_SCALES 0x2u

/* Shared expert.  [P3] Command-A-Plus multi-stream page,
 * Cohere2MoeSparseMoeBlock.forward: a shared expert runs on the same input
 * as the routed experts and the layer returns routed + shared, halved under
 * the 'average' combination strategy.  With MOE_SHARED_EXPERT the weights
 * hold num_experts + 1 experts and the last one is the shared expert: an
 * NVFP4 SwiGLU expert of the routed shape applied to every token with weight
 * 1, its input quantized per token like the routed experts' (it joins the
 * grouped GEMMs as one more group of T rows).  The router still chooses
 * among the first num_experts (logits stay [T, num_experts]).  The finalize
 * adds it to the weighted routed sum: out = bf16(c * (sum_j w_j y_j + y_s)),
 * c = 1, or 0.5 with MOE_SHARED_AVERAGE (which requires MOE_SHARED_EXPERT).
 * The deterministic finalize adds y_s after the k routed terms. */
#define MOE_SHARED_EXPERT 0x4u
#define MOE_SHARED_AVERAGE 0x8u

/* W4A16: bf16 activations, NVFP4 weights.  The pages only name this variant
 * ([P3] "Related work": a CuTe DSL NVFP4 W4A16 mode); read here as: no
 * activation is quantized — x itself (bf16) is GEMM1's input and the SwiGLU
 * output rounded to bf16 (nearest even) is GEMM2's input; the weights stay
 * NVFP4 (dequantized exactly to bf16 for bf16 MFMA), the outputs are scaled
 * by 1 / g_w only.  Not combinable with MOE_STATIC_ACT_SCALES
 * (NVFP4_ERR_INVALID_ARG). */
#define MOE_W4A16 0x10u

typedef struct moe_config {
  int64_t max_num_tokens; /* token ceiling: every buffer is sized from it once */
  int64_t hidden;         /* H: multiple of 128 */
  int64_t inter;          /* I: multiple of 128 */
  int32_t num_experts;    /* E: routed experts, 1..1024 */
  int32_t top_k;          /* k: 1..min(16, E) */
  uint32_t flags;         /* OR of the MOE_* flags above, or 0 */
} moe_config;

/* NVFP4 expert weights in the row-major boundary layout, device pointers
 * (the input of moe_pack_weights; refresh_scales_inplace takes the scales in
 * this layout).  w13 rows [0, I) are the gate projection (w1) and rows
 * [I, 2I) the up projection (w3); act = silu(gate) * up.
 *   w13_codes  u8 [E, 2I, H/2], 16-byte aligned   w13_scales u8 [E, 2I, H/16]
 *   w13_gscale f32 [E]                            (per-expert global scale)
 *   w2_codes   u8 [E, H, I/2],  16-byte aligned   w2_scales  u8 [E, H, I/16]
 *   w2_gscale  f32 [E]
 * For a workspace the dims must equal its own: num_experts = E, or E + 1
 * with MOE_SHARED_EXPERT (expert E is the shared one), and (H, I). */
typedef struct moe_nvfp4_weights {
  int64_t num_experts, hidden, inter;
  const void* w13_codes;
  const void* w13_scales;
  const float* w13_gscale;
  const void* w2_codes;
  const void* w2_scales;
  const float* w2_gscale;
} moe_nvfp4_weights;

/* Expert weights packed for the kernels, in caller-owned device memory.
 * w13 and w2 each hold the matrix's codes and block scales as "unit
 * records": a unit is four 16-row MMA fragments of one expert (for W13 gate
 * rows 32j..32j+31 with the matching up rows I+32j..; for W2 rows
 * 64j..64j+63), and the record of (unit, 128-wide K step) is 4608 bytes (4 KB
 * of codes, one lane's 32 codes per 16 bytes, then 512 bytes of their E4M3
 * scales), so that one wave reads a record as five contiguous spans.  This is
 * the kernels' analogue of the *_blockscale_mma copies of [P1]
 * "Implementation breakdown" item 3, here for codes and scales together.
 * Records are expert-major: expert e's records start at e times the
 * per-expert size (moe_packed_bytes with num_experts = 1), so experts can be
 * packed in pieces.
 *   w13        u8 [moe_packed_bytes w13], 16-byte aligned
 *   w13_gscale f32 [E]  per-expert global scales (copied at bind)
 *   w2         u8 [moe_packed_bytes w2], 16-byte aligned
 *   w2_gscale  f32 [E] */
typedef struct moe_nvfp4_packed {
  int64_t num_experts, hidden, inter;
  const void* w13;
  const float* w13_gscale;
  const void* w2;
  const float* w2_gscale;
} moe_nvfp4_packed;

/*
 * Bytes of the packed W13 and W2 buffers for E experts of hidden size H and
 * intermediate size I (multiples of 128).  Host-only, no device access.
 * NVFP4_ERR_INVALID_ARG for bad dims or NULL outputs.
 */
int moe_packed_bytes(int64_t num_experts, int64_t hidden, int64_t inter, int64_t* w13_bytes,
                     int64_t* w2_bytes);

/*
 * Pack row-major NVFP4 weights into the unit-record layout (the online
 * weight conversion's last step, [P1] "Feature and motivation"; done once
 * per weight load).  w13_packed_dev / w2_packed_dev are caller-owned device
 * buffers of moe_packed_bytes(w->num_experts, ...) bytes, 16-byte aligned,
 * not overlapping the inputs.  With NULL code pointers in `w` only the
 * scale bytes of the records are written (the codes already there stay).
 * The global scales in `w` are not read.  Enqueued on `stream`; the inputs
 * must stay valid until that work has run.
 */
int moe_pack_weights(const moe_nvfp4_weights* w, void* w13_packed_dev, void* w2_packed_dev, void* stream);

typedef struct moe_workspace moe_workspace;

/*
 * Create a workspace: every device buffer of the forward is allocated here,
 * once, from cfg->max_num_tokens ([P2] "Feature and motivation" and
 * "Implementation breakdown" items 1-3: sizing from the first forward's batch
 * crashed later, larger batches; the ceiling comes from configuration).
 * moe_token_ceiling() computes that ceiling from serving limits.
 * Limits: 1 <= max_num_tokens <= 2^24, max_num_tokens * top_k <= 2^30 and
 * max_num_tokens * hidden < 2^30 (the prefill kernels address one token
 * operand of fp16 rows with 32-bit byte offsets); otherwise
 * NVFP4_ERR_INVALID_ARG.
 * Synchronizes the device (allocation).  *out receives the handle.
 */
int moe_workspace_create(const moe_config* cfg, void* stream, moe_workspace** out);

/*
 * Bind packed expert weights (moe_pack_weights).  The packed records are
 * BORROWED: the caller owns them and must keep them alive, at the same
 * addresses, for as long as the workspace runs forwards; reloading codes in
 * place (moe_pack_weights into the same buffers) is picked up by the next
 * forward, captured graphs included.  The per-expert global scales are
 * COPIED into library-owned buffers.  May be called once per workspace.
 * Enqueued on `stream`; the global-scale arrays must stay valid until that
 * copy has run.  Dims must match the workspace (NVFP4_ERR_INVALID_ARG).
 */
int moe_workspace_bind_weights(moe_workspace* ws, const moe_nvfp4_packed* w, void* stream);

/*
 * Forward of the layer on T tokens:
 *   quantize x per token -> router top-k -> expandInputRows permutation ->
 *   grouped GEMM1 (gate+up) with SwiGLU -> per-row re-quantization ->
 *   grouped GEMM2 -> weighted finalize.
 * ([P3] "Feature and motivation": routing, expandInputRows, activation and
 * finalize around the expert GEMM; [P1] "Implementation breakdown" item 2:
 * quantize per token, then run the experts with the per-token scale.)
 * Router: the k largest logits (ties to the smaller expert index, slots in
 * descending order), weights = softmax over the chosen k.
 *
 *   x_dev        bf16 [T, H], 16-byte aligned
 *   logits_dev   f32 [T, E]
 *   T            0..max_num_tokens (0: no-op; above: NVFP4_ERR_TOO_MANY_TOKENS,
 *                message "num_tokens (T) exceeds max_num_tokens (M)")
 *   out_dev      bf16 [T, H], 16-byte aligned; must not overlap x_dev or
 *                logits_dev (NVFP4_ERR_ALIAS; [P3] "Implementation breakdown"
 *                item 2: in-place MoE output raced with a reader of the input)
 * No allocation and no host synchronization: the call can be captured in a
 * HIP graph.  One stream at a time per workspace.
 */
int moe_nvfp4_forward(moe_workspace* ws, const void* x_dev, const float* logits_dev, int64_t T,
                      void* out_dev, void* stream);

/*
 * The same forward for activations the caller has already quantized, as the
 * runner of [P1] "Implementation breakdown" item 2 is handed them (FP4 codes,
 * block scales and the per-token global scale, consumed by the expert GEMMs
 * as they are).  Step Q1 is skipped; everything after it is
 * moe_nvfp4_forward's, so codes that nvfp4_quantize_per_token wrote for x
 * give exactly moe_nvfp4_forward(x)'s output (bit for bit with
 * MOE_DETERMINISTIC_FINALIZE).
 *
 *   x_codes_dev   u8 [T, H/2], two E2M1 codes per byte (even element in the
 *                 low nibble), 16-byte aligned
 *   x_scales_dev  u8 [T, H/16], E4M3 block scales, 16-byte aligned; no NaN
 *                 byte (0x7F / 0xFF) is checked for: one gives NaN outputs
 *   x_gscale_dev  f32 [T], encode-direction global scales (a value is
 *                 code x scale / g), 4-byte aligned, finite and > 0
 *   logits_dev, T, out_dev, stream   as for moe_nvfp4_forward; out must not
 *                 overlap the three activation arrays (NVFP4_ERR_ALIAS)
 * The three arrays are read in place (borrowed for the call's duration on
 * `stream`) and never written.  With MOE_STATIC_ACT_SCALES only the GEMM2
 * input scale (scales[1]) is used.  A MOE_W4A16 workspace returns
 * NVFP4_ERR_INVALID_ARG (it takes bf16 activations).  No allocation and no
 * host synchronization.
 */
int moe_nvfp4_forward_quantized(moe_workspace* ws, const void* x_codes_dev, const void* x_scales_dev,
                                const float* x_gscale_dev, const float* logits_dev, int64_t T,
                                void* out_dev, void* stream);

/*
 * The forward without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  It computes exactly what moe_nvfp4_forward computes for
 * a workspace of configuration *cfg bound to *w (bit for bit with
 * MOE_DETERMINISTIC_FINALIZE), with no allocation: every intermediate lives
 * in one fixed 64 MiB device array inside the library, which each GPU the
 * library runs on holds until the process ends.
 *   cfg          dims and flags as for moe_workspace_create; T may not exceed
 *                cfg->max_num_tokens (NVFP4_ERR_TOO_MANY_TOKENS).
 *                MOE_STATIC_ACT_SCALES is not supported (NVFP4_ERR_INVALID_ARG)
 *   w            packed weights (moe_pack_weights), read in place together
 *                with its global-scale arrays for the call's duration
 *   x_dev, logits_dev, T, out_dev, stream   as for moe_nvfp4_forward
 * A forward whose intermediates exceed the array (for example more than
 * about 840 tokens of a 2048 x 768 x 128-expert top-8 layer, about 270 of a
 * 7168 x 2048 x 256-expert one) returns NVFP4_ERR_INVALID_ARG, naming the
 * largest token count that fits, and launches nothing.  All calls on one GPU
 * share that GPU's array, and it keeps the last call's contents: calls that
 * overlap on one GPU (other streams, other threads) race.  The first call on
 * each device looks the array's address up (make it outside graph capture).
 */
int moe_nvfp4_forward_noalloc(const moe_config* cfg, const moe_nvfp4_packed* w, const void* x_dev,
                              const float* logits_dev, int64_t T, void* out_dev, void* stream);

/*
 * Scale reload after a weight update ([P1] "Implementation breakdown" item 3
 * and "Source snippets", refresh_cutedsl_standard_scales_for_weight_update):
 * the new block scales are written INTO the bound packed records (the
 * caller's buffers, at the addresses bound) and the new global scales INTO
 * the workspace's copies, so addresses captured by a HIP graph stay valid.
 * `w` carries the new scales in the row-major layout; its code pointers must
 * be NULL (the codes live in the caller's packed buffers and are reloaded
 * there with moe_pack_weights; otherwise NVFP4_ERR_INVALID_ARG).  Dims that
 * differ from the bound ones return NVFP4_ERR_METADATA_CHANGED
 * ("recapture is required") and change nothing.  Enqueued on `stream`,
 * ordered with forwards on the same stream.
 */
int refresh_scales_inplace(moe_workspace* ws, const moe_nvfp4_weights* w, void* stream);

/*
 * Static activation scales (workspaces created with MOE_STATIC_ACT_SCALES):
 * copies scales_dev[0] = g_x (global scale of x) and scales_dev[1] = g_a
 * (global scale of GEMM2's input), binary32 encode-direction scales
 * (dequantized value = code * block scale / g), finite and > 0, from device
 * memory INTO the workspace, so a captured forward keeps its addresses and
 * uses the new values on its next replay.  Must be called before the first
 * forward; a forward before it returns NVFP4_ERR_INVALID_ARG.  Enqueued on
 * `stream`; the caller's buffer must stay valid until that work has run.
 * NVFP4_ERR_INVALID_ARG for a workspace without the flag or NULL pointers.
 */
int moe_workspace_set_act_scales(moe_workspace* ws, const float* scales_dev, void* stream);

/* Free library-owned memory (never the caller's packed weights).  NULL is a
 * no-op.  Synchronizes the device. */
int moe_workspace_destroy(moe_workspace* ws);

/*
 * Token ceiling of one forward from serving limits ([P2] "Source snippets",
 * cutedsl_moe_max_num_tokens): max(max_prefill, piecewise_max if > 0,
 * graph_max_bs * (spec_draft_tokens if > 0 else 1)).  piecewise_max = 0
 * means piecewise graphs are disabled.  Host-only, no device access.
 */
int moe_token_ceiling(int64_t max_prefill, int64_t piecewise_max, int64_t graph_max_bs,
                      int64_t spec_draft_tokens, int64_t* out);

/*
 * Read-only access to the workspace's intermediate buffers (for tests and
 * inspection).  Returns the device pointer and byte size of one buffer;
 * contents are those of the last forward on the workspace.
 *   MOE_BUF_XQ_CODES  u8 [T, H/2]     MOE_BUF_XQ_SCALES u8 [T, H/16]
 *   MOE_BUF_XQ_GSCALE f32 [T]         MOE_BUF_TOPK_IDS  i32 [T, k]
 *   MOE_BUF_TOPK_W    f32 [T, k]      MOE_BUF_COUNTS    i32 [E]
 *   MOE_BUF_OFFSETS   i32 [E + 1]     MOE_BUF_PERM      i32 [T*k] (row -> t*k+j)
 *   MOE_BUF_INV       i32 [T*k]       ((t*k+j) -> row)
 *   MOE_BUF_ACT       f32 [Rt, I]     SwiGLU output per expanded row
 *   MOE_BUF_A2_CODES  u8 [Rt, I/2]    MOE_BUF_A2_SCALES u8 [Rt, I/16]
 *   MOE_BUF_A2_GSCALE f32 [Rt]        re-quantized activation
 *   MOE_BUF_A2_16     16-bit [Rt, I]  GEMM2's 16-bit input when the tiled
 *                     GEMMs run: fp16 of the re-quantized act, or (W4A16)
 *                     act rounded to bf16
 * where Rt = T*k, plus T with MOE_SHARED_EXPERT: rows [0, T*k) are the
 * routed rows in expert order, row T*k + t the shared expert's row of token
 * t.
 * (sizes are reported for max_num_tokens rows)
 */
typedef enum moe_buffer_id {
  MOE_BUF_XQ_CODES = 0,
  MOE_BUF_XQ_SCALES,
  MOE_BUF_XQ_GSCALE,
  MOE_BUF_TOPK_IDS,
  MOE_BUF_TOPK_W,
  MOE_BUF_COUNTS,
  MOE_BUF_OFFSETS,
  MOE_BUF_PERM,
  MOE_BUF_INV,
  MOE_BUF_ACT,
  MOE_BUF_A2_CODES,
  MOE_BUF_A2_SCALES,
  MOE_BUF_A2_GSCALE,
  MOE_BUF_A2_16,
  MOE_BUF_COUNT_
} moe_buffer_id;

int moe_workspace_buffer(const moe_workspace* ws, int32_t id, void** ptr_out, int64_t* bytes_out);

/*
 * Per-stage timing (inspection and benchmarks).  With events != NULL, every
 * later forward on the workspace records the five caller-owned hipEvent_t
 * handles events[0..4] on its stream: events[0] before the prologue kernel
 * (quantize + route + permute), events[1] after it, events[2] after GEMM1 +
 * SwiGLU, events[3] after GEMM2 (with the fused re-quantization), events[4]
 * after the finalize.  The handles are copied; pass new ones before each
 * forward to keep several forwards' timings.  NULL stops recording.
 */
int moe_workspace_set_stage_events(moe_workspace* ws, void* const* events);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_MOE_H */
