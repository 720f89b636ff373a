/*
 * qsmoe.h -- C ABI of the MI355X (gfx950) routed-expert MoE layer library.
 *
 * The layer is the DeepSeek-V4 MoE FFN as the following pages describe it
 * (cited by page title and section):
 *   [PR1192] mlx-lm pull request "Add DeepSeek-v4 (Flash/Pro)"
 *   [CARD4]  model card "mlx-community / DeepSeek-V4-Flash-4bit"
 *   [ALPHA]  model card "DeepSeek-V4-Flash-MLX-4bit"
 *   [PR1190] mlx-lm pull request "Add DeepSeek-V4 model and safetensors/tokenizer
 *            fallback handling"
 *   [SERVE]  model card "DeepSeek-V4-Flash-0731-MLX-Serve-mixed-2-3-8bit"
 *
 *   1. route    -- fp32 gate logits, sqrtsoftplus scores, per-expert bias,
 *                  top-k (or the tid2eid hash table), renormalised weights;
 *   2. permute  -- bucket the T*k (token, slot) assignments by expert;
 *   3. experts  -- per assignment, SwiGLU over group-quantised gate/up/down
 *                  projections (affine b-bit or MXFP4), plus the shared expert;
 *   4. combine  -- weighted sum of the k expert outputs (+ shared) per token.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array pointers are DEVICE pointers owned by the caller. The library
 *    never allocates or frees device memory; all scratch comes from the
 *    caller's workspace `ws` (size from moe_workspace_size or the per-call
 *    sizes below). Descriptor structs are host memory, read during the call.
 *  - Every call only enqueues work on `stream` and returns: no host sync, no
 *    host readback of routing. Weights and inputs must stay valid until the
 *    enqueued work completes.
 *  - Host validation happens before anything is enqueued; a negative status
 *    means nothing was launched. T == 0 returns MOE_OK with no launch.
 *  - Device-side precondition violations (a token id outside [0, vocab), a
 *    tid2eid entry or a top-k id outside [0, E)) OR a code into the sticky
 *    error word at the start of `ws`; the offending id is replaced by 0 (and
 *    a hash-routed token's weights by 0) so that every access stays in
 *    bounds. Read it with moe_device_error, clear it with moe_workspace_init.
 *  - Layouts are row-major. A quantised projection is [rows = out][cols = in]
 *    per expert, codes packed along cols (the contraction dimension).
 *  - bf16 arrays are passed as uint16_t bit patterns.
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef QSMOE_H
#define QSMOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, k > E, ...            */
  MOE_ERR_UNSUPPORTED = -2, /* a format/bits/group/shape the kernels lack      */
  MOE_ERR_ALIGNMENT = -3,   /* a pointer not 16-byte aligned                   */
  MOE_ERR_WORKSPACE = -4,   /* workspace null or smaller than required         */
  MOE_ERR_HIP = -5          /* a HIP launch or runtime call failed             */
} moe_status;

typedef enum { MOE_FMT_AFFINE = 0, MOE_FMT_MXFP4 = 1, MOE_FMT_MXFP8 = 2 } moe_format;
typedef enum { MOE_ROUTE_TOPK = 0, MOE_ROUTE_HASH = 1 } moe_route_mode;
typedef enum { MOE_OUT_BF16 = 0, MOE_OUT_F32 = 1 } moe_out_dtype;

/* Device error bits ORed into the workspace's error word. */
#define MOE_DEVERR_TOKEN_ID 1  /* token id outside [0, vocab)                  */
#define MOE_DEVERR_HASH_ID 2   /* tid2eid entry outside [0, E)                  */
#define MOE_DEVERR_EXPERT_ID 4 /* top-k id passed to moe_permute outside [0, E) */
#define MOE_DEVERR_QUANT_INPUT 8 /* moe_quantize_affine: a NaN/inf weight, or a group's
                                    scale or bias beyond fp16 (outputs unspecified) */

/*
 * One stacked quantised projection: num_experts matrices of [rows][cols].
 *
 * MOE_FMT_AFFINE ([PR1192] pre-stacked expert patch: {weight, scales, biases}
 * triplets; [SERVE]: packs byte-compatible with MLX's affine layout; bit
 * widths and groups from [CARD4] "Conversion" and the [SERVE] precision
 * table): element (e, r, c) has the unsigned code q = bits [c*b, c*b + b) of
 * row (e, r)'s LSB-first bit stream over little-endian uint32 words (a 3-bit
 * code may straddle two words), and the value
 *     w = scale[e][r][c / g] * q + bias[e][r][c / g]
 * with fp16 scale and bias.  bits in {2, 3, 4, 8}, g in {32, 64, 128}.
 *   codes  : uint32 [E][rows][cols * bits / 32]
 *   scales : fp16   [E][rows][cols / g]
 *   biases : fp16   [E][rows][cols / g]
 *
 * MOE_FMT_MXFP4 ([PR1192] mxfp4 dequantize with group_size 32, bits 4;
 * [ALPHA]: FP4 e2m1 packed two per byte; [PR1190]: e8m0 = 2^(b - 127)):
 * byte j of a row holds element 2j in its low nibble and 2j+1 in its high
 * nibble; nibble n decodes to (-1)^(n >> 3) * {0, .5, 1, 1.5, 2, 3, 4, 6}[n & 7]
 * (OCP MX e2m1), times 2^(s - 127) for the row's scale byte s of that group of
 * 32 (s = 255 is NaN).  bits = 4, g = 32.
 *   codes  : uint32 [E][rows][cols / 8]
 *   scales : uint8  [E][rows][cols / 32]
 *   biases : NULL
 *
 * MOE_FMT_MXFP8 ([PR1192] FP8-to-bf16 requantization report: E4M3 bytes
 * viewed as uint32 words with E8M0 block scales expanded to one per 32, read
 * by mx.dequantize with group_size 32, bits 8, mode "mxfp8"; [PR1190]:
 * MXFP8-quantized MoE layers, F8_E4M3 kept as uint8): byte j of a row holds
 * element j as OCP FP8 E4M3 (bit 7 sign, 4 exponent bits with bias 7, 3
 * mantissa bits; exponent 0 subnormal; S.1111.111 NaN; largest 448), times
 * 2^(s - 127) for the row's scale byte s of that group of 32.  bits = 8,
 * g = 32.
 *   codes  : uint32 [E][rows][cols / 4]
 *   scales : uint8  [E][rows][cols / 32]
 *   biases : NULL
 *
 * Requirements: cols % 32 == 0, cols % g == 0, cols <= 8192, rows >= 1;
 * codes 16-byte aligned, scales/biases 4-byte aligned.
 */
typedef struct {
  int32_t format;      /* moe_format                         */
  int32_t bits;
  int32_t group_size;
  int32_t rows;        /* output features                    */
  int32_t cols;        /* input features (contraction)       */
  int32_t num_experts;
  const uint32_t* codes;
  const void* scales;
  const void* biases;
} moe_qtensor;

/* SwiGLU expert weights: gate = w1 [I][d], up = w3 [I][d], down = w2 [d][I]
 * ([PR1192] pre-stacked rename: w1 -> gate_proj, w2 -> down_proj,
 * w3 -> up_proj). y = W2 (silu(W1 x) * (W3 x)), with the product rounded to
 * bf16 (round to nearest even) before the down projection. gate and up share
 * format, bits and group; down may differ ([SERVE] precision table: gate/up
 * 2-bit g128 with down 3-bit g128). */
typedef struct {
  moe_qtensor gate, up, down;
} moe_experts;

/*
 * Router.
 *  MOE_ROUTE_TOPK: l[t][e] = sum_i x[t][i] * weight[e][i] in fp32 ([PR1192]
 *    cross-reference table, row "MoE gate dtype"); s = sqrt(softplus(l))
 *    ([CARD4] "Architecture"), evaluated as sqrt(max(l,0) + log1p(exp(-|l|)))
 *    (the logaddexp form of [PR1192]'s review notes); key = s + bias[e]; the
 *    top_k experts by key descending, ties to the lower expert index, in that
 *    order; weights w_j = routed_scale * s_j / sum_j s_j (the bias ranks only;
 *    [ALPHA] "REAP-pruned builds": the router renormalises over the selected
 *    experts).
 *  MOE_ROUTE_HASH: ids[t][j] = tid2eid[token_ids[t]][j] in table order
 *    ([CARD4] "Architecture": deterministic tid2eid table for the first
 *    layers; [ALPHA]: tid2eid[vocab, 6]); weights as above from those experts'
 *    fp32 logits; no bias.
 *  weight : fp32 [E][hidden]; bias : fp32 [E] or NULL; tid2eid : int32
 *  [vocab][top_k] (hash mode only). 1 <= top_k <= min(E, 8), E <= 1024,
 *  hidden % 32 == 0.
 */
typedef struct {
  int32_t mode;        /* moe_route_mode */
  int32_t num_experts;
  int32_t top_k;
  int32_t hidden;
  int32_t vocab;       /* hash mode */
  const float* weight;
  const float* bias;
  const int32_t* tid2eid;
  float routed_scale;  /* 1.0f for the layers here */
} moe_router;

/* A whole layer. `shared` (nullable) is the always-on shared expert, added to
 * every token with weight 1 after the routed sum ([ALPHA] "Why mixed-4_8bit"
 * and the [SERVE] precision table name the shared experts). routed.*.num_experts
 * must equal router.num_experts; shared->*.num_experts must be 1. */
typedef struct {
  moe_router router;
  moe_experts routed;
  const moe_experts* shared;
} moe_layer;

/* Bytes of workspace moe_forward needs for every token count up to
 * max_tokens (0 on an invalid layer): never smaller for a larger max_tokens,
 * so a buffer sized once (e.g. before graph capture) serves every T <=
 * max_tokens. The same size serves every other entry point. */
size_t moe_workspace_size(const moe_layer* layer, int32_t max_tokens);

/*
 * Where moe_forward keeps its intermediates in the workspace, for inspection
 * after the call (tests, routing statistics). Byte offsets from the start of
 * `ws`; 0 marks a region the call does not write for this layer and T.
 *   ids      int32 [T][k]   routed expert ids, slot order (key descending)
 *   weights  fp32  [T][k]   combine weights
 *   logits   fp32  [T][E]   router logits (top-k routing; hash routing on the
 *                           fused path only)
 *   keys     uint64 [T][E]  ranking key of every expert: bits 63..32 are the
 *                           fp32 key s + bias mapped so that unsigned order is
 *                           numeric order (key >= 0: bits | 0x80000000; key < 0:
 *                           ~bits), bits 31..0 are 0xFFFFFFFF - e; the top-k
 *                           takes the k largest values (ties: lower index)
 *   scores   fp32  [T][E]   sqrtsoftplus scores s of every expert
 *   offsets  int32 [E+1], perm int32 [T*k]   buckets (general path only)
 *   h        bf16  [T*k][I]  silu(gate) * up rounded to bf16: bucket order
 *                           (row p belongs to assignment perm[p]) on the
 *                           general path, slot order t*k + j on the fused path
 *   h_shared bf16  [T][I_shared] (shared expert)
 *   y_slot   fp32  [T*k][d]  (general path only), y_shared fp32 [T][d] (general
 *            path, and the fused path of a single token)
 * fused = 1 when moe_forward takes the three-launch small-batch path. total =
 * the bytes moe_forward needs for exactly T tokens. Errors: INVALID_ARG (T <
 * 1, null out, invalid layer), UNSUPPORTED.
 */
typedef struct {
  size_t total;
  size_t ids, weights, logits, keys, scores, offsets, perm, h, h_shared, y_slot, y_shared;
  int32_t fused;
} moe_ws_layout;

moe_status moe_workspace_layout(const moe_layer* layer, int32_t T, moe_ws_layout* out);

/* Zero the workspace header, which holds the device error word (a small
 * kernel; capturable). */
moe_status moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/* Step 1 (the router as moe_router defines it). x_bf16 [T][hidden];
 * token_ids int32 [T] (hash mode, else may be NULL); outputs topk_ids int32
 * [T][top_k], topk_w fp32 [T][top_k]. In top-k mode ws needs 256 + A(4*T*E)
 * + A(8*T*E) + A(4*T*E) bytes, A() rounding up to a multiple of 256, and
 * holds after the call: logits fp32 [T][E] at byte 256, then the packed
 * ranking keys uint64 [T][E] and the scores fp32 [T][E] (formats as in
 * moe_ws_layout). Hash mode needs 256 bytes. */
moe_status moe_route(const moe_router* router, const uint16_t* x_bf16, const int32_t* token_ids,
                     int32_t T, int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Step 2. A stable counting sort of the T*k assignments a = t*k + j by
 * expert topk_ids[a], so that each of the stacked experts ([PR1192]: experts
 * pre-stacked as switch_mlp.{gate,up,down}_proj, one weight tensor per
 * projection over all experts) runs once over one contiguous bucket of its
 * assignments: expert_offsets int32 [E+1] (exclusive prefix sum of the
 * per-expert counts; offsets[E] = T*k), perm int32 [T*k] (assignment indices
 * bucketed by expert, ascending within a bucket). Ids outside [0, E) set
 * MOE_DEVERR_EXPERT_ID and count as expert 0. ws needs 256 bytes. */
moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                       int32_t* expert_offsets, int32_t* perm, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* Step 3. For each bucketed assignment a (token t = a / k) of expert e:
 * y_slot[a] = expert_e(x[t]) in fp32, written in assignment order a, so row
 * t*k + j is token t's j-th expert. If `shared` is non-NULL, y_shared[t] =
 * shared(x[t]) for every token (y_shared may be NULL only when shared is).
 * y_slot fp32 [T*k][hidden], y_shared fp32 [T][hidden]. ws: see
 * moe_workspace_size. */
moe_status moe_expert_ffn(const moe_experts* routed, const moe_experts* shared,
                          const uint16_t* x_bf16, int32_t T, int32_t k,
                          const int32_t* expert_offsets, const int32_t* perm, float* y_slot,
                          float* y_shared, void* ws, size_t ws_bytes, hipStream_t stream);

/* Step 4. The weighted combine: each token's output is its selected
 * experts' outputs times their router weights ([ALPHA] "REAP-pruned builds":
 * router weight x expert output, renormalised over the kept experts), plus
 * the shared expert's output ([ALPHA] "Why mixed-4_8bit"):
 * out[t] = sum_{j=0..k-1} topk_w[t][j] * y_slot[t*k + j] (j in order) +
 * y_shared[t] (if non-NULL), accumulated in fp32 with one writer per output
 * element (no atomics); stored as bf16 (round to nearest even) or fp32 per
 * out_dtype. y_slot fp32 [T*k][d], topk_w fp32 [T][k], y_shared fp32 [T][d]
 * or NULL, out [T][d]. d % 4 == 0; y_slot, y_shared 16-byte aligned, out
 * 8-byte (bf16) or 16-byte (fp32) aligned. Errors: INVALID_ARG, UNSUPPORTED
 * (d), ALIGNMENT, HIP. */
moe_status moe_combine(const float* y_slot, const float* topk_w, const float* y_shared, int32_t T,
                       int32_t k, int32_t d, int32_t out_dtype, void* out, hipStream_t stream);

/* Steps 1-4 in one call: out [T][hidden] (bf16 or fp32). token_ids is needed
 * in hash mode only. ws >= moe_workspace_size(layer, T). */
moe_status moe_forward(const moe_layer* layer, const uint16_t* x_bf16, const int32_t* token_ids,
                       int32_t T, int32_t out_dtype, void* out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same launches and results as moe_forward, with the workspace taken from a
 * library-owned device array of 64 MiB instead of a caller buffer. Each GPU
 * the library runs on holds its own copy of the array until the process ends;
 * its address is resolved on the first call on each device. The caller still
 * passes inputs and outputs (same rules as moe_forward). Every call on a GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialised by the caller. The
 * device error word is cleared at the start of each call and is not reported
 * (out-of-range ids are still clamped in bounds). Allocates nothing, makes no
 * hipMalloc/hipFree and no host synchronisation. Errors: as moe_forward, and
 * MOE_ERR_WORKSPACE when moe_workspace_layout(layer, T).total exceeds the
 * 64 MiB (e.g. T = 512 at hidden 4096, intermediate 2048, top-6 fits; the
 * 4096-token prefill does not), before anything is launched.
 */
moe_status moe_forward_noalloc(const moe_layer* layer, const uint16_t* x_bf16, const int32_t* token_ids,
                               int32_t T, int32_t out_dtype, void* out, hipStream_t stream);

/* Test and inspection helpers (not on the hot path). */

/* Router logits only: logits fp32 [T][E] (top-k mode's first kernel). */
moe_status moe_router_logits(const moe_router* router, const uint16_t* x_bf16, int32_t T,
                             float* logits, hipStream_t stream);

/* moe_forward with timing probes: kernel i is launched with the event pair
 * events[2i] (start) and events[2i+1] (stop), which the dispatch itself
 * timestamps when the kernel begins and ends, so their elapsed time is the
 * kernel's execution time alone. Its name (a static string) goes to names[i]
 * and the number of kernels to *n_kernels. n_events must be at least twice
 * the number of kernels (at most 16 are launched, so 32 always suffice);
 * otherwise MOE_ERR_INVALID_ARG after the step has run. The caller creates
 * the events (timing enabled). Same results as moe_forward. */
moe_status moe_forward_probed(const moe_layer* layer, const uint16_t* x_bf16, const int32_t* token_ids,
                              int32_t T, int32_t out_dtype, void* out, void* ws, size_t ws_bytes,
                              hipStream_t stream, hipEvent_t* events, int32_t n_events, const char** names,
                              int32_t* n_kernels);

/* Measurement kernels (not part of the layer): the scale for HBM byte
 * counters and the achievable rates beside the nominal peaks.
 * moe_probe_stream: mode 0 reads every byte of buf [bytes] once (16 bytes per
 * lane, consecutive lanes on consecutive pieces: bytes of traffic); mode 1
 * reads the first 32 bytes of every 128-byte line (bytes / 4 requested);
 * mode 2 writes every byte once (bytes written). Modes 0 and 1 run 2048
 * workgroups; workgroup i stores the XOR of the words it read into sink[i]
 * (device uint32 [2048], overwritten), so the XOR of the 2048 words is that
 * of every word read. bytes > 0 and a multiple of 128; buf 16-byte aligned.
 * Errors: INVALID_ARG, ALIGNMENT, HIP. */
moe_status moe_probe_stream(void* buf, size_t bytes, int32_t mode, uint32_t* sink, hipStream_t stream);

/* moe_probe_mfma: `workgroups` workgroups of 4 waves, each wave `iters` rounds
 * of 8 independent V_MFMA_F32_32X32X16_BF16 (2 * 32 * 32 * 16 flops each), no
 * memory traffic. out: device uint64 [5], out[4] zeroed by the caller; wave 0
 * of workgroup 0 writes its shader-clock counter (s_memtime) before and after
 * its loop to out[0], out[1] and the 100 MHz wall clock to out[2], out[3]:
 * the sustained shader clock is (out[1] - out[0]) / ((out[3] - out[2]) / 1e8).
 * Errors: INVALID_ARG, ALIGNMENT, HIP. */
moe_status moe_probe_mfma(int32_t workgroups, int32_t iters, uint64_t* out, hipStream_t stream);

/* Synchronises `stream`, then copies the workspace error word to *code_out. */
moe_status moe_device_error(const void* ws, int32_t* code_out, hipStream_t stream);

/*
 * Plain min/max affine quantisation of bf16 weights: the conversion step
 * before the layer ([CARD4] "Conversion": mlx_lm.convert -q --q-bits b
 * --q-group-size g; [SERVE] contrasts its calibrated search with plain
 * min/max). Produces a MOE_FMT_AFFINE projection for one matrix (call per
 * expert, or once on E stacked matrices as rows = E * rows). Per group of g
 * inputs of a row, in fp32 with IEEE rounding (the pages give the recipe,
 * not its arithmetic; this is the reading taken):
 *     scale = fp16_rne((max - min) / (2^b - 1)),  bias = fp16_rne(min),
 *     q = clamp(rint((w - bias) / scale), 0, 2^b - 1), q = 0 if scale == 0.
 *   w_bf16 : device bf16 [rows][cols], 16-byte aligned
 *   codes  : device uint32 [rows][cols * bits / 32], 16-byte aligned (written)
 *   scales, biases : device fp16 [rows][cols / g], 2-byte aligned (written)
 *   err    : device int32 or NULL; MOE_DEVERR_QUANT_INPUT is ORed in for a
 *            NaN/inf weight or a group whose scale or bias overflows fp16.
 * bits in {2, 3, 4, 8}, g in {32, 64, 128}, cols % g == 0, rows >= 0.
 * Asynchronous on `stream`; allocates nothing. Errors: INVALID_ARG (null or
 * negative), UNSUPPORTED (bits, g, cols), ALIGNMENT, HIP.
 */
moe_status moe_quantize_affine(const uint16_t* w_bf16, int64_t rows, int32_t cols, int32_t bits, int32_t group_size,
                               uint32_t* codes, uint16_t* scales, uint16_t* biases, int32_t* err,
                               hipStream_t stream);

/*
 * mHC mix matrices (an op beside the MoE layer): [CARD4] "Architecture": the
 * residual stream is hc_mult = 4 parallel copies recombined by a
 * doubly-stochastic, Sinkhorn-normalised mix matrix; [PR1192] review notes:
 * unfused, a softmax followed by iterations of a sum and a division (~40
 * launches per call). For each of T tokens: m = softmax over each row of the
 * n x n logits, then `iters` rounds of dividing each column by its sum + eps
 * and then each row by its sum + eps (the pages give neither the round count
 * nor eps; 10 rounds and eps = 0 make the pages' ~40 unfused launches). fp32,
 * one launch, allocates nothing.
 *   logits : device fp32 [T][n][n]
 *   out    : device fp32 [T][n][n] (may be logits itself)
 * n in {2, 4, 8}; T >= 0; iters >= 0; eps >= 0 and finite. Rows whose
 * softmax leaves a column all zero (logit spreads beyond ~80 in fp32) give
 * NaN when eps = 0. Errors: INVALID_ARG, UNSUPPORTED (n), ALIGNMENT (4-byte),
 * HIP.
 */
moe_status moe_mhc_sinkhorn(const float* logits, int64_t T, int32_t n, int32_t iters, float eps, float* out,
                            hipStream_t stream);

const char* moe_status_string(moe_status status);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSMOE_H */
