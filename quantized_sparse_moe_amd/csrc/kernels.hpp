// Internal launch interface between the C ABI (host.hip) and the kernel
// translation units. Everything here is already validated by the caller.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsmoe {

// Kernel launch used by every launcher. When moe_forward_probed is active on
// this thread, the launch takes the next pair of timing events, which the
// dispatch itself timestamps at kernel start and end (no launch gap inside).
bool probe_events(hipEvent_t* start, hipEvent_t* stop);

#define QSMOE_LAUNCH(KERNEL, GRID, BLOCK, LDS, STREAM, ...)                                    \
  do {                                                                                         \
    hipEvent_t qsmoe_ev0_, qsmoe_ev1_;                                                         \
    if (::qsmoe::probe_events(&qsmoe_ev0_, &qsmoe_ev1_))                                       \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, STREAM, qsmoe_ev0_, qsmoe_ev1_, 0,       \
                            __VA_ARGS__);                                                      \
    else                                                                                       \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, STREAM, __VA_ARGS__);                       \
  } while (0)

// One stacked quantised projection as the kernels see it.
struct QMat {
  const uint32_t* codes;  // [n][rows][row_words]
  const void* scales;     // fp16 (affine) or uint8 e8m0 (mxfp4), [n][rows][row_groups]
  const uint16_t* biases; // fp16 (affine) or null
  int32_t fmt;            // 0 affine, 1 mxfp4
  int32_t bits;
  int32_t group;
  int32_t rows;
  int32_t cols;
  int32_t row_words;      // cols * bits / 32
  int32_t row_groups;     // cols / group
  int32_t gshift;         // log2(group / 32)
};

// Router ---------------------------------------------------------------------
hipError_t launch_router_logits(const uint16_t* x, const float* wr, int T, int E, int d, float* logits,
                                hipStream_t s);
// keys / scores (nullable): every expert's packed ranking key and score, as
// the small-batch path keeps them.
hipError_t launch_router_topk(const float* logits, const float* bias, int T, int E, int k, float routed_scale,
                              int32_t* ids, float* w, uint64_t* keys, float* scores, hipStream_t s);
hipError_t launch_router_hash(const uint16_t* x, const float* wr, const int32_t* token_ids,
                              const int32_t* tid2eid, int T, int E, int k, int d, int vocab, float routed_scale,
                              int32_t* ids, float* w, int32_t* err, hipStream_t s);

// Bucketing ------------------------------------------------------------------
hipError_t launch_permute(const int32_t* ids, int n, int E, int32_t* offsets, int32_t* perm, int32_t* err,
                          hipStream_t s);

// Experts (GEMV path: few tokens per expert) ---------------------------------
// Routed mode: expert_offsets/perm given, n_buckets = min(T*k, E).
// Shared mode: one expert, bucket b covers tokens [b*NT, b*NT + NT).
struct GateUpArgs {
  QMat gate, up;           // rows = I, cols = d
  const uint16_t* x;       // bf16 [T][d]
  int32_t T, k, E;
  const int32_t* offsets;  // routed only
  const int32_t* perm;     // routed only
  int32_t shared;
  uint16_t* h;             // bf16 [T*k][I] in bucketed order (routed) or [T][I] (shared)
  int32_t ksplit = 1;      // MFMA path only: > 1 writes fp32 partials to part instead of h
  float* part = nullptr;
};
hipError_t launch_gateup(const GateUpArgs& a, hipStream_t s);

struct DownArgs {
  QMat down;               // rows = d, cols = I
  const uint16_t* h;       // bf16, as written by launch_gateup
  int32_t T, k, E;
  const int32_t* offsets;
  const int32_t* perm;
  int32_t shared;
  float* y;                // fp32 [T*k][d] in assignment order (routed) or [T][d] (shared)
  int32_t ksplit = 1;      // MFMA path only: > 1 writes fp32 partials to part instead of y
  float* part = nullptr;
};
hipError_t launch_down(const DownArgs& a, hipStream_t s);

// Experts (MFMA grouped GEMM path: many tokens per expert, MXFP4) ------------
bool mfma_supported(const QMat& m, bool gateup, int64_t T, int k);
// K slices for the shared expert's projection at T tokens (1: no split), and
// the finishers of a split: h = bf16(silu(sum g) * sum u), y = sum of slices.
int mfma_shared_ksplit(const QMat& m, bool gateup, int T);
hipError_t launch_swiglu_parts(const float* part, int ks, int n, int I, uint16_t* h, hipStream_t s);
hipError_t launch_sum_parts(const float* part, int ks, int64_t count, float* y, hipStream_t s);
hipError_t launch_mfma_gateup(const GateUpArgs& a, hipStream_t s);
hipError_t launch_mfma_down(const DownArgs& a, hipStream_t s);

// Fused small-batch path (T <= 4 tokens, top-k routing) ------------------------
struct DecodeArgs {
  const uint16_t* x;       // bf16 [T][d]
  int32_t T, d, E, k;
  float routed_scale;
  const float* wr;         // router weight fp32 [E][d]
  const float* bias;       // fp32 [E] or null
  float* logits;           // workspace fp32 [T][E]
  uint64_t* keys;          // workspace [T][E] ranking keys (score + bias, ~index)
  float* scores;           // workspace fp32 [T][E] sqrtsoftplus scores
  QMat gate, up, down;     // routed experts
  uint16_t* h;             // workspace bf16 [T*k][I] (slot order)
  int32_t has_shared;
  QMat sgate, sup, sdown;  // shared expert (affine 8-bit) when has_shared
  uint16_t* h_sh;          // workspace bf16 [T][I_shared]
  void* out;               // bf16 or fp32 [T][d]
  int32_t out_f32;
  int32_t n_logit_blocks;  // workgroups of launch 1 that compute logits (set by its launcher)
  int32_t* ids;            // workspace int32 [T][k], written by launch 2
  float* w;                // workspace fp32 [T][k], written by launch 2
  int32_t hash;            // tid2eid routing: ids from the table, weights from the launch-1 scores
  const int32_t* token_ids;  // [T] (hash)
  const int32_t* tid2eid;    // [vocab][k] (hash)
  int32_t vocab;
  int32_t* err;            // workspace error word
  float* y_sh;             // workspace fp32 [T][d]: the shared expert's output (single token)
};
bool decode_path_supported(const DecodeArgs& a);
hipError_t launch_dec_router(const DecodeArgs& a, hipStream_t s);
hipError_t launch_dec_gateup(const DecodeArgs& a, hipStream_t s);
hipError_t launch_dec_down_combine(const DecodeArgs& a, hipStream_t s);
// Launch 2 computes the shared expert's down projection into y_sh (single token).
bool dec_shared_in_gateup(const DecodeArgs& a);

// Combine --------------------------------------------------------------------
hipError_t launch_combine(const float* y_slot, const float* w, const float* y_shared, int T, int k, int d,
                          int out_f32, void* out, hipStream_t s);

// Affine quantiser (conversion step before the layer) ------------------------
hipError_t launch_quantize_affine(const uint16_t* w, int64_t rows, int cols, int bits, int group, uint32_t* codes,
                                  uint16_t* scales, uint16_t* biases, int32_t* err, hipStream_t s);

// mHC Sinkhorn mix matrices -------------------------------------------------
hipError_t launch_mhc_sinkhorn(const float* logits, int64_t T, int n, int iters, float eps, float* out,
                               hipStream_t s);

// Measurement kernels -----------------------------------------------------------
// mode 0: read every byte of buf once (16 bytes per lane); 1: read the first
// 32 bytes of every 128-byte line; 2: write every byte once.
hipError_t launch_probe_stream(const void* buf, size_t bytes, int mode, uint32_t* sink, hipStream_t s);
hipError_t launch_probe_mfma(int workgroups, int iters, uint64_t* out, hipStream_t s);

// Workspace ------------------------------------------------------------------
hipError_t launch_fill_i32(int32_t* p, int32_t v, int n, hipStream_t s);

// Does a GEMV kernel exist for this projection shape/format?
bool gemv_supported(const QMat& m);

}  // namespace qsmoe
