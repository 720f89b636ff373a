// Expert SwiGLU as a quantised grouped GEMV (few tokens per expert).
//
// Projections are group-quantised, affine b-bit (w = scale * q + bias, fp16
// scale and bias per group; {weight, scales, biases} triplets of the
// pre-stacked experts in mlx-lm PR "Add DeepSeek-v4 (Flash/Pro)"; bit widths
// and groups from "mlx-community / DeepSeek-V4-Flash-4bit" (Conversion) and
// the precision table of "DeepSeek-V4-Flash-0731-MLX-Serve-mixed-2-3-8bit")
// or MXFP4 (e2m1 nibbles, one e8m0 exponent per 32 values; the same PR's
// mxfp4 dequantize, the FP4 e2m1 format of "DeepSeek-V4-Flash-MLX-4bit").
// gate = w1, up = w3, down = w2 (the PR's pre-stacked rename); the SwiGLU
// product silu(w1 x) * (w3 x) is rounded to bf16 before the down projection.
//
// Layout of the work: one launch covers every (virtual bucket, output row)
// unit of a projection, where a virtual bucket is up to NT bucketed positions
// of one expert (or NT tokens of the shared expert). A workgroup stages the
// expert offsets in LDS and derives each expert's first virtual bucket once;
// the units are then split evenly over all waves of the grid, so routing skew
// never leaves CUs idle and the lookup, the activations and the first rows
// are fetched once per wave rather than once per small tile. Within a row,
// lane l owns the 32-code chunks c = l + 64 m (m < CPL), so one 16-byte load
// per lane per chunk covers a contiguous 1 KB of a 4-bit row per wave, and the
// NT tokens' activations stay in registers for all rows, packed as bf16 pairs
// in the order the codes are unpacked. Codes are turned into bf16
// pairs with integer ops only (for b <= 4 the exact value off + q with
// off = 2^b, one shift and one and-or per pair), dotted with v_dot2_f32_bf16
// into fp32, and the group's scale and bias are applied once per 32-code chunk:
//   sum_i x_i (s q_i + b) = s * sum_i x_i (q_i + off) + (b - off * s) * sum_i x_i.
// MXFP4 nibbles become exact bf16 with v_cvt_scalef32_pk_bf16_fp4 (scale 1),
// and the chunk sum is multiplied by the e8m0 power of two in fp32.
#include <algorithm>

#include "ffn_core.hpp"

namespace qsmoe {

// ---------------------------------------------------------------------------
static int chunks_per_lane(int cols) { return cols <= 2048 ? 1 : (cols <= 4096 ? 2 : 4); }

bool gemv_supported(const QMat& m) {
  if (m.cols % 32 != 0 || m.cols > 8192 || m.rows < 1) return false;
  if (m.fmt == 0) return m.bits == 2 || m.bits == 3 || m.bits == 4 || m.bits == 8;
  if (m.fmt == 2) return m.bits == 8 && m.group == 32;
  return m.fmt == 1 && m.bits == 4 && m.group == 32;
}

// Tokens handled per pass over the rows, from the mean bucket size (the
// activations of NT tokens x CPL chunks are held in registers).
constexpr int kGemvMaxTokenChunks = 8;  // NT * CPL activation chunks held in registers
static int tokens_per_pass(int T, int k, int E, int cpl, int shared) {
  const int buckets = shared ? 1 : (T * k < E ? T * k : E);
  const int per = shared ? T : (T * k + buckets - 1) / buckets;
  int nt = per <= 1 ? 1 : (per <= 2 ? 2 : 4);
  while (nt * cpl > kGemvMaxTokenChunks) nt >>= 1;
  return nt;
}

#define QSMOE_FMT_SWITCH(FMT_, BITS_, ...)                   \
  if ((FMT_) == 0 && (BITS_) == 4) {                         \
    constexpr int F = 0, B = 4;                              \
    __VA_ARGS__                                              \
  } else if ((FMT_) == 0 && (BITS_) == 2) {                  \
    constexpr int F = 0, B = 2;                              \
    __VA_ARGS__                                              \
  } else if ((FMT_) == 0 && (BITS_) == 3) {                  \
    constexpr int F = 0, B = 3;                              \
    __VA_ARGS__                                              \
  } else if ((FMT_) == 0 && (BITS_) == 8) {                  \
    constexpr int F = 0, B = 8;                              \
    __VA_ARGS__                                              \
  } else if ((FMT_) == 2) {                                  \
    constexpr int F = 2, B = 8;                              \
    __VA_ARGS__                                              \
  } else {                                                   \
    constexpr int F = 1, B = 4;                              \
    __VA_ARGS__                                              \
  }

#define QSMOE_SHAPE_SWITCH(CPL_, NT_, ...)                   \
  if ((CPL_) == 1 && (NT_) == 1) {                           \
    constexpr int CP = 1, NTK = 1;                           \
    __VA_ARGS__                                              \
  } else if ((CPL_) == 1 && (NT_) == 2) {                    \
    constexpr int CP = 1, NTK = 2;                           \
    __VA_ARGS__                                              \
  } else if ((CPL_) == 1) {                                  \
    constexpr int CP = 1, NTK = 4;                           \
    __VA_ARGS__                                              \
  } else if ((CPL_) == 2 && (NT_) == 1) {                    \
    constexpr int CP = 2, NTK = 1;                           \
    __VA_ARGS__                                              \
  } else if ((CPL_) == 2 && (NT_) == 2) {                   \
    constexpr int CP = 2, NTK = 2;                           \
    __VA_ARGS__                                              \
  } else if ((CPL_) == 2) {                                  \
    constexpr int CP = 2, NTK = 4;                           \
    __VA_ARGS__                                              \
  } else {                                                   \
    constexpr int CP = 4, NTK = 1;                           \
    __VA_ARGS__                                              \
  }

// Workgroups of a streaming launch: enough waves to keep every CU busy, few
// enough that each wave streams several rows.
static unsigned stream_grid(int T, int k, int E, int nt, int rows, int shared) {
  const int64_t vb_max = shared ? (T + nt - 1) / nt : std::min<int64_t>(static_cast<int64_t>(T) * k, E) +
                                                          static_cast<int64_t>(T) * k / nt;
  const int64_t units = vb_max * rows;
  const int64_t wg = (units + 7) / 8;  // at least two rows per wave
  return static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(wg, 512)));
}

hipError_t launch_gateup(const GateUpArgs& g, hipStream_t s) {
  const int cpl = chunks_per_lane(g.gate.cols);
  const int nt = tokens_per_pass(g.T, g.k, g.E, cpl, g.shared);
  StreamArgs a{g.gate, g.up, g.x, g.T, g.k, g.E, g.offsets, g.perm, g.shared, g.h, nullptr};
  const dim3 grid(stream_grid(g.T, g.k, g.E, nt, g.gate.rows, g.shared)), block(256);
  QSMOE_FMT_SWITCH(g.gate.fmt, g.gate.bits, QSMOE_SHAPE_SWITCH(cpl, nt, {
    QSMOE_LAUNCH((k_ffn_stream<F, B, CP, NTK, true>), grid, block, 0, s, a);
  }))
  return hipGetLastError();
}

hipError_t launch_down(const DownArgs& d, hipStream_t s) {
  const int cpl = chunks_per_lane(d.down.cols);
  const int nt = tokens_per_pass(d.T, d.k, d.E, cpl, d.shared);
  StreamArgs a{d.down, d.down, d.h, d.T, d.k, d.E, d.offsets, d.perm, d.shared, nullptr, d.y};
  const dim3 grid(stream_grid(d.T, d.k, d.E, nt, d.down.rows, d.shared)), block(256);
  QSMOE_FMT_SWITCH(d.down.fmt, d.down.bits, QSMOE_SHAPE_SWITCH(cpl, nt, {
    QSMOE_LAUNCH((k_ffn_stream<F, B, CP, NTK, false>), grid, block, 0, s, a);
  }))
  return hipGetLastError();
}

}  // namespace qsmoe
