// Expert SwiGLU as an MFMA grouped GEMM, for buckets with many tokens
// (prefill). Same layer as the GEMV path (stacked gate/up/down of mlx-lm PR
// "Add DeepSeek-v4 (Flash/Pro)"; MXFP4 = e2m1 nibbles with one e8m0 exponent
// per 32 inputs, the native expert format named on "DeepSeek-V4-Flash-MLX-4bit",
// which "DeepSeek-V4-Flash-0731-MLX-Serve-mixed-2-3-8bit" notes is exact in bf16).
//
// Tiles. A workgroup of 4 waves owns 128 bucketed tokens of one expert and
// 64 output rows of gate and the same 64 rows of up (so the SwiGLU epilogue
// has g and u in the same lane), or 128 output rows of down. Each wave takes
// all 128 tokens and its own 32 columns (16 rows of gate + 16 of up, or 32
// rows of down): 16 accumulator tiles of V_MFMA_F32_16X16X32_BF16. Every
// weight fragment a wave converts to bf16 then feeds up to 8 MFMAs, and no
// two waves convert the same weights; the conversion, not the MFMA, is what
// bounds a layout in which fragments are reused less.
//
// K is consumed 128 at a time. The activations of the tile (gathered through
// perm for gate/up; contiguous bucketed h rows for down) are staged in LDS,
// double-buffered, with a padded row stride so the 16 lanes reading one
// fragment hit distinct banks. Weights go straight from HBM into registers:
// for each 16-row block, lane l loads 16 bytes (32 e2m1 codes) of row l % 16
// and the one e8m0 byte of that 32-group, one K step ahead of use; the codes
// become exact bf16 with v_cvt_scalef32_pk_bf16_fp4 (the scale applied in the
// conversion). Within a K step the 128 inputs are assigned to MFMA passes so
// that lane group g = l / 16 always holds inputs 32 g .. 32 g + 31: pass s
// uses inputs 32 g + 8 s .. + 7, for A and B alike (a sum does not care which
// pass adds which input).
//
// Work split. Tiles are (expert m-tile, n-tile) pairs; the number of
// m-tiles depends on the routing, so the grid is an upper bound and each
// workgroup derives the real count from expert_offsets (staged in LDS).
// Pairs are dealt to the 8 XCDs in contiguous runs (blockIdx % 8 picks the
// XCD), so the workgroups sharing an m-tile's activations and an expert's
// weights run on the same L2. M-blocks of 16 past the bucket's end skip their
// MFMAs.
#include <algorithm>
#include <type_traits>

#include "ffn_core.hpp"

namespace qsmoe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;  // plain 16-byte register quad

constexpr int kMT = 128;                 // tokens per workgroup tile
constexpr int kKT = 128;                 // inputs per K step
constexpr int kALdsStride = kKT + 8;     // bf16 elements per LDS row (272 bytes)
constexpr int kRB = 2;                   // 16-column blocks per wave
constexpr int kMB = kMT / 16;            // 16-token blocks per wave

struct MfmaArgs {
  QMat m0, m1;             // gate, up (GATEUP) or down
  const uint16_t* x;       // gate/up: activations [T][cols]; down: h [T*k][cols] (bucketed order)
  int32_t T, k, E;
  const int32_t* offsets;
  const int32_t* perm;
  uint16_t* h;             // gate/up output [T*k][I]
  float* y;                // down output [T*k][d] (assignment order)
};

__device__ __forceinline__ bf16x8_t fp4_to_bf16x8(uint32_t word, float scale) {
  uint32_t r[4];
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3));
  return __builtin_bit_cast(bf16x8_t, r);
}

template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void k_mfma_mxfp4(MfmaArgs a) {
  constexpr int NTILE = GATEUP ? 64 : 128;    // output rows per workgroup (per matrix)
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int32_t s_mt[kMaxExperts + 1];
  __shared__ int32_t s_src[kMT];
  __shared__ __attribute__((aligned(16))) uint16_t s_a[2][kMT][kALdsStride];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int wn = wave;
  const int n = a.T * a.k;
  const QMat& q0 = a.m0;
  const int rows = q0.rows, cols = q0.cols;

  // m-tiles per expert (exclusive scan of ceil(count / kMT))
  for (int i = tid; i <= a.E; i += 256) s_off[i] = min(max(a.offsets[i], 0), n);
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int e0 = 0; e0 < a.E; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < a.E ? (max(s_off[e + 1] - s_off[e], 0) + kMT - 1) / kMT : 0;
      int incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      if (e < a.E) s_mt[e] = carry + incl - c;
      carry += __shfl(incl, 63);
    }
    if (lane == 0) s_mt[a.E] = carry;
  }
  __syncthreads();
  const int n_ntiles = rows / NTILE;
  const int64_t pairs = static_cast<int64_t>(s_mt[a.E]) * n_ntiles;
  const int64_t per_xcd = (pairs + 7) / 8;
  const int64_t local = blockIdx.x / 8;
  if (local >= per_xcd) return;
  const int64_t pair = (blockIdx.x % 8) * per_xcd + local;
  if (pair >= pairs) return;
  const int mtile = static_cast<int>(pair / n_ntiles), ntile = static_cast<int>(pair % n_ntiles);

  // expert of this m-tile
  int e = 0;
  for (int e0 = 0; e0 < a.E; e0 += 64) {
    const int ee = e0 + lane;
    const bool hit = ee < a.E && s_mt[ee] <= mtile && mtile < s_mt[ee + 1];
    const uint64_t m = __ballot(hit);
    if (m) {
      e = e0 + __ffsll(static_cast<unsigned long long>(m)) - 1;
      break;
    }
  }
  const int p0 = s_off[e] + (mtile - s_mt[e]) * kMT;
  const int count = min(kMT, s_off[e + 1] - p0);
  if (tid < kMT) {
    const int p = p0 + min(tid, count - 1);
    s_src[tid] = GATEUP ? min(max(a.perm[p] / a.k, 0), a.T - 1) : p;
  }
  __syncthreads();

  // A staging: in round i (0..7) thread t copies 16 bytes, chunk t % 16 of
  // token row t / 16 + 16 i, so 16 consecutive lanes read one row's 256
  // contiguous bytes of the K step.
  const int a_chunk = tid & 15, a_row0 = tid >> 4;
  uint32_t a_off[8];  // element offsets of this thread's 8 rows (+ its chunk)
#pragma unroll
  for (int i = 0; i < 8; ++i) a_off[i] = static_cast<uint32_t>(s_src[a_row0 + 16 * i]) * cols + a_chunk * 8;
  auto load_a = [&](u32x4_t (&ar)[8], int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ar[i] = *reinterpret_cast<const u32x4_t*>(a.x + a_off[i] + k0);
  };
  auto store_a = [&](const u32x4_t (&ar)[8], int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t*>(&s_a[buf][a_row0 + 16 * i][a_chunk * 8]) = ar[i];
  };

  // B: this wave's 2 column blocks (gate/up: 16 rows of gate + the same 16 of up)
  const QMat w0 = expert_slice(a.m0, e);
  const QMat w1 = expert_slice(a.m1, e);
  const int g = lane >> 4, r16 = lane & 15;
  const int row0 = ntile * NTILE + wn * (GATEUP ? 16 : 32) + r16;  // row of block 0 for this lane
  const size_t rw = static_cast<size_t>(w0.row_words), rg = static_cast<size_t>(w0.row_groups);
  // byte addresses of this lane's rows: block rb is row0 + 16 rb (down) or
  // row0 of gate (rb = 0) / up (rb = 1)
  const uint8_t* c0 = reinterpret_cast<const uint8_t*>(w0.codes) + (static_cast<size_t>(row0) * rw + 4 * g) * 4;
  const uint8_t* c1 = reinterpret_cast<const uint8_t*>(w1.codes) + (static_cast<size_t>(row0) * rw + 4 * g) * 4;
  const uint8_t* e0p = static_cast<const uint8_t*>(w0.scales) + static_cast<size_t>(row0) * rg + g;
  const uint8_t* e1p = static_cast<const uint8_t*>(w1.scales) + static_cast<size_t>(row0) * rg + g;
  const size_t cstep = 16 * rw * 4, estep = 16 * rg;
  auto load_b = [&](u32x4_t (&bv)[kRB], uint32_t (&sv)[kRB], int k0) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const bool second = GATEUP && rb == 1;
      const int blk = GATEUP ? 0 : rb;
      const uint8_t* cp = (second ? c1 : c0) + blk * cstep + k0 / 2;
      const uint8_t* ep = (second ? e1p : e0p) + blk * estep + k0 / 32;
      bv[rb] = *reinterpret_cast<const u32x4_t*>(cp);
      sv[rb] = *ep;
    }
  };

  f32x4_t acc[kMB][kRB];
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < kRB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // the K loop, specialised on the number of 16-token blocks that hold
  // tokens, so that no MFMA sits behind a branch
  const int valid_mb = min(kMB, (count + 15) / 16);
  const int nsteps = cols / kKT;
  // Software pipeline over K steps: during step ks the activations of step
  // ks + 2 and the weights of step ks + 1 are in flight, the activations of
  // step ks + 1 (already in registers) go to the other LDS buffer at the end.
  // Register sets alternate between even and odd steps (loop unrolled by 2).
  u32x4_t a_reg0[8], a_reg1[8];
  u32x4_t b_reg0[kRB], b_reg1[kRB];
  uint32_t e_reg0[kRB], e_reg1[kRB];
  auto kloop = [&](auto nmb_tag) {
    constexpr int NMB = decltype(nmb_tag)::value;
    auto step = [&](int ks, u32x4_t (&a_ld)[8], const u32x4_t (&a_st)[8], const u32x4_t (&b_use)[kRB],
                    const uint32_t (&e_use)[kRB], u32x4_t (&b_ld)[kRB], uint32_t (&e_ld)[kRB]) {
      const int buf = ks & 1;
      load_a(a_ld, min(ks + 2, nsteps - 1) * kKT);
      load_b(b_ld, e_ld, min(ks + 1, nsteps - 1) * kKT);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8_t af[NMB > 0 ? NMB : 1];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          af[mb] = *reinterpret_cast<const bf16x8_t*>(&s_a[buf][mb * 16 + r16][32 * g + 8 * s]);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          if constexpr (NMB > 0) {
            const bf16x8_t bf = fp4_to_bf16x8(b_use[rb][s], e8m0_to_f32(e_use[rb]));
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
              acc[mb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], bf, acc[mb][rb], 0, 0, 0);
          }
        }
      }
      if (ks + 1 < nsteps) store_a(a_st, buf ^ 1);
      __syncthreads();
    };
    load_a(a_reg0, 0);
    load_b(b_reg0, e_reg0, 0);
    store_a(a_reg0, 0);
    load_a(a_reg0, min(1, nsteps - 1) * kKT);
    __syncthreads();
    for (int ks = 0; ks < nsteps; ks += 2) {
      step(ks, a_reg1, a_reg0, b_reg0, e_reg0, b_reg1, e_reg1);
      if (ks + 1 < nsteps) step(ks + 1, a_reg0, a_reg1, b_reg1, e_reg1, b_reg0, e_reg0);
    }
  };
  switch (valid_mb) {
    case 8: kloop(std::integral_constant<int, 8>{}); break;
    case 7: kloop(std::integral_constant<int, 7>{}); break;
    case 6: kloop(std::integral_constant<int, 6>{}); break;
    case 5: kloop(std::integral_constant<int, 5>{}); break;
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    default: kloop(std::integral_constant<int, 1>{}); break;
  }

  // epilogue: lane holds rows 4 * g + i (tokens) of column r16 (output row)
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    if (mb >= valid_mb) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = mb * 16 + 4 * g + i;
      if (tl >= count) continue;
      if constexpr (GATEUP) {
        a.h[static_cast<size_t>(p0 + tl) * rows + row0] =
            static_cast<uint16_t>(f32_to_bf16_rne(silu(acc[mb][0][i]) * acc[mb][1][i]));
      } else {
        const int slot = min(max(a.perm[p0 + tl], 0), n - 1);
        float* yrow = a.y + static_cast<size_t>(slot) * rows + row0;
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) yrow[rb * 16] = acc[mb][rb][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
bool mfma_supported(const QMat& gate, const QMat& down, int64_t T, int k) {
  // activation rows are addressed with 32-bit element offsets
  if (T * k * std::max(gate.cols, down.cols) >= (int64_t{1} << 31)) return false;
  return gate.fmt == 1 && down.fmt == 1 && gate.cols % kKT == 0 && down.cols % kKT == 0 && gate.rows % 64 == 0 &&
         down.rows % 128 == 0;
}

static unsigned mfma_grid(int T, int k, int E, int rows, int ntile) {
  const int64_t tk = static_cast<int64_t>(T) * k;
  const int64_t mtiles = (tk + kMT - 1) / kMT + std::min<int64_t>(tk, E);
  const int64_t pairs = mtiles * (rows / ntile);
  return static_cast<unsigned>(((pairs + 7) / 8) * 8);
}

hipError_t launch_mfma_gateup(const GateUpArgs& g, hipStream_t s) {
  MfmaArgs a{g.gate, g.up, g.x, g.T, g.k, g.E, g.offsets, g.perm, g.h, nullptr};
  hipLaunchKernelGGL((k_mfma_mxfp4<true>), dim3(mfma_grid(g.T, g.k, g.E, g.gate.rows, 64)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mfma_down(const DownArgs& d, hipStream_t s) {
  MfmaArgs a{d.down, d.down, d.h, d.T, d.k, d.E, d.offsets, d.perm, nullptr, d.y};
  hipLaunchKernelGGL((k_mfma_mxfp4<false>), dim3(mfma_grid(d.T, d.k, d.E, d.down.rows, 128)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qsmoe
