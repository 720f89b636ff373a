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

constexpr int kKT = 128;                 // inputs per K step
constexpr int kALdsStride = kKT + 8;     // bf16 elements per LDS row (272 bytes)

struct MfmaArgs {
  QMat m0, m1;             // gate, up (GATEUP) or down
  const uint16_t* x;       // gate/up: activations [T][cols]; down: h [T*k][cols] (bucketed order)
  int32_t T, k, E;
  const int32_t* offsets;  // routed only
  const int32_t* perm;     // routed only
  int32_t shared;          // one expert over all T tokens in token order (k = E = 1)
  uint16_t* h;             // gate/up output [T*k][I]
  float* y;                // down output [T*k][d] (assignment order)
  int32_t ksplit;          // K slices (affine only); > 1: fp32 partial sums to part
  float* part;             // [ksplit][T*k][2 I] (gate/up: g then u) or [ksplit][T*k][d]
};

typedef __attribute__((address_space(1))) void global_void_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// direct global -> LDS load of 16 bytes per lane (gfx950's
// GLOBAL_LOAD_LDS_DWORDX4): lane l's bytes land at lds + 16 l; lds must be
// the same for the whole wave. Counted by vmcnt, like any vector load.
__device__ __forceinline__ void load_lds16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((global_void_t*)(src), (lds_void_t*)(lds), 16, 0, 0);
}

// s_waitcnt vmcnt(0), leaving the LDS/scalar and export counters alone
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
__device__ __forceinline__ void vmem_wait_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }
// Workgroup barrier that leaves the wave's N newest vector loads in flight
// (N < 16): s_waitcnt vmcnt(N) lgkmcnt(0), then s_barrier between
// compiler-only fences (they keep LDS accesses from moving across; a release
// fence would make the wave wait for every load in flight, since the compiler
// cannot tell direct-to-LDS loads from register loads). Loads complete in
// order, so everything older than the N newest has landed.
template <int N>
__device__ __forceinline__ void barrier_keep() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ bf16x8_t fp4_to_bf16x8(uint32_t word, float scale) {
  uint32_t r[4];
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3));
  return __builtin_bit_cast(bf16x8_t, r);
}

// Which (expert m-tile, n-tile) pair this workgroup computes. Tiles are MT
// bucketed tokens of one expert; an expert with c tokens has ceil(c / MT)
// m-tiles, counted from expert_offsets with a wave scan (staged in LDS).
// Pairs are dealt to the 8 XCDs in contiguous runs (blockIdx % 8 picks the
// XCD), so the workgroups sharing an m-tile's activations and an expert's
// weights run on the same L2. Returns false (for the whole workgroup) when
// the grid's upper bound left this workgroup without a pair.
struct Tile {
  int e, p0, count, ntile, kslice;
};

template <int MT>
__device__ bool tile_of_block(const MfmaArgs& a, int n_ntiles, int32_t* s_off, int32_t* s_mt, Tile& t) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int n = a.T * a.k;
  for (int i = tid; i <= a.E; i += blockDim.x) s_off[i] = a.shared ? (i == 0 ? 0 : n) : min(max(a.offsets[i], 0), n);
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int e0 = 0; e0 < a.E; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < a.E ? (max(s_off[e + 1] - s_off[e], 0) + MT - 1) / MT : 0;
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
  const int ks = max(a.ksplit, 1);
  const int64_t pairs = static_cast<int64_t>(s_mt[a.E]) * n_ntiles * ks;
  const int64_t per_xcd = (pairs + 7) / 8;
  const int64_t local = blockIdx.x / 8;
  if (local >= per_xcd) return false;
  const int64_t pair = (blockIdx.x % 8) * per_xcd + local;
  if (pair >= pairs) return false;
  int mtile;
  if (ks == 1) {
    mtile = static_cast<int>(pair / n_ntiles);
    t.ntile = static_cast<int>(pair % n_ntiles);
    t.kslice = 0;
  } else {
    // K-split: the m-tiles of one (n-tile, K slice) weight block are adjacent
    const int64_t mt = s_mt[a.E];
    mtile = static_cast<int>(pair % mt);
    const int64_t wb = pair / mt;
    t.ntile = static_cast<int>(wb / ks);
    t.kslice = static_cast<int>(wb % ks);
  }
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
  t.e = e;
  t.p0 = s_off[e] + (mtile - s_mt[e]) * MT;
  t.count = min(MT, s_off[e + 1] - t.p0);
  return true;
}

template <bool GATEUP, int MT, int RB>
__global__ __launch_bounds__(256, 2) void k_mfma_mxfp4(MfmaArgs a) {
  constexpr int HB = GATEUP ? RB / 2 : RB;    // 16-row blocks per matrix per wave
  constexpr int NTILE = 4 * HB * 16;          // output rows per workgroup (per matrix)
  constexpr int MB = MT / 16;                 // 16-token blocks per wave
  constexpr int ACH = MT * 16 / 256;          // 16-byte activation chunks per thread per K step
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int32_t s_mt[kMaxExperts + 1];
  __shared__ int32_t s_src[MT];
  __shared__ __attribute__((aligned(16))) uint16_t s_a[2][MT][kALdsStride];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int wn = wave;
  const int n = a.T * a.k;
  const int rows = a.m0.rows, cols = a.m0.cols;
  Tile t;
  if (!tile_of_block<MT>(a, rows / NTILE, s_off, s_mt, t)) return;
  const int e = t.e, p0 = t.p0, count = t.count, ntile = t.ntile;
  if (tid < MT) {
    const int p = p0 + min(tid, count - 1);
    s_src[tid] = GATEUP && !a.shared ? min(max(a.perm[p] / a.k, 0), a.T - 1) : p;
  }
  __syncthreads();

  // A staging: in round i (0..7) thread t copies 16 bytes, chunk t % 16 of
  // token row t / 16 + 16 i, so 16 consecutive lanes read one row's 256
  // contiguous bytes of the K step.
  const int a_chunk = tid & 15, a_row0 = tid >> 4;
  uint32_t a_off[ACH];  // element offsets of this thread's rows (+ its chunk)
#pragma unroll
  for (int i = 0; i < ACH; ++i) a_off[i] = static_cast<uint32_t>(s_src[a_row0 + 16 * i]) * cols + a_chunk * 8;
  auto load_a = [&](u32x4_t (&ar)[ACH], int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) ar[i] = *reinterpret_cast<const u32x4_t*>(a.x + a_off[i] + k0);
  };
  auto store_a = [&](const u32x4_t (&ar)[ACH], int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<u32x4_t*>(&s_a[buf][a_row0 + 16 * i][a_chunk * 8]) = ar[i];
  };

  // B: this wave's RB column blocks (gate/up: HB blocks of gate + the same rows of up)
  const QMat w0 = expert_slice(a.m0, e);
  const QMat w1 = expert_slice(a.m1, e);
  const int g = lane >> 4, r16 = lane & 15;
  const int row0 = ntile * NTILE + wn * HB * 16 + r16;  // row of block 0 for this lane
  const size_t rw = static_cast<size_t>(w0.row_words), rg = static_cast<size_t>(w0.row_groups);
  // byte addresses of this lane's rows: block rb is row0 + 16 (rb % HB) of
  // gate or down (rb < HB) / up (rb >= HB)
  const uint8_t* c0 = reinterpret_cast<const uint8_t*>(w0.codes) + (static_cast<size_t>(row0) * rw + 4 * g) * 4;
  const uint8_t* c1 = reinterpret_cast<const uint8_t*>(w1.codes) + (static_cast<size_t>(row0) * rw + 4 * g) * 4;
  const uint8_t* e0p = static_cast<const uint8_t*>(w0.scales) + static_cast<size_t>(row0) * rg + g;
  const uint8_t* e1p = static_cast<const uint8_t*>(w1.scales) + static_cast<size_t>(row0) * rg + g;
  const size_t cstep = 16 * rw * 4, estep = 16 * rg;
  auto load_b = [&](u32x4_t (&bv)[RB], uint32_t (&sv)[RB], int k0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bool second = GATEUP && rb >= HB;
      const int blk = rb % HB;
      const uint8_t* cp = (second ? c1 : c0) + blk * cstep + k0 / 2;
      const uint8_t* ep = (second ? e1p : e0p) + blk * estep + k0 / 32;
      bv[rb] = *reinterpret_cast<const u32x4_t*>(cp);
      sv[rb] = *ep;
    }
  };

  f32x4_t acc[MB][RB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // the K loop, specialised on the number of 16-token blocks that hold
  // tokens, so that no MFMA sits behind a branch
  const int valid_mb = min(MB, (count + 15) / 16);
  const int nsteps = cols / kKT;
  // Software pipeline over K steps: during step ks the activations of step
  // ks + 2 and the weights of step ks + 1 are in flight, the activations of
  // step ks + 1 (already in registers) go to the other LDS buffer at the end.
  // Register sets alternate between even and odd steps (loop unrolled by 2).
  u32x4_t a_reg0[ACH], a_reg1[ACH];
  u32x4_t b_reg0[RB], b_reg1[RB];
  uint32_t e_reg0[RB], e_reg1[RB];
  auto kloop = [&](auto nmb_tag) {
    constexpr int NMB = decltype(nmb_tag)::value;
    auto step = [&](int ks, u32x4_t (&a_ld)[ACH], const u32x4_t (&a_st)[ACH], const u32x4_t (&b_use)[RB],
                    const uint32_t (&e_use)[RB], u32x4_t (&b_ld)[RB], uint32_t (&e_ld)[RB]) {
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
        for (int rb = 0; rb < RB; ++rb) {
          if constexpr (NMB > 0) {
            const bf16x8_t bf = fp4_to_bf16x8(b_use[rb][s], e8m0_to_f32(e_use[rb]));
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
              acc[mb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], bf, acc[mb][rb], 0, 0, 0);
          }
        }
      }
      store_a(a_st, buf ^ 1);  // after the last step: unused, harmless
      lds_barrier();
    };
    load_a(a_reg0, 0);
    load_b(b_reg0, e_reg0, 0);
    store_a(a_reg0, 0);
    load_a(a_reg0, min(1, nsteps - 1) * kKT);
    lds_barrier();
    int ks = 0;
    for (; ks + 2 <= nsteps; ks += 2) {
      step(ks, a_reg1, a_reg0, b_reg0, e_reg0, b_reg1, e_reg1);
      step(ks + 1, a_reg0, a_reg1, b_reg1, e_reg1, b_reg0, e_reg0);
    }
    if (ks < nsteps) step(ks, a_reg1, a_reg0, b_reg0, e_reg0, b_reg1, e_reg1);
  };
  if constexpr (MB == 8) {
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
  } else {
    switch (valid_mb) {
      case 4: kloop(std::integral_constant<int, 4>{}); break;
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      default: kloop(std::integral_constant<int, 1>{}); break;
    }
  }

  // epilogue: lane holds rows 4 * g + i (tokens) of column r16 (output row)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= valid_mb) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = mb * 16 + 4 * g + i;
      if (tl >= count) continue;
      if constexpr (GATEUP) {
        uint16_t* hrow = a.h + static_cast<size_t>(p0 + tl) * rows + row0;
#pragma unroll
        for (int rb = 0; rb < HB; ++rb)
          hrow[rb * 16] = static_cast<uint16_t>(f32_to_bf16_rne(silu(acc[mb][rb][i]) * acc[mb][rb + HB][i]));
      } else {
        const int slot = a.shared ? p0 + tl : min(max(a.perm[p0 + tl], 0), n - 1);
        float* yrow = a.y + static_cast<size_t>(slot) * rows + row0;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) yrow[rb * 16] = acc[mb][rb][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MXFP4 grouped GEMM on 32 x 32 tiles (V_MFMA_F32_32X32X16_BF16), weights
// staged through LDS, two workgroups per CU.
//
// Workgroup: 128 bucketed tokens x 256 output columns: 128 rows of gate and
// the same 128 rows of up, or 256 rows of down. Its 4 waves split the
// columns; each takes all 128 tokens x 64 columns (gate/up: 32 rows of gate
// + the same 32 of up, so the SwiGLU pairs meet in one lane) as 4 x 2
// accumulator tiles of 32 x 32. Operand layouts (checked on the device): A
// lane l holds row l % 32, inputs 8 (l / 32) .. + 7 of the pass; B lane l
// holds column l % 32 and the same inputs; element i of D in lane l is row
// 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32. In a 128-input K step lane
// group g = l / 32 holds inputs 64 g .. 64 g + 63, pass p (0..7) using inputs
// 64 g + 8 p .. + 7 for A and B alike (the sum does not care which pass adds
// which input), so a lane's weights for the step are 32 contiguous bytes of
// its row with the two e8m0 exponents over them.
//
// Loads. Every operand goes from HBM straight into LDS
// (GLOBAL_LOAD_LDS_DWORDX4, 16 bytes per lane, no staging registers):
//  - activations (gathered through perm for gate/up; contiguous bucketed h
//    rows for down), double-buffered one K step ahead: a load instruction
//    covers 4 tile rows x 256 bytes; rows of 256 bytes, slot s of row r
//    holding input chunk s ^ (r % 16), so the 16 rows that 16 lanes read at
//    once hold a chunk in 16 different slots;
//  - weights: each wave loads its own 64 rows x 64 bytes of the step, 16 rows
//    x 64 contiguous bytes per instruction (a load straight into the B operand
//    layout touches 32 rows per instruction, and a 64-lane load costs about
//    in proportion to the 128-byte lines it touches: measured on this GPU,
//    34 against 20 bytes per clock per CU from L2). A row's four 16-byte
//    chunks sit at slot c ^ ((r / 4) % 4) of its 64 bytes, so the 16 rows that
//    16 lanes read at once cover all 64 banks. The rows are private to the
//    wave, so a single buffer suffices: the wave copies the step's 32 bytes
//    per lane and block into registers, then issues the next step's loads
//    into the same place;
//  - the e8m0 bytes of 4 K steps in one 16-byte load per block, 4 steps ahead.
// The LDS budget (2 x 32 KB activations + 16 KB weights, the set-up's
// offsets aliased into the weight buffer) leaves room for two workgroups per
// CU, which hide each other's barriers, set-up and epilogue. The weights
// become exact bf16 with v_cvt_scalef32_pk_bf16_fp4 (the scale applied in the
// conversion).
template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void k_mfma_mxfp4_w(MfmaArgs a) {
  typedef __attribute__((ext_vector_type(16))) float f32x16_t;
  constexpr int MT = 128;
  constexpr int NB = 2;                              // 32-column blocks per wave
  constexpr int WR = 32 * NB;                        // weight rows per wave
  constexpr int NTILE = GATEUP ? 2 * WR : 4 * WR;    // rows per matrix per workgroup
  constexpr int ACH = MT * 16 / 256;                 // 16-byte activation chunks per thread per step
  constexpr int WCH = WR * 4 / 64;                   // weight load instructions per wave per step
  constexpr int ABUF = MT * kKT * 2;                 // bytes per activation buffer
  extern __shared__ __attribute__((aligned(16))) uint8_t s_lds[];
  uint16_t* const s_a0 = reinterpret_cast<uint16_t*>(s_lds);
  uint16_t* const s_a1 = reinterpret_cast<uint16_t*>(s_lds + ABUF);
  uint8_t* const s_w = s_lds + 2 * ABUF;             // 4 waves x WR rows x 64 bytes
  // the set-up's expert offsets, m-tile starts and gather rows live in the
  // weight buffer until its first load
  int32_t* const s_off = reinterpret_cast<int32_t*>(s_w);
  int32_t* const s_mt = s_off + a.E + 1;
  int32_t* const s_src = s_off;

  const int tid = threadIdx.x, lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const int n = a.T * a.k;
  const int rows = a.m0.rows, cols = a.m0.cols;
  Tile t;
  if (!tile_of_block<MT>(a, rows / NTILE, s_off, s_mt, t)) return;
  const int e = __builtin_amdgcn_readfirstlane(t.e), p0 = __builtin_amdgcn_readfirstlane(t.p0);
  const int count = __builtin_amdgcn_readfirstlane(t.count), ntile = __builtin_amdgcn_readfirstlane(t.ntile);
  __syncthreads();  // every wave is done with s_off / s_mt
  if (tid < MT) {
    const int p = p0 + min(tid, count - 1);
    s_src[tid] = GATEUP && !a.shared ? min(max(a.perm[p] / a.k, 0), a.T - 1) : p;
  }
  __syncthreads();
  // activations: round i of wave w fills the 1 KB of tile rows 4 b .. 4 b + 3,
  // b = ACH w + i (wave w: rows 32 w .. 32 w + 31). Rows past the tile's
  // tokens repeat its last token.
  uint32_t a_off[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int row = 4 * (ACH * wave + i) + (lane >> 4), slot = lane & 15;
    a_off[i] = static_cast<uint32_t>(s_src[row]) * cols + 8 * (slot ^ (row & 15));
  }
  __syncthreads();  // s_src is read: the weight buffer is free
  auto load_a = [&](uint16_t* buf, int k) {
    const uint16_t* const base = a.x + k * kKT;
#pragma unroll
    for (int i = 0; i < ACH; ++i) load_lds16(base + a_off[i], buf + (ACH * wave + i) * 512);
  };
  // fragment reads: lane (r32, g) takes chunk 8 g + p of its row in pass p
  const int xr = r32 & 15;
  const int a_rd = r32 * kKT + 8 * ((8 * g) ^ (xr & 8));

  // weights: block b of the wave is rows wrow(b) .. + 31 of gate (b = 0) and
  // up (b = 1), or of down
  const QMat w0 = expert_slice(a.m0, e);
  const QMat w1 = expert_slice(a.m1, e);
  const size_t rb_bytes = static_cast<size_t>(w0.row_words) * 4, rg = static_cast<size_t>(w0.row_groups);
  auto wrow = [&](int b) { return GATEUP ? ntile * NTILE + 32 * wave : ntile * NTILE + WR * wave + 32 * b; };
  const uint8_t* wbase[NB];
  const uint8_t* sbase[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const QMat& m = (GATEUP && b == 1) ? w1 : w0;
    wbase[b] = reinterpret_cast<const uint8_t*>(m.codes) + static_cast<size_t>(wrow(b)) * rb_bytes;
    sbase[b] = static_cast<const uint8_t*>(m.scales) + static_cast<size_t>(wrow(b) + r32) * rg;
  }
  // weight load instruction i covers the wave's rows 16 i .. 16 i + 15
  // (block i / 2): lane l takes row 16 i + l / 4, LDS slot l % 4, global
  // chunk (l % 4) ^ ((row / 4) % 4)
  uint32_t w_off[WCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int rl = 16 * i + (lane >> 2);
    const int c = (lane & 3) ^ ((rl >> 2) & 3);
    w_off[i] = static_cast<uint32_t>((rl & 31) * rb_bytes + 16 * c);
  }
  uint8_t* const w_lds = s_w + WR * wave * 64;
  auto load_w = [&](int k) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) load_lds16(wbase[i / 2] + k * (kKT / 2) + w_off[i], w_lds + 16 * i * 64);
  };
  // block b, half h (passes 4 h .. 4 h + 3) is chunk 2 g + h of row 32 b + r32
  uint32_t w_rd[NB][2];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int rl = 32 * b + r32;
#pragma unroll
    for (int h = 0; h < 2; ++h) w_rd[b][h] = rl * 64 + 16 * ((2 * g + h) ^ ((rl >> 2) & 3));
  }

  const int nmt = min(MT / 32, (count + 31) / 32);  // 32-token blocks with tokens
  const int nsteps = cols / kKT;                     // a multiple of 4
  // a wave whose activation rows all lie in blocks without tokens loads none
  const bool a_need = wave < nmt;

  // K loop specialised on the number of token blocks with tokens: the
  // accumulators and MFMAs of empty blocks do not exist
  auto kloop = [&](auto nmt_tag) {
    constexpr int NMT = decltype(nmt_tag)::value;
    f32x16_t acc[NMT][NB];
#pragma unroll
    for (int i = 0; i < NMT; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = f32x16_t{};
    // e8m0 bytes of 4 K steps per block (byte 4 j + 2 g + h: group 2 g + h
    // of step j), the current chunk and the next
    u32x4_t scn[NB], s_nxt[NB];
    auto load_sn = [&](u32x4_t (&dst)[NB], int k0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) dst[b] = *reinterpret_cast<const u32x4_t*>(sbase[b] + k0 / 32);
    };
    auto step = [&](auto j_tag, int ks) {
      constexpr int J = decltype(j_tag)::value;
      const uint16_t* const rda = (J & 1) ? s_a1 : s_a0;
      uint16_t* const wra = (J & 1) ? s_a0 : s_a1;
      const int kn = min(ks + 1, nsteps - 1);
      // this step's weights into registers; the next step's then go to LDS
      u32x4_t wv[NB][2];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int h = 0; h < 2; ++h) wv[b][h] = *reinterpret_cast<const u32x4_t*>(w_lds + w_rd[b][h]);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): read before the next loads overwrite
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (a_need) load_a(wra, kn);
      load_w(kn);
      // first step of a chunk: the scales of the chunk after this one (the
      // end-of-step wait leaves them in flight)
      if constexpr (J == 0) load_sn(s_nxt, min(ks + 4, nsteps - 4) * kKT);
      __builtin_amdgcn_sched_barrier(0);
      float sc[NB][2];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint32_t sw = scn[b][J] >> (16 * g);
        sc[b][0] = e8m0_to_f32(sw & 0xffu);
        sc[b][1] = e8m0_to_f32((sw >> 8) & 0xffu);
      }
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        bf16x8_t af[NMT];
        const int off = a_rd + 8 * (p ^ (xr & 7));
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) af[mt] = *reinterpret_cast<const bf16x8_t*>(rda + 32 * mt * kKT + off);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const bf16x8_t bf = fp4_to_bf16x8(wv[b][p >> 2][p & 3], sc[b][p >> 2]);
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt)
            acc[mt][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bf, acc[mt][b], 0, 0, 0);
        }
      }
      if constexpr (J == 3) {
#pragma unroll
        for (int b = 0; b < NB; ++b) scn[b] = s_nxt[b];
      }
      // the next step's operands have landed (J == 0: all but the NB scale
      // loads)
      barrier_keep<J == 0 ? NB : 0>();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    load_sn(scn, 0);
    if (a_need) load_a(s_a0, 0);
    load_w(0);
    vmem_wait_all();
    lds_barrier();
    for (int ks = 0; ks < nsteps; ks += 4) {
      step(I0{}, ks);
      step(I1{}, ks + 1);
      step(I2{}, ks + 2);
      step(I3{}, ks + 3);
    }

    // epilogue: element i of lane l is token 32 mt + 8 (i / 4) + 4 g + i % 4
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tl = 32 * mt + 8 * (i >> 2) + 4 * g + (i & 3);
        if (tl >= count) continue;
        if constexpr (GATEUP) {
          a.h[static_cast<size_t>(p0 + tl) * rows + wrow(0) + r32] =
              static_cast<uint16_t>(f32_to_bf16_rne(silu_fast(acc[mt][0][i]) * acc[mt][1][i]));
        } else {
          const int slot = a.shared ? p0 + tl : min(max(a.perm[p0 + tl], 0), n - 1);
          float* yrow = a.y + static_cast<size_t>(slot) * rows;
#pragma unroll
          for (int b = 0; b < NB; ++b) yrow[wrow(b) + r32] = acc[mt][b][i];
        }
      }
    }
  };
  switch (nmt) {
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    default: kloop(std::integral_constant<int, 1>{}); break;
  }
}

// LDS of k_mfma_mxfp4_w: two activation buffers and the 4 waves' weight rows
constexpr size_t kMxwLds = 2 * 128 * kKT * 2 + 4 * 64 * 64;

// ---------------------------------------------------------------------------
// Affine b-bit experts, b in {2, 3, 4} (w = s q + b per group of G inputs,
// fp16 s and b).
//
// Codes become exact bf16 without a multiply: 3-bit codes in the top bits of
// the mantissa of 2^b give the value off + q, off = 2^b (code_pair); 4-bit
// and 2-bit codes go through the e4m3 and e2m1 converters and give q itself
// (off = 0; see CVT4 and CVT2 below). Each MFMA pass covers 32 consecutive
// inputs, so all of them lie in one group per output row, and per group the
// kernel gets
//   D[m][n] = sum_k x[m][k] (off + q[n][k])   and   X[m] = sum_k x[m][k]
// (X from an extra MFMA against a B operand of ones), then adds
//   s[n] D[m][n] + (b[n] - off s[n]) X[m]
// = sum_k x[m][k] (s[n] q[n][k] + b[n]) to the fp32 accumulator: exact
// products, fp32 sums, the group's scale and bias applied once per group.
//
// This layout serves buckets of a few tokens (hash routing, mid-size
// batches), where the weight stream is the cost. Tiles: MT (16 or 32)
// bucketed tokens x RB * 16 columns per wave (gate/up: RB/2 blocks of gate
// and the same rows of up), 4 waves per workgroup. Each wave streams its 64
// weight rows in macro steps of ROWB bytes per row (128 bytes: 1 K step of
// 8-bit codes, 2 of 4-bit, 4 of 2-bit; 96 bytes, 2 K steps, of 3-bit, which
// keeps that format's staging registers and LDS slot small): every load
// instruction covers 8 rows of the macro step, so it touches few cache
// lines; reading 16 rows x 32 bytes per instruction instead measured 25 %
// less bandwidth from the same number of bytes. The macro step is staged
// in registers one macro step ahead and written to the wave's own padded
// LDS slot, from which lane
// group g of pass s reads the 8-code chunk of inputs 32 s + 8 g .. + 7 and
// recasts it as one word (code i at bit b i, code i + 4 at bit 16 + b i).
// Scales and biases are fetched once per 4 K steps (lane group q holds step
// q) and broadcast with a lane shuffle. A chunk's 8 codes decode
// to bf16 in the order (0, 4, 1, 5, 2, 6, 3, 7) with one shift and one and-or
// per pair; the activations are stored to LDS in that same order within each
// 8-input chunk.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4_t interleave_halves(const u32x4_t& v) {
  // (x0 x1)(x2 x3)(x4 x5)(x6 x7) -> (x0 x4)(x1 x5)(x2 x6)(x3 x7)
  return u32x4_t{(v[0] & 0xffffu) | (v[2] << 16), (v[0] >> 16) | (v[2] & 0xffff0000u),
                 (v[1] & 0xffffu) | (v[3] << 16), (v[1] >> 16) | (v[3] & 0xffff0000u)};
}

// A chunk of 8 codes as the bf16 pairs (v_i, v_{i+4}), i = 0..3, where v is
// 2^b + q for 2-, 3- and 4-bit codes (chunk word: code i at bit BITS i, code
// i + 4 at bit 16 + BITS i) and q itself for 8-bit codes (two words, code i
// in byte i % 4 of word i / 4; the byte converts exactly to fp32, whose top
// half is the exact bf16).
template <int BITS>
__device__ __forceinline__ bf16x8_t chunk_to_bf16x8(const uint32_t (&f)[BITS == 8 ? 2 : 1]) {
  if constexpr (BITS == 8) {
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = static_cast<float>((f[0] >> (8 * i)) & 0xffu);
      const float hi = static_cast<float>((f[1] >> (8 * i)) & 0xffu);
      r[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
    }
    return __builtin_bit_cast(bf16x8_t, r);
  } else {
    const uint32_t k = code_base_pair<BITS>();
    const uint32_t w = f[0];
    const u32x4_t r{code_pair<BITS, 0>(w, k), code_pair<BITS, BITS>(w, k), code_pair<BITS, 2 * BITS>(w, k),
                    code_pair<BITS, 3 * BITS>(w, k)};
    return __builtin_bit_cast(bf16x8_t, r);
  }
}

// MXFP8: a chunk of 8 E4M3 codes (code i in byte i % 4 of word i / 4) as the
// exact bf16 pairs (v_i, v_{i+4}), i = 0..3: v_perm gathers bytes
// (c0, c4, c1, c5) and (c2, c6, c3, c7), and each 16-bit half converts to a
// bf16 pair (scale 1: the e8m0 scale multiplies the group's dot product).
__device__ __forceinline__ bf16x8_t e4m3_chunk_to_bf16x8(const uint32_t (&f)[2]) {
  const uint32_t a = __builtin_amdgcn_perm(f[1], f[0], 0x05010400u);
  const uint32_t b = __builtin_amdgcn_perm(f[1], f[0], 0x07030602u);
  const u32x4_t r{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a, 1.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a, 1.0f, true)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.0f, true))};
  return __builtin_bit_cast(bf16x8_t, r);
}

constexpr int kAffRB = 4;  // 16-column blocks per wave (affine)

// workgroups per CU the register budget is cut for: 3 (168 VGPRs) for the
// 4-bit, 64-group, 16-token down projection, which needs only a few more
// (measured: 304 -> 294 us at 512 tokens; the gate/up one spills more and
// got slower, 626 -> 647 us), else 2
template <bool GATEUP, int BITS, int G, int MT>
constexpr int aff_min_wg() {
  return (!GATEUP && BITS == 4 && G == 64 && MT == 16) ? 3 : 2;
}

// FMT 0: affine codes as above; FMT 2: MXFP8 (BITS 8, G 32), E4M3 codes with
// one e8m0 scale per group and no bias, so no X term.
template <bool GATEUP, int BITS, int G, int MT, int FMT = 0>
__global__ __launch_bounds__(256, (aff_min_wg<GATEUP, BITS, G, MT>())) void k_mfma_affine(MfmaArgs a) {
  static_assert(FMT == 0 || (FMT == 2 && BITS == 8 && G == 32), "MXFP8 is 8-bit codes in groups of 32");
  constexpr int RB = kAffRB;
  constexpr int HB = GATEUP ? RB / 2 : RB;           // row blocks per matrix per wave
  constexpr int NTILE = 4 * HB * 16;                 // rows per matrix per workgroup
  constexpr int PPG = G / 32;                        // MFMA passes per group
  constexpr int GPS = kKT / G;                       // groups per K step
  constexpr int MB = MT / 16;
  constexpr int ACH = (MT * 16 + 255) / 256;         // 16-byte activation chunks per thread per step
  extern __shared__ int32_t s_dyn[];  // expert offsets and m-tile starts, E + 1 each
  int32_t* const s_off = s_dyn;
  int32_t* const s_mt = s_dyn + a.E + 1;
  __shared__ int32_t s_src[MT];
  __shared__ __attribute__((aligned(16))) uint16_t s_a[2][MT][kALdsStride];
  // weight macro steps: ROWB bytes of each of a wave's 64 rows
  constexpr int QW = BITS == 8 ? 2 : 1;         // words per 8-code chunk as read
  // 2-bit codes in groups of 64 or 128 decode through the e2m1 converter:
  // a code q in the low two bits of a nibble is the e2m1 value q / 2, so
  // with the conversion's scale 2 each masked nibble pair becomes the exact
  // bf16 pair (q, q') with no code offset. A 32-bit word of 16 codes serves
  // two passes of a lane group (its even-indexed codes, then its odd ones),
  // so a pass covers inputs 64 t + 16 g + (0, 2, .., 14) or (1, 3, .., 15):
  // 64 inputs, one group. The activations are stored in LDS in that order
  // (each 16-input block as its 8 even-indexed then its 8 odd-indexed inputs).
  constexpr bool CVT2 = BITS == 2 && G >= 64 && FMT == 0;
  // 4-bit codes decode through the e4m3 converter: a byte q in 0..15 is the
  // E4M3 value q 2^-9 (subnormal below 8, exponent 1 from 8 on), so with the
  // conversion's scale 2^9 the nibbles of a chunk word, masked into bytes
  // (even-indexed codes, then after a shift by 4 the odd ones), become the
  // exact bf16 values q with no code offset: the chunk's 8 codes in the order
  // (0, 2, 4, 6, 1, 3, 5, 7), and the activations are stored in LDS in that
  // order within each 8-input chunk.
  constexpr bool CVT4 = BITS == 4 && FMT == 0;
  constexpr float kOff = (BITS == 8 || CVT2 || CVT4) ? 0.0f : static_cast<float>(1 << BITS);  // value of code 0 as decoded
  constexpr int LPR = 8;                        // lanes per row in one load
  constexpr int BPL = BITS == 3 ? 12 : 16;      // bytes per lane in one load
  constexpr int ROWB = LPR * BPL;               // bytes per row per macro step
  constexpr int SPM = ROWB * 8 / (BITS * kKT);  // K steps per macro step
  constexpr int RPI = 64 / LPR;                 // rows per load
  constexpr int NIM = 64 / RPI;                 // loads per macro step
  constexpr int LSTR = ROWB + 16;               // LDS bytes per row (padded against bank conflicts)
  constexpr int BW = BPL / 4;
  static_assert(4 % SPM == 0 && RB * 16 == 64, "macro steps tile the unrolled rounds and 64 rows");
  __shared__ __attribute__((aligned(16))) uint32_t s_b[4][64 * LSTR / 4];  // per wave

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int n = a.T * a.k;
  const int rows = a.m0.rows, cols = a.m0.cols;
  Tile t;
  if (!tile_of_block<MT>(a, rows / NTILE, s_off, s_mt, t)) return;
  // tile coordinates are wave-uniform: keep them (and the addresses built
  // from them) in scalar registers
  const int e = __builtin_amdgcn_readfirstlane(t.e), p0 = __builtin_amdgcn_readfirstlane(t.p0);
  const int count = __builtin_amdgcn_readfirstlane(t.count), ntile = __builtin_amdgcn_readfirstlane(t.ntile);
  const int kslice = __builtin_amdgcn_readfirstlane(t.kslice);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  if (tid < MT) {
    const int p = p0 + min(tid, count - 1);
    s_src[tid] = GATEUP && !a.shared ? min(max(a.perm[p] / a.k, 0), a.T - 1) : p;
  }
  __syncthreads();

  // activations: round i, thread t copies chunk t % 16 of row t / 16 + 16 i
  // (threads beyond the tile's rows repeat the last row's copy)
  const int a_chunk = tid & 15;
  int a_row[ACH];
  uint32_t a_off[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    a_row[i] = min((tid >> 4) + 16 * i, MT - 1);
    a_off[i] = static_cast<uint32_t>(s_src[a_row[i]]) * cols + a_chunk * 8;
  }
  auto load_a = [&](u32x4_t (&ar)[ACH], int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) ar[i] = *reinterpret_cast<const u32x4_t*>(a.x + a_off[i] + k0);
  };
  auto store_a = [&](const u32x4_t (&ar)[ACH], int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      if constexpr (CVT2) {
        // inputs 8 c .. 8 c + 7 (c = a_chunk): half c % 2 of 16-input block c / 2
        const u32x4_t v = ar[i];
        const uint32_t e0 = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);
        const uint32_t e1 = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);
        const uint32_t o0 = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);
        const uint32_t o1 = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);
        uint16_t* blk = &s_a[buf][a_row[i]][16 * (a_chunk >> 1) + 4 * (a_chunk & 1)];
        *reinterpret_cast<uint2*>(blk) = make_uint2(e0, e1);
        *reinterpret_cast<uint2*>(blk + 8) = make_uint2(o0, o1);
      } else if constexpr (CVT4) {
        // inputs 8 c .. 8 c + 7 as (0, 2, 4, 6, 1, 3, 5, 7)
        const u32x4_t v = ar[i];
        *reinterpret_cast<u32x4_t*>(&s_a[buf][a_row[i]][a_chunk * 8]) =
            u32x4_t{__builtin_amdgcn_perm(v[1], v[0], 0x05040100u), __builtin_amdgcn_perm(v[3], v[2], 0x05040100u),
                    __builtin_amdgcn_perm(v[1], v[0], 0x07060302u), __builtin_amdgcn_perm(v[3], v[2], 0x07060302u)};
      } else {
        *reinterpret_cast<u32x4_t*>(&s_a[buf][a_row[i]][a_chunk * 8]) = interleave_halves(ar[i]);
      }
    }
  };

  // weights: wave row R (0..63) is row rbase0 + 16 (R / 16 % HB) + R % 16 of
  // gate (R / 16 < HB) or up; load i of a macro step covers wave rows
  // RPI i .. + RPI - 1, lane l reading BPL bytes at byte (l % LPR) BPL of row
  // RPI i + l / LPR.
  const QMat w0 = expert_slice(a.m0, e);
  const QMat w1 = expert_slice(a.m1, e);
  const int g = lane >> 4, r16 = lane & 15;
  const int rbase0 = ntile * NTILE + wave_u * HB * 16;
  const int rbase = rbase0 + r16;
  const int rg = w0.row_groups, row_bytes = w0.row_words * 4;
  const int lrow = lane / LPR, lbyte = (lane % LPR) * BPL;
  // wave-uniform bases (rows rbase0 ..) and 32-bit lane offsets
  const char* cb0 = reinterpret_cast<const char*>(w0.codes) + static_cast<size_t>(rbase0) * row_bytes;
  const char* cb1 = reinterpret_cast<const char*>(w1.codes) + static_cast<size_t>(rbase0) * row_bytes;
  const uint16_t* s0p = static_cast<const uint16_t*>(w0.scales) + static_cast<size_t>(rbase0) * rg;
  const uint16_t* s1p = static_cast<const uint16_t*>(w1.scales) + static_cast<size_t>(rbase0) * rg;
  const uint16_t* b0p = FMT == 0 ? w0.biases + static_cast<size_t>(rbase0) * rg : nullptr;
  const uint16_t* b1p = FMT == 0 ? w1.biases + static_cast<size_t>(rbase0) * rg : nullptr;
  // MXFP8: one e8m0 byte per group, so a step's 4 groups are one word
  const uint8_t* e0p = static_cast<const uint8_t*>(w0.scales) + static_cast<size_t>(rbase0) * rg;
  const uint8_t* e1p = static_cast<const uint8_t*>(w1.scales) + static_cast<size_t>(rbase0) * rg;
  const uint32_t lrow_off = static_cast<uint32_t>(lrow * row_bytes), sc_off = static_cast<uint32_t>(r16 * rg);
  const int nsteps = cols / kKT;
  // this workgroup's K steps [ks_begin, ks_end) (the host makes slices a
  // multiple of SPM steps)
  const int slice = nsteps / max(a.ksplit, 1);
  const int ks_begin = kslice * slice, ks_end = ks_begin + slice;

  uint32_t stg[NIM][BW];
  // the macro step that starts at K step ks (past the end: clamped, unused)
  auto load_macro = [&](int ks) {
    const uint32_t o = lrow_off + min((ks / SPM) * ROWB + lbyte, row_bytes - BPL);
#pragma unroll
    for (int i = 0; i < NIM; ++i) {
      const int rb = RPI * i / 16;
      const char* p = (rb >= HB ? cb1 : cb0) + static_cast<size_t>(16 * (rb % HB) + RPI * i % 16) * row_bytes + o;
      if constexpr (BW == 4) {
        // gate/up codes non-temporally (measured at 512 tokens: 4-bit gate/up
        // 630 -> 587 us, 2-bit at 64 tokens 290 -> 278 us; the down
        // projection, whose weights more m-tiles share, got slower, and so
        // did the MXFP4 GEMM, which re-reads each expert per 128 tokens)
        u32x4_t v;
        if constexpr (GATEUP)
          v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        else
          v = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
        for (int w = 0; w < 4; ++w) stg[i][w] = v[w];
      } else {
#pragma unroll
        for (int w = 0; w < BW; ++w) stg[i][w] = reinterpret_cast<const uint32_t*>(p)[w];
      }
    }
  };
  char* const sb_w = reinterpret_cast<char*>(&s_b[wave][0]) + lrow * LSTR + lbyte;
  auto store_macro = [&]() {
#pragma unroll
    for (int i = 0; i < NIM; ++i) {
      char* d = sb_w + RPI * i * LSTR;
      if constexpr (BW == 4) {
        *reinterpret_cast<u32x4_t*>(d) = u32x4_t{stg[i][0], stg[i][1], stg[i][2], stg[i][3]};
      } else {
#pragma unroll
        for (int w = 0; w < BW; ++w) reinterpret_cast<uint32_t*>(d)[w] = stg[i][w];
      }
    }
  };
  // chunk c = 16 jm + 4 s + g of row 16 rb + r16 of the macro step in LDS
  const char* const sb_r = reinterpret_cast<const char*>(&s_b[wave][0]) + r16 * LSTR;
  const int g3w = (3 * g) >> 2, g3sh = 8 * ((3 * g) & 3);  // 3-bit: word and bit of chunk g
  auto read_chunk = [&](int rb, int s, int jm, uint32_t (&c)[QW]) {
    const char* row = sb_r + 16 * rb * LSTR;
    if constexpr (BITS == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(row + 8 * (16 * jm + 4 * s + g));
      c[0] = v.x;
      c[QW - 1] = v.y;
    } else if constexpr (BITS == 4) {
      c[0] = *reinterpret_cast<const uint32_t*>(row + 4 * (16 * jm + 4 * s + g));
    } else if constexpr (CVT2) {
      // passes 2 t, 2 t + 1 (t = s / 2) share the word of codes
      // 64 t + 16 g .. + 15 of the step
      c[0] = *reinterpret_cast<const uint32_t*>(row + 32 * jm + 16 * (s >> 1) + 4 * g);
    } else if constexpr (BITS == 2) {
      // codes 0..3 in byte 0, 4..7 in byte 1 -> bytes 0 and 2
      const uint32_t h = *reinterpret_cast<const uint16_t*>(row + 2 * (16 * jm + 4 * s + g));
      c[0] = (h & 0xffu) | ((h << 8) & 0xff0000u);
    } else {
      // 24 bits at byte 3 c: funnel-shift from the two words that hold them,
      // then move codes 4..7 (bits 12..23) up to bit 16
      const uint32_t* w = reinterpret_cast<const uint32_t*>(row) + 12 * jm + 3 * s + g3w;
      const uint32_t v = __builtin_amdgcn_alignbit(w[1], w[0], g3sh);
      c[0] = (v & 0xfffu) | ((v << 4) & 0x0fff0000u);
    }
  };
  // Scales and biases of K steps ks0 .. ks0 + 3: lane group q holds step
  // ks0 + q, so the 4 lane groups of a row read 4 steps' values (contiguous)
  // with one request per row and array.
  constexpr int SWS = GPS == 1 ? 1 : GPS / 2;  // 32-bit words per row per step
  struct Scales {
    uint32_t s[RB][SWS], b[RB][SWS];
  };
  auto load_scales = [&](Scales& sc, int ks0) {
    const int kq = min(ks0 + g, nsteps - 1) * GPS;  // first group of that step
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if constexpr (FMT == 2) {
        const uint8_t* ep = (rb >= HB ? e1p : e0p) + static_cast<size_t>(16 * (rb % HB)) * rg + (sc_off + kq);
        sc.s[rb][0] = *reinterpret_cast<const uint32_t*>(ep);
        continue;
      }
      const uint16_t* sp = (rb >= HB ? s1p : s0p) + static_cast<size_t>(16 * (rb % HB)) * rg + (sc_off + kq);
      const uint16_t* bp = (rb >= HB ? b1p : b0p) + static_cast<size_t>(16 * (rb % HB)) * rg + (sc_off + kq);
      if constexpr (GPS == 1) {
        sc.s[rb][0] = *sp;
        sc.b[rb][0] = *bp;
      } else {
#pragma unroll
        for (int w = 0; w < SWS; ++w) {
          sc.s[rb][w] = reinterpret_cast<const uint32_t*>(sp)[w];
          sc.b[rb][w] = reinterpret_cast<const uint32_t*>(bp)[w];
        }
      }
    }
  };

  f32x4_t acc[MB][RB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int valid_mb = min(MB, (count + 15) / 16);
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  u32x4_t a_reg0[ACH], a_reg1[ACH];
  Scales sc_cur, sc_nxt;

  auto kloop = [&](auto nmb_tag) {
    constexpr int NMB = decltype(nmb_tag)::value;
    // step ks = round base + J; weights one macro step ahead, activations
    // two steps ahead
    auto step = [&](int ks, auto j_tag, u32x4_t (&a_ld)[ACH], const u32x4_t (&a_st)[ACH]) {
      constexpr int J = decltype(j_tag)::value;
      constexpr int JM = J % SPM;
      const int buf = ks & 1;
      if constexpr (JM == 0) {
        // a macro step begins: its staged codes go to the wave's LDS slot and
        // the next macro step's loads are issued (two macro steps in flight,
        // in a second set of staging registers, measured slower: 631 -> 656
        // us for the 4-bit gate/up at 512 tokens)
        store_macro();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        load_macro(ks + SPM);
      }
      load_a(a_ld, min(ks + 2, nsteps - 1) * kKT);
      if constexpr (J % 4 == 0) load_scales(sc_nxt, ks + 4);
      uint32_t qw[RB][4][QW];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (!CVT2 || (s & 1) == 0) read_chunk(rb, s, JM, qw[rb][s]);  // CVT2: one word per two passes
        }
      // this step's scales and biases live in lane group J % 4
      uint32_t sw[RB][SWS], bw[RB][SWS];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int w = 0; w < SWS; ++w) {
          sw[rb][w] = __shfl(sc_cur.s[rb][w], (J & 3) * 16 + r16);
          bw[rb][w] = FMT == 0 ? __shfl(sc_cur.b[rb][w], (J & 3) * 16 + r16) : 0u;
        }

      // group j's scale and bias applied to its partial tiles: after all
      // groups' MFMAs (more independent work between an MFMA and its use), or
      // right after each group's when two m-blocks of several groups would
      // not fit the register file
      constexpr bool EPI_EACH = NMB == 2 && GPS >= 2;
      f32x4_t dg[GPS][NMB][RB], xg[GPS][NMB];
      auto epilogue = [&](int j) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if constexpr (FMT == 2) {
            const float sc = e8m0_to_f32((sw[rb][0] >> (8 * j)) & 0xffu);
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[mb][rb][i] = fmaf(sc, dg[j][mb][rb][i], acc[mb][rb][i]);
            continue;
          }
          const float sc = f16_to_f32(static_cast<uint16_t>(sw[rb][j / 2] >> (16 * (j & 1))));
          const float bb = f16_to_f32(static_cast<uint16_t>(bw[rb][j / 2] >> (16 * (j & 1))));
          const float bc = kOff == 0.0f ? bb : fmaf(-kOff, sc, bb);
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[mb][rb][i] = fmaf(sc, dg[j][mb][rb][i], fmaf(bc, xg[j][mb][i], acc[mb][rb][i]));
        }
      };
#pragma unroll
      for (int j = 0; j < GPS; ++j) {
#pragma unroll
        for (int pp = 0; pp < PPG; ++pp) {
          const int s = j * PPG + pp;
          bf16x8_t af[NMB];
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            const int ao = CVT2 ? 64 * (s >> 1) + 16 * g + 8 * (s & 1) : 32 * s + 8 * g;
            af[mb] = *reinterpret_cast<const bf16x8_t*>(&s_a[buf][mb * 16 + r16][ao]);
          }
          if constexpr (FMT == 0) {
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
              xg[j][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  af[mb], ones, pp == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : xg[j][mb], 0, 0, 0);
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            bf16x8_t bf;
            if constexpr (FMT == 2) {
              bf = e4m3_chunk_to_bf16x8(qw[rb][s]);
            } else if constexpr (CVT2) {
              const uint32_t w = qw[rb][s & ~1][0];
              const uint32_t m = ((s & 1) ? (w >> 2) : w) & 0x33333333u;
              const u32x4_t r{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m, 2.0f, 0)),
                              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m, 2.0f, 1)),
                              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m, 2.0f, 2)),
                              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m, 2.0f, 3))};
              bf = __builtin_bit_cast(bf16x8_t, r);
            } else if constexpr (CVT4) {
              const uint32_t w = qw[rb][s][0];
              const uint32_t ev = w & 0x0f0f0f0fu, od = (w >> 4) & 0x0f0f0f0fu;
              const u32x4_t r{
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, 512.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, 512.0f, true)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, 512.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, 512.0f, true))};
              bf = __builtin_bit_cast(bf16x8_t, r);
            } else {
              bf = chunk_to_bf16x8<BITS>(qw[rb][s]);
            }
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
              dg[j][mb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  af[mb], bf, pp == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : dg[j][mb][rb], 0, 0, 0);
          }
        }
        if constexpr (EPI_EACH) epilogue(j);
      }
      if constexpr (!EPI_EACH) {
#pragma unroll
        for (int j = 0; j < GPS; ++j) epilogue(j);
      }
      if constexpr (J % 4 == 3) sc_cur = sc_nxt;
      store_a(a_st, buf ^ 1);  // after the last step: unused, harmless
      lds_barrier();
    };
    using J0 = std::integral_constant<int, 0>;
    using J1 = std::integral_constant<int, 1>;
    using J2 = std::integral_constant<int, 2>;
    using J3 = std::integral_constant<int, 3>;
    using J4 = std::integral_constant<int, 4>;
    using J5 = std::integral_constant<int, 5>;
    using J6 = std::integral_constant<int, 6>;
    using J7 = std::integral_constant<int, 7>;
    load_scales(sc_cur, ks_begin);
    load_macro(ks_begin);
    load_a(a_reg0, ks_begin * kKT);
    store_a(a_reg0, 0);
    load_a(a_reg0, min(ks_begin + 1, nsteps - 1) * kKT);
    lds_barrier();
    int ks = ks_begin;
    for (; ks + 8 <= ks_end; ks += 8) {
      step(ks, J0{}, a_reg1, a_reg0);
      step(ks + 1, J1{}, a_reg0, a_reg1);
      step(ks + 2, J2{}, a_reg1, a_reg0);
      step(ks + 3, J3{}, a_reg0, a_reg1);
      step(ks + 4, J4{}, a_reg1, a_reg0);
      step(ks + 5, J5{}, a_reg0, a_reg1);
      step(ks + 6, J6{}, a_reg1, a_reg0);
      step(ks + 7, J7{}, a_reg0, a_reg1);
    }
    if (ks < ks_end) step(ks, J0{}, a_reg1, a_reg0);
    if (ks + 1 < ks_end) step(ks + 1, J1{}, a_reg0, a_reg1);
    if (ks + 2 < ks_end) step(ks + 2, J2{}, a_reg1, a_reg0);
    if (ks + 3 < ks_end) step(ks + 3, J3{}, a_reg0, a_reg1);
    if (ks + 4 < ks_end) step(ks + 4, J4{}, a_reg1, a_reg0);
    if (ks + 5 < ks_end) step(ks + 5, J5{}, a_reg0, a_reg1);
    if (ks + 6 < ks_end) step(ks + 6, J6{}, a_reg1, a_reg0);
  };
  if constexpr (MB == 2) {
    if (valid_mb == 2)
      kloop(std::integral_constant<int, 2>{});
    else
      kloop(std::integral_constant<int, 1>{});
  } else {
    kloop(std::integral_constant<int, 1>{});
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= valid_mb) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = mb * 16 + 4 * g + i;
      if (tl >= count) continue;
      if (a.ksplit > 1) {
        // partial sums of this K slice, reduced in slice order by the finisher
        const int width = GATEUP ? 2 * rows : rows;
        float* prow = a.part + (static_cast<size_t>(kslice) * n + (p0 + tl)) * width + rbase;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) prow[(GATEUP && rb >= HB ? rows : 0) + (rb % HB) * 16] = acc[mb][rb][i];
      } else if constexpr (GATEUP) {
        uint16_t* hrow = a.h + static_cast<size_t>(p0 + tl) * rows + rbase;
#pragma unroll
        for (int rb = 0; rb < HB; ++rb)
          hrow[rb * 16] = static_cast<uint16_t>(f32_to_bf16_rne(silu(acc[mb][rb][i]) * acc[mb][rb + HB][i]));
      } else {
        const int slot = a.shared ? p0 + tl : min(max(a.perm[p0 + tl], 0), n - 1);
        float* yrow = a.y + static_cast<size_t>(slot) * rows + rbase;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) yrow[rb * 16] = acc[mb][rb][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
static bool affine_mfma_ok(const QMat& m) {
  // 3-bit codes with groups of 32 exceed the register file in this layout
  // and stay on the streaming path
  if (m.bits == 3 && m.group == 32) return false;
  return m.fmt == 0 && (m.bits == 2 || m.bits == 3 || m.bits == 4 || m.bits == 8) &&
         (m.group == 32 || m.group == 64 || m.group == 128);
}

bool mfma_supported(const QMat& m, bool gateup, int64_t T, int k) {
  // activation rows are addressed with 32-bit element offsets
  if (T * k * m.cols >= (int64_t{1} << 31) || m.cols % kKT != 0) return false;
  if (m.fmt == 1) return m.bits == 4 && m.group == 32 && m.rows % (gateup ? 64 : 128) == 0;
  if (m.fmt == 2) return m.bits == 8 && m.group == 32 && m.rows % ((gateup ? 32 : 64) * kAffRB) == 0;
  return affine_mfma_ok(m) && m.rows % ((gateup ? 32 : 64) * kAffRB) == 0;
}

static unsigned mfma_grid(int T, int k, int E, int rows, int ntile, int mt, int ksplit = 1) {
  const int64_t tk = static_cast<int64_t>(T) * k;
  const int64_t mtiles = (tk + mt - 1) / mt + std::min<int64_t>(tk, E);
  const int64_t pairs = mtiles * (rows / ntile) * std::max(ksplit, 1);
  return static_cast<unsigned>(((pairs + 7) / 8) * 8);
}

template <bool GATEUP, int BITS, int MT>
static void launch_affine(const MfmaArgs& a, hipStream_t s) {
  constexpr int NTILE = (GATEUP ? 32 : 64) * kAffRB;
  const dim3 grid(mfma_grid(a.T, a.k, a.E, a.m0.rows, NTILE, MT, a.ksplit));
  const size_t lds = static_cast<size_t>(2) * (a.E + 1) * sizeof(int32_t);
  if constexpr (MT == 16 && BITS != 3) {
    if (a.m0.group == 32) {
      QSMOE_LAUNCH((k_mfma_affine<GATEUP, BITS, 32, 16>), grid, dim3(256), lds, s, a);
      return;
    }
  }
  if (a.m0.group == 64)
    QSMOE_LAUNCH((k_mfma_affine<GATEUP, BITS, 64, MT>), grid, dim3(256), lds, s, a);
  else
    QSMOE_LAUNCH((k_mfma_affine<GATEUP, BITS, 128, MT>), grid, dim3(256), lds, s, a);
}

template <bool GATEUP>
static hipError_t launch_mfma(const MfmaArgs& a, hipStream_t s) {
  const QMat& m = a.m0;
  constexpr int kMxwN = GATEUP ? 128 : 256;  // k_mfma_mxfp4_w's rows per workgroup (per matrix)
  if (m.fmt == 1 && m.rows % kMxwN == 0 && m.cols % (4 * kKT) == 0 && 2 * (a.E + 1) * 4 <= 4 * 64 * 64 &&
      reinterpret_cast<uintptr_t>(a.m0.scales) % 16 == 0 && reinterpret_cast<uintptr_t>(a.m1.scales) % 16 == 0) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_mfma_mxfp4_w<GATEUP>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMxwLds);
    if (attr != hipSuccess) return attr;
    QSMOE_LAUNCH((k_mfma_mxfp4_w<GATEUP>), dim3(mfma_grid(a.T, a.k, a.E, m.rows, kMxwN, 128)), dim3(256), kMxwLds, s,
                 a);
  } else if (m.fmt == 1) {
    // measured: gate/up best with 128-token tiles x 32 columns per wave, down
    // with 64-token tiles x 64 columns per wave
    constexpr int MT = GATEUP ? 128 : 64, RB = GATEUP ? 2 : 4;
    constexpr int NTILE = 4 * (GATEUP ? RB / 2 : RB) * 16;
    if (m.rows % NTILE == 0) {
      QSMOE_LAUNCH((k_mfma_mxfp4<GATEUP, MT, RB>), dim3(mfma_grid(a.T, a.k, a.E, m.rows, NTILE, MT)),
                         dim3(256), 0, s, a);
    } else {
      constexpr int NT2 = GATEUP ? 64 : 128;
      QSMOE_LAUNCH((k_mfma_mxfp4<GATEUP, 128, 2>), dim3(mfma_grid(a.T, a.k, a.E, m.rows, NT2, 128)),
                         dim3(256), 0, s, a);
    }
  } else if (m.fmt == 2) {
    // MXFP8: the 8-bit affine layout with E4M3 decode and e8m0 group scales
    constexpr int NTILE = (GATEUP ? 32 : 64) * kAffRB;
    const size_t lds = static_cast<size_t>(2) * (a.E + 1) * sizeof(int32_t);
    // 32-token tiles from 8 tokens per expert on average, as for the affine
    // codes (no bias term here, so groups of 32 fit the larger tile: 223
    // VGPRs; measured at 512 tokens: gate/up 830 -> 691 us, down 464 -> 437 us)
    if (static_cast<int64_t>(a.T) * a.k < 8LL * a.E)
      QSMOE_LAUNCH((k_mfma_affine<GATEUP, 8, 32, 16, 2>), dim3(mfma_grid(a.T, a.k, a.E, m.rows, NTILE, 16, a.ksplit)),
                   dim3(256), lds, s, a);
    else
      QSMOE_LAUNCH((k_mfma_affine<GATEUP, 8, 32, 32, 2>), dim3(mfma_grid(a.T, a.k, a.E, m.rows, NTILE, 32, a.ksplit)),
                   dim3(256), lds, s, a);
  } else if (m.bits == 2) {
    launch_affine<GATEUP, 2, 16>(a, s);
  } else if (m.bits == 3) {
    launch_affine<GATEUP, 3, 16>(a, s);
  } else if (static_cast<int64_t>(a.T) * a.k < 8LL * a.E || m.group == 32) {
    // buckets average under 8 tokens (or 4 groups per step). From 8 on, 32-token
    // tiles: fewer buckets need a second tile, whose weights stream again
    // (measured at 512 tokens, ~12 per expert: 4-bit gate/up 582 -> 549 us)
    if (m.bits == 8)
      launch_affine<GATEUP, 8, 16>(a, s);
    else
      launch_affine<GATEUP, 4, 16>(a, s);
  } else if (m.bits == 8) {
    launch_affine<GATEUP, 8, 32>(a, s);
  } else {
    launch_affine<GATEUP, 4, 32>(a, s);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K-split (shared expert at small T): too few (m-tile, n-tile) pairs to fill
// the chip, so each pair's K range is split over ksplit workgroups, which
// write fp32 partial sums; the finishers add the slices in slice order
// (deterministic), then apply SwiGLU and round h to bf16 (gate/up) or store
// y (down).
int mfma_shared_ksplit(const QMat& m, bool gateup, int T) {
  if (m.fmt != 0) return 1;
  const int mt = T < 16 ? 16 : (m.bits < 4 || m.group == 32 ? 16 : 32);
  const int ntile = (gateup ? 32 : 64) * kAffRB;
  const int pairs = ((T + mt - 1) / mt) * (m.rows / ntile);
  const int nsteps = m.cols / kKT;
  int ks = 1;
  // slices of a multiple of 4 K steps (so of every format's macro step)
  while (pairs * ks < 256 && nsteps % (ks * 2) == 0 && (nsteps / (ks * 2)) % 4 == 0) ks *= 2;
  return ks;
}

__global__ __launch_bounds__(256) void k_swiglu_parts(const float* __restrict__ part, int ks, int n, int I,
                                                      uint16_t* __restrict__ h) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(n) * I) return;
  const int64_t p = i / I, r = i - p * I;
  float g = 0.0f, u = 0.0f;
  for (int s = 0; s < ks; ++s) {
    const float* row = part + (static_cast<int64_t>(s) * n + p) * 2 * I;
    g += row[r];
    u += row[I + r];
  }
  h[i] = static_cast<uint16_t>(f32_to_bf16_rne(silu(g) * u));
}

__global__ __launch_bounds__(256) void k_sum_parts(const float* __restrict__ part, int ks, int64_t count,
                                                   float* __restrict__ y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count) return;
  float v = 0.0f;
  for (int s = 0; s < ks; ++s) v += part[static_cast<int64_t>(s) * count + i];
  y[i] = v;
}

hipError_t launch_swiglu_parts(const float* part, int ks, int n, int I, uint16_t* h, hipStream_t s) {
  const int64_t count = static_cast<int64_t>(n) * I;
  QSMOE_LAUNCH(k_swiglu_parts, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256), 0, s, part, ks, n, I, h);
  return hipGetLastError();
}

hipError_t launch_sum_parts(const float* part, int ks, int64_t count, float* y, hipStream_t s) {
  QSMOE_LAUNCH(k_sum_parts, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256), 0, s, part, ks, count, y);
  return hipGetLastError();
}

// Shared mode (one expert over all tokens) takes k = E = 1.
hipError_t launch_mfma_gateup(const GateUpArgs& g, hipStream_t s) {
  const int k = g.shared ? 1 : g.k, E = g.shared ? 1 : g.E;
  return launch_mfma<true>(
      MfmaArgs{g.gate, g.up, g.x, g.T, k, E, g.offsets, g.perm, g.shared, g.h, nullptr, g.ksplit, g.part}, s);
}

hipError_t launch_mfma_down(const DownArgs& d, hipStream_t s) {
  const int k = d.shared ? 1 : d.k, E = d.shared ? 1 : d.E;
  return launch_mfma<false>(
      MfmaArgs{d.down, d.down, d.h, d.T, k, E, d.offsets, d.perm, d.shared, nullptr, d.y, d.ksplit, d.part}, s);
}

}  // namespace qsmoe
