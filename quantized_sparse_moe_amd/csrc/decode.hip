// Fused small-batch (decode) path of the layer: three launches instead of
// eight when a step has at most 4 tokens, top-k routing and at most 256
// experts.
//
//   1. k_dec_router: the fp32 router logits (one workgroup per expert) with each
//      expert's score and ranking key, and on the remaining workgroups the
//      shared expert's gate/up + SwiGLU (no routing needed).
//   2. k_dec_gateup: each workgroup selects the top-k from the keys (same
//      selection as moe_route, so the ids are bit-identical) and streams the
//      selected experts' gate/up rows; no bucketing kernel is needed because
//      each (token, slot) is its own bucket when tokens are this few.
//   3. k_dec_down_combine: per output row, the k selected experts' down rows
//      and the shared expert's down row are dotted with their own h vectors
//      (all held in registers), weighted by the router weights and summed in
//      one reduction: down projection, shared expert and combine in one pass,
//      without atomics (one writer per output element).
//
// The layer's definition is that of the general path (router: fp32 gate of
// mlx-lm PR "Add DeepSeek-v4 (Flash/Pro)", sqrtsoftplus of
// "mlx-community / DeepSeek-V4-Flash-4bit"; experts: the same PR's stacked
// gate/up/down; shared expert of "DeepSeek-V4-Flash-MLX-4bit"); only the
// order of the fp32 additions in the combine differs.
#include <algorithm>
#include <type_traits>

#include "decode_core.hpp"

namespace qsmoe {

// Launch 1: router logits of one expert per workgroup (split-K over its four
// waves), with the expert's score and ranking key for every token; the
// remaining workgroups stream the shared expert's gate/up, which needs no
// routing.
template <int TT, int SCPL, int SNT>
__global__ __launch_bounds__(256) void k_dec_router(DecodeArgs a) {
  __shared__ float s_part[4 * TT];
  if (static_cast<int>(blockIdx.x) < a.n_logit_blocks) {
    logits_wg<TT>(a.x, a.wr, a.T, a.E, a.d, blockIdx.x, 0, a.logits, s_part, a.bias, a.keys, a.scores);
  } else if constexpr (SNT > 0) {
    StreamArgs sa{a.sgate, a.sup, a.x, a.T, a.k, 1, nullptr, nullptr, 1, a.h_sh, nullptr};
    ffn_stream_body<0, 8, SCPL, SNT, true>(sa, blockIdx.x - a.n_logit_blocks, gridDim.x - a.n_logit_blocks, nullptr,
                                           nullptr);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Launch 2. Every workgroup first selects each token's top-k from the
// launch-1 keys (wave t: token t, keys in registers; same selection as
// moe_route, so the ids are bit-identical; workgroup 0 also publishes ids and
// weights for launch 3), then streams the (token, slot) x row units of the
// selected experts' gate/up, split evenly over all waves.
template <int F, int B, int CPL>
__global__ __launch_bounds__(256) void k_dec_gateup(DecodeArgs a) {
  __shared__ int32_t s_ids[kDecMaxT * kDecMaxK];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  if (wave < a.T) {
    int id;
    float wt;
    dec_token_head(a, wave, blockIdx.x == 0, id, wt);
    if (lane < a.k) {
      s_ids[wave * a.k + lane] = id;
      if (blockIdx.x == 0) {
        a.ids[wave * a.k + lane] = id;
        a.w[wave * a.k + lane] = wt;
      }
    }
  }
  __syncthreads();
  const int rows = a.gate.rows, nchunks = a.gate.cols >> 5;
  const int64_t total = static_cast<int64_t>(a.T) * a.k * rows;
  const int64_t W = static_cast<int64_t>(gridDim.x) * 4, gw = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  int64_t u = total * gw / W;
  const int64_t u_end = total * (gw + 1) / W;
  while (u < u_end) {
    const int slot = static_cast<int>(u / rows);
    const int r_begin = static_cast<int>(u - static_cast<int64_t>(slot) * rows);
    const int r_end = static_cast<int>(min<int64_t>(rows, r_begin + (u_end - u)));
    const int t = slot / a.k;
    const uint16_t* xrow[1] = {a.x + static_cast<size_t>(t) * a.d};
    const bool xvalid[1] = {true};
    XRaw<CPL, 1> xw;
    load_x_raw<CPL, 1>(xw, xrow, lane, nchunks);
    const int e = min(max(__builtin_amdgcn_readfirstlane(s_ids[slot]), 0), a.E - 1);
    const QMat q0 = expert_slice(a.gate, e), q1 = expert_slice(a.up, e);
    uint16_t* hs = a.h + static_cast<size_t>(slot) * rows;
    stream_rows<F, B, CPL, 1, true, 1>(q0, q1, xw, xvalid, r_begin, r_end, lane, nchunks,
                                    [&](int, int r, float g, float up) {
                                      hs[r] = static_cast<uint16_t>(f32_to_bf16_rne(silu(g) * up));
                                    });
    u += r_end - r_begin;
  }
  __syncthreads();
}

// The shared expert's down rows [*ctr, end) of the single token, taken one
// at a time from an LDS counter (next row's loads issued before the current
// row is computed): y_sh[r] = down row r . h_sh, fp32. Takes no further row
// once *stop is non-zero (stop may be null). Requires end > 0.
__device__ __forceinline__ void dec_shared_down_rows(const DecodeArgs& a, uint32_t* ctr, uint32_t end, int lane,
                                                     const uint32_t* stop) {
  const int nchunks = a.sdown.cols >> 5;
  auto grab = [&]() -> uint32_t {
    if (stop != nullptr && __hip_atomic_load(stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u) return end;
    uint32_t v = 0;
    if (lane == 0) v = atomicAdd(ctr, 1u);
    return __builtin_amdgcn_readfirstlane(v);
  };
  const uint16_t* srow[1] = {a.h_sh};
  const bool sv[1] = {true};
  XRaw<1, 1> hw;
  load_x_raw<1, 1>(hw, srow, lane, nchunks);
  RowRegs<0, 8, 1> A, Bb;
  XRegs<0, 8, 1, 1> hs;
  auto compute = [&](const RowRegs<0, 8, 1>& r, uint32_t u) {
    const float v[1] = {row_dot_one<0, 8, 1, 1>(r, hs, 0, lane, nchunks)};
    const float y = wave_reduce_multi<1>(v);
    if (reduce_multi_writer<1>(lane)) a.y_sh[u] = y;
  };
  uint32_t u0 = grab();
  load_row<0, 8, 1>(A, a.sdown, min(u0, end - 1), lane, nchunks);
  finish_x<0, 8, 1, 1>(hs, hw, sv, lane, nchunks);
  if (u0 >= end) return;
  while (true) {
    const uint32_t u1 = grab();
    load_row<0, 8, 1>(Bb, a.sdown, min(u1, end - 1), lane, nchunks);
    compute(A, u0);
    if (u1 >= end) break;
    const uint32_t u2 = grab();
    load_row<0, 8, 1>(A, a.sdown, min(u2, end - 1), lane, nchunks);
    compute(Bb, u1);
    if (u2 >= end) break;
    u0 = u2;
  }
}

// The routed (slot, row) units [*ctr, u_end) of k_dec_gateup1 (u_end > 0).
template <int F, int B, int CPL, bool FULL>
__device__ __forceinline__ void dec_gateup1_rows(const DecodeArgs& a, const int32_t* s_ids, uint32_t* ctr,
                                                 uint32_t u_end, const XRaw<CPL, 1>& xw, int lane) {
  const int rows = a.gate.rows, nchunks = FULL ? 64 * CPL : a.gate.cols >> 5;
  const bool xvalid[1] = {true};
  auto grab = [&]() -> uint32_t {
    uint32_t v = 0;
    if (lane == 0) v = atomicAdd(ctr, 1u);
    return __builtin_amdgcn_readfirstlane(v);
  };
  using Batch = RowBatch<F, B, CPL, true, 1>;
  // loads are unconditional: a unit past the end reloads the last one
  auto load_unit = [&](Batch& bt, uint32_t u) {
    const uint32_t uc = min(u, u_end - 1);
    const int slot = static_cast<int>(uc / rows), r = static_cast<int>(uc - static_cast<uint32_t>(slot) * rows);
    const int e = min(max(__builtin_amdgcn_readfirstlane(s_ids[slot]), 0), a.E - 1);
    load_batch<F, B, CPL, true, 1>(bt, expert_slice(a.gate, e), expert_slice(a.up, e), r, r + 1, lane, nchunks);
  };
  XRegs<F, B, CPL, 1> xr;
  auto compute_unit = [&](const Batch& bt, uint32_t u) {
    const int slot = static_cast<int>(u / rows), r = static_cast<int>(u - static_cast<uint32_t>(slot) * rows);
    uint16_t* hs = a.h + static_cast<size_t>(slot) * rows;
    auto store = [&](int, int rr, float g, float up) {
      hs[rr] = static_cast<uint16_t>(f32_to_bf16_rne(silu(g) * up));
    };
    compute_batch<F, B, CPL, 1, true, 1>(bt, xr, r, r + 1, lane, nchunks, store);
  };
  Batch A, Bb;
  uint32_t u0 = grab();
  load_unit(A, u0);
  finish_x<F, B, CPL, 1>(xr, xw, xvalid, lane, nchunks);
  if (u0 < u_end) {
    while (true) {
      const uint32_t u1 = grab();
      load_unit(Bb, u1);
      compute_unit(A, u0);
      if (u1 >= u_end) break;
      const uint32_t u2 = grab();
      load_unit(A, u2);
      compute_unit(Bb, u1);
      if (u2 >= u_end) break;
      u0 = u2;
    }
  }
}

// Launch 2 for a single token: one 512-thread workgroup per CU takes an equal
// share of the (slot, row) units, and inside it the 8 waves take rows one at
// a time from an LDS counter, the next row's loads issued before the current
// row is computed. Two waves share each SIMD and the older one is issued
// first: with a fixed split per wave (or per workgroup, two per CU) the
// younger half measured ~20 % slower and the launch ended with it.
// While wave 0 selects the top-k, the other waves stream the shared
// expert's down rows of the workgroup's share of the output rows (SHD: the
// layer has a shared expert; it needs no routing, and launch 3 then only adds
// y_sh); every wave joins the routed rows once the ids are in LDS, and the
// shared rows left over are taken by the waves that run out of routed rows.
// FULL: the input width is exactly 64 CPL chunks of 32 (every lane's
// chunks exist): validity masks and address clamps fold away.
template <int F, int B, int CPL, bool FULL, bool SHD>
__global__ __launch_bounds__(512) void k_dec_gateup1(DecodeArgs a) {
  __shared__ int32_t s_ids[kDecMaxK];
  __shared__ uint32_t s_next, s_sh_next, s_ready;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int rows = a.gate.rows, nchunks = FULL ? 64 * CPL : a.gate.cols >> 5;
  const uint32_t G = gridDim.x, b = blockIdx.x;
  const uint32_t total = static_cast<uint32_t>(a.k) * rows;
  const uint32_t u_begin = static_cast<uint32_t>(static_cast<uint64_t>(total) * b / G);
  const uint32_t u_end = static_cast<uint32_t>(static_cast<uint64_t>(total) * (b + 1) / G);
  const uint32_t d_rows = SHD ? static_cast<uint32_t>(a.sdown.rows) : 0u;
  const uint32_t r0 = static_cast<uint32_t>(static_cast<uint64_t>(d_rows) * b / G);
  const uint32_t r1 = static_cast<uint32_t>(static_cast<uint64_t>(d_rows) * (b + 1) / G);
  if (threadIdx.x == 0) {
    s_next = u_begin;
    s_sh_next = r0;
    s_ready = 0;
  }
  const uint16_t* xrow[1] = {a.x};
  const bool xvalid[1] = {true};
  XRaw<CPL, 1> xw;
  load_x_raw<CPL, 1>(xw, xrow, lane, nchunks);
  __syncthreads();
  if (wave == 0) {
    int id;
    float wt;
    dec_token_head(a, 0, b == 0, id, wt);
    if (lane < a.k) {
      s_ids[lane] = id;
      if (b == 0) {
        a.ids[lane] = id;
        a.w[lane] = wt;
      }
    }
    __hip_atomic_store(&s_ready, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else if constexpr (SHD) {
    if (r0 < r1) dec_shared_down_rows(a, &s_sh_next, r1, lane, &s_ready);
  }
  // the ids (wave 0 always stores them; the poll is bounded all the same)
  for (uint32_t it = 0; it < kLdsSpinLimit; ++it) {
    if (__hip_atomic_load(&s_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u) break;
    __builtin_amdgcn_s_sleep(1);
  }
  if (u_begin < u_end) dec_gateup1_rows<F, B, CPL, FULL>(a, s_ids, &s_next, u_end, xw, lane);
  if constexpr (SHD) {
    if (r0 < r1) dec_shared_down_rows(a, &s_sh_next, r1, lane, nullptr);
  }
}

// ---------------------------------------------------------------------------
// Output row r of token t: the lane's partial of the shared row (ysh) plus the
// weighted partials of the k routed rows, reduced over the wave, plus the
// shared expert's output when launch 2 computed it (ypre), and stored.
template <int F, int B, int K>
__device__ __forceinline__ void dec_finish_row(const RoutedRows<F, B, K>& b, const XRegs<F, B, 1, K>& hx,
                                               const float (&wj)[K], float ysh, float ypre, const DecodeArgs& a, int t,
                                               int r, bool valid, int lane, int nchunks) {
  float v[1] = {ysh};
#pragma unroll
  for (int j = 0; j < K; ++j) v[0] += wj[j] * row_dot_one<F, B, 1, K>(b.r[j], hx, j, lane, nchunks);
  const float y = wave_reduce_multi<1>(v) + ypre;
  if (reduce_multi_writer<1>(lane) && valid) {
    const size_t o = static_cast<size_t>(t) * a.down.rows + r;
    if (a.out_f32)
      static_cast<float*>(a.out)[o] = y;
    else
      static_cast<uint16_t*>(a.out)[o] = static_cast<uint16_t>(f32_to_bf16_rne(y));
  }
}

constexpr int kDecSegRows = 4;  // output rows per segment of a wave's range

// Launch 3: per (token, output row) unit, the k selected experts' down rows
// and the shared expert's down row against their own h vectors, weighted and
// summed in one reduction (SHM 1; SHM 2: launch 2 computed the shared
// expert's output y_sh, which is added; SHM 0: no shared expert). A wave's rows go in segments of kDecSegRows: the
// segment's shared rows are loaded first (for the first segment, before the
// routing ids are even read, so that stream hides the ids' round trip), then
// its routed rows, one row ahead of the arithmetic.
// FULL: both input widths (intermediate sizes) are exactly 64 chunks of 32.
template <int F, int B, int K, int SHM, bool FULL>
__global__ __launch_bounds__(256) void k_dec_down_combine(DecodeArgs a) {
  constexpr bool SH = SHM == 1, PRE = SHM == 2;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int rows = a.down.rows, I = FULL ? 2048 : a.down.cols, nchunks = I >> 5;
  const int Ish = SH ? (FULL ? 2048 : a.sdown.cols) : 32, nchunks_sh = Ish >> 5;
  const int64_t total = static_cast<int64_t>(a.T) * rows;
  const int64_t W = static_cast<int64_t>(gridDim.x) * 4, gw = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  int64_t u = total * gw / W;
  const int64_t u_end = total * (gw + 1) / W;
  while (u < u_end) {
    const int t = static_cast<int>(u / rows);
    const int r_begin = static_cast<int>(u - static_cast<int64_t>(t) * rows);
    const int r_end = static_cast<int>(min<int64_t>(rows, r_begin + (u_end - u)));
    // shared h and the first segment's shared rows: no routing needed
    RowRegs<0, 8, 1> rs[kDecSegRows];
    XRaw<1, 1> hsw;
    const uint16_t* srow[1] = {a.h_sh + static_cast<size_t>(t) * Ish};
    const bool sv[1] = {true};
    if constexpr (SH) {
      load_x_raw<1, 1>(hsw, srow, lane, nchunks_sh);
#pragma unroll
      for (int i = 0; i < kDecSegRows; ++i) load_row<0, 8, 1>(rs[i], a.sdown, min(r_begin + i, r_end - 1), lane, nchunks_sh);
    }
    // ids, weights and the routed h rows
    int id_raw[K];
    float wj[K];
    const uint16_t* hrow[K];
    bool hvalid[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const bool ok = j < a.k;
      const int jj = ok ? j : 0;
      id_raw[j] = a.ids[t * a.k + jj];
      wj[j] = a.w[t * a.k + jj];
      wj[j] = ok ? wj[j] : 0.0f;
      hrow[j] = a.h + static_cast<size_t>(t * a.k + jj) * I;
      hvalid[j] = ok;
    }
    XRaw<1, K> hw;
    load_x_raw<1, K>(hw, hrow, lane, nchunks);
    XRegs<0, 8, 1, 1> hsx;
    if constexpr (SH) finish_x<0, 8, 1, 1>(hsx, hsw, sv, lane, nchunks_sh);
    QMat qd[K];
#pragma unroll
    for (int j = 0; j < K; ++j)
      qd[j] = expert_slice(a.down, min(max(__builtin_amdgcn_readfirstlane(id_raw[j]), 0), a.E - 1));
    XRegs<F, B, 1, K> hx;
    auto segment = [&](int seg0, auto first_tag) {
      constexpr bool FIRST = decltype(first_tag)::value;
      if constexpr (SH && !FIRST) {
#pragma unroll
        for (int i = 0; i < kDecSegRows; ++i)
          load_row<0, 8, 1>(rs[i], a.sdown, min(seg0 + i, r_end - 1), lane, nchunks_sh);
      }
      RoutedRows<F, B, K> A, Bb;
      dec_load_routed<F, B, K>(A, qd, min(seg0, r_end - 1), lane, nchunks);
      float ypre[kDecSegRows];
#pragma unroll
      for (int i = 0; i < kDecSegRows; ++i)
        ypre[i] = PRE ? a.y_sh[static_cast<size_t>(t) * rows + min(seg0 + i, r_end - 1)] : 0.0f;
      if constexpr (FIRST) {
        finish_x<F, B, 1, K>(hx, hw, hvalid, lane, nchunks);
      }
      float ysh[kDecSegRows];
#pragma unroll
      for (int i = 0; i < kDecSegRows; ++i)
        ysh[i] = SH ? row_dot_one<0, 8, 1, 1>(rs[i], hsx, 0, lane, nchunks_sh) : 0.0f;
      dec_load_routed<F, B, K>(Bb, qd, min(seg0 + 1, r_end - 1), lane, nchunks);
      dec_finish_row<F, B, K>(A, hx, wj, ysh[0], ypre[0], a, t, seg0, seg0 < r_end, lane, nchunks);
      dec_load_routed<F, B, K>(A, qd, min(seg0 + 2, r_end - 1), lane, nchunks);
      dec_finish_row<F, B, K>(Bb, hx, wj, ysh[1], ypre[1], a, t, seg0 + 1, seg0 + 1 < r_end, lane, nchunks);
      dec_load_routed<F, B, K>(Bb, qd, min(seg0 + 3, r_end - 1), lane, nchunks);
      dec_finish_row<F, B, K>(A, hx, wj, ysh[2], ypre[2], a, t, seg0 + 2, seg0 + 2 < r_end, lane, nchunks);
      dec_finish_row<F, B, K>(Bb, hx, wj, ysh[3], ypre[3], a, t, seg0 + 3, seg0 + 3 < r_end, lane, nchunks);
    };
    static_assert(kDecSegRows == 4, "the segment body is unrolled for 4 rows");
    segment(r_begin, std::true_type{});
    for (int seg0 = r_begin + kDecSegRows; seg0 < r_end; seg0 += kDecSegRows) segment(seg0, std::false_type{});
    u += r_end - r_begin;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
static int dec_cpl(int cols) { return cols <= 2048 ? 1 : (cols <= 4096 ? 2 : 4); }

bool decode_path_supported(const DecodeArgs& a) {
  if (a.T < 1 || a.T > kDecMaxT || a.k > kDecMaxK || a.E > 256 || a.d % 32 != 0) return false;
  if (a.down.cols > 2048) return false;
  if (a.has_shared) {
    if (a.sgate.fmt != 0 || a.sgate.bits != 8 || a.sdown.fmt != 0 || a.sdown.bits != 8) return false;
    if (a.sdown.cols > 2048) return false;
  }
  return true;
}

// Grid sizing of launches 2 and 3: at most kDecMaxWg workgroups, at least
// the given rows per wave (measured: 2 rows per wave for gate/up and the
// shared gate/up, 4 for the down projection).
constexpr int64_t kDecMaxWg = 512;
constexpr int kDecGuMinRows = 2;
constexpr int kDecShMinRows = 2;
constexpr int kDecDnMinRows = 4;

// Workgroups for `units` rows with at least `min_rows` rows per wave.
static unsigned dec_grid(int64_t units, int min_rows = 2) {
  const int64_t per_wg = 4 * min_rows;
  return static_cast<unsigned>(
      std::max<int64_t>(1, std::min<int64_t>((units + per_wg - 1) / per_wg, kDecMaxWg)));
}

#define QSMOE_DEC_FMT(FMT_, BITS_, ...)                      \
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

// Tokens per pass of the shared expert's gate/up (0: no shared expert).
static int dec_shared_nt(const DecodeArgs& a, int cpl) {
  if (!a.has_shared) return 0;
  int nt = a.T <= 1 ? 1 : (a.T <= 2 ? 2 : 4);
  while (nt * cpl > 4) nt >>= 1;
  return nt;
}

hipError_t launch_dec_router(const DecodeArgs& a0, hipStream_t s) {
  DecodeArgs a = a0;
  a.n_logit_blocks = a.E;
  const int scpl = a.has_shared ? dec_cpl(a.sgate.cols) : 1;
  const int snt = dec_shared_nt(a, scpl);
  unsigned grid = a.n_logit_blocks;
  if (snt > 0) grid += dec_grid(static_cast<int64_t>((a.T + snt - 1) / snt) * a.sgate.rows, kDecShMinRows);
  const int tt = a.T <= 1 ? 1 : (a.T <= 2 ? 2 : 4);
#define QSMOE_K1(CP, NT_)                                                                   \
  do {                                                                                      \
    if (tt == 1)                                                                            \
      QSMOE_LAUNCH((k_dec_router<1, CP, NT_>), dim3(grid), dim3(256), 0, s, a);       \
    else if (tt == 2)                                                                       \
      QSMOE_LAUNCH((k_dec_router<2, CP, NT_>), dim3(grid), dim3(256), 0, s, a);       \
    else                                                                                    \
      QSMOE_LAUNCH((k_dec_router<4, CP, NT_>), dim3(grid), dim3(256), 0, s, a);       \
  } while (0)
  if (snt == 0) QSMOE_K1(1, 0);
  else if (scpl == 1 && snt == 1) QSMOE_K1(1, 1);
  else if (scpl == 1 && snt == 2) QSMOE_K1(1, 2);
  else if (scpl == 1) QSMOE_K1(1, 4);
  else if (scpl == 2 && snt == 1) QSMOE_K1(2, 1);
  else if (scpl == 2) QSMOE_K1(2, 2);
  else QSMOE_K1(4, 1);
#undef QSMOE_K1
  return hipGetLastError();
}

static int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

// Launch 2 of a single token runs one 512-thread workgroup per CU
// (k_dec_gateup1; a hidden size above 4096 would spill at 512 threads).
static bool dec_single_token(const DecodeArgs& a) {
  return a.T == 1 && dec_cpl(a.gate.cols) <= 2 && device_cus() > 0;
}

bool dec_shared_in_gateup(const DecodeArgs& a) { return a.has_shared && dec_single_token(a); }

hipError_t launch_dec_gateup(const DecodeArgs& a, hipStream_t s) {
  const int cpl = dec_cpl(a.gate.cols);
  if (dec_single_token(a)) {
    const dim3 grid(static_cast<unsigned>(device_cus())), block(512);
    const bool full = a.gate.cols == 2048 * cpl;
#define QSMOE_K2(CP, FU)                                                                   \
  do {                                                                                     \
    if (a.has_shared)                                                                      \
      QSMOE_LAUNCH((k_dec_gateup1<F, B, CP, FU, true>), grid, block, 0, s, a);             \
    else                                                                                   \
      QSMOE_LAUNCH((k_dec_gateup1<F, B, CP, FU, false>), grid, block, 0, s, a);            \
  } while (0)
    QSMOE_DEC_FMT(a.gate.fmt, a.gate.bits, {
      if (cpl == 1 && full)
        QSMOE_K2(1, true);
      else if (cpl == 1)
        QSMOE_K2(1, false);
      else if (full)
        QSMOE_K2(2, true);
      else
        QSMOE_K2(2, false);
    })
#undef QSMOE_K2
    return hipGetLastError();
  }
  const dim3 grid(dec_grid(static_cast<int64_t>(a.T) * a.k * a.gate.rows, kDecGuMinRows)), block(256);
  QSMOE_DEC_FMT(a.gate.fmt, a.gate.bits, {
    if (cpl == 1)
      QSMOE_LAUNCH((k_dec_gateup<F, B, 1>), grid, block, 0, s, a);
    else if (cpl == 2)
      QSMOE_LAUNCH((k_dec_gateup<F, B, 2>), grid, block, 0, s, a);
    else
      QSMOE_LAUNCH((k_dec_gateup<F, B, 4>), grid, block, 0, s, a);
  })
  return hipGetLastError();
}

hipError_t launch_dec_down_combine(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(dec_grid(static_cast<int64_t>(a.T) * a.down.rows, kDecDnMinRows)), block(256);
  const size_t lds = 0;
  const int K = a.k <= 2 ? 2 : (a.k <= 4 ? 4 : (a.k <= 6 ? 6 : 8));
  const int shm = !a.has_shared ? 0 : (dec_shared_in_gateup(a) ? 2 : 1);
  const bool full = a.down.cols == 2048 && (shm != 1 || a.sdown.cols == 2048);
#define QSMOE_K3S(K_, SHM_)                                                                            \
  do {                                                                                                 \
    if (full)                                                                                          \
      QSMOE_LAUNCH((k_dec_down_combine<F, B, K_, SHM_, true>), grid, block, lds, s, a);                \
    else                                                                                               \
      QSMOE_LAUNCH((k_dec_down_combine<F, B, K_, SHM_, false>), grid, block, lds, s, a);               \
  } while (0)
#define QSMOE_K3(K_)            \
  do {                          \
    if (shm == 2)               \
      QSMOE_K3S(K_, 2);         \
    else if (shm == 1)          \
      QSMOE_K3S(K_, 1);         \
    else                        \
      QSMOE_K3S(K_, 0);         \
  } while (0)
  QSMOE_DEC_FMT(a.down.fmt, a.down.bits, {
    if (K == 2) QSMOE_K3(2);
    else if (K == 4) QSMOE_K3(4);
    else if (K == 6) QSMOE_K3(6);
    else QSMOE_K3(8);
  })
#undef QSMOE_K3
#undef QSMOE_K3S
  return hipGetLastError();
}

}  // namespace qsmoe
