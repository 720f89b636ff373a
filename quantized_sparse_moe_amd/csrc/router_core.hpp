// Routing core shared by the router kernels and the fused small-batch path:
// the fp32 logit GEMV of a wave and the per-token top-k, so both compute
// bit-identical logits, ids and weights.
#pragma once

#include "common.hpp"

namespace qsmoe {

// Order-preserving map of an fp32 key and expert index to a 64-bit value:
// larger key first, equal keys -> lower index first.
__device__ __forceinline__ uint64_t pack_key(float key, int e) {
  const uint32_t u = __float_as_uint(key);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(0xffffffffu - static_cast<uint32_t>(e));
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(v)), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, 0xF, 0xF, true);
  const uint64_t o = (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
  return o > v ? o : v;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), l);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Wave maximum: DPP within each row of 16 lanes (quad swaps, half-row and row
// mirrors), then the four row results through readlane. Uniform result.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0xB1>(v);
  v = dpp_max_step<0x4E>(v);
  v = dpp_max_step<0x141>(v);
  v = dpp_max_step<0x140>(v);
  uint64_t m = readlane_u64(v, 0);
  const uint64_t r1 = readlane_u64(v, 16), r2 = readlane_u64(v, 32), r3 = readlane_u64(v, 48);
  m = r1 > m ? r1 : m;
  m = r2 > m ? r2 : m;
  m = r3 > m ? r3 : m;
  return m;
}

// Score and ranking key of expert e for logit l: s = sqrt(softplus(l)) and
// the packed (s + bias, ~e) key.
__device__ __forceinline__ void score_key(float l, const float* __restrict__ bias, int e, float& s, uint64_t& key) {
  s = sqrtsoftplus(l);
  key = pack_key(s + (bias ? bias[e] : 0.0f), e);
}

// Logits of expert e for tokens t0 .. t0+TT-1 (clamped to T) by the four
// waves of a workgroup: wave w takes the columns [w d/4, (w+1) d/4) (d % 32
// == 0; the quarter boundaries are multiples of 8), its lanes striding them 8
// values at a time (32 B of Wr, 16 B of x per token) with every load of the
// quarter (up to 1024 columns) issued in one batch, then one multi-value wave
// reduction; wave 0 adds the four partial sums in wave order. The order of
// every addition is fixed, so every caller gets identical logits. With
// `keys`, the writer lane also stores each token's score and ranking key.
// Must be called by all four waves of the workgroup with the same e and t0;
// s_part holds 4 * TT floats of LDS.
template <int TT>
__device__ __forceinline__ void logits_wg(const uint16_t* __restrict__ x, const float* __restrict__ wr, int T, int E,
                                          int d, int e, int t0, float* __restrict__ logits, float* s_part,
                                          const float* __restrict__ bias = nullptr, uint64_t* keys = nullptr,
                                          float* scores = nullptr) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int q8 = d >> 3;  // columns in units of 8
  const int c_begin = ((q8 * wave) >> 2) << 3, c_end = ((q8 * (wave + 1)) >> 2) << 3;
  float acc[TT];
#pragma unroll
  for (int j = 0; j < TT; ++j) acc[j] = 0.0f;
  const float* wrow = wr + static_cast<size_t>(e) * d;
  constexpr int kSteps = 2;  // 2 * 512 columns per batch
  for (int base0 = c_begin + lane * 8; base0 < c_end; base0 += kSteps * 512) {
    float4 w0[kSteps], w1[kSteps];
    uint4 xv[kSteps][TT];
#pragma unroll
    for (int q = 0; q < kSteps; ++q) {
      const int c = min(base0 + q * 512, d - 8);
      w0[q] = *reinterpret_cast<const float4*>(wrow + c);
      w1[q] = *reinterpret_cast<const float4*>(wrow + c + 4);
#pragma unroll
      for (int j = 0; j < TT; ++j) {
        const int t = min(t0 + j, T - 1);
        xv[q][j] = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * d + c);
      }
    }
#pragma unroll
    for (int q = 0; q < kSteps; ++q) {
      if (base0 + q * 512 >= c_end) break;
#pragma unroll
      for (int j = 0; j < TT; ++j) {
        float a = acc[j];
        a = fmaf(bf16_to_f32(xv[q][j].x & 0xffffu), w0[q].x, a);
        a = fmaf(bf16_to_f32(xv[q][j].x >> 16), w0[q].y, a);
        a = fmaf(bf16_to_f32(xv[q][j].y & 0xffffu), w0[q].z, a);
        a = fmaf(bf16_to_f32(xv[q][j].y >> 16), w0[q].w, a);
        a = fmaf(bf16_to_f32(xv[q][j].z & 0xffffu), w1[q].x, a);
        a = fmaf(bf16_to_f32(xv[q][j].z >> 16), w1[q].y, a);
        a = fmaf(bf16_to_f32(xv[q][j].w & 0xffffu), w1[q].z, a);
        a = fmaf(bf16_to_f32(xv[q][j].w >> 16), w1[q].w, a);
        acc[j] = a;
      }
    }
  }
  const float r = wave_reduce_multi<TT>(acc);
  const int j = reduce_multi_index<TT>(lane);
  if (reduce_multi_writer<TT>(lane)) s_part[wave * TT + j] = r;
  __syncthreads();
  if (wave == 0 && reduce_multi_writer<TT>(lane) && t0 + j < T) {
    const float l = ((s_part[j] + s_part[TT + j]) + s_part[2 * TT + j]) + s_part[3 * TT + j];
    const size_t o = static_cast<size_t>(t0 + j) * E + e;
    logits[o] = l;
    if (keys != nullptr) score_key(l, bias, e, scores[o], keys[o]);
  }
}

// Top-k selection by one wave over the E keys and scores staged in LDS
// (private to the wave): k rounds of a wave arg-max over packed (key, ~index)
// retire one expert each. The bias only ranks; the weights are the selected
// unbiased scores renormalised (1/k if their sum is 0). Lane j < k receives
// the j-th id and weight.
__device__ __forceinline__ void topk_rounds(uint64_t* s_key, const float* s_s, int E, int k, float routed_scale,
                                            int& id_out, float& w_out) {
  const int lane = lane_id();
  int sel_e = 0;
  float sel_s = 0.0f, total = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
    for (int e = lane; e < E; e += 64) best = s_key[e] > best ? s_key[e] : best;
    best = wave_max_u64(best);
    const int e = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
    const float sj = s_s[e];
    if ((e & 63) == lane) s_key[e] = 0;
    total += sj;
    if (lane == j) {
      sel_e = e;
      sel_s = sj;
    }
  }
  id_out = sel_e;
  w_out = (total > 0.0f ? sel_s / total : 1.0f / static_cast<float>(k)) * routed_scale;
}

// Top-k selection by one wave with the keys and scores of up to 256 experts
// held in registers (expert e = lane + 64 i): no LDS round trip per round.
// Same selection order and arithmetic as topk_rounds.
__device__ __forceinline__ void topk_rounds_reg(uint64_t (&key)[4], const float (&sc)[4], int k, float routed_scale,
                                                int& id_out, float& w_out) {
  const int lane = lane_id();
  int sel_e = 0;
  float sel_s = 0.0f, total = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0] > key[1] ? key[0] : key[1];
    const uint64_t b2 = key[2] > key[3] ? key[2] : key[3];
    best = b2 > best ? b2 : best;
    best = wave_max_u64(best);
    const int e = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
    float mine = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (key[i] == best) {
        mine = sc[i];
        key[i] = 0;
      }
    }
    const float sj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), e & 63));
    total += sj;
    if (lane == j) {
      sel_e = e;
      sel_s = sj;
    }
  }
  id_out = sel_e;
  w_out = (total > 0.0f ? sel_s / total : 1.0f / static_cast<float>(k)) * routed_scale;
}

// Top-k of one token by one wave from its logits (scores and keys computed
// here, staged in LDS: s_key E uint64, s_s E floats; also stored to keys_t /
// scores_t when those are given).
__device__ __forceinline__ void topk_wave(const float* __restrict__ logits_t, const float* __restrict__ bias, int E,
                                          int k, float routed_scale, uint64_t* s_key, float* s_s, int& id_out,
                                          float& w_out, uint64_t* __restrict__ keys_t = nullptr,
                                          float* __restrict__ scores_t = nullptr) {
  for (int e = lane_id(); e < E; e += 64) {
    score_key(logits_t[e], bias, e, s_s[e], s_key[e]);
    if (keys_t != nullptr) {
      keys_t[e] = s_key[e];
      scores_t[e] = s_s[e];
    }
  }
  topk_rounds(s_key, s_s, E, k, routed_scale, id_out, w_out);
}

}  // namespace qsmoe
