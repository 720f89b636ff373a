// Pieces shared by the fused small-batch (decode) kernels: their limits, the
// per-token head that selects each token's experts (the top-k from the
// router's keys, or the tid2eid hash route; every decode kernel selects
// bit-identical ids) and the row helpers of the down projection.
#pragma once

#include "ffn_core.hpp"
#include "router_core.hpp"

namespace qsmoe {

constexpr int kDecMaxT = 4;
constexpr int kDecMaxK = 8;
constexpr uint32_t kLdsSpinLimit = 1u << 24;  // polls of a workgroup-local flag before giving up
// Hash route of token t by one wave (the pages' tid2eid table, as k_hash):
// lane j < k takes expert tid2eid[token][j]; the weights are the launch-1
// scores of those experts renormalised over the k slots (summed in slot
// order). A token id or table entry out of range sets the device error word
// (publish: one workgroup only), the id becomes 0 and the token's weights 0.
__device__ __forceinline__ void dec_hash_head(const DecodeArgs& a, int t, bool publish, int& id, float& wt) {
  const int lane = lane_id();
  int tok = a.token_ids[t];
  bool ok = true;
  if (tok < 0 || tok >= a.vocab) {
    if (publish && lane == 0) set_device_error(a.err, 1);
    tok = 0;
    ok = false;
  }
  int e = lane < a.k ? a.tid2eid[static_cast<size_t>(tok) * a.k + lane] : 0;
  const bool bad = lane < a.k && (e < 0 || e >= a.E);
  if (__ballot(bad) != 0) {
    if (publish && lane == 0) set_device_error(a.err, 2);
    ok = false;
  }
  e = (bad || lane >= a.k) ? 0 : e;
  const float s = lane < a.k ? a.scores[static_cast<size_t>(t) * a.E + e] : 0.0f;
  float total = 0.0f;
  for (int j = 0; j < a.k; ++j) total += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), j));
  id = e;
  wt = ok ? (total > 0.0f ? s / total : 1.0f / static_cast<float>(a.k)) * a.routed_scale : 0.0f;
}

// Ids and weights of token `t` by one wave (lane j < k receives slot j):
// the top-k of launch 1's keys (same selection as moe_route) or the hash
// route. `publish` marks the one workgroup that stores errors.
__device__ __forceinline__ void dec_token_head(const DecodeArgs& a, int t, bool publish, int& id, float& wt) {
  if (a.hash) {
    dec_hash_head(a, t, publish, id, wt);
    return;
  }
  const int lane = lane_id();
  uint64_t key[4];
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    const bool ok = e < a.E;
    const size_t o = static_cast<size_t>(t) * a.E + (ok ? e : 0);
    key[i] = a.keys[o];
    sc[i] = a.scores[o];
    key[i] = ok ? key[i] : 0;
  }
  topk_rounds_reg(key, sc, a.k, a.routed_scale, id, wt);
}

// Partial (this lane's) dot of one row with token j's activations.
template <int F, int B, int CPL, int NT>
__device__ __forceinline__ float row_dot_one(const RowRegs<F, B, CPL>& r, const XRegs<F, B, CPL, NT>& xr, int j,
                                             int lane, int nchunks) {
  using C = Codec<F, B>;
  float acc = 0.0f;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const bool ok = lane + 64 * m < nchunks;
    uint32_t p[16];
    C::pairs(r.w[m], p);
    float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      d0 = dot2_bf16(p[i], xr.px[j][m][i], d0);
      d1 = dot2_bf16(p[i + 1], xr.px[j][m][i + 1], d1);
    }
    const float d = d0 + d1;
    if constexpr (F == 0) {
      const float s = ok ? f16_to_f32(static_cast<uint16_t>(r.s[m])) : 0.0f;
      const float b = ok ? f16_to_f32(static_cast<uint16_t>(r.b[m])) : 0.0f;
      acc += s * d + (b - C::kOff * s) * xr.xs[j][m];
    } else {
      acc += d * (ok ? e8m0_to_f32(r.s[m]) : 0.0f);
    }
  }
  return acc;
}

// The k selected experts' down rows of one output row, as loaded by a wave.
template <int F, int B, int K>
struct RoutedRows {
  RowRegs<F, B, 1> r[K];
};

template <int F, int B, int K>
__device__ __forceinline__ void dec_load_routed(RoutedRows<F, B, K>& b, const QMat (&qd)[K], int r, int lane,
                                                int nchunks) {
#pragma unroll
  for (int j = 0; j < K; ++j) load_row<F, B, 1>(b.r[j], qd[j], r, lane, nchunks);
}

}  // namespace qsmoe
