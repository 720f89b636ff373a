// Router kernels: fp32 gate logits, sqrtsoftplus scoring with per-expert bias
// and wave-level top-k, and the tid2eid hash route.
//
// The gate is computed in fp32 from the bf16 activations (mlx-lm PR "Add
// DeepSeek-v4 (Flash/Pro)", cross-reference table row "MoE gate dtype");
// scores are sqrt(softplus(l)) ("mlx-community / DeepSeek-V4-Flash-4bit",
// "Architecture") evaluated in the overflow-free logaddexp form the same PR's
// review notes ask for.
#include "kernels.hpp"
#include "router_core.hpp"

namespace qsmoe {

// ---------------------------------------------------------------------------
// Logits, few tokens: one wave per (expert, TT tokens).
// ---------------------------------------------------------------------------
template <int TT>
__global__ __launch_bounds__(256) void k_logits_gemv(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                     int T, int E, int d, float* __restrict__ logits) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e < E) logits_wave<TT>(x, wr, T, E, d, e, blockIdx.y * TT, logits);
}

// ---------------------------------------------------------------------------
// Logits, many tokens: 64 tokens x 64 experts per workgroup, K step 32 staged
// through LDS in fp32, 4x4 outputs per thread. Requires d % 32 == 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_logits_tiled(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                      int T, int E, int d, float* __restrict__ logits) {
  __shared__ float xs[32][64 + 4];
  __shared__ float ws[32][64 + 4];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.y * 64, e0 = blockIdx.x * 64;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  const int lr = tid >> 2, lc = (tid & 3) * 8;  // loader: row (token / expert), 8 columns
  const int lt = min(t0 + lr, T - 1), le = min(e0 + lr, E - 1);
  for (int k0 = 0; k0 < d; k0 += 32) {
    const uint4 xv = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(lt) * d + k0 + lc);
    const float4 w0 = *reinterpret_cast<const float4*>(wr + static_cast<size_t>(le) * d + k0 + lc);
    const float4 w1 = *reinterpret_cast<const float4*>(wr + static_cast<size_t>(le) * d + k0 + lc + 4);
    __syncthreads();
    xs[lc + 0][lr] = bf16_to_f32(xv.x & 0xffffu);
    xs[lc + 1][lr] = bf16_to_f32(xv.x >> 16);
    xs[lc + 2][lr] = bf16_to_f32(xv.y & 0xffffu);
    xs[lc + 3][lr] = bf16_to_f32(xv.y >> 16);
    xs[lc + 4][lr] = bf16_to_f32(xv.z & 0xffffu);
    xs[lc + 5][lr] = bf16_to_f32(xv.z >> 16);
    xs[lc + 6][lr] = bf16_to_f32(xv.w & 0xffffu);
    xs[lc + 7][lr] = bf16_to_f32(xv.w >> 16);
    ws[lc + 0][lr] = w0.x;
    ws[lc + 1][lr] = w0.y;
    ws[lc + 2][lr] = w0.z;
    ws[lc + 3][lr] = w0.w;
    ws[lc + 4][lr] = w1.x;
    ws[lc + 5][lr] = w1.y;
    ws[lc + 6][lr] = w1.z;
    ws[lc + 7][lr] = w1.w;
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(&xs[kk][ty * 4]);
      const float4 b = *reinterpret_cast<const float4*>(&ws[kk][tx * 4]);
      const float av[4] = {a.x, a.y, a.z, a.w};
      const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) logits[static_cast<size_t>(t) * E + e] = acc[i][j];
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token (keys staged in LDS, 12 bytes per expert).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const float* __restrict__ bias,
                                              int T, int E, int k, float routed_scale, int32_t* __restrict__ ids,
                                              float* __restrict__ w) {
  extern __shared__ uint64_t lds_keys[];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  uint64_t* s_key = lds_keys + static_cast<size_t>(wave) * E;
  float* s_s = reinterpret_cast<float*>(lds_keys + static_cast<size_t>(4) * E) + static_cast<size_t>(wave) * E;
  int id;
  float wt;
  topk_wave(logits + static_cast<size_t>(t) * E, bias, E, k, routed_scale, s_key, s_s, id, wt);
  if (lane < k) {
    ids[static_cast<size_t>(t) * k + lane] = id;
    w[static_cast<size_t>(t) * k + lane] = wt;
  }
}

// ---------------------------------------------------------------------------
// Hash route: one wave per token. ids from tid2eid[token], logits of those k
// experts, sqrtsoftplus, renormalised weights. Out-of-range token ids or
// table entries set the device error word; the id becomes 0 and the token's
// weights 0 so every access stays in bounds.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_hash(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                              const int32_t* __restrict__ token_ids,
                                              const int32_t* __restrict__ tid2eid, int T, int E, int k, int d,
                                              int vocab, float routed_scale, int32_t* __restrict__ ids,
                                              float* __restrict__ w, int32_t* err) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int tok = token_ids[t];
  bool ok = true;
  if (tok < 0 || tok >= vocab) {
    if (lane == 0) set_device_error(err, 1);
    tok = 0;
    ok = false;
  }
  int eid[8];
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc[j] = 0.0f;
    eid[j] = 0;
    if (j < k) {
      int e = tid2eid[static_cast<size_t>(tok) * k + j];
      if (e < 0 || e >= E) {
        if (lane == 0) set_device_error(err, 2);
        e = 0;
        ok = false;
      }
      eid[j] = e;
    }
  }
  const uint16_t* xr = x + static_cast<size_t>(t) * d;
  for (int base = lane * 8; base < d; base += 64 * 8) {
    const uint4 xv = *reinterpret_cast<const uint4*>(xr + base);
    const float xf[8] = {bf16_to_f32(xv.x & 0xffffu), bf16_to_f32(xv.x >> 16), bf16_to_f32(xv.y & 0xffffu),
                         bf16_to_f32(xv.y >> 16),     bf16_to_f32(xv.z & 0xffffu), bf16_to_f32(xv.z >> 16),
                         bf16_to_f32(xv.w & 0xffffu), bf16_to_f32(xv.w >> 16)};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        const float* wrow = wr + static_cast<size_t>(eid[j]) * d + base;
        const float4 w0 = *reinterpret_cast<const float4*>(wrow);
        const float4 w1 = *reinterpret_cast<const float4*>(wrow + 4);
        float a = acc[j];
        a = fmaf(xf[0], w0.x, a);
        a = fmaf(xf[1], w0.y, a);
        a = fmaf(xf[2], w0.z, a);
        a = fmaf(xf[3], w0.w, a);
        a = fmaf(xf[4], w1.x, a);
        a = fmaf(xf[5], w1.y, a);
        a = fmaf(xf[6], w1.z, a);
        a = fmaf(xf[7], w1.w, a);
        acc[j] = a;
      }
    }
  }
  float tot[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) tot[j] = wave_sum(acc[j]);
  float s[8], total = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    s[j] = j < k ? sqrtsoftplus(tot[j]) : 0.0f;
    total += s[j];
  }
  if (lane < k) {
    float sj = 0.0f;
    int ej = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j == lane) {
        sj = s[j];
        ej = eid[j];
      }
    float wj = total > 0.0f ? sj / total : 1.0f / static_cast<float>(k);
    ids[static_cast<size_t>(t) * k + lane] = ej;
    w[static_cast<size_t>(t) * k + lane] = ok ? wj * routed_scale : 0.0f;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_router_logits(const uint16_t* x, const float* wr, int T, int E, int d, float* logits,
                                hipStream_t s) {
  if (T > 16) {
    dim3 grid((E + 63) / 64, (T + 63) / 64);
    hipLaunchKernelGGL(k_logits_tiled, grid, dim3(256), 0, s, x, wr, T, E, d, logits);
  } else if (T == 1) {
    hipLaunchKernelGGL(k_logits_gemv<1>, dim3((E + 3) / 4, 1), dim3(256), 0, s, x, wr, T, E, d, logits);
  } else if (T == 2) {
    hipLaunchKernelGGL(k_logits_gemv<2>, dim3((E + 3) / 4, 1), dim3(256), 0, s, x, wr, T, E, d, logits);
  } else {
    hipLaunchKernelGGL(k_logits_gemv<4>, dim3((E + 3) / 4, (T + 3) / 4), dim3(256), 0, s, x, wr, T, E, d, logits);
  }
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, const float* bias, int T, int E, int k, float routed_scale,
                              int32_t* ids, float* w, hipStream_t s) {
  const size_t lds = static_cast<size_t>(4) * E * (sizeof(uint64_t) + sizeof(float));
  hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), lds, s, logits, bias, T, E, k, routed_scale, ids, w);
  return hipGetLastError();
}

hipError_t launch_router_hash(const uint16_t* x, const float* wr, const int32_t* token_ids,
                              const int32_t* tid2eid, int T, int E, int k, int d, int vocab, float routed_scale,
                              int32_t* ids, float* w, int32_t* err, hipStream_t s) {
  hipLaunchKernelGGL(k_hash, dim3((T + 3) / 4), dim3(256), 0, s, x, wr, token_ids, tid2eid, T, E, k, d, vocab,
                     routed_scale, ids, w, err);
  return hipGetLastError();
}

}  // namespace qsmoe
