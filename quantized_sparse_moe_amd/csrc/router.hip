// Router kernels: fp32 gate logits, sqrtsoftplus scoring with per-expert bias
// and wave-level top-k, and the tid2eid hash route.
//
// The gate is computed in fp32 from the bf16 activations (mlx-lm PR "Add
// DeepSeek-v4 (Flash/Pro)", cross-reference table row "MoE gate dtype");
// scores are sqrt(softplus(l)) ("mlx-community / DeepSeek-V4-Flash-4bit",
// "Architecture") evaluated in the overflow-free logaddexp form the same PR's
// review notes ask for.
#include "common.hpp"
#include "kernels.hpp"

namespace qsmoe {

// ---------------------------------------------------------------------------
// Logits, few tokens: one wave per (expert, TT tokens); lanes stride the
// hidden dimension 8 values at a time (32 B of Wr, 16 B of x per token).
// ---------------------------------------------------------------------------
template <int TT>
__global__ __launch_bounds__(256) void k_logits_gemv(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                     int T, int E, int d, float* __restrict__ logits) {
  const int lane = lane_id();
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t0 = blockIdx.y * TT;
  if (e >= E) return;
  float acc[TT];
#pragma unroll
  for (int j = 0; j < TT; ++j) acc[j] = 0.0f;
  const float* wrow = wr + static_cast<size_t>(e) * d;
  for (int base = lane * 8; base < d; base += 64 * 8) {
    const float4 w0 = *reinterpret_cast<const float4*>(wrow + base);
    const float4 w1 = *reinterpret_cast<const float4*>(wrow + base + 4);
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      const int t = min(t0 + j, T - 1);
      const uint4 xv = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * d + base);
      float a = acc[j];
      a = fmaf(bf16_to_f32(xv.x & 0xffffu), w0.x, a);
      a = fmaf(bf16_to_f32(xv.x >> 16), w0.y, a);
      a = fmaf(bf16_to_f32(xv.y & 0xffffu), w0.z, a);
      a = fmaf(bf16_to_f32(xv.y >> 16), w0.w, a);
      a = fmaf(bf16_to_f32(xv.z & 0xffffu), w1.x, a);
      a = fmaf(bf16_to_f32(xv.z >> 16), w1.y, a);
      a = fmaf(bf16_to_f32(xv.w & 0xffffu), w1.z, a);
      a = fmaf(bf16_to_f32(xv.w >> 16), w1.w, a);
      acc[j] = a;
    }
  }
  const float r = wave_reduce_multi<TT>(acc);
  const int j = reduce_multi_index<TT>(lane);
  if (reduce_multi_writer<TT>(lane) && t0 + j < T) logits[static_cast<size_t>(t0 + j) * E + e] = r;
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

// Order-preserving map of an fp32 key and expert index to a 64-bit value:
// larger key first, equal keys -> lower index first.
__device__ __forceinline__ uint64_t pack_key(float key, int e) {
  const uint32_t u = __float_as_uint(key);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(0xffffffffu - static_cast<uint32_t>(e));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token. Each lane holds EPL experts (e = lane + 64 i).
// k rounds of a wave arg-max over packed (key, ~index); the winner's owner
// retires it. Weights are the selected unbiased scores renormalised.
// ---------------------------------------------------------------------------
template <int EPL>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const float* __restrict__ bias,
                                              int T, int E, int k, float routed_scale, int32_t* __restrict__ ids,
                                              float* __restrict__ w) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float s[EPL];
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      s[i] = sqrtsoftplus(logits[static_cast<size_t>(t) * E + e]);
      key[i] = pack_key(s[i] + (bias ? bias[e] : 0.0f), e);
    } else {
      s[i] = 0.0f;
      key[i] = 0;
    }
  }
  int sel_e = 0;
  float sel_s = 0.0f, total = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
    float se = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (key[i] == best) {
        se = s[i];
        key[i] = 0;
      }
    }
    const float sj = __shfl(se, e & 63);
    total += sj;
    if (lane == j) {
      sel_e = e;
      sel_s = sj;
    }
  }
  if (lane < k) {
    const float wj = total > 0.0f ? sel_s / total : 1.0f / static_cast<float>(k);
    ids[static_cast<size_t>(t) * k + lane] = sel_e;
    w[static_cast<size_t>(t) * k + lane] = wj * routed_scale;
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
  if (T > 16 && d % 32 == 0) {
    dim3 grid((E + 63) / 64, (T + 63) / 64);
    hipLaunchKernelGGL(k_logits_tiled, grid, dim3(256), 0, s, x, wr, T, E, d, logits);
  } else if (T == 1) {
    hipLaunchKernelGGL(k_logits_gemv<1>, dim3((E + 3) / 4, T), dim3(256), 0, s, x, wr, T, E, d, logits);
  } else if (T == 2) {
    hipLaunchKernelGGL(k_logits_gemv<2>, dim3((E + 3) / 4, 1), dim3(256), 0, s, x, wr, T, E, d, logits);
  } else {
    hipLaunchKernelGGL(k_logits_gemv<4>, dim3((E + 3) / 4, (T + 3) / 4), dim3(256), 0, s, x, wr, T, E, d, logits);
  }
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, const float* bias, int T, int E, int k, float routed_scale,
                              int32_t* ids, float* w, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(k_topk<1>, grid, block, 0, s, logits, bias, T, E, k, routed_scale, ids, w);
  else if (E <= 128)
    hipLaunchKernelGGL(k_topk<2>, grid, block, 0, s, logits, bias, T, E, k, routed_scale, ids, w);
  else if (E <= 256)
    hipLaunchKernelGGL(k_topk<4>, grid, block, 0, s, logits, bias, T, E, k, routed_scale, ids, w);
  else if (E <= 512)
    hipLaunchKernelGGL(k_topk<8>, grid, block, 0, s, logits, bias, T, E, k, routed_scale, ids, w);
  else
    hipLaunchKernelGGL(k_topk<16>, grid, block, 0, s, logits, bias, T, E, k, routed_scale, ids, w);
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
