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
// Logits, few tokens: one workgroup per (expert, TT tokens), split-K over
// its four waves.
// ---------------------------------------------------------------------------
template <int TT>
__global__ __launch_bounds__(256) void k_logits_gemv(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                     int T, int E, int d, float* __restrict__ logits) {
  __shared__ float s_part[4 * TT];
  logits_wg<TT>(x, wr, T, E, d, blockIdx.x, blockIdx.y * TT, logits, s_part);
}

// ---------------------------------------------------------------------------
// Logits, many tokens: MFMA with the fp32 gate split into three bf16 terms.
//
// Truncating w to its top 16 bits gives hi (exact bf16); the remainder w - hi
// is exact in fp32 and carries at most 16 significant bits, so a second
// truncation gives mid and a third remainder lo that is itself exact in bf16
// (8 + 8 + 8 bits cover fp32's 24-bit significand). Every x*hi, x*mid, x*lo
// product of two bf16 values is exact in fp32, so three bf16 MFMAs with fp32
// accumulation give x.w to fp32 accumulation error, as an fp32 dot product
// would, at bf16 matrix-core rate.
//
// Workgroup: MB*16 tokens x 64 experts; its four waves each take every fourth
// 32-wide K step over the whole tile and the partial tiles are added in wave
// order through LDS, so the result does not depend on timing. Fragments are
// loaded straight from global memory in the V_MFMA_F32_16X16X32_BF16 operand
// layout (lane l: row l % 16, inputs 8 (l / 16) .. + 7 of the step).
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

__device__ __forceinline__ void split3_bf16x8(const u32x4_t& w0, const u32x4_t& w1, bf16x8_t& hi, bf16x8_t& mid,
                                              bf16x8_t& lo) {
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t bits = j < 4 ? w0[j] : w1[j - 4];
    const uint32_t hb = bits & 0xffff0000u;
    const float r1 = __uint_as_float(bits) - __uint_as_float(hb);
    const uint32_t mb = __float_as_uint(r1) & 0xffff0000u;
    const float r2 = r1 - __uint_as_float(mb);
    const uint32_t lb = __float_as_uint(r2) >> 16;  // exact: r2 has at most 8 significant bits
    if (j & 1) {
      h[j >> 1] |= hb;
      m[j >> 1] |= mb;
      l[j >> 1] |= lb << 16;
    } else {
      h[j >> 1] = hb >> 16;
      m[j >> 1] = mb >> 16;
      l[j >> 1] = lb;
    }
  }
  hi = __builtin_bit_cast(bf16x8_t, h);
  mid = __builtin_bit_cast(bf16x8_t, m);
  lo = __builtin_bit_cast(bf16x8_t, l);
}

template <int MB>
__global__ __launch_bounds__(256) void k_logits_mfma(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                     int T, int E, int d, float* __restrict__ logits) {
  constexpr int NB = 4;  // 16-expert blocks per workgroup
  __shared__ f32x4_t s_part[3][MB * NB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int t0 = blockIdx.y * (MB * 16), e0 = blockIdx.x * (NB * 16);
  const uint16_t* xa[MB];
  const float* wb[NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) xa[mb] = x + static_cast<size_t>(min(t0 + mb * 16 + r16, T - 1)) * d + 8 * g;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wb[nb] = wr + static_cast<size_t>(min(e0 + nb * 16 + r16, E - 1)) * d + 8 * g;

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nsteps = d / 32;
  for (int ks = wave; ks < nsteps; ks += 4) {
    const int k0 = ks * 32;
    bf16x8_t af[MB];
    u32x4_t bw[NB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) af[mb] = *reinterpret_cast<const bf16x8_t*>(xa[mb] + k0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      bw[nb][0] = *reinterpret_cast<const u32x4_t*>(wb[nb] + k0);
      bw[nb][1] = *reinterpret_cast<const u32x4_t*>(wb[nb] + k0 + 4);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      bf16x8_t hi, mid, lo;
      split3_bf16x8(bw[nb][0], bw[nb][1], hi, mid, lo);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], lo, acc[mb][nb], 0, 0, 0);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], mid, acc[mb][nb], 0, 0, 0);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], hi, acc[mb][nb], 0, 0, 0);
      }
    }
  }

  // fixed-order reduction of the four waves' partial tiles
  if (wave > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s_part[wave - 1][mb * NB + nb][lane] = acc[mb][nb];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4_t v = acc[mb][nb];
#pragma unroll
      for (int w = 0; w < 3; ++w) v += s_part[w][mb * NB + nb][lane];
      const int e = e0 + nb * 16 + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + mb * 16 + 4 * g + i;
        if (t < T && e < E) logits[static_cast<size_t>(t) * E + e] = v[i];
      }
    }
  }
}

// Mid-size batches (16 < T <= 256): the tile above leaves most of the chip
// idle (4 x T/16 workgroups), so here a workgroup takes 16 tokens x 16
// experts and its 16 waves split K (wave w takes K steps w, w + 16, ...). A
// wave issues the loads of all its steps (up to kLogitsU) before the first
// MFMA, so one memory round trip covers its share; steps past the end get a
// zero A fragment. Partial tiles are added in wave order through LDS.
constexpr int kLogitsWaves = 16;
constexpr int kLogitsU = 8;

__global__ __launch_bounds__(kLogitsWaves * 64) void k_logits_mfma_ksplit(const uint16_t* __restrict__ x,
                                                                          const float* __restrict__ wr, int T,
                                                                          int E, int d,
                                                                          float* __restrict__ logits) {
  __shared__ f32x4_t s_part[kLogitsWaves - 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int t0 = blockIdx.y * 16, e0 = blockIdx.x * 16;
  const uint16_t* xa = x + static_cast<size_t>(min(t0 + r16, T - 1)) * d + 8 * g;
  const float* wb = wr + static_cast<size_t>(min(e0 + r16, E - 1)) * d + 8 * g;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nsteps = d / 32;
  for (int base = wave; base < nsteps; base += kLogitsWaves * kLogitsU) {
    bf16x8_t af[kLogitsU];
    u32x4_t bw[kLogitsU][2];
#pragma unroll
    for (int u = 0; u < kLogitsU; ++u) {
      const int k0 = min(base + u * kLogitsWaves, nsteps - 1) * 32;
      af[u] = *reinterpret_cast<const bf16x8_t*>(xa + k0);
      bw[u][0] = *reinterpret_cast<const u32x4_t*>(wb + k0);
      bw[u][1] = *reinterpret_cast<const u32x4_t*>(wb + k0 + 4);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the first MFMA
#pragma unroll
    for (int u = 0; u < kLogitsU; ++u) {
      const bool ok = base + u * kLogitsWaves < nsteps;
      const bf16x8_t a = ok ? af[u] : bf16x8_t{};
      bf16x8_t hi, mid, lo;
      split3_bf16x8(bw[u][0], bw[u][1], hi, mid, lo);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, lo, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, mid, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hi, acc, 0, 0, 0);
    }
  }
  if (wave > 0) s_part[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kLogitsWaves - 1; ++w) acc += s_part[w][lane];
  const int e = e0 + r16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * g + i;
    if (t < T && e < E) logits[static_cast<size_t>(t) * E + e] = acc[i];
  }
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token (keys staged in LDS, 12 bytes per expert); every
// expert's packed key and score also go to `keys` / `scores` when given.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const float* __restrict__ bias,
                                              int T, int E, int k, float routed_scale, int32_t* __restrict__ ids,
                                              float* __restrict__ w, uint64_t* __restrict__ keys,
                                              float* __restrict__ scores) {
  extern __shared__ uint64_t lds_keys[];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  uint64_t* s_key = lds_keys + static_cast<size_t>(wave) * E;
  float* s_s = reinterpret_cast<float*>(lds_keys + static_cast<size_t>(4) * E) + static_cast<size_t>(wave) * E;
  int id;
  float wt;
  const size_t o = static_cast<size_t>(t) * E;
  topk_wave(logits + o, bias, E, k, routed_scale, s_key, s_s, id, wt, keys ? keys + o : nullptr,
            scores ? scores + o : nullptr);
  if (lane < k) {
    ids[static_cast<size_t>(t) * k + lane] = id;
    w[static_cast<size_t>(t) * k + lane] = wt;
  }
}

// ---------------------------------------------------------------------------
// Hash route: one workgroup per token. ids from tid2eid[token], logits of
// those k experts (the 4 waves take interleaved 512-input slices of the
// hidden dimension and their partial sums meet in LDS), sqrtsoftplus,
// renormalised weights. Out-of-range token ids or table entries set the
// device error word; the id becomes 0 and the token's weights 0 so every
// access stays in bounds. (One wave per token walked its 6 router rows in
// 8 dependent rounds: 24 us for 512 tokens.)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_hash(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                              const int32_t* __restrict__ token_ids,
                                              const int32_t* __restrict__ tid2eid, int T, int E, int k, int d,
                                              int vocab, float routed_scale, int32_t* __restrict__ ids,
                                              float* __restrict__ w, int32_t* err) {
  __shared__ float s_part[4][8];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int t = blockIdx.x;
  int tok = token_ids[t];
  bool ok = true;
  if (tok < 0 || tok >= vocab) {
    if (threadIdx.x == 0) set_device_error(err, 1);
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
        if (threadIdx.x == 0) set_device_error(err, 2);
        e = 0;
        ok = false;
      }
      eid[j] = e;
    }
  }
  const uint16_t* xr = x + static_cast<size_t>(t) * d;
#pragma unroll 2
  for (int base = threadIdx.x * 8; base < d; base += 256 * 8) {
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
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = wave_sum(acc[j]);
    if (lane == 0) s_part[wave][j] = p;
  }
  __syncthreads();
  if (wave != 0) return;
  float s[8], total = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float tot = (s_part[0][j] + s_part[1][j]) + (s_part[2][j] + s_part[3][j]);
    s[j] = j < k ? sqrtsoftplus(tot) : 0.0f;
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
// Largest T for the K-split logits kernel (16 x 16 tiles, K over 16 waves);
// above it the 64 x 64-tile kernel. Measured: T=512 29 vs 50 us, T=4096 215
// vs 58 us.
constexpr int kLogitsKsplitMaxT = 512;
hipError_t launch_router_logits(const uint16_t* x, const float* wr, int T, int E, int d, float* logits,
                                hipStream_t s) {
  if (T > kLogitsKsplitMaxT) {
    QSMOE_LAUNCH(k_logits_mfma<4>, dim3((E + 63) / 64, (T + 63) / 64), dim3(256), 0, s, x, wr, T, E, d,
                       logits);
  } else if (T > 16) {
    QSMOE_LAUNCH(k_logits_mfma_ksplit, dim3((E + 15) / 16, (T + 15) / 16), dim3(kLogitsWaves * 64), 0, s, x, wr,
                 T, E, d, logits);
  } else if (T == 1) {
    QSMOE_LAUNCH(k_logits_gemv<1>, dim3(E, 1), dim3(256), 0, s, x, wr, T, E, d, logits);
  } else if (T == 2) {
    QSMOE_LAUNCH(k_logits_gemv<2>, dim3(E, 1), dim3(256), 0, s, x, wr, T, E, d, logits);
  } else {
    QSMOE_LAUNCH(k_logits_gemv<4>, dim3(E, (T + 3) / 4), dim3(256), 0, s, x, wr, T, E, d, logits);
  }
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, const float* bias, int T, int E, int k, float routed_scale,
                              int32_t* ids, float* w, uint64_t* keys, float* scores, hipStream_t s) {
  const size_t lds = static_cast<size_t>(4) * E * (sizeof(uint64_t) + sizeof(float));
  QSMOE_LAUNCH(k_topk, dim3((T + 3) / 4), dim3(256), lds, s, logits, bias, T, E, k, routed_scale, ids, w, keys,
               scores);
  return hipGetLastError();
}

hipError_t launch_router_hash(const uint16_t* x, const float* wr, const int32_t* token_ids,
                              const int32_t* tid2eid, int T, int E, int k, int d, int vocab, float routed_scale,
                              int32_t* ids, float* w, int32_t* err, hipStream_t s) {
  if (T == 0) return hipSuccess;
  QSMOE_LAUNCH(k_hash, dim3(T), dim3(256), 0, s, x, wr, token_ids, tid2eid, T, E, k, d, vocab, routed_scale, ids,
               w, err);
  return hipGetLastError();
}

}  // namespace qsmoe
