// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsmoe {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// e8m0 exponent byte -> 2^(b - 127) as fp32 (b = 0 is the subnormal 2^-127,
// b = 255 is NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  uint32_t bits = b == 0 ? 0x00400000u : (b == 255 ? 0x7fc00000u : (b << 23));
  return __uint_as_float(bits);
}

__device__ __forceinline__ float sqrtsoftplus(float l) {
  return sqrtf(fmaxf(l, 0.0f) + log1pf(expf(-fabsf(l))));
}

// Workgroup barrier that orders LDS accesses only: global loads issued
// before it stay in flight (a plain __syncthreads also waits for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
// The same with the division as a reciprocal (at most ~3 fp32 ulps apart,
// 8 fewer instructions); below z = -64, where the reciprocal of 1 + e^-z
// would leave the normal range, the exact division.
__device__ __forceinline__ float silu_fast(float z) {
  const float d = 1.0f + expf(-z);
  if (z > -64.0f) return z * __builtin_amdgcn_rcpf(d);
  return z / d;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Exchange with a partner lane that differs in bit log2(mask): masks 1 and 2
// are quad permutations, 4 and 8 the half-row / row mirrors (which flip the
// target bit too), 16 and 32 go through ds_bpermute. For sums the pairing
// only needs to flip the bit; the six pairings together reach all 64 lanes.
__device__ __forceinline__ float xchg(float v, int mask) {
  switch (mask) {
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
    case 4: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
    case 8: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));
    default: return __shfl_xor(v, mask);
  }
}

// Reduce N values (N a power of two, N <= 64) across the wave at once.
// Each halving step keeps half of the values per lane and exchanges the other
// half with the partner lane, so the cost is about N + 6 shuffles instead of
// 6N. On return every lane holds the wave total of value index
// reduce_multi_index<N>(lane).
template <int N>
__device__ __forceinline__ float wave_reduce_multi(const float (&v)[N]) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "the halving exchange needs a power-of-two count");
  float cur[N];
#pragma unroll
  for (int i = 0; i < N; ++i) cur[i] = v[i];
  const int lane = lane_id();
  int mask = 32;
#pragma unroll
  for (int n = N; n > 1; n >>= 1) {
    const bool upper = (lane & mask) != 0;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      float send = upper ? cur[i] : cur[i + n / 2];
      float keep = upper ? cur[i + n / 2] : cur[i];
      cur[i] = keep + xchg(send, mask);
    }
    mask >>= 1;
  }
  float r = cur[0];
#pragma unroll
  for (; mask >= 1; mask >>= 1) r += xchg(r, mask);
  return r;
}

template <int N>
__device__ __forceinline__ int reduce_multi_index(int lane) {
  int idx = 0, mask = 32;
#pragma unroll
  for (int n = N; n > 1; n >>= 1) {
    if (lane & mask) idx += n / 2;
    mask >>= 1;
  }
  return idx;
}

// The lanes that write value index reduce_multi_index<N>: the lowest lane of
// each group of 64/N lanes.
template <int N>
__device__ __forceinline__ bool reduce_multi_writer(int lane) {
  return (lane & (64 / N - 1)) == 0;
}

// The b-th (0-based) expert with a non-empty bucket, or -1. Every lane of the
// wave gets the same answer.
__device__ __forceinline__ int find_bucket_expert(const int32_t* __restrict__ offsets, int E, int b) {
  const int lane = lane_id();
  int base = 0;
  for (int e0 = 0; e0 < E; e0 += kWave) {
    const int e = e0 + lane;
    const bool nonempty = e < E && offsets[e + 1] > offsets[e];
    const uint64_t m = __ballot(nonempty);
    const int cnt = __popcll(m);
    if (b < base + cnt) {
      const int want = b - base;
      const int before = __popcll(m & ((1ull << lane) - 1ull));
      const uint64_t hit = __ballot(nonempty && before == want);
      return e0 + __ffsll(static_cast<unsigned long long>(hit)) - 1;
    }
    base += cnt;
  }
  return -1;
}

__device__ __forceinline__ void set_device_error(int32_t* err, int code) {
  if (err) atomicOr(err, code);
}

}  // namespace qsmoe
