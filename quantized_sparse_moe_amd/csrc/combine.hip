// Weighted combine back to token order, without atomics: each output element
// has exactly one writer, which gathers the token's k expert rows (written in
// assignment order t*k + j) in fixed j order and then adds the shared expert.
// The router weights multiply the expert outputs ("DeepSeek-V4-Flash-MLX-4bit",
// "REAP-pruned builds": router weight times expert output is each expert's
// contribution).
#include "common.hpp"
#include "kernels.hpp"

namespace qsmoe {

template <int OUT_F32>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y_slot, const float* __restrict__ w,
                                                 const float* __restrict__ y_shared, int T, int k, int d,
                                                 void* __restrict__ out) {
  const int nblk = (d / 4 + 255) / 256;
  const int t = blockIdx.x / nblk;
  const int i = ((blockIdx.x % nblk) * 256 + threadIdx.x) * 4;
  if (i >= d) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* base = y_slot + static_cast<size_t>(t) * k * d + i;
  for (int j = 0; j < k; ++j) {
    const float wj = w[static_cast<size_t>(t) * k + j];
    const float4 v = *reinterpret_cast<const float4*>(base + static_cast<size_t>(j) * d);
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  if (y_shared) {
    const float4 v = *reinterpret_cast<const float4*>(y_shared + static_cast<size_t>(t) * d + i);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  if constexpr (OUT_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + static_cast<size_t>(t) * d + i) = acc;
  } else {
    uint2 o;
    o.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
    o.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + static_cast<size_t>(t) * d + i) = o;
  }
}

hipError_t launch_combine(const float* y_slot, const float* w, const float* y_shared, int T, int k, int d,
                          int out_f32, void* out, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((d / 4 + 255) / 256) * T), block(256);
  if (out_f32)
    QSMOE_LAUNCH(k_combine<1>, grid, block, 0, s, y_slot, w, y_shared, T, k, d, out);
  else
    QSMOE_LAUNCH(k_combine<0>, grid, block, 0, s, y_slot, w, y_shared, T, k, d, out);
  return hipGetLastError();
}

__global__ void k_fill_i32(int32_t* p, int32_t v, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, int n, hipStream_t s) {
  QSMOE_LAUNCH(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace qsmoe
