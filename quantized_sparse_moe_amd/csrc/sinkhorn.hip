// mHC mix matrices, an op beside the MoE layer (model card
// "mlx-community / DeepSeek-V4-Flash-4bit", section "Architecture": the
// residual stream is hc_mult = 4 parallel copies recombined by a
// doubly-stochastic, Sinkhorn-normalised mix matrix; mlx-lm pull request
// "Add DeepSeek-v4 (Flash/Pro)", review notes: unfused, the normalisation is
// a softmax followed by iterations of a sum and a division, ~40 launches per
// call). Per token: softmax over each row of the n x n logits, then `iters`
// rounds of dividing every column by its sum (+ eps) and then every row by
// its sum (+ eps). One lane per matrix element: a token's n x n lanes are
// consecutive within a wave (n * n divides 64), so a row sum is an xor
// shuffle over the n lanes of the row and a column sum one over the lanes n
// apart; the logits are read once (coalesced) and the result written once,
// in one launch. (One thread per token, its matrix in registers, ran each
// token's ~300 divisions in one dependent chain on 1/16 of the lanes: 10.4 us
// per 4096 tokens.)
#include "common.hpp"
#include "kernels.hpp"

namespace qsmoe {

template <int N>
__global__ __launch_bounds__(256) void k_mhc_sinkhorn(const float* logits, int64_t T, int iters, float eps,
                                                      float* out) {
  constexpr int NN = N * N;
  static_assert(64 % NN == 0, "a matrix's lanes lie in one wave");
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // element of logits[T][N][N]
  const bool valid = e < T * NN;  // whole matrices are valid or not: 256 % NN == 0
  float v = valid ? logits[e] : 0.0f;
  float mx = v;
#pragma unroll
  for (int o = 1; o < N; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  v = expf(v - mx);
  float s = v;
#pragma unroll
  for (int o = 1; o < N; o <<= 1) s += __shfl_xor(s, o);
  v = v / s;
  for (int it = 0; it < iters; ++it) {
    float c = v;
#pragma unroll
    for (int o = N; o < NN; o <<= 1) c += __shfl_xor(c, o);
    v = v / (c + eps);
    float r = v;
#pragma unroll
    for (int o = 1; o < N; o <<= 1) r += __shfl_xor(r, o);
    v = v / (r + eps);
  }
  if (valid) out[e] = v;
}

hipError_t launch_mhc_sinkhorn(const float* logits, int64_t T, int n, int iters, float eps, float* out,
                               hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((T * n * n + 255) / 256));
  if (n == 2)
    QSMOE_LAUNCH(k_mhc_sinkhorn<2>, grid, dim3(256), 0, s, logits, T, iters, eps, out);
  else if (n == 4)
    QSMOE_LAUNCH(k_mhc_sinkhorn<4>, grid, dim3(256), 0, s, logits, T, iters, eps, out);
  else
    QSMOE_LAUNCH(k_mhc_sinkhorn<8>, grid, dim3(256), 0, s, logits, T, iters, eps, out);
  return hipGetLastError();
}

}  // namespace qsmoe
