// mHC mix matrices, an op beside the MoE layer (model card
// "mlx-community / DeepSeek-V4-Flash-4bit", section "Architecture": the
// residual stream is hc_mult = 4 parallel copies recombined by a
// doubly-stochastic, Sinkhorn-normalised mix matrix; mlx-lm pull request
// "Add DeepSeek-v4 (Flash/Pro)", review notes: unfused, the normalisation is
// a softmax followed by iterations of a sum and a division, ~40 launches per
// call). Per token: softmax over each row of the n x n logits, then `iters`
// rounds of dividing every column by its sum (+ eps) and then every row by
// its sum (+ eps). One lane per matrix element: a token's n x n lanes are
// consecutive within a wave (n * n divides 64), so a row sum pairs the n
// lanes of the row and a column sum the lanes n apart, by DPP lane moves
// within 16 lanes (only n = 8's column steps across 16 and 32 lanes go
// through LDS shuffles); the logits are read once (coalesced) and the result
// written once, in one launch. (With every step an LDS shuffle, a chain of
// 40 round trips over 10 rounds, 4096 tokens at n = 4 took 3.9-4.5 us.) (One thread per token, its matrix in registers, ran each
// token's ~300 divisions in one dependent chain on 1/16 of the lanes: 10.4 us
// per 4096 tokens.)
#include "common.hpp"
#include "kernels.hpp"

namespace qsmoe {

// A lane's value moved by a DPP lane pattern (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xb1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kDppRor4 = 0x124;       // rotate by 4 within 16
constexpr int kDppRor8 = 0x128;       // rotate by 8 within 16

// Sum over the N consecutive lanes of a matrix row: every lane of the row
// gets the same bits (each step adds a lane's value and its partner's).
template <int N>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_mov<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp_mov<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp_mov<kDppHalfMirror>(x);
  return x;
}

// Sum over the N lanes of a matrix column (stride N, NN lanes per matrix).
template <int N>
__device__ __forceinline__ float col_sum(float x) {
  if constexpr (N == 2) {
    x += dpp_mov<kDppXor2>(x);
  } else if constexpr (N == 4) {
    x += dpp_mov<kDppRor8>(x);  // lanes i, i + 8 of the 16
    x += dpp_mov<kDppRor4>(x);  // ... and i + 4, i + 12
  } else {
    x += dpp_mov<kDppRor8>(x);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
  }
  return x;
}

template <int N>
__global__ __launch_bounds__(256) void k_mhc_sinkhorn(const float* logits, int64_t T, int iters, float eps,
                                                      float* out) {
  constexpr int NN = N * N;
  static_assert(64 % NN == 0, "a matrix's lanes lie in one wave");
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // element of logits[T][N][N]
  const bool valid = e < T * NN;  // whole matrices are valid or not: 256 % NN == 0
  float v = valid ? logits[e] : 0.0f;
  float mx = v;
  mx = fmaxf(mx, dpp_mov<kDppXor1>(mx));
  if constexpr (N >= 4) mx = fmaxf(mx, dpp_mov<kDppXor2>(mx));
  if constexpr (N >= 8) mx = fmaxf(mx, dpp_mov<kDppHalfMirror>(mx));
  v = expf(v - mx);
  v = v / row_sum<N>(v);
  for (int it = 0; it < iters; ++it) {
    v = v / (col_sum<N>(v) + eps);
    v = v / (row_sum<N>(v) + eps);
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
