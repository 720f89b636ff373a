// Plain min/max affine quantisation of bf16 weights: the conversion step
// before the layer (model card "mlx-community / DeepSeek-V4-Flash-4bit",
// section "Conversion": mlx_lm.convert -q --q-bits 4 --q-group-size 64; the
// "MLX-Serve-mixed-2-3-8bit" card contrasts its calibrated search with plain
// min/max). Per group of G inputs of a row:
//   scale = fp16((max - min) / (2^b - 1)), bias = fp16(min),
//   q = clamp(rint((w - bias) / scale), 0, 2^b - 1)   (q = 0 if scale == 0),
// every step in fp32 with IEEE rounding (round-to-nearest-even conversions,
// correctly rounded division, rint ties to even), so the integer codes are
// reproducible bit for bit. Codes are packed as the layer reads them: one
// LSB-first bit stream over little-endian uint32 words along the row.
#include <hip/hip_fp16.h>

#include "common.hpp"
#include "kernels.hpp"

namespace qsmoe {

// One lane per 32-input chunk: its 32 weights (4 x 16-byte loads), the
// group's min and max over the G / 32 lanes of the group (consecutive lanes,
// xor shuffles), its 32 codes into BITS whole words. The first lane of a
// group writes the group's scale and bias.
template <int BITS, int G>
__global__ __launch_bounds__(256) void k_quantize_affine(const uint16_t* __restrict__ w, int64_t nchunks,
                                                         uint32_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                         uint16_t* __restrict__ biases, int32_t* err) {
  constexpr int LPG = G / 32;  // lanes per group
  const int64_t chunk = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const bool valid = chunk < nchunks;
  const int64_t c = valid ? chunk : nchunks - 1;  // the lanes past the end stay in the shuffles
  const uint4* src = reinterpret_cast<const uint4*>(w + c * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 u = src[q];
    const uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * q + 2 * i] = bf16_to_f32(p[i] & 0xffffu);
      v[8 * q + 2 * i + 1] = bf16_to_f32(p[i] >> 16);
    }
  }
  float lo = v[0], hi = v[0];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    lo = fminf(lo, v[i]);
    hi = fmaxf(hi, v[i]);
  }
#pragma unroll
  for (int o = 1; o < LPG; o <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
  }
  constexpr float kLevels = static_cast<float>((1 << BITS) - 1);
  const __half s16 = __float2half_rn((hi - lo) / kLevels);
  const __half b16 = __float2half_rn(lo);
  const float s = __half2float(s16), b = __half2float(b16);
  uint32_t word[BITS];
#pragma unroll
  for (int j = 0; j < BITS; ++j) word[j] = 0;
  // rint of the correctly rounded quotient fl(fl(w - b) / s) without a
  // subtraction and a division per weight: with r the correctly rounded 1 / s,
  // tr = fma(w, r, -fl(b r)) lies within 2^-22 |(w - b) / s| + 2^-24 |b r| of
  // that quotient, so both round to the same integer unless tr is that close
  // to a half-integer. |(w - b) / s| is at most tmax (the rounding steps are
  // monotonic and every finite weight lies in [lo, hi]), which gives one
  // distance for the lane, with a 4x margin. Only weights closer than that to
  // a half-integer, and all of a group with scale 0, a non-finite scale, an
  // offset so large that the distance reaches 1/4, or NaN weights (whose test
  // fails), take the subtraction and the division.
  const float r = 1.0f / s;
  const float br = b * r;
  const float tmax = fmaxf(fabsf(lo - b), fabsf(hi - b)) * r;
  const float tol = (fmaxf(tmax, 1.0f) + fabsf(br)) * 0x1p-20f;
  const float lim = (s > 0.0f && tol < 0.25f) ? 0.5f - tol : -1.0f;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float tr = fmaf(v[i], r, -br);
    float t = rintf(tr);
    if (!(fabsf(tr - t) < lim)) {
      t = s == 0.0f ? 0.0f : rintf((v[i] - b) / s);
      finite = finite && isfinite(v[i]);
    }
    const uint32_t q = static_cast<uint32_t>(fminf(fmaxf(t, 0.0f), kLevels));
    const int bit = i * BITS, wi = bit >> 5, off = bit & 31;
    word[wi] |= q << off;
    if (off + BITS > 32) word[wi + 1] |= q >> (32 - off);
  }
  // infinities show in the scale or the bias; NaN weights only here
  if (valid && (!finite || !isfinite(s) || !isfinite(b))) set_device_error(err, 8);
  if (!valid) return;
  uint32_t* dst = codes + c * BITS;
#pragma unroll
  for (int j = 0; j < BITS; ++j) dst[j] = word[j];
  if (c % LPG == 0) {
    scales[c / LPG] = __half_as_ushort(s16);
    biases[c / LPG] = __half_as_ushort(b16);
  }
}

template <int BITS>
static void launch_quantize_bits(const uint16_t* w, int64_t nchunks, int group, uint32_t* codes, uint16_t* scales,
                                 uint16_t* biases, int32_t* err, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((nchunks + 255) / 256));
  if (group == 32)
    QSMOE_LAUNCH((k_quantize_affine<BITS, 32>), grid, dim3(256), 0, s, w, nchunks, codes, scales, biases, err);
  else if (group == 64)
    QSMOE_LAUNCH((k_quantize_affine<BITS, 64>), grid, dim3(256), 0, s, w, nchunks, codes, scales, biases, err);
  else
    QSMOE_LAUNCH((k_quantize_affine<BITS, 128>), grid, dim3(256), 0, s, w, nchunks, codes, scales, biases, err);
}

hipError_t launch_quantize_affine(const uint16_t* w, int64_t rows, int cols, int bits, int group, uint32_t* codes,
                                  uint16_t* scales, uint16_t* biases, int32_t* err, hipStream_t s) {
  const int64_t nchunks = rows * (cols / 32);
  if (nchunks == 0) return hipSuccess;
  switch (bits) {
    case 2: launch_quantize_bits<2>(w, nchunks, group, codes, scales, biases, err, s); break;
    case 3: launch_quantize_bits<3>(w, nchunks, group, codes, scales, biases, err, s); break;
    case 4: launch_quantize_bits<4>(w, nchunks, group, codes, scales, biases, err, s); break;
    default: launch_quantize_bits<8>(w, nchunks, group, codes, scales, biases, err, s); break;
  }
  return hipGetLastError();
}

}  // namespace qsmoe
