// Expert SwiGLU as a quantised grouped GEMV (few tokens per expert).
//
// Projections are group-quantised, affine b-bit (w = scale * q + bias, fp16
// scale and bias per group; {weight, scales, biases} triplets of the
// pre-stacked experts in mlx-lm PR "Add DeepSeek-v4 (Flash/Pro)"; bit widths
// and groups from "mlx-community / DeepSeek-V4-Flash-4bit" (Conversion) and
// the precision table of "DeepSeek-V4-Flash-0731-MLX-Serve-mixed-2-3-8bit")
// or MXFP4 (e2m1 nibbles, one e8m0 exponent per 32 values; the same PR's
// mxfp4 dequantize, the FP4 e2m1 format of "DeepSeek-V4-Flash-MLX-4bit").
// gate = w1, up = w3, down = w2 (the PR's pre-stacked rename); the SwiGLU
// product silu(w1 x) * (w3 x) is rounded to bf16 before the down projection.
//
// Layout of the work: a workgroup of 4 waves owns 16 consecutive output rows
// of one expert; each wave streams 4 rows. Within a row, lane l owns the
// 32-code chunks c = l + 64 m (m < CPL), so one 16-byte load per lane per
// chunk covers a contiguous 1 KB of a 4-bit row per wave. The activations of
// the NT tokens being processed stay in registers for all rows, packed as
// bf16 pairs in the order the codes are unpacked. Codes are turned into bf16
// pairs with integer ops only (for b <= 4, bf16 bits 0x4300 | q are the exact
// value 128 + q), dotted with v_dot2_f32_bf16 into fp32, and the group's
// scale and bias are applied once per 32-code chunk:
//   sum_i x_i (s q_i + b) = s * sum_i x_i (q_i + off) + (b - off * s) * sum_i x_i.
// MXFP4 nibbles become exact bf16 with v_cvt_scalef32_pk_bf16_fp4 (scale 1),
// and the chunk sum is multiplied by the e8m0 power of two in fp32.
#include "common.hpp"
#include "kernels.hpp"

namespace qsmoe {

constexpr int kRowsPerWave = 4;
constexpr int kRowsPerBlock = 16;

template <int FMT, int BITS>
struct Codec;

// Affine 4-bit: word j holds codes 8j..8j+7; pair m = 4j + i is (8j+i, 8j+i+4).
template <>
struct Codec<0, 4> {
  static constexpr float kOff = 128.0f;
  static constexpr int lo(int m) { return 8 * (m >> 2) + (m & 3); }
  static constexpr int hi(int m) { return lo(m) + 4; }
  __device__ static __forceinline__ void pairs(const uint32_t (&w)[4], uint32_t (&p)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[4 * j + i] = ((w[j] >> (4 * i)) & 0x000f000fu) | 0x43004300u;
  }
};

// Affine 2-bit: word j holds codes 16j..16j+15; pair m = 8j + i is (16j+i, 16j+i+8).
template <>
struct Codec<0, 2> {
  static constexpr float kOff = 128.0f;
  static constexpr int lo(int m) { return 16 * (m >> 3) + (m & 7); }
  static constexpr int hi(int m) { return lo(m) + 8; }
  __device__ static __forceinline__ void pairs(const uint32_t (&w)[2], uint32_t (&p)[16]) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) p[8 * j + i] = ((w[j] >> (2 * i)) & 0x00030003u) | 0x43004300u;
  }
};

// Affine 3-bit: 32 codes in a 96-bit stream; pair m is (m, m+16).
template <>
struct Codec<0, 3> {
  static constexpr float kOff = 128.0f;
  static constexpr int lo(int m) { return m; }
  static constexpr int hi(int m) { return m + 16; }
  __device__ static __forceinline__ uint32_t code(const uint32_t (&w)[3], int c) {
    const int bit = 3 * c, word = bit >> 5, off = bit & 31;
    if (off <= 29) return (w[word] >> off) & 7u;
    return ((w[word] >> off) | (w[word + 1] << (32 - off))) & 7u;
  }
  __device__ static __forceinline__ void pairs(const uint32_t (&w)[3], uint32_t (&p)[16]) {
#pragma unroll
    for (int m = 0; m < 16; ++m) p[m] = code(w, m) | (code(w, m + 16) << 16) | 0x43004300u;
  }
};

// Affine 8-bit: word j holds codes 4j..4j+3; pair m = 2j + h is (4j+2h, 4j+2h+1).
// Codes up to 255 are exact in bf16: convert to fp32 and keep the top half.
template <>
struct Codec<0, 8> {
  static constexpr float kOff = 0.0f;
  static constexpr int lo(int m) { return 2 * m; }
  static constexpr int hi(int m) { return 2 * m + 1; }
  __device__ static __forceinline__ void pairs(const uint32_t (&w)[8], uint32_t (&p)[16]) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float fa = static_cast<float>((w[j] >> (16 * h)) & 0xffu);
        const float fb = static_cast<float>((w[j] >> (16 * h + 8)) & 0xffu);
        p[2 * j + h] = (__float_as_uint(fa) >> 16) | (__float_as_uint(fb) & 0xffff0000u);
      }
  }
};

// MXFP4: byte b of word j holds codes 8j+2b (low nibble) and 8j+2b+1.
template <>
struct Codec<1, 4> {
  static constexpr float kOff = 0.0f;
  static constexpr int lo(int m) { return 2 * m; }
  static constexpr int hi(int m) { return 2 * m + 1; }
  __device__ static __forceinline__ void pairs(const uint32_t (&w)[4], uint32_t (&p)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[4 * j + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], 1.0f, 0));
      p[4 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], 1.0f, 1));
      p[4 * j + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], 1.0f, 2));
      p[4 * j + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], 1.0f, 3));
    }
  }
};

// Activations of NT tokens for the lane's CPL chunks.
template <int FMT, int BITS, int CPL, int NT>
struct XRegs {
  uint32_t px[NT][CPL][16];
  float xs[NT][CPL];
};

template <int FMT, int BITS, int CPL, int NT>
__device__ __forceinline__ void load_x(XRegs<FMT, BITS, CPL, NT>& xr, const uint16_t* const (&xrow)[NT], int lane,
                                       int nchunks) {
  using C = Codec<FMT, BITS>;
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
      const int c = lane + 64 * m;
      uint32_t xw[16];
      if (xrow[j] != nullptr && c < nchunks) {
        const uint4* src = reinterpret_cast<const uint4*>(xrow[j] + 32 * c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = src[q];
          xw[4 * q + 0] = v.x;
          xw[4 * q + 1] = v.y;
          xw[4 * q + 2] = v.z;
          xw[4 * q + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) xw[q] = 0;
      }
      float sum = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) sum += bf16_to_f32(xw[q] & 0xffffu) + bf16_to_f32(xw[q] >> 16);
      xr.xs[j][m] = sum;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int a = C::lo(i), b = C::hi(i);
        const uint32_t xa = (xw[a >> 1] >> (16 * (a & 1))) & 0xffffu;
        const uint32_t xb = (xw[b >> 1] >> (16 * (b & 1))) & 0xffffu;
        xr.px[j][m][i] = xa | (xb << 16);
      }
    }
}

// One quantised row as loaded by one lane.
template <int FMT, int BITS, int CPL>
struct RowRegs {
  uint32_t w[CPL][BITS];
  float s[CPL];
  float b[CPL];
};

template <int FMT, int BITS, int CPL>
__device__ __forceinline__ void load_row(RowRegs<FMT, BITS, CPL>& r, const QMat& q, size_t row_index, int lane,
                                         int nchunks) {
  const uint32_t* codes = q.codes + row_index * q.row_words;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = lane + 64 * m;
    if (c < nchunks) {
      const uint32_t* src = codes + c * BITS;
      if constexpr (BITS == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(src);
        r.w[m][0] = v.x;
        r.w[m][1] = v.y;
        r.w[m][2] = v.z;
        r.w[m][3] = v.w;
      } else if constexpr (BITS == 8) {
        const uint4 v0 = reinterpret_cast<const uint4*>(src)[0];
        const uint4 v1 = reinterpret_cast<const uint4*>(src)[1];
        r.w[m][0] = v0.x;
        r.w[m][1] = v0.y;
        r.w[m][2] = v0.z;
        r.w[m][3] = v0.w;
        r.w[m][4] = v1.x;
        r.w[m][5] = v1.y;
        r.w[m][6] = v1.z;
        r.w[m][7] = v1.w;
      } else if constexpr (BITS == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(src);
        r.w[m][0] = v.x;
        r.w[m][1] = v.y;
      } else {
        r.w[m][0] = src[0];
        r.w[m][1] = src[1];
        r.w[m][2] = src[2];
      }
      const size_t g = row_index * q.row_groups + (c >> q.gshift);
      if constexpr (FMT == 0) {
        r.s[m] = f16_to_f32(static_cast<const uint16_t*>(q.scales)[g]);
        r.b[m] = f16_to_f32(q.biases[g]);
      } else {
        r.s[m] = e8m0_to_f32(static_cast<const uint8_t*>(q.scales)[g]);
        r.b[m] = 0.0f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < BITS; ++i) r.w[m][i] = 0;
      r.s[m] = 0.0f;
      r.b[m] = 0.0f;
    }
  }
}

template <int FMT, int BITS, int CPL, int NT>
__device__ __forceinline__ void row_dot(const RowRegs<FMT, BITS, CPL>& r, const XRegs<FMT, BITS, CPL, NT>& xr,
                                        float* acc) {
  using C = Codec<FMT, BITS>;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    uint32_t p[16];
    C::pairs(r.w[m], p);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        d0 = dot2_bf16(p[i], xr.px[j][m][i], d0);
        d1 = dot2_bf16(p[i + 1], xr.px[j][m][i + 1], d1);
      }
      const float d = d0 + d1;
      if constexpr (FMT == 0)
        acc[j] += r.s[m] * d + (r.b[m] - C::kOff * r.s[m]) * xr.xs[j][m];
      else
        acc[j] += d * r.s[m];
    }
  }
}

__device__ __forceinline__ QMat expert_slice(const QMat& q, int e) {
  QMat r = q;
  const size_t rows = static_cast<size_t>(q.rows);
  r.codes = q.codes + static_cast<size_t>(e) * rows * q.row_words;
  if (q.fmt == 0) {
    r.scales = static_cast<const uint16_t*>(q.scales) + static_cast<size_t>(e) * rows * q.row_groups;
    r.biases = q.biases + static_cast<size_t>(e) * rows * q.row_groups;
  } else {
    r.scales = static_cast<const uint8_t*>(q.scales) + static_cast<size_t>(e) * rows * q.row_groups;
  }
  return r;
}

// Which expert and which range of bucketed positions this workgroup serves.
__device__ __forceinline__ bool bucket_range(int bucket, int shared, int T, int NTtok, const int32_t* offsets,
                                             int E, int n, int& e, int& p0, int& p1) {
  if (shared) {
    e = 0;
    p0 = bucket * NTtok;
    p1 = min(T, p0 + NTtok);
    return p0 < p1;
  }
  e = find_bucket_expert(offsets, E, bucket);
  if (e < 0) return false;
  // clamp to [0, n) so that malformed offsets cannot index out of bounds
  p0 = max(0, min(offsets[e], n));
  p1 = max(p0, min(offsets[e + 1], n));
  return p0 < p1;
}

// Token of bucketed position p (routed): perm holds assignment a = t*k + j.
__device__ __forceinline__ int token_of(const int32_t* perm, int p, int k, int T) {
  return min(max(perm[p] / k, 0), T - 1);
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU: h[p][r] = bf16(silu(gate_r . x) * (up_r . x))
// ---------------------------------------------------------------------------
template <int FMT, int BITS, int CPL, int NT>
__global__ __launch_bounds__(256) void k_gateup(GateUpArgs a) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int rows = a.gate.rows;
  const int row_tiles = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int bucket = blockIdx.x / row_tiles, tile = blockIdx.x % row_tiles;
  int e, p0, p1;
  if (!bucket_range(bucket, a.shared, a.T, NT, a.offsets, a.E, a.T * a.k, e, p0, p1)) return;
  const QMat g = expert_slice(a.gate, e), u = expert_slice(a.up, e);
  const int nchunks = g.cols >> 5;
  const int r0 = tile * kRowsPerBlock + wave * kRowsPerWave;
  if (r0 >= rows) return;
  for (int p = p0; p < p1; p += NT) {
    const uint16_t* xrow[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int pj = p + j;
      if (pj < p1) {
        const int t = a.shared ? pj : token_of(a.perm, pj, a.k, a.T);
        xrow[j] = a.x + static_cast<size_t>(t) * g.cols;
      } else {
        xrow[j] = nullptr;
      }
    }
    XRegs<FMT, BITS, CPL, NT> xr;
    load_x<FMT, BITS, CPL, NT>(xr, xrow, lane, nchunks);
    RowRegs<FMT, BITS, CPL> rg[kRowsPerWave], ru[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int r = min(r0 + i, rows - 1);
      load_row<FMT, BITS, CPL>(rg[i], g, r, lane, nchunks);
      load_row<FMT, BITS, CPL>(ru[i], u, r, lane, nchunks);
    }
    float ag[kRowsPerWave * NT], au[kRowsPerWave * NT];
#pragma unroll
    for (int i = 0; i < kRowsPerWave * NT; ++i) ag[i] = au[i] = 0.0f;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      row_dot<FMT, BITS, CPL, NT>(rg[i], xr, ag + i * NT);
      row_dot<FMT, BITS, CPL, NT>(ru[i], xr, au + i * NT);
    }
    constexpr int N = kRowsPerWave * NT;
    const float gs = wave_reduce_multi<N>(ag);
    const float us = wave_reduce_multi<N>(au);
    const int v = reduce_multi_index<N>(lane);
    const int ri = v / NT, j = v % NT;
    if (reduce_multi_writer<N>(lane) && p + j < p1 && r0 + ri < rows)
      a.h[static_cast<size_t>(p + j) * rows + r0 + ri] = static_cast<uint16_t>(f32_to_bf16_rne(silu(gs) * us));
  }
}

// ---------------------------------------------------------------------------
// down: y[a][r] = down_r . h[p]  (a = perm[p] routed, a = p shared)
// ---------------------------------------------------------------------------
template <int FMT, int BITS, int CPL, int NT>
__global__ __launch_bounds__(256) void k_down(DownArgs a) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int rows = a.down.rows;
  const int row_tiles = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int bucket = blockIdx.x / row_tiles, tile = blockIdx.x % row_tiles;
  int e, p0, p1;
  if (!bucket_range(bucket, a.shared, a.T, NT, a.offsets, a.E, a.T * a.k, e, p0, p1)) return;
  const QMat dn = expert_slice(a.down, e);
  const int cols = dn.cols, nchunks = cols >> 5;
  const int r0 = tile * kRowsPerBlock + wave * kRowsPerWave;
  if (r0 >= rows) return;
  for (int p = p0; p < p1; p += NT) {
    const uint16_t* xrow[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) xrow[j] = (p + j < p1) ? a.h + static_cast<size_t>(p + j) * cols : nullptr;
    XRegs<FMT, BITS, CPL, NT> xr;
    load_x<FMT, BITS, CPL, NT>(xr, xrow, lane, nchunks);
    RowRegs<FMT, BITS, CPL> rr[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) load_row<FMT, BITS, CPL>(rr[i], dn, min(r0 + i, rows - 1), lane, nchunks);
    float acc[kRowsPerWave * NT];
#pragma unroll
    for (int i = 0; i < kRowsPerWave * NT; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) row_dot<FMT, BITS, CPL, NT>(rr[i], xr, acc + i * NT);
    constexpr int N = kRowsPerWave * NT;
    const float ys = wave_reduce_multi<N>(acc);
    const int v = reduce_multi_index<N>(lane);
    const int ri = v / NT, j = v % NT;
    if (reduce_multi_writer<N>(lane) && p + j < p1 && r0 + ri < rows) {
      const int slot = a.shared ? p + j : min(max(a.perm[p + j], 0), a.T * a.k - 1);
      a.y[static_cast<size_t>(slot) * rows + r0 + ri] = ys;
    }
  }
}

// ---------------------------------------------------------------------------
static int chunks_per_lane(int cols) { return cols <= 2048 ? 1 : (cols <= 4096 ? 2 : 4); }

bool gemv_supported(const QMat& m) {
  if (m.cols % 32 != 0 || m.cols > 8192 || m.rows < 1) return false;
  if (m.fmt == 0) return m.bits == 2 || m.bits == 3 || m.bits == 4 || m.bits == 8;
  return m.fmt == 1 && m.bits == 4 && m.group == 32;
}

// Tokens handled per pass over the rows, from the mean bucket size.
static int tokens_per_pass(int T, int k, int E, int cpl, int shared) {
  const int buckets = shared ? 1 : (T * k < E ? T * k : E);
  const int per = shared ? T : (T * k + buckets - 1) / buckets;
  int nt = per <= 1 ? 1 : (per <= 2 ? 2 : 4);
  while (nt * cpl > 4) nt >>= 1;
  return nt;
}

#define QSMOE_FMT_SWITCH(FMT_, BITS_, ...)                   \
  if ((FMT_) == 0 && (BITS_) == 4) {                         \
    constexpr int F = 0, B = 4;                              \
    __VA_ARGS__                                              \
  } else if ((FMT_) == 0 && (BITS_) == 2) {                  \
    constexpr int F = 0, B = 2;                              \
    __VA_ARGS__                                              \
  } else if ((FMT_) == 0 && (BITS_) == 3) {                  \
    constexpr int F = 0, B = 3;                              \
    __VA_ARGS__                                              \
  } else if ((FMT_) == 0 && (BITS_) == 8) {                  \
    constexpr int F = 0, B = 8;                              \
    __VA_ARGS__                                              \
  } else {                                                   \
    constexpr int F = 1, B = 4;                              \
    __VA_ARGS__                                              \
  }

#define QSMOE_SHAPE_SWITCH(CPL_, NT_, ...)                   \
  if ((CPL_) == 1 && (NT_) == 1) {                           \
    constexpr int CP = 1, NTK = 1;                           \
    __VA_ARGS__                                              \
  } else if ((CPL_) == 1 && (NT_) == 2) {                    \
    constexpr int CP = 1, NTK = 2;                           \
    __VA_ARGS__                                              \
  } else if ((CPL_) == 1) {                                  \
    constexpr int CP = 1, NTK = 4;                           \
    __VA_ARGS__                                              \
  } else if ((CPL_) == 2 && (NT_) == 1) {                    \
    constexpr int CP = 2, NTK = 1;                           \
    __VA_ARGS__                                              \
  } else if ((CPL_) == 2) {                                  \
    constexpr int CP = 2, NTK = 2;                           \
    __VA_ARGS__                                              \
  } else {                                                   \
    constexpr int CP = 4, NTK = 1;                           \
    __VA_ARGS__                                              \
  }

hipError_t launch_gateup(const GateUpArgs& a, hipStream_t s) {
  const int cpl = chunks_per_lane(a.gate.cols);
  const int nt = tokens_per_pass(a.T, a.k, a.E, cpl, a.shared);
  const int row_tiles = (a.gate.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int buckets = a.shared ? (a.T + nt - 1) / nt : (a.T * a.k < a.E ? a.T * a.k : a.E);
  const dim3 grid(static_cast<unsigned>(buckets) * row_tiles), block(256);
  QSMOE_FMT_SWITCH(a.gate.fmt, a.gate.bits, QSMOE_SHAPE_SWITCH(cpl, nt, {
    hipLaunchKernelGGL((k_gateup<F, B, CP, NTK>), grid, block, 0, s, a);
  }))
  return hipGetLastError();
}

hipError_t launch_down(const DownArgs& a, hipStream_t s) {
  const int cpl = chunks_per_lane(a.down.cols);
  const int nt = tokens_per_pass(a.T, a.k, a.E, cpl, a.shared);
  const int row_tiles = (a.down.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int buckets = a.shared ? (a.T + nt - 1) / nt : (a.T * a.k < a.E ? a.T * a.k : a.E);
  const dim3 grid(static_cast<unsigned>(buckets) * row_tiles), block(256);
  QSMOE_FMT_SWITCH(a.down.fmt, a.down.bits, QSMOE_SHAPE_SWITCH(cpl, nt, {
    hipLaunchKernelGGL((k_down<F, B, CP, NTK>), grid, block, 0, s, a);
  }))
  return hipGetLastError();
}

}  // namespace qsmoe
