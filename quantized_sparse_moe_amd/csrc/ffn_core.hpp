// Quantised-row streaming core shared by the expert kernels: code unpacking
// per format, activations held in registers, branch-free row loads, the
// per-row dot products and the (virtual bucket, row) streaming loop.
#pragma once

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace qsmoe {

template <int FMT, int BITS>
struct Codec;

// Affine b-bit codes (b <= 4) become exact bf16 values without a multiply:
// with the exponent of 2^b and the code in the top b bits of the 7-bit
// mantissa, the bits (0x3F80 + (b << 7)) | (q << (7 - b)) are the value
// 2^b + q. The offset 2^b is the smallest that keeps integer steps, so the
// sums the kernels form (x times 2^b + q, the offset removed through the
// group's sum of x) carry the least cancellation: 16 + q for 4-bit codes
// instead of 128 + q.
template <int BITS>
constexpr uint32_t kCodeBase = 0x3F80u + (static_cast<uint32_t>(BITS) << 7);  // bf16 bits of 2^BITS

// The pair (2^b, 2^b) as a vector register: with one operand already in a
// VGPR, "(w >> n) & mask | k" compiles to a single v_and_or_b32 (the mask
// takes the one scalar operand a VOP3 may read).
template <int BITS>
__device__ __forceinline__ uint32_t code_base_pair() {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(kCodeBase<BITS> * 0x10001u), 0xE4, 0xF,
                                                        0xF, false));
}

// Code fields at bit `at` of each 16-bit half of w moved to the top BITS bits
// of the bf16 mantissa (bit 7 - BITS), masked, with the exponent of 2^BITS.
template <int BITS, int AT>
__device__ __forceinline__ uint32_t code_pair(uint32_t w, uint32_t k) {
  constexpr int kTop = 7 - BITS;
  constexpr uint32_t kMask = ((1u << BITS) - 1u) * 0x10001u << kTop;
  if constexpr (AT >= kTop)
    return ((w >> (AT - kTop)) & kMask) | k;
  else
    return ((w << (kTop - AT)) & kMask) | k;
}

// Affine 4-bit: word j holds codes 8j..8j+7; pair m = 4j + i is (8j+i, 8j+i+4).
template <>
struct Codec<0, 4> {
  static constexpr float kOff = 16.0f;
  static constexpr int lo(int m) { return 8 * (m >> 2) + (m & 3); }
  static constexpr int hi(int m) { return lo(m) + 4; }
  __device__ static __forceinline__ void pairs(const uint32_t (&w)[4], uint32_t (&p)[16]) {
    const uint32_t k = code_base_pair<4>();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[4 * j + 0] = code_pair<4, 0>(w[j], k);
      p[4 * j + 1] = code_pair<4, 4>(w[j], k);
      p[4 * j + 2] = code_pair<4, 8>(w[j], k);
      p[4 * j + 3] = code_pair<4, 12>(w[j], k);
    }
  }
};

// Affine 2-bit: word j holds codes 16j..16j+15; pair m = 8j + i is (16j+i, 16j+i+8).
template <>
struct Codec<0, 2> {
  // A 2-bit code q in the low two bits of a nibble is the e2m1 value q / 2:
  // masking word j with 0x33333333 leaves its even-indexed codes in the
  // nibbles (its odd-indexed ones after a shift by 2), and
  // v_cvt_scalef32_pk_bf16_fp4 at scale 2 turns each byte into the exact bf16
  // pair of its two codes (3 masks and 8 conversions per 16 codes; no code
  // offset). Pair m = 8j + r is (16j + 4r, 16j + 4r + 2) for r < 4 and
  // (16j + 4(r - 4) + 1, 16j + 4(r - 4) + 3) for r >= 4.
  static constexpr float kOff = 0.0f;
  static constexpr int lo(int m) { return 16 * (m >> 3) + 4 * (m & 3) + ((m >> 2) & 1); }
  static constexpr int hi(int m) { return lo(m) + 2; }
  __device__ static __forceinline__ void pairs(const uint32_t (&w)[2], uint32_t (&p)[16]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t m0 = w[j] & 0x33333333u, m1 = (w[j] >> 2) & 0x33333333u;
#define QSMOE_CVT2(K_)                                                                                        \
  p[8 * j + K_] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m0, 2.0f, K_));     \
  p[8 * j + 4 + K_] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m1, 2.0f, K_));
      QSMOE_CVT2(0)
      QSMOE_CVT2(1)
      QSMOE_CVT2(2)
      QSMOE_CVT2(3)
#undef QSMOE_CVT2
    }
  }
};

// Affine 3-bit: 32 codes in a 96-bit stream; pair m is (m, m+16).
template <>
struct Codec<0, 3> {
  static constexpr float kOff = 8.0f;
  static constexpr int lo(int m) { return m; }
  static constexpr int hi(int m) { return m + 16; }
  __device__ static __forceinline__ uint32_t code(const uint32_t (&w)[3], int c) {
    const int bit = 3 * c, word = bit >> 5, off = bit & 31;
    if (off <= 29) return (w[word] >> off) & 7u;
    return ((w[word] >> off) | (w[word + 1] << (32 - off))) & 7u;
  }
  __device__ static __forceinline__ void pairs(const uint32_t (&w)[3], uint32_t (&p)[16]) {
    const uint32_t k = code_base_pair<3>();
#pragma unroll
    for (int m = 0; m < 16; ++m) p[m] = (code(w, m) << 4) | (code(w, m + 16) << 20) | k;
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

// MXFP8: byte b of word j holds code 4j+b (OCP E4M3); pair m = 2j + h is
// (4j+2h, 4j+2h+1). Every finite E4M3 value is exact in bf16, so the scaled
// conversion runs with scale 1 and the e8m0 scale multiplies the dot product.
template <>
struct Codec<2, 8> {
  static constexpr float kOff = 0.0f;
  static constexpr int lo(int m) { return 2 * m; }
  static constexpr int hi(int m) { return 2 * m + 1; }
  __device__ static __forceinline__ void pairs(const uint32_t (&w)[8], uint32_t (&p)[16]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[2 * j + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], 1.0f, false));
      p[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], 1.0f, true));
    }
  }
};

// Activations of NT tokens for the lane's CPL chunks.
template <int FMT, int BITS, int CPL, int NT>
struct XRegs {
  uint32_t px[NT][CPL][16];
  float xs[NT][CPL];
};

// Loads are issued without branches: an out-of-range chunk (or a missing
// token) loads from a clamped, always valid address and is masked to zero
// afterwards. A branch around a load makes the compiler wait for it before
// leaving the branch, which would serialise every row's memory round trip.
// Activations are fetched in two phases so that callers can put weight loads
// in flight between issuing them (load_x_raw) and consuming them (finish_x).
template <int CPL, int NT>
struct XRaw {
  uint32_t w[NT][CPL][16];
};

template <int CPL, int NT>
__device__ __forceinline__ void load_x_raw(XRaw<CPL, NT>& xw, const uint16_t* const (&xrow)[NT], int lane,
                                           int nchunks) {
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
      const int c = min(lane + 64 * m, nchunks - 1);
      const uint4* src = reinterpret_cast<const uint4*>(xrow[j] + 32 * c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = src[q];
        xw.w[j][m][4 * q + 0] = v.x;
        xw.w[j][m][4 * q + 1] = v.y;
        xw.w[j][m][4 * q + 2] = v.z;
        xw.w[j][m][4 * q + 3] = v.w;
      }
    }
}

template <int FMT, int BITS, int CPL, int NT>
__device__ __forceinline__ void finish_x(XRegs<FMT, BITS, CPL, NT>& xr, const XRaw<CPL, NT>& xw,
                                         const bool (&xvalid)[NT], int lane, int nchunks) {
  using C = Codec<FMT, BITS>;
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
      const bool ok = xvalid[j] && lane + 64 * m < nchunks;
      uint32_t v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = ok ? xw.w[j][m][q] : 0u;
      float sum = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) sum += bf16_to_f32(v[q] & 0xffffu) + bf16_to_f32(v[q] >> 16);
      xr.xs[j][m] = sum;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int a = C::lo(i), b = C::hi(i);
        const uint32_t xa = (v[a >> 1] >> (16 * (a & 1))) & 0xffffu;
        const uint32_t xb = (v[b >> 1] >> (16 * (b & 1))) & 0xffffu;
        xr.px[j][m][i] = xa | (xb << 16);
      }
    }
}

template <int FMT, int BITS, int CPL, int NT>
__device__ __forceinline__ void load_x(XRegs<FMT, BITS, CPL, NT>& xr, const uint16_t* const (&xrow)[NT],
                                       const bool (&xvalid)[NT], int lane, int nchunks) {
  XRaw<CPL, NT> xw;
  load_x_raw<CPL, NT>(xw, xrow, lane, nchunks);
  finish_x<FMT, BITS, CPL, NT>(xr, xw, xvalid, lane, nchunks);
}

// 4-bit weight codes are read exactly once per launch: load them
// non-temporally (measured: 2 % faster decode, no effect on the other
// streaming launches; slower for the 8-bit shared rows, which keep plain loads).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_stream_t;
__device__ __forceinline__ uint4 load_stream16(const uint32_t* p) {
  const u32x4_stream_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_stream_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// One quantised row as loaded by one lane: raw code words and raw scale /
// bias bits, converted only when the row is consumed.
template <int FMT, int BITS, int CPL>
struct RowRegs {
  uint32_t w[CPL][BITS];
  uint32_t s[CPL];
  uint32_t b[CPL];
};

template <int FMT, int BITS, int CPL>
__device__ __forceinline__ void load_row(RowRegs<FMT, BITS, CPL>& r, const QMat& q, size_t row_index, int lane,
                                         int nchunks) {
  const uint32_t* codes = q.codes + row_index * q.row_words;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = min(lane + 64 * m, nchunks - 1);
    const uint32_t* src = codes + c * BITS;
    if constexpr (BITS == 4) {
      const uint4 v = load_stream16(src);
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
      r.s[m] = static_cast<const uint16_t*>(q.scales)[g];
      r.b[m] = q.biases[g];
    } else {
      r.s[m] = static_cast<const uint8_t*>(q.scales)[g];
      r.b[m] = 0;
    }
  }
}

template <int FMT, int BITS, int CPL, int NT>
__device__ __forceinline__ void row_dot(const RowRegs<FMT, BITS, CPL>& r, const XRegs<FMT, BITS, CPL, NT>& xr,
                                        float* acc, int lane, int nchunks) {
  using C = Codec<FMT, BITS>;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const bool ok = lane + 64 * m < nchunks;
    uint32_t p[16];
    C::pairs(r.w[m], p);
    float s, b;
    if constexpr (FMT == 0) {
      s = ok ? f16_to_f32(static_cast<uint16_t>(r.s[m])) : 0.0f;
      b = ok ? f16_to_f32(static_cast<uint16_t>(r.b[m])) : 0.0f;
    } else {
      s = ok ? e8m0_to_f32(r.s[m]) : 0.0f;
      b = 0.0f;
    }
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
        acc[j] += s * d + (b - C::kOff * s) * xr.xs[j][m];
      else
        acc[j] += d * s;
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

// Work of one launch: the (virtual bucket, row) units of one projection (or of
// the gate/up pair). A virtual bucket is up to NT consecutive bucketed
// positions of one expert (routed) or NT consecutive tokens (shared). The
// units are split evenly over all waves of the grid, whatever the routing.
struct StreamArgs {
  QMat m0, m1;           // gate and up (GATEUP), or down
  const uint16_t* x;     // gate/up: activations [T][cols]; down: h [*][cols]
  int32_t T, k, E;
  const int32_t* offsets;
  const int32_t* perm;
  int32_t shared;
  uint16_t* h;           // gate/up output
  float* y;              // down output
};

constexpr int kMaxExperts = 1024;

// Rows [r_begin, r_end) of q0 (and q1) against the activations in xr. Rows
// go in batches of BR per wave, double-buffered: the next batch's loads are
// issued before the current batch is computed, so every wave keeps memory
// requests in flight while it works. store(j, row, v0, v1) is called once per
// (token j, row) by one lane. Small batches keep fewer bytes in flight per
// wave, which lowers the queueing latency when every wave of the chip streams
// at once; the callers pick BR per projection.
template <int FMT, int BITS, int CPL, bool GATEUP, int BR>
struct RowBatch {
  RowRegs<FMT, BITS, CPL> r0[BR];
  RowRegs<FMT, BITS, CPL> r1[GATEUP ? BR : 1];
};

template <int FMT, int BITS, int CPL, bool GATEUP, int BR>
__device__ __forceinline__ void load_batch(RowBatch<FMT, BITS, CPL, GATEUP, BR>& b, const QMat& q0,
                                           const QMat& q1, int r0, int r_end, int lane, int nchunks) {
#pragma unroll
  for (int i = 0; i < BR; ++i) {
    const int r = min(r0 + i, r_end - 1);
    load_row<FMT, BITS, CPL>(b.r0[i], q0, r, lane, nchunks);
    if constexpr (GATEUP) load_row<FMT, BITS, CPL>(b.r1[i], q1, r, lane, nchunks);
  }
}

template <int FMT, int BITS, int CPL, int NT, bool GATEUP, int BR, class Store>
__device__ __forceinline__ void compute_batch(const RowBatch<FMT, BITS, CPL, GATEUP, BR>& b,
                                              const XRegs<FMT, BITS, CPL, NT>& xr, int r0, int r_end, int lane,
                                              int nchunks, Store& store) {
  constexpr int N = BR * NT;
  float acc0[N], acc1[N];
#pragma unroll
  for (int i = 0; i < N; ++i) acc0[i] = acc1[i] = 0.0f;
#pragma unroll
  for (int i = 0; i < BR; ++i) {
    row_dot<FMT, BITS, CPL, NT>(b.r0[i], xr, acc0 + i * NT, lane, nchunks);
    if constexpr (GATEUP) row_dot<FMT, BITS, CPL, NT>(b.r1[i], xr, acc1 + i * NT, lane, nchunks);
  }
  const float s0 = wave_reduce_multi<N>(acc0);
  const float s1 = GATEUP ? wave_reduce_multi<N>(acc1) : 0.0f;
  const int v = reduce_multi_index<N>(lane);
  const int ri = v / NT, j = v % NT;
  if (reduce_multi_writer<N>(lane) && r0 + ri < r_end) store(j, r0 + ri, s0, s1);
}

template <int FMT, int BITS, int CPL, int NT, bool GATEUP, int BR, class Store>
__device__ __forceinline__ void stream_rows(const QMat& q0, const QMat& q1, const XRaw<CPL, NT>& xw,
                                            const bool (&xvalid)[NT], int r_begin, int r_end, int lane,
                                            int nchunks, Store store) {
  // The prefetches are unconditional (rows clamped to r_end - 1): a load
  // behind a branch makes the compiler assume the worst at the join and wait
  // for every load in flight, which would undo the double buffering. The
  // activations (issued by the caller) are unpacked once the first rows are
  // in flight.
  RowBatch<FMT, BITS, CPL, GATEUP, BR> A, B;
  int r = r_begin;
  load_batch<FMT, BITS, CPL, GATEUP, BR>(A, q0, q1, r, r_end, lane, nchunks);
  XRegs<FMT, BITS, CPL, NT> xr;
  finish_x<FMT, BITS, CPL, NT>(xr, xw, xvalid, lane, nchunks);
  while (true) {
    load_batch<FMT, BITS, CPL, GATEUP, BR>(B, q0, q1, r + BR, r_end, lane, nchunks);
    compute_batch<FMT, BITS, CPL, NT, GATEUP, BR>(A, xr, r, r_end, lane, nchunks, store);
    if (r + BR >= r_end) break;
    load_batch<FMT, BITS, CPL, GATEUP, BR>(A, q0, q1, r + 2 * BR, r_end, lane, nchunks);
    compute_batch<FMT, BITS, CPL, NT, GATEUP, BR>(B, xr, r + BR, r_end, lane, nchunks, store);
    if (r + 2 * BR >= r_end) break;
    r += 2 * BR;
  }
}

// One launch's share of the (virtual bucket, row) units of a projection (or
// of the gate/up pair), for workgroup `bid` of `nblk`. s_off / s_vb are LDS
// scratch of kMaxExperts + 1 ints each (unused in shared mode).
template <int FMT, int BITS, int CPL, int NT, bool GATEUP>
__device__ __forceinline__ void ffn_stream_body(const StreamArgs& a, int bid, int nblk, int32_t* s_off,
                                                int32_t* s_vb) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int rows = a.m0.rows, cols = a.m0.cols, nchunks = cols >> 5;
  const int n = a.shared ? a.T : a.T * a.k;
  int n_vb;
  if (a.shared) {
    n_vb = (a.T + NT - 1) / NT;
  } else {
    for (int i = threadIdx.x; i <= a.E; i += blockDim.x) s_off[i] = min(max(a.offsets[i], 0), n);
    __syncthreads();
    if (wave == 0) {
      // exclusive scan of ceil(count / NT) over experts -> first virtual bucket of each expert
      int carry = 0;
      for (int e0 = 0; e0 < a.E; e0 += 64) {
        const int e = e0 + lane;
        const int cnt = e < a.E ? max(s_off[e + 1] - s_off[e], 0) : 0;
        const int c = (cnt + NT - 1) / NT;
        int incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o);
          if (lane >= o) incl += y;
        }
        if (e < a.E) s_vb[e] = carry + incl - c;
        carry += __shfl(incl, 63);
      }
      if (lane == 0) s_vb[a.E] = carry;
    }
    __syncthreads();
    n_vb = s_vb[a.E];
  }
  const int64_t total = static_cast<int64_t>(n_vb) * rows;
  const int64_t W = static_cast<int64_t>(nblk) * 4, gw = static_cast<int64_t>(bid) * 4 + wave;
  int64_t u = total * gw / W;
  const int64_t u_end = total * (gw + 1) / W;

  while (u < u_end) {
    const int vb = static_cast<int>(u / rows);
    const int r_begin = static_cast<int>(u - static_cast<int64_t>(vb) * rows);
    const int r_end = static_cast<int>(min<int64_t>(rows, r_begin + (u_end - u)));
    int e, p0, p1;
    if (a.shared) {
      e = 0;
      p0 = vb * NT;
      p1 = min(a.T, p0 + NT);
    } else {
      // the expert whose virtual buckets contain vb
      e = 0;
      for (int e0 = 0; e0 < a.E; e0 += 64) {
        const int ee = e0 + lane;
        const bool hit = ee < a.E && s_vb[ee] <= vb && vb < s_vb[ee + 1];
        const uint64_t m = __ballot(hit);
        if (m) {
          e = e0 + __ffsll(static_cast<unsigned long long>(m)) - 1;
          break;
        }
      }
      p0 = s_off[e] + (vb - s_vb[e]) * NT;
      p1 = min(p0 + NT, s_off[e + 1]);
    }
    const QMat q0 = expert_slice(a.m0, e);
    const QMat q1 = GATEUP ? expert_slice(a.m1, e) : q0;

    const uint16_t* xrow[NT];
    bool xvalid[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      xvalid[j] = p0 + j < p1;
      const int p = xvalid[j] ? p0 + j : p0;
      int src = p;
      if (GATEUP && !a.shared) src = min(max(a.perm[p] / a.k, 0), a.T - 1);
      xrow[j] = a.x + static_cast<size_t>(src) * cols;
    }
    XRaw<CPL, NT> xw;
    load_x_raw<CPL, NT>(xw, xrow, lane, nchunks);

    if constexpr (GATEUP) {
      stream_rows<FMT, BITS, CPL, NT, true, 1>(q0, q1, xw, xvalid, r_begin, r_end, lane, nchunks,
                                            [&](int j, int r, float g, float u) {
                                              if (p0 + j < p1)
                                                a.h[static_cast<size_t>(p0 + j) * rows + r] =
                                                    static_cast<uint16_t>(f32_to_bf16_rne(silu(g) * u));
                                            });
    } else {
      stream_rows<FMT, BITS, CPL, NT, false, 2>(q0, q1, xw, xvalid, r_begin, r_end, lane, nchunks,
                                             [&](int j, int r, float y, float) {
                                               if (p0 + j < p1) {
                                                 const int slot = a.shared ? p0 + j : min(max(a.perm[p0 + j], 0), n - 1);
                                                 a.y[static_cast<size_t>(slot) * rows + r] = y;
                                               }
                                             });
    }
    u += r_end - r_begin;
  }
}

template <int FMT, int BITS, int CPL, int NT, bool GATEUP>
__global__ __launch_bounds__(256) void k_ffn_stream(StreamArgs a) {
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int32_t s_vb[kMaxExperts + 1];
  ffn_stream_body<FMT, BITS, CPL, NT, GATEUP>(a, blockIdx.x, gridDim.x, s_off, s_vb);
}

}  // namespace qsmoe
