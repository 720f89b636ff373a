// Measurement kernels: memory streams of known traffic (the scale for HBM
// byte counters and the achievable read bandwidth) and a dense MFMA loop (the
// sustained shader clock and bf16 matrix rate). Not part of the layer.
#include "common.hpp"
#include "kernels.hpp"

namespace qsmoe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int kProbeBlocks = 2048;  // workgroups of the stream kernels (8 per CU); words of the sink

// Mode 0: every byte of [src, src + bytes) read once, 16 bytes per lane,
// consecutive lanes on consecutive 16-byte pieces. Mode 1: the first 32 bytes
// of every 128-byte line (two 16-byte loads per lane, lanes 128 bytes apart).
// The XOR of the words a workgroup read goes to sink[workgroup] (a plain
// store: atomics on one word from every workgroup would serialise and cost
// more than a small read), so no load can be dropped. bytes is a multiple of
// 128.
template <int MODE>
__global__ __launch_bounds__(256) void k_probe_read(const u32x4_t* __restrict__ src, size_t bytes,
                                                    uint32_t* __restrict__ sink) {
  const size_t n_threads = static_cast<size_t>(gridDim.x) * 256;
  const size_t tid = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  u32x4_t acc = u32x4_t{0u, 0u, 0u, 0u};
  if constexpr (MODE == 0) {
    const size_t n = bytes / 16;
#pragma unroll 4
    for (size_t i = tid; i < n; i += n_threads) {
      const u32x4_t v = __builtin_nontemporal_load(src + i);
      acc ^= v;
    }
  } else {
    const size_t lines = bytes / 128;
#pragma unroll 4
    for (size_t i = tid; i < lines; i += n_threads) {
      const u32x4_t a = __builtin_nontemporal_load(src + 8 * i);
      const u32x4_t b = __builtin_nontemporal_load(src + 8 * i + 1);
      acc ^= a ^ b;
    }
  }
  uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v ^= __shfl_xor(v, m);
  __shared__ uint32_t s_x[4];
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_x[0] ^ s_x[1] ^ s_x[2] ^ s_x[3];
}

// Every 16-byte piece of [dst, dst + bytes) written once with its index.
__global__ __launch_bounds__(256) void k_probe_write(u32x4_t* __restrict__ dst, size_t bytes) {
  const size_t n_threads = static_cast<size_t>(gridDim.x) * 256;
  const size_t n = bytes / 16;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += n_threads) {
    const uint32_t lo = static_cast<uint32_t>(i);
    __builtin_nontemporal_store(u32x4_t{lo, lo, lo, lo}, dst + i);
  }
}

// Dense bf16 MFMA: every wave runs `iters` rounds of 8 independent
// V_MFMA_F32_32X32X16_BF16 chains (no memory traffic in the loop). Wave 0 of
// workgroup 0 records the shader-clock counter (s_memtime) and the 100 MHz
// wall clock (s_memrealtime) around its loop into out[0..3]; each wave adds
// one accumulator element to out[4] so the loop stays live.
__global__ __launch_bounds__(256) void k_probe_mfma(int iters, uint64_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u + lane, 0x3f803f80u, 0x3c003c00u, 0x3f80u));
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, make_uint4(0x3c003c00u, 0x3f803f80u + lane, 0x3f80u, 0x3c003c00u));
  f32x16_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16_t{};
  const bool rec = blockIdx.x == 0 && threadIdx.x == 0;
  uint64_t c0 = 0, w0 = 0;
  if (rec) {
    c0 = clock64();
    w0 = wall_clock64();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  if (rec) {
    const uint64_t c1 = clock64(), w1 = wall_clock64();
    out[0] = c0;
    out[1] = c1;
    out[2] = w0;
    out[3] = w1;
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][lane & 15];
  if (lane == 0) atomicAdd(reinterpret_cast<unsigned long long*>(out + 4), static_cast<unsigned long long>(s > 0.0f));
}

hipError_t launch_probe_stream(const void* buf, size_t bytes, int mode, uint32_t* sink, hipStream_t s) {
  if (mode == 0)
    QSMOE_LAUNCH(k_probe_read<0>, dim3(kProbeBlocks), dim3(256), 0, s, static_cast<const u32x4_t*>(buf), bytes, sink);
  else if (mode == 1)
    QSMOE_LAUNCH(k_probe_read<1>, dim3(kProbeBlocks), dim3(256), 0, s, static_cast<const u32x4_t*>(buf), bytes, sink);
  else
    QSMOE_LAUNCH(k_probe_write, dim3(kProbeBlocks), dim3(256), 0, s, static_cast<u32x4_t*>(const_cast<void*>(buf)),
                 bytes);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int workgroups, int iters, uint64_t* out, hipStream_t s) {
  QSMOE_LAUNCH(k_probe_mfma, dim3(workgroups), dim3(256), 0, s, iters, out);
  return hipGetLastError();
}

}  // namespace qsmoe
