// Bucketing of the T*k (token, slot) assignments by expert: a stable counting
// sort in one workgroup of 16 waves.
//
// The stacked expert tensors (mlx-lm PR "Add DeepSeek-v4 (Flash/Pro)",
// pre-stacked switch_mlp.{gate,up,down}_proj) are run over contiguous buckets
// of assignments, so each expert's weights are streamed once per step.
//
// Wave w owns a contiguous segment of assignments. Pass 1 counts per (wave,
// expert) with LDS atomic adds; a scan over (expert, wave) gives every wave
// its base per expert; in pass 2, lanes holding the same expert id are
// grouped with one ballot per id bit (the group's lowest lane is its
// leader), each lane writes perm[base + rank-within-group] and the leader
// advances the base. (The workgroup runs on one CU, where a wave64 VALU
// instruction takes 4 cycles: grouping in both passes cost ~40 us for 24576
// assignments.) Order within a bucket
// is ascending assignment index, i.e. the sort is stable. Each lane loads the
// ids of kPermBatch consecutive 64-wide rows at once, so one memory latency is
// paid per batch rather than per row; up to kPermKeep batches per wave stay
// in registers for pass 2. When perm fits in LDS beside the histograms,
// pass 2 scatters into LDS and the result is written out with whole-row
// stores (scattered 4-byte global stores from one CU cost ~1 line each).
#include "common.hpp"
#include "kernels.hpp"

namespace qsmoe {

constexpr int kPermWaves = 16;
constexpr int kPermBatch = 8;
constexpr int kPermKeep = 4;                    // batches per wave kept in registers
constexpr size_t kPermLdsMax = 144 * 1024;      // dynamic LDS limit of the kernel

// The valid lanes whose id equals this lane's: per id bit, keep the lanes
// whose bit agrees (the ballot of set bits, complemented where this lane's
// bit is clear). Invalid lanes are cleared by the first ballot alone.
__device__ __forceinline__ uint64_t same_id_mask(bool valid, int id, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const uint32_t bit = (static_cast<uint32_t>(id) >> b) & 1u;
    const uint64_t bb = __ballot(bit != 0);
    const uint64_t flip = static_cast<uint64_t>(bit) - 1ull;  // 0 or all ones
    m &= bb ^ flip;
  }
  return m;
}

__global__ __launch_bounds__(kPermWaves * 64) void k_permute(const int32_t* __restrict__ ids, int n, int E,
                                                             int nbits, int staged, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm, int32_t* err) {
  extern __shared__ int32_t lds[];
  int32_t* hist = lds;                        // [kPermWaves][E]
  int32_t* wave_tot = lds + kPermWaves * E;   // [kPermWaves] scan scratch
  int32_t* perm_lds = wave_tot + kPermWaves;  // [n] when staged
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  const int nthreads = kPermWaves * 64;
  for (int i = tid; i < kPermWaves * E; i += nthreads) hist[i] = 0;
  __syncthreads();

  const int seg = ((n + kPermWaves - 1) / kPermWaves + 63) & ~63;
  const int s0 = min(n, w * seg), s1 = min(n, s0 + seg);
  const uint64_t lt_mask = (1ull << lane) - 1ull;

  // pass 1: per-wave histogram (the first kPermKeep batches' ids are kept)
  int keep[kPermKeep][kPermBatch];
  int bi = 0;
  for (int base = s0; base < s1; base += 64 * kPermBatch, ++bi) {
    int idv[kPermBatch];
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u) {
      const int a = base + u * 64 + lane;
      idv[u] = a < s1 ? ids[a] : 0;
    }
#pragma unroll
    for (int k = 0; k < kPermKeep; ++k)
      if (bi == k) {
#pragma unroll
        for (int u = 0; u < kPermBatch; ++u) keep[k][u] = idv[u];
      }
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u) {
      const int a = base + u * 64 + lane;
      const bool valid = a < s1;
      int id = idv[u];
      if (valid && (id < 0 || id >= E)) {
        set_device_error(err, 4);
        id = 0;
      }
      if (valid) atomicAdd(&hist[w * E + id], 1);
    }
  }
  __syncthreads();

  // per-expert totals, exclusive scan over experts, per-wave bases
  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += nthreads) {
    const int e = e0 + tid;
    int tot = 0;
    if (e < E)
      for (int v = 0; v < kPermWaves; ++v) tot += hist[v * E + e];
    // inclusive wave scan
    int incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wave_tot[w] = incl;
    __syncthreads();
    int wave_base = 0, chunk_total = 0;
    for (int v = 0; v < kPermWaves; ++v) {
      if (v < w) wave_base += wave_tot[v];
      chunk_total += wave_tot[v];
    }
    const int excl = carry + wave_base + incl - tot;
    if (e < E) {
      offsets[e] = excl;
      int run = excl;
      for (int v = 0; v < kPermWaves; ++v) {
        const int c = hist[v * E + e];
        hist[v * E + e] = run;
        run += c;
      }
    }
    carry += chunk_total;
    __syncthreads();
  }
  if (tid == 0) offsets[E] = n;
  __syncthreads();

  // pass 2: stable scatter
  bi = 0;
  for (int base = s0; base < s1; base += 64 * kPermBatch, ++bi) {
    int idv[kPermBatch];
    if (bi < kPermKeep) {
#pragma unroll
      for (int k = 0; k < kPermKeep; ++k)
        if (bi == k) {
#pragma unroll
          for (int u = 0; u < kPermBatch; ++u) idv[u] = keep[k][u];
        }
    } else {
#pragma unroll
      for (int u = 0; u < kPermBatch; ++u) {
        const int a = base + u * 64 + lane;
        idv[u] = a < s1 ? ids[a] : 0;
      }
    }
#pragma unroll
    for (int u = 0; u < kPermBatch; ++u) {
      const int a = base + u * 64 + lane;
      const bool valid = a < s1;
      int id = idv[u];
      if (id < 0 || id >= E) id = 0;
      const uint64_t m = same_id_mask(valid, id, nbits);
      if (valid) {
        const int pos = hist[w * E + id] + __popcll(m & lt_mask);
        if (staged)
          perm_lds[pos] = a;
        else
          perm[pos] = a;
      }
      if (valid && (m & lt_mask) == 0) hist[w * E + id] += __popcll(m);
    }
  }
  if (staged) {
    __syncthreads();
    for (int i = tid; i < n; i += nthreads) perm[i] = perm_lds[i];
  }
}

hipError_t launch_permute(const int32_t* ids, int n, int E, int32_t* offsets, int32_t* perm, int32_t* err,
                          hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const size_t hist_lds = (static_cast<size_t>(kPermWaves) * E + kPermWaves) * sizeof(int32_t);
  const size_t staged_lds = hist_lds + static_cast<size_t>(n) * sizeof(int32_t);
  const int staged = staged_lds <= kPermLdsMax ? 1 : 0;
  // up to 1024 experts (64 KiB of histograms), or a staged perm, needs more
  // than the default 64 KiB of dynamic LDS
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k_permute),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kPermLdsMax);
  if (attr != hipSuccess) return attr;
  QSMOE_LAUNCH(k_permute, dim3(1), dim3(kPermWaves * 64), staged ? staged_lds : hist_lds, s, ids, n, E, nbits,
               staged, offsets, perm, err);
  return hipGetLastError();
}

}  // namespace qsmoe
