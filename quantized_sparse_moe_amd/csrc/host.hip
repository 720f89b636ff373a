// C ABI of the MoE layer library: host validation, workspace carving and the
// launch sequence. Nothing here allocates device memory or synchronises,
// except moe_device_error, which exists for tests.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "qsmoe.h"
#include "kernels.hpp"

using namespace qsmoe;

namespace {

// Every workspace starts with a 256-byte header; int32 [0] is the sticky
// device error word. moe_workspace_init zeroes the header.
constexpr size_t kHeader = 256;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int ilog2(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

moe_status check_qtensor(const moe_qtensor& q, int experts, int rows, int cols) {
  if (q.codes == nullptr || q.scales == nullptr) return MOE_ERR_INVALID_ARG;
  if (q.rows != rows || q.cols != cols || q.num_experts != experts || rows < 1 || cols < 1) return MOE_ERR_INVALID_ARG;
  if (q.format == MOE_FMT_AFFINE) {
    if (q.biases == nullptr) return MOE_ERR_INVALID_ARG;
    if (!(q.bits == 2 || q.bits == 3 || q.bits == 4 || q.bits == 8)) return MOE_ERR_UNSUPPORTED;
    if (!(q.group_size == 32 || q.group_size == 64 || q.group_size == 128)) return MOE_ERR_UNSUPPORTED;
    if (!aligned(q.scales, 2) || !aligned(q.biases, 2)) return MOE_ERR_ALIGNMENT;
  } else if (q.format == MOE_FMT_MXFP4) {
    if (q.bits != 4 || q.group_size != 32) return MOE_ERR_UNSUPPORTED;
  } else if (q.format == MOE_FMT_MXFP8) {
    if (q.bits != 8 || q.group_size != 32) return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  if (cols % 32 != 0 || cols % q.group_size != 0 || cols > 8192) return MOE_ERR_UNSUPPORTED;
  if (!aligned(q.codes, 16)) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

QMat to_qmat(const moe_qtensor& q) {
  QMat m;
  m.codes = q.codes;
  m.scales = q.scales;
  m.biases = static_cast<const uint16_t*>(q.format == MOE_FMT_AFFINE ? q.biases : nullptr);
  m.fmt = q.format;
  m.bits = q.bits;
  m.group = q.group_size;
  m.rows = q.rows;
  m.cols = q.cols;
  m.row_words = q.cols * q.bits / 32;
  m.row_groups = q.cols / q.group_size;
  m.gshift = ilog2(q.group_size / 32);
  return m;
}

// Shape of an expert set: d = gate.cols, I = gate.rows.
moe_status check_experts(const moe_experts& x, int experts, int d_expected) {
  const int d = x.gate.cols, I = x.gate.rows;
  if (d_expected > 0 && d != d_expected) return MOE_ERR_INVALID_ARG;
  moe_status s;
  if ((s = check_qtensor(x.gate, experts, I, d)) != MOE_OK) return s;
  if ((s = check_qtensor(x.up, experts, I, d)) != MOE_OK) return s;
  if ((s = check_qtensor(x.down, experts, d, I)) != MOE_OK) return s;
  if (x.up.format != x.gate.format || x.up.bits != x.gate.bits || x.up.group_size != x.gate.group_size)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_router(const moe_router& r) {
  if (r.weight == nullptr) return MOE_ERR_INVALID_ARG;
  if (r.num_experts < 1 || r.num_experts > 1024) return MOE_ERR_UNSUPPORTED;
  if (r.top_k < 1 || r.top_k > r.num_experts || r.top_k > 8) return MOE_ERR_INVALID_ARG;
  if (r.hidden < 32 || r.hidden % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (!aligned(r.weight, 16)) return MOE_ERR_ALIGNMENT;
  if (r.bias != nullptr && !aligned(r.bias, 4)) return MOE_ERR_ALIGNMENT;
  if (r.mode == MOE_ROUTE_HASH) {
    if (r.tid2eid == nullptr || r.vocab < 1) return MOE_ERR_INVALID_ARG;
    if (!aligned(r.tid2eid, 4)) return MOE_ERR_ALIGNMENT;
  } else if (r.mode != MOE_ROUTE_TOPK) {
    return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

moe_status check_layer(const moe_layer* L) {
  if (L == nullptr) return MOE_ERR_INVALID_ARG;
  moe_status s;
  if ((s = check_router(L->router)) != MOE_OK) return s;
  if ((s = check_experts(L->routed, L->router.num_experts, L->router.hidden)) != MOE_OK) return s;
  if (L->shared && (s = check_experts(*L->shared, 1, L->router.hidden)) != MOE_OK) return s;
  return MOE_OK;
}

// moe_route's workspace in top-k mode: header | logits fp32 [T][E] | packed
// keys uint64 [T][E] | scores fp32 [T][E] (each region 256-byte aligned).
struct RouteLayout {
  size_t logits, keys, scores, total;
};

RouteLayout route_layout(const moe_router& r, int T) {
  const size_t te = static_cast<size_t>(T) * r.num_experts;
  RouteLayout l{kHeader, 0, 0, kHeader};
  if (r.mode != MOE_ROUTE_TOPK) return l;
  l.keys = l.logits + align_up(te * 4);
  l.scores = l.keys + align_up(te * 8);
  l.total = l.scores + align_up(te * 4);
  return l;
}

// fp32 partial sums of the shared expert's K-split projections, bounded for
// every token count up to T: the slice count only falls as T grows (it is 1
// from some T_cap on), so slices(8) * min(T, T_cap) rows always suffice.
size_t shared_part_bytes(const moe_experts& sh, int T) {
  auto rows_bound = [T](const QMat& m, bool gateup) -> size_t {
    const int ks8 = mfma_shared_ksplit(m, gateup, 8);
    if (ks8 <= 1) return 0;
    int tcap = 8;
    while (mfma_shared_ksplit(m, gateup, tcap) > 1) tcap *= 2;
    return static_cast<size_t>(ks8) * std::min(T, tcap);
  };
  const QMat g = to_qmat(sh.gate), dn = to_qmat(sh.down);
  const size_t a = rows_bound(g, true) * 2 * g.rows * 4, b = rows_bound(dn, false) * dn.rows * 4;
  return align_up(std::max(a, b));
}

size_t ffn_ws_bytes(const moe_experts& routed, const moe_experts* shared, int T, int k) {
  size_t b = kHeader + align_up(static_cast<size_t>(T) * k * routed.gate.rows * 2);
  if (shared) b += align_up(static_cast<size_t>(T) * shared->gate.rows * 2) + shared_part_bytes(*shared, T);
  return b;
}

struct FwdLayout {
  size_t ids, w, logits, keys, scores, offsets, perm, h, h_sh, sh_part, y_slot, y_sh, total;
};

// The fused small-batch path takes at most this many tokens (the decode
// kernels check the rest of their conditions themselves).
constexpr int kSmallBatch = 4;

FwdLayout forward_layout(const moe_layer& L, int T) {
  const int k = L.router.top_k, E = L.router.num_experts, d = L.router.hidden;
  const size_t tk = static_cast<size_t>(T) * k;
  FwdLayout f;
  size_t o = kHeader;
  f.ids = o;
  o += align_up(tk * 4);
  f.w = o;
  o += align_up(tk * 4);
  // logits, packed ranking keys and scores of every expert: top-k routing,
  // and hash routing on the small-batch path (whose launch 1 computes every
  // expert's logit and score)
  const bool small = T <= kSmallBatch;
  const bool all_experts = L.router.mode == MOE_ROUTE_TOPK || small;
  const size_t te = static_cast<size_t>(T) * E;
  f.logits = o;
  o += all_experts ? align_up(te * 4) : 0;
  f.keys = o;
  o += all_experts ? align_up(te * 8) : 0;
  f.scores = o;
  o += all_experts ? align_up(te * 4) : 0;
  f.offsets = o;
  o += align_up((E + 1) * 4);
  f.perm = o;
  o += align_up(tk * 4);
  f.h = o;
  o += align_up(tk * L.routed.gate.rows * 2);
  f.h_sh = o;
  o += L.shared ? align_up(static_cast<size_t>(T) * L.shared->gate.rows * 2) : 0;
  f.sh_part = o;
  o += L.shared ? shared_part_bytes(*L.shared, T) : 0;
  f.y_slot = o;
  o += align_up(tk * d * 4);
  f.y_sh = o;
  o += L.shared ? align_up(static_cast<size_t>(T) * d * 4) : 0;
  f.total = o;
  return f;
}

// Optional timing probe of moe_forward_probed: every launch takes the next
// (start, stop) event pair, timestamped by the dispatch itself, and the
// name given to mark() labels the launches made since the previous mark().
struct Probe {
  hipEvent_t* events;
  int32_t n_events;
  const char** names;
  int32_t count;   // launches that took an event pair
  int32_t named;   // launches already labelled
  bool overflow;
};
thread_local Probe* g_probe = nullptr;

}  // namespace

namespace qsmoe {
bool probe_events(hipEvent_t* start, hipEvent_t* stop) {
  if (g_probe == nullptr) return false;
  Probe& p = *g_probe;
  if (2 * (p.count + 1) > p.n_events) {
    p.overflow = true;
    return false;
  }
  *start = p.events[2 * p.count];
  *stop = p.events[2 * p.count + 1];
  p.count += 1;
  return true;
}
}  // namespace qsmoe

namespace {

hipError_t mark(hipError_t launched, const char* name, hipStream_t) {
  if (g_probe == nullptr) return launched;
  Probe& p = *g_probe;
  for (; p.named < p.count; ++p.named) p.names[p.named] = name;
  return launched;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

moe_status run_route(const moe_router& r, const uint16_t* x, const int32_t* token_ids, int T, int32_t* ids,
                     float* w, float* logits, uint64_t* keys, float* scores, int32_t* err, hipStream_t s) {
  hipError_t e;
  if (r.mode == MOE_ROUTE_HASH) {
    e = mark(launch_router_hash(x, r.weight, token_ids, r.tid2eid, T, r.num_experts, r.top_k, r.hidden, r.vocab,
                                r.routed_scale, ids, w, err, s),
             "router_hash", s);
    return hip_status(e);
  }
  if ((e = mark(launch_router_logits(x, r.weight, T, r.num_experts, r.hidden, logits, s), "router_logits", s)) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return hip_status(mark(
      launch_router_topk(logits, r.bias, T, r.num_experts, r.top_k, r.routed_scale, ids, w, keys, scores, s),
      "router_topk", s));
}

bool mfma_worthwhile(const QMat& m, int T, int k, int E) {
  const int64_t per_expert = m.fmt == 0 && m.bits < 4 ? 1 : 4;
  return static_cast<int64_t>(T) * k >= per_expert * E;
}

moe_status run_ffn(const moe_experts& routed, const moe_experts* shared, const uint16_t* x, int T, int k, int E,
                   const int32_t* offsets, const int32_t* perm, float* y_slot, float* y_sh, uint16_t* h,
                   uint16_t* h_sh, float* sh_part, hipStream_t s) {
  // The shared expert (every token, token order) is a dense GEMM on the
  // matrix cores from 8 tokens on (K split over workgroups while its tiles
  // are too few to fill the chip), a streaming GEMV below that.
  bool sh_mfma = false;
  int ks_gu = 1, ks_dn = 1;
  if (shared) {
    const QMat sg = to_qmat(shared->gate), sd = to_qmat(shared->down);
    sh_mfma = T >= 8 && mfma_supported(sg, true, T, 1) && mfma_supported(sd, false, T, 1);
    if (sh_mfma) {
      ks_gu = mfma_shared_ksplit(sg, true, T);
      ks_dn = mfma_shared_ksplit(sd, false, T);
    }
    GateUpArgs g{sg, to_qmat(shared->up), x, T, k, 1, nullptr, nullptr, 1, h_sh, ks_gu, sh_part};
    if (sh_mfma) {
      if (mark(launch_mfma_gateup(g, s), "shared_gateup_mfma", s) != hipSuccess) return MOE_ERR_HIP;
      if (ks_gu > 1 && mark(launch_swiglu_parts(sh_part, ks_gu, T, sg.rows, h_sh, s), "shared_swiglu", s) !=
                           hipSuccess)
        return MOE_ERR_HIP;
    } else if (mark(launch_gateup(g, s), "shared_gateup", s) != hipSuccess) {
      return MOE_ERR_HIP;
    }
  }
  // Grouped GEMM on the matrix cores once buckets average enough tokens
  // (measured crossovers: 4 per expert for 4-bit codes, 1 for 2- and 3-bit,
  // whose GEMV decode costs more per byte); each projection picks its own
  // path (both keep h in bucket order).
  const QMat qg = to_qmat(routed.gate), qd = to_qmat(routed.down);
  const bool mfma_gu = mfma_worthwhile(qg, T, k, E) && mfma_supported(qg, true, T, k);
  const bool mfma_dn = mfma_worthwhile(qd, T, k, E) && mfma_supported(qd, false, T, k);
  GateUpArgs g{to_qmat(routed.gate), to_qmat(routed.up), x, T, k, E, offsets, perm, 0, h};
  if (mfma_gu) {
    if (mark(launch_mfma_gateup(g, s), "routed_gateup_mfma", s) != hipSuccess) return MOE_ERR_HIP;
  } else if (mark(launch_gateup(g, s), "routed_gateup", s) != hipSuccess) {
    return MOE_ERR_HIP;
  }
  if (shared) {
    DownArgs dn{to_qmat(shared->down), h_sh, T, k, 1, nullptr, nullptr, 1, y_sh, ks_dn, sh_part};
    if (sh_mfma) {
      if (mark(launch_mfma_down(dn, s), "shared_down_mfma", s) != hipSuccess) return MOE_ERR_HIP;
      if (ks_dn > 1 && mark(launch_sum_parts(sh_part, ks_dn, static_cast<int64_t>(T) * dn.down.rows, y_sh, s),
                            "shared_sum", s) != hipSuccess)
        return MOE_ERR_HIP;
    } else if (mark(launch_down(dn, s), "shared_down", s) != hipSuccess) {
      return MOE_ERR_HIP;
    }
  }
  DownArgs dn{to_qmat(routed.down), h, T, k, E, offsets, perm, 0, y_slot};
  if (mfma_dn) return hip_status(mark(launch_mfma_down(dn, s), "routed_down_mfma", s));
  return hip_status(mark(launch_down(dn, s), "routed_down", s));
}

}  // namespace

extern "C" {

const char* moe_version(void) { return "qsmoe 0.1.0 (gfx950)"; }

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported format or shape";
    case MOE_ERR_ALIGNMENT: return "misaligned pointer";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

moe_status moe_quantize_affine(const uint16_t* w_bf16, int64_t rows, int32_t cols, int32_t bits, int32_t group_size,
                               uint32_t* codes, uint16_t* scales, uint16_t* biases, int32_t* err,
                               hipStream_t stream) {
  if (rows < 0 || cols < 0) return MOE_ERR_INVALID_ARG;
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 8)) return MOE_ERR_UNSUPPORTED;
  if (!(group_size == 32 || group_size == 64 || group_size == 128)) return MOE_ERR_UNSUPPORTED;
  if (cols % group_size != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (w_bf16 == nullptr || codes == nullptr || scales == nullptr || biases == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(w_bf16, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(biases, 2) ||
      !aligned(err, 4))
    return MOE_ERR_ALIGNMENT;
  return hip_status(launch_quantize_affine(w_bf16, rows, cols, bits, group_size, codes, scales, biases, err, stream));
}

moe_status moe_mhc_sinkhorn(const float* logits, int64_t T, int32_t n, int32_t iters, float eps, float* out,
                            hipStream_t stream) {
  if (T < 0 || iters < 0 || !(eps >= 0.0f) || eps == INFINITY) return MOE_ERR_INVALID_ARG;
  if (!(n == 2 || n == 4 || n == 8)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (logits == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(out, 4)) return MOE_ERR_ALIGNMENT;
  return hip_status(launch_mhc_sinkhorn(logits, T, n, iters, eps, out, stream));
}

size_t moe_workspace_size(const moe_layer* layer, int32_t max_tokens) {
  if (max_tokens < 0 || check_layer(layer) != MOE_OK) return 0;
  // Every region grows with T, but the small-batch regions of a hash layer
  // exist only up to kSmallBatch tokens: the larger of the two layouts serves
  // every T <= max_tokens.
  const int mt = max_tokens > 0 ? max_tokens : 1;
  return std::max(forward_layout(*layer, std::min(mt, kSmallBatch)).total, forward_layout(*layer, mt).total);
}

moe_status moe_workspace_layout(const moe_layer* layer, int32_t T, moe_ws_layout* out) {
  if (out == nullptr || T < 1) return MOE_ERR_INVALID_ARG;
  moe_status s = check_layer(layer);
  if (s != MOE_OK) return s;
  const moe_layer& L = *layer;
  const FwdLayout f = forward_layout(L, T);
  const bool small = T <= kSmallBatch, all_experts = L.router.mode == MOE_ROUTE_TOPK || small;
  DecodeArgs da{};
  da.T = T;
  da.d = L.router.hidden;
  da.E = L.router.num_experts;
  da.k = L.router.top_k;
  da.gate = to_qmat(L.routed.gate);
  da.up = to_qmat(L.routed.up);
  da.down = to_qmat(L.routed.down);
  da.has_shared = L.shared != nullptr;
  if (L.shared) {
    da.sgate = to_qmat(L.shared->gate);
    da.sup = to_qmat(L.shared->up);
    da.sdown = to_qmat(L.shared->down);
  }
  const bool fused = decode_path_supported(da);
  *out = moe_ws_layout{};
  out->total = f.total;
  out->fused = fused ? 1 : 0;
  out->ids = f.ids;
  out->weights = f.w;
  out->logits = all_experts ? f.logits : 0;
  out->keys = all_experts ? f.keys : 0;
  out->scores = all_experts ? f.scores : 0;
  out->offsets = fused ? 0 : f.offsets;
  out->perm = fused ? 0 : f.perm;
  out->h = f.h;
  out->h_shared = L.shared ? f.h_sh : 0;
  out->y_slot = fused ? 0 : f.y_slot;
  const bool y_sh = L.shared && (!fused || dec_shared_in_gateup(da));
  out->y_shared = y_sh ? f.y_sh : 0;
  return MOE_OK;
}

moe_status moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (ws == nullptr || ws_bytes < kHeader) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  return hip_status(launch_fill_i32(static_cast<int32_t*>(ws), 0, static_cast<int>(kHeader / 4), stream));
}

moe_status moe_router_logits(const moe_router* router, const uint16_t* x_bf16, int32_t T, float* logits,
                             hipStream_t stream) {
  if (router == nullptr || T < 0) return MOE_ERR_INVALID_ARG;
  moe_status s = check_router(*router);
  if (s != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (x_bf16 == nullptr || logits == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16)) return MOE_ERR_ALIGNMENT;
  return hip_status(launch_router_logits(x_bf16, router->weight, T, router->num_experts, router->hidden, logits,
                                         stream));
}

moe_status moe_route(const moe_router* router, const uint16_t* x_bf16, const int32_t* token_ids, int32_t T,
                     int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (router == nullptr || T < 0) return MOE_ERR_INVALID_ARG;
  moe_status s = check_router(*router);
  if (s != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (x_bf16 == nullptr || topk_ids == nullptr || topk_w == nullptr) return MOE_ERR_INVALID_ARG;
  if (router->mode == MOE_ROUTE_HASH && token_ids == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16)) return MOE_ERR_ALIGNMENT;
  const RouteLayout rl = route_layout(*router, T);
  if (ws == nullptr || ws_bytes < rl.total) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  return run_route(*router, x_bf16, token_ids, T, topk_ids, topk_w, at<float>(ws, rl.logits),
                   at<uint64_t>(ws, rl.keys), at<float>(ws, rl.scores), at<int32_t>(ws, 0), stream);
}

moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* expert_offsets,
                       int32_t* perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (E < 1 || E > 1024) return MOE_ERR_UNSUPPORTED;
  if (k < 1 || k > E || k > 8) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (topk_ids == nullptr || expert_offsets == nullptr || perm == nullptr) return MOE_ERR_INVALID_ARG;
  if (ws == nullptr || ws_bytes < kHeader) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  return hip_status(launch_permute(topk_ids, T * k, E, expert_offsets, perm, at<int32_t>(ws, 0), stream));
}

moe_status moe_expert_ffn(const moe_experts* routed, const moe_experts* shared, const uint16_t* x_bf16, int32_t T,
                          int32_t k, const int32_t* expert_offsets, const int32_t* perm, float* y_slot,
                          float* y_shared, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (routed == nullptr || T < 0) return MOE_ERR_INVALID_ARG;
  const int E = routed->gate.num_experts;
  moe_status s = check_experts(*routed, E, 0);
  if (s != MOE_OK) return s;
  if (E < 1 || E > 1024) return MOE_ERR_UNSUPPORTED;
  if (k < 1 || k > E || k > 8) return MOE_ERR_INVALID_ARG;
  if (shared && (s = check_experts(*shared, 1, routed->gate.cols)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (x_bf16 == nullptr || expert_offsets == nullptr || perm == nullptr || y_slot == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (shared) {
    if (y_shared == nullptr) return MOE_ERR_INVALID_ARG;
    if (!aligned(y_shared, 16)) return MOE_ERR_ALIGNMENT;
  }
  if (!aligned(x_bf16, 16) || !aligned(y_slot, 16)) return MOE_ERR_ALIGNMENT;
  if (ws == nullptr || ws_bytes < ffn_ws_bytes(*routed, shared, T, k)) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  uint16_t* h = at<uint16_t>(ws, kHeader);
  const size_t o_sh = kHeader + align_up(static_cast<size_t>(T) * k * routed->gate.rows * 2);
  uint16_t* h_sh = at<uint16_t>(ws, o_sh);
  float* sh_part =
      shared ? at<float>(ws, o_sh + align_up(static_cast<size_t>(T) * shared->gate.rows * 2)) : nullptr;
  return run_ffn(*routed, shared, x_bf16, T, k, E, expert_offsets, perm, y_slot, y_shared, h, h_sh, sh_part,
                 stream);
}

moe_status moe_combine(const float* y_slot, const float* topk_w, const float* y_shared, int32_t T, int32_t k,
                       int32_t d, int32_t out_dtype, void* out, hipStream_t stream) {
  if (T < 0 || k < 1 || d < 1) return MOE_ERR_INVALID_ARG;
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32) return MOE_ERR_INVALID_ARG;
  if (d % 4 != 0) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (y_slot == nullptr || topk_w == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(y_slot, 16) || !aligned(out, 8) || (y_shared && !aligned(y_shared, 16))) return MOE_ERR_ALIGNMENT;
  if (out_dtype == MOE_OUT_F32 && !aligned(out, 16)) return MOE_ERR_ALIGNMENT;
  return hip_status(launch_combine(y_slot, topk_w, y_shared, T, k, d, out_dtype == MOE_OUT_F32, out, stream));
}

}  // extern "C"

namespace {

// moe_forward's checks of everything but the workspace. T == 0 passes (the
// caller returns MOE_OK without a launch).
moe_status check_forward_args(const moe_layer* layer, const uint16_t* x_bf16, const int32_t* token_ids, int32_t T,
                              int32_t out_dtype, const void* out) {
  if (T < 0) return MOE_ERR_INVALID_ARG;
  moe_status s = check_layer(layer);
  if (s != MOE_OK) return s;
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (x_bf16 == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
  if (layer->router.mode == MOE_ROUTE_HASH && token_ids == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16) || !aligned(out, 16)) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

// The launch sequence of one forward on a validated layer and a workspace of
// at least f.total bytes.
moe_status run_forward(const moe_layer& L, const uint16_t* x_bf16, const int32_t* token_ids, int32_t T,
                       int32_t out_dtype, void* out, void* ws, const FwdLayout& f, hipStream_t stream) {
  moe_status s;
  const int k = L.router.top_k, E = L.router.num_experts, d = L.router.hidden;
  if (L.router.mode == MOE_ROUTE_TOPK || L.router.mode == MOE_ROUTE_HASH) {
    DecodeArgs da{};
    da.hash = L.router.mode == MOE_ROUTE_HASH;
    da.token_ids = token_ids;
    da.tid2eid = L.router.tid2eid;
    da.vocab = L.router.vocab;
    da.err = at<int32_t>(ws, 0);
    da.x = x_bf16;
    da.T = T;
    da.d = d;
    da.E = E;
    da.k = k;
    da.routed_scale = L.router.routed_scale;
    da.wr = L.router.weight;
    da.bias = L.router.bias;
    da.logits = at<float>(ws, f.logits);
    da.keys = at<uint64_t>(ws, f.keys);
    da.scores = at<float>(ws, f.scores);
    da.gate = to_qmat(L.routed.gate);
    da.up = to_qmat(L.routed.up);
    da.down = to_qmat(L.routed.down);
    da.h = at<uint16_t>(ws, f.h);
    da.has_shared = L.shared != nullptr;
    if (L.shared) {
      da.sgate = to_qmat(L.shared->gate);
      da.sup = to_qmat(L.shared->up);
      da.sdown = to_qmat(L.shared->down);
      da.h_sh = at<uint16_t>(ws, f.h_sh);
      da.y_sh = at<float>(ws, f.y_sh);
    }
    da.out = out;
    da.out_f32 = out_dtype == MOE_OUT_F32;
    da.ids = at<int32_t>(ws, f.ids);
    da.w = at<float>(ws, f.w);
    if (decode_path_supported(da)) {
      if (mark(launch_dec_router(da, stream), "dec_router", stream) != hipSuccess) return MOE_ERR_HIP;
      if (mark(launch_dec_gateup(da, stream), "dec_gateup", stream) != hipSuccess) return MOE_ERR_HIP;
      return hip_status(mark(launch_dec_down_combine(da, stream), "dec_down_combine", stream));
    }
  }
  int32_t* err = at<int32_t>(ws, 0);
  int32_t* ids = at<int32_t>(ws, f.ids);
  float* w = at<float>(ws, f.w);
  int32_t* offsets = at<int32_t>(ws, f.offsets);
  int32_t* perm = at<int32_t>(ws, f.perm);
  float* y_slot = at<float>(ws, f.y_slot);
  float* y_sh = L.shared ? at<float>(ws, f.y_sh) : nullptr;
  if ((s = run_route(L.router, x_bf16, token_ids, T, ids, w, at<float>(ws, f.logits), at<uint64_t>(ws, f.keys),
                     at<float>(ws, f.scores), err, stream)) != MOE_OK)
    return s;
  if (mark(launch_permute(ids, T * k, E, offsets, perm, err, stream), "permute", stream) != hipSuccess)
    return MOE_ERR_HIP;
  if ((s = run_ffn(L.routed, L.shared, x_bf16, T, k, E, offsets, perm, y_slot, y_sh, at<uint16_t>(ws, f.h),
                   at<uint16_t>(ws, f.h_sh), at<float>(ws, f.sh_part), stream)) != MOE_OK)
    return s;
  return hip_status(
      mark(launch_combine(y_slot, w, y_sh, T, k, d, out_dtype == MOE_OUT_F32, out, stream), "combine", stream));
}

// The allocation-free variant's workspace: one array per GPU, resolved to its
// device address once per device (hipGetSymbolAddress with that device
// current); host code uses only the resolved address.
constexpr size_t kStaticScratchBytes = size_t{64} << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status static_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_layer* layer, const uint16_t* x_bf16, const int32_t* token_ids, int32_t T,
                       int32_t out_dtype, void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status s = check_forward_args(layer, x_bf16, token_ids, T, out_dtype, out);
  if (s != MOE_OK || T == 0) return s;
  if (ws == nullptr) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  const FwdLayout f = forward_layout(*layer, T);
  if (ws_bytes < f.total) return MOE_ERR_WORKSPACE;
  return run_forward(*layer, x_bf16, token_ids, T, out_dtype, out, ws, f, stream);
}

moe_status moe_forward_noalloc(const moe_layer* layer, const uint16_t* x_bf16, const int32_t* token_ids, int32_t T,
                               int32_t out_dtype, void* out, hipStream_t stream) {
  moe_status s = check_forward_args(layer, x_bf16, token_ids, T, out_dtype, out);
  if (s != MOE_OK || T == 0) return s;
  const FwdLayout f = forward_layout(*layer, T);
  if (f.total > kStaticScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((s = static_scratch(&ws)) != MOE_OK) return s;
  // the sticky error word starts each call at zero (a kernel, not a memset)
  if (launch_fill_i32(static_cast<int32_t*>(ws), 0, static_cast<int>(kHeader / 4), stream) != hipSuccess)
    return MOE_ERR_HIP;
  return run_forward(*layer, x_bf16, token_ids, T, out_dtype, out, ws, f, stream);
}

moe_status moe_forward_probed(const moe_layer* layer, const uint16_t* x_bf16, const int32_t* token_ids, int32_t T,
                              int32_t out_dtype, void* out, void* ws, size_t ws_bytes, hipStream_t stream,
                              hipEvent_t* events, int32_t n_events, const char** names, int32_t* n_kernels) {
  if (events == nullptr || names == nullptr || n_kernels == nullptr || n_events < 2) return MOE_ERR_INVALID_ARG;
  Probe p{events, n_events, names, 0, 0, false};
  *n_kernels = 0;
  g_probe = &p;
  const moe_status s = moe_forward(layer, x_bf16, token_ids, T, out_dtype, out, ws, ws_bytes, stream);
  g_probe = nullptr;
  *n_kernels = p.count;
  if (s == MOE_OK && p.overflow) return MOE_ERR_INVALID_ARG;
  return s;
}

moe_status moe_probe_stream(void* buf, size_t bytes, int32_t mode, uint32_t* sink, hipStream_t stream) {
  if (buf == nullptr || bytes == 0 || bytes % 128 != 0 || mode < 0 || mode > 2) return MOE_ERR_INVALID_ARG;
  if (mode != 2 && sink == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(buf, 16) || (sink != nullptr && !aligned(sink, 4))) return MOE_ERR_ALIGNMENT;
  return hip_status(launch_probe_stream(buf, bytes, mode, sink, stream));
}

moe_status moe_probe_mfma(int32_t workgroups, int32_t iters, uint64_t* out, hipStream_t stream) {
  if (workgroups < 1 || iters < 1 || out == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(out, 8)) return MOE_ERR_ALIGNMENT;
  return hip_status(launch_probe_mfma(workgroups, iters, out, stream));
}

moe_status moe_device_error(const void* ws, int32_t* code_out, hipStream_t stream) {
  if (ws == nullptr || code_out == nullptr) return MOE_ERR_INVALID_ARG;
  if (hipStreamSynchronize(stream) != hipSuccess) return MOE_ERR_HIP;
  return hip_status(hipMemcpy(code_out, ws, sizeof(int32_t), hipMemcpyDeviceToHost));
}

}  // extern "C"
