// C ABI of libmoe: argument validation, workspace carving and the launch sequence of
// the layer's forward pass.  The contract of every entry point is documented in
// include/moe.h.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "moe_internal.h"

namespace moe {

static moe_status_t validate(const moe_desc_t* d) {
  if (!d) return MOE_E_NULL;
  if (d->T < 0 || d->d_model <= 0 || d->n_experts < 1 || d->d_ff <= 0 || d->top_k < 1 ||
      d->top_k > d->n_experts || d->n_shared < 0 || d->n_shared > 1 ||
      !isfinite(d->capacity_factor))
    return MOE_E_SHAPE;
  if (d->dtype != MOE_DTYPE_F32 && d->dtype != MOE_DTYPE_BF16) return MOE_E_UNSUPPORTED;
  if (d->out_dtype != MOE_DTYPE_F32 && d->out_dtype != MOE_DTYPE_BF16) return MOE_E_UNSUPPORTED;
  if (d->n_experts > kMaxExperts || d->top_k > kMaxTopK) return MOE_E_UNSUPPORTED;
  if (d->d_model % 64 || d->d_ff % 64 || d->d_model > 65536 || d->d_ff > 65536)
    return MOE_E_UNSUPPORTED;
  // 32-bit element offsets inside the kernels.  T is bounded first, so that with every
  // other field already bounded above none of the products below can overflow.
  if (d->T > (int64_t)INT32_MAX / 32) return MOE_E_UNSUPPORTED;
  const int64_t rows = d->T * d->top_k + d->n_shared * d->T;
  if (rows > (int64_t)INT32_MAX || d->T * d->d_model > (int64_t)INT32_MAX ||
      rows * d->d_ff > (int64_t)INT32_MAX || d->d_ff * d->d_model > (int64_t)INT32_MAX)
    return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

Workspace carve_workspace(const moe_desc_t& d, void* base) {
  const RoutePlan rp = route_plan(d);
  const int64_t TK = d.T * d.top_k, E = d.n_experts;
  const int64_t rows = TK + d.n_shared * d.T;
  const int64_t nbd = ceil_div(TK, kDispatchChunk);
  const int64_t nbh = rp.n_blocks > nbd ? rp.n_blocks : nbd;
  const size_t esz = d.dtype == MOE_DTYPE_BF16 ? 2 : 4;
  char* p = (char*)base;
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? (void*)(p + off) : nullptr;
    off += align256(bytes > 0 ? bytes : 1);
    return r;
  };
  Workspace w{};
  w.topk_idx = (int32_t*)take(TK * 4);
  w.topk_w = (float*)take(TK * 4);
  w.p_part = (float*)take(rp.n_blocks * E * 4);
  w.cnt_part = (int32_t*)take(nbh * E * 4);
  w.counts = (int32_t*)take(E * 4);
  w.ctr = (int32_t*)take(kTileCounters * 4);
  w.offsets = (int32_t*)take((E + 1) * 4);
  w.perm_src = (int32_t*)take(TK * 4);
  w.slot_pos = (int32_t*)take(TK * 4);
  w.cand = (int32_t*)take(TK * 4);
  w.offer = (int32_t*)take(TK * 4);
  w.ocounts = (int32_t*)take(E * 4);
  w.H = take((size_t)rows * d.d_ff * esz);
  w.Yp = (float*)take((size_t)rows * d.d_model * 4);
  w.bytes = off;   // monotone in T
  return w;
}

static moe_status_t check_ws(const moe_desc_t& d, void* ws, size_t bytes, Workspace& w) {
  w = carve_workspace(d, ws);
  if (!ws || bytes < w.bytes || ((uintptr_t)ws & 255u)) return MOE_E_WORKSPACE;
  return MOE_OK;
}

// Per-expert capacity C = max(floor(cf k T / E), k) ("Mixture-of-experts in practice",
// routing-math section: the expected load k T / E times the capacity factor, truncated,
// at least k), -1 without a capacity (cf <= 0).  The product is exact on the float32 cf
// of the descriptor: cf = m 2^s with an integer m < 2^24, so floor(m k T 2^s / E) is
// integer arithmetic (m k T < 2^54 under validate()'s bounds) and no evaluation order or
// rounding enters.  A C above T k keeps every assignment (an expert holds at most one
// slot per token), so it is reported as T k, which also keeps C within 32 bits.
static int64_t capacity_of(const moe_desc_t& d) {
  if (!(d.capacity_factor > 0.0f)) return -1;
  const int64_t all = d.T * d.top_k;
  int e2 = 0;
  const float fr = frexpf(d.capacity_factor, &e2);        // cf = fr 2^e2, fr in [0.5, 1)
  const uint64_t m = (uint64_t)ldexpf(fr, 24);             // exact: 24 significant bits
  const int s = e2 - 24;                                   // cf = m 2^s
  const unsigned __int128 num = (unsigned __int128)m * (uint64_t)d.top_k * (uint64_t)d.T;
  const uint64_t E = (uint64_t)d.n_experts;
  int64_t raw;
  if (num == 0) {
    raw = 0;
  } else if (s >= 0) {
    // num >= 1 and E <= 2^10, so a shift of 50 or more gives at least 2^40 > T k
    raw = s >= 50 ? all : (int64_t)std::min<unsigned __int128>((num << s) / E, all);
  } else {
    const unsigned __int128 q = num / E;
    raw = -s >= 64 ? 0 : (int64_t)std::min<unsigned __int128>(q >> -s, all);
  }
  return raw < d.top_k ? d.top_k : raw;
}

#define MOE_HIP(call)                       \
  do {                                      \
    if ((call) != hipSuccess) return MOE_E_HIP; \
  } while (0)

static bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

static ExpertWeights plain_weights(const void* g, const void* u, const void* dn) {
  return ExpertWeights{g, u, dn, nullptr, nullptr, nullptr, false};
}

// 8-bit weights: a bf16 layer, and every scale array given for the weights given.
static moe_status_t check_fp8(const moe_desc_t& d, const ExpertWeights& ew) {
  if (!ew.fp8) return MOE_OK;
  if (d.dtype != MOE_DTYPE_BF16) return MOE_E_UNSUPPORTED;
  if ((ew.gate && !ew.s_gate) || (ew.up && !ew.s_up) || (ew.down && !ew.s_down))
    return MOE_E_NULL;
  if (!aligned4(ew.s_gate) || !aligned4(ew.s_up) || !aligned4(ew.s_down))
    return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

static moe_status_t experts_impl(const moe_desc_t* desc, const void* x, const int32_t* perm_src,
                                 const int32_t* offsets, const ExpertWeights& ew, float* Yp,
                                 void* H, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  const moe_desc_t& d = *desc;
  const bool any = d.T > 0;
  if (!offsets || !ew.gate || !ew.up || !ew.down || (any && (!x || !perm_src || !Yp)))
    return MOE_E_NULL;
  if ((st = check_fp8(d, ew)) != MOE_OK) return st;
  if (!aligned16(x) || !aligned16(ew.gate) || !aligned16(ew.up) || !aligned16(ew.down) ||
      !aligned16(Yp) || (H && !aligned16(H)))
    return MOE_E_UNSUPPORTED;
  Workspace w;
  if ((st = check_ws(d, workspace, workspace_bytes, w)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  void* h = H ? H : w.H;
  MOE_HIP(launch_zero_i32(w.ctr, kTileCounters, s));
  MOE_HIP(launch_gate_up(d, token_choice_rows(d), x, perm_src, offsets, ew, h, w.ctr, s));
  MOE_HIP(launch_down(d, token_choice_rows(d), h, offsets, ew, Yp, w.ctr + kTileCounters / 2, s));
  return MOE_OK;
}

// Work counters of an optional workspace (NULL: static tile order).
static moe_status_t optional_ctr(const moe_desc_t& d, void* ws, size_t bytes, int32_t** ctr) {
  *ctr = nullptr;
  if (!ws) return MOE_OK;
  Workspace w;
  const moe_status_t st = check_ws(d, ws, bytes, w);
  if (st == MOE_OK) *ctr = w.ctr;
  return st;
}

static moe_status_t gate_up_impl(const moe_desc_t* desc, const void* x, const int32_t* perm_src,
                                 const int32_t* offsets, const ExpertWeights& ew, void* H,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  if (!offsets || !ew.gate || !ew.up || (desc->T > 0 && (!x || !perm_src || !H)))
    return MOE_E_NULL;
  if ((st = check_fp8(*desc, ew)) != MOE_OK) return st;
  if (!aligned16(x) || !aligned16(ew.gate) || !aligned16(ew.up) || !aligned16(H))
    return MOE_E_UNSUPPORTED;
  int32_t* ctr;
  if ((st = optional_ctr(*desc, workspace, workspace_bytes, &ctr)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (ctr) MOE_HIP(launch_zero_i32(ctr, kTileCounters / 2, s));
  MOE_HIP(launch_gate_up(*desc, token_choice_rows(*desc), x, perm_src, offsets, ew, H, ctr, s));
  return MOE_OK;
}

static moe_status_t down_impl(const moe_desc_t* desc, const void* H, const int32_t* offsets,
                              const ExpertWeights& ew, float* Yp, void* workspace,
                              size_t workspace_bytes, void* stream) {
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  if (!offsets || !ew.down || (desc->T > 0 && (!H || !Yp))) return MOE_E_NULL;
  if ((st = check_fp8(*desc, ew)) != MOE_OK) return st;
  if (!aligned16(H) || !aligned16(ew.down) || !aligned16(Yp)) return MOE_E_UNSUPPORTED;
  int32_t* ctr;
  if ((st = optional_ctr(*desc, workspace, workspace_bytes, &ctr)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (ctr) MOE_HIP(launch_zero_i32(ctr + kTileCounters / 2, kTileCounters / 2, s));
  MOE_HIP(launch_down(*desc, token_choice_rows(*desc), H, offsets, ew, Yp,
                      ctr ? ctr + kTileCounters / 2 : nullptr, s));
  return MOE_OK;
}

// Round-0 ranks (from the block histograms in blk, chunked by chunk), offers to the
// next-best candidates, and the final placement: offsets, perm_src, slot_pos.
static hipError_t dispatch_next_best(const moe_desc_t& d, const int32_t* topk_idx,
                                     const int32_t* cand, int chunk, int32_t* blk,
                                     const int32_t* counts, const Workspace& w,
                                     int32_t* offsets, int32_t* perm_src, int32_t* slot_pos,
                                     hipStream_t s) {
  const int64_t TK = d.T * d.top_k, C = capacity_of(d);
  const int E = (int)d.n_experts, k = (int)d.top_k;
  hipError_t e;
  if ((e = launch_ranks(topk_idx, TK, E, chunk, blk, slot_pos, s)) != hipSuccess) return e;
  if ((e = launch_offers(slot_pos, cand, d.T, k, E, C, w.offer, blk, s)) != hipSuccess) return e;
  if ((e = launch_expert_scan(blk, ceil_div(TK, kDispatchChunk), E, nullptr, d.T, k, w.ocounts,
                              nullptr, nullptr, nullptr, 0, s)) != hipSuccess)
    return e;
  return launch_place_next_best(topk_idx, w.offer, TK, E, C, counts, w.ocounts, blk, offsets,
                                perm_src, slot_pos, s);
}

static moe_status_t forward_impl(const moe_desc_t* desc, const void* x, const void* W_router,
                                 const float* router_bias, const ExpertWeights& ew, void* out,
                                 float* f, float* p, void* workspace, size_t workspace_bytes,
                                 void* stream, bool next_best = false) {
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  const moe_desc_t& d = *desc;
  if (next_best && !(d.capacity_factor > 0.0f)) return MOE_E_SHAPE;
  if (!W_router || !ew.gate || !ew.up || !ew.down || (d.T > 0 && (!x || !out)))
    return MOE_E_NULL;
  if ((st = check_fp8(d, ew)) != MOE_OK) return st;
  if (!aligned16(x) || !aligned16(W_router) || !aligned16(ew.gate) || !aligned16(ew.up) ||
      !aligned16(ew.down) || !aligned16(out))
    return MOE_E_UNSUPPORTED;
  Workspace w;
  if ((st = check_ws(d, workspace, workspace_bytes, w)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const RoutePlan rp = route_plan(d);
  const int64_t TK = d.T * d.top_k;
  const int E = (int)d.n_experts;
  const int64_t C = capacity_of(d);
  const int chunk = rp.BT * (int)d.top_k;   // the route blocks' histograms serve dispatch
  if (rp.n_blocks == 1 && !next_best && d.dtype == MOE_DTYPE_BF16) {
    // one route block holds the whole batch: it also does the dispatch (decode sizes)
    const RouteDispatch fd{C, w.counts, w.offsets, w.perm_src, w.slot_pos, f, p, w.ctr,
                           kTileCounters};
    MOE_HIP(launch_route(d, x, W_router, router_bias, w.topk_idx, w.topk_w, nullptr, nullptr,
                         nullptr, w.p_part, w.cnt_part, s, &fd));
  } else {
    MOE_HIP(launch_route(d, x, W_router, router_bias, w.topk_idx, w.topk_w, nullptr, nullptr,
                         next_best ? w.cand : nullptr, w.p_part, w.cnt_part, s));
    MOE_HIP(launch_expert_scan(w.cnt_part, rp.n_blocks, E, w.p_part, d.T, (int)d.top_k,
                               w.counts, f, p, w.ctr, kTileCounters, s));
    if (next_best)
      MOE_HIP(dispatch_next_best(d, w.topk_idx, w.cand, chunk, w.cnt_part, w.counts, w,
                                 w.offsets, w.perm_src, w.slot_pos, s));
    else
      MOE_HIP(launch_scatter(w.topk_idx, TK, E, chunk, C, w.cnt_part, w.counts, w.offsets,
                             w.perm_src, w.slot_pos, s));
  }
  const GemmRows rows = token_choice_rows(d);
  MOE_HIP(launch_gate_up(d, rows, x, w.perm_src, w.offsets, ew, w.H, w.ctr, s));
  MOE_HIP(launch_down(d, rows, w.H, w.offsets, ew, w.Yp, w.ctr + kTileCounters / 2, s));
  MOE_HIP(launch_combine(d, w.Yp, w.slot_pos, w.topk_w, out, s));
  return MOE_OK;
}

// ---- expert choice
int64_t expert_choice_capacity(const moe_desc_t& d) {
  const int64_t C = capacity_of(d);
  if (C < 0) return -1;
  return C < d.T ? C : d.T;
}

static GemmRows expert_choice_rows(const moe_desc_t& d) {
  return {d.n_experts * expert_choice_capacity(d), 1};
}

// validate() plus what expert choice needs: a capacity factor > 0, T within the select
// kernel's reach, and the E C + S T rows within 32-bit element offsets.
static moe_status_t validate_ec(const moe_desc_t* d) {
  moe_status_t st = validate(d);
  if (st != MOE_OK) return st;
  if (!(d->capacity_factor > 0.0f)) return MOE_E_SHAPE;
  if (d->T > kMaxExpertChoiceTokens) return MOE_E_UNSUPPORTED;
  const int64_t rows = expert_choice_rows(*d).routed + d->n_shared * d->T;
  if (rows > (int64_t)INT32_MAX || rows * d->d_ff > (int64_t)INT32_MAX ||
      rows * d->d_model > (int64_t)INT32_MAX)
    return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

WorkspaceEC carve_workspace_ec(const moe_desc_t& d, void* base) {
  const RoutePlan rp = route_plan(d);
  const GemmRows gr = expert_choice_rows(d);
  const int64_t E = d.n_experts, TE = d.T * E;
  const int64_t rows = gr.routed + d.n_shared * d.T;
  const size_t esz = d.dtype == MOE_DTYPE_BF16 ? 2 : 4;
  char* p = (char*)base;
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? (void*)(p + off) : nullptr;
    off += align256(bytes > 0 ? bytes : 1);
    return r;
  };
  WorkspaceEC w{};
  w.p_part = (float*)take(rp.n_blocks * E * 4);
  w.cnt_part = (int32_t*)take(rp.n_blocks * E * 4);
  w.counts = (int32_t*)take(E * 4);
  w.ctr = (int32_t*)take(kTileCounters * 4);
  w.offsets = (int32_t*)take((E + 1) * 4);
  w.probs = (float*)take(TE * 4);
  w.slot = (int32_t*)take(TE * 4);
  w.perm_src = (int32_t*)take(gr.routed * 4);
  w.H = take((size_t)rows * d.d_ff * esz);
  w.Yp = (float*)take((size_t)rows * d.d_model * 4);
  w.bytes = off;
  return w;
}

static moe_status_t check_ws_ec(const moe_desc_t& d, void* ws, size_t bytes, WorkspaceEC& w) {
  w = carve_workspace_ec(d, ws);
  if (!ws || bytes < w.bytes || ((uintptr_t)ws & 255u)) return MOE_E_WORKSPACE;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_str(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_E_NULL: return "MOE_E_NULL: a required pointer is NULL";
    case MOE_E_SHAPE: return "MOE_E_SHAPE: inconsistent or out-of-range sizes";
    case MOE_E_UNSUPPORTED: return "MOE_E_UNSUPPORTED: outside what the kernels implement";
    case MOE_E_WORKSPACE: return "MOE_E_WORKSPACE: workspace missing, misaligned or too small";
    case MOE_E_HIP: return "MOE_E_HIP: a HIP launch failed";
    case MOE_E_SCRATCH:
      return "MOE_E_SCRATCH: the layer needs more scratch than the static device buffer holds";
  }
  return "unknown moe_status_t";
}

moe_status_t moe_validate(const moe_desc_t* desc) { return validate(desc); }

size_t moe_workspace_bytes(const moe_desc_t* desc) {
  if (validate(desc) != MOE_OK) return 0;
  return carve_workspace(*desc, nullptr).bytes;
}

int64_t moe_capacity(const moe_desc_t* desc) {
  if (validate(desc) != MOE_OK) return -1;
  return capacity_of(*desc);
}

moe_status_t moe_route(const moe_desc_t* desc, const void* x, const void* W_router,
                       const float* router_bias, int32_t* topk_idx, float* topk_w, float* gap,
                       float* f, float* p, void* workspace, size_t workspace_bytes,
                       void* stream) {
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  const moe_desc_t& d = *desc;
  const bool any = d.T > 0;   // with no tokens, token-sized buffers may be NULL
  if (!W_router || (any && (!x || !topk_idx || !topk_w))) return MOE_E_NULL;
  if (!aligned16(x) || !aligned16(W_router)) return MOE_E_UNSUPPORTED;
  Workspace w;
  if ((st = check_ws(d, workspace, workspace_bytes, w)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const RoutePlan rp = route_plan(d);
  MOE_HIP(launch_route(d, x, W_router, router_bias, topk_idx, topk_w, gap, nullptr, nullptr,
                       w.p_part, w.cnt_part, s));
  if (f || p)
    MOE_HIP(launch_expert_scan(w.cnt_part, rp.n_blocks, (int)d.n_experts, w.p_part, d.T,
                               (int)d.top_k, w.counts, f, p, nullptr, 0, s));
  return MOE_OK;
}

moe_status_t moe_dispatch(const moe_desc_t* desc, const int32_t* topk_idx, int32_t* counts,
                          int32_t* offsets, int32_t* perm_src, int32_t* slot_pos,
                          void* workspace, size_t workspace_bytes, void* stream) {
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  const moe_desc_t& d = *desc;
  if (!counts || !offsets || (d.T > 0 && (!topk_idx || !perm_src || !slot_pos)))
    return MOE_E_NULL;
  Workspace w;
  if ((st = check_ws(d, workspace, workspace_bytes, w)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const int64_t TK = d.T * d.top_k;
  const int E = (int)d.n_experts;
  const int64_t C = capacity_of(d);
  MOE_HIP(launch_hist(topk_idx, TK, E, kDispatchChunk, w.cnt_part, s));
  MOE_HIP(launch_expert_scan(w.cnt_part, ceil_div(TK, kDispatchChunk), E, nullptr, d.T,
                             (int)d.top_k, counts, nullptr, nullptr, nullptr, 0, s));
  MOE_HIP(launch_scatter(topk_idx, TK, E, kDispatchChunk, C, w.cnt_part, counts, offsets,
                         perm_src, slot_pos, s));
  return MOE_OK;
}

moe_status_t moe_experts(const moe_desc_t* desc, const void* x, const int32_t* perm_src,
                         const int32_t* offsets, const void* W_gate, const void* W_up,
                         const void* W_down, float* Yp, void* H, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return experts_impl(desc, x, perm_src, offsets, plain_weights(W_gate, W_up, W_down), Yp, H,
                      workspace, workspace_bytes, stream);
}

moe_status_t moe_experts_gate_up(const moe_desc_t* desc, const void* x, const int32_t* perm_src,
                                 const int32_t* offsets, const void* W_gate, const void* W_up,
                                 void* H, void* workspace, size_t workspace_bytes, void* stream) {
  return gate_up_impl(desc, x, perm_src, offsets, plain_weights(W_gate, W_up, nullptr), H,
                      workspace, workspace_bytes, stream);
}

moe_status_t moe_experts_down(const moe_desc_t* desc, const void* H, const int32_t* offsets,
                              const void* W_down, float* Yp, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return down_impl(desc, H, offsets, plain_weights(nullptr, nullptr, W_down), Yp, workspace,
                   workspace_bytes, stream);
}

moe_status_t moe_combine(const moe_desc_t* desc, const float* Yp, const int32_t* slot_pos,
                         const float* topk_w, void* out, void* stream) {
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  const moe_desc_t& d = *desc;
  if (d.T > 0 && (!Yp || !slot_pos || !topk_w || !out)) return MOE_E_NULL;
  if (!aligned16(Yp) || !aligned16(out)) return MOE_E_UNSUPPORTED;
  MOE_HIP(launch_combine(d, Yp, slot_pos, topk_w, out, (hipStream_t)stream));
  return MOE_OK;
}

moe_status_t moe_forward(const moe_desc_t* desc, const void* x, const void* W_router,
                         const float* router_bias, const void* W_gate, const void* W_up,
                         const void* W_down, void* out, float* f, float* p, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return forward_impl(desc, x, W_router, router_bias, plain_weights(W_gate, W_up, W_down), out,
                      f, p, workspace, workspace_bytes, stream);
}

// ---- 8-bit expert weights
moe_status_t moe_forward_fp8(const moe_desc_t* desc, const void* x, const void* W_router,
                             const float* router_bias, const uint8_t* Wq_gate,
                             const uint8_t* Wq_up, const uint8_t* Wq_down, const float* s_gate,
                             const float* s_up, const float* s_down, void* out, float* f,
                             float* p, void* workspace, size_t workspace_bytes, void* stream) {
  const ExpertWeights ew{Wq_gate, Wq_up, Wq_down, s_gate, s_up, s_down, true};
  return forward_impl(desc, x, W_router, router_bias, ew, out, f, p, workspace, workspace_bytes,
                      stream);
}

moe_status_t moe_experts_fp8(const moe_desc_t* desc, const void* x, const int32_t* perm_src,
                             const int32_t* offsets, const uint8_t* Wq_gate,
                             const uint8_t* Wq_up, const uint8_t* Wq_down, const float* s_gate,
                             const float* s_up, const float* s_down, float* Yp, void* H,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const ExpertWeights ew{Wq_gate, Wq_up, Wq_down, s_gate, s_up, s_down, true};
  return experts_impl(desc, x, perm_src, offsets, ew, Yp, H, workspace, workspace_bytes,
                      stream);
}

moe_status_t moe_experts_gate_up_fp8(const moe_desc_t* desc, const void* x,
                                     const int32_t* perm_src, const int32_t* offsets,
                                     const uint8_t* Wq_gate, const uint8_t* Wq_up,
                                     const float* s_gate, const float* s_up, void* H,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  const ExpertWeights ew{Wq_gate, Wq_up, nullptr, s_gate, s_up, nullptr, true};
  return gate_up_impl(desc, x, perm_src, offsets, ew, H, workspace, workspace_bytes, stream);
}

moe_status_t moe_experts_down_fp8(const moe_desc_t* desc, const void* H, const int32_t* offsets,
                                  const uint8_t* Wq_down, const float* s_down, float* Yp,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  const ExpertWeights ew{nullptr, nullptr, Wq_down, nullptr, nullptr, s_down, true};
  return down_impl(desc, H, offsets, ew, Yp, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- expert-choice routing
extern "C" {

size_t moe_workspace_bytes_expert_choice(const moe_desc_t* desc) {
  if (validate_ec(desc) != MOE_OK) return 0;
  return carve_workspace_ec(*desc, nullptr).bytes;
}

int64_t moe_capacity_expert_choice(const moe_desc_t* desc) {
  if (validate_ec(desc) != MOE_OK) return -1;
  return expert_choice_capacity(*desc);
}

moe_status_t moe_route_expert_choice(const moe_desc_t* desc, const void* x,
                                     const void* W_router, float* probs, int32_t* offsets,
                                     int32_t* perm_src, int32_t* slot, float* f, float* p,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  moe_status_t st = validate_ec(desc);
  if (st != MOE_OK) return st;
  const moe_desc_t& d = *desc;
  if (!W_router || !offsets || (d.T > 0 && (!x || !probs || !perm_src || !slot)))
    return MOE_E_NULL;
  if (!aligned16(x) || !aligned16(W_router)) return MOE_E_UNSUPPORTED;
  WorkspaceEC w;
  if ((st = check_ws_ec(d, workspace, workspace_bytes, w)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const RoutePlan rp = route_plan(d);
  const int E = (int)d.n_experts;
  if (d.T == 0) {   // no tokens: empty groups, f and P zero
    MOE_HIP(launch_zero_i32(offsets, E + 1, s));
    if (f || p)
      MOE_HIP(launch_expert_scan(w.cnt_part, 0, E, nullptr, 0, (int)d.top_k, w.counts, f, p,
                                 nullptr, 0, s));
    return MOE_OK;
  }
  MOE_HIP(launch_route(d, x, W_router, nullptr, nullptr, nullptr, nullptr, probs, nullptr,
                       w.p_part, w.cnt_part, s));
  if (p)
    MOE_HIP(launch_expert_scan(w.cnt_part, rp.n_blocks, E, w.p_part, d.T, (int)d.top_k,
                               w.counts, nullptr, p, nullptr, 0, s));
  MOE_HIP(launch_ec_select(probs, (int)d.T, E, (int)expert_choice_capacity(d), perm_src, offsets,
                           slot, f, s));
  return MOE_OK;
}

moe_status_t moe_combine_expert_choice(const moe_desc_t* desc, const float* Yp,
                                       const int32_t* slot, const float* probs, void* out,
                                       void* stream) {
  moe_status_t st = validate_ec(desc);
  if (st != MOE_OK) return st;
  const moe_desc_t& d = *desc;
  if (d.T > 0 && (!Yp || !slot || !probs || !out)) return MOE_E_NULL;
  if (!aligned16(Yp) || !aligned16(out)) return MOE_E_UNSUPPORTED;
  MOE_HIP(launch_ec_combine(d, expert_choice_rows(d).routed, Yp, slot, probs, out,
                            (hipStream_t)stream));
  return MOE_OK;
}

moe_status_t moe_forward_expert_choice(const moe_desc_t* desc, const void* x,
                                       const void* W_router, const void* W_gate,
                                       const void* W_up, const void* W_down, void* out, float* f,
                                       float* p, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  moe_status_t st = validate_ec(desc);
  if (st != MOE_OK) return st;
  const moe_desc_t& d = *desc;
  if (!W_router || !W_gate || !W_up || !W_down || (d.T > 0 && (!x || !out))) return MOE_E_NULL;
  if (!aligned16(x) || !aligned16(W_router) || !aligned16(W_gate) || !aligned16(W_up) ||
      !aligned16(W_down) || !aligned16(out))
    return MOE_E_UNSUPPORTED;
  WorkspaceEC w;
  if ((st = check_ws_ec(d, workspace, workspace_bytes, w)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const RoutePlan rp = route_plan(d);
  const int E = (int)d.n_experts;
  const GemmRows rows = expert_choice_rows(d);
  const ExpertWeights ew = plain_weights(W_gate, W_up, W_down);
  if (d.T == 0) {   // no tokens: f and P are zero
    if (f || p)
      MOE_HIP(launch_expert_scan(w.cnt_part, 0, E, nullptr, 0, (int)d.top_k, w.counts, f, p,
                                 nullptr, 0, s));
    return MOE_OK;
  }
  MOE_HIP(launch_route(d, x, W_router, nullptr, nullptr, nullptr, nullptr, w.probs, nullptr,
                       w.p_part, w.cnt_part, s));
  // P from the route blocks' partial sums; also clears the GEMMs' work counters
  MOE_HIP(launch_expert_scan(w.cnt_part, rp.n_blocks, E, w.p_part, d.T, (int)d.top_k, w.counts,
                             nullptr, p, w.ctr, kTileCounters, s));
  MOE_HIP(launch_ec_select(w.probs, (int)d.T, E, (int)expert_choice_capacity(d), w.perm_src,
                           w.offsets, w.slot, f, s));
  MOE_HIP(launch_gate_up(d, rows, x, w.perm_src, w.offsets, ew, w.H, w.ctr, s));
  MOE_HIP(launch_down(d, rows, w.H, w.offsets, ew, w.Yp, w.ctr + kTileCounters / 2, s));
  MOE_HIP(launch_ec_combine(d, rows.routed, w.Yp, w.slot, w.probs, out, s));
  return MOE_OK;
}

}  // extern "C"

// ---- capacity overflow to the next-best expert
extern "C" {

moe_status_t moe_forward_next_best(const moe_desc_t* desc, const void* x, const void* W_router,
                                   const float* router_bias, const void* W_gate,
                                   const void* W_up, const void* W_down, void* out, float* f,
                                   float* p, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return forward_impl(desc, x, W_router, router_bias, plain_weights(W_gate, W_up, W_down), out,
                      f, p, workspace, workspace_bytes, stream, true);
}

moe_status_t moe_route_next_best(const moe_desc_t* desc, const void* x, const void* W_router,
                                 const float* router_bias, int32_t* topk_idx, float* topk_w,
                                 int32_t* cand, float* f, float* p, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  const moe_desc_t& d = *desc;
  if (!W_router || (d.T > 0 && (!x || !topk_idx || !topk_w || !cand))) return MOE_E_NULL;
  if (!aligned16(x) || !aligned16(W_router)) return MOE_E_UNSUPPORTED;
  Workspace w;
  if ((st = check_ws(d, workspace, workspace_bytes, w)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const RoutePlan rp = route_plan(d);
  MOE_HIP(launch_route(d, x, W_router, router_bias, topk_idx, topk_w, nullptr, nullptr, cand,
                       w.p_part, w.cnt_part, s));
  if (f || p)
    MOE_HIP(launch_expert_scan(w.cnt_part, rp.n_blocks, (int)d.n_experts, w.p_part, d.T,
                               (int)d.top_k, w.counts, f, p, nullptr, 0, s));
  return MOE_OK;
}

moe_status_t moe_dispatch_next_best(const moe_desc_t* desc, const int32_t* topk_idx,
                                    const int32_t* cand, int32_t* counts, int32_t* offsets,
                                    int32_t* perm_src, int32_t* slot_pos, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  const moe_desc_t& d = *desc;
  if (!(d.capacity_factor > 0.0f)) return MOE_E_SHAPE;
  if (!counts || !offsets || (d.T > 0 && (!topk_idx || !cand || !perm_src || !slot_pos)))
    return MOE_E_NULL;
  Workspace w;
  if ((st = check_ws(d, workspace, workspace_bytes, w)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const int64_t TK = d.T * d.top_k;
  const int E = (int)d.n_experts;
  MOE_HIP(launch_hist(topk_idx, TK, E, kDispatchChunk, w.cnt_part, s));
  MOE_HIP(launch_expert_scan(w.cnt_part, ceil_div(TK, kDispatchChunk), E, nullptr, d.T,
                             (int)d.top_k, counts, nullptr, nullptr, nullptr, 0, s));
  MOE_HIP(dispatch_next_best(d, topk_idx, cand, kDispatchChunk, w.cnt_part, counts, w, offsets,
                             perm_src, slot_pos, s));
  return MOE_OK;
}

}  // extern "C"

// ---- allocation-free entry point
namespace moe {

// The scratch of moe_forward_noalloc.  On the host `scratch` names a stand-in, not device
// memory: host code never passes it to a kernel, a memset or a copy; it uses the address
// hipGetSymbolAddress returns for the current device (each GPU holds its own copy).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

static std::atomic<void*> scratch_addr[kMaxDevices];
static std::mutex scratch_mu;

// Device address of the current device's scratch, looked up on its first use.
static moe_status_t device_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_E_UNSUPPORTED;
  void* ptr = scratch_addr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    ptr = scratch_addr[dev].load(std::memory_order_acquire);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
        return MOE_E_HIP;
      scratch_addr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return MOE_OK;
}

}  // namespace moe

extern "C" moe_status_t moe_forward_noalloc(const moe_desc_t* desc, const void* x,
                                            const void* W_router, const float* router_bias,
                                            const void* W_gate, const void* W_up,
                                            const void* W_down, void* out, float* f, float* p,
                                            void* stream) {
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  if (carve_workspace(*desc, nullptr).bytes > MOE_NOALLOC_SCRATCH_BYTES) return MOE_E_SCRATCH;
  void* ws = nullptr;
  if ((st = device_scratch(&ws)) != MOE_OK) return st;
  return forward_impl(desc, x, W_router, router_bias, plain_weights(W_gate, W_up, W_down), out,
                      f, p, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}
