// Internal declarations shared by the HIP translation units of libmoe (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef uint16_t bf16_t;

// Upper limits enforced by moe_validate.
constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 16;
// Devices whose per-device facts (CU count, kernel attributes, static scratch address) the
// library caches.
constexpr int kMaxDevices = 64;

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

__device__ inline float bf16_to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// float32 -> bfloat16, round to nearest, ties to even (inputs are finite).
__device__ inline bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// ---------------------------------------------------------------- route plan
// One route block handles BT = 16 * TPW tokens with 4 waves: EW waves split the
// (padded) experts into slabs of 16 * EPW, KS = 4 / EW waves split the reduction.
struct RoutePlan {
  int EPW, TPW, KS, BT, E_pad;
  int64_t n_blocks;
};
RoutePlan route_plan(const moe_desc_t& d);

// ---------------------------------------------------------------- workspace
struct Workspace {
  int32_t* topk_idx;   // [T*k]
  float* topk_w;       // [T*k]
  float* p_part;       // [route blocks][E]
  int32_t* cnt_part;   // [max(route blocks, dispatch blocks)][E]  (block histograms -> bases)
  int32_t* counts;     // [E]
  int32_t* offsets;    // [E+1]
  int32_t* perm_src;   // [T*k]
  int32_t* slot_pos;   // [T*k]
  void* H;             // [T*k + S*T, F] dtype
  float* Yp;           // [T*k + S*T, d]
  int32_t* ctr;        // kTileCounters work counters of the grouped GEMMs
  int32_t* cand;       // [T*k] next-best candidates (overflow redirect)
  int32_t* offer;      // [T*k] expert offered each dropped assignment, or -1
  int32_t* ocounts;    // [E] offers per expert
  size_t bytes;        // total size
};
Workspace carve_workspace(const moe_desc_t& d, void* base);

// Expert-choice layers: probabilities and slot matrix [T, E], E*C routed rows.
struct WorkspaceEC {
  float* p_part;       // [route blocks][E]
  int32_t* cnt_part;   // [route blocks][E]
  int32_t* counts;     // [E]
  int32_t* offsets;    // [E+1]
  float* probs;        // [T, E]
  int32_t* slot;       // [T, E]
  int32_t* perm_src;   // [E*C]
  void* H;             // [E*C + S*T, F] dtype
  float* Yp;           // [E*C + S*T, d]
  int32_t* ctr;        // kTileCounters
  size_t bytes;        // total size
};
// C of an expert-choice layer: min(T, max(floor(cf k T / E), k)); -1 when cf <= 0.
int64_t expert_choice_capacity(const moe_desc_t& d);
WorkspaceEC carve_workspace_ec(const moe_desc_t& d, void* base);

constexpr int kDispatchChunk = 1024;   // assignments per histogram block in moe_dispatch

// ---------------------------------------------------------------- launchers
// gap (optional, [T]): s_(k) - s_(k+1) of each token's selection scores (+inf if k == E).
// probs (optional, [T, E]): the router probabilities.  With topk_idx NULL no top-k is
// taken (and the block histograms stay zero).  cand (optional, [T, k]): the experts
// ranked k+1 .. 2k by selection score, -1 past E.
// Dispatch done by the route kernel itself when it runs as one block (bf16 layers, T at
// most one block's tokens): counts, f, P, offsets, perm_src and slot_pos as the
// histogram / scan / scatter kernels give them, and nzero work counters cleared.
struct RouteDispatch {
  int64_t C;   // capacity, < 0: none
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm_src;
  int32_t* slot_pos;
  float* f;
  float* p;
  int32_t* zero;
  int nzero;
};
hipError_t launch_route(const moe_desc_t& d, const void* x, const void* W_router,
                        const float* bias, int32_t* topk_idx, float* topk_w, float* gap,
                        float* probs, int32_t* cand, float* p_part, int32_t* cnt_part,
                        hipStream_t s, const RouteDispatch* fused = nullptr);
hipError_t launch_hist(const int32_t* idx, int64_t NA, int E, int chunk, int32_t* blk_cnt,
                       hipStream_t s);
// zero (optional): nzero <= 256 int32 that block 0 also sets to zero.
hipError_t launch_expert_scan(int32_t* blk, int64_t nb, int E, const float* p_part, int64_t T,
                              int k, int32_t* counts, float* f, float* p, int32_t* zero,
                              int nzero, hipStream_t s);
hipError_t launch_scatter(const int32_t* idx, int64_t NA, int E, int chunk, int64_t C,
                          const int32_t* blk_base, const int32_t* counts, int32_t* offsets,
                          int32_t* perm_src, int32_t* slot_pos, hipStream_t s);
// Overflow to the next-best expert (C >= 0), after hist + expert_scan of topk_idx:
//  ranks   rank0[i] = stable rank of assignment i within its top-k expert
//  offers  offer[i] = cand[t, m] for the m-th assignment of token t with rank0 >= C (-1
//          otherwise), and the block histograms of the offers (chunk kDispatchChunk)
//  place   (after expert_scan of those histograms -> ocounts) offsets of kept0 + accepted
//          offers, and the final slot_pos / perm_src.  rank0 may live in slot_pos.
hipError_t launch_ranks(const int32_t* idx, int64_t NA, int E, int chunk,
                        const int32_t* blk_base, int32_t* rank0, hipStream_t s);
hipError_t launch_offers(const int32_t* rank0, const int32_t* cand, int64_t T, int k, int E,
                         int64_t C, int32_t* offer, int32_t* blk, hipStream_t s);
hipError_t launch_place_next_best(const int32_t* idx, const int32_t* offer, int64_t NA, int E,
                                  int64_t C, const int32_t* counts, const int32_t* ocounts,
                                  const int32_t* offer_base, int32_t* offsets,
                                  int32_t* perm_src, int32_t* slot_pos, hipStream_t s);
// Expert weights as the grouped GEMMs take them: tensors of desc.dtype, or (fp8 set, bf16
// layers only) e4m3 codes with one float32 scale per output row.
struct ExpertWeights {
  const void* gate;
  const void* up;
  const void* down;
  const float* s_gate;   // [E + S, F]
  const float* s_up;     // [E + S, F]
  const float* s_down;   // [E + S, d]
  bool fp8;
};
// Rows of the grouped GEMMs: `routed` expert-contiguous rows (offsets[E] of them at most),
// row r taking token perm_src[r] / token_div, then the shared expert's T rows.
struct GemmRows {
  int64_t routed;   // T*k (token choice) or E*C (expert choice)
  int token_div;    // k (perm_src holds t*k + j) or 1 (perm_src holds t)
};
inline GemmRows token_choice_rows(const moe_desc_t& d) { return {d.T * d.top_k, (int)d.top_k}; }
hipError_t launch_gate_up(const moe_desc_t& d, const GemmRows& rows, const void* x,
                          const int32_t* perm_src, const int32_t* offsets,
                          const ExpertWeights& ew, void* H, int32_t* ctr, hipStream_t s);
// ctr: NULL (static tile order) or 8 int32 work counters, zero at launch.
hipError_t launch_down(const moe_desc_t& d, const GemmRows& rows, const void* H,
                       const int32_t* offsets, const ExpertWeights& ew, float* Yp,
                       int32_t* ctr, hipStream_t s);
// Sets n int32 to zero (a kernel, so that it may sit in a captured graph).
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);
constexpr int kTileCounters = 16;   // 8 per grouped GEMM
hipError_t launch_combine(const moe_desc_t& d, const float* Yp, const int32_t* slot_pos,
                          const float* topk_w, void* out, hipStream_t s);

// Expert choice: expert e takes the C tokens with the largest probs[:, e] (ties to the
// lower token), rows [e C, (e+1) C) in ascending token order; slot [T, E] gets each
// (token, expert)'s row or -1; f (optional) the share of the E*C assignments.
// Needs T <= kMaxExpertChoiceTokens.
constexpr int kMaxExpertChoiceTokens = 32768;
hipError_t launch_ec_select(const float* probs, int T, int E, int C, int32_t* perm_src,
                            int32_t* offsets, int32_t* slot, float* f, hipStream_t s);
// out[t] = sum over e ascending with slot[t, e] >= 0 of probs[t, e] * Yp[slot[t, e]]
// (+ Yp[shared_row0 + t] with a shared expert).
hipError_t launch_ec_combine(const moe_desc_t& d, int64_t shared_row0, const float* Yp,
                             const int32_t* slot, const float* probs, void* out, hipStream_t s);

}  // namespace moe
