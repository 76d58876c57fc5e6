/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse mixture-of-experts FFN forward pass.
 *
 * The layer (pages cited by title and section):
 *   router     logits = x W_r^T, no bias; p = softmax(logits)
 *              ("Chapter 30: Mixture of Experts", LLM Transformer book, 30.2.3)
 *   top-k      the k experts with the largest selection score s = p + b, where b is an
 *              optional per-expert selection bias that changes only the choice
 *              ("Mixture of Experts (MoE) memo", iwashi.co, DeepSeek-V3 aux-loss-free
 *              section); ties go to the lower expert index; slots ordered by s, highest
 *              first
 *   renorm     w_tj = p[t, idx_tj] / sum_j p[t, idx_tj]   (book 30.2.3 step 4)
 *   statistics f_e = #assignments to e / (T k) (before any capacity drop);
 *              P_e = mean_t p[t, e]   (memo, auxiliary-loss section)
 *   dispatch   the T*k assignments, flattened row-major (i = t*k + j), are grouped by
 *              expert in stable order; with a capacity C = max(floor(cf k T / E), k) (the
 *              product exact on the float32 cf; see moe_capacity) the first C of
 *              each expert are kept, the rest dropped
 *              ("Mixture-of-experts in practice: routing, load balancing and parallel
 *              configuration", deepseekmodel.com, routing-math and expert-parallel
 *              sections)
 *   experts    o = W_down (SiLU(W_gate x) * (W_up x)) per kept assignment (book 30.2.4);
 *              the optional shared expert runs on every token (book 30.4.5)
 *   combine    y_t = sum over kept j of w_tj o_tj  (+ shared_t); dropped slots give 0
 *              (book 30.6.1; practice, capacity section)
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; everything is row-major:
 *       x [T, d]; W_router [E, d]; router_bias [E] float32;
 *       W_gate, W_up [E + S, F, d]; W_down [E + S, d, F]  (S = n_shared; the shared
 *       expert's weights are appended at index E);  out [T, d].
 *     x, W_router and the expert weights have desc->dtype; out has desc->out_dtype.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; outputs are valid once the caller synchronises the stream.
 *   - The library never allocates, frees or synchronises.  Scratch memory comes from
 *     the caller's workspace (size from moe_workspace_bytes).  Calls that share a
 *     workspace must not overlap; calls with distinct workspaces may run concurrently.
 *   - With T == 0 the token-sized buffers (x, out, topk_*, perm_src, slot_pos, H, Yp)
 *     may be NULL; weights, offsets and counts are always required.
 *   - All arguments are validated on the host before anything is enqueued; an invalid
 *     call returns a nonzero status and enqueues nothing.  MOE_E_HIP reports a failed
 *     kernel launch (hipGetLastError).  Non-finite inputs are undefined behaviour.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;

typedef enum {
  MOE_OK = 0,
  MOE_E_NULL = 1,         /* a required pointer is NULL */
  MOE_E_SHAPE = 2,        /* inconsistent or out-of-range sizes */
  MOE_E_UNSUPPORTED = 3,  /* valid layer, but outside what the kernels implement */
  MOE_E_WORKSPACE = 4,    /* workspace NULL or smaller than moe_workspace_bytes */
  MOE_E_HIP = 5,          /* a HIP launch failed */
  MOE_E_SCRATCH = 6       /* moe_forward_noalloc: the layer needs more scratch than the
                             library's static device buffer holds */
} moe_status_t;

/* Layer description shared by every entry point.
 * Supported: T >= 0; 1 <= E <= 512; 1 <= top_k <= min(E, 16); n_shared in {0, 1};
 * d_model and d_ff positive multiples of 64 (at most 65536); dtype and out_dtype each
 * MOE_DTYPE_F32 or MOE_DTYPE_BF16.  capacity_factor <= 0 disables the capacity limit;
 * a NaN or infinite capacity_factor is MOE_E_SHAPE. */
typedef struct {
  int64_t T;                /* tokens (batch * sequence, flattened) */
  int64_t d_model;          /* d */
  int64_t n_experts;        /* E, routed experts */
  int64_t d_ff;             /* F, expert hidden size (the shared expert uses the same F) */
  int64_t top_k;            /* k */
  int64_t n_shared;         /* S: 0 or 1 always-on shared expert */
  float capacity_factor;    /* cf; <= 0: no capacity limit */
  int32_t dtype;            /* moe_dtype_t of x, W_router, W_gate, W_up, W_down */
  int32_t out_dtype;        /* moe_dtype_t of out */
} moe_desc_t;

/* Human-readable name of a status code (static storage). */
const char* moe_status_str(moe_status_t status);

/* Host-only check of a description: returns MOE_OK or the status any entry point would
 * return for it.  Makes no HIP call. */
moe_status_t moe_validate(const moe_desc_t* desc);

/* Bytes of workspace that moe_forward and each stage entry point take for `desc` (0 if
 * desc is invalid).  Makes no HIP call.  The workspace must be 256-byte aligned.  The
 * size grows with T, so a workspace sized for a larger T (all other fields equal) also
 * serves a smaller T. */
size_t moe_workspace_bytes(const moe_desc_t* desc);

/* Capacity C for `desc`: max(floor(cf * k * T / E), k), or -1 when cf <= 0 (no limit)
 * or desc is invalid.  ("Mixture-of-experts in practice", routing-math section.)  The
 * product is exact on the float32 value of capacity_factor (no rounding, no evaluation
 * order: cf = 0.7 is 0.699999988..., so k T / E = 10 gives C = 6); a C above T * k
 * keeps every assignment and is returned as T * k.  Makes no HIP call. */
int64_t moe_capacity(const moe_desc_t* desc);

/* The whole layer: route -> dispatch -> experts -> combine.
 *   router_bias  [E] float32 selection bias, or NULL for none
 *   out          [T, d] in desc->out_dtype
 *   f, p         [E] float32 statistics f_e and P_e, or NULL to skip
 * Errors: MOE_E_NULL (x, W_router, W_gate, W_up, W_down, out), MOE_E_SHAPE,
 * MOE_E_UNSUPPORTED, MOE_E_WORKSPACE, MOE_E_HIP. */
moe_status_t moe_forward(const moe_desc_t* desc, const void* x, const void* W_router,
                         const float* router_bias, const void* W_gate, const void* W_up,
                         const void* W_down, void* out, float* f, float* p,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Router, softmax, top-k on p + bias, renormalisation, statistics.
 * ("Chapter 30", 30.2.3; "MoE memo", auxiliary-loss and DeepSeek-V3 sections.)
 *   topk_idx [T, k] int32   chosen experts, slot order = selection score descending
 *   topk_w   [T, k] float32 renormalised weights from the unbiased probabilities
 *   gap      [T] float32 or NULL: s_(k) - s_(k+1), the k-th largest selection score minus
 *            the (k+1)-th (+inf when k == E); how close the token is to routing otherwise
 *   f, p     [E] float32 or NULL
 * Errors: MOE_E_NULL (x, W_router, topk_idx, topk_w), MOE_E_SHAPE, MOE_E_UNSUPPORTED,
 * MOE_E_WORKSPACE, MOE_E_HIP. */
moe_status_t moe_route(const moe_desc_t* desc, const void* x, const void* W_router,
                       const float* router_bias, int32_t* topk_idx, float* topk_w,
                       float* gap, float* f, float* p, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Expert histogram, capacity, prefix sum and the stable permutation.
 * ("Mixture-of-experts in practice", expert-parallel section: flatten, stable sort by
 * expert, bincount; routing-math section: capacity.)
 *   topk_idx [T, k] int32 in [0, E)   (any routing, e.g. an external one)
 *   counts   [E] int32      assignments per expert before the capacity cut
 *   offsets  [E + 1] int32  exclusive prefix sum of min(counts, C); offsets[E] = N kept
 *   perm_src [T * k] int32  perm_src[pos] = t*k + j of the assignment in row pos
 *                           (entries at pos >= N are left untouched)
 *   slot_pos [T * k] int32  row of assignment t*k + j, or -1 when it was dropped
 * An expert id outside [0, E) is treated as a dropped assignment: slot_pos = -1 and it
 * is not counted.
 * Errors: MOE_E_NULL (any pointer), MOE_E_SHAPE, MOE_E_UNSUPPORTED, MOE_E_WORKSPACE,
 * MOE_E_HIP. */
moe_status_t moe_dispatch(const moe_desc_t* desc, const int32_t* topk_idx, int32_t* counts,
                          int32_t* offsets, int32_t* perm_src, int32_t* slot_pos,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Grouped SwiGLU experts over the expert-contiguous rows ("Chapter 30", 30.2.4).
 * Row pos in [offsets[e], offsets[e+1]) is token perm_src[pos] / k run through expert
 * e.  With n_shared = 1, rows T*k + t (t < T) are token t through the shared expert.
 *   Yp [T*k + S*T, d] float32  o = W_down h for every such row (other rows untouched)
 *   H  [T*k + S*T, F] in dtype, or NULL: h = SiLU(W_gate x) * (W_up x) (rounded to
 *      bf16 for bf16 layers); when NULL the workspace holds it.
 * Errors: MOE_E_NULL (x, perm_src, offsets, W_gate, W_up, W_down, Yp), MOE_E_SHAPE,
 * MOE_E_UNSUPPORTED, MOE_E_WORKSPACE, MOE_E_HIP. */
moe_status_t moe_experts(const moe_desc_t* desc, const void* x, const int32_t* perm_src,
                         const int32_t* offsets, const void* W_gate, const void* W_up,
                         const void* W_down, float* Yp, void* H, void* workspace,
                         size_t workspace_bytes, void* stream);

/* The two kernels of moe_experts, one launch each, for callers that stage them:
 *   moe_experts_gate_up:  H = SiLU(X W_gate^T) * (X W_up^T) on the grouped rows
 *                         (H [T*k + S*T, F] in dtype; rows outside the groups untouched)
 *   moe_experts_down:     Yp = H W_down^T on the same rows (Yp [T*k + S*T, d] float32)
 * Row/group layout as for moe_experts.  The workspace is optional: with one (sized as for
 * moe_forward) the output tiles are handed out to the CUs dynamically through a few
 * counters kept in it, without (NULL) in a fixed order; the results are identical.
 * Errors: MOE_E_NULL (any pointer), MOE_E_SHAPE, MOE_E_UNSUPPORTED, MOE_E_WORKSPACE
 * (a workspace given but too small or misaligned), MOE_E_HIP. */
moe_status_t moe_experts_gate_up(const moe_desc_t* desc, const void* x, const int32_t* perm_src,
                                 const int32_t* offsets, const void* W_gate, const void* W_up,
                                 void* H, void* workspace, size_t workspace_bytes, void* stream);
moe_status_t moe_experts_down(const moe_desc_t* desc, const void* H, const int32_t* offsets,
                              const void* W_down, float* Yp, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ---- 8-bit expert weights ("Chapter 30", 30.4.6: FP8 halves the bytes each operation
 * moves; "Mixture-of-experts in practice", section on quantisation and routing: the router
 * stays in high precision, the expert weights carry the quantisation).
 * The expert weights are e4m3 codes (the "fn" encoding: sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinities, largest finite value 448) with one float32 scale per
 * output row:  W[e][n][:] = s[e][n] * decode(Wq[e][n][:]).
 *   Wq_gate, Wq_up [E + S, F, d] uint8;  s_gate, s_up [E + S, F] float32
 *   Wq_down        [E + S, d, F] uint8;  s_down      [E + S, d] float32
 * x, W_router and the activations stay in desc->dtype, which must be MOE_DTYPE_BF16
 * (else MOE_E_UNSUPPORTED); the codes are widened exactly to bf16 for the MFMAs and the
 * scales are applied to the fp32 sums (h = SiLU(s_g * (x.q_g)) * (s_u * (x.q_u)), o =
 * s_d * (h.q_d)).  Workspace, streams, layouts of the other tensors and the error rules are
 * those of the bf16 entry points; the code arrays must be 16-byte aligned, the scale arrays
 * 4-byte aligned, and a NULL scale array for given codes is MOE_E_NULL. */
moe_status_t moe_forward_fp8(const moe_desc_t* desc, const void* x, const void* W_router,
                             const float* router_bias, const uint8_t* Wq_gate,
                             const uint8_t* Wq_up, const uint8_t* Wq_down, const float* s_gate,
                             const float* s_up, const float* s_down, void* out, float* f,
                             float* p, void* workspace, size_t workspace_bytes, void* stream);
moe_status_t moe_experts_fp8(const moe_desc_t* desc, const void* x, const int32_t* perm_src,
                             const int32_t* offsets, const uint8_t* Wq_gate,
                             const uint8_t* Wq_up, const uint8_t* Wq_down, const float* s_gate,
                             const float* s_up, const float* s_down, float* Yp, void* H,
                             void* workspace, size_t workspace_bytes, void* stream);
moe_status_t moe_experts_gate_up_fp8(const moe_desc_t* desc, const void* x,
                                     const int32_t* perm_src, const int32_t* offsets,
                                     const uint8_t* Wq_gate, const uint8_t* Wq_up,
                                     const float* s_gate, const float* s_up, void* H,
                                     void* workspace, size_t workspace_bytes, void* stream);
moe_status_t moe_experts_down_fp8(const moe_desc_t* desc, const void* H, const int32_t* offsets,
                                  const uint8_t* Wq_down, const float* s_down, float* Yp,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Weighted combine back to token order ("Chapter 30", 30.6.1 and 30.4.5):
 *   out[t] = sum_{j ascending, slot_pos[t*k+j] >= 0} topk_w[t,j] * Yp[slot_pos[t*k+j]]
 *            + (n_shared ? Yp[T*k + t] : 0)
 * summed in float32, written in out_dtype.  Needs no workspace.
 * Errors: MOE_E_NULL (Yp, slot_pos, topk_w, out), MOE_E_SHAPE, MOE_E_UNSUPPORTED,
 * MOE_E_HIP. */
moe_status_t moe_combine(const moe_desc_t* desc, const float* Yp, const int32_t* slot_pos,
                         const float* topk_w, void* out, void* stream);

/* ---- Capacity overflow to the next-best expert ("Chapter 30", 30.5.2: tokens past an
 * expert's capacity are dropped or handed to the next-best expert).  One redirect round:
 * round 0 is the capacity cut of moe_dispatch (each expert keeps its first C assignments
 * in row-major (token, slot) order); the m-th assignment of token t dropped there (slot
 * order) is offered to cand[t, m], the token's (k+1+m)-th best expert by selection score
 * (ties to the lower index; -1 past E); every expert takes the offers in row-major order
 * while its rows stay within C; the rest are dropped.  An expert's rows are its round-0
 * assignments, then its accepted offers, each in row-major order.  A redirected slot keeps
 * its weight topk_w[t, j]; the combine is moe_combine.  f and P are those of moe_forward.
 * capacity_factor must be > 0 (else MOE_E_SHAPE).  Workspace: moe_workspace_bytes.
 *   moe_route_next_best    moe_route plus cand [T, k] int32
 *   moe_dispatch_next_best moe_dispatch with the redirect (counts = the top-k histogram)
 *   moe_forward_next_best  the whole layer (arguments as moe_forward) */
moe_status_t moe_forward_next_best(const moe_desc_t* desc, const void* x, const void* W_router,
                                   const float* router_bias, const void* W_gate,
                                   const void* W_up, const void* W_down, void* out, float* f,
                                   float* p, void* workspace, size_t workspace_bytes,
                                   void* stream);
moe_status_t moe_route_next_best(const moe_desc_t* desc, const void* x, const void* W_router,
                                 const float* router_bias, int32_t* topk_idx, float* topk_w,
                                 int32_t* cand, float* f, float* p, void* workspace,
                                 size_t workspace_bytes, void* stream);
moe_status_t moe_dispatch_next_best(const moe_desc_t* desc, const int32_t* topk_idx,
                                    const int32_t* cand, int32_t* counts, int32_t* offsets,
                                    int32_t* perm_src, int32_t* slot_pos, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ---- Expert-choice routing ("Mixture of Experts (MoE) memo", routing section: the
 * expert-choice row of the routing-design table, every expert picks the tokens that suit
 * it and loads come out equal; "Mixture-of-experts in practice", top-k section: each
 * expert takes its top-C tokens by its capacity, no token is dropped for capacity, and a
 * token's routing depends on the whole batch, so it fits encoders, not causal decoding).
 *   p[t, :]  = softmax(x[t] W_router^T) (no selection bias)
 *   C        = min(T, max(floor(capacity_factor * top_k * T / E), top_k)), top_k read as
 *              the average number of experts per token; capacity_factor must be > 0
 *   expert e takes the C tokens with the largest p[t, e] (float32; equal values go to the
 *   lower token index) as rows [e C, (e + 1) C) of the grouped GEMMs, in ascending token
 *   order;
 *   out[t]   = sum over the experts e that took t, ascending, of p[t, e] * FFN_e(x[t])
 *              (+ the shared expert, weight 1); a token no expert took gives 0 (+ shared).
 *   f_e = C / (E C) (1/E), P_e = mean_t p[t, e].
 * Tensors and errors as for token choice; in addition a capacity_factor <= 0 is
 * MOE_E_SHAPE and T > 32768 is MOE_E_UNSUPPORTED.  The workspace comes from
 * moe_workspace_bytes_expert_choice (0 for an invalid description). */
size_t moe_workspace_bytes_expert_choice(const moe_desc_t* desc);
/* C as above, or -1 for an invalid description. */
int64_t moe_capacity_expert_choice(const moe_desc_t* desc);
/* Router probabilities probs [T, E] float32, the selection as offsets [E + 1] (e C),
 * perm_src [E C] (token of each row) and slot [T, E] (row of (t, e), or -1), f and P
 * (each optional, [E]).  Needs the workspace. */
moe_status_t moe_route_expert_choice(const moe_desc_t* desc, const void* x,
                                     const void* W_router, float* probs, int32_t* offsets,
                                     int32_t* perm_src, int32_t* slot, float* f, float* p,
                                     void* workspace, size_t workspace_bytes, void* stream);
/* out[t] = sum_{e ascending, slot[t, e] >= 0} probs[t, e] * Yp[slot[t, e]]
 *          (+ Yp[E C + t] with a shared expert), float32 sums written in out_dtype. */
moe_status_t moe_combine_expert_choice(const moe_desc_t* desc, const float* Yp,
                                       const int32_t* slot, const float* probs, void* out,
                                       void* stream);
/* The whole layer with expert-choice routing (router, selection, grouped SwiGLU GEMMs
 * over the E C rows and the shared expert's T rows, combine). */
moe_status_t moe_forward_expert_choice(const moe_desc_t* desc, const void* x,
                                       const void* W_router, const void* W_gate,
                                       const void* W_up, const void* W_down, void* out, float* f,
                                       float* p, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* ---- Allocation-free entry point.
 * For callers that cannot allocate device memory or call hipMalloc at all: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Same layer and
 * arguments as moe_forward, without the workspace: its scratch is a static device buffer
 * inside the library, MOE_NOALLOC_SCRATCH_BYTES per GPU, that each GPU the library is
 * loaded on holds until the process ends.  The caller still passes inputs and outputs.
 *   - A layer whose moe_workspace_bytes exceeds MOE_NOALLOC_SCRATCH_BYTES returns
 *     MOE_E_SCRATCH and enqueues nothing (decode-sized and small prefill batches fit:
 *     e.g. T 16 of a d 4096, d_ff 14336, top-2 layer needs about 2 MB).
 *   - Every call on one GPU uses that GPU's single buffer: calls that overlap on one GPU
 *     (other streams, other threads) race and must be ordered by the caller.  The buffer
 *     keeps the last call's contents; each call clears what it needs at zero by kernel.
 *   - The first call on each device looks the buffer's address up (a host query, no
 *     allocation); make it outside graph capture.
 *   - Calls no hipMalloc, hipFree or other allocating routine. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_forward_noalloc(const moe_desc_t* desc, const void* x, const void* W_router,
                                 const float* router_bias, const void* W_gate, const void* W_up,
                                 const void* W_down, void* out, float* f, float* p,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
