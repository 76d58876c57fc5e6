// Router: logits = x W_r^T, softmax, top-k on the selection score p + bias, renormalised
// weights, per-block partial sums of p and per-block expert histograms.
//
// "Chapter 30: Mixture of Experts" (LLM Transformer book), 30.2.3 steps 1-4;
// "Mixture of Experts (MoE) memo" (iwashi.co), DeepSeek-V3 aux-loss-free section (the
// bias only changes the choice); "Mixture-of-experts in practice" (deepseekmodel.com),
// routing-math section (bias-free gate, always renormalise).
//
// bf16 layers: the logits GEMM runs on MFMA (v_mfma_f32_16x16x32_bf16, fp32
// accumulation).  One block = 4 wave64s over BT tokens.  EW waves split the experts
// into slabs of 16*EPW; KS = 4/EW waves split the reduction over d.  A wave's rows of a
// 64-wide k chunk are loaded 8 lanes per 128-byte row segment and put into MFMA operand
// order through a wave-private LDS buffer; lane group g of MFMA half h takes the 8 k values
// at 16 g + 8 h for A and B alike, so the sum is over the same pairs as a plain dot product.
// The top-k runs one wavefront per token; its reductions move data between lanes with DPP
// and v_permlane16/32_swap (no LDS round trips).
#include <math.h>

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Lane exchanges for wave-wide reductions.  Inside a 16-lane row: DPP quad swaps (1,0,3,2)
// and (2,3,0,1), then the half-row and row mirrors; across rows: v_permlane16_swap and
// v_permlane32_swap, which hand every lane the values of both rows (or halves) of its pair.
// After each step every lane of the group holds op(a, b) of the same two values, so with a
// commutative op all 64 lanes end with the same bits.
constexpr int DPP_QUAD_1032 = 0xB1, DPP_QUAD_2301 = 0x4E, DPP_HALF_MIRROR = 0x141,
              DPP_MIRROR = 0x140;

template <int CTRL>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

template <class Op>
__device__ inline float wave_reduce(float v, Op op) {
  v = op(v, dpp_f<DPP_QUAD_1032>(v));
  v = op(v, dpp_f<DPP_QUAD_2301>(v));
  v = op(v, dpp_f<DPP_HALF_MIRROR>(v));
  v = op(v, dpp_f<DPP_MIRROR>(v));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return op(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ inline float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ inline float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}

// (v, e) <- the better of (v, e) and (ov, oe): larger score, lower expert on equal scores.
// Written without short-circuit operators so that it compiles to compares and selects
// (a branch per compare, with its exec-mask bookkeeping, made each top-k round ~10x slower).
__device__ inline void take_better(float& v, int& e, float ov, int oe) {
  const bool better = (ov > v) | ((ov == v) & (oe < e));
  v = better ? ov : v;
  e = better ? oe : e;
}
template <int CTRL>
__device__ inline void argmax_step(float& v, int& e) {
  const float ov = dpp_f<CTRL>(v);
  const int oe = dpp_i<CTRL>(e);
  take_better(v, e, ov, oe);
}
// Wave-wide argmax of (score, expert); every lane ends with the winner.
__device__ inline void wave_argmax(float& v, int& e) {
  argmax_step<DPP_QUAD_1032>(v, e);
  argmax_step<DPP_QUAD_2301>(v, e);
  argmax_step<DPP_HALF_MIRROR>(v, e);
  argmax_step<DPP_MIRROR>(v, e);
  {
    const auto rv = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                     false, false);
    const auto re = __builtin_amdgcn_permlane16_swap((unsigned)e, (unsigned)e, false, false);
    v = __uint_as_float(rv[0]);
    e = (int)re[0];
    take_better(v, e, __uint_as_float(rv[1]), (int)re[1]);
  }
  {
    const auto rv = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                     false, false);
    const auto re = __builtin_amdgcn_permlane32_swap((unsigned)e, (unsigned)e, false, false);
    v = __uint_as_float(rv[0]);
    e = (int)re[0];
    take_better(v, e, __uint_as_float(rv[1]), (int)re[1]);
  }
}

// Softmax + top-k + renorm for the tokens of one block, logits in LDS rows of E_PAD.
// Waves take tokens tt = wave, wave + 4, ...  Accumulates p into psum (per lane, expert
// lane + 64 i) and the chosen experts into the LDS histogram cnt.  probs (optional)
// receives every p; k = 0 takes no top-k.  cand (optional, [T, k]) receives the experts
// ranked k+1 .. 2k by selection score (-1 past E).
template <int E_PAD>
__device__ inline void route_tail(const float* lg, int BT, int t0, int T, int E, int k,
                                  const float* __restrict__ bias, int32_t* __restrict__ topk_idx,
                                  float* __restrict__ topk_w, float* __restrict__ gap,
                                  float* __restrict__ probs, int32_t* __restrict__ cand,
                                  float* psum, int* cnt) {
  constexpr int NV = (E_PAD + 63) / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float bv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    bv[i] = (bias != nullptr && e < E) ? bias[e] : 0.0f;
  }
  for (int tt = w; tt < BT; tt += 4) {
    const int t = t0 + tt;
    if (t >= T) break;
    const float* row = lg + (size_t)tt * E_PAD;
    float v[NV];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      v[i] = (e < E) ? row[e] : -INFINITY;
      m = fmaxf(m, v[i]);
    }
    m = wave_max(m);
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      v[i] = (e < E) ? expf(v[i] - m) : 0.0f;
      sum += v[i];
    }
    sum = wave_sum(sum);
    const float inv = 1.0f / sum;
    float s[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      v[i] = v[i] * inv;                       // p
      psum[i] += v[i];
      s[i] = (e < E) ? v[i] + bv[i] : -INFINITY;   // selection score, fp32
      if (probs != nullptr && e < E) probs[(size_t)t * E + e] = v[i];
    }
    unsigned taken = 0;
    int my_idx = 0, my_cand = -1;
    float my_p = 0.0f, s_k = 0.0f, tot = 0.0f;
    // k rounds of wavefront argmax, then the candidates (extra rounds) and/or one more
    // for the gap
    const int extra = cand != nullptr ? min(k, E - k) : 0;
    const int rounds = k + max(extra, gap != nullptr ? 1 : 0);
    for (int r = 0; r < rounds; ++r) {
      float bvv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        const bool ok = (((taken >> i) & 1u) == 0u) & (e < E) &
                        ((s[i] > bvv) | ((s[i] == bvv) & (e < be)));
        bvv = ok ? s[i] : bvv;
        be = ok ? e : be;
      }
      wave_argmax(bvv, be);
      if (r >= k) {
        if (r == k && gap != nullptr && lane == 0) gap[t] = s_k - bvv;   // +inf when k == E
        if (r - k < extra) {   // candidate r - k: the (r+1)-th best expert
          const bool ok = be < E;
          if (ok && lane == (be & 63)) taken |= 1u << (be >> 6);
          if (lane == r - k) my_cand = ok ? be : -1;
        }
        continue;
      }
      s_k = bvv;
      const bool ok = be < E;   // always true for finite inputs and k <= E
      const int owner = ok ? (be & 63) : 0, slot = ok ? (be >> 6) : 0;
      float pp = 0.0f;
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (i == slot) pp = v[i];
      if (ok && lane == owner) taken |= 1u << slot;
      pp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pp), owner));
      tot += pp;   // sum of the chosen p in slot order
      if (lane == r) {
        my_idx = be;
        my_p = pp;
      }
      if (lane == 0 && be < E) atomicAdd(&cnt[be], 1);
    }
    if (lane < k) {
      topk_idx[(size_t)t * k + lane] = my_idx;
      topk_w[(size_t)t * k + lane] = my_p / tot;
      if (cand != nullptr) cand[(size_t)t * k + lane] = lane < extra ? my_cand : -1;
    }
  }
}

// Reductions over one token's segment of SEG = 16 or 32 lanes (DPP inside a row, then a
// permlane16 swap to join the two rows of a 32-lane segment); every lane of the segment
// ends with the same bits.
template <int SEG, class Op>
__device__ inline float seg_reduce(float v, Op op) {
  v = op(v, dpp_f<DPP_QUAD_1032>(v));
  v = op(v, dpp_f<DPP_QUAD_2301>(v));
  v = op(v, dpp_f<DPP_HALF_MIRROR>(v));
  v = op(v, dpp_f<DPP_MIRROR>(v));
  if constexpr (SEG == 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return v;
}
// (v, e, p) <- the better candidate (larger v, then lower e), p travelling with it.
template <int CTRL>
__device__ inline void seg_argmax_step(float& v, int& e, float& p) {
  const float ov = dpp_f<CTRL>(v), op_ = dpp_f<CTRL>(p);
  const int oe = dpp_i<CTRL>(e);
  const bool better = (ov > v) | ((ov == v) & (oe < e));   // compares and selects only
  v = better ? ov : v;
  e = better ? oe : e;
  p = better ? op_ : p;
}
template <int SEG>
__device__ inline void seg_argmax(float& v, int& e, float& p) {
  seg_argmax_step<DPP_QUAD_1032>(v, e, p);
  seg_argmax_step<DPP_QUAD_2301>(v, e, p);
  seg_argmax_step<DPP_HALF_MIRROR>(v, e, p);
  seg_argmax_step<DPP_MIRROR>(v, e, p);
  if constexpr (SEG == 32) {
    const auto rv = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                     false, false);
    const auto re = __builtin_amdgcn_permlane16_swap((unsigned)e, (unsigned)e, false, false);
    const auto rp = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(p),
                                                     false, false);
    v = __uint_as_float(rv[0]);
    e = (int)re[0];
    p = __uint_as_float(rp[0]);
    const float ov = __uint_as_float(rv[1]);
    const int oe = (int)re[1];
    const bool better = (ov > v) | ((ov == v) & (oe < e));
    v = better ? ov : v;
    e = better ? oe : e;
    p = better ? __uint_as_float(rp[1]) : p;
  }
}

// route_tail for E_PAD <= 32: a wave takes 64 / E_PAD tokens at once, one segment of
// E_PAD lanes per token (lane = expert), so the reductions of several tokens run side by
// side instead of one token after the other.  Same results as route_tail (the sums of p
// and of the chosen p run over the same values; only their order within a segment
// differs) and the same outputs.
template <int E_PAD>
__device__ inline void route_tail_packed(const float* lg, int BT, int t0, int T, int E, int k,
                                         const float* __restrict__ bias,
                                         int32_t* __restrict__ topk_idx,
                                         float* __restrict__ topk_w, float* __restrict__ gap,
                                         float* __restrict__ probs, int32_t* __restrict__ cand,
                                         float* psum, int* cnt) {
  static_assert(E_PAD == 16 || E_PAD == 32, "one or two 16-lane rows per token");
  constexpr int G = 64 / E_PAD;   // tokens per wave and pass
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = lane % E_PAD, sg = lane / E_PAD, seg0 = sg * E_PAD;
  const float bv = (bias != nullptr && e < E) ? bias[e] : 0.0f;
  float ps = 0.0f;
  const int extra = cand != nullptr ? min(k, E - k) : 0;
  const int rounds = k + max(extra, gap != nullptr ? 1 : 0);
  for (int tb = 0; tb < BT; tb += 4 * G) {
    const int tt = tb + w * G + sg;
    const int t = t0 + tt;
    const bool tok = tt < BT && t < T;   // segments past the batch compute, never write
    const float x = (tok && e < E) ? lg[(size_t)tt * E_PAD + e] : -INFINITY;
    const float m = seg_reduce<E_PAD>(x, [](float a, float b) { return fmaxf(a, b); });
    float pe = (tok && e < E) ? expf(x - m) : 0.0f;
    const float sum = seg_reduce<E_PAD>(pe, [](float a, float b) { return a + b; });
    pe = tok ? pe * (1.0f / sum) : 0.0f;   // p
    ps += pe;
    if (probs != nullptr && tok && e < E) probs[(size_t)t * E + e] = pe;
    const float sc = (e < E) ? pe + bv : -INFINITY;   // selection score, fp32
    bool taken = false;
    int my_idx = 0, my_cand = -1;
    float my_p = 0.0f, s_k = 0.0f, tot = 0.0f;
    for (int r = 0; r < rounds; ++r) {
      float bvv = (!taken && e < E) ? sc : -INFINITY;
      int be = (!taken && e < E) ? e : 0x7fffffff;
      float bp = pe;
      seg_argmax<E_PAD>(bvv, be, bp);
      const bool ok = be < E;
      if (r >= k) {
        if (r == k && gap != nullptr && tok && lane == seg0) gap[t] = s_k - bvv;
        if (r - k < extra) {
          if (ok && e == be) taken = true;
          if (lane == seg0 + r - k) my_cand = ok ? be : -1;
        }
        continue;
      }
      s_k = bvv;
      if (ok && e == be) taken = true;
      tot += bp;   // sum of the chosen p in slot order
      if (lane == seg0 + r) {
        my_idx = be;
        my_p = bp;
      }
      if (tok && lane == seg0 && ok) atomicAdd(&cnt[be], 1);
    }
    if (tok && e < k) {
      topk_idx[(size_t)t * k + e] = my_idx;
      topk_w[(size_t)t * k + e] = my_p / tot;
      if (cand != nullptr) cand[(size_t)t * k + e] = e < extra ? my_cand : -1;
    }
  }
  // the segments' partial sums of p, per expert, into lanes 0 .. E_PAD - 1
  {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(ps), __float_as_uint(ps),
                                                      false, false);
    float v = ps;
    if constexpr (E_PAD == 16) v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                      false, false);
    v = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
    psum[0] = v;
  }
}

// Writes the block's partial sum of p and its expert histogram (fixed order).
template <int E_PAD>
__device__ inline void route_block_stats(const float* psum, float (*pw)[E_PAD], const int* cnt,
                                         int E, float* __restrict__ p_part,
                                         int32_t* __restrict__ cnt_part) {
  constexpr int NV = (E_PAD + 63) / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (lane + 64 * i < E_PAD) pw[w][lane + 64 * i] = psum[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    p_part[(size_t)blockIdx.x * E + e] = ((pw[0][e] + pw[1][e]) + pw[2][e]) + pw[3][e];
    cnt_part[(size_t)blockIdx.x * E + e] = cnt[e];
  }
}

// One-block launches (fd.offsets set): the block's histogram is the whole batch's, so the
// dispatch follows in the same kernel: counts, f and P exactly as the expert scan forms
// them from the one block's partials, offsets of min(count, C), and each assignment's
// stable rank within its expert counted directly over the (at most 512) assignments.
template <int E_PAD>
__device__ inline void route_fused_dispatch(const RouteDispatch& fd, const float (*pw)[E_PAD],
                                            const int* cnt, int T, int E, int k,
                                            const int32_t* __restrict__ topk_idx) {
  __shared__ int offs[kMaxExperts + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int e = tid; e < E; e += blockDim.x) {
    const int c = cnt[e];
    fd.counts[e] = c;
    if (fd.f) fd.f[e] = (float)((double)c / (double)((int64_t)T * k));
    if (fd.p) fd.p[e] = (float)((double)(((pw[0][e] + pw[1][e]) + pw[2][e]) + pw[3][e]) / (double)T);
  }
  if (tid < 64) {   // offsets: exclusive scan of min(count, C), 64 experts at a time
    int run = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      int v = e < E ? cnt[e] : 0;
      if (fd.C >= 0 && v > fd.C) v = (int)fd.C;
      int incl = v;
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
      }
      if (e < E) offs[e] = run + incl - v;
      run += __shfl(incl, 63, 64);
    }
    if (lane == 0) offs[E] = run;
  }
  for (int i = tid; i < fd.nzero; i += blockDim.x) fd.zero[i] = 0;
  __syncthreads();
  for (int e = tid; e <= E; e += blockDim.x) fd.offsets[e] = offs[e];
  const int n = T * k;
  for (int i = tid; i < n; i += blockDim.x) {
    const int e = topk_idx[i];
    if ((unsigned)e >= (unsigned)E) {   // no expert (non-finite scores): dropped
      fd.slot_pos[i] = -1;
      continue;
    }
    int r = 0;
    for (int i2 = 0; i2 < i; ++i2) r += topk_idx[i2] == e ? 1 : 0;
    const bool keep = fd.C < 0 || (int64_t)r < fd.C;
    const int pos = offs[e] + r;
    fd.slot_pos[i] = keep ? pos : -1;
    if (keep) fd.perm_src[pos] = i;
  }
}

template <int EPW, int TPW, int KS, int R>
__global__ __launch_bounds__(256) void route_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Wr, const float* __restrict__ bias,
    int T, int d, int E, int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ gap, float* __restrict__ probs, int32_t* __restrict__ cand,
    float* __restrict__ p_part, int32_t* __restrict__ cnt_part, RouteDispatch fd) {
  constexpr int EW = 4 / KS;
  constexpr int E_PAD = 16 * EPW * EW;
  constexpr int BT = 16 * TPW;
  constexpr int NV = (E_PAD + 63) / 64;
  __shared__ float lg[KS][BT][E_PAD];
  __shared__ float pw[4][E_PAD];
  __shared__ int cnt[E_PAD];
  __shared__ __align__(16) unsigned char rbuf[4 * 16 * (TPW + EPW) * 128];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ew = w / KS, ks = w % KS;
  const int t0 = blockIdx.x * BT;
  const int r = lane & 15, g = lane >> 4;
  for (int e = threadIdx.x; e < E_PAD; e += blockDim.x) cnt[e] = 0;

  // Row segments: 16 bytes per lane, 8 lanes per 128-byte row segment of a 64-wide k chunk
  // (the loads coalesce; a lane per row, as the MFMA operand layout has it, runs the load
  // path at a quarter of its rate).  Segment i of the lane: token row 8 i + lane / 8 of the
  // block (i < 2 TPW), then expert row 8 (i - 2 TPW) + lane / 8 of the wave's slab, chunk
  // lane % 8.  Expert rows past E (padding of the last slab) read row E-1 and token rows
  // past T read row T-1; their logits are never used.  32-bit element offsets: T d and E d
  // are below 2^31.
  constexpr int NSEG = 2 * (TPW + EPW);
  int soff[NSEG];
#pragma unroll
  for (int i = 0; i < NSEG; ++i) {
    const int rr = 8 * (i < 2 * TPW ? i : i - 2 * TPW) + (lane >> 3);
    const int row = i < 2 * TPW ? min(t0 + rr, T - 1) : min(ew * EPW * 16 + rr, E - 1);
    soff[i] = row * d + 8 * (lane & 7);
  }
  // The wave's LDS buffer of one chunk: its 16 TPW token rows, then its 16 EPW expert rows,
  // 128 bytes each, 16-byte chunk c of row r at position c ^ ((r / 2) % 8) (conflict-free
  // stores and fragment reads).  Written and read by this wave only, in program order, so no
  // barrier.  Fragment (row r, k16 half h) of lane group g: chunk 2 g + h.
  unsigned char* wbuf = rbuf + w * (16 * (TPW + EPW) * 128);
  int swr[NSEG], frd[2];
#pragma unroll
  for (int i = 0; i < NSEG; ++i) {
    const int row = 8 * i + (lane >> 3);
    swr[i] = row * 128 + 16 * ((lane & 7) ^ ((row >> 1) & 7));
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) frd[h] = r * 128 + 16 * ((2 * g + h) ^ ((r >> 1) & 7));
  floatx4 acc[TPW][EPW];
#pragma unroll
  for (int tb = 0; tb < TPW; ++tb)
#pragma unroll
    for (int eb = 0; eb < EPW; ++eb) acc[tb][eb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // This wave's 64-wide k chunks are c = ks + KS*j, j < nj.  Their row segments go through a
  // ring of R register slots, loaded R-1 chunks ahead of the MFMAs.  Whole passes over
  // the ring run unguarded (a load past the end reads the last chunk again, a valid
  // address, and is never used); the remaining chunks, already loaded, finish after the
  // loop.  No loaded value is touched before its chunk's turn, so the loads of the next
  // R-1 chunks stay in flight while a chunk's MFMAs run.
  const int nchunk = d / 64;
  const int nj = (nchunk - ks + KS - 1) / KS;
  u32x4 seg[R][NSEG];
#define R_LOAD(SLOT, j)                                                                     \
  {                                                                                         \
    const int c_ = ks + KS * min((j), nj - 1);                                              \
    _Pragma("unroll") for (int i = 0; i < NSEG; ++i)                                        \
      seg[SLOT][i] = *reinterpret_cast<const u32x4*>((i < 2 * TPW ? x : Wr) + soff[i] + c_ * 64); \
  }
#define R_MFMA(SLOT)                                                                        \
  {                                                                                         \
    _Pragma("unroll") for (int i = 0; i < NSEG; ++i)                                        \
      *reinterpret_cast<u32x4*>(wbuf + swr[i]) = seg[SLOT][i];                              \
    _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                         \
      bf16x8 fa_[TPW], fb_[EPW];                                                            \
      _Pragma("unroll") for (int tb = 0; tb < TPW; ++tb)                                    \
        fa_[tb] = *reinterpret_cast<const bf16x8*>(wbuf + tb * 16 * 128 + frd[h]);          \
      _Pragma("unroll") for (int eb = 0; eb < EPW; ++eb)                                    \
        fb_[eb] = *reinterpret_cast<const bf16x8*>(wbuf + (TPW + eb) * 16 * 128 + frd[h]);  \
      _Pragma("unroll") for (int tb = 0; tb < TPW; ++tb)                                    \
        _Pragma("unroll") for (int eb = 0; eb < EPW; ++eb)                                  \
          acc[tb][eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa_[tb], fb_[eb], acc[tb][eb], \
                                                                0, 0, 0);                   \
    }                                                                                       \
  }
  if (nj > 0) {
#pragma unroll
    for (int q = 0; q < R - 1; ++q) R_LOAD(q, q);
    int j0 = 0;
    for (; j0 + R <= nj; j0 += R) {
#pragma unroll
      for (int q = 0; q < R; ++q) {
        R_LOAD((q + R - 1) % R, j0 + q + R - 1);
        __builtin_amdgcn_sched_barrier(0);   // keep each load group ahead of the MFMAs
        R_MFMA(q);
      }
    }
    // The last nj - j0 < R chunks are already in slots 0 .. nj - j0 - 1.
#pragma unroll
    for (int q = 0; q < R - 1; ++q)
      if (j0 + q < nj) R_MFMA(q);
  }
#undef R_LOAD
#undef R_MFMA
  // D[m][n] of a 16x16 MFMA block sits in lane n + 16*(m/4), register m%4.
#pragma unroll
  for (int tb = 0; tb < TPW; ++tb)
#pragma unroll
    for (int eb = 0; eb < EPW; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lg[ks][tb * 16 + 4 * g + i][(ew * EPW + eb) * 16 + r] = acc[tb][eb][i];
  __syncthreads();
  if (KS > 1) {
    for (int idx = threadIdx.x; idx < BT * E_PAD; idx += blockDim.x) {
      float* base = &lg[0][0][0];
      float v = base[idx];
      for (int q = 1; q < KS; ++q) v += base[q * BT * E_PAD + idx];
      base[idx] = v;
    }
    __syncthreads();
  }
  float psum[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) psum[i] = 0.0f;
  if constexpr (E_PAD <= 32)
    route_tail_packed<E_PAD>(&lg[0][0][0], BT, t0, T, E, k, bias, topk_idx, topk_w, gap, probs,
                             cand, psum, cnt);
  else
    route_tail<E_PAD>(&lg[0][0][0], BT, t0, T, E, k, bias, topk_idx, topk_w, gap, probs, cand,
                      psum, cnt);
  __syncthreads();
  route_block_stats<E_PAD>(psum, pw, cnt, E, p_part, cnt_part);
  if (fd.offsets != nullptr) {
    __syncthreads();   // the top-k indices written above are visible to the whole block
    route_fused_dispatch<E_PAD>(fd, pw, cnt, T, E, k, topk_idx);
  }
}

// fp32 layers: plain FMA dot products (small correctness-sized layers).
template <int E_PAD>
__global__ __launch_bounds__(256) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ Wr, const float* __restrict__ bias,
    int T, int d, int E, int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ gap, float* __restrict__ probs, int32_t* __restrict__ cand,
    float* __restrict__ p_part, int32_t* __restrict__ cnt_part) {
  constexpr int BT = 16;
  constexpr int NV = (E_PAD + 63) / 64;
  __shared__ float lg[BT][E_PAD];
  __shared__ float pw[4][E_PAD];
  __shared__ int cnt[E_PAD];
  const int t0 = blockIdx.x * BT;
  for (int e = threadIdx.x; e < E_PAD; e += blockDim.x) cnt[e] = 0;
  for (int idx = threadIdx.x; idx < BT * E; idx += blockDim.x) {
    const int tt = idx / E, e = idx % E;
    const int t = min(t0 + tt, T - 1);
    const float4* xa = reinterpret_cast<const float4*>(x + (size_t)t * d);
    const float4* wb = reinterpret_cast<const float4*>(Wr + (size_t)e * d);
    float acc = 0.0f;
    for (int i = 0; i < d / 4; ++i) {
      const float4 a = xa[i], b = wb[i];
      acc = fmaf(a.x, b.x, acc);
      acc = fmaf(a.y, b.y, acc);
      acc = fmaf(a.z, b.z, acc);
      acc = fmaf(a.w, b.w, acc);
    }
    lg[tt][e] = acc;
  }
  __syncthreads();
  float psum[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) psum[i] = 0.0f;
  route_tail<E_PAD>(&lg[0][0], BT, t0, T, E, k, bias, topk_idx, topk_w, gap, probs, cand, psum,
                    cnt);
  __syncthreads();
  route_block_stats<E_PAD>(psum, pw, cnt, E, p_part, cnt_part);
}

RoutePlan route_plan(const moe_desc_t& d) {
  RoutePlan p{};
  const int E = (int)d.n_experts;
  if (d.dtype == MOE_DTYPE_F32) {
    int ep = 64;
    while (ep < E) ep *= 2;
    p.EPW = 0;
    p.TPW = 1;
    p.KS = 1;
    p.BT = 16;
    p.E_pad = ep;
  } else {
    int EW;
    if (E <= 16) {
      EW = 1;
      p.EPW = 1;
    } else if (E <= 32) {
      EW = 2;
      p.EPW = 1;
    } else if (E <= 64) {
      // every wave takes all 64 (padded) experts over a quarter of d, so each token row is
      // loaded once per block instead of once per wave (Switch-shaped router, E 64, T 16384:
      // 62 -> 40 us against four 16-expert slabs over the whole d; at E 256 two 128-expert
      // slabs over half of d were slower than four slabs, 0.26 against 0.20 ms)
      EW = 1;
      p.EPW = 4;
    } else {
      EW = 4;
      int epw = 1;
      while (epw * 64 < E) epw *= 2;
      p.EPW = epw;
    }
    p.KS = 4 / EW;
    p.TPW = ((EW == 4 || p.EPW == 4) && p.EPW <= 4 && ceil_div(d.T, 32) >= 256) ? 2 : 1;
    p.BT = 16 * p.TPW;
    p.E_pad = 16 * p.EPW * EW;
  }
  p.n_blocks = ceil_div(d.T, p.BT);
  return p;
}

hipError_t launch_route(const moe_desc_t& d, const void* x, const void* W_router,
                        const float* bias, int32_t* topk_idx, float* topk_w, float* gap,
                        float* probs, int32_t* cand, float* p_part, int32_t* cnt_part,
                        hipStream_t s, const RouteDispatch* fused) {
  const RoutePlan rp = route_plan(d);
  if (rp.n_blocks == 0) return hipSuccess;
  const int T = (int)d.T, dm = (int)d.d_model, E = (int)d.n_experts;
  const int k = topk_idx != nullptr ? (int)d.top_k : 0;
  const dim3 grid((unsigned)rp.n_blocks), block(256);
  if (d.dtype == MOE_DTYPE_F32) {
    if (fused != nullptr) return hipErrorInvalidValue;   // bf16 layers only
    const float* xx = (const float*)x;
    const float* ww = (const float*)W_router;
#define MOE_ROUTE_F32(EP)                                                                     \
  if (rp.E_pad == EP) {                                                                       \
    hipLaunchKernelGGL(route_f32_kernel<EP>, grid, block, 0, s, xx, ww, bias, T, dm, E, k,    \
                       topk_idx, topk_w, gap, probs, cand, p_part, cnt_part);                 \
    return hipGetLastError();                                                                 \
  }
    MOE_ROUTE_F32(64)
    MOE_ROUTE_F32(128)
    MOE_ROUTE_F32(256)
    MOE_ROUTE_F32(512)
#undef MOE_ROUTE_F32
    return hipErrorInvalidValue;
  }
  const bf16_t* xx = (const bf16_t*)x;
  const bf16_t* ww = (const bf16_t*)W_router;
  RouteDispatch fd{};
  if (fused != nullptr) {
    if (rp.n_blocks != 1 || k == 0 || (int64_t)T * k > 512) return hipErrorInvalidValue;
    fd = *fused;
  }
// R: ring slots of k-chunk fragments (8 (EPW + TPW) VGPRs each).  Eight for the one-slab
// layouts of small batches (latency-bound: one or few blocks); fewer where many blocks
// share a CU and registers decide how many (measured: the Switch-shaped router takes
// 61 us with 4 slots, 66 us with 8).  The loads in flight (2 (EPW + TPW) per slot) stay
// within what vmcnt counts.
#define MOE_ROUTE_BF16(EPW_, TPW_, KS_)                                                      \
  if (rp.EPW == EPW_ && rp.TPW == TPW_ && rp.KS == KS_) {                                     \
    constexpr int R_ = (EPW_ + TPW_) <= 2 ? 8 : (EPW_ + TPW_) <= 3 ? 4 : 2;                   \
    hipLaunchKernelGGL((route_bf16_kernel<EPW_, TPW_, KS_, R_>), grid, block, 0, s, xx, ww,   \
                       bias, T, dm, E, k, topk_idx, topk_w, gap, probs, cand, p_part,         \
                       cnt_part, fd);                                                         \
    return hipGetLastError();                                                                 \
  }
  MOE_ROUTE_BF16(1, 1, 4)
  MOE_ROUTE_BF16(1, 1, 2)
  MOE_ROUTE_BF16(1, 1, 1)
  MOE_ROUTE_BF16(1, 2, 1)
  MOE_ROUTE_BF16(2, 1, 1)
  MOE_ROUTE_BF16(2, 2, 1)
  MOE_ROUTE_BF16(4, 1, 1)
  MOE_ROUTE_BF16(4, 2, 1)
  MOE_ROUTE_BF16(8, 1, 1)
  MOE_ROUTE_BF16(4, 1, 4)
  MOE_ROUTE_BF16(4, 2, 4)
#undef MOE_ROUTE_BF16
  return hipErrorInvalidValue;
}

}  // namespace moe
