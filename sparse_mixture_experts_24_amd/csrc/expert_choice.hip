// Expert-choice routing: every expert takes the C tokens with the largest router
// probability, and the combine weights each expert's output by that probability.
//
// "Mixture of Experts (MoE) memo" (iwashi.co), routing section: in the expert-choice row
// of the routing-design table each expert picks the tokens that suit it, so every
// expert's load is the same; "Mixture-of-experts in practice" (deepseekmodel.com), top-k
// section: each expert takes its top-C tokens according to its capacity, no token is
// dropped for capacity, and the choice depends on the whole batch.
//
// Selection: one block per expert.  Probabilities are non-negative floats, so their bit
// patterns order like the values; the C-th largest key is found by a most-significant-
// digit radix select (four 8-bit passes over an LDS histogram), then a token is taken if
// its key is larger, or equal and among the first (C - #larger) equal keys in token
// order.  Two block-wide scans in token order give each taken token its row.
#include "moe_internal.h"

namespace moe {

constexpr int EC_THREADS = 1024;

// Exclusive prefix sum of v over the block's threads in thread order; *total gets the
// sum.  wsum: 16 ints of LDS.  Contains barriers: every thread must call it.
__device__ inline int block_exclusive_scan(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int NW = EC_THREADS / 64;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int q = 0; q < NW; ++q) {
    const int x = wsum[q];
    before += q < w ? x : 0;
    all += x;
  }
  __syncthreads();   // wsum is free again on return
  *total = all;
  return before + incl - v;
}

// KPT: tokens per thread (T <= 1024 KPT); thread i holds tokens [i KPT, (i + 1) KPT).
template <int KPT>
__global__ __launch_bounds__(EC_THREADS) void ec_select_kernel(
    const float* __restrict__ probs, int T, int E, int C, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot, float* __restrict__ f) {
  __shared__ int hist[256];
  __shared__ int wsum[EC_THREADS / 64];
  __shared__ unsigned sh_digit;
  __shared__ int sh_rem;
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t0 = tid * KPT;
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int t = t0 + j;
    key[j] = t < T ? __float_as_uint(probs[(size_t)t * E + e]) : 0u;
  }

  // Radix select of the C-th largest key, most significant byte first.
  uint32_t prefix = 0, mask = 0;
  int remaining = C;   // how many of the keys matching prefix are still to be taken
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (t0 + j < T && (key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & 255u], 1);
    __syncthreads();
    if (w == 0) {
      // lane l holds digits 255 - 4l .. 252 - 4l (descending); counts above a digit are
      // the lanes before plus the digits before it in the lane
      int c[4], own = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = hist[255 - 4 * lane - q];
        own += c[q];
      }
      int incl = own;
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
      }
      int above = incl - own;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (above < remaining && above + c[q] >= remaining) {   // exactly one digit
          sh_digit = (unsigned)(255 - 4 * lane - q);
          sh_rem = remaining - above;
        }
        above += c[q];
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    remaining = sh_rem;
  }
  const uint32_t kappa = prefix;   // the C-th largest key
  const int need = remaining;      // keys equal to kappa that are taken, first in token order

  int eq = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) eq += (t0 + j < T && key[j] == kappa) ? 1 : 0;
  int total;
  int eq_rank = block_exclusive_scan(eq, wsum, &total);
  unsigned taken = 0;
  int n_taken = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (t0 + j >= T) continue;
    bool take = key[j] > kappa;
    if (key[j] == kappa) {
      take = eq_rank < need;
      ++eq_rank;
    }
    if (take) {
      taken |= 1u << j;
      ++n_taken;
    }
  }
  int row = block_exclusive_scan(n_taken, wsum, &total);
  const int64_t base = (int64_t)e * C;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int t = t0 + j;
    if (t >= T) continue;
    if ((taken >> j) & 1u) {
      perm_src[base + row] = t;
      slot[(size_t)t * E + e] = (int32_t)(base + row);
      ++row;
    } else {
      slot[(size_t)t * E + e] = -1;
    }
  }
  if (tid == 0) {
    offsets[e] = (int32_t)base;
    if (e == E - 1) offsets[E] = (int32_t)(base + C);
    if (f) f[e] = C > 0 ? 1.0f / (float)E : 0.0f;   // every expert takes C of the E C rows
  }
}

hipError_t launch_ec_select(const float* probs, int T, int E, int C, int32_t* perm_src,
                            int32_t* offsets, int32_t* slot, float* f, hipStream_t s) {
  if (E <= 0) return hipSuccess;
  const dim3 grid((unsigned)E), block(EC_THREADS);
#define MOE_EC_SELECT(KPT_)                                                                   \
  if (T <= EC_THREADS * KPT_) {                                                               \
    hipLaunchKernelGGL(ec_select_kernel<KPT_>, grid, block, 0, s, probs, T, E, C, perm_src,   \
                       offsets, slot, f);                                                     \
    return hipGetLastError();                                                                 \
  }
  MOE_EC_SELECT(1)
  MOE_EC_SELECT(2)
  MOE_EC_SELECT(4)
  MOE_EC_SELECT(8)
  MOE_EC_SELECT(16)
  MOE_EC_SELECT(32)
#undef MOE_EC_SELECT
  return hipErrorInvalidValue;
}

template <typename OutT>
__device__ inline void ec_store4(OutT* out, int64_t i, float4 v);
template <>
__device__ inline void ec_store4<float>(float* out, int64_t i, float4 v) {
  *reinterpret_cast<float4*>(out + i) = v;
}
template <>
__device__ inline void ec_store4<bf16_t>(bf16_t* out, int64_t i, float4 v) {
  const uint32_t lo = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
  *reinterpret_cast<uint2*>(out + i) = make_uint2(lo, hi);
}

// One block per token.  Wave 0 lists the token's taken experts in ascending order (row and
// weight, through LDS); then each thread sums float4 columns over the list, four rows in
// flight at a time.
template <typename OutT>
__global__ __launch_bounds__(256) void ec_combine_kernel(const float* __restrict__ Yp,
                                                         const int32_t* __restrict__ slot,
                                                         const float* __restrict__ probs, int E,
                                                         int d, int shared, int64_t shared_row0,
                                                         OutT* __restrict__ out) {
  constexpr int KB = 4;
  __shared__ int rows[kMaxExperts];
  __shared__ float wts[kMaxExperts];
  __shared__ int n_sh;
  const int t = blockIdx.x, lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    int n = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int pos = e < E ? slot[(size_t)t * E + e] : -1;
      const uint64_t m = __ballot(pos >= 0);
      const int before = __popcll(m & ((1ull << lane) - 1ull));
      if (pos >= 0) {
        rows[n + before] = pos;
        wts[n + before] = probs[(size_t)t * E + e];
      }
      n += __popcll(m);
    }
    if (lane == 0) n_sh = n;
  }
  __syncthreads();
  const int n = n_sh;
  const int64_t srow = shared_row0 + t;
  for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < n; j0 += KB) {
      float4 v[KB];
#pragma unroll
      for (int q = 0; q < KB; ++q) {
        const int j = j0 + q;
        const int64_t off = (int64_t)(j < n ? rows[j] : rows[j0]) * d + c;
        v[q] = *reinterpret_cast<const float4*>(Yp + off);
      }
#pragma unroll
      for (int q = 0; q < KB; ++q) {
        if (j0 + q >= n) break;
        const float wj = wts[j0 + q];
        acc.x = fmaf(wj, v[q].x, acc.x);
        acc.y = fmaf(wj, v[q].y, acc.y);
        acc.z = fmaf(wj, v[q].z, acc.z);
        acc.w = fmaf(wj, v[q].w, acc.w);
      }
    }
    if (shared) {
      const float4 v = *reinterpret_cast<const float4*>(Yp + srow * d + c);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    ec_store4<OutT>(out, (int64_t)t * d + c, acc);
  }
}

hipError_t launch_ec_combine(const moe_desc_t& d, int64_t shared_row0, const float* Yp,
                             const int32_t* slot, const float* probs, void* out, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  const dim3 grid((unsigned)d.T), block(256);
  const int E = (int)d.n_experts, dm = (int)d.d_model, sh = (int)d.n_shared;
  if (d.out_dtype == MOE_DTYPE_F32)
    hipLaunchKernelGGL(ec_combine_kernel<float>, grid, block, 0, s, Yp, slot, probs, E, dm, sh,
                       shared_row0, (float*)out);
  else
    hipLaunchKernelGGL(ec_combine_kernel<bf16_t>, grid, block, 0, s, Yp, slot, probs, E, dm, sh,
                       shared_row0, (bf16_t*)out);
  return hipGetLastError();
}

}  // namespace moe
