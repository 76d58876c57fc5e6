// Weighted combine back to token order:
//   out[t] = sum_{j ascending, slot kept} w[t,j] * Yp[slot_pos[t,j]]  (+ Yp[T*k + t])
// "Chapter 30: Mixture of Experts" (LLM Transformer book), 30.6.1 (weighted sum of the
// chosen experts' outputs) and 30.4.5 (shared expert added); "Mixture-of-experts in
// practice" (deepseekmodel.com), capacity section (a dropped assignment contributes 0).
//
// HBM-bound gather: one block per token row, float4 loads of the k expert rows, fp32
// sums in a fixed slot order (deterministic, no atomics), one coalesced row write.
#include "moe_internal.h"

namespace moe {

template <typename OutT>
__device__ inline void store4(OutT* out, int64_t i, float4 v);
template <>
__device__ inline void store4<float>(float* out, int64_t i, float4 v) {
  *reinterpret_cast<float4*>(out + i) = v;
}
template <>
__device__ inline void store4<bf16_t>(bf16_t* out, int64_t i, float4 v) {
  const uint32_t lo = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
  *reinterpret_cast<uint2*>(out + i) = make_uint2(lo, hi);
}

// Yp2 (optional): second partial of a K-split down GEMM; a slot's output is Yp + Yp2.
template <typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Yp,
                                                      const float* __restrict__ Yp2,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ w, int T, int k,
                                                      int d, int shared, OutT* __restrict__ out) {
  const int t = blockIdx.x;
  __shared__ int sp[kMaxTopK];
  __shared__ float sw[kMaxTopK];
  if (threadIdx.x < k) {
    sp[threadIdx.x] = slot_pos[(int64_t)t * k + threadIdx.x];
    sw[threadIdx.x] = w[(int64_t)t * k + threadIdx.x];
  }
  __syncthreads();
  const int64_t srow = (int64_t)T * k + t;
  for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int pos = sp[j];
      if (pos < 0) continue;
      float4 v = *reinterpret_cast<const float4*>(Yp + (int64_t)pos * d + c);
      if (Yp2) {
        const float4 v2 = *reinterpret_cast<const float4*>(Yp2 + (int64_t)pos * d + c);
        v.x += v2.x;
        v.y += v2.y;
        v.z += v2.z;
        v.w += v2.w;
      }
      const float wj = sw[j];
      acc.x = fmaf(wj, v.x, acc.x);
      acc.y = fmaf(wj, v.y, acc.y);
      acc.z = fmaf(wj, v.z, acc.z);
      acc.w = fmaf(wj, v.w, acc.w);
    }
    if (shared) {
      float4 v = *reinterpret_cast<const float4*>(Yp + srow * d + c);
      if (Yp2) {
        const float4 v2 = *reinterpret_cast<const float4*>(Yp2 + srow * d + c);
        v.x += v2.x;
        v.y += v2.y;
        v.z += v2.z;
        v.w += v2.w;
      }
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    store4<OutT>(out, (int64_t)t * d + c, acc);
  }
}

hipError_t launch_combine(const moe_desc_t& d, const float* Yp, const float* Yp2,
                          const int32_t* slot_pos, const float* topk_w, void* out, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  const dim3 grid((unsigned)d.T), block(256);
  const int T = (int)d.T, k = (int)d.top_k, dm = (int)d.d_model, sh = (int)d.n_shared;
  if (d.out_dtype == MOE_DTYPE_F32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, s, Yp, Yp2, slot_pos, topk_w, T, k, dm,
                       sh, (float*)out);
  else
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, block, 0, s, Yp, Yp2, slot_pos, topk_w, T, k, dm,
                       sh, (bf16_t*)out);
  return hipGetLastError();
}

}  // namespace moe
