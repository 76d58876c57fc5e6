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

// The slots are read KB at a time (KB = 8 for k > 4: the fine-grained layer's 8 slots and
// its shared row in one batch), all loads of a batch issued before any is used (a dropped
// slot loads row 0 and contributes nothing), so each thread keeps up to KB + 1 16-byte
// loads in flight; the sum runs over the slots in ascending order, the shared row last.
template <typename OutT, int KB>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Yp,
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
    // the shared expert's row is loaded with the first batch of slots, added after all
    float4 vs = make_float4(0.f, 0.f, 0.f, 0.f);
    if (shared) vs = *reinterpret_cast<const float4*>(Yp + srow * d + c);
    for (int j0 = 0; j0 < k; j0 += KB) {
      float4 v[KB];
      bool ok[KB];
#pragma unroll
      for (int q = 0; q < KB; ++q) {
        const int j = j0 + q;
        const int pos = j < k ? sp[j] : -1;
        ok[q] = pos >= 0;
        const int64_t off = (int64_t)(ok[q] ? pos : 0) * d + c;
        v[q] = *reinterpret_cast<const float4*>(Yp + off);
      }
#pragma unroll
      for (int q = 0; q < KB; ++q) {
        if (!ok[q]) continue;
        const float wj = sw[j0 + q];
        acc.x = fmaf(wj, v[q].x, acc.x);
        acc.y = fmaf(wj, v[q].y, acc.y);
        acc.z = fmaf(wj, v[q].z, acc.z);
        acc.w = fmaf(wj, v[q].w, acc.w);
      }
    }
    if (shared) {
      acc.x += vs.x;
      acc.y += vs.y;
      acc.z += vs.z;
      acc.w += vs.w;
    }
    store4<OutT>(out, (int64_t)t * d + c, acc);
  }
}

template <typename OutT>
static void launch_combine_o(const moe_desc_t& d, const float* Yp, const int32_t* slot_pos,
                             const float* topk_w, OutT* out, hipStream_t s) {
  const dim3 grid((unsigned)d.T), block(256);
  const int T = (int)d.T, k = (int)d.top_k, dm = (int)d.d_model, sh = (int)d.n_shared;
  if (k == 1)
    hipLaunchKernelGGL((combine_kernel<OutT, 1>), grid, block, 0, s, Yp, slot_pos, topk_w, T, k,
                       dm, sh, out);
  else if (k == 2)
    hipLaunchKernelGGL((combine_kernel<OutT, 2>), grid, block, 0, s, Yp, slot_pos, topk_w, T, k,
                       dm, sh, out);
  else if (k <= 4)
    hipLaunchKernelGGL((combine_kernel<OutT, 4>), grid, block, 0, s, Yp, slot_pos, topk_w, T, k,
                       dm, sh, out);
  else
    hipLaunchKernelGGL((combine_kernel<OutT, 8>), grid, block, 0, s, Yp, slot_pos, topk_w, T, k,
                       dm, sh, out);
}

hipError_t launch_combine(const moe_desc_t& d, const float* Yp, const int32_t* slot_pos,
                          const float* topk_w, void* out, hipStream_t s) {
  if (d.T == 0) return hipSuccess;
  if (d.out_dtype == MOE_DTYPE_F32)
    launch_combine_o<float>(d, Yp, slot_pos, topk_w, (float*)out, s);
  else
    launch_combine_o<bf16_t>(d, Yp, slot_pos, topk_w, (bf16_t*)out, s);
  return hipGetLastError();
}

}  // namespace moe
