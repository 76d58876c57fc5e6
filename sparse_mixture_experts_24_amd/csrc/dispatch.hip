// Dispatch: expert histogram, capacity cut, prefix sum and the stable permutation of
// the T*k (token, slot) assignments into expert-contiguous order.
//
// "Mixture-of-experts in practice" (deepseekmodel.com), expert-parallel section: the
// assignments are flattened row-major and stably grouped by expert with a bincount;
// routing-math section: per-expert capacity from the expected load, at least k.
// "Chapter 30" (LLM Transformer book), 30.5.2: overflow beyond the capacity is dropped.
//
// Three passes, none of whose results depend on atomic ordering:
//   hist     block b counts the experts of assignments [b*chunk, (b+1)*chunk) with LDS
//            atomics (integer adds commute) -> blk[b][e]
//   scan     one block per expert: exclusive prefix over blocks (blk -> base), total
//            = count (and the f, P statistics when the router's partials are given)
//   scatter  every block derives offsets = exclusive scan of kept = min(count, C) over
//            the experts; block b walks its chunk in order, 256 per round; the rank of an
//            assignment among equal experts inside a wavefront comes from ballots on
//            the bits of the expert id, across wavefronts from LDS counts, across
//            rounds and blocks from the running base: rank = stable position within
//            the expert; keep iff rank < C; row = offsets[e] + rank.
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int64_t NA,
                                                   int E, int chunk, int32_t* __restrict__ blk) {
  __shared__ int h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * chunk;
  for (int q = threadIdx.x; q < chunk; q += blockDim.x) {
    const int64_t i = base + q;
    if (i < NA) {
      const int e = idx[i];
      if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) blk[(int64_t)blockIdx.x * E + e] = h[e];
}

hipError_t launch_hist(const int32_t* idx, int64_t NA, int E, int chunk, int32_t* blk,
                       hipStream_t s) {
  const int64_t nb = ceil_div(NA, chunk);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(hist_kernel, dim3((unsigned)nb), dim3(256), 0, s, idx, NA, E, chunk, blk);
  return hipGetLastError();
}

// One block per expert e: the exclusive prefix over histogram blocks of blk[b][e] (in
// place: the blocks' bases), the total count, and optionally the statistics
//   f_e = count_e / (T k),  P_e = sum_b p_part[b][e] / T
// (p summed per thread over a fixed stride of blocks, then by a fixed tree: the result
// does not depend on timing).
__global__ __launch_bounds__(256) void expert_scan_kernel(int32_t* __restrict__ blk, int64_t nb,
                                                          int E, const float* __restrict__ p_part,
                                                          int64_t T, int k, int32_t* __restrict__ counts,
                                                          float* __restrict__ f, float* __restrict__ p,
                                                          int32_t* __restrict__ zero, int nzero) {
  __shared__ int wsum[4];
  __shared__ float red[256];
  const int e = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  if (e == 0 && t < nzero) zero[t] = 0;   // the grouped GEMMs' work counters, if asked
  int run = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += 256) {
    const int64_t b = b0 + t;
    const int v = b < nb ? blk[b * E + e] : 0;
    int incl = v;
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int before = run;
    for (int q = 0; q < w; ++q) before += wsum[q];
    if (b < nb) blk[b * E + e] = before + incl - v;
    run += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  float ps = 0.0f;
  if (p_part) {
    for (int64_t b = t; b < nb; b += 256) ps += p_part[b * E + e];
    red[t] = ps;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (t < o) red[t] += red[t + o];
      __syncthreads();
    }
  }
  if (t == 0) {
    counts[e] = run;
    if (f) f[e] = T > 0 ? (float)((double)run / (double)(T * k)) : 0.0f;
    if (p) p[e] = (T > 0 && p_part) ? (float)((double)red[0] / (double)T) : 0.0f;
  }
}

hipError_t launch_expert_scan(int32_t* blk, int64_t nb, int E, const float* p_part, int64_t T,
                              int k, int32_t* counts, float* f, float* p, int32_t* zero,
                              int nzero, hipStream_t s) {
  hipLaunchKernelGGL(expert_scan_kernel, dim3(E), dim3(256), 0, s, blk, nb, E, p_part, T, k,
                     counts, f, p, zero, zero ? nzero : 0);
  return hipGetLastError();
}

// offsets = exclusive scan over experts of kept_e = min(count_e, C) (C < 0: no limit),
// computed by every block into LDS; block 0 also writes it out.
__device__ inline void block_offsets(const int32_t* __restrict__ counts, int E, int64_t C,
                                     int* offs, int32_t* __restrict__ offsets_out) {
  __shared__ int wsum[4];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int run = 0;
  for (int e0 = 0; e0 < E; e0 += 256) {
    const int e = e0 + t;
    int v = 0;
    if (e < E) {
      v = counts[e];
      if (C >= 0 && v > C) v = (int)C;
    }
    int incl = v;
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int before = run;
    for (int q = 0; q < w; ++q) before += wsum[q];
    if (e < E) offs[e] = before + incl - v;
    run += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (t == 0) offs[E] = run;
  __syncthreads();
  if (blockIdx.x == 0 && offsets_out)
    for (int e = t; e <= E; e += blockDim.x) offsets_out[e] = offs[e];
}

__global__ __launch_bounds__(256) void scatter_kernel(
    const int32_t* __restrict__ idx, int64_t NA, int E, int chunk, int64_t C,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ slot_pos) {
  __shared__ int run[kMaxExperts];
  __shared__ int wc[4][kMaxExperts];
  __shared__ int offsets[kMaxExperts + 1];
  block_offsets(counts, E, C, offsets, offsets_out);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool has_work = (int64_t)blockIdx.x * chunk < NA;   // (NA == 0: offsets only)
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    run[e] = has_work ? blk_base[(int64_t)blockIdx.x * E + e] : 0;
    wc[0][e] = wc[1][e] = wc[2][e] = wc[3][e] = 0;
  }
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * chunk;
  for (int q0 = 0; q0 < chunk; q0 += 256) {
    const int64_t i = base + q0 + threadIdx.x;
    const bool inb = (q0 + (int)threadIdx.x < chunk) && i < NA;
    const int ev = inb ? idx[i] : 0;
    const bool valid = inb && (unsigned)ev < (unsigned)E;   // out-of-range ids: dropped
    const int e = valid ? ev : 0;
    if (inb && !valid) slot_pos[i] = -1;
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t m = __ballot(on);
      peers &= on ? m : ~m;
    }
    const int lrank = __popcll(peers & below);
    if (valid && lrank == 0) wc[w][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int r = run[e] + lrank;
      for (int q = 0; q < w; ++q) r += wc[q][e];
      const bool keep = (C < 0) || ((int64_t)r < C);
      const int pos = offsets[e] + r;
      slot_pos[i] = keep ? pos : -1;
      if (keep) perm_src[pos] = (int32_t)i;
    }
    __syncthreads();
    for (int ee = threadIdx.x; ee < E; ee += blockDim.x) {
      run[ee] += wc[0][ee] + wc[1][ee] + wc[2][ee] + wc[3][ee];
      wc[0][ee] = wc[1][ee] = wc[2][ee] = wc[3][ee] = 0;
    }
    __syncthreads();
  }
}

hipError_t launch_scatter(const int32_t* idx, int64_t NA, int E, int chunk, int64_t C,
                          const int32_t* blk_base, const int32_t* counts, int32_t* offsets,
                          int32_t* perm_src, int32_t* slot_pos, hipStream_t s) {
  // at least one block, so that the offsets are written even with no assignments
  const int64_t nb = NA > 0 ? ceil_div(NA, chunk) : 1;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)nb), dim3(256), 0, s, idx, NA, E, chunk, C,
                     blk_base, counts, offsets, perm_src, slot_pos);
  return hipGetLastError();
}

}  // namespace moe
