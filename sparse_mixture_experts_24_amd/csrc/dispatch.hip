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
//   scan     one block: per expert, exclusive prefix over blocks (blk -> base), totals
//            = counts, kept = min(count, C), offsets = exclusive scan of kept
//   scatter  block b walks its chunk in order, 256 assignments per round; the rank of an
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

// One block of 1024 threads.  C < 0: no capacity limit.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ blk, int64_t nb, int E,
                                                    int64_t C, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int kept[1024];
  __shared__ int wsum[16];
  const int t = threadIdx.x;
  int kv = 0;
  if (t < E) {
    int run = 0;
    for (int64_t b = 0; b < nb; ++b) {
      const int c = blk[b * E + t];
      blk[b * E + t] = run;
      run += c;
    }
    counts[t] = run;
    kv = (C < 0 || run < C) ? run : (int)C;
  }
  // exclusive scan of kept over experts: wave inclusive scan, then across waves
  const int lane = t & 63, w = t >> 6;
  int incl = kv;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0;
  for (int q = 0; q < w; ++q) before += wsum[q];
  kept[t] = before + incl - kv;   // exclusive
  __syncthreads();
  if (t < E) offsets[t] = kept[t];
  if (t == E - 1) offsets[E] = kept[t] + kv;
}

hipError_t launch_scan(int32_t* blk, int64_t nb, int E, int64_t C, int32_t* counts,
                       int32_t* offsets, hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, blk, nb, E, C, counts, offsets);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void scatter_kernel(
    const int32_t* __restrict__ idx, int64_t NA, int E, int chunk, int64_t C,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_src, int32_t* __restrict__ slot_pos) {
  __shared__ int run[kMaxExperts];
  __shared__ int wc[4][kMaxExperts];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    run[e] = blk_base[(int64_t)blockIdx.x * E + e];
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
                          const int32_t* blk_base, const int32_t* offsets, int32_t* perm_src,
                          int32_t* slot_pos, hipStream_t s) {
  const int64_t nb = ceil_div(NA, chunk);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)nb), dim3(256), 0, s, idx, NA, E, chunk, C,
                     blk_base, offsets, perm_src, slot_pos);
  return hipGetLastError();
}

}  // namespace moe
