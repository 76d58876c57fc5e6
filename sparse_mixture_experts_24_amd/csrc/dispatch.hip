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
//
// Overflow handed to the next-best expert ("Chapter 30", 30.5.2: tokens past the
// capacity are dropped or go to the next-best expert), one redirect round:
//   ranks    the scatter's stable ranks, kept raw (rank0)
//   offers   the m-th assignment of token t with rank0 >= C (slot order) is offered to
//            cand[t, m], the token's (k+1+m)-th best expert; block histograms of offers
//   scan     offer bases and counts per expert
//   place    offsets of kept0_e + accepted_e (kept0 = min(count, C), accepted = the first
//            C - kept0 offers in row-major order); round-0 rows first, then accepted
//            offers, each in row-major order.
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
// computed by every block into LDS; block 0 also writes it out.  With ocounts (offers per
// expert) kept_e also takes min(ocount_e, C - min(count_e, C)) accepted offers, and kept0
// (LDS) receives min(count_e, C).
__device__ inline void block_offsets(const int32_t* __restrict__ counts, int E, int64_t C,
                                     int* offs, int32_t* __restrict__ offsets_out,
                                     const int32_t* __restrict__ ocounts = nullptr,
                                     int* kept0 = nullptr) {
  __shared__ int wsum[4];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int run = 0;
  for (int e0 = 0; e0 < E; e0 += 256) {
    const int e = e0 + t;
    int v = 0;
    if (e < E) {
      v = counts[e];
      if (C >= 0 && v > C) v = (int)C;
      if (kept0) kept0[e] = v;
      if (ocounts) v += min(ocounts[e], (int)C - v);
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

// RANKS: write each assignment's raw stable rank (or -1 for an out-of-range id) to
// slot_pos instead of placing it (no offsets, no perm_src).
template <bool RANKS>
__global__ __launch_bounds__(256) void scatter_kernel(
    const int32_t* __restrict__ idx, int64_t NA, int E, int chunk, int64_t C,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ slot_pos) {
  __shared__ int run[kMaxExperts];
  __shared__ int wc[4][kMaxExperts];
  __shared__ int offsets[kMaxExperts + 1];
  if (!RANKS) block_offsets(counts, E, C, offsets, offsets_out);
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
      if (RANKS) {
        slot_pos[i] = r;
      } else {
        const bool keep = (C < 0) || ((int64_t)r < C);
        const int pos = offsets[e] + r;
        slot_pos[i] = keep ? pos : -1;
        if (keep) perm_src[pos] = (int32_t)i;
      }
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
  hipLaunchKernelGGL(scatter_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, idx, NA, E,
                     chunk, C, blk_base, counts, offsets, perm_src, slot_pos);
  return hipGetLastError();
}

hipError_t launch_ranks(const int32_t* idx, int64_t NA, int E, int chunk,
                        const int32_t* blk_base, int32_t* rank0, hipStream_t s) {
  const int64_t nb = ceil_div(NA, chunk);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_kernel<true>, dim3((unsigned)nb), dim3(256), 0, s, idx, NA, E,
                     chunk, (int64_t)-1, blk_base, nullptr, nullptr, nullptr, rank0);
  return hipGetLastError();
}

// Block b: assignments [b chunk, (b+1) chunk) with chunk = kDispatchChunk.
__global__ __launch_bounds__(256) void offers_kernel(const int32_t* __restrict__ rank0,
                                                     const int32_t* __restrict__ cand, int64_t NA,
                                                     int k, int E, int64_t C,
                                                     int32_t* __restrict__ offer,
                                                     int32_t* __restrict__ blk) {
  __shared__ int h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kDispatchChunk;
  for (int q = threadIdx.x; q < kDispatchChunk; q += blockDim.x) {
    const int64_t i = base + q;
    if (i >= NA) break;
    int target = -1;
    if ((int64_t)rank0[i] >= C) {   // dropped by the capacity (an invalid id has rank -1)
      const int64_t t0 = i - i % k;
      int m = 0;
      for (int64_t i2 = t0; i2 < i; ++i2) m += ((int64_t)rank0[i2] >= C) ? 1 : 0;
      const int c = cand[t0 + m];     // m < k: at most k - 1 earlier slots
      if ((unsigned)c < (unsigned)E) target = c;
    }
    offer[i] = target;
    if (target >= 0) atomicAdd(&h[target], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) blk[(int64_t)blockIdx.x * E + e] = h[e];
}

hipError_t launch_offers(const int32_t* rank0, const int32_t* cand, int64_t T, int k, int E,
                         int64_t C, int32_t* offer, int32_t* blk, hipStream_t s) {
  const int64_t NA = T * k, nb = ceil_div(NA, kDispatchChunk);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(offers_kernel, dim3((unsigned)nb), dim3(256), 0, s, rank0, cand, NA, k, E,
                     C, offer, blk);
  return hipGetLastError();
}

// Block b: assignments [b chunk, (b+1) chunk), chunk = kDispatchChunk.  slot_pos holds
// rank0 on entry.  Offers are ranked per expert in row-major order like the scatter
// (ballots on the expert bits inside a wavefront, LDS counts across wavefronts, running
// bases across rounds and blocks).
__global__ __launch_bounds__(256) void place_next_best_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ offer, int64_t NA, int E,
    int64_t C, const int32_t* __restrict__ counts, const int32_t* __restrict__ ocounts,
    const int32_t* __restrict__ offer_base, int32_t* __restrict__ offsets_out,
    int32_t* __restrict__ perm_src, int32_t* __restrict__ slot_pos) {
  __shared__ int run[kMaxExperts];
  __shared__ int wc[4][kMaxExperts];
  __shared__ int offsets[kMaxExperts + 1];
  __shared__ int kept0[kMaxExperts];
  block_offsets(counts, E, C, offsets, offsets_out, ocounts, kept0);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool has_work = (int64_t)blockIdx.x * kDispatchChunk < NA;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    run[e] = has_work ? offer_base[(int64_t)blockIdx.x * E + e] : 0;
    wc[0][e] = wc[1][e] = wc[2][e] = wc[3][e] = 0;
  }
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kDispatchChunk;
  for (int q0 = 0; q0 < kDispatchChunk; q0 += 256) {
    const int64_t i = base + q0 + threadIdx.x;
    const bool inb = i < NA;
    const int r0 = inb ? slot_pos[i] : -1;
    const int ov = inb ? offer[i] : -1;
    const bool off = ov >= 0;
    const int e = off ? ov : 0;
    uint64_t peers = __ballot(off);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t m = __ballot(on);
      peers &= on ? m : ~m;
    }
    const int lrank = __popcll(peers & below);
    if (off && lrank == 0) wc[w][e] = __popcll(peers);
    __syncthreads();
    if (inb) {
      int pos = -1;
      if (r0 >= 0 && (int64_t)r0 < C) {
        pos = offsets[idx[i]] + r0;                 // kept in round 0
      } else if (off) {
        int r = run[e] + lrank;
        for (int q = 0; q < w; ++q) r += wc[q][e];
        if ((int64_t)r < C - kept0[e]) pos = offsets[e] + kept0[e] + r;
      }
      slot_pos[i] = pos;
      if (pos >= 0) perm_src[pos] = (int32_t)i;
    }
    __syncthreads();
    for (int ee = threadIdx.x; ee < E; ee += blockDim.x) {
      run[ee] += wc[0][ee] + wc[1][ee] + wc[2][ee] + wc[3][ee];
      wc[0][ee] = wc[1][ee] = wc[2][ee] = wc[3][ee] = 0;
    }
    __syncthreads();
  }
}

hipError_t launch_place_next_best(const int32_t* idx, const int32_t* offer, int64_t NA, int E,
                                  int64_t C, const int32_t* counts, const int32_t* ocounts,
                                  const int32_t* offer_base, int32_t* offsets,
                                  int32_t* perm_src, int32_t* slot_pos, hipStream_t s) {
  const int64_t nb = NA > 0 ? ceil_div(NA, kDispatchChunk) : 1;
  hipLaunchKernelGGL(place_next_best_kernel, dim3((unsigned)nb), dim3(256), 0, s, idx, offer, NA,
                     E, C, counts, ocounts, offer_base, offsets, perm_src, slot_pos);
  return hipGetLastError();
}

}  // namespace moe
