// Grouped SwiGLU experts: for every expert (group) g the rows [row_begin_g,
// row_begin_g + M_g) of the expert-contiguous order run through
//   H = SiLU(X W_gate[g]^T) * (X W_up[g]^T)      (gate/up GEMM, fused epilogue)
//   Yp = H W_down[g]^T                             (down GEMM)
// "Chapter 30: Mixture of Experts" (LLM Transformer book), 30.2.4: w1 through SiLU,
// w3 linear, w2 back to d; "Mixture-of-experts in practice" (deepseekmodel.com),
// expert-parallel section: with the tokens of each expert contiguous, one grouped GEMM
// computes all experts of the layer at once instead of one small GEMM per expert.
//
// bf16 kernels (gfx950), persistent, over a tile table (per-group tile prefix) built on
// the device from the dispatch offsets, so skewed per-expert counts need no host round
// trip; tiles are ordered (group, n-tile, m-tile) and dealt to the XCDs in windows of
// consecutive tiles, so the m-tiles that share a weight tile run on the same L2:
//   * gemm_w8_kernel (batches in which a group can be large; bf16 or 8-bit weights): 8 waves in
//     ping-pong pairs per SIMD, 64..256-row x 256-weight-row tiles, token rows and weights
//     both staged through LDS;
//   * gemm_bf16_kernel (batches in which no group can be large: fewer tokens than the
//     small-group bound): 4 waves, 64-row streaming tiles and barrier-free skinny tiles
//     for groups of at most 32 rows;
//   * v_mfma_f32_32x32x16_bf16 accumulators; for the gate/up GEMM a wave holds the gate
//     and up blocks of the same columns, so SiLU(g)*u is formed in registers and H is
//     stored once, in bf16;
//   * the X rows of the gate/up GEMM are gathered on the fly through perm_src (the
//     permuted activations are never materialised);
//   * every tile kind walks K in the same 64-wide steps, k-slot order and rotation, so an
//     output element sums in the same order whichever tile computes it.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
// Native vector type for 16-byte global/LDS moves (HIP's uint4 struct is copied through
// memory and would keep the staging registers in scratch).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const void* A;          // gated: x [T, K]; down: H [rows, K]
  const int32_t* perm_src;
  const int32_t* offsets; // [E+1]
  const void* B0;         // gated: W_gate; down: W_down   [G, N, K]
  const void* B1;         // gated: W_up
  void* out;              // gated: H [rows, N] (dtype); down: Yp [rows, N] fp32
  int64_t shared_row0;    // T*k: first row of the shared expert
  int T, topk, E, G, N, K, n_tiles;
  int narrow_small;       // small groups take half-width tiles (gate/up 64, down 128 columns)
  int skinny_all;         // every group has at most 32 rows (static order: streamed tiles)
  int* ctr;               // NULL, or 8 per-XCD unit counters, zero at launch
  const float* sc0;       // 8-bit weights: per-row scales of B0 [G, N] (else unused)
  const float* sc1;       // 8-bit weights: per-row scales of B1 (gated)
};

// 8 e4m3 codes (bytes of lo, then hi; byte j = k-slot j) -> 8 bf16 operands.  Every e4m3
// value is exact in bf16; the per-row scale is applied to the accumulated sums.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Geometry of group g.
__device__ inline void group_rows(const GemmArgs& a, int g, int64_t& row_begin, int& M) {
  if (g < a.E) {
    row_begin = a.offsets[g];
    M = a.offsets[g + 1] - a.offsets[g];
  } else {
    row_begin = a.shared_row0;
    M = a.T;
  }
}

// Builds, in LDS, the exclusive prefix over groups of their tile counts (the tile
// table) from the dispatch offsets; tiles[G] is the total.  tile_count(M) gives a group's
// number of tiles from its row count.  Wavefront 0 scans the groups 64 at a time.  Ends
// with a barrier.
template <typename CountFn>
__device__ inline void build_tile_table(const GemmArgs& a, CountFn tile_count, int* tiles) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int run = 0;
    for (int base = 0; base < a.G; base += 64) {
      const int g = base + lane;
      int c = 0;
      if (g < a.G) c = tile_count((g < a.E) ? a.offsets[g + 1] - a.offsets[g] : a.T);
      int incl = c;
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      if (g < a.G) tiles[g] = run + incl - c;
      run += __shfl(incl, 63, 64);
    }
    if (lane == 0) tiles[a.G] = run;
  }
  __syncthreads();
}

// tile -> group: the g with tiles[g] <= tile < tiles[g + 1] (a group with tiles).
__device__ inline int find_group(const int* tiles, int G, int64_t tile) {
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tiles[mid] <= tile) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Source row (in A) of row m of group g, for m < M.
template <bool GATED>
__device__ inline int64_t a_source_row(const GemmArgs& a, int g, int64_t row_begin, int m) {
  if (!GATED) return row_begin + m;                 // H rows are already grouped
  if (g < a.E) return a.perm_src[row_begin + m] / a.topk;
  return m;                                          // shared expert: token m
}

__device__ inline float silu_f(float z) { return z / (1.0f + expf(-z)); }
// SiLU with the hardware exp2 and reciprocal (a few ulp of fp32); used where h is then
// rounded to bf16, whose step is 2^16 times coarser.
__device__ inline float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// ------------------------------------------------------------------ bf16 MFMA tiles
// Output tiles of 64 to 256 rows (256-row tiles for large groups, with the remainder in one
// tile of 64, 128, 192 or 256 rows; 64-row tiles for small groups, so small experts do not
// pay for 256-row MFMA tiles) by 128 h columns (gate/up: the gate rows of those columns
// and the matching up rows) or 256 output columns (down).
//   * K is walked in 64-wide steps; inside a step the MFMA k-slots are permuted: k16 step s,
//     lane half g uses the physical columns [32g + 8s, 32g + 8s + 8), for A and B alike;
//   * token rows are staged through LDS rows padded to 72 bf16 (LDK), so the fragment
//     reads of a wavefront hit distinct banks.
constexpr int BK = 64, LDK = BK + 8;
constexpr int BM_BIG = 256, BM_SMALL = 64;
// Row counts from which a group takes 256-row tiles (and a 64- to 256-row remainder)
// instead of 64-row tiles.  gate/up: a group of 65-128 rows runs faster as one 128-row tile
// (its weights read once) than as two 64-row tiles; the down GEMM's 64-row tiles, 256
// columns wide, stay ahead up to 80 rows.  (Measured on the Switch-shaped layer, whose groups hold 32-320 rows:
// gate/up 1.13 -> 1.07 ms, down 0.59 -> 0.56 ms against one bound of 128 rows for both.)
constexpr int SMALL_GROUP_ROWS_GATED = 65, SMALL_GROUP_ROWS_DOWN = 81;

// Tile shape of a group with M rows: 256-row tiles for large groups, 64-row tiles for
// small ones.  Columns per tile: gate/up 128 (each wave one 32-column block of gate and
// the same block of up); down 256, or 128 for small groups when the host finds the
// whole launch short of tiles (decode-sized batches, where the GEMM streams weights and
// every CU must take part).
template <bool GATED>
__device__ inline bool small_group(int M) {
  return M < (GATED ? SMALL_GROUP_ROWS_GATED : SMALL_GROUP_ROWS_DOWN);
}
// Rows of m-tile mt (tiles start at mt * B in large groups, mt * 64 in small ones): large
// groups are cut into tiles of B rows (256, or 192 for down GEMMs whose rounds that fills
// better, see down_tile_rows) and put their remainder in one tile of 64, 128, 192 or B
// rows, whichever is the smallest that holds it.
template <bool GATED>
__device__ inline int m_tile_rows(int M, int mt, int B) {
  if (small_group<GATED>(M)) return BM_SMALL;
  const int r = M - mt * B;
  return r > 192 ? B : r > 128 ? 192 : r > 64 ? 128 : 64;
}
template <bool GATED>
__device__ inline int tile_cols(bool small, int narrow_small) {
  const bool narrow = small && narrow_small;
  return GATED ? (narrow ? 64 : 128) : (narrow ? 128 : 256);
}

// Epilogue of a tile: D[m][n] of a 32x32 block sits in lane n + 32*((m/4)%2), register
// 4*(m/8) + m%4.  Gate/up: h = SiLU(g) * u -> bf16 into an LDS tile [BM][128 + 8] (the A
// stages are free: every block barrier of the K loop is behind), then 16-byte row stores.
// Down: fp32 stores of the lanes' columns.
template <int MB, int NB, bool GATED, bool FP8>
__device__ __forceinline__ void store_tile(const floatx16 (&acc)[MB][NB], bf16_t* smem,
                                           void* outp, int64_t row_begin, int M, int m0,
                                           int ncol0, int N, const int (&bcol)[NB],
                                           const float (&scl)[NB]) {
  constexpr int BMT = 32 * MB;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 31, fg = lane >> 5;
  if (GATED) {
    constexpr int HLD = 136;
    bf16_t* Ht = smem;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mb * 32 + 8 * (r >> 2) + 4 * fg + (r & 3);
        const float gv = FP8 ? acc[mb][0][r] * scl[0] : acc[mb][0][r];
        const float uv = FP8 ? acc[mb][NB - 1][r] * scl[NB - 1] : acc[mb][NB - 1][r];
        Ht[row * HLD + 32 * w + fr] = f32_to_bf16(silu_fast(gv) * uv);
      }
    __syncthreads();
    bf16_t* H = (bf16_t*)outp;
#pragma unroll 4
    for (int i = 0; i < BMT / 16; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 4, cc = (c & 15) * 8;
      const int m = m0 + row, n = ncol0 + cc;   // N % 64 == 0: n < N implies n + 8 <= N
      if (m < M && n < N)
        *reinterpret_cast<u32x4*>(H + (row_begin + m) * N + n) =
            *reinterpret_cast<const u32x4*>(Ht + row * HLD + cc);
    }
    __syncthreads();   // the next tile's prologue overwrites the LDS
  } else {
    float* Y = (float*)outp;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int n = bcol[nb];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + mb * 32 + 8 * (r >> 2) + 4 * fg + (r & 3);
          if (m < M && n < N)
            Y[(row_begin + m) * N + n] = FP8 ? acc[mb][nb][r] * scl[nb] : acc[mb][nb][r];
        }
      }
  }
}

// Per-row weight scales of the lane's NB output columns (1 for bf16 weights).
template <int NB, bool GATED, bool FP8>
__device__ __forceinline__ void load_scales(const GemmArgs& a, int g, const int (&bcol)[NB],
                                            float (&scl)[NB]) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float* sc = (GATED && nb >= NB / 2) ? a.sc1 : a.sc0;
    scl[nb] = FP8 ? sc[(int64_t)g * a.N + min(bcol[nb], a.N - 1)] : 1.0f;
  }
}

// A 64-row tile whose work is streaming its weights (small groups: decode, the tail of
// skewed or capacity-limited routing).  The weights are read with whole 128-byte row
// segments per 8 lanes (the loads coalesce into full HBM bursts) and put into MFMA order through
// a wave-private LDS buffer: two stages of [NB*32 rows][64 bf16], 16-byte chunks XOR
// swizzled (chunk c of row r at c ^ ((r/2)%8)) so both the stores and the fragment reads
// are conflict-free.  P steps of weights are in flight per wave (P register sets).
constexpr int SB_STAGE = 2 * 32 * BK;                 // bf16 per wave stage, NB <= 2
constexpr size_t SMALL_LDS_BYTES =
    (size_t)(2 * 64 * LDK + 4 * 2 * SB_STAGE) * sizeof(bf16_t);   // A stages + B buffers
// Steps of weights in flight per wave (measured on decode-sized launches: about 16 KB
// (two-block tiles) to 32 KB (one-block down tiles) per wave is best; more is slower).
constexpr int STREAM_P2 = 2, STREAM_P1 = 8;
// Tiles whose group has at most 32 rows left take the barrier-free skinny tile, with 4 K
// steps of weights and tokens in flight per wave.  (Measured on decode-sized launches: with
// each tile drained before the next one, 2 steps were best for bf16 weights; with the tiles
// of a launch streamed back to back, 4 steps take the Mixtral decode gate/up from 0.332 to
// 0.309 ms and the 8-bit one from 0.217 to 0.194 ms; 6 or 8 steps are no faster.)
constexpr int SKINNY_ROWS = 32;
constexpr int SKINNY_P = 4;
constexpr size_t KERNEL_LDS_BYTES = SMALL_LDS_BYTES;
// 8-bit weights: a K step of a row is 64 bytes, read by 4 lanes (16 rows per load); the
// wave-private stage holds [NB*32 rows][64 bytes], 16-byte chunk c of row r at position
// c ^ ((r/4)%4), and a fragment is one 8-byte read, converted to bf16 after the read.
template <int NB, bool GATED, int P, bool FP8>
__device__ __forceinline__ void gemm_bf16_tile_stream(const GemmArgs& a, bf16_t* smem, int g,
                                                      int64_t row_begin, int M, int m0,
                                                      int ncol0, int k0, int nk, int rot,
                                                      void* outp) {
  static_assert(!GATED || NB == 2, "gate/up tiles pair one gate and one up block per wave");
  static_assert(P % 2 == 0, "the step loop is unrolled by P (even: two LDS stages)");
  constexpr int MB = 2, BMT = 64, STAGE = BMT * LDK;
  constexpr int NL = FP8 ? 2 * NB : 4 * NB;     // B loads per step
  constexpr int WB = FP8 ? 1 : 2;               // bytes per weight
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const int fr = lane & 31, fg = lane >> 5;
  const bf16_t* A = (const bf16_t*)a.A + k0 * BK;
  const int K = a.K, N = a.N;
  bf16_t* Bw = smem + 2 * STAGE + w * 2 * SB_STAGE;   // this wave's two B stages

  int aoff[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = m0 + lr + 32 * i;
    aoff[i] = m < M ? m : 0;
  }
  if (GATED && g < a.E) {
#pragma unroll
    for (int i = 0; i < MB; ++i) aoff[i] = a.perm_src[row_begin + aoff[i]];
#pragma unroll
    for (int i = 0; i < MB; ++i) aoff[i] = aoff[i] / a.topk * K + lc;
  } else {
    const int base = GATED ? 0 : (int)row_begin;
#pragma unroll
    for (int i = 0; i < MB; ++i) aoff[i] = (base + aoff[i]) * K + lc;
  }
  // B load j (j < NL): block nb = j / 4, rows r = 8 (j % 4) + lane / 8 of the block, the
  // lane's 16-byte chunk c = lane % 8; stored at chunk position c ^ ((r / 2) % 8).
  const char* pbl[NL];   // byte addresses
  int bst[NL];           // byte offsets in the wave's stage
  int bcol[NB];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int nb = FP8 ? j / 2 : j / 4;
    const int r = FP8 ? 16 * (j % 2) + (lane >> 2) : 8 * (j % 4) + (lane >> 3);
    const int c = FP8 ? lane & 3 : lane & 7;
    const int n = GATED ? ncol0 + 32 * w + r : ncol0 + 32 * NB * w + 32 * nb + r;
    const char* base = (const char*)((GATED && nb == 1) ? a.B1 : a.B0);
    pbl[j] = base + (((int64_t)g * N + min(n, N - 1)) * K + k0 * BK) * WB + 16 * c;
    bst[j] = FP8 ? (nb * 32 + r) * BK + 16 * (c ^ ((r >> 2) & 3))
                 : 2 * ((nb * 32 + r) * BK + 8 * (c ^ ((r >> 1) & 7)));
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    bcol[nb] = GATED ? ncol0 + 32 * w + fr : ncol0 + 32 * NB * w + 32 * nb + fr;
  int brd[4];   // fragment read offsets: row fr of a block, k16 step s of lane half fg
#pragma unroll
  for (int s = 0; s < 4; ++s)
    brd[s] = FP8 ? fr * BK + 16 * ((2 * fg + (s >> 1)) ^ ((fr >> 2) & 3)) + 8 * (s & 1)
                 : 2 * (fr * BK + 8 * ((4 * fg + s) ^ ((fr >> 1) & 7)));

  floatx16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  u32x4 rb[P][NL];   // weights of steps in flight: set q holds step t with t % P == q
  u32x4 ra[MB];

  // Step t reads K step (t + rot) mod nk (see k_rotation).
#define MOE_KSTEP(t) ((min((t), nk - 1) + rot) - ((min((t), nk - 1) + rot) >= nk ? nk : 0))
#define MOE_SLOAD_B(q, t)                                                                  \
  _Pragma("unroll") for (int j = 0; j < NL; ++j)                                           \
    rb[q][j] = *reinterpret_cast<const u32x4*>(pbl[j] + MOE_KSTEP(t) * BK * WB);
#define MOE_SSTORE_B(q, st)                                                                \
  _Pragma("unroll") for (int j = 0; j < NL; ++j)                                           \
    *reinterpret_cast<u32x4*>((char*)Bw + (st) * SB_STAGE * 2 + bst[j]) = rb[q][j];
#define MOE_SLOAD_A(t)                                                                     \
  _Pragma("unroll") for (int i = 0; i < MB; ++i)                                           \
    ra[i] = *reinterpret_cast<const u32x4*>(A + aoff[i] + MOE_KSTEP(t) * BK);
#define MOE_SSTORE_A(st)                                                                   \
  _Pragma("unroll") for (int i = 0; i < MB; ++i)                                           \
    *reinterpret_cast<u32x4*>(smem + (st) * STAGE + (lr + 32 * i) * LDK + lc) = ra[i];
  // K step t: the weights of step t+1 go from their register set into this wave's LDS
  // stage (t+1)%2 and the set is refilled with step t+1+P; the MFMAs of step t read the
  // stages t%2; the token rows of step t+1 are stored; block barrier.  Steps t >= nk
  // (padding to a multiple of P) see zero token rows.
#define MOE_SSTEP(t, q1)                                                                   \
  {                                                                                        \
    MOE_SLOAD_A(min((t) + 1, nk - 1));                                                     \
    MOE_SSTORE_B(q1, ((t) + 1) & 1);                                                       \
    MOE_SLOAD_B(q1, (t) + 1 + P);                                                          \
    const bf16_t* As_ = smem + ((t) & 1) * STAGE;                                          \
    const bf16_t* Bs_ = Bw + ((t) & 1) * SB_STAGE;                                         \
    _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                        \
      bf16x8 af[MB], bfr[NB];                                                              \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                    \
        af[mb] = *reinterpret_cast<const bf16x8*>(As_ + (mb * 32 + fr) * LDK + 32 * fg + 8 * s); \
      _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) {                                  \
        const char* bp_ = (const char*)Bs_ + nb * 32 * BK * WB + brd[s];                   \
        if constexpr (FP8) {                                                               \
          const uint2 q_ = *reinterpret_cast<const uint2*>(bp_);                           \
          bfr[nb] = e4m3x8_to_bf16(q_.x, q_.y);                                            \
        } else {                                                                           \
          bfr[nb] = *reinterpret_cast<const bf16x8*>(bp_);                                 \
        }                                                                                  \
      }                                                                                    \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                    \
        _Pragma("unroll") for (int nb = 0; nb < NB; ++nb)                                  \
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], \
                                                                0, 0, 0);                  \
    }                                                                                      \
    if ((t) + 1 >= nk) {                                                                   \
      _Pragma("unroll") for (int i = 0; i < MB; ++i) ra[i] = u32x4{0u, 0u, 0u, 0u};        \
    }                                                                                      \
    MOE_SSTORE_A(((t) + 1) & 1);                                                           \
    __syncthreads();                                                                       \
  }

  // Prologue: weights of steps 0..P-1 requested, step 0's stored; token rows of step 0.
#pragma unroll
  for (int q = 0; q < P; ++q) MOE_SLOAD_B(q, q);
  MOE_SSTORE_B(0, 0);
  MOE_SLOAD_B(0, P);
  MOE_SLOAD_A(0);
  MOE_SSTORE_A(0);
  __syncthreads();
  const int nkp = (nk + P - 1) / P * P;
  for (int kt = 0; kt < nkp; kt += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) MOE_SSTEP(kt + u, (u + 1) % P);   // (u: the macros use j)
  }
#undef MOE_KSTEP
#undef MOE_SLOAD_B
#undef MOE_SSTORE_B
#undef MOE_SLOAD_A
#undef MOE_SSTORE_A
#undef MOE_SSTEP
  float scl[NB];
  load_scales<NB, GATED, FP8>(a, g, bcol, scl);
  store_tile<MB, NB, GATED, FP8>(acc, smem, outp, row_begin, M, m0, ncol0, N, bcol, scl);
}

// Coordinates of one tile of the table: group, its rows, the tile's first row and column,
// and its K rotation.
struct TileAt {
  int g, M, m0, ncol0, rot;
  int64_t row_begin;
};

// One tile, as a sequence of length one for gemm_skinny_stream.
struct OneTile {
  TileAt t;
  __device__ bool get(int r, TileAt& out) const {
    out = t;
    return r == 0;
  }
};

// Tiles of at most 32 rows (decode-sized groups): every wave computes all of the tile's rows
// against its own weight rows and reads its token fragments straight from global memory (the
// few rows are L1/L2 hits), so the K loop has no block barrier and no LDS traffic for the
// tokens.  The weights stream as in gemm_bf16_tile_stream (whole row segments per load,
// through the wave's swizzled LDS stages); P steps of weights and tokens are in flight.
//
// The block walks a sequence of such tiles (units.get(r, tile) for r = 0, 1, ... while it
// returns true) as one stream: the loads of a tile's last P steps are those of the next
// tile's first P steps, so the pipeline does not drain between tiles and each tile's
// epilogue overlaps the next tile's first loads.  (Each tile takes nkp = nk rounded up to P
// steps; steps past nk multiply zero token fragments.)  The epilogue's LDS transpose sits
// past the four waves' weight stages, which hold the next tile's first step meanwhile.
//
// Gate/up with NB == 1 (64-column tiles, for launches whose tiles would leave much of a
// last round idle): the wave's 32 weight rows are 16 gate rows and the 16 matching up rows
// and the MFMA is taken transposed (D[weight row][token]), so a lane holds gate and up of
// one (token, h) in registers r and r + 8.
template <int NB, bool GATED, int P, bool FP8, typename Units>
__device__ __forceinline__ void gemm_skinny_stream(const GemmArgs& a, bf16_t* smem,
                                                   const Units& units) {
  constexpr bool PAIRED = GATED && NB == 1;
  static_assert(P % 2 == 0, "the step loop is unrolled by P (even: two LDS stages)");
  constexpr int MB = 1;
  constexpr int NL = FP8 ? 2 * NB : 4 * NB;     // B loads per step
  constexpr int WB = FP8 ? 1 : 2;               // bytes per weight
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int fr = lane & 31, fg = lane >> 5;
  const bf16_t* A = (const bf16_t*)a.A;
  const int K = a.K, N = a.N, nk = K / BK, nkp = (nk + P - 1) / P * P;
  bf16_t* Bw = smem + w * 2 * SB_STAGE;          // this wave's two B stages
  bf16_t* Ht = smem + 4 * 2 * SB_STAGE;          // epilogue transpose, past every wave's stages

  // Per-tile addressing: the lane's token row (row fr of the tile; rows past M read row 0
  // of the group, their results are never stored; lane half fg reads k 32 fg .. 32 fg + 31)
  // and its weight row segments.
  struct Addr {
    const char* pbl[NL];
    int aoff, rot;
  };
  auto addr_of = [&](const TileAt& u, Addr& ad) {
    const int m = u.m0 + fr < u.M ? u.m0 + fr : 0;
    if (GATED && u.g < a.E) ad.aoff = a.perm_src[u.row_begin + m] / a.topk * K;
    else ad.aoff = ((GATED ? 0 : (int)u.row_begin) + m) * K;
    ad.aoff += 32 * fg;
    ad.rot = u.rot;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int nb = FP8 ? j / 2 : j / 4;
      const int r = FP8 ? 16 * (j % 2) + (lane >> 2) : 8 * (j % 4) + (lane >> 3);
      const int c = FP8 ? lane & 3 : lane & 7;
      const int n = PAIRED  ? u.ncol0 + 16 * w + (r & 15)
                    : GATED ? u.ncol0 + 32 * w + r
                            : u.ncol0 + 32 * NB * w + 32 * nb + r;
      const char* base = (const char*)((PAIRED ? r >= 16 : (GATED && nb == 1)) ? a.B1 : a.B0);
      ad.pbl[j] = base + (((int64_t)u.g * N + min(n, N - 1)) * K) * WB + 16 * c;
    }
  };
  int bst[NL];   // byte offset of each B load in the wave's stage
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int r = FP8 ? 16 * (j % 2) + (lane >> 2) : 8 * (j % 4) + (lane >> 3);
    const int c = FP8 ? lane & 3 : lane & 7;
    const int nb = FP8 ? j / 2 : j / 4;
    bst[j] = FP8 ? (nb * 32 + r) * BK + 16 * (c ^ ((r >> 2) & 3))
                 : 2 * ((nb * 32 + r) * BK + 8 * (c ^ ((r >> 1) & 7)));
  }
  int brd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    brd[s] = FP8 ? fr * BK + 16 * ((2 * fg + (s >> 1)) ^ ((fr >> 2) & 3)) + 8 * (s & 1)
                 : 2 * (fr * BK + 8 * ((4 * fg + s) ^ ((fr >> 1) & 7)));

  floatx16 acc[MB][NB];
  u32x4 rb[P][NL];       // weights of steps in flight: set q holds step t with t % P == q
  bf16x8 ra[P][4];       // token fragments of the same steps (k16 steps 0..3)

  // Tile step t reads K step (t + rot) mod nk (see k_rotation); steps past nk are clamped.
#define MOE_KROT(ad, t) ((min((t), nk - 1) + (ad).rot) - ((min((t), nk - 1) + (ad).rot) >= nk ? nk : 0))
#define MOE_KLOAD(q, ad, t)                                                                \
  {                                                                                        \
    const int ks_ = MOE_KROT(ad, t);                                                       \
    _Pragma("unroll") for (int j = 0; j < NL; ++j)                                         \
      rb[q][j] = *reinterpret_cast<const u32x4*>((ad).pbl[j] + ks_ * BK * WB);             \
    _Pragma("unroll") for (int s = 0; s < 4; ++s)                                          \
      ra[q][s] = *reinterpret_cast<const bf16x8*>(A + (ad).aoff + ks_ * BK + 8 * s);       \
  }
#define MOE_KSTORE_B(q, st)                                                                \
  _Pragma("unroll") for (int j = 0; j < NL; ++j)                                           \
    *reinterpret_cast<u32x4*>((char*)Bw + (st) * SB_STAGE * 2 + bst[j]) = rb[q][j];
  // Tile step t (weights in stage t % 2, tokens in set t % P): the weights of step t+1 go
  // from their registers into the other stage, and the set is refilled with step lt of the
  // tile whose addresses are ad (step t+P of this tile, or step t+P-nkp of the next).
  // Steps t >= nk multiply zero token fragments.
#define MOE_KSTEP_BODY(t, q0, q1, ad, lt)                                                  \
  {                                                                                        \
    MOE_KSTORE_B(q1, ((t) + 1) & 1);                                                       \
    const char* Bs_ = (const char*)Bw + ((t) & 1) * SB_STAGE * 2;                          \
    const bool live_ = (t) < nk;                                                           \
    _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                        \
      const bf16x8 af_ = live_ ? ra[q0][s] : bf16x8{};                                     \
      _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) {                                  \
        const char* bp_ = Bs_ + nb * 32 * BK * WB + brd[s];                                \
        bf16x8 bfr_;                                                                       \
        if constexpr (FP8) {                                                               \
          const uint2 q_ = *reinterpret_cast<const uint2*>(bp_);                           \
          bfr_ = e4m3x8_to_bf16(q_.x, q_.y);                                               \
        } else {                                                                           \
          bfr_ = *reinterpret_cast<const bf16x8*>(bp_);                                    \
        }                                                                                  \
        if constexpr (PAIRED)                                                              \
          acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr_, af_, acc[0][nb], 0, 0, \
                                                               0);                         \
        else                                                                               \
          acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af_, bfr_, acc[0][nb], 0, 0, \
                                                               0);                         \
      }                                                                                    \
    }                                                                                      \
    MOE_KLOAD(q0, ad, lt);                                                                 \
  }

  TileAt cur;
  if (!units.get(0, cur)) return;
  Addr ac;
  addr_of(cur, ac);
  // Prologue: steps 0..P-1 of the first tile requested; step 0's weights stored.
#pragma unroll
  for (int q = 0; q < P; ++q) MOE_KLOAD(q, ac, q);
  MOE_KSTORE_B(0, 0);
  for (int r = 0;; ++r) {
    TileAt nxt;
    const bool more = units.get(r + 1, nxt);
    Addr an;
    if (more) addr_of(nxt, an);
    else an = ac;   // past the last tile: this tile's last step again (in bounds, unused)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[0][j][v] = 0.0f;
    for (int kt = 0; kt < nkp - P; kt += P) {
#pragma unroll
      for (int u = 0; u < P; ++u) MOE_KSTEP_BODY(kt + u, u, (u + 1) % P, ac, kt + u + P);
    }
    // the last P steps request the next tile's first P steps (set u holds its step u)
#pragma unroll
    for (int u = 0; u < P; ++u)
      MOE_KSTEP_BODY(nkp - P + u, u, (u + 1) % P, an, more ? u : nk - 1);
    // epilogue of this tile
    if constexpr (PAIRED) {
      // acc[0][0][r] (r < 8): gate row 8(r/4) + 4 fg + r%4 of the wave's 16, token fr;
      // r + 8: the matching up row.  h -> bf16 into an LDS tile [32][64 + 8], then 16-byte
      // row stores (one per thread).
      constexpr int HLD = 72;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        uint32_t pk[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r0 = 4 * q + 2 * i;
          float gv[2], uv[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            gv[e] = acc[0][0][r0 + e];
            uv[e] = acc[0][0][r0 + e + 8];
            if constexpr (FP8) {
              const int64_t hrow =
                  (int64_t)cur.g * N + min(cur.ncol0 + 16 * w + 8 * q + 4 * fg + 2 * i + e, N - 1);
              gv[e] *= a.sc0[hrow];
              uv[e] *= a.sc1[hrow];
            }
          }
          pk[i] = (uint32_t)f32_to_bf16(silu_fast(gv[0]) * uv[0]) |
                  ((uint32_t)f32_to_bf16(silu_fast(gv[1]) * uv[1]) << 16);
        }
        *reinterpret_cast<uint2*>(Ht + fr * HLD + 16 * w + 8 * q + 4 * fg) =
            make_uint2(pk[0], pk[1]);
      }
      __syncthreads();
      bf16_t* Hout = (bf16_t*)a.out;
      const int tid = threadIdx.x, row = tid >> 3, cc = (tid & 7) * 8;
      const int m = cur.m0 + row, n = cur.ncol0 + cc;   // N % 64 == 0: n < N => n + 8 <= N
      if (m < cur.M && n < N)
        *reinterpret_cast<u32x4*>(Hout + (cur.row_begin + m) * N + n) =
            *reinterpret_cast<const u32x4*>(Ht + row * HLD + cc);
      __syncthreads();   // the next tile's epilogue rewrites the transpose
    } else {
      int bcol[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        bcol[nb] = GATED ? cur.ncol0 + 32 * w + fr : cur.ncol0 + 32 * NB * w + 32 * nb + fr;
      float scl[NB];
      load_scales<NB, GATED, FP8>(a, cur.g, bcol, scl);
      store_tile<MB, NB, GATED, FP8>(acc, Ht, a.out, cur.row_begin, cur.M, cur.m0, cur.ncol0, N,
                                     bcol, scl);
    }
    if (!more) break;
    cur = nxt;
    ac = an;
  }
#undef MOE_KROT
#undef MOE_KLOAD
#undef MOE_KSTORE_B
#undef MOE_KSTEP_BODY
}

// First K step of a tile: tiles running at the same time start at different K offsets, so
// their weight streams spread over the HBM channels instead of all reading the same column
// range of rows at a common stride.  A function of the expert and the output columns only
// (in units of the large tiles' width, whatever the tile kind), so the summation order of
// an output element does not depend on the rest of the batch.  Blocks of W8_NBLOCK
// consecutive large-tile column blocks share a start: the 8-wave kernel runs such a block's
// n-tiles of the same m-tiles together (8 m-tiles x 4 n-tiles per XCD window), and with a
// common K position they read each token-row chunk from L2 once for the block (prefill
// 2.86 -> 2.83 ms, fine-grained 7.46 -> 7.34 ms, Switch 1.75 -> 1.73 ms, decode 0.484 ->
// 0.480 ms against a start per column block).
constexpr int W8_NBLOCK = 4;
template <bool GATED>
__device__ inline int k_rotation(int g, int ncol0, int nk) {
  const unsigned cb = (unsigned)ncol0 / (GATED ? 128u : 256u);
  return (int)((cb / W8_NBLOCK + 13u * (unsigned)g) % (unsigned)nk);
}

// The tiles of a launch in which every group fits a skinny tile (at most 32 rows): the
// block's units first, first + stride, ... of the static order, below total.
template <bool GATED>
struct StaticSkinnyTiles {
  const GemmArgs* a;
  const int* tiles;
  int64_t first, stride, total;
  __device__ bool get(int r, TileAt& t) const {
    const int64_t tile = first + (int64_t)r * stride;
    if (tile >= total) return false;
    t.g = find_group(tiles, a->G, tile);
    group_rows(*a, t.g, t.row_begin, t.M);
    const int mt_g = (t.M + BM_SMALL - 1) / BM_SMALL;
    const int local = (int)(tile - tiles[t.g]);       // ordered (n-tile, m-tile)
    t.m0 = (local % mt_g) * BM_SMALL;
    t.ncol0 = (local / mt_g) * tile_cols<GATED>(true, a->narrow_small);
    t.rot = k_rotation<GATED>(t.g, t.ncol0, a->K / BK);
    return true;
  }
};

// One tile of gemm_bf16_kernel's table: a 64-row tile (the kernel runs batches in which
// no group is large, every group as 64-row tiles), streaming or skinny.
template <bool GATED, bool FP8>
__device__ __forceinline__ void gemm_bf16_unit(const GemmArgs& a, bf16_t* smem,
                                               const int* tiles, int64_t tile) {
  const int nk = a.K / BK;
  const int g = find_group(tiles, a.G, tile);
  int64_t row_begin;
  int M;
  group_rows(a, g, row_begin, M);
  const int narrow = a.narrow_small;
  const int mt_g = (M + BM_SMALL - 1) / BM_SMALL;
  const int local = (int)(tile - tiles[g]);          // ordered (n-tile, m-tile)
  const int mt = local % mt_g;
  const int ncol0 = (local / mt_g) * tile_cols<GATED>(true, narrow);
  const int rot = k_rotation<GATED>(g, ncol0, nk);
  if (M - mt * BM_SMALL <= SKINNY_ROWS) {
    // (gate/up takes 64-column tiles only when every group fits a skinny tile)
    const OneTile one{TileAt{g, M, mt * BM_SMALL, ncol0, rot, row_begin}};
    if (!narrow)
      gemm_skinny_stream<2, GATED, SKINNY_P, FP8>(a, smem, one);
    else
      gemm_skinny_stream<1, GATED, SKINNY_P, FP8>(a, smem, one);
  }
  else if (GATED || !narrow)
    gemm_bf16_tile_stream<2, GATED, STREAM_P2, FP8>(a, smem, g, row_begin, M, mt * BM_SMALL, ncol0,
                                               0, nk, rot, a.out);
  else if constexpr (!GATED)
    gemm_bf16_tile_stream<1, GATED, STREAM_P1, FP8>(a, smem, g, row_begin, M, mt * BM_SMALL, ncol0,
                                               0, nk, rot, a.out);
}

// Persistent kernel for batches in which no group is large (fewer tokens than the
// small-group bound): every group as 64-row tiles, in table order (group, n-tile, m-tile),
// dealt to the 8 XCDs (blocks are dispatched to XCDs round-robin) in windows of 32
// consecutive units, so that the m-tiles sharing a weight tile run at the same time on one
// L2.  Without counters block b takes unit 32 (8 r + b % 8) + b / 8 of round r (grid of
// 256).  With counters (a.ctr, 8 ints, zero at launch) each block takes its XCD's next unit
// when it is free, and an XCD that runs out helps the others.
template <bool GATED, bool FP8>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmArgs a) {
  extern __shared__ __align__(16) bf16_t smem[];
  __shared__ int tiles[kMaxExperts + 2];
  __shared__ long long next_unit;
  const int N = a.N, bn = tile_cols<GATED>(true, a.narrow_small);
  build_tile_table(a, [N, bn](int M) {
    return ((M + BM_SMALL - 1) / BM_SMALL) * ((N + bn - 1) / bn);
  }, tiles);   // ends with a barrier
  const int64_t total = tiles[a.G];
  const int x = blockIdx.x & 7;
  if (a.ctr == nullptr) {
    const int per = gridDim.x >> 3;
    const int64_t first = (int64_t)x * per + (blockIdx.x >> 3);
    if (a.skinny_all) {
      // every tile is a skinny one: the block streams its units without draining
      const StaticSkinnyTiles<GATED> units{&a, tiles, first, gridDim.x, total};
      if (a.narrow_small)
        gemm_skinny_stream<1, GATED, SKINNY_P, FP8>(a, smem, units);
      else
        gemm_skinny_stream<2, GATED, SKINNY_P, FP8>(a, smem, units);
      return;
    }
    for (int64_t unit = first; unit < total; unit += gridDim.x)
      gemm_bf16_unit<GATED, FP8>(a, smem, tiles, unit);
    return;
  }
  for (;;) {
    if (threadIdx.x == 0) {
      // XCD xr's c-th unit: the units are dealt out to the XCDs in windows of W
      // consecutive ones, round-robin (the static order's windows); an XCD whose windows
      // are used up takes the next XCD's in turn.
      constexpr int W = 32;
      long long u = -1;
      for (int r = 0; r < 8 && u < 0; ++r) {
        const int xr = (x + r) & 7;
        const int c = atomicAdd(&a.ctr[xr], 1);
        const int64_t cand = ((int64_t)(c / W) * 8 + xr) * W + c % W;
        if (cand < total) u = cand;
      }
      next_unit = u;
    }
    __syncthreads();
    const int64_t unit = next_unit;
    __syncthreads();   // read by all before thread 0 writes the next one
    if (unit < 0) break;
    gemm_bf16_unit<GATED, FP8>(a, smem, tiles, unit);
  }
}

// ------------------------------------------------------------------ 8-wave bf16 kernel
// Every tile of a bf16 GEMM whose batch can hold a large group: 256-row tiles with a
// 64/128/192/256-row remainder tile for large groups, 64-row tiles for small ones (as in
// gemm_bf16_kernel).  Eight waves, two per SIMD, both operands staged through LDS, and
// the two waves of a SIMD in ping-pong: group 0 (waves 0-3) and group 1 (waves 4-7, one
// phase behind) alternate between a memory phase (the fragment reads of half a K step and
// the LDS stores of half the staged data) and a compute phase (that half step's MFMAs, with
// the global loads of half of the step two ahead issued between them), each phase ending
// in a block barrier, so one wave of every SIMD issues MFMAs while the other waits on LDS.
// (Measured on the Mixtral prefill layer: gate/up 1.81 -> 1.69 ms, down 1.07 -> 0.99 ms
// against the 4-wave tiles; with both waves of a SIMD in the same phase it is no faster.)
//
// A tile is 64*MH rows x 128*NB weight rows.  Gate/up (NB = 2): the 128 gate rows of the
// tile's 128 output columns and the matching 128 up rows; wave (wm, wn) = (w / 4, w % 4)
// takes rows [32 MH wm, 32 MH (wm + 1)) against gate rows 32 wn .. 32 wn + 31 and the same
// up rows, so SiLU(g) * u is formed in registers.  Down: output columns 32 NB wn ..
// 32 NB wn + 32 NB - 1 of the tile (NB = 1: a 128-column half, see gemm_w8_kernel).
// The K steps, the k-slot permutation and the K rotation are those of the 4-wave tiles, so
// every output element sums in the same order whichever kernel computes it.
// 8-bit weights: the stage holds the weight rows as their e4m3 codes (64 bytes per row and
// K step, 16-byte chunk c of row r at position c ^ ((r / 4) % 4)), widened to bf16 after the
// fragment read; the per-row scales are applied to the sums in the epilogue.
constexpr int W8_A_BYTES = BM_BIG * LDK * 2;                      // token rows of a stage
constexpr int W8_STAGE_BF16 = 2 * W8_A_BYTES;                     // + 256 weight rows, bf16
constexpr int W8_STAGE_FP8 = W8_A_BYTES + BM_BIG * BK;            // + 256 rows of codes
constexpr size_t W8_LDS_BYTES = 2 * W8_STAGE_BF16;                // 147456

// Row height of the down GEMM's large tiles, 256 or 192, chosen per launch from the
// dispatch offsets (every block computes the same value).  Estimated time of a launch:
// rounds x mean unit cost, where a unit of r rows costs 31 + r (the 256-row tile's K loop
// took 1/0.777 of the 192-row one's per launch on the Mixtral-shaped prefill layer) and
// the rounds n / grid are rounded up to the next half (the last round's column halves,
// dynamic order) or whole.  Few rounds: the quantisation decides (Mixtral-shaped prefill,
// 576 units = 2.25 rounds of 256-row tiles against 768 = 3 of 192-row ones: down 0.946 ->
// 0.882 ms; Switch-shaped 0.524 -> 0.515); many rounds: the padded work decides
// (fine-grained layer: 256, where 192 ran 3.5% slower).  The summation order does not
// depend on the tile shape, so neither do the results.  Wave 0; ends with a barrier.
__device__ inline int down_tile_rows(const GemmArgs& a, const int* offs, bool halves,
                                     int* out) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int64_t NT = (a.N + 255) / 256;
    long long n[2] = {0, 0}, w[2] = {0, 0};
    for (int base = 0; base < a.G; base += 64) {
      const int g = base + lane;
      const int M = g < a.G ? (g < a.E ? offs[g + 1] - offs[g] : a.T) : 0;
      if (M > 0) {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const int B = v == 0 ? 256 : 192;
          if (small_group<false>(M)) {
            const int mt = (M + BM_SMALL - 1) / BM_SMALL;
            n[v] += mt * NT;
            w[v] += mt * NT * (31 + BM_SMALL);
          } else {
            const int mt = (M + B - 1) / B;
            n[v] += mt * NT;
            w[v] += NT * ((mt - 1) * (31 + B) + 31 + m_tile_rows<false>(M, mt - 1, B));
          }
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 2; ++v)
      for (int o = 32; o > 0; o >>= 1) {
        n[v] += __shfl_xor(n[v], o, 64);
        w[v] += __shfl_xor(w[v], o, 64);
      }
    if (lane == 0) {
      double est[2];
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        if (n[v] == 0) {
          est[v] = 0.0;
          continue;
        }
        const double R = (double)n[v] / (double)gridDim.x, fl = floor(R), fr = R - fl;
        const double rounds = fr == 0.0 ? fl : (halves && fr <= 0.5) ? fl + 0.5 : fl + 1.0;
        est[v] = rounds * (double)w[v] / (double)n[v];
      }
      *out = est[1] < 0.98 * est[0] ? 192 : 256;
    }
  }
  __syncthreads();
  return *out;
}

// The next unit of a block that claims its units through the per-XCD counters: the
// counter of the block's own XCD is bumped when a tile's K loop ends, and the claim is
// resolved (falling back to the other XCDs' counters once its own are spent) and
// published in LDS after the tile's epilogue, so the atomic's round trip overlaps the
// epilogue while the unit still goes to a block that is about to be free.  (Claimed when
// the tile starts instead, a block holds its next unit a whole tile ahead: prefill down
// 0.93 -> 0.99 ms, the last rounds lose their balance.)
struct W8Claim {
  long long* slot;   // LDS; nullptr: static order
  int x;             // the block's XCD
  int64_t total;     // units in the launch
};
constexpr int W8_WINDOW = 32;   // consecutive units dealt to one XCD
__device__ inline long long w8_resolve_claim(const GemmArgs& a, const W8Claim& c, int first) {
  int v = first;
  for (int r = 0; r < 8; ++r) {
    const int xr = (c.x + r) & 7;
    if (r > 0) v = atomicAdd(&a.ctr[xr], 1);
    const int64_t cand = ((int64_t)(v / W8_WINDOW) * 8 + xr) * W8_WINDOW + v % W8_WINDOW;
    if (cand < c.total) return cand;
  }
  return -1;
}

template <int MH, int NB, bool GATED, bool FP8>
__device__ __forceinline__ void w8_tile(const GemmArgs& a, bf16_t* smem, int g,
                                        int64_t row_begin, int M, int m0, int ncol0, int nk,
                                        int rot, const W8Claim& claim) {
  static_assert(!GATED || NB == 2, "gate/up tiles pair the gate and up blocks in a wave");
  constexpr int STAGE = FP8 ? W8_STAGE_FP8 : W8_STAGE_BF16;      // bytes
  constexpr int NBL = FP8 ? NB : 2 * NB;   // 16-byte weight chunks per thread and step
  constexpr int NCH = MH + NBL;            // 16-byte chunks staged per thread and step
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int lr = tid >> 3, lc = (tid & 7) * 8;       // token loads: rows lr + 64 i, k lc
  const int fr = lane & 31, fg = lane >> 5;
  const bf16_t* A = (const bf16_t*)a.A;
  char* sm = (char*)smem;
  const int K = a.K, N = a.N;

  // Token rows (element offsets; the host bounds T*d and rows*F below 2^31).
  int aoff[MH];
#pragma unroll
  for (int i = 0; i < MH; ++i) {
    const int m = m0 + lr + 64 * i;
    aoff[i] = m < M ? m : 0;
  }
  // Routed gate/up rows: the slot indices are loaded here and turned into token-row
  // offsets in the prologue, after the weight rows of step 0 are requested (those do not
  // depend on them), so the two round trips overlap.
  const bool gathered = GATED && g < a.E;
  if (gathered) {
#pragma unroll
    for (int i = 0; i < MH; ++i) aoff[i] = a.perm_src[row_begin + aoff[i]];
  } else {
    const int base = GATED ? 0 : (int)row_begin;     // shared expert: token m; down: row
#pragma unroll
    for (int i = 0; i < MH; ++i) aoff[i] = (base + aoff[i]) * K + lc;
  }
  // Weight chunks: this expert's matrices (wave-uniform) + 32-bit byte offsets (N K < 2^31).
  // bf16: chunk i is row lr + 64 i at k lc (gate/up: i = 0, 1 gate rows, 2, 3 the matching
  // up rows); 8-bit: row tid / 4 + 128 i, 16-byte chunk tid % 4 (gate/up: i = 0 gate, 1 up).
  typedef typename std::conditional<FP8, uint8_t, bf16_t>::type WT;
  const WT* Bm[2] = {(const WT*)a.B0 + (int64_t)g * N * K,
                     (const WT*)(GATED ? a.B1 : a.B0) + (int64_t)g * N * K};
  int boff[NBL], bst[NBL];   // element offsets in the matrix, byte offsets in a stage
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    const int j = FP8 ? (tid >> 2) + 128 * i : lr + 64 * i;
    const int n = GATED ? ncol0 + (j & 127) : ncol0 + j;
    boff[i] = min(n, N - 1) * K + (FP8 ? 16 * (tid & 3) : lc);
    bst[i] = FP8 ? W8_A_BYTES + j * BK + 16 * ((tid & 3) ^ ((j >> 2) & 3))
                 : W8_A_BYTES + (j * LDK + lc) * 2;
  }
  // Fragment reads: token rows (bf16 offsets of row 32 MH wm + fr, lane half fg), weight
  // rows (byte offsets of the nb-th 32-row block, row fr; 8-bit: per k16 step pair).
  const int ard = (32 * MH * wm + fr) * LDK + 32 * fg;
  int brd[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int R = (GATED ? 128 * nb + 32 * wn : 32 * NB * wn + 32 * nb) + fr;
    brd[nb] = FP8 ? W8_A_BYTES + R * BK : W8_A_BYTES + (R * LDK + 32 * fg) * 2;
  }
  const int bx0 = 16 * ((2 * fg) ^ ((fr >> 2) & 3)), bx1 = 16 * ((2 * fg + 1) ^ ((fr >> 2) & 3));

  floatx16 acc[MH][NB];
#pragma unroll
  for (int i = 0; i < MH; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  // Register sets of staged chunks (i < MH token rows, then weight rows): set q holds step
  // t with t % PF == q, PF steps ahead of the MFMAs; more for the smaller tiles, whose work
  // per step is smaller against the same load latency and which have the registers (Switch
  // layer gate/up 1.00 -> 0.97 ms, its 8-bit variant 0.78 -> 0.76 ms and down 0.44 -> 0.42
  // ms, against one set for every tile; deeper sets for the 64- and 128-row tiles, 6 and 4,
  // were no faster).
  constexpr int PF = MH == 1 ? 4 : MH == 2 ? 3 : MH == 3 ? 2 : 1;
  u32x4 st[PF][NCH];

  // Step t reads K step (t + rot) mod nk (see k_rotation); loads past the last step are
  // clamped to it (in bounds, never used).
#define W8_KSTEP(t) ((min((t), nk - 1) + rot) - ((min((t), nk - 1) + rot) >= nk ? nk : 0))
#define W8_LOAD_CHUNK(q, i, t)                                                             \
  {                                                                                        \
    const int ks_ = W8_KSTEP(t);                                                           \
    if ((i) < MH)                                                                          \
      st[q][i] = *reinterpret_cast<const u32x4*>(A + aoff[(i) < MH ? (i) : 0] + ks_ * BK); \
    else                                                                                   \
      st[q][i] = *reinterpret_cast<const u32x4*>(                                          \
          Bm[(i) >= MH + NBL / 2 ? 1 : 0] + boff[(i) >= MH ? (i) - MH : 0] + ks_ * BK);    \
  }
#define W8_STORE_CHUNK(q, i, s)                                                            \
  {                                                                                        \
    const int o_ = (i) < MH ? ((lr + 64 * (i)) * LDK + lc) * 2 : bst[(i) >= MH ? (i) - MH : 0]; \
    *reinterpret_cast<u32x4*>(sm + (s) * STAGE + o_) = st[q][i];                           \
  }
#define W8_READ(af, bf, s0, s)                                                             \
  {                                                                                        \
    const bf16_t* SA_ = (const bf16_t*)(sm + (s0) * STAGE);                                \
    _Pragma("unroll") for (int mb = 0; mb < MH; ++mb)                                      \
      af[mb] = *reinterpret_cast<const bf16x8*>(SA_ + ard + mb * 32 * LDK + 8 * (s));      \
    _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) {                                    \
      if constexpr (FP8) {                                                                 \
        const uint2 q_ = *reinterpret_cast<const uint2*>(                                  \
            sm + (s0) * STAGE + brd[nb] + ((s) >> 1 ? bx1 : bx0) + 8 * ((s) & 1));         \
        bf[nb] = e4m3x8_to_bf16(q_.x, q_.y);                                               \
      } else {                                                                             \
        bf[nb] = *reinterpret_cast<const bf16x8*>(sm + (s0) * STAGE + brd[nb] + 16 * (s)); \
      }                                                                                    \
    }                                                                                      \
  }
#define W8_MFMA(af, bf)                                                                    \
  _Pragma("unroll") for (int mb = 0; mb < MH; ++mb)                                        \
    _Pragma("unroll") for (int nb = 0; nb < NB; ++nb)                                      \
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bf[nb], acc[mb][nb], 0, 0, 0);

  // Prologue: step 0 in stage 0, steps 1 .. PF in the register sets.
  if constexpr (GATED) {
#pragma unroll
    for (int i = MH; i < NCH; ++i) W8_LOAD_CHUNK(0, i, 0);   // weight rows of step 0
    __builtin_amdgcn_sched_barrier(0);
    if (gathered) {
#pragma unroll
      for (int i = 0; i < MH; ++i) aoff[i] = aoff[i] / a.topk * K + lc;
    }
#pragma unroll
    for (int i = 0; i < MH; ++i) W8_LOAD_CHUNK(0, i, 0);      // token rows of step 0
  } else {
#pragma unroll
    for (int i = 0; i < NCH; ++i) W8_LOAD_CHUNK(0, i, 0);
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) W8_STORE_CHUNK(0, i, 0);
  // Steps 1 .. PF in the loop's own order (gate/up: pinned by scheduling barriers): the
  // vector-memory counter retires loads in issue order, and the counts the compiler waits
  // for at the top of the K loop must also hold on entry, or every step waits for loads
  // issued one phase earlier.  (The down GEMM is left as it was: its 256-row loop already
  // waits exactly, and with the pinning and the loop shape below, for all of its tiles or
  // only the 64-192-row ones, the prefill down GEMM ran 1-3% slower.)
  if constexpr (GATED) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 1; q <= PF; ++q)
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      W8_LOAD_CHUNK(q % PF, i, q);
      if constexpr (GATED) __builtin_amdgcn_sched_barrier(0);
    }
  __syncthreads();
  if (wm == 1) __syncthreads();   // group 1 runs one phase behind
  // One K step t (u = t % PF, unrolled, names the register sets).  Stage t & 1 holds step
  // t.  Half step h: the memory phase reads its two k16 steps and stores chunks
  // [NCH h / 2, NCH (h + 1) / 2) of step t+1 from set q1 into the other stage, last read
  // during step t-1 by both groups; the compute phase runs the MFMAs and reloads those
  // chunks of set q1 with step t+1+PF.
#define W8_STEP(u, t)                                                                      \
  {                                                                                        \
    const int q1 = ((u) + 1) % PF;   /* the set holding step t+1 */                       \
    _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                        \
      bf16x8 af[2][MH], bfr[2][NB];                                                        \
      W8_READ(af[0], bfr[0], (t) & 1, 2 * h);                                              \
      W8_READ(af[1], bfr[1], (t) & 1, 2 * h + 1);                                          \
      _Pragma("unroll") for (int i = NCH * h / 2; i < NCH * (h + 1) / 2; ++i)              \
        W8_STORE_CHUNK(q1, i, ((t) + 1) & 1);                                              \
      __builtin_amdgcn_sched_barrier(0);                                                   \
      __syncthreads();                                                                     \
      W8_MFMA(af[0], bfr[0]);                                                              \
      _Pragma("unroll") for (int i = NCH * h / 2; i < NCH * (h + 1) / 2; ++i)              \
        W8_LOAD_CHUNK(q1, i, (t) + 1 + PF);                                                \
      W8_MFMA(af[1], bfr[1]);                                                              \
      __builtin_amdgcn_sched_barrier(0);                                                   \
      __syncthreads();                                                                     \
    }                                                                                      \
  }
  if constexpr (GATED) {
    // Whole groups of PF steps in the loop, the last nk % PF after it: a loop body left
    // early joins the loop head with a partial group's loads in flight, and the compiler
    // then waits at every step as if the last-issued set came first.
    int t0 = 0;
    for (; t0 + PF <= nk; t0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) W8_STEP(u, t0 + u);
    }
#pragma unroll
    for (int u = 0; u + 1 < PF; ++u)
      if (t0 + u < nk) W8_STEP(u, t0 + u);   // uniform: every wave takes the same steps
  } else {
    for (int t0 = 0; t0 < nk; t0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int t = t0 + u;
        if (t >= nk) break;   // uniform: every wave takes the same steps
        W8_STEP(u, t);
      }
    }
  }
#undef W8_STEP
  if (wm == 0) __syncthreads();   // the groups' barrier counts match again
  int claimed = 0;
  if (claim.slot != nullptr && tid == 0) claimed = atomicAdd(&a.ctr[claim.x], 1);
#undef W8_KSTEP
#undef W8_LOAD_CHUNK
#undef W8_STORE_CHUNK
#undef W8_READ
#undef W8_MFMA

  if constexpr (GATED) {
    // h = SiLU(g) * u -> bf16 through an LDS tile [64 MH][128 + 8] (the stages are free:
    // the last phase ended with a barrier), then 16-byte row stores.
    float sg = 1.0f, su = 1.0f;
    if constexpr (FP8) {
      const int n = min(ncol0 + 32 * wn + fr, N - 1);
      sg = a.sc0[(int64_t)g * N + n];
      su = a.sc1[(int64_t)g * N + n];
    }
    constexpr int HLD = 136;
    bf16_t* Ht = smem;
#pragma unroll
    for (int mb = 0; mb < MH; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * MH * wm + 32 * mb + 8 * (r >> 2) + 4 * fg + (r & 3);
        const float gv = FP8 ? acc[mb][0][r] * sg : acc[mb][0][r];
        const float uv = FP8 ? acc[mb][1][r] * su : acc[mb][1][r];
        Ht[row * HLD + 32 * wn + fr] = f32_to_bf16(silu_fast(gv) * uv);
      }
    __syncthreads();
    bf16_t* H = (bf16_t*)a.out;
#pragma unroll
    for (int i = 0; i < 2 * MH; ++i) {
      const int c = tid + 512 * i;
      const int row = c >> 4, cc = (c & 15) * 8;
      const int m = m0 + row, n = ncol0 + cc;   // N % 64 == 0: n < N implies n + 8 <= N
      if (m < M && n < N)
        *reinterpret_cast<u32x4*>(H + (row_begin + m) * N + n) =
            *reinterpret_cast<const u32x4*>(Ht + row * HLD + cc);
    }
    __syncthreads();   // the next tile's prologue overwrites the LDS
  } else {
    float* Y = (float*)a.out;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = ncol0 + 32 * NB * wn + 32 * nb + fr;
      const float sc = FP8 ? a.sc0[(int64_t)g * N + min(n, N - 1)] : 1.0f;
#pragma unroll
      for (int mb = 0; mb < MH; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 32 * MH * wm + 32 * mb + 8 * (r >> 2) + 4 * fg + (r & 3);
          if (m < M && n < N) Y[(row_begin + m) * N + n] = FP8 ? acc[mb][nb][r] * sc : acc[mb][nb][r];
        }
    }
  }
  if (claim.slot != nullptr && tid == 0) *claim.slot = w8_resolve_claim(a, claim, claimed);
}

// One work unit of the 8-wave kernel's table: a tile, or (down GEMM, units from split0
// on) column half v & 1 of tile split0 + v / 2, with the whole tile's K rotation.
template <bool GATED, bool FP8>
__device__ __forceinline__ void w8_unit(const GemmArgs& a, bf16_t* smem, const int* tiles,
                                        const int* offs, int bmb, int64_t unit, int64_t split0,
                                        int nk, const W8Claim& claim) {
  constexpr int COLS = GATED ? 128 : 256;   // output columns per tile
  int half = -1;
  if (!GATED && unit >= split0) {
    const int64_t v = unit - split0;
    unit = split0 + v / 2;
    half = (int)(v & 1);
  }
  const int g = find_group(tiles, a.G, unit);
  int64_t row_begin;
  int M;
  if (g < a.E) {   // the dispatch offsets, copied into LDS at launch
    row_begin = offs[g];
    M = offs[g + 1] - offs[g];
  } else {
    row_begin = a.shared_row0;
    M = a.T;
  }
  const int bm = small_group<GATED>(M) ? BM_SMALL : bmb;
  const int mt_g = (M + bm - 1) / bm;
  // A group's tiles in blocks of W8_NBLOCK n-tiles (the last block may be narrower); within
  // a block m-tile major, so a window of 32 consecutive units is 8 m-tiles x 4 n-tiles
  // sharing their K positions.
  const int local = (int)(unit - tiles[g]);
  const int NT = (a.N + COLS - 1) / COLS, full = NT / W8_NBLOCK;
  int mt, nt;
  if (local < full * mt_g * W8_NBLOCK) {
    const int nb = local / (mt_g * W8_NBLOCK), rem = local % (mt_g * W8_NBLOCK);
    mt = rem / W8_NBLOCK;
    nt = nb * W8_NBLOCK + rem % W8_NBLOCK;
  } else {
    const int rem = local - full * mt_g * W8_NBLOCK, wd = NT - full * W8_NBLOCK;
    mt = rem / wd;
    nt = full * W8_NBLOCK + rem % wd;
  }
  const int ncol0 = nt * COLS;
  const int rows = m_tile_rows<GATED>(M, mt, bmb);
  const int rot = k_rotation<GATED>(g, ncol0, nk);
  const int m0 = mt * bm;
  if constexpr (!GATED) {
    if (half >= 0) {
      const int nc = ncol0 + 128 * half;
      if (nc >= a.N) {   // a tile that holds no second half (N % 256 <= 128)
        if (claim.slot != nullptr && threadIdx.x == 0)
          *claim.slot = w8_resolve_claim(a, claim, atomicAdd(&a.ctr[claim.x], 1));
        return;
      }
      if (rows == 256) w8_tile<4, 1, false, FP8>(a, smem, g, row_begin, M, m0, nc, nk, rot, claim);
      else if (rows == 192) w8_tile<3, 1, false, FP8>(a, smem, g, row_begin, M, m0, nc, nk, rot, claim);
      else if (rows == 128) w8_tile<2, 1, false, FP8>(a, smem, g, row_begin, M, m0, nc, nk, rot, claim);
      else w8_tile<1, 1, false, FP8>(a, smem, g, row_begin, M, m0, nc, nk, rot, claim);
      return;
    }
  }
  if (rows == 256) w8_tile<4, 2, GATED, FP8>(a, smem, g, row_begin, M, m0, ncol0, nk, rot, claim);
  else if (rows == 192) w8_tile<3, 2, GATED, FP8>(a, smem, g, row_begin, M, m0, ncol0, nk, rot, claim);
  else if (rows == 128) w8_tile<2, 2, GATED, FP8>(a, smem, g, row_begin, M, m0, ncol0, nk, rot, claim);
  else w8_tile<1, 2, GATED, FP8>(a, smem, g, row_begin, M, m0, ncol0, nk, rot, claim);
}

// Persistent 8-wave kernel over the tile table, in the order and XCD windows of
// gemm_bf16_kernel (static, or claimed through the 8 per-XCD counters
// a.ctr); the down GEMM with counters cuts a last round that is at most half full into
// column halves, as there.
template <bool GATED, bool FP8>
__global__ __launch_bounds__(512, 1) void gemm_w8_kernel(GemmArgs a) {
  extern __shared__ __align__(16) bf16_t smem[];
  __shared__ int tiles[kMaxExperts + 2];
  __shared__ int offs[kMaxExperts + 1];
  __shared__ long long next_unit;
  constexpr int COLS = GATED ? 128 : 256;
  const int N = a.N;
  __shared__ int bmb_s;
  for (int i = threadIdx.x; i <= a.E; i += blockDim.x) offs[i] = a.offsets[i];
  int bmb = BM_BIG;
  if constexpr (!GATED) {
    __syncthreads();
    bmb = down_tile_rows(a, offs, a.ctr != nullptr, &bmb_s);
  }
  build_tile_table(a, [N, bmb](int M) {
    const int bm = small_group<GATED>(M) ? BM_SMALL : bmb;
    return ((M + bm - 1) / bm) * ((N + COLS - 1) / COLS);
  }, tiles);   // ends with a barrier: offs is visible too
  const int64_t whole = tiles[a.G];
  const int nk = a.K / BK;
  int64_t split0 = whole;
  if (!GATED && a.ctr != nullptr) {
    const int64_t r = whole % gridDim.x;
    if (r > 0 && 2 * r <= (int64_t)gridDim.x) split0 = whole - r;
  }
  const int64_t total = split0 + 2 * (whole - split0);
  const int x = blockIdx.x & 7;
  if (a.ctr == nullptr) {
    const int per = gridDim.x >> 3;
    const int64_t first = (int64_t)x * per + (blockIdx.x >> 3);
    const W8Claim none{nullptr, x, total};
    for (int64_t unit = first; unit < total; unit += gridDim.x)
      w8_unit<GATED, FP8>(a, smem, tiles, offs, bmb, unit, split0, nk, none);
    return;
  }
  // Units claimed through the per-XCD counters: the first here, each next one by the
  // current unit (thread 0 writes it to next_unit at the unit's end).
  const W8Claim claim{&next_unit, x, total};
  if (threadIdx.x == 0) next_unit = w8_resolve_claim(a, claim, atomicAdd(&a.ctr[x], 1));
  __syncthreads();
  int64_t unit = next_unit;
  __syncthreads();   // read by all before thread 0 writes the next one
  while (unit >= 0) {
    w8_unit<GATED, FP8>(a, smem, tiles, offs, bmb, unit, split0, nk, claim);
    __syncthreads();
    unit = next_unit;
    __syncthreads();
  }
}

// ------------------------------------------------------------------ fp32 kernel
// Plain FMA tiles of 64x64 (gate/up: 64 rows x 64 gate + 64 up columns), BK 16.
template <bool GATED>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int TM = 64, TN = 64, TK = 16;
  __shared__ float As[TK][TM + 4];
  __shared__ float Bs[GATED ? 2 : 1][TK][TN + 4];
  __shared__ int tiles[kMaxExperts + 2];
  const int nt = a.n_tiles;
  build_tile_table(a, [nt](int M) { return (M + 63) / 64 * nt; }, tiles);   // 64 x 64 tiles
  const int64_t total = tiles[a.G];
  const int64_t tile = blockIdx.x;
  if (tile >= total) return;
  const int g = find_group(tiles, a.G, tile);
  int64_t row_begin;
  int M;
  group_rows(a, g, row_begin, M);
  const int mt_g = (M + 63) / 64;
  const int64_t local = tile - tiles[g];
  const int m0 = (int)(local % mt_g) * TM;
  const int n0 = (int)(local / mt_g) * TN;
  const float* A = (const float*)a.A;
  const float* B0 = (const float*)a.B0;
  const float* B1 = (const float*)a.B1;
  const int K = a.K, N = a.N;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[2][4][4] = {};
  // loader: 64 rows x 16 k = 1024 floats = 256 threads x 4
  const int lrow = threadIdx.x >> 2, lk = (threadIdx.x & 3) * 4;
  const int am = m0 + lrow;
  const int64_t asrc = a_source_row<GATED>(a, g, row_begin, am < M ? am : 0);
  const int bn = min(n0 + lrow, N - 1);
  for (int k0 = 0; k0 < K; k0 += TK) {
    const float4 va = *reinterpret_cast<const float4*>(A + asrc * K + k0 + lk);
    As[lk + 0][lrow] = va.x; As[lk + 1][lrow] = va.y; As[lk + 2][lrow] = va.z; As[lk + 3][lrow] = va.w;
    const float4 vb = *reinterpret_cast<const float4*>(B0 + ((int64_t)g * N + bn) * K + k0 + lk);
    Bs[0][lk + 0][lrow] = vb.x; Bs[0][lk + 1][lrow] = vb.y; Bs[0][lk + 2][lrow] = vb.z; Bs[0][lk + 3][lrow] = vb.w;
    if (GATED) {
      const float4 vu = *reinterpret_cast<const float4*>(B1 + ((int64_t)g * N + bn) * K + k0 + lk);
      Bs[GATED ? 1 : 0][lk + 0][lrow] = vu.x; Bs[GATED ? 1 : 0][lk + 1][lrow] = vu.y;
      Bs[GATED ? 1 : 0][lk + 2][lrow] = vu.z; Bs[GATED ? 1 : 0][lk + 3][lrow] = vu.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int q = 0; q < (GATED ? 2 : 1); ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float bv = Bs[q][kk][tx * 4 + j];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[q][i][j] = fmaf(av[i], bv, acc[q][i][j]);
        }
    }
    __syncthreads();
  }
  float* out = (float*)a.out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const float v = GATED ? silu_f(acc[0][i][j]) * acc[1][i][j] : acc[0][i][j];
      out[(row_begin + m) * N + n] = v;
    }
  }
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(64), 0, s, p, n);
  return hipGetLastError();
}

// Facts about the current device, looked up once per device (the library may drive
// several GPUs from several threads).

static int device_cu_count() {
  static std::atomic<int> cached[kMaxDevices];   // 0: not looked up yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// The grouped GEMM kernels take more dynamic LDS than the default limit: raised once per
// device and kernel (a repeated call from a racing thread sets the same value again).
template <bool GATED, bool FP8>
static hipError_t allow_kernel_lds() {
  static std::atomic<bool> done[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute((const void*)gemm_bf16_kernel<GATED, FP8>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)KERNEL_LDS_BYTES);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) done[dev].store(true, std::memory_order_release);
  return hipSuccess;
}

template <bool GATED, bool FP8>
static hipError_t allow_w8_lds() {
  static std::atomic<bool> done[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute((const void*)gemm_w8_kernel<GATED, FP8>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)W8_LDS_BYTES);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) done[dev].store(true, std::memory_order_release);
  return hipSuccess;
}

// bf16 layers with a batch in which some group may be large (a group holds at most T
// rows): the whole GEMM runs in the 8-wave kernel (small groups as 64-row tiles there; on
// the Switch-shaped layer this beats sending them to gemm_bf16_kernel's streaming tiles in
// a second launch: gate/up 1.05 -> 1.01 ms, down 0.61 -> 0.52 ms).  Decode-sized batches
// stay with gemm_bf16_kernel.  Returns whether it launched.
template <bool GATED>
static hipError_t run_w8(const GemmArgs& a, const moe_desc_t& d, bool fp8, hipStream_t s,
                         bool* launched) {
  *launched = false;
  if (d.dtype != MOE_DTYPE_BF16 || d.T < (GATED ? SMALL_GROUP_ROWS_GATED : SMALL_GROUP_ROWS_DOWN))
    return hipSuccess;
  hipError_t e = fp8 ? allow_w8_lds<GATED, true>() : allow_w8_lds<GATED, false>();
  if (e != hipSuccess) return e;
  const int64_t grid = round_up(device_cu_count(), 8);
  if (fp8)
    hipLaunchKernelGGL((gemm_w8_kernel<GATED, true>), dim3((unsigned)grid), dim3(512), W8_LDS_BYTES, s, a);
  else
    hipLaunchKernelGGL((gemm_w8_kernel<GATED, false>), dim3((unsigned)grid), dim3(512), W8_LDS_BYTES, s, a);
  e = hipGetLastError();
  *launched = e == hipSuccess;
  return e;
}

template <bool GATED, bool FP8>
static hipError_t run_bf16(const GemmArgs& a, int64_t max_tiles, hipStream_t s) {
  const hipError_t e = allow_kernel_lds<GATED, FP8>();
  if (e != hipSuccess) return e;
  int64_t grid = device_cu_count();
  if (max_tiles < grid) grid = max_tiles;
  grid = round_up(grid, 8);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<GATED, FP8>), dim3((unsigned)grid), dim3(256),
                     KERNEL_LDS_BYTES, s, a);
  return hipGetLastError();
}

template <bool GATED>
static hipError_t run_f32(const GemmArgs& a, int64_t max_m_tiles, hipStream_t s) {
  const int64_t grid = max_m_tiles * a.n_tiles;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_f32_kernel<GATED>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

static GemmArgs base_args(const moe_desc_t& d, const GemmRows& rows, const int32_t* offsets) {
  GemmArgs a{};
  a.offsets = offsets;
  a.shared_row0 = rows.routed;
  a.T = (int)d.T;
  a.topk = rows.token_div;
  a.E = (int)d.n_experts;
  a.G = (int)(d.n_experts + d.n_shared);
  return a;
}

// Dynamic tile order pays off where tile costs differ (large groups with 64-, 128- or
// 256-row remainder tiles); for decode-sized batches (all groups small, every tile alike)
// the counter round trip per tile is pure cost.  Taken when the groups average at least
// 128 rows.
static bool dynamic_tiles(const moe_desc_t& d, const GemmRows& rows) {
  return rows.routed >= (int64_t)2 * BM_SMALL * d.n_experts;
}

// Share of the CU slots of the last round left idle by n equal tiles on cus CUs.
static double idle_fraction(int64_t n, int64_t cus) {
  if (n <= 0) return 0.0;
  const int64_t slots = ceil_div(n, cus) * cus;
  return (double)(slots - n) / (double)slots;
}

// Upper bound of sum_g ceil(M_g / bm): ceil(routed / bm) + E (+ ceil(T / bm) shared).
static int64_t max_m_tiles(const moe_desc_t& d, const GemmRows& rows, int bm) {
  return ceil_div(rows.routed, bm) + d.n_experts + (d.n_shared ? ceil_div(d.T, bm) : 0);
}

hipError_t launch_gate_up(const moe_desc_t& d, const GemmRows& rows, const void* x,
                          const int32_t* perm_src, const int32_t* offsets,
                          const ExpertWeights& ew, void* H, int32_t* ctr, hipStream_t s) {
  const bool bf = d.dtype == MOE_DTYPE_BF16;
  GemmArgs a = base_args(d, rows, offsets);
  a.A = x;
  a.perm_src = perm_src;
  a.B0 = ew.gate;
  a.B1 = ew.up;
  a.sc0 = ew.s_gate;
  a.sc1 = ew.s_up;
  a.out = H;
  a.N = (int)d.d_ff;
  a.K = (int)d.d_model;
  a.n_tiles = (int)ceil_div(d.d_ff, 64);   // fp32 kernel: 64-column tiles
  a.ctr = dynamic_tiles(d, rows) ? ctr : nullptr;
  a.skinny_all = d.T <= SKINNY_ROWS && a.ctr == nullptr;   // a group holds at most T rows
  {
    // Every group fits a skinny tile (at most T rows each): take 64-column tiles when that
    // leaves less of the last round idle, e.g. 8 experts x 14336 columns give 896 tiles of
    // 128 (3.5 rounds of a 256-CU chip) but 1792 of 64 (7 rounds).
    const int64_t groups = std::min<int64_t>(d.n_experts + d.n_shared, rows.routed + d.n_shared);
    const int64_t cus = device_cu_count();
    a.narrow_small = d.T <= SKINNY_ROWS &&
                     idle_fraction(groups * ceil_div(d.d_ff, 64), cus) + 0.02 <
                         idle_fraction(groups * ceil_div(d.d_ff, 128), cus);
  }
  const int64_t mt = max_m_tiles(d, rows, BM_SMALL) * ceil_div(d.d_ff, 64);
  if (!bf) return run_f32<true>(a, max_m_tiles(d, rows, 64), s);
  {
    bool launched = false;
    const hipError_t e = run_w8<true>(a, d, ew.fp8, s, &launched);
    if (e != hipSuccess || launched) return e;
  }
  return ew.fp8 ? run_bf16<true, true>(a, mt, s) : run_bf16<true, false>(a, mt, s);
}

hipError_t launch_down(const moe_desc_t& d, const GemmRows& rows, const void* H,
                       const int32_t* offsets, const ExpertWeights& ew, float* Yp,
                       int32_t* ctr, hipStream_t s) {
  const bool bf = d.dtype == MOE_DTYPE_BF16;
  GemmArgs a = base_args(d, rows, offsets);
  a.A = H;
  a.B0 = ew.down;
  a.sc0 = ew.s_down;
  a.out = Yp;
  a.N = (int)d.d_model;
  a.K = (int)d.d_ff;
  a.n_tiles = (int)ceil_div(d.d_model, 64);
  {
    // narrow down tiles for small groups only when even the most groups that can exist
    // would give fewer than two 256-column tiles per CU
    const int64_t groups = std::min<int64_t>(d.n_experts + d.n_shared, rows.routed + d.n_shared);
    a.narrow_small = groups * ceil_div(d.d_model, 256) < 2 * (int64_t)device_cu_count();
  }
  a.ctr = dynamic_tiles(d, rows) ? ctr : nullptr;
  a.skinny_all = d.T <= SKINNY_ROWS && a.ctr == nullptr;
  const int64_t mt = max_m_tiles(d, rows, BM_SMALL) * ceil_div(d.d_model, 128);
  if (!bf) return run_f32<false>(a, max_m_tiles(d, rows, 64), s);
  {
    bool launched = false;
    const hipError_t e = run_w8<false>(a, d, ew.fp8, s, &launched);
    if (e != hipSuccess || launched) return e;
  }
  return ew.fp8 ? run_bf16<false, true>(a, mt, s) : run_bf16<false, false>(a, mt, s);
}

}  // namespace moe
