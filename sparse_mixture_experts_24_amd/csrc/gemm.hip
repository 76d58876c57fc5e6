// Grouped SwiGLU experts: for every expert (group) g the rows [row_begin_g,
// row_begin_g + M_g) of the expert-contiguous order run through
//   H = SiLU(X W_gate[g]^T) * (X W_up[g]^T)      (gate/up GEMM, fused epilogue)
//   Yp = H W_down[g]^T                             (down GEMM)
// "Chapter 30: Mixture of Experts" (LLM Transformer book), 30.2.4: w1 through SiLU,
// w3 linear, w2 back to d; "Mixture-of-experts in practice" (deepseekmodel.com),
// expert-parallel section: with the tokens of each expert contiguous, one grouped GEMM
// computes all experts of the layer at once instead of one small GEMM per expert.
//
// bf16 kernel (gfx950):
//   * one 256x256 output tile per iteration of a persistent loop; 4 wave64s, each a
//     128x128 sub-tile held in 16 v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 per
//     lane); for the gate/up GEMM a wave's 128 columns are 64 gate + the matching 64 up
//     columns, so SiLU(g)*u is formed in registers and H is stored once, in bf16;
//   * K is walked in 64-wide steps through two LDS stages (rows padded to 72 bf16 so
//     that a wavefront's 16-byte fragment reads hit distinct banks); the next step's
//     global loads are in flight while the current step's 64 MFMAs run;
//   * the X rows of the gate/up GEMM are gathered on the fly through perm_src (the
//     permuted activations are never materialised);
//   * the tile table (per-group m-tile prefix) is built on the device from the
//     dispatch offsets, so skewed per-expert counts need no host round trip; tiles are
//     ordered (group, n-tile, m-tile), and each XCD takes a contiguous run of them, so
//     the m-tiles that share a weight tile run on the same L2.
#include <math.h>

#include <algorithm>

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

// Weight registers of one K step: bf16 [nb][k16 step] operands, or the 32 code bytes of
// each lane for 8-bit weights (k16 step s in bytes [8s, 8s + 8)).
template <bool FP8, int NB>
struct BRegs {
  bf16x8 v[NB][4];
  __device__ __forceinline__ bf16x8 op(int nb, int s) const { return v[nb][s]; }
};
template <int NB>
struct BRegs<true, NB> {
  u32x4 v[NB][2];
  __device__ __forceinline__ bf16x8 op(int nb, int s) const {
    const u32x4 q = v[nb][s >> 1];
    return (s & 1) ? e4m3x8_to_bf16(q[2], q[3]) : e4m3x8_to_bf16(q[0], q[1]);
  }
};

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

// ------------------------------------------------------------------ bf16 MFMA kernel
// Output tile BM x BN, BN = 256 (gate/up: 128 gate + the matching 128 up columns).
// BM = 32*MB rows: 256 for groups that are not small (small_group below; the last tile
// of a group 64, 128, 192 or 256 rows, to fit the remainder), 64 for small ones, so small
// experts (decode, the tail of skewed or capacity-limited routing) do not pay for 256-row
// MFMA tiles.  Wave w owns B rows [64w, 64w + 64) of the tile (gate/up: 32 gate + 32 up)
// and all BM A rows: MB x 2 blocks of 32x32 accumulators.
//   * B (the weights) goes straight from global memory into MFMA operand registers,
//     three register sets deep: the set for K-step t+2 is issued at step t, so a weight
//     load has two steps of work to arrive;
//   * A (the token rows) is staged once per block through LDS (two stages, rows padded to
//     72 bf16 so fragment reads hit distinct banks) and read by all four waves;
//   * inside a 64-wide K step the MFMA k-slots are permuted: step s, lane half g uses the
//     physical columns [32g + 8s, 32g + 8s + 8), for A and B alike, so each lane's B data
//     for the whole step is 64 contiguous bytes of one weight row;
//   * each K step is one scheduling region in which the fragment reads of k16 step s+1
//     and the global loads are interleaved with the MFMAs of step s.
constexpr int BK = 64, LDK = BK + 8;
constexpr int BM_BIG = 256, BM_SMALL = 64;
// Row counts from which a group takes the MFMA tiles instead of 64-row tiles.  gate/up: a
// group of 65-128 rows runs faster as one 128-row tile (its weights read once) than as
// two 64-row streaming tiles; the down GEMM's 64-row tiles, 256 columns wide, stay ahead
// up to 80 rows.  (Measured on the Switch-shaped layer, whose groups hold 32-320 rows:
// gate/up 1.13 -> 1.07 ms, down 0.59 -> 0.56 ms against one bound of 128 rows for both.)
constexpr int SMALL_GROUP_ROWS_GATED = 65, SMALL_GROUP_ROWS_DOWN = 81;
constexpr size_t GEMM_LDS_BYTES = 2 * BM_BIG * LDK * sizeof(bf16_t);   // 73728

// Tile shape of a group with M rows: 256-row tiles for large groups, 64-row tiles for
// small ones.  Columns per tile: gate/up 128 (each wave one 32-column block of gate and
// the same block of up); down 256, or 128 for small groups when the host finds the
// whole launch short of tiles (decode-sized batches, where the GEMM streams weights and
// every CU must take part).
template <bool GATED>
__device__ inline bool small_group(int M) {
  return M < (GATED ? SMALL_GROUP_ROWS_GATED : SMALL_GROUP_ROWS_DOWN);
}
// Rows of m-tile mt (tiles start at mt * 256 in large groups, mt * 64 in small ones):
// large groups take 256-row tiles and put their remainder in one tile of 64, 128, 192 or
// 256 rows, whichever is the smallest that holds it.
template <bool GATED>
__device__ inline int m_tile_rows(int M, int mt) {
  if (small_group<GATED>(M)) return BM_SMALL;
  const int r = M - mt * BM_BIG;
  return r > 192 ? BM_BIG : r > 128 ? 192 : r > 64 ? 128 : 64;
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
// skewed or capacity-limited routing).  Same math as gemm_bf16_tile<2, NB, GATED>, but the
// weights are read with whole 128-byte row segments per 8 lanes (HBM-friendly, where the
// register-direct layout has 32 rows x 32 bytes per load) and put into MFMA order through
// a wave-private LDS buffer: two stages of [NB*32 rows][64 bf16], 16-byte chunks XOR
// swizzled (chunk c of row r at c ^ ((r/2)%8)) so both the stores and the fragment reads
// are conflict-free.  P steps of weights are in flight per wave (P register sets).
constexpr int SB_STAGE = 2 * 32 * BK;                 // bf16 per wave stage, NB <= 2
constexpr size_t SMALL_LDS_BYTES =
    (size_t)(2 * 64 * LDK + 4 * 2 * SB_STAGE) * sizeof(bf16_t);   // A stages + B buffers
// Steps of weights in flight per wave (measured on decode-sized launches: about 16 KB
// (two-block tiles) to 32 KB (one-block down tiles) per wave is best; more is slower).
constexpr int STREAM_P2 = 2, STREAM_P1 = 8;
// Tiles whose group has at most 32 rows left take the barrier-free skinny tile, with 2
// (bf16 weights) or 4 (8-bit weights: half the bytes per step) K steps in flight per wave
// (measured on decode-sized launches; deeper is slower).
constexpr int SKINNY_ROWS = 32;
template <bool FP8>
constexpr int skinny_p() { return FP8 ? 4 : 2; }
constexpr size_t KERNEL_LDS_BYTES =
    GEMM_LDS_BYTES > SMALL_LDS_BYTES ? GEMM_LDS_BYTES : SMALL_LDS_BYTES;
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

// A tile of at most 32 rows (decode-sized groups): every wave computes all of them against
// its own weight rows and reads its token fragments straight from global memory (the few
// rows are L1/L2 hits), so the K loop has no block barrier and no LDS traffic for the
// tokens.  The weights stream as in gemm_bf16_tile_stream (whole row segments per load,
// through the wave's swizzled LDS stages); P steps of weights and tokens are in flight.
//
// Gate/up with NB == 1 (64-column tiles, for launches whose tiles would leave much of a
// last round idle): the wave's 32 weight rows are 16 gate rows and the 16 matching up rows
// and the MFMA is taken transposed (D[weight row][token]), so a lane holds gate and up of
// one (token, h) in registers r and r + 8.
template <int NB, bool GATED, int P, bool FP8>
__device__ __forceinline__ void gemm_bf16_tile_skinny(const GemmArgs& a, bf16_t* smem, int g,
                                                      int64_t row_begin, int M, int m0,
                                                      int ncol0, int k0, int nk, int rot,
                                                      void* outp) {
  constexpr bool PAIRED = GATED && NB == 1;
  static_assert(P % 2 == 0, "the step loop is unrolled by P (even: two LDS stages)");
  constexpr int MB = 1;
  constexpr int NL = FP8 ? 2 * NB : 4 * NB;     // B loads per step
  constexpr int WB = FP8 ? 1 : 2;               // bytes per weight
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int fr = lane & 31, fg = lane >> 5;
  const bf16_t* A = (const bf16_t*)a.A + k0 * BK;
  const int K = a.K, N = a.N;
  bf16_t* Bw = smem + w * 2 * SB_STAGE;          // this wave's two B stages

  // token row of this lane's fragments: row fr of the tile (rows past M read row 0 of the
  // group; their results are never stored); lane half fg reads k 32 fg .. 32 fg + 31
  int aoff;
  {
    const int m = m0 + fr < M ? m0 + fr : 0;
    if (GATED && g < a.E) aoff = a.perm_src[row_begin + m] / a.topk * K;
    else aoff = ((GATED ? 0 : (int)row_begin) + m) * K;
    aoff += 32 * fg;
  }
  const char* pbl[NL];
  int bst[NL];
  int bcol[NB];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int nb = FP8 ? j / 2 : j / 4;
    const int r = FP8 ? 16 * (j % 2) + (lane >> 2) : 8 * (j % 4) + (lane >> 3);
    const int c = FP8 ? lane & 3 : lane & 7;
    const int n = PAIRED  ? ncol0 + 16 * w + (r & 15)
                  : GATED ? ncol0 + 32 * w + r
                          : ncol0 + 32 * NB * w + 32 * nb + r;
    const char* base =
        (const char*)((PAIRED ? r >= 16 : (GATED && nb == 1)) ? a.B1 : a.B0);
    pbl[j] = base + (((int64_t)g * N + min(n, N - 1)) * K + k0 * BK) * WB + 16 * c;
    bst[j] = FP8 ? (nb * 32 + r) * BK + 16 * (c ^ ((r >> 2) & 3))
                 : 2 * ((nb * 32 + r) * BK + 8 * (c ^ ((r >> 1) & 7)));
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    bcol[nb] = GATED ? ncol0 + 32 * w + fr : ncol0 + 32 * NB * w + 32 * nb + fr;
  int brd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    brd[s] = FP8 ? fr * BK + 16 * ((2 * fg + (s >> 1)) ^ ((fr >> 2) & 3)) + 8 * (s & 1)
                 : 2 * (fr * BK + 8 * ((4 * fg + s) ^ ((fr >> 1) & 7)));

  floatx16 acc[MB][NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][j][r] = 0.0f;

  u32x4 rb[P][NL];       // weights of steps in flight: set q holds step t with t % P == q
  bf16x8 ra[P][4];       // token fragments of the same steps (k16 steps 0..3)

#define MOE_KSTEP(t) ((min((t), nk - 1) + rot) - ((min((t), nk - 1) + rot) >= nk ? nk : 0))
#define MOE_KLOAD(q, t)                                                                    \
  {                                                                                        \
    _Pragma("unroll") for (int j = 0; j < NL; ++j)                                         \
      rb[q][j] = *reinterpret_cast<const u32x4*>(pbl[j] + MOE_KSTEP(t) * BK * WB);         \
    _Pragma("unroll") for (int s = 0; s < 4; ++s)                                          \
      ra[q][s] = *reinterpret_cast<const bf16x8*>(A + aoff + MOE_KSTEP(t) * BK + 8 * s);   \
  }
#define MOE_KSTORE_B(q, st)                                                                \
  _Pragma("unroll") for (int j = 0; j < NL; ++j)                                           \
    *reinterpret_cast<u32x4*>((char*)Bw + (st) * SB_STAGE * 2 + bst[j]) = rb[q][j];
  // K step t (weights in stage t % 2, tokens in set t % P): the weights of step t+1 go from
  // their registers into the other stage and the set is refilled with step t+1+P.  Steps
  // t >= nk (padding to a multiple of P) multiply zero token fragments.
#define MOE_KSTEP_BODY(t, q0, q1)                                                          \
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
    MOE_KLOAD(q0, (t) + P);                                                                \
  }

  // Prologue: steps 0..P-1 requested; step 0's weights stored.  Step t's set q0 = t % P is
  // reloaded with step t+P after its MFMAs; set q1 = (t+1) % P was requested P-1 steps ago.
#pragma unroll
  for (int q = 0; q < P; ++q) MOE_KLOAD(q, q);
  MOE_KSTORE_B(0, 0);
  const int nkp = (nk + P - 1) / P * P;
  for (int kt = 0; kt < nkp; kt += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) MOE_KSTEP_BODY(kt + u, u, (u + 1) % P);   // (u: macros use j, s)
  }
#undef MOE_KSTEP
#undef MOE_KLOAD
#undef MOE_KSTORE_B
#undef MOE_KSTEP_BODY
  __syncthreads();   // every wave is done with its LDS stages before the epilogue uses LDS
  if constexpr (PAIRED) {
    // acc[0][0][r] (r < 8): gate row 8(r/4) + 4 fg + r%4 of the wave's 16, token fr;
    // r + 8: the matching up row.  h -> bf16 into an LDS tile [32][64 + 8], then 16-byte
    // row stores (one per thread).
    constexpr int HLD = 72;
    bf16_t* Ht = smem;
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
            const int64_t hrow = (int64_t)g * N + min(ncol0 + 16 * w + 8 * q + 4 * fg + 2 * i + e, N - 1);
            gv[e] *= a.sc0[hrow];
            uv[e] *= a.sc1[hrow];
          }
        }
        pk[i] = (uint32_t)f32_to_bf16(silu_fast(gv[0]) * uv[0]) |
                ((uint32_t)f32_to_bf16(silu_fast(gv[1]) * uv[1]) << 16);
      }
      *reinterpret_cast<uint2*>(Ht + fr * HLD + 16 * w + 8 * q + 4 * fg) = make_uint2(pk[0], pk[1]);
    }
    __syncthreads();
    bf16_t* Hout = (bf16_t*)outp;
    const int tid = threadIdx.x, row = tid >> 3, cc = (tid & 7) * 8;
    const int m = m0 + row, n = ncol0 + cc;   // N % 64 == 0: n < N implies n + 8 <= N
    if (m < M && n < N)
      *reinterpret_cast<u32x4*>(Hout + (row_begin + m) * N + n) =
          *reinterpret_cast<const u32x4*>(Ht + row * HLD + cc);
    __syncthreads();   // the next tile's prologue overwrites the LDS
  } else {
    float scl[NB];
    load_scales<NB, GATED, FP8>(a, g, bcol, scl);
    store_tile<MB, NB, GATED, FP8>(acc, smem, outp, row_begin, M, m0, ncol0, N, bcol, scl);
  }
}

// One output tile over K steps [k0, k0 + nk) (callers pass the whole K), into outp.
template <int MB, int NB, bool GATED, bool FP8>
__device__ __forceinline__ void gemm_bf16_tile(const GemmArgs& a, bf16_t* smem, int g,
                                               int64_t row_begin, int M, int m0, int ncol0,
                                               int k0, int nk, int rot, void* outp) {
  static_assert(!GATED || NB == 2, "gate/up tiles pair one gate and one up block per wave");
  constexpr int BMT = 32 * MB;
  constexpr int STAGE = BMT * LDK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = tid >> 3, lc = (tid & 7) * 8;       // A load: row lr + 32i, k offset lc
  const int fr = lane & 31, fg = lane >> 5;          // fragment row / lane half
  const bf16_t* A = (const bf16_t*)a.A + k0 * BK;
  const int K = a.K, N = a.N;

  // A: element offsets (32-bit; the host bounds T*d and rows*F below 2^31).  The
  // perm_src gathers of the routed rows are issued together, then converted.
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
    const int base = GATED ? 0 : (int)row_begin;     // shared expert: token m; down: row
#pragma unroll
    for (int i = 0; i < MB; ++i) aoff[i] = (base + aoff[i]) * K + lc;
  }
  // B: this lane's NB weight rows (one per n-block), 32 contiguous k per lane half
  // (64 bytes of bf16, or 32 bytes of 8-bit codes)
  constexpr int WB = FP8 ? 1 : 2;                    // bytes per weight
  const char* pb[NB];
  int bcol[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = GATED ? ncol0 + 32 * w + fr : ncol0 + 32 * NB * w + 32 * nb + fr;
    const char* base = (const char*)((GATED && nb == 1) ? a.B1 : a.B0);
    bcol[nb] = n;
    pb[nb] = base + (((int64_t)g * N + min(n, N - 1)) * K + 32 * fg + k0 * BK) * WB;
  }

  floatx16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  BRegs<FP8, NB> b0, b1, b2;   // three B register sets
  u32x4 ra[MB];

  // Step t reads K step (t + rot) mod nk (see k_rotation).
#define MOE_KSTEP(t) ((min((t), nk - 1) + rot) - ((min((t), nk - 1) + rot) >= nk ? nk : 0))
#define MOE_LOAD_B(set, t)                                                                 \
  _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) {                                      \
    if constexpr (FP8) {                                                                   \
      _Pragma("unroll") for (int h = 0; h < 2; ++h)                                        \
        set.v[nb][h] = *reinterpret_cast<const u32x4*>(pb[nb] + MOE_KSTEP(t) * BK + 16 * h); \
    } else {                                                                               \
      _Pragma("unroll") for (int s = 0; s < 4; ++s)                                        \
        set.v[nb][s] =                                                                     \
            *reinterpret_cast<const bf16x8*>(pb[nb] + MOE_KSTEP(t) * BK * 2 + 16 * s);     \
    }                                                                                      \
  }
#define MOE_LOAD_A(t)                                                                      \
  _Pragma("unroll") for (int i = 0; i < MB; ++i)                                           \
    ra[i] = *reinterpret_cast<const u32x4*>(A + aoff[i] + MOE_KSTEP(t) * BK);
#define MOE_STORE_A(st)                                                                    \
  {                                                                                        \
    bf16_t* As_ = smem + (st) * STAGE;                                                     \
    _Pragma("unroll") for (int i = 0; i < MB; ++i)                                         \
      *reinterpret_cast<u32x4*>(As_ + (lr + 32 * i) * LDK + lc) = ra[i];                   \
  }
#define MOE_READ_A(af, st, s)                                                              \
  _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                        \
    af[mb] = *reinterpret_cast<const bf16x8*>(smem + (st) * STAGE + (mb * 32 + fr) * LDK + \
                                              32 * fg + 8 * (s));
#define MOE_MFMA(af, set, s)                                                               \
  _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                        \
    _Pragma("unroll") for (int nb = 0; nb < NB; ++nb)                                      \
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], set.op(nb, s),          \
                                                            acc[mb][nb], 0, 0, 0);
#define MOE_COMPUTE(set, st)                                                               \
  {                                                                                        \
    bf16x8 fa[MB], fb[MB];                                                                 \
    MOE_READ_A(fa, st, 0);                                                                 \
    MOE_READ_A(fb, st, 1);                                                                 \
    MOE_MFMA(fa, set, 0);                                                                  \
    MOE_READ_A(fa, st, 2);                                                                 \
    MOE_MFMA(fb, set, 1);                                                                  \
    MOE_READ_A(fb, st, 3);                                                                 \
    MOE_MFMA(fa, set, 2);                                                                  \
    MOE_MFMA(fb, set, 3);                                                                  \
  }
  // Region order: the 2*MB fragment reads of k16 steps 0 and 1, then per k16 step s a
  // quarter of the MB + 4*NB global loads and MB x {NB MFMAs, (read for step s+2)}.
#define MOE_INTERLEAVE(s, reads)                                                           \
  {                                                                                        \
    constexpr int NGL_ = MB + 4 * NB;                                                      \
    __builtin_amdgcn_sched_group_barrier(0x020, NGL_ * ((s) + 1) / 4 - NGL_ * (s) / 4, 0); \
    _Pragma("unroll") for (int j_ = 0; j_ < MB; ++j_) {                                    \
      __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);                                  \
      if (reads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                        \
    }                                                                                      \
  }
  // Steps t >= nk (padding the step count up to a multiple of 3) read zero A rows, so the
  // accumulators are unchanged, and the loop body has no exits.
#define MOE_STEP_END(t, cur, nxt2)                                                             \
  {                                                                                        \
    MOE_LOAD_A(min((t) + 1, nk - 1));                                                      \
    MOE_LOAD_B(nxt2, (t) + 2);                                                             \
    MOE_COMPUTE(cur, (t) & 1);                                                             \
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * MB, 0);                                \
    MOE_INTERLEAVE(0, 1)                                                                   \
    MOE_INTERLEAVE(1, 1)                                                                   \
    MOE_INTERLEAVE(2, 0)                                                                   \
    MOE_INTERLEAVE(3, 0)                                                                   \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    if ((t) + 1 >= nk) {                                                                   \
      _Pragma("unroll") for (int i = 0; i < MB; ++i) ra[i] = u32x4{0u, 0u, 0u, 0u};        \
    }                                                                                      \
    MOE_STORE_A(((t) + 1) & 1);                                                            \
    __syncthreads();                                                                       \
  }

  // Scheduling of a k16 step of the first half: a quarter of the weight loads, then MB x
  // {NB MFMAs, one fragment read for the second half}.
#define MOE_SGB_HALF                                                                       \
  __builtin_amdgcn_sched_group_barrier(0x020, 2 * NB, 0);                                  \
  _Pragma("unroll") for (int j_ = 0; j_ < MB; ++j_) {                                      \
    __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);                                    \
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                     \
  }
  // K step t (rows in stage t & 1, weights in set cur; the registers ra hold the rows of
  // step t+1, requested halfway through step t-1).  Halfway through the step, after the
  // MFMAs of k16 steps 0 and 1, ra goes to the other stage (read last during step t-1,
  // before the barrier that ended it) and is refilled with the rows of step t+2, so the
  // LDS writes overlap the MFMAs of k16 steps 2 and 3 instead of stalling the step's end.
#define MOE_STEP(t, cur, nxt2)                                                             \
  {                                                                                        \
    MOE_LOAD_B(nxt2, (t) + 2);                                                             \
    {                                                                                      \
      bf16x8 fa[MB], fb[MB];                                                               \
      MOE_READ_A(fa, (t) & 1, 0);                                                          \
      MOE_READ_A(fb, (t) & 1, 1);                                                          \
      MOE_MFMA(fa, cur, 0);                                                                \
      MOE_READ_A(fa, (t) & 1, 2);                                                          \
      MOE_MFMA(fb, cur, 1);                                                                \
      MOE_READ_A(fb, (t) & 1, 3);                                                          \
      MOE_STORE_A(((t) + 1) & 1);                                                          \
      MOE_LOAD_A(min((t) + 2, nk - 1));                                                    \
      MOE_MFMA(fa, cur, 2);                                                                \
      MOE_MFMA(fb, cur, 3);                                                                \
    }                                                                                      \
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * MB, 0);                                \
    MOE_SGB_HALF                                                                           \
    MOE_SGB_HALF                                                                           \
    __builtin_amdgcn_sched_group_barrier(0x200, MB, 0);                                    \
    __builtin_amdgcn_sched_group_barrier(0x020, MB / 2, 0);                                \
    __builtin_amdgcn_sched_group_barrier(0x008, NB * MB, 0);                               \
    __builtin_amdgcn_sched_group_barrier(0x020, MB - MB / 2, 0);                           \
    __builtin_amdgcn_sched_group_barrier(0x008, NB * MB, 0);                               \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    __syncthreads();                                                                       \
  }

  // Gate/up 256-row tiles store their next rows halfway through each step; the other tiles
  // (down, and the 128/64-row remainders) store them at the end of the step: the mid-step
  // order needs more registers live across the step and spills there.
  if constexpr (GATED && MB == 8) {
  MOE_LOAD_B(b0, 0);
  MOE_LOAD_B(b1, 1);
  MOE_LOAD_A(0);
  MOE_STORE_A(0);
  MOE_LOAD_A(min(1, nk - 1));
  __syncthreads();
  // Whole triples of steps (the B register sets rotate with period 3), then the last
  // nk % 3 steps; loads past the last step are clamped to it (in bounds, never used).
  int kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
    MOE_STEP(kt, b0, b2);
    MOE_STEP(kt + 1, b1, b0);
    MOE_STEP(kt + 2, b2, b1);
  }
  if (kt < nk) MOE_STEP(kt, b0, b2);
  if (kt + 1 < nk) MOE_STEP(kt + 1, b1, b0);
  } else {
  MOE_LOAD_B(b0, 0);
  MOE_LOAD_B(b1, 1);
  MOE_LOAD_A(0);
  MOE_STORE_A(0);
  __syncthreads();
  const int nk3 = (nk + 2) / 3 * 3;
  for (int kt = 0; kt < nk3; kt += 3) {
    MOE_STEP_END(kt, b0, b2);
    MOE_STEP_END(kt + 1, b1, b0);
    MOE_STEP_END(kt + 2, b2, b1);
  }
  }
#undef MOE_KSTEP
#undef MOE_LOAD_B
#undef MOE_LOAD_A
#undef MOE_STORE_A
#undef MOE_READ_A
#undef MOE_MFMA
#undef MOE_SGB_HALF
#undef MOE_STEP
#undef MOE_COMPUTE
#undef MOE_INTERLEAVE
#undef MOE_STEP_END

  float scl[NB];
  load_scales<NB, GATED, FP8>(a, g, bcol, scl);
  store_tile<MB, NB, GATED, FP8>(acc, smem, outp, row_begin, M, m0, ncol0, N, bcol, scl);
}

// First K step of a tile: tiles running at the same time start at different K offsets, so
// their weight streams spread over the HBM channels instead of all reading the same column
// range of rows at a common stride.  A function of the expert and the output columns only
// (in units of the large tiles' width, whatever the tile kind), so the summation order of
// an output element does not depend on the rest of the batch.
template <bool GATED>
__device__ inline int k_rotation(int g, int ncol0, int nk) {
  const unsigned cb = (unsigned)ncol0 / (GATED ? 128u : 256u);
  return (int)((cb + 13u * (unsigned)g) % (unsigned)nk);
}

// One work unit: a tile of the table built in LDS.  Units from split0 on are the
// launch's last tiles cut in two column halves (down GEMM only, see gemm_bf16_kernel):
// unit split0 + 2 v + h is column half h of tile unit split0 + v.  Only 256- and 192-row
// tiles are cut; of another tile, half 0 is the whole tile and half 1 is empty.
template <bool GATED, bool FP8>
__device__ __forceinline__ void gemm_bf16_unit(const GemmArgs& a, bf16_t* smem,
                                               const int* tiles, int64_t ntile, int64_t unit,
                                               int64_t split0) {
  int half = -1;   // -1: the whole tile; 0 or 1: that column half
  if (unit >= split0) {
    const int64_t v = unit - split0;
    unit = split0 + v / 2;
    half = (int)(v & 1);
  }
  const int64_t tile = unit;
  const int k0 = 0, nk = a.K / BK;
  void* outp = a.out;
  const int g = find_group(tiles, a.G, tile);
  int64_t row_begin;
  int M;
  group_rows(a, g, row_begin, M);
  const bool sm = small_group<GATED>(M);
  const int narrow = a.narrow_small;
  const int mt_g = (M + (sm ? BM_SMALL : BM_BIG) - 1) / (sm ? BM_SMALL : BM_BIG);
  const int local = (int)(tile - tiles[g]);          // ordered (n-tile, m-tile)
  const int mt = local % mt_g;
  const int ncol0 = (local / mt_g) * tile_cols<GATED>(sm, narrow);
  const int rows = m_tile_rows<GATED>(M, mt);
  const int rot = k_rotation<GATED>(g, ncol0, nk);
  if constexpr (!GATED) {
    if (half >= 0) {
      // A column half has the whole tile's K walk (rot depends on the 256-column block
      // only), so every output element sums in the same order as in the whole tile.
      const int nc = ncol0 + 128 * half;
      if (nc >= a.N) return;   // a tile that holds no second half (N % 256 <= 128)
      if (!sm && rows == BM_BIG) {
        gemm_bf16_tile<BM_BIG / 32, 1, GATED, FP8>(a, smem, g, row_begin, M, mt * BM_BIG, nc, k0,
                                                   nk, rot, outp);
        return;
      }
      if (!sm && rows == 192) {
        gemm_bf16_tile<192 / 32, 1, GATED, FP8>(a, smem, g, row_begin, M, mt * BM_BIG, nc, k0,
                                                nk, rot, outp);
        return;
      }
      if (half == 1) return;
    }
  }
  if (!sm && rows == BM_BIG)
    gemm_bf16_tile<BM_BIG / 32, 2, GATED, FP8>(a, smem, g, row_begin, M, mt * BM_BIG, ncol0, k0, nk,
                                          rot, outp);
  else if (!sm && rows == 192)
    gemm_bf16_tile<192 / 32, 2, GATED, FP8>(a, smem, g, row_begin, M, mt * BM_BIG, ncol0, k0, nk,
                                       rot, outp);
  else if (!sm && rows == 128)
    gemm_bf16_tile<128 / 32, 2, GATED, FP8>(a, smem, g, row_begin, M, mt * BM_BIG, ncol0, k0, nk,
                                       rot, outp);
  else if (!sm)
    gemm_bf16_tile<BM_SMALL / 32, 2, GATED, FP8>(a, smem, g, row_begin, M, mt * BM_BIG, ncol0, k0,
                                            nk, rot, outp);
  else if (M - mt * BM_SMALL <= SKINNY_ROWS) {
    // (gate/up takes 64-column tiles only when every group fits a skinny tile)
    if (!narrow)
      gemm_bf16_tile_skinny<2, GATED, skinny_p<FP8>(), FP8>(a, smem, g, row_begin, M,
                                                            mt * BM_SMALL, ncol0, k0, nk, rot,
                                                            outp);
    else
      gemm_bf16_tile_skinny<1, GATED, skinny_p<FP8>(), FP8>(a, smem, g, row_begin, M,
                                                            mt * BM_SMALL, ncol0, k0, nk, rot,
                                                            outp);
  }
  else if (GATED || !narrow)
    gemm_bf16_tile_stream<2, GATED, STREAM_P2, FP8>(a, smem, g, row_begin, M, mt * BM_SMALL, ncol0,
                                               k0, nk, rot, outp);
  else if constexpr (!GATED)
    gemm_bf16_tile_stream<1, GATED, STREAM_P1, FP8>(a, smem, g, row_begin, M, mt * BM_SMALL, ncol0,
                                               k0, nk, rot, outp);
}

// Persistent kernel over the work units in table order (group, n-tile, m-tile), dealt to
// the 8 XCDs (blocks are dispatched to XCDs round-robin) in windows of 32 consecutive
// units, so that the m-tiles sharing a weight tile run at the same time on one L2.
// Down GEMM with the dynamic order: when the units leave a last round at most half full
// (r = units mod grid, 0 < 2 r <= grid), the last r units are cut into 2 r column halves,
// so that the last round has work for more blocks and ends about half a unit earlier.
// Without counters block b takes unit 32 (8 r + b % 8) + b / 8 of round r (grid of 256).
// With counters (a.ctr, 8 ints, zero at launch) each block takes its XCD's next unit
// when it is free, so blocks that drew cheap tiles (a group's 64- or 128-row remainder)
// take more, and an XCD that runs out helps the others.
template <bool GATED, bool FP8>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmArgs a) {
  extern __shared__ __align__(16) bf16_t smem[];
  __shared__ int tiles[kMaxExperts + 2];
  __shared__ long long next_unit;
  const int N = a.N, narrow = a.narrow_small;
  auto tile_count = [N, narrow](int M) {
    const bool sm = small_group<GATED>(M);
    const int bm = sm ? BM_SMALL : BM_BIG, bn = tile_cols<GATED>(sm, narrow);
    return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  };
  build_tile_table(a, tile_count, tiles);   // ends with a barrier
  const int64_t ntile = tiles[a.G];
  const int64_t whole = ntile;               // work units: the tiles
  int64_t split0 = whole;                    // first unit cut in column halves
  if (!GATED && a.ctr != nullptr) {
    const int64_t r = whole % gridDim.x;
    if (r > 0 && 2 * r <= (int64_t)gridDim.x) split0 = whole - r;
  }
  const int64_t total = split0 + 2 * (whole - split0);
  const int x = blockIdx.x & 7;
  if (a.ctr == nullptr) {
    const int per = gridDim.x >> 3;
    for (int64_t unit = (int64_t)x * per + (blockIdx.x >> 3); unit < total; unit += gridDim.x)
      gemm_bf16_unit<GATED, FP8>(a, smem, tiles, ntile, unit, split0);
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
    gemm_bf16_unit<GATED, FP8>(a, smem, tiles, ntile, unit, split0);
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

static int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

template <bool GATED, bool FP8>
static hipError_t run_bf16(const GemmArgs& a, int64_t max_tiles, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_kernel<GATED, FP8>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)KERNEL_LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
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
  const int64_t mt = max_m_tiles(d, rows, BM_SMALL) * ceil_div(d.d_model, 128);
  if (!bf) return run_f32<false>(a, max_m_tiles(d, rows, 64), s);
  return ew.fp8 ? run_bf16<false, true>(a, mt, s) : run_bf16<false, false>(a, mt, s);
}

}  // namespace moe
