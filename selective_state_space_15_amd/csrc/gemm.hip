// Linear layers of the Mamba-2 mixer on gfx950: y = x W^T (+ residual), bf16 in and
// out, fp32 accumulation on MFMA, with an optional RMSNorm of each x row folded into
// the operand load.
//
// The mixer around the hot path is in_proj -> conv1d + SiLU -> SSD -> SiLU(z) gate ->
// out_proj (the Mamba-2 block the Video-Ma2mba model card's architecture diagram and
// the arXiv index page's "Builds on" list name); the full block adds an RMSNorm before
// in_proj, a gated RMSNorm before out_proj and the residual.  Those are exactly the
// two options here:
//   norm:     x_row <- x_row * rsqrt(mean_k x_row[k]^2 + eps) * g[k]   (over the K
//             entries the product reduces over, so the norm is computed while the
//             workgroup streams the row block anyway)
//   residual: y <- y + r   (added in fp32 before the one rounding to bf16)
//
// Shape of the work: one workgroup of 4 waves computes a BM x BN block of y; the waves
// form a 2 x 2 grid of WM x WN sub-blocks of 16 x 16 MFMA tiles
// (v_mfma_f32_16x16x32_bf16).  Each K-tile of 64 is staged in LDS row-major (K
// contiguous, rows padded by 16 bytes against bank conflicts), in two buffers so that a
// tile is staged while the other is read; the 16-byte row pieces of the tile two ahead
// are loaded into registers while the MFMAs run on the current one.  Row
// and column indices past M / N are clamped for the loads and masked at the store.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace ssd {
namespace {

constexpr int kBK = 64;               // K per LDS tile
constexpr int kLd = kBK + 8;          // LDS row stride (elements): 144 bytes
constexpr int kLinThreads = 256;
// 16-byte pieces as a native vector (HIP's uint4 struct is copied through private
// memory when an array of it is loaded from global memory)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// block tile of y per workgroup (compile-time; 128 x 128 unless built otherwise)
#ifndef SSD_LINEAR_BM
#define SSD_LINEAR_BM 128
#endif
#ifndef SSD_LINEAR_BN
#define SSD_LINEAR_BN 128
#endif
// waves per SIMD the register budget is sized for
#ifndef SSD_LINEAR_WAVES
#define SSD_LINEAR_WAVES 2
#endif
// 256 x 256 blocks for large problems (0: the small blocks everywhere)
#ifndef SSD_LINEAR_BIG
#define SSD_LINEAR_BIG 1
#endif

struct LinArgs {
  const uint16_t* x;  // A operand: [M][ldx] (K contiguous) or, transposed, [K][ldx]
  int64_t ldx;
  const uint16_t* w;  // B operand: [N][ldw] (K contiguous) or, transposed, [K][ldw]
  int64_t ldw;
  const float* g;  // RMSNorm gain [K] (NORM)
  float eps;
  const uint16_t* r;  // residual [M][ldr] (RES)
  int64_t ldr;
  void* y;            // [M][ldy]: bf16, or fp32 (OF32)
  int64_t ldy;
  int64_t M, K;
  int N;
  int accumulate;     // OF32: y += product
  int tiles_n;
  int64_t tiles;
};

// Sum over the 8 consecutive lanes 8q .. 8q+7, in each of them.
__device__ __forceinline__ float sum8(float v) {
  v += dpp_f<kDppQuad1032>(0.f, v);
  v += dpp_f<kDppQuad2301>(0.f, v);
  v += dpp_f<kDppRowHalfMirror>(0.f, v);
  return v;
}

// LDS tile of one operand for one K-tile of 64: K-contiguous operands are staged as
// [rows][64 + 8], transposed ones (stored [K][rows] in memory) as [64][rows + 8]; the
// MFMA fragments of the latter are read with the gfx950 LDS transpose loads.
template <int ROWS, bool TR, int NT = kLinThreads>
struct OpTile {
  static constexpr int ld = TR ? ROWS + 8 : kLd;
  static constexpr int elems = TR ? kBK * ld : ROWS * kLd;
  static constexpr int pieces = ROWS * kBK / 8 / NT;  // 16-byte pieces per thread
  static_assert(pieces * 8 * NT == ROWS * kBK, "the tile splits evenly over the threads");
  // piece i of thread t: (row, k) of the tile it covers
  __device__ static __forceinline__ int row(int t, int i) {
    return TR ? 8 * ((t + NT * i) % (ROWS / 8)) : (t + NT * i) / 8;
  }
  __device__ static __forceinline__ int kk(int t, int i) {
    return TR ? (t + NT * i) / (ROWS / 8) : 8 * ((t + NT * i) % 8);
  }
  __device__ static __forceinline__ int lds_off(int t, int i) {
    return TR ? kk(t, i) * ld + row(t, i) : row(t, i) * kLd + kk(t, i);
  }
};

// One K-tile's pieces of an operand into registers.  rows: the block's first row r0
// and the operand's row count R (rows past it are clamped: their products land in
// masked outputs); K-tile k0 of K (reduction entries past K read as zero).
template <int ROWS, bool TR, bool RAG, int NT, int NP>
__device__ __forceinline__ void load_op(u32x4 (&v)[NP], uint32_t& keep, const uint16_t* base,
                                        int64_t ld, int64_t r0, int64_t R, int64_t k0, int64_t K) {
  using OT = OpTile<ROWS, TR, NT>;
  const int t = threadIdx.x;
  keep = 0;
  if constexpr (TR) {
    const uint16_t* tb = base + k0 * ld + r0;  // uniform
#pragma unroll
    for (int i = 0; i < OT::pieces; ++i) {
      const int64_t rr = r0 + OT::row(t, i);
      const int cr = static_cast<int>((rr + 8 <= R ? rr : R - 8) - r0);
      const int kr = OT::kk(t, i);
      const bool kin = !RAG || k0 + kr < K;
      const int kc = kin ? kr : static_cast<int>(K - 1 - k0);
      v[i] = *reinterpret_cast<const u32x4*>(
          byte_off(tb, static_cast<uint32_t>((static_cast<int64_t>(kc) * ld + cr) * 2)));
      keep |= (kin ? 1u : 0u) << i;
    }
  } else {
    const uint16_t* tb = base + r0 * ld + k0;  // uniform
#pragma unroll
    for (int i = 0; i < OT::pieces; ++i) {
      const int64_t rr = r0 + OT::row(t, i);
      const int cr = static_cast<int>((rr < R ? rr : R - 1) - r0);
      // a ragged K (a multiple of 8) ends inside the last tile: pieces past it read the
      // last valid piece and are zeroed
      const int kr = OT::kk(t, i);
      const bool kin = !RAG || k0 + kr < K;
      const int kc = kin ? kr : static_cast<int>(K - 8 - k0);
      v[i] = *reinterpret_cast<const u32x4*>(
          byte_off(tb, static_cast<uint32_t>((static_cast<int64_t>(cr) * ld + kc) * 2)));
      keep |= (kin ? 1u : 0u) << i;
    }
  }
}

// The pieces into the LDS tile; pieces past K (clear bits of keep) become zeros here,
// where the values are consumed, not right after their loads.
template <int ROWS, bool TR, bool RAG, int NT, int NP>
__device__ __forceinline__ void store_op(const u32x4 (&v)[NP], uint32_t keep, uint16_t* s) {
  using OT = OpTile<ROWS, TR, NT>;
#pragma unroll
  for (int i = 0; i < OT::pieces; ++i) {
    const bool k = !RAG || ((keep >> i) & 1u);
    *reinterpret_cast<u32x4*>(s + OT::lds_off(threadIdx.x, i)) =
        u32x4{k ? v[i].x : 0u, k ? v[i].y : 0u, k ? v[i].z : 0u, k ? v[i].w : 0u};
  }
}

// RMSNorm bookkeeping of one K-tile (K-contiguous x only): the rows' squares
// (unscaled) go into ss, and the x pieces become x * g[k] rounded to the bf16 operand.
template <int AV>
__device__ __forceinline__ void norm_pieces(u32x4 (&ra)[AV], float (&ss)[AV], const float* gp) {
  const float4 g0 = *reinterpret_cast<const float4*>(gp);
  const float4 g1 = *reinterpret_cast<const float4*>(gp + 4);
  const float gk[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
  for (int i = 0; i < AV; ++i) {
    const uint32_t wd[4] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float v0 = __uint_as_float(wd[q] << 16), v1 = __uint_as_float(wd[q] & 0xffff0000u);
      ss[i] += v0 * v0 + v1 * v1;
      o[q] = f2bf2(v0 * gk[2 * q], v1 * gk[2 * q + 1]);
    }
    ra[i] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

// The MFMAs of one staged K-tile: the wave's TM x TN tiles of 16 x 16 at (wm, wn).
template <int TM, int TN, int BM, int BN, bool TA, bool TB>
__device__ __forceinline__ void mma_tile(f32x4 (&acc)[TM][TN], const uint16_t* sA, const uint16_t* sB,
                                         int wm, int wn, int r, int kg) {
#pragma unroll
  for (int kk = 0; kk < kBK; kk += 32) {
    bf16x8 af[TM], bfr[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af[i] = frag<uint16_t, !TA>::get(sA, OpTile<BM, TA>::ld, wm + 16 * i + r, kk + 8 * kg);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bfr[j] = frag<uint16_t, !TB>::get(sB, OpTile<BN, TB>::ld, wn + 16 * j + r, kk + 8 * kg);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma_step(af[i], bfr[j], acc[i][j]);
  }
}

// Launch shapes: block tile BM x BN computed by a WGM x WGN grid of waves, WPS waves per
// SIMD of register budget, and DEPTH K-tiles loaded ahead into registers.
// RAG: a ragged K (not whole K-tiles) is supported.
template <int BM_, int BN_, int WGM_, int WGN_, int WPS_, int DEPTH_, bool RAG_>
struct LinShape {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, WPS = WPS_, DEPTH = DEPTH_;
  static constexpr bool rag = RAG_;
  static constexpr int threads = 64 * WGM * WGN;
};
// 128 x 128 blocks of 4 waves (two workgroups per CU), two K-tiles ahead
using LinSmall = LinShape<SSD_LINEAR_BM, SSD_LINEAR_BN, 2, 2, SSD_LINEAR_WAVES, 2, true>;
// 256 x 256 blocks of 8 waves with 128 x 64 wave tiles (one workgroup per CU, 147 KB of
// double-buffered LDS), one K-tile ahead: 2.7 times fewer LDS bytes per flop than the
// 64 x 64 wave tiles, for problems with enough blocks to fill the GPU
using LinBig = LinShape<256, 256, 2, 4, 2, 1, true>;

template <typename S, bool TA, bool TB, bool NORM, bool RES, bool OF32, bool RAG>
__global__ void __launch_bounds__(S::threads) __attribute__((amdgpu_waves_per_eu(S::WPS, S::WPS)))
linear_kernel(LinArgs a) {
  static_assert(!(NORM && TA), "the norm prologue needs K-contiguous rows");
  static_assert(!(NORM && RAG), "the norm prologue needs whole K-tiles");
  constexpr int BM = S::BM, BN = S::BN, NT = S::threads;
  constexpr int WM = BM / S::WGM, WN = BN / S::WGN;  // wave sub-block
  constexpr int TM = WM / 16, TN = WN / 16;            // MFMA tiles per wave
  using OA = OpTile<BM, TA, NT>;
  using OB = OpTile<BN, TB, NT>;
  constexpr int AV = OA::pieces, BV = OB::pieces;
  // operand tiles during the K loop, double-buffered (even K-tiles in buffer 0, odd in
  // buffer 1: a tile is staged while the waves may still read the other, one barrier per
  // K-tile); the bf16 output block afterwards
  constexpr int kOpElems = 2 * (OA::elems + OB::elems);
  constexpr int kOutElems = OF32 ? 8 : BM * (BN + 8);
  __shared__ __align__(16) uint16_t smem[kOpElems > kOutElems ? kOpElems : kOutElems];
  __shared__ float s_rstd[NORM ? BM : 1];
  uint16_t* const sA0 = smem;
  uint16_t* const sB0 = smem + OA::elems;
  uint16_t* const sA1 = smem + OA::elems + OB::elems;
  uint16_t* const sB1 = sA1 + OA::elems;

  const int tid = threadIdx.x, wave = tid >> 6;
  // Tile order: consecutive logical ids run on one XCD (xcd_remap); they walk groups of
  // kGroupM row blocks, all column blocks of a group, row block fastest -- so the row
  // blocks of a group and each column block stay in that XCD's L2 while they are reused
  // (row block first would stream every column block of w through L2 once per row block).
  constexpr int64_t kGroupM = 8;
  const int64_t lid = xcd_remap(blockIdx.x, a.tiles);
  const int64_t tiles_m = a.tiles / a.tiles_n;
  const int64_t grp = lid / (kGroupM * a.tiles_n), in_grp = lid % (kGroupM * a.tiles_n);
  const int64_t gm_rows = tiles_m - grp * kGroupM < kGroupM ? tiles_m - grp * kGroupM : kGroupM;
  const int64_t m0 = (grp * kGroupM + in_grp % gm_rows) * BM;
  const int64_t n0 = (in_grp / gm_rows) * BN;
  const int wm = (wave / S::WGN) * WM, wn = (wave % S::WGN) * WN;

  float ss[AV];
#pragma unroll
  for (int i = 0; i < AV; ++i) ss[i] = 0.f;
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lane = tid & 63, r = lane & 15, kg = lane >> 4;
  const int64_t nk = (a.K + kBK - 1) / kBK;

  // One K-tile: norm bookkeeping, stage to its LDS buffer, one barrier (the tile is
  // visible, and every wave is past the MFMAs of the tile two back, which used this
  // buffer), refill the registers with the tile two ahead (clamped to the last: no
  // branch), then the MFMAs on the staged tile.
#define SSD_LINEAR_STEPR(ra, rb, ka, kb, kt, sA, sB, R, NKT)                                     \
  do {                                                                                           \
    if constexpr (NORM) norm_pieces<AV>(ra, ss, a.g + (kt) * kBK + OA::kk(tid, 0));              \
    store_op<BM, TA, R, NT>(ra, ka, sA);                                                         \
    store_op<BN, TB, R, NT>(rb, kb, sB);                                                         \
    __syncthreads();                                                                             \
    const int64_t kn_ = (kt) + S::DEPTH < (NKT) ? (kt) + S::DEPTH : (NKT) - 1;                  \
    load_op<BM, TA, R, NT>(ra, ka, a.x, a.ldx, m0, a.M, kn_ * kBK, a.K);                         \
    load_op<BN, TB, R, NT>(rb, kb, a.w, a.ldw, n0, a.N, kn_ * kBK, a.K);                         \
    mma_tile<TM, TN, BM, BN, TA, TB>(acc, sA, sB, wm, wn, r, kg);                                \
  } while (0)
#define SSD_LINEAR_STEP(ra, rb, ka, kb, kt, sA, sB) SSD_LINEAR_STEPR(ra, rb, ka, kb, kt, sA, sB, RAG, nk)

  int64_t kt = 0;
  if constexpr (S::DEPTH == 2) {
    // two tiles in flight: register set 0 holds even tiles, set 1 odd ones
    u32x4 a0[AV], b0[BV], a1[AV], b1[BV];
    uint32_t ka0, kb0, ka1, kb1;
    load_op<BM, TA, RAG, NT>(a0, ka0, a.x, a.ldx, m0, a.M, 0, a.K);
    load_op<BN, TB, RAG, NT>(b0, kb0, a.w, a.ldw, n0, a.N, 0, a.K);
    load_op<BM, TA, RAG, NT>(a1, ka1, a.x, a.ldx, m0, a.M, (nk > 1 ? 1 : 0) * kBK, a.K);
    load_op<BN, TB, RAG, NT>(b1, kb1, a.w, a.ldw, n0, a.N, (nk > 1 ? 1 : 0) * kBK, a.K);
    for (; kt + 1 < nk; kt += 2) {
      SSD_LINEAR_STEP(a0, b0, ka0, kb0, kt, sA0, sB0);
      SSD_LINEAR_STEP(a1, b1, ka1, kb1, kt + 1, sA1, sB1);
    }
    if (kt < nk) SSD_LINEAR_STEP(a0, b0, ka0, kb0, kt, sA0, sB0);
  } else if constexpr (!RAG) {
    // one tile in flight; the LDS buffers still alternate
    u32x4 a0[AV], b0[BV];
    uint32_t ka0, kb0;
    load_op<BM, TA, false, NT>(a0, ka0, a.x, a.ldx, m0, a.M, 0, a.K);
    load_op<BN, TB, false, NT>(b0, kb0, a.w, a.ldw, n0, a.N, 0, a.K);
    for (; kt + 1 < nk; kt += 2) {
      SSD_LINEAR_STEP(a0, b0, ka0, kb0, kt, sA0, sB0);
      SSD_LINEAR_STEP(a0, b0, ka0, kb0, kt + 1, sA1, sB1);
    }
    if (kt < nk) SSD_LINEAR_STEP(a0, b0, ka0, kb0, kt, sA0, sB0);
  } else {
    // ragged K, one tile in flight: every K-tile but the last is whole, so the loop runs
    // over those with the whole-tile loads and stores (the masked forms do not fit these
    // blocks' registers), and the last tile is loaded, masked and multiplied after it.
    u32x4 a0[AV], b0[BV];
    uint32_t ka0 = 0, kb0 = 0;
    const int64_t nw = nk - 1;  // whole K-tiles
    if (nw > 0) {
      load_op<BM, TA, false, NT>(a0, ka0, a.x, a.ldx, m0, a.M, 0, a.K);
      load_op<BN, TB, false, NT>(b0, kb0, a.w, a.ldw, n0, a.N, 0, a.K);
      for (; kt + 1 < nw; kt += 2) {
        SSD_LINEAR_STEPR(a0, b0, ka0, kb0, kt, sA0, sB0, false, nw);
        SSD_LINEAR_STEPR(a0, b0, ka0, kb0, kt + 1, sA1, sB1, false, nw);
      }
      if (kt < nw) SSD_LINEAR_STEPR(a0, b0, ka0, kb0, kt, sA0, sB0, false, nw);
    }
    load_op<BM, TA, true, NT>(a0, ka0, a.x, a.ldx, m0, a.M, nw * kBK, a.K);
    load_op<BN, TB, true, NT>(b0, kb0, a.w, a.ldw, n0, a.N, nw * kBK, a.K);
    __syncthreads();  // every wave is past the MFMAs that read buffer 0
    store_op<BM, TA, true, NT>(a0, ka0, sA0);
    store_op<BN, TB, true, NT>(b0, kb0, sB0);
    __syncthreads();
    mma_tile<TM, TN, BM, BN, TA, TB>(acc, sA0, sB0, wm, wn, r, kg);
  }
#undef SSD_LINEAR_STEP
#undef SSD_LINEAR_STEPR

  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const float t = sum8(ss[i]);
      if ((tid & 7) == 0) s_rstd[OA::row(tid, i)] = rsqrtf(t / static_cast<float>(a.K) + a.eps);
    }
  }
  __syncthreads();  // operand tiles dead; s_rstd complete

  if constexpr (OF32) {
    // fp32 result (weight gradients), optionally added to what y holds
    float* y = static_cast<float*>(a.y);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t gm = m0 + wm + 16 * i + 4 * kg + e;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int64_t gn = n0 + wn + 16 * j + r;
          if (gm < a.M && gn < a.N) {
            float* p = y + gm * a.ldy + gn;
            *p = a.accumulate ? *p + acc[i][j][e] : acc[i][j][e];
          }
        }
      }
    return;
  } else {
    // stage the block as bf16 rows in LDS (after the norm scale and the residual, in
    // fp32), then store 16-byte row pieces
    constexpr int kOutLd = BN + 8;
    uint16_t* sC = smem;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = wm + 16 * i + 4 * kg + e;
        const float sc = NORM ? s_rstd[row] : 1.f;
        int64_t gm = m0 + row;
        gm = gm < a.M ? gm : a.M - 1;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = wn + 16 * j + r;
          float v = acc[i][j][e] * sc;
          if constexpr (RES) {
            int64_t gn = n0 + col;
            gn = gn < a.N ? gn : a.N - 1;
            v += bf2f(a.r[gm * a.ldr + gn]);
          }
          sC[row * kOutLd + col] = f2bf(v);
        }
      }
    }
    __syncthreads();
    uint16_t* y = static_cast<uint16_t*>(a.y);
    constexpr int kPieces = BM * BN / 8;
#pragma unroll
    for (int q = 0; q < kPieces / NT; ++q) {
      const int p = tid + NT * q;
      const int row = p / (BN / 8), c8 = 8 * (p % (BN / 8));
      const int64_t gm = m0 + row;
      const int64_t gn = n0 + c8;
      if (gm < a.M && gn < a.N)
        *reinterpret_cast<u32x4*>(y + gm * a.ldy + gn) = *reinterpret_cast<const u32x4*>(sC + row * kOutLd + c8);
    }
  }
}

template <typename S, bool TA, bool TB, bool NORM, bool RES, bool OF32>
hipError_t launch_linear_s(const LinArgs& a0, hipStream_t s) {
  LinArgs a = a0;
  a.tiles_n = static_cast<int>((a.N + S::BN - 1) / S::BN);
  a.tiles = ((a.M + S::BM - 1) / S::BM) * a.tiles_n;
  const dim3 grid(static_cast<unsigned>(a.tiles)), block(S::threads);
  if (a.K % kBK == 0)
    hipLaunchKernelGGL((linear_kernel<S, TA, TB, NORM, RES, OF32, false>), grid, block, 0, s, a);
  else if constexpr (!NORM && S::rag)
    hipLaunchKernelGGL((linear_kernel<S, TA, TB, NORM, RES, OF32, true>), grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// The big blocks where they make at least four full waves of workgroups (one per CU), or
// half a wave for long K, no operand is smaller than a block and there is no norm
// prologue (it does not fit the big blocks' registers); the small ones otherwise.
template <bool TA, bool TB, bool NORM, bool RES, bool OF32>
hipError_t launch_linear_t(const LinArgs& a, hipStream_t s) {
  if constexpr (!NORM) {
    const int64_t big_tiles = ((a.M + 255) / 256) * ((a.N + 255) / 256);
    // long K (the weight gradients over a whole batch of tokens): a block's work is long
    // enough that half the CUs with big blocks beat the small ones (65,536 tokens: 650 ->
    // 930 TFLOP/s at 200 and 420 blocks)
    const bool enough = big_tiles >= 4 * 256 || (a.K >= 16384 && big_tiles >= 128);
    if (SSD_LINEAR_BIG && a.M >= 256 && a.N >= 256 && enough)
      return launch_linear_s<LinBig, TA, TB, NORM, RES, OF32>(a, s);
  }
  return launch_linear_s<LinSmall, TA, TB, NORM, RES, OF32>(a, s);
}

}  // namespace

hipError_t launch_linear(const LinearProblem& lp, hipStream_t s) {
  LinArgs a{};
  a.x = static_cast<const uint16_t*>(lp.x);
  a.ldx = lp.ldx;
  a.w = static_cast<const uint16_t*>(lp.w);
  a.ldw = lp.ldw;
  a.g = lp.norm_w;
  a.eps = lp.eps;
  a.r = static_cast<const uint16_t*>(lp.residual);
  a.ldr = lp.ldr;
  a.y = lp.y;
  a.ldy = lp.ldy;
  a.M = lp.M;
  a.N = static_cast<int>(lp.N);
  a.K = lp.K;
  TimingScope ts(kKLinear, s);
  const bool norm = lp.norm_w != nullptr, res = lp.residual != nullptr;
  if (norm && res) return launch_linear_t<false, false, true, true, false>(a, s);
  if (norm) return launch_linear_t<false, false, true, false, false>(a, s);
  if (res) return launch_linear_t<false, false, false, true, false>(a, s);
  return launch_linear_t<false, false, false, false, false>(a, s);
}

// dx[M][K] = dy[M][N] w[N][K]  (the input gradient of y = x w^T)
hipError_t launch_linear_dgrad(int64_t M, int64_t N, int64_t K, const void* dy, int64_t lddy,
                               const void* w, int64_t ldw, void* dx, int64_t lddx, hipStream_t s) {
  LinArgs a{};
  a.x = static_cast<const uint16_t*>(dy);  // A = dy, reduction over N (contiguous)
  a.ldx = lddy;
  a.w = static_cast<const uint16_t*>(w);   // B[k][n] = w[n][k]: stored [N][K], transposed
  a.ldw = ldw;
  a.y = dx;
  a.ldy = lddx;
  a.M = M;
  a.N = static_cast<int>(K);
  a.K = N;
  TimingScope ts(kKLinear, s);
  return launch_linear_t<false, true, false, false, false>(a, s);
}

// dw[N][K] (+)= dy[M][N]^T x[M][K]  (the weight gradient of y = x w^T, fp32)
hipError_t launch_linear_wgrad(int64_t M, int64_t N, int64_t K, const void* dy, int64_t lddy,
                               const void* x, int64_t ldx, float* dw, int64_t lddw, int accumulate,
                               hipStream_t s) {
  LinArgs a{};
  a.x = static_cast<const uint16_t*>(dy);  // A[n][m] = dy[m][n]: stored [M][N], transposed
  a.ldx = lddy;
  a.w = static_cast<const uint16_t*>(x);   // B[k][m] = x[m][k]: stored [M][K], transposed
  a.ldw = ldx;
  a.y = dw;
  a.ldy = lddw;
  a.M = N;
  a.N = static_cast<int>(K);
  a.K = M;
  a.accumulate = accumulate;
  TimingScope ts(kKLinear, s);
  return launch_linear_t<true, true, false, false, true>(a, s);
}

}  // namespace ssd
