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
// contiguous, rows padded by 16 bytes against bank conflicts); the next tile's 16-byte
// row pieces are loaded into registers while the MFMAs run on the current one.  Row
// and column indices past M / N are clamped for the loads and masked at the store.
#include <hip/hip_runtime.h>

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

struct LinArgs {
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* w;
  int64_t ldw;
  const float* g;  // RMSNorm gain [K] (NORM)
  float eps;
  const uint16_t* r;  // residual [M][ldr] (RES)
  int64_t ldr;
  uint16_t* y;
  int64_t ldy;
  int64_t M;
  int N, K;
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

// RMSNorm bookkeeping of one K-tile: the rows' squares (unscaled) go into ss, and the
// x pieces become x * g[k] rounded to the bf16 operand.
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

// One K-tile's 16-byte row pieces of x and w into registers (tile kt; the pieces'
// offsets are relative to the block's first rows).
template <int AV, int BV>
__device__ __forceinline__ void load_tile(u32x4 (&ra)[AV], u32x4 (&rb)[BV], const uint16_t* xb,
                                          const uint32_t (&xo)[AV], const uint16_t* wb,
                                          const uint32_t (&wo)[BV], int kt) {
  const uint32_t kb = static_cast<uint32_t>(kt * kBK * 2);
#pragma unroll
  for (int i = 0; i < AV; ++i) ra[i] = *reinterpret_cast<const u32x4*>(byte_off(xb, xo[i] + kb));
#pragma unroll
  for (int i = 0; i < BV; ++i) rb[i] = *reinterpret_cast<const u32x4*>(byte_off(wb, wo[i] + kb));
}

// The pieces into the LDS tiles: piece i of this thread at row lrow + 32 i.
template <int AV, int BV>
__device__ __forceinline__ void store_tile(const u32x4 (&ra)[AV], const u32x4 (&rb)[BV], uint16_t* sA,
                                           uint16_t* sB, int off) {
  constexpr int kStep = (kLinThreads / 8) * kLd;
#pragma unroll
  for (int i = 0; i < AV; ++i) *reinterpret_cast<u32x4*>(sA + off + kStep * i) = ra[i];
#pragma unroll
  for (int i = 0; i < BV; ++i) *reinterpret_cast<u32x4*>(sB + off + kStep * i) = rb[i];
}

// The MFMAs of one staged K-tile: the wave's TM x TN tiles of 16 x 16 at (wm, wn).
template <int TM, int TN>
__device__ __forceinline__ void mma_tile(f32x4 (&acc)[TM][TN], const uint16_t* sA, const uint16_t* sB,
                                         int wm, int wn, int r, int kg) {
#pragma unroll
  for (int kk = 0; kk < kBK; kk += 32) {
    bf16x8 af[TM], bfr[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = frag<uint16_t, true>::get(sA, kLd, wm + 16 * i + r, kk + 8 * kg);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[j] = frag<uint16_t, true>::get(sB, kLd, wn + 16 * j + r, kk + 8 * kg);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma_step(af[i], bfr[j], acc[i][j]);
  }
}

template <int BM, int BN, bool NORM, bool RES>
__global__ void __launch_bounds__(kLinThreads) __attribute__((amdgpu_waves_per_eu(SSD_LINEAR_WAVES, SSD_LINEAR_WAVES)))
linear_kernel(LinArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;   // wave sub-block
  constexpr int TM = WM / 16, TN = WN / 16;  // MFMA tiles per wave
  constexpr int AV = BM * 8 / kLinThreads;   // 16-byte A pieces per thread per K-tile
  constexpr int BV = BN * 8 / kLinThreads;
  constexpr int kRowsPerPass = kLinThreads / 8;  // rows one pass of the block covers
  // operand tiles during the K loop; the bf16 output block afterwards
  constexpr int kOpElems = (BM + BN) * kLd;
  constexpr int kOutElems = BM * (BN + 8);
  __shared__ __align__(16) uint16_t smem[kOpElems > kOutElems ? kOpElems : kOutElems];
  __shared__ float s_rstd[BM];
  uint16_t* sA = smem;
  uint16_t* sB = smem + BM * kLd;

  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t lid = xcd_remap(blockIdx.x, a.tiles);
  const int64_t m0 = (lid / a.tiles_n) * BM;
  const int n0 = static_cast<int>(lid % a.tiles_n) * BN;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;

  // loader: piece (row = tid / 8 + 32 i, k = 8 (tid % 8)) of each tile, addressed as
  // the block's first row (uniform) plus a 32-bit byte offset per piece; rows past M
  // or N are clamped to the last one
  const int lrow = tid >> 3, lk = 8 * (tid & 7);
  const uint16_t* xb = a.x + m0 * a.ldx;
  const uint16_t* wb = a.w + static_cast<int64_t>(n0) * a.ldw;
  uint32_t xo[AV], wo[BV];
#pragma unroll
  for (int i = 0; i < AV; ++i) {
    int64_t m = m0 + lrow + kRowsPerPass * i;
    m = (m < a.M ? m : a.M - 1) - m0;
    xo[i] = static_cast<uint32_t>((m * a.ldx + lk) * 2);
  }
#pragma unroll
  for (int i = 0; i < BV; ++i) {
    int n = n0 + lrow + kRowsPerPass * i;
    n = (n < a.N ? n : a.N - 1) - n0;
    wo[i] = static_cast<uint32_t>((static_cast<int64_t>(n) * a.ldw + lk) * 2);
  }

  float ss[AV];
#pragma unroll
  for (int i = 0; i < AV; ++i) ss[i] = 0.f;
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lane = tid & 63, r = lane & 15, kg = lane >> 4;
  const int nk = a.K / kBK;

  // one K-tile: norm bookkeeping, stage to LDS, refill the registers with the tile two
  // ahead (clamped to the last: no branch), then the MFMAs on the staged tile
#define SSD_LINEAR_STEP(ra, rb, kt)                                                              \
  do {                                                                                           \
    if constexpr (NORM) norm_pieces<AV>(ra, ss, a.g + (kt) * kBK + lk);                         \
    __syncthreads(); /* every wave is done reading the previous tile */                         \
    store_tile<AV, BV>(ra, rb, sA, sB, lrow * kLd + lk);                                        \
    __syncthreads();                                                                             \
    load_tile<AV, BV>(ra, rb, xb, xo, wb, wo, (kt) + 2 < nk ? (kt) + 2 : nk - 1);               \
    mma_tile<TM, TN>(acc, sA, sB, wm, wn, r, kg);                                                \
  } while (0)

  // two tiles in flight: buffer 0 holds even tiles, buffer 1 odd ones
  u32x4 a0[AV], b0[BV], a1[AV], b1[BV];
  load_tile<AV, BV>(a0, b0, xb, xo, wb, wo, 0);
  load_tile<AV, BV>(a1, b1, xb, xo, wb, wo, nk > 1 ? 1 : 0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    SSD_LINEAR_STEP(a0, b0, kt);
    SSD_LINEAR_STEP(a1, b1, kt + 1);
  }
  if (kt < nk) SSD_LINEAR_STEP(a0, b0, kt);
#undef SSD_LINEAR_STEP

  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const float t = sum8(ss[i]);
      if ((tid & 7) == 0) s_rstd[lrow + kRowsPerPass * i] = rsqrtf(t / static_cast<float>(a.K) + a.eps);
    }
  }
  __syncthreads();  // operand tiles dead; s_rstd complete

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
          int gn = n0 + col;
          gn = gn < a.N ? gn : a.N - 1;
          v += bf2f(a.r[gm * a.ldr + gn]);
        }
        sC[row * kOutLd + col] = f2bf(v);
      }
    }
  }
  __syncthreads();
  constexpr int kPieces = BM * BN / 8;
#pragma unroll
  for (int q = 0; q < kPieces / kLinThreads; ++q) {
    const int p = tid + kLinThreads * q;
    const int row = p / (BN / 8), c8 = 8 * (p % (BN / 8));
    const int64_t gm = m0 + row;
    const int gn = n0 + c8;
    if (gm < a.M && gn < a.N)
      *reinterpret_cast<u32x4*>(a.y + gm * a.ldy + gn) =
          *reinterpret_cast<const u32x4*>(sC + row * kOutLd + c8);
  }
}

template <int BM, int BN, bool NORM, bool RES>
hipError_t launch_linear_t(const LinArgs& a0, hipStream_t s) {
  LinArgs a = a0;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.tiles = ((a.M + BM - 1) / BM) * a.tiles_n;
  hipLaunchKernelGGL((linear_kernel<BM, BN, NORM, RES>), dim3(static_cast<unsigned>(a.tiles)),
                     dim3(kLinThreads), 0, s, a);
  return hipGetLastError();
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
  a.y = static_cast<uint16_t*>(lp.y);
  a.ldy = lp.ldy;
  a.M = lp.M;
  a.N = static_cast<int>(lp.N);
  a.K = static_cast<int>(lp.K);
  TimingScope ts(kKLinear, s);
  const bool norm = lp.norm_w != nullptr, res = lp.residual != nullptr;
  constexpr int BM = SSD_LINEAR_BM, BN = SSD_LINEAR_BN;
  if (norm && res) return launch_linear_t<BM, BN, true, true>(a, s);
  if (norm) return launch_linear_t<BM, BN, true, false>(a, s);
  if (res) return launch_linear_t<BM, BN, false, true>(a, s);
  return launch_linear_t<BM, BN, false, false>(a, s);
}

}  // namespace ssd
