// RMSNorm of the full Mamba-2 block on gfx950 (the block the Video-Ma2mba model card
// and the arXiv index page's "Builds on" list name: a norm before in_proj and a gated
// norm -- over the SiLU(z)-gated hot-path output -- before out_proj), forward and
// backward, for rows of bf16 activations:
//
//   forward   r = (mean_k x[k]^2 + eps)^(-1/2),   y[k] = x[k] r g[k]
//   backward  dx[k] = r g[k] dy[k] - x[k] r^3 / K * sum_j g[j] dy[j] x[j]   (+ dres[k])
//             dg[k] = sum over rows of dy[k] x[k] r
//
// One wave per row (16-byte pieces, the row's sums by DPP wave reductions).  dg is a
// column sum over rows: each wave keeps the partial of the rows it visits (a fixed
// grid-stride assignment), the partials go to scratch and an ordered column sum adds
// them, so the result is the same on every run.
#include "common.hpp"
#include "launch.hpp"

namespace ssd {
namespace {

constexpr int kNormThreads = 256;
constexpr int kNormWaves = kNormThreads / kWave;
constexpr int kNormMaxPieces = 10;   // 16-byte pieces per lane: K <= 64 * 8 * 10 = 5120
constexpr int kNormBwdBlocks = 256;  // workgroups of the backward (dg partial rows = 4x this)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void unpack8(const u32x4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __uint_as_float(w[q] << 16);
    f[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  return u32x4{f2bf2(f[0], f[1]), f2bf2(f[2], f[3]), f2bf2(f[4], f[5]), f2bf2(f[6], f[7])};
}

struct NormArgs {
  int64_t M;
  int K;
  const uint16_t* x;
  int64_t ldx;
  const float* g;
  float eps;
  const uint16_t* dy;
  int64_t lddy;
  const uint16_t* dres;
  int64_t ldres;
  uint16_t* out;  // y (forward) or dx (backward)
  int64_t ldo;
  float* rstd;     // forward: [M] or null
  float* dg_part;  // backward: [kNormBwdBlocks * kNormWaves][K]
};

__global__ void __launch_bounds__(kNormThreads) rmsnorm_fwd_kernel(NormArgs a) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t m = blockIdx.x * static_cast<int64_t>(kNormWaves) + wave;
  if (m >= a.M) return;
  const int np = a.K / 8;
  const uint16_t* xr = a.x + m * a.ldx;
  u32x4 v[kNormMaxPieces];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kNormMaxPieces; ++j) {
    const int p = lane + kWave * j;
    if (p < np) {
      v[j] = *reinterpret_cast<const u32x4*>(xr + 8 * p);
      float f[8];
      unpack8(v[j], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
    }
  }
  const float r = rsqrtf(wave_sum(ss) / static_cast<float>(a.K) + a.eps);
  if (a.rstd && lane == 0) a.rstd[m] = r;
  uint16_t* yr = a.out + m * a.ldo;
#pragma unroll
  for (int j = 0; j < kNormMaxPieces; ++j) {
    const int p = lane + kWave * j;
    if (p < np) {
      float f[8];
      unpack8(v[j], f);
      const float4 g0 = *reinterpret_cast<const float4*>(a.g + 8 * p);
      const float4 g1 = *reinterpret_cast<const float4*>(a.g + 8 * p + 4);
      const float gk[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= r * gk[e];
      *reinterpret_cast<u32x4*>(yr + 8 * p) = pack8(f);
    }
  }
}

__global__ void __launch_bounds__(kNormThreads) rmsnorm_bwd_kernel(NormArgs a) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t wid = blockIdx.x * static_cast<int64_t>(kNormWaves) + wave;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * kNormWaves;
  const int np = a.K / 8;
  float dgp[kNormMaxPieces][8];
#pragma unroll
  for (int j = 0; j < kNormMaxPieces; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) dgp[j][e] = 0.f;
  for (int64_t m = wid; m < a.M; m += nw) {
    const uint16_t* xr = a.x + m * a.ldx;
    const uint16_t* dr = a.dy + m * a.lddy;
    u32x4 xv[kNormMaxPieces], dv[kNormMaxPieces];
    float ss = 0.f, s = 0.f;
#pragma unroll
    for (int j = 0; j < kNormMaxPieces; ++j) {
      const int p = lane + kWave * j;
      if (p < np) {
        xv[j] = *reinterpret_cast<const u32x4*>(xr + 8 * p);
        dv[j] = *reinterpret_cast<const u32x4*>(dr + 8 * p);
        float xf[8], df[8];
        unpack8(xv[j], xf);
        unpack8(dv[j], df);
        const float4 g0 = *reinterpret_cast<const float4*>(a.g + 8 * p);
        const float4 g1 = *reinterpret_cast<const float4*>(a.g + 8 * p + 4);
        const float gk[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ss += xf[e] * xf[e];
          s += gk[e] * df[e] * xf[e];
        }
      }
    }
    const float r = rsqrtf(wave_sum(ss) / static_cast<float>(a.K) + a.eps);
    const float c = r * r * r * wave_sum(s) / static_cast<float>(a.K);
    uint16_t* outr = a.out + m * a.ldo;
#pragma unroll
    for (int j = 0; j < kNormMaxPieces; ++j) {
      const int p = lane + kWave * j;
      if (p < np) {
        float xf[8], df[8], rf[8];
        unpack8(xv[j], xf);
        unpack8(dv[j], df);
        if (a.dres) {
          unpack8(*reinterpret_cast<const u32x4*>(a.dres + m * a.ldres + 8 * p), rf);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) rf[e] = 0.f;
        }
        const float4 g0 = *reinterpret_cast<const float4*>(a.g + 8 * p);
        const float4 g1 = *reinterpret_cast<const float4*>(a.g + 8 * p + 4);
        const float gk[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] = r * gk[e] * df[e] - xf[e] * c + rf[e];
          dgp[j][e] += df[e] * xf[e] * r;
        }
        *reinterpret_cast<u32x4*>(outr + 8 * p) = pack8(o);
      }
    }
  }
  float* part = a.dg_part + wid * a.K;
#pragma unroll
  for (int j = 0; j < kNormMaxPieces; ++j) {
    const int p = lane + kWave * j;
    if (p < np) {
      *reinterpret_cast<float4*>(part + 8 * p) = make_float4(dgp[j][0], dgp[j][1], dgp[j][2], dgp[j][3]);
      *reinterpret_cast<float4*>(part + 8 * p + 4) = make_float4(dgp[j][4], dgp[j][5], dgp[j][6], dgp[j][7]);
    }
  }
}

// dg[k] (+)= sum of the partial rows, in row order.
__global__ void __launch_bounds__(256) rmsnorm_dg_kernel(const float* part, int64_t rows, int K, float* dg,
                                                         int accumulate) {
  const float v = block_colsum(part, rows, K);
  const int64_t col = blockIdx.x * static_cast<int64_t>(kWave) + threadIdx.x;
  if (threadIdx.x < kWave && col < K) dg[col] = accumulate ? dg[col] + v : v;
}

}  // namespace

size_t rmsnorm_bwd_workspace_bytes(int64_t K) {
  return static_cast<size_t>(kNormBwdBlocks) * kNormWaves * K * sizeof(float);
}

int rmsnorm_max_k() { return kWave * 8 * kNormMaxPieces; }

hipError_t launch_rmsnorm_fwd(int64_t M, int K, const void* x, int64_t ldx, const float* g, float eps,
                              void* y, int64_t ldy, float* rstd, hipStream_t s) {
  NormArgs a{};
  a.M = M;
  a.K = K;
  a.x = static_cast<const uint16_t*>(x);
  a.ldx = ldx;
  a.g = g;
  a.eps = eps;
  a.out = static_cast<uint16_t*>(y);
  a.ldo = ldy;
  a.rstd = rstd;
  TimingScope ts(kKNorm, s);
  hipLaunchKernelGGL(rmsnorm_fwd_kernel, dim3(static_cast<unsigned>((M + kNormWaves - 1) / kNormWaves)),
                     dim3(kNormThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(int64_t M, int K, const void* x, int64_t ldx, const float* g, float eps,
                              const void* dy, int64_t lddy, const void* dres, int64_t ldres, void* dx,
                              int64_t lddx, float* dg, int accumulate, void* ws, hipStream_t s) {
  NormArgs a{};
  a.M = M;
  a.K = K;
  a.x = static_cast<const uint16_t*>(x);
  a.ldx = ldx;
  a.g = g;
  a.eps = eps;
  a.dy = static_cast<const uint16_t*>(dy);
  a.lddy = lddy;
  a.dres = static_cast<const uint16_t*>(dres);
  a.ldres = ldres;
  a.out = static_cast<uint16_t*>(dx);
  a.ldo = lddx;
  a.dg_part = static_cast<float*>(ws);
  TimingScope ts(kKNorm, s);
  hipLaunchKernelGGL(rmsnorm_bwd_kernel, dim3(kNormBwdBlocks), dim3(kNormThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !dg) return e;
  hipLaunchKernelGGL(rmsnorm_dg_kernel, dim3(static_cast<unsigned>((K + kWave - 1) / kWave)), dim3(256), 0, s,
                     static_cast<const float*>(ws), static_cast<int64_t>(kNormBwdBlocks) * kNormWaves, K, dg,
                     accumulate);
  return hipGetLastError();
}

}  // namespace ssd
