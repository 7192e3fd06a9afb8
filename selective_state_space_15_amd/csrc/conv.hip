// Causal depthwise conv1d (+ bias, optional SiLU) on gfx950, forward and backward.
//
//   pre[t, c] = b[c] + sum_{k<K} w[c, k] * xin[t - K + 1 + k, c],   out = silu(pre) or pre
//   xin[t < 0] = carried conv state (the last K-1 inputs of the previous segment)
//
// This is the Conv1d that the Video-Ma2mba review (pith.science verdict for arXiv
// 2411.19460, skeptic critique) notes precedes the SSD in a Mamba-2 block, which
// is why a sequence checkpoint must carry the conv buffer as well as h.
//
// Forward: one thread per (batch, 16-row tile, 16-byte channel vector); all 19 raw
// rows are loaded up front (independent loads in flight), the taps are applied in
// registers and the 16 output rows are stored as 16-byte vectors.  Adjacent threads
// take adjacent channel vectors, so every row access is coalesced.
//
// Backward: one thread per (batch, 64-row tile, channel vector) walks its rows with
// a sliding register window; dpre = dout * silu'(pre) is recomputed from the raw
// rows, dx[tau] = sum_k dpre[tau + K-1-k] w[k] (plus the gradient of the returned
// conv state for the last K-1 rows), and per-tile partial sums of dw and db go to
// scratch for an ordered reduction (deterministic, no atomics).
#include "common.hpp"
#include "launch.hpp"

namespace ssd {

namespace {

constexpr int kRowsF = 16;  // rows per thread, forward
constexpr int kRowsB = 64;  // rows per thread, backward

struct ConvFwdArgs {
  int64_t B, L;
  int C, K, silu;
  const void* x;
  int64_t x_sb, x_st;
  int x_c0;           // channel offset of the processed range inside x rows
  const void* st;     // carried state rows (null = zeros)
  int64_t st_sb, st_st;
  int st_c0;
  const float* w;     // [C][K] of the processed range
  const float* bias;  // [C] or null
  void* out;
  int64_t o_sb, o_st;
  int o_c0;
};

template <typename IO>
__global__ void __launch_bounds__(256) conv_fwd_kernel(ConvFwdArgs a) {
  using T = io_traits<IO>;
  using E = typename T::elem;
  constexpr int V = T::vec;
  const int ncv = a.C / V;
  const int64_t ntile = (a.L + kRowsF - 1) / kRowsF;
  const int64_t gid = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (gid >= a.B * ntile * ncv) return;
  const int cv = static_cast<int>(gid % ncv);
  const int64_t tile = (gid / ncv) % ntile;
  const int64_t b = gid / (static_cast<int64_t>(ncv) * ntile);
  const int c = cv * V;
  const int K = a.K;
  const int64_t t0 = tile * kRowsF;
  const E* xb = static_cast<const E*>(a.x) + b * a.x_sb + a.x_c0 + c;
  const E* sb = a.st ? static_cast<const E*>(a.st) + b * a.st_sb + a.st_c0 + c : nullptr;

  uint4 in[kRowsF + 3];  // raw rows t0-3 .. t0+15
#pragma unroll
  for (int i = 0; i < kRowsF + 3; ++i) {
    const int64_t t = t0 - 3 + i;
    in[i] = make_uint4(0u, 0u, 0u, 0u);
    if (t >= a.L) {
    } else if (t >= 0) {
      in[i] = *reinterpret_cast<const uint4*>(xb + t * a.x_st);
    } else if (sb && t >= -(K - 1)) {
      in[i] = *reinterpret_cast<const uint4*>(sb + (t + K - 1) * a.st_st);
    }
  }
  float w4[4][V], bias[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    bias[v] = a.bias ? a.bias[c + v] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = j - (4 - K);  // taps right-aligned on 4
      w4[j][v] = kk >= 0 ? a.w[(c + v) * K + kk] : 0.f;
    }
  }
  E* ob = static_cast<E*>(a.out) + b * a.o_sb + a.o_c0 + c;
#pragma unroll
  for (int r = 0; r < kRowsF; ++r) {
    const int64_t t = t0 + r;
    if (t < a.L) {
      float o[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float pre = bias[v];
#pragma unroll
        for (int j = 0; j < 4; ++j) pre = fmaf(w4[j][v], raw_elem<IO>(in[r + j], v), pre);
        o[v] = a.silu ? siluf_(pre) : pre;
      }
      store_vec16<IO>(ob + t * a.o_st, o);
    }
  }
}

}  // namespace

// Conv forward over channels [c0, c0 + C) of the rows of `x`, writing channels
// [o_c0, o_c0 + C) of `out`.  Weights / bias pointers refer to channel c0.
hipError_t launch_conv_fwd_range(int bf16, int64_t B, int64_t L, int C, int K, int silu, View x,
                                 int x_c0, View st, int st_c0, const float* w, const float* bias,
                                 MView out, int o_c0, hipStream_t s) {
  ConvFwdArgs a{};
  a.B = B;
  a.L = L;
  a.C = C;
  a.K = K;
  a.silu = silu;
  a.x = x.p;
  a.x_sb = x.sb;
  a.x_st = x.st;
  a.x_c0 = x_c0;
  a.st = st.p;
  a.st_sb = st.sb;
  a.st_st = st.st;
  a.st_c0 = st_c0;
  a.w = w;
  a.bias = bias;
  a.out = out.p;
  a.o_sb = out.sb;
  a.o_st = out.st;
  a.o_c0 = o_c0;
  const int V = bf16 ? 8 : 4;
  const int64_t n = B * ((L + kRowsF - 1) / kRowsF) * (C / V);
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(conv_fwd_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(conv_fwd_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

size_t bc_prepass_bytes(const Problem& pr) {
  if (pr.K == 0) return 0;
  const size_t n = static_cast<size_t>(pr.B) * pr.L * 2 * pr.G * pr.N * (pr.bf16 ? 2 : 4);
  return (n + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_bc_prepass(const Problem& pr, void* dst, hipStream_t s) {
  const int hp = pr.H * pr.P, gn2 = 2 * pr.G * pr.N;
  const MView out{dst, pr.L * gn2, gn2};
  return launch_conv_fwd_range(pr.bf16, pr.B, pr.L, gn2, pr.K, 1, pr.xbc, hp, pr.cs_in, hp,
                               pr.conv_w + static_cast<int64_t>(hp) * pr.K,
                               pr.conv_b ? pr.conv_b + hp : nullptr, out, 0, s);
}

hipError_t launch_conv_fwd(const ConvProblem& cp, MView out, MView state_out, hipStream_t s) {
  hipError_t e = launch_conv_fwd_range(cp.bf16, cp.B, cp.L, static_cast<int>(cp.C), cp.K, cp.silu,
                                       cp.x, 0, cp.state_in, 0, cp.w, cp.b, out, 0, s);
  if (e != hipSuccess || !state_out.p) return e;
  // returned state: the last K-1 inputs (reuse the SSD conv-state copy with Cd = C)
  Problem pr{};
  pr.bf16 = cp.bf16;
  pr.B = cp.B;
  pr.L = cp.L;
  pr.H = 1;
  pr.P = static_cast<int>(cp.C);
  pr.N = 0;
  pr.G = 1;
  pr.K = cp.K;
  pr.xbc = cp.x;
  pr.cs_in = cp.state_in;
  return launch_conv_state_out(pr, state_out, s);
}

}  // namespace ssd
