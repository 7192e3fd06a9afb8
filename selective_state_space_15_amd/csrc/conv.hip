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
// Backward: one thread per (batch, 32-row tile, 4 channels) walks its rows with a
// sliding register window; dpre = dout * silu'(pre) is recomputed from the raw
// rows, dx[tau] = sum_k dpre[tau + K-1-k] w[k] (plus the gradient of the returned
// conv state for the last K-1 rows), and per-tile partial sums of dw and db go to
// scratch for an ordered reduction (deterministic, no atomics).
#include "common.hpp"
#include "launch.hpp"

namespace ssd {

namespace {

constexpr int kRowsF = 16;  // rows per thread, forward
constexpr int kRowsB = 32;  // rows per thread, backward

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
  void* out_lo;  // optional: out value minus its rounding to the I/O dtype (same layout)
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
      if (a.out_lo) {
        float lo[V];
#pragma unroll
        for (int v = 0; v < V; ++v) lo[v] = o[v] - T::to_f(T::from_f(o[v]));
        store_vec16<IO>(static_cast<E*>(a.out_lo) + b * a.o_sb + a.o_c0 + c + t * a.o_st, lo);
      }
    }
  }
}

// ------------------------------------------------------------------ backward
constexpr int kBatch = 4;  // output rows per step of the backward register window

struct ConvBwdArgs {
  int64_t B, L;
  int C, K, silu;
  const void* x;  // raw rows
  int64_t x_sb, x_st;
  const void* st;  // carried state rows (null = zeros)
  int64_t st_sb, st_st;
  const float* w;
  const float* bias;
  // gradient of the conv output: a view (standalone) or the fused SSD sources
  const void* g;
  int64_t g_sb, g_st;
  const float* dbc;  // fused: dB | dC of group g at [(g * per_g * B + b) * L + t][2N] (fp32)
  int per_g, hp, G, N;
  const void* dso;  // gradient of the returned state rows (null = zero)
  int64_t dso_sb, dso_st;
  void* dx;
  int64_t dx_sb, dx_st;
  void* dsi;  // gradient of the carried-in state rows (null = skip)
  int64_t dsi_sb, dsi_st;
  float* part;  // [B][ntile][C][5]: dw taps 0..K-1, db at 4
};

// Four channels of I/O elements: 8 bytes of bf16 or 16 bytes of fp32, held in a uint4.
template <typename IO>
struct quad;
template <>
struct quad<bf16_t> {
  __device__ static __forceinline__ uint4 load(const uint16_t* p) {
    const uint2 r = *reinterpret_cast<const uint2*>(p);
    return make_uint4(r.x, r.y, 0u, 0u);
  }
  __device__ static __forceinline__ float get(const uint4& r, int v) {
    const uint32_t w = v < 2 ? r.x : r.y;
    return __uint_as_float((v & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ static __forceinline__ void store(uint16_t* p, const float* f) {
    *reinterpret_cast<uint2*>(p) = make_uint2(f2bf2(f[0], f[1]), f2bf2(f[2], f[3]));
  }
};
template <>
struct quad<float> {
  __device__ static __forceinline__ uint4 load(const float* p) {
    return *reinterpret_cast<const uint4*>(p);
  }
  __device__ static __forceinline__ float get(const uint4& r, int v) {
    return __uint_as_float(v == 0 ? r.x : v == 1 ? r.y : v == 2 ? r.z : r.w);
  }
  __device__ static __forceinline__ void store(float* p, const float* f) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
};
__device__ __forceinline__ float word_f(const uint4& r, int v) {
  return __uint_as_float(v == 0 ? r.x : v == 1 ? r.y : v == 2 ? r.z : r.w);
}

// One work item = (batch, kRowsB-row tile, 4 channels).  The thread walks the tile's
// rows kBatch at a time with a register window: raw[i] holds raw row tau0 - 3 + i
// and dp[i] holds dpre of row tau0 + i, so each step loads only kBatch new raw rows
// and kBatch new gradient rows, and those of the next step are in flight while
// this one computes.  Row pointers advance by a stride per step (no 64-bit
// multiplies per row).  INTERIOR tiles (all rows they touch inside the sequence,
// no carried-state rows, no returned-state rows) run without any masking; the
// first and last tiles take the general path, where rows outside the sequence
// read a valid row and are masked to zero after the load.
template <typename IO, bool FUSED, bool INTERIOR>
__device__ __forceinline__ void conv_bwd_tile(const ConvBwdArgs& a, int64_t b, int64_t tile, int c) {
  using T = io_traits<IO>;
  using E = typename T::elem;
  using Qd = quad<IO>;
  const int64_t ntile = (a.L + kRowsB - 1) / kRowsB;
  const int K = a.K;

  float w4[4][4], bias[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    bias[v] = a.bias ? a.bias[c + v] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = j - (4 - K);  // taps right-aligned on 4: tap j reads row t - 3 + j
      w4[j][v] = kk >= 0 ? a.w[(c + v) * K + kk] : 0.f;
    }
  }
  const E* xb = static_cast<const E*>(a.x) + b * a.x_sb + c;
  const E* sb = a.st ? static_cast<const E*>(a.st) + b * a.st_sb + c : nullptr;
  const int64_t xst = a.x_st;
  auto raw_row = [&](int64_t t) -> uint4 {
    if constexpr (INTERIOR) {
      return Qd::load(xb + t * xst);
    } else {
      const E* p = xb;
      bool ok = false;
      if (t >= 0 && t < a.L) {
        p = xb + t * xst;
        ok = true;
      } else if (sb && t < 0 && t >= -(K - 1)) {
        p = sb + (t + K - 1) * a.st_st;
        ok = true;
      }
      return keep_if(ok, Qd::load(p));
    }
  };
  // gradient rows: I/O-typed view, or (fused, B / C channels) the fp32 group sums
  const bool from_f32 = FUSED && c >= a.hp;
  const E* gb = nullptr;
  int64_t g_st = 0;
  const float* fb = nullptr;
  const int64_t f_st = 2LL * a.N;
  if (FUSED) {
    if (from_f32) {
      const int gn = a.G * a.N, rel = c - a.hp;
      const bool isC = rel >= gn;
      const int g = (isC ? rel - gn : rel) / a.N, n0 = (isC ? rel - gn : rel) % a.N;
      fb = a.dbc + ((static_cast<int64_t>(g) * a.per_g * a.B + b) * a.L) * f_st + (isC ? a.N : 0) + n0;
    } else {
      gb = static_cast<const E*>(a.g) + b * a.L * a.hp + c;
      g_st = a.hp;
    }
  } else {
    gb = static_cast<const E*>(a.g) + b * a.g_sb + c;
    g_st = a.g_st;
  }
  auto grad_row = [&](int64_t t) -> uint4 {
    const bool ok = INTERIOR || (t >= 0 && t < a.L);
    const int64_t tt = ok ? t : 0;
    uint4 v;
    if (from_f32)
      v = *reinterpret_cast<const uint4*>(fb + tt * f_st);
    else
      v = Qd::load(gb + tt * g_st);
    return INTERIOR ? v : keep_if(ok, v);
  };
  auto unpack = [&](const uint4& r, float* f) {
#pragma unroll
    for (int v = 0; v < 4; ++v) f[v] = Qd::get(r, v);
  };
  auto unpack_grad = [&](const uint4& r, float* f) {
#pragma unroll
    for (int v = 0; v < 4; ++v) f[v] = from_f32 ? word_f(r, v) : Qd::get(r, v);
  };
  // dpre of row t from its four raw rows (rows t-3 .. t) and its gradient g
  const bool silu = a.silu != 0;
  auto dpre_row = [&](int64_t t, const float (*rw)[4], const float* gv, float* d) {
    const bool ok = INTERIOR || (t >= 0 && t < a.L);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float pre = bias[v];
#pragma unroll
      for (int j = 0; j < 4; ++j) pre = fmaf(w4[j][v], rw[j][v], pre);
      const float dv = silu ? gv[v] * dsiluf_(pre) : gv[v];
      d[v] = ok ? dv : 0.f;
    }
  };

  float dw[4][4], db[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    db[v] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) dw[j][v] = 0.f;
  }
  E* dxb = static_cast<E*>(a.dx) + b * a.dx_sb + c;
  const E* dsob = a.dso ? static_cast<const E*>(a.dso) + b * a.dso_sb + c : nullptr;
  E* dsib = a.dsi ? static_cast<E*>(a.dsi) + b * a.dsi_sb + c : nullptr;
  const int64_t t_lo = tile * kRowsB;
  // tile 0 also produces the gradient of the carried-in state rows (tau < 0)
  const int64_t tau_begin = tile == 0 ? -(K - 1) : t_lo;
  const int64_t tau_end = t_lo + kRowsB < a.L ? t_lo + kRowsB : a.L;

  float raw[kBatch + 6][4];   // raw row tau0 - 3 + i
  float dp[kBatch + 3][4];    // dpre of row tau0 + i
  int64_t tau0 = tau_begin;
  {
    uint4 r0[6], g0[3];
#pragma unroll
    for (int i = 0; i < 6; ++i) r0[i] = raw_row(tau0 - 3 + i);
#pragma unroll
    for (int i = 0; i < 3; ++i) g0[i] = grad_row(tau0 + i);
#pragma unroll
    for (int i = 0; i < 6; ++i) unpack(r0[i], raw[i]);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      float gv[4];
      unpack_grad(g0[i], gv);
      dpre_row(tau0 + i, raw + i, gv, dp[i]);
    }
  }
  uint4 nraw[kBatch], ngr[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    nraw[i] = raw_row(tau0 + 3 + i);
    ngr[i] = grad_row(tau0 + 3 + i);
  }
  E* dxrow = dxb + tau0 * a.dx_st;  // advanced by kBatch rows per step
  const int64_t dx_step = kBatch * a.dx_st;
  for (; tau0 < tau_end; tau0 += kBatch, dxrow += dx_step) {
    float cgr[kBatch][4];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      unpack(nraw[i], raw[6 + i]);
      unpack_grad(ngr[i], cgr[i]);
    }
    // next step's rows (harmless past the tile: masked or simply unused)
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      nraw[i] = raw_row(tau0 + kBatch + 3 + i);
      ngr[i] = grad_row(tau0 + kBatch + 3 + i);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) dpre_row(tau0 + 3 + i, raw + 3 + i, cgr[i], dp[3 + i]);
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int64_t tau = tau0 + r;
      if (INTERIOR || tau < tau_end) {
        float o[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float acc = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) acc = fmaf(w4[j][v], dp[r + 3 - j][v], acc);
          o[v] = acc;
        }
        if constexpr (!INTERIOR) {
          const int64_t js = tau - (a.L - (K - 1));  // row of the returned state
          if (dsob && js >= 0) {
            const uint4 d = Qd::load(dsob + js * a.dso_st);
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] += Qd::get(d, v);
          }
        }
        if (INTERIOR || tau >= 0) {
          Qd::store(dxrow + r * a.dx_st, o);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            db[v] += dp[r][v];
#pragma unroll
            for (int j = 0; j < 4; ++j) dw[j][v] = fmaf(dp[r][v], raw[r + j][v], dw[j][v]);
          }
        } else if (dsib) {
          Qd::store(dsib + (tau + K - 1) * a.dsi_st, o);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 6; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) raw[i][v] = raw[i + kBatch][v];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) dp[i][v] = dp[i + kBatch][v];
  }
  float* pp = a.part + ((b * ntile + tile) * a.C + c) * 5;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = j - (4 - K);
      if (kk >= 0) pp[v * 5 + kk] = dw[j][v];
    }
    pp[v * 5 + 4] = db[v];
  }
}

template <typename IO, bool FUSED>
__device__ __forceinline__ void conv_bwd_item(const ConvBwdArgs& a, int64_t gid) {
  const int ncq = a.C / 4;
  const int64_t ntile = (a.L + kRowsB - 1) / kRowsB;
  const int c = static_cast<int>(gid % ncq) * 4;
  const int64_t tile = (gid / ncq) % ntile;
  const int64_t b = gid / (static_cast<int64_t>(ncq) * ntile);
  // interior: rows t_lo - 3 .. t_lo + kRowsB + 2 * kBatch + 2 (prefetch reach) inside
  // the sequence, and none of the last K - 1 rows (gradient of the returned state)
  const int64_t t_lo = tile * kRowsB;
  const bool interior = tile > 0 && t_lo + kRowsB + 2 * kBatch + 3 <= a.L - (a.K - 1);
  if (interior)
    conv_bwd_tile<IO, FUSED, true>(a, b, tile, c);
  else
    conv_bwd_tile<IO, FUSED, false>(a, b, tile, c);
}

// Grid-stride over the (batch, tile, 4-channel) items: the grid is sized to what
// the device holds at once, so no partial last round of workgroups.
template <typename IO, bool FUSED>
__global__ void __launch_bounds__(256) conv_bwd_kernel(ConvBwdArgs a) {
  const int64_t ntile = (a.L + kRowsB - 1) / kRowsB;
  const int64_t total = a.B * ntile * (a.C / 4);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t gid = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; gid < total;
       gid += stride)
    conv_bwd_item<IO, FUSED>(a, gid);
}

// dw[c][k], db[c]: ordered sums of the per-(batch, tile) partials ([n_bt][C][5])
__global__ void __launch_bounds__(256) conv_params_kernel(const float* part, int64_t n_bt, int C,
                                                          int K, float* dw, float* db,
                                                          int accumulate) {
  const float acc = block_colsum(part, n_bt, static_cast<int64_t>(C) * 5);
  const int i = blockIdx.x * kWave + threadIdx.x;
  if (threadIdx.x >= kWave || i >= C * 5) return;
  const int c = i / 5, k = i % 5;
  if (k < 4 && k >= K) return;
  float* dst = k == 4 ? (db ? db + c : nullptr) : (dw ? dw + c * K + k : nullptr);
  if (!dst) return;
  *dst = accumulate ? *dst + acc : acc;
}

template <typename IO, bool FUSED>
void launch_conv_bwd_kernel(const ConvBwdArgs& a, int64_t n, hipStream_t s) {
  const int64_t cap = resident_blocks(reinterpret_cast<const void*>(conv_bwd_kernel<IO, FUSED>), 256);
  int64_t blocks = (n + 255) / 256;
  if (cap > 0 && blocks > cap) blocks = cap;
  hipLaunchKernelGGL((conv_bwd_kernel<IO, FUSED>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     s, a);
}

hipError_t run_conv_bwd(ConvBwdArgs a, int bf16, bool fused, float* dw, float* db, int accumulate,
                        hipStream_t s) {
  const int64_t ntile = (a.L + kRowsB - 1) / kRowsB;
  const int64_t n = a.B * ntile * (a.C / 4);
  TimingScope ts(kKConvBwd, s);
  if (bf16) {
    if (fused)
      launch_conv_bwd_kernel<bf16_t, true>(a, n, s);
    else
      launch_conv_bwd_kernel<bf16_t, false>(a, n, s);
  } else {
    if (fused)
      launch_conv_bwd_kernel<float, true>(a, n, s);
    else
      launch_conv_bwd_kernel<float, false>(a, n, s);
  }
  hipLaunchKernelGGL(conv_params_kernel, dim3(static_cast<unsigned>((a.C * 5 + kWave - 1) / kWave)),
                     dim3(256), 0, s, a.part, a.B * ntile, a.C, a.K, dw, db, accumulate);
  return hipGetLastError();
}

}  // namespace

size_t conv_bwd_partials_bytes(int64_t B, int64_t L, int64_t C) {
  const int64_t ntile = (L + kRowsB - 1) / kRowsB;
  return static_cast<size_t>(B) * ntile * C * 5 * sizeof(float);
}

size_t conv_bwd_workspace_bytes(int64_t B, int64_t L, int64_t C) {
  return conv_bwd_partials_bytes(B, L, C);
}

hipError_t launch_conv_bwd(const ConvProblem& cp, View dout, View dstate_out, MView dx, float* dw,
                           float* db, MView dstate_in, int accumulate, void* ws, hipStream_t s) {
  ConvBwdArgs a{};
  a.B = cp.B;
  a.L = cp.L;
  a.C = static_cast<int>(cp.C);
  a.K = cp.K;
  a.silu = cp.silu;
  a.x = cp.x.p;
  a.x_sb = cp.x.sb;
  a.x_st = cp.x.st;
  a.st = cp.state_in.p;
  a.st_sb = cp.state_in.sb;
  a.st_st = cp.state_in.st;
  a.w = cp.w;
  a.bias = cp.b;
  a.g = dout.p;
  a.g_sb = dout.sb;
  a.g_st = dout.st;
  a.dso = dstate_out.p;
  a.dso_sb = dstate_out.sb;
  a.dso_st = dstate_out.st;
  a.dx = dx.p;
  a.dx_sb = dx.sb;
  a.dx_st = dx.st;
  a.dsi = dstate_in.p;
  a.dsi_sb = dstate_in.sb;
  a.dsi_st = dstate_in.st;
  a.part = static_cast<float*>(ws);
  return run_conv_bwd(a, cp.bf16, false, dw, db, accumulate, s);
}

// Conv backward of the SSD entry point: the post-conv gradient of the x channels
// comes from `dx_ws` ([B][L][H*P], I/O dtype), that of the B and C channels from
// the fp32 sums over each group's head blocks, held in the partial slot of the
// group's first block (slot g * per_g of a [slots][B][L][2N] array).
hipError_t launch_conv_bwd_fused(const Problem& pr, const void* dx_ws, const float* dbc_sum,
                                 int per_g, View dcs_out, MView dxbc, float* dconv_w, float* dconv_b,
                                 MView dcs_in, int accumulate, void* ws, hipStream_t s) {
  ConvBwdArgs a{};
  a.B = pr.B;
  a.L = pr.L;
  a.C = pr.H * pr.P + 2 * pr.G * pr.N;
  a.K = pr.K;
  a.silu = 1;
  a.x = pr.xbc.p;
  a.x_sb = pr.xbc.sb;
  a.x_st = pr.xbc.st;
  a.st = pr.cs_in.p;
  a.st_sb = pr.cs_in.sb;
  a.st_st = pr.cs_in.st;
  a.w = pr.conv_w;
  a.bias = pr.conv_b;
  a.g = dx_ws;
  a.dbc = dbc_sum;
  a.per_g = per_g;
  a.hp = pr.H * pr.P;
  a.G = pr.G;
  a.N = pr.N;
  a.dso = dcs_out.p;
  a.dso_sb = dcs_out.sb;
  a.dso_st = dcs_out.st;
  a.dx = dxbc.p;
  a.dx_sb = dxbc.sb;
  a.dx_st = dxbc.st;
  a.dsi = dcs_in.p;
  a.dsi_sb = dcs_in.sb;
  a.dsi_st = dcs_in.st;
  a.part = static_cast<float*>(ws);
  return run_conv_bwd(a, pr.bf16, true, dconv_w, dconv_b, accumulate, s);
}

// Conv forward over channels [c0, c0 + C) of the rows of `x`, writing channels
// [o_c0, o_c0 + C) of `out`.  Weights / bias pointers refer to channel c0.
hipError_t launch_conv_fwd_range(int bf16, int64_t B, int64_t L, int C, int K, int silu, View x,
                                 int x_c0, View st, int st_c0, const float* w, const float* bias,
                                 MView out, int o_c0, hipStream_t s, void* out_lo) {
  ConvFwdArgs a{};
  a.out_lo = out_lo;
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

hipError_t launch_bc_prepass(const Problem& pr, void* dst, void* dst_lo, hipStream_t s) {
  TimingScope ts(kKBcPrepass, s);
  const int hp = pr.H * pr.P, gn2 = 2 * pr.G * pr.N;
  const MView out{dst, pr.L * gn2, gn2};
  return launch_conv_fwd_range(pr.bf16, pr.B, pr.L, gn2, pr.K, 1, pr.xbc, hp, pr.cs_in, hp,
                               pr.conv_w + static_cast<int64_t>(hp) * pr.K,
                               pr.conv_b ? pr.conv_b + hp : nullptr, out, 0, s,
                               pr.bf16 ? dst_lo : nullptr);
}

size_t x_prepass_bytes(const Problem& pr) {
  if (pr.K == 0) return 0;
  const size_t n = static_cast<size_t>(pr.B) * pr.L * pr.H * pr.P * (pr.bf16 ? 2 : 4);
  return (n + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_x_prepass(const Problem& pr, void* dst, hipStream_t s) {
  TimingScope ts(kKBcPrepass, s);
  const int hp = pr.H * pr.P;
  const MView out{dst, pr.L * hp, hp};
  return launch_conv_fwd_range(pr.bf16, pr.B, pr.L, hp, pr.K, 1, pr.xbc, 0, pr.cs_in, 0, pr.conv_w,
                               pr.conv_b, out, 0, s, nullptr);
}

hipError_t launch_conv_fwd(const ConvProblem& cp, MView out, MView state_out, hipStream_t s) {
  TimingScope ts(kKConvFwd, s);
  hipError_t e = launch_conv_fwd_range(cp.bf16, cp.B, cp.L, static_cast<int>(cp.C), cp.K, cp.silu,
                                       cp.x, 0, cp.state_in, 0, cp.w, cp.b, out, 0, s, nullptr);
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
