// Causal depthwise conv1d (+ bias, optional SiLU) on gfx950, forward and backward.
//
//   pre[t, c] = b[c] + sum_{k<K} w[c, k] * xin[t - K + 1 + k, c],   out = silu(pre) or pre
//   xin[t < 0] = carried conv state (the last K-1 inputs of the previous segment)
//
// This is the Conv1d that the Video-Ma2mba review (pith.science verdict for arXiv
// 2411.19460, skeptic critique) notes precedes the SSD in a Mamba-2 block, which
// is why a sequence checkpoint must carry the conv buffer as well as h.
//
// Forward: one thread per (batch, 8-row tile, 16-byte channel vector); all 11 raw
// rows are loaded up front (independent loads in flight), the taps are applied in
// registers and the 8 output rows are stored as 16-byte vectors.  Adjacent threads
// take adjacent channel vectors, so every row access is coalesced.
//
// Backward: one workgroup per (batch, 64-row tile, 64 channels) stages the tile's raw
// and gradient rows in LDS (all loads in flight at once), then each thread walks 16
// rows of one channel with a sliding register window; dpre = dout * silu'(pre) is
// recomputed from the raw rows, dx[tau] = sum_k dpre[tau + K-1-k] w[k] (plus the
// gradient of the returned conv state for the last K-1 rows), and per-tile partial
// sums of dw and db go to scratch for an ordered reduction (deterministic, no atomics).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace ssd {

namespace {

constexpr int kRowsF = 8;      // rows per thread, forward
constexpr int kTileRows = 64;  // rows per workgroup, backward
constexpr int kTileCh = 64;    // channels per workgroup, backward
constexpr int kSegRows = 16;   // rows per thread, backward (four segments per tile)

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
  // channels c >= split (relative to x_c0) go to out2 at channel c - split instead
  // (with out2_lo as out_lo); split >= C: everything goes to out
  int split;
  void* out2;
  int64_t o2_sb, o2_st;
  void* out2_lo;
};

// K is a template parameter so that every load is straight-line code: a load under a
// branch, a select right after a load, or control flow that merges registers with
// loads in flight makes the compiler wait for every outstanding memory operation
// (the previous rows' stores included) inside each output row.
template <typename IO, int K>
__global__ void __launch_bounds__(256) conv_fwd_kernel(ConvFwdArgs a) {
  using T = io_traits<IO>;
  using E = typename T::elem;
  constexpr int V = T::vec;
  static_assert(K >= 1 && K <= 4, "taps are right-aligned on 4");
  const int ncv = a.C / V;
  const int64_t ntile = (a.L + kRowsF - 1) / kRowsF;
  // consecutive workgroups (consecutive row tiles) on one XCD: each XCD writes one
  // contiguous token range, the range the chunk kernels after it (xcd_remap over
  // chunks or chunk groups) give to the same XCD, so part of what they read of these
  // rows is still in that XCD's L2
  const int64_t gid = xcd_remap(blockIdx.x, gridDim.x) * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (gid >= a.B * ntile * ncv) return;
  const int cv = static_cast<int>(gid % ncv);
  const int64_t tile = (gid / ncv) % ntile;
  const int64_t b = gid / (static_cast<int64_t>(ncv) * ntile);
  const int c = cv * V;
  const int64_t t0 = tile * kRowsF;
  const E* xb = static_cast<const E*>(a.x) + b * a.x_sb + a.x_c0 + c;
  const bool has_st = a.st != nullptr;
  const E* sb = has_st ? static_cast<const E*>(a.st) + b * a.st_sb + a.st_c0 + c : xb;
  const int64_t sst = has_st ? a.st_st : 0;

  // weights of the V channels: [C][K] rows of consecutive channels are contiguous, V*K
  // floats from a 16-byte aligned offset (the pointer is checked 16-byte aligned)
  constexpr int NWV = V * K / 4;
  float wf[V * K];
  {
    const float4* wv = reinterpret_cast<const float4*>(a.w + static_cast<int64_t>(c) * K);
#pragma unroll
    for (int q = 0; q < NWV; ++q) {
      const float4 v4 = wv[q];
      wf[4 * q] = v4.x;
      wf[4 * q + 1] = v4.y;
      wf[4 * q + 2] = v4.z;
      wf[4 * q + 3] = v4.w;
    }
  }
  const bool has_bias = a.bias != nullptr;
  const float* bp = has_bias ? a.bias + c : a.w;  // any valid address without a bias
  float bias_raw[V];
#pragma unroll
  for (int v = 0; v < V; v += 4) {
    const float4 v4 = *reinterpret_cast<const float4*>(bp + v);
    bias_raw[v] = v4.x;
    bias_raw[v + 1] = v4.y;
    bias_raw[v + 2] = v4.z;
    bias_raw[v + 3] = v4.w;
  }
  // raw rows t0-3 .. t0+kRowsF-1 from rows clamped into [0, L), and the carried-state rows
  // for the three rows before the tile (used on the first tile only)
  uint4 in[kRowsF + 3], sin[3];
#pragma unroll
  for (int i = 0; i < kRowsF + 3; ++i) {
    const int64_t t = t0 - 3 + i;
    const int64_t tc = t < 0 ? 0 : (t >= a.L ? a.L - 1 : t);
    in[i] = *reinterpret_cast<const uint4*>(xb + tc * a.x_st);
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int j = i + K - 4;  // state row of t = -3 + i (valid for j >= 0)
    sin[i] = *reinterpret_cast<const uint4*>(sb + (j < 0 ? 0 : j) * sst);
  }

  const bool second = c >= a.split;  // a vector never straddles the split (split % V == 0)
  E* ob = second ? static_cast<E*>(a.out2) + b * a.o2_sb + (c - a.split)
                 : static_cast<E*>(a.out) + b * a.o_sb + a.o_c0 + c;
  E* olb = second ? (a.out2_lo ? static_cast<E*>(a.out2_lo) + b * a.o2_sb + (c - a.split) : nullptr)
                  : (a.out_lo ? static_cast<E*>(a.out_lo) + b * a.o_sb + a.o_c0 + c : nullptr);
  const int64_t ost = second ? a.o2_st : a.o_st;

  // row index i (t = t0 - 3 + i): the carried-state row before the sequence, zero
  // outside the sequence and before the carried state -- resolved once per row on the
  // packed words, so each tap reads a plain element
#pragma unroll
  for (int i = 0; i < kRowsF + 3; ++i) {
    const int64_t t = t0 - 3 + i;
    uint4 v = in[i];
    if (i < 3) {
      const bool from_st = t < 0;
      v = make_uint4(from_st ? sin[i].x : v.x, from_st ? sin[i].y : v.y, from_st ? sin[i].z : v.z,
                     from_st ? sin[i].w : v.w);
    }
    const bool ok = t < a.L && t >= -(K - 1) && (t >= 0 || has_st);
    in[i] = keep_if(ok, v);
  }
  auto raw = [&](int i, int v) __attribute__((always_inline)) { return raw_elem<IO>(in[i], v); };
  float bias[V];
#pragma unroll
  for (int v = 0; v < V; ++v) bias[v] = has_bias ? bias_raw[v] : 0.f;
  // SILU is the (uniform) activation flag as a compile-time value: one branch for the
  // tile instead of a select per element
  auto row = [&](int r, float* o, auto silu_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float pre = bias[v];
#pragma unroll
      for (int k = 0; k < K; ++k) pre = fmaf(wf[v * K + k], raw(r + 4 - K + k, v), pre);
      o[v] = decltype(silu_tag)::value ? siluf_(pre) : pre;
    }
  };
  auto put = [&](int r, const float* o) __attribute__((always_inline)) {
    store_vec16<IO>(ob + (t0 + r) * ost, o);
    if (olb) {
      float lo[V];
#pragma unroll
      for (int v = 0; v < V; ++v) lo[v] = o[v] - T::to_f(T::from_f(o[v]));
      store_vec16<IO>(olb + (t0 + r) * ost, lo);
    }
  };
  auto tile_rows = [&](auto silu_tag) __attribute__((always_inline)) {
    if (t0 + kRowsF <= a.L) {
#pragma unroll
      for (int r = 0; r < kRowsF; ++r) {
        float o[V];
        row(r, o, silu_tag);
        put(r, o);
      }
    } else {
#pragma unroll
      for (int r = 0; r < kRowsF; ++r) {
        float o[V];
        row(r, o, silu_tag);
        if (t0 + r < a.L) put(r, o);
      }
    }
  };
  if (a.silu)
    tile_rows(std::true_type{});
  else
    tile_rows(std::false_type{});
}

// ------------------------------------------------------------------ backward

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

// One workgroup = (batch, kTileRows-row tile, kTileCh channels).  The tile's raw rows
// (with the 3-row halo on each side) and its gradient rows (with 3 rows below) are
// first loaded as 16-byte vectors, every load in flight at once, into LDS (the
// gradient as fp32).  Then thread (channel cl, segment s) walks rows
// [t_lo + kSegRows s, t_lo + kSegRows (s + 1)) with a register window: dpre of rows tau .. tau + 3
// and raw rows tau - 3 .. tau + 3, so each row reads one raw and one gradient value
// from LDS.  Rows outside the sequence are zero; tile 0 also produces the gradient of
// the carried-in state rows (tau < 0), and the last K-1 rows add the gradient of the
// returned state.  The dw / db sums of the four segments are added in segment order
// and written as one partial per (batch, tile, channel).
template <typename IO, bool FUSED>
__global__ void __launch_bounds__(256) conv_bwd_kernel(ConvBwdArgs a) {
  using T = io_traits<IO>;
  using E = typename T::elem;
  constexpr int V = T::vec;                  // channels per 16-byte I/O vector
  constexpr int RROWS = kTileRows + 6;       // raw rows t_lo - 3 .. t_lo + kTileRows + 2
  constexpr int GROWS = kTileRows + 3;       // gradient rows t_lo .. t_lo + kTileRows + 2
  constexpr int RVPR = kTileCh / V;          // raw vectors per row
  constexpr int NRV = (RROWS * RVPR + 255) / 256;
  constexpr int GVPR_F = kTileCh / 4;        // fp32 gradient vectors per row
  constexpr int NGV = (GROWS * GVPR_F + 255) / 256;  // slots for the widest gradient case
  static_assert(kTileRows == 4 * kSegRows, "four row segments per tile");
  __shared__ __align__(16) E sR[RROWS * kTileCh];
  __shared__ __align__(16) float sG[GROWS * kTileCh];

  // channel blocks: the I/O-gradient channels [0, xlim) in blocks of kTileCh, then (fused)
  // the fp32-gradient B / C channels [hp, C); a block never mixes the two
  const int xlim = FUSED ? a.hp : a.C;
  const int nxb = (xlim + kTileCh - 1) / kTileCh;
  const int ncb = nxb + (FUSED ? (a.C - a.hp + kTileCh - 1) / kTileCh : 0);
  const int64_t ntile = (a.L + kTileRows - 1) / kTileRows;
  // consecutive workgroups on one XCD: one contiguous token range per XCD, as in the
  // chunk kernels before it
  const int64_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = static_cast<int>(wg % ncb);
  const int64_t tile = (wg / ncb) % ntile;
  const int64_t b = wg / (static_cast<int64_t>(ncb) * ntile);
  const bool from_f32 = FUSED && cb >= nxb;
  const int c0 = from_f32 ? a.hp + (cb - nxb) * kTileCh : cb * kTileCh;
  const int climit = from_f32 ? a.C : xlim;  // channels of this block: [c0, min(c0 + kTileCh, climit))
  const int64_t t_lo = tile * kTileRows;
  const int K = a.K;
  const int tid = threadIdx.x;

  // ---- tile loads.  Every load is unconditional, from a clamped (valid) address,
  // and all of them are in flight together; the masks (rows outside the sequence,
  // channels past the block) are applied where the values go to LDS.  A load under a
  // branch, or a select right after it, would make the wave wait for it at once.
  const bool has_st = a.st != nullptr;
  const E* xb = static_cast<const E*>(a.x) + b * a.x_sb;
  const E* sbp = has_st ? static_cast<const E*>(a.st) + b * a.st_sb : xb;
  const int64_t sst = has_st ? a.st_st : 0;
  // thread tid loads the vectors tid + 256 q; 256 is a multiple of the vectors per row,
  // so its column is the same in every row: the column is resolved once and each load
  // adds a row offset
  static_assert(256 % RVPR == 0, "raw vectors per row divide the block");
  const int rcv = (tid % RVPR) * V;
  const int rcc = c0 + rcv < climit ? c0 + rcv : c0;
  const E* xcol = xb + rcc;
  const E* scol = sbp + rcc;
  uint4 rr[NRV];
#pragma unroll
  for (int q = 0; q < NRV; ++q) {
    const int row = min(tid / RVPR + (256 / RVPR) * q, RROWS - 1);
    const int64_t t = t_lo - 3 + row;
    const bool in_st = has_st && t < 0 && t >= -(K - 1);
    const int64_t tc = t < 0 ? 0 : (t >= a.L ? a.L - 1 : t);
    const E* src = in_st ? scol + (t + K - 1) * sst : xcol + tc * a.x_st;
    rr[q] = *reinterpret_cast<const uint4*>(src);
  }
  // gradient rows: 16-byte vectors of cw channels (the I/O view, or the fp32 group
  // sums for the fused B / C channels); gvpr = vectors per row (a power of two)
  const int gsh = from_f32 ? 4 : (V == 8 ? 3 : 4);
  const int cw = from_f32 ? 4 : V;
  // as for the raw rows, the column of a thread's gradient vectors is the same in every
  // row: its address is resolved once (the block is uniformly I/O or fp32 gradients, so
  // only one kind is computed), and each row adds rows x the row stride
  uint4 gr[NGV];
  {
    const int gcv = (tid & ((1 << gsh) - 1)) * cw;
    const int gcc = c0 + gcv < climit ? c0 + gcv : c0;
    const char* gcol;
    int64_t gst;  // bytes between rows
    if constexpr (FUSED) {
      if (from_f32) {
        // fp32 group sums [group][B][L][2N] of B (first N) and C (next N)
        const int gn = a.G * a.N, lgN = __builtin_ctz(a.N);  // N is a power of two
        const int rel = gcc - a.hp;
        const bool isC = rel >= gn;
        const int rc = isC ? rel - gn : rel;
        gcol = reinterpret_cast<const char*>(
            a.dbc + ((static_cast<int64_t>(rc >> lgN) * a.per_g * a.B + b) * a.L) * (2LL * a.N) +
            (isC ? a.N : 0) + (rc & (a.N - 1)));
        gst = 2LL * a.N * sizeof(float);
      } else {
        gcol = reinterpret_cast<const char*>(static_cast<const E*>(a.g) + b * a.L * a.hp + gcc);
        gst = static_cast<int64_t>(a.hp) * sizeof(E);
      }
    } else {
      gcol = reinterpret_cast<const char*>(static_cast<const E*>(a.g) + b * a.g_sb + gcc);
      gst = a.g_st * static_cast<int64_t>(sizeof(E));
    }
    const int growq = 256 >> gsh;  // rows one pass of the block covers
#pragma unroll
    for (int q = 0; q < NGV; ++q) {
      const int row = min((tid >> gsh) + growq * q, GROWS - 1);
      const int64_t t = t_lo + row;
      const int64_t tt = t < a.L ? t : a.L - 1;
      gr[q] = *reinterpret_cast<const uint4*>(gcol + tt * gst);
    }
  }
  // gradient of the returned state rows L-(K-1) .. L-1 (zero without one), fp32 in LDS
  __shared__ float sDso[3][kTileCh];
  uint4 dso_v;
  constexpr int DVPR = kTileCh / V;
  const bool has_dso = a.dso != nullptr;
  {
    const int k = min(tid, 3 * DVPR - 1);
    const int js = k / DVPR, cv = (k % DVPR) * V;
    const int cc = c0 + cv < climit ? c0 + cv : c0;
    const E* src = has_dso ? static_cast<const E*>(a.dso) + b * a.dso_sb + (js < K - 1 ? js : 0) * a.dso_st + cc
                           : xb + cc;
    dso_v = *reinterpret_cast<const uint4*>(src);
  }
  // this thread's channel: taps (right-aligned on 4: tap j reads row t - 3 + j) and bias
  const int cl = tid % kTileCh, seg = tid / kTileCh;
  const int c = c0 + cl;
  const bool cvalid = c < climit;
  const int cwc = cvalid ? c : c0;
  float w4[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int kk = jj - (4 - K);
    w4[jj] = a.w[cwc * K + (kk >= 0 ? kk : 0)];
  }
  const float bias_raw = a.bias ? a.bias[cwc] : 0.f;

  // ---- masks, then LDS
#pragma unroll
  for (int q = 0; q < NRV; ++q) {
    const int k = tid + 256 * q;
    const int row = k / RVPR, cv = (k % RVPR) * V;
    const int64_t t = t_lo - 3 + row;
    const bool in_seq = t >= 0 && t < a.L;
    const bool in_st = has_st && t < 0 && t >= -(K - 1);
    const bool ok = c0 + cv < climit && (in_seq || in_st);
    if (k < RROWS * RVPR) *reinterpret_cast<uint4*>(sR + row * kTileCh + cv) = keep_if(ok, rr[q]);
  }
#pragma unroll
  for (int q = 0; q < NGV; ++q) {
    const int k = tid + 256 * q;
    const int row = k >> gsh, cv = (k & ((1 << gsh) - 1)) * cw;
    const bool ok = c0 + cv < climit && t_lo + row < a.L;
    if (k < (GROWS << gsh)) {
      float* dst = sG + row * kTileCh + cv;
      if (from_f32) {
        *reinterpret_cast<uint4*>(dst) = keep_if(ok, gr[q]);
      } else {
        const uint4 gk = keep_if(ok, gr[q]);  // masked as packed words, then widened
        float f[V];
#pragma unroll
        for (int v = 0; v < V; ++v) f[v] = raw_elem<IO>(gk, v);
#pragma unroll
        for (int v = 0; v < V; v += 4) *reinterpret_cast<float4*>(dst + v) = make_float4(f[v], f[v + 1], f[v + 2], f[v + 3]);
      }
    }
  }
  if (tid < 3 * DVPR) {
    const int js = tid / DVPR, cv = (tid % DVPR) * V;
    const bool ok = has_dso && js < K - 1;
#pragma unroll
    for (int v = 0; v < V; ++v) sDso[js][cv + v] = ok ? raw_elem<IO>(dso_v, v) : 0.f;
  }
  for (int jj = 0; jj < 4; ++jj)
    if (jj < 4 - K || !cvalid) w4[jj] = 0.f;
  const float bias = cvalid ? bias_raw : 0.f;
  __syncthreads();

  // ---- the row walk: thread (channel cl, segment seg) produces dx of rows
  // r0 .. r0 + kSegRows - 1 with a register window (raw rows tau-3 .. tau+3, dpre of
  // rows tau .. tau+3); tile 0's first segment also the carried-state rows -(K-1)..-1
  const bool silu = a.silu != 0;
  const int64_t r0 = t_lo + seg * kSegRows;
  const int lr0 = seg * kSegRows;  // r0 - t_lo
  auto raw_l = [&](int lr) __attribute__((always_inline)) {  // raw row t_lo + lr (lr >= -3)
    return T::lds_to_f(sR[(lr + 3) * kTileCh + cl]);
  };
  auto dpre_l = [&](int lr, const float* rw4) __attribute__((always_inline)) {  // row t_lo + lr >= t_lo
    float pre = bias;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) pre = fmaf(w4[jj], rw4[jj], pre);
    const float gv = sG[lr * kTileCh + cl];  // zero outside the sequence
    return silu ? gv * dsiluf_(pre) : gv;
  };
  float dw[4] = {0.f, 0.f, 0.f, 0.f}, db = 0.f;
  // carried-state rows (tile 0, segment 0: one whole wave)
  if (tile == 0 && seg == 0 && a.dsi != nullptr) {
    E* dsib = static_cast<E*>(a.dsi) + b * a.dsi_sb + cwc;
    for (int tau = -(K - 1); tau < 0; ++tau) {
      // o = sum_j w[j] dpre(tau + 3 - j); dpre of rows outside [0, L) is zero
      float o = 0.f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int t = tau + 3 - jj;
        if (t >= 0 && t < a.L) {
          float rw4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) rw4[i] = raw_l(t - 3 + i);
          o = fmaf(w4[jj], dpre_l(t, rw4), o);
        }
      }
      const int64_t js = tau - (a.L - (K - 1));
      if (js >= 0) o += sDso[js][cl];
      if (cvalid) dsib[(tau + K - 1) * a.dsi_st] = T::from_f(o);
    }
  }
  // the walk's dx rows, stored afterwards through LDS as 16-byte row vectors
  float outv[kSegRows];
#pragma unroll
  for (int r = 0; r < kSegRows; ++r) outv[r] = 0.f;
  auto walk = [&](auto edge_tag) __attribute__((always_inline)) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    float rw[7], d[4];
#pragma unroll
    for (int i = 0; i < 6; ++i) rw[i] = raw_l(lr0 - 3 + i);
#pragma unroll
    for (int i = 0; i < 3; ++i) d[i] = dpre_l(lr0 + i, rw + i);
#pragma unroll
    for (int r = 0; r < kSegRows; ++r) {
      const int lr = lr0 + r;
      rw[6] = raw_l(lr + 3);
      d[3] = dpre_l(lr + 3, rw + 3);
      float o = 0.f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) o = fmaf(w4[jj], d[3 - jj], o);
      db += d[0];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dw[jj] = fmaf(d[0], rw[jj], dw[jj]);
      if constexpr (EDGE) {
        const int64_t js = t_lo + lr - (a.L - (K - 1));
        if (js >= 0 && js < K - 1) o += sDso[js][cl];
      }
      outv[r] = o;
#pragma unroll
      for (int i = 0; i < 6; ++i) rw[i] = rw[i + 1];
#pragma unroll
      for (int i = 0; i < 3; ++i) d[i] = d[i + 1];
    }
  };
  // interior tiles: every row is inside the sequence and none is a returned-state row
  if (t_lo + kTileRows <= a.L - (K - 1))
    walk(std::false_type{});
  else if (r0 < a.L)
    walk(std::true_type{});
  // ---- dx rows and the dw / db partials go through the tiles' LDS once every thread
  // is done with it: dx as [row][channel] in the gradient tile, then stored as 16-byte
  // row vectors; dw / db of the four segments added in segment order, one partial per
  // (batch, tile, channel)
  __syncthreads();
  E* sO = reinterpret_cast<E*>(sG);  // [kTileRows][kTileCh]
  static_assert(kTileRows * kTileCh * sizeof(E) <= sizeof(sG), "dx rows fit the gradient tile");
#pragma unroll
  for (int r = 0; r < kSegRows; ++r) sO[(lr0 + r) * kTileCh + cl] = T::from_f(outv[r]);
  float* sPart = reinterpret_cast<float*>(sR);  // [4 segments][5][kTileCh]
  static_assert(4 * 5 * kTileCh * sizeof(float) <= sizeof(sR), "partials fit the raw tile");
#pragma unroll
  for (int j = 0; j < 4; ++j) sPart[(seg * 5 + j) * kTileCh + cl] = dw[j];
  sPart[(seg * 5 + 4) * kTileCh + cl] = db;
  __syncthreads();
  {
    constexpr int OV = kTileCh / V;  // vectors per row
    static_assert(kTileRows * OV % 256 == 0, "dx vectors tile the block");
    E* dxt = static_cast<E*>(a.dx) + b * a.dx_sb + t_lo * a.dx_st + c0;
#pragma unroll
    for (int q = 0; q < kTileRows * OV / 256; ++q) {
      const int k = tid + 256 * q;
      const int row = k / OV, cv = (k % OV) * V;
      if (t_lo + row < a.L && c0 + cv < climit)
        *reinterpret_cast<uint4*>(dxt + row * a.dx_st + cv) = *reinterpret_cast<const uint4*>(sO + row * kTileCh + cv);
    }
  }
  if (seg == 0 && cvalid) {
    float* pp = a.part + ((b * ntile + tile) * a.C + c) * 5;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const float v = ((sPart[j * kTileCh + cl] + sPart[(5 + j) * kTileCh + cl]) + sPart[(10 + j) * kTileCh + cl]) +
                      sPart[(15 + j) * kTileCh + cl];
      const int kk = j - (4 - K);
      if (j == 4)
        pp[4] = v;
      else if (kk >= 0)
        pp[kk] = v;
    }
  }
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
void launch_conv_bwd_kernel(const ConvBwdArgs& a, hipStream_t s) {
  const int64_t ntile = (a.L + kTileRows - 1) / kTileRows;
  const int xlim = FUSED ? a.hp : a.C;
  const int64_t ncb = (xlim + kTileCh - 1) / kTileCh + (FUSED ? (a.C - a.hp + kTileCh - 1) / kTileCh : 0);
  const int64_t blocks = a.B * ntile * ncb;
  hipLaunchKernelGGL((conv_bwd_kernel<IO, FUSED>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
}

hipError_t launch_conv_fwd_kernel(int bf16, const ConvFwdArgs& a, dim3 grid, hipStream_t s) {
#define SSD_CONV_FWD(IO, KK)                                                          \
  if (a.K == KK) {                                                                    \
    hipLaunchKernelGGL((conv_fwd_kernel<IO, KK>), grid, dim3(256), 0, s, a);          \
    return hipGetLastError();                                                         \
  }
  if (bf16) {
    SSD_CONV_FWD(bf16_t, 4)
    SSD_CONV_FWD(bf16_t, 3)
    SSD_CONV_FWD(bf16_t, 2)
  } else {
    SSD_CONV_FWD(float, 4)
    SSD_CONV_FWD(float, 3)
    SSD_CONV_FWD(float, 2)
  }
#undef SSD_CONV_FWD
  return hipErrorInvalidValue;
}

hipError_t run_conv_bwd(ConvBwdArgs a, int bf16, bool fused, float* dw, float* db, int accumulate,
                        hipStream_t s) {
  const int64_t ntile = (a.L + kTileRows - 1) / kTileRows;
  TimingScope ts(kKConvBwd, s);
  if (bf16) {
    if (fused)
      launch_conv_bwd_kernel<bf16_t, true>(a, s);
    else
      launch_conv_bwd_kernel<bf16_t, false>(a, s);
  } else {
    if (fused)
      launch_conv_bwd_kernel<float, true>(a, s);
    else
      launch_conv_bwd_kernel<float, false>(a, s);
  }
  hipLaunchKernelGGL(conv_params_kernel, dim3(static_cast<unsigned>((a.C * 5 + kWave - 1) / kWave)),
                     dim3(256), 0, s, a.part, a.B * ntile, a.C, a.K, dw, db, accumulate);
  return hipGetLastError();
}

}  // namespace

size_t conv_bwd_partials_bytes(int64_t B, int64_t L, int64_t C) {
  const int64_t ntile = (L + kTileRows - 1) / kTileRows;
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
  a.split = C;  // one output
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
  return launch_conv_fwd_kernel(bf16, a, grid, s);
}

size_t bc_prepass_bytes(const Problem& pr) {
  if (pr.K == 0) return 0;
  const size_t n = static_cast<size_t>(pr.B) * pr.L * 2 * pr.G * pr.N * (pr.bf16 ? 2 : 4);
  return (n + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_bc_prepass(const Problem& pr, void* dst, void* dst_lo, hipStream_t s, int kind) {
  TimingScope ts(kind, s);
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

hipError_t launch_xbc_prepass(const Problem& pr, void* xp, void* bc, void* bc_lo, hipStream_t s) {
  TimingScope ts(kKXbcPrepass, s);
  const int hp = pr.H * pr.P, gn2 = 2 * pr.G * pr.N, C = hp + gn2;
  ConvFwdArgs a{};
  a.B = pr.B;
  a.L = pr.L;
  a.C = C;
  a.K = pr.K;
  a.silu = 1;
  a.x = pr.xbc.p;
  a.x_sb = pr.xbc.sb;
  a.x_st = pr.xbc.st;
  a.x_c0 = 0;
  a.st = pr.cs_in.p;
  a.st_sb = pr.cs_in.sb;
  a.st_st = pr.cs_in.st;
  a.st_c0 = 0;
  a.w = pr.conv_w;
  a.bias = pr.conv_b;
  a.out = xp;
  a.o_sb = pr.L * hp;
  a.o_st = hp;
  a.o_c0 = 0;
  a.out_lo = nullptr;
  a.split = hp;
  a.out2 = bc;
  a.o2_sb = pr.L * gn2;
  a.o2_st = gn2;
  a.out2_lo = pr.bf16 ? bc_lo : nullptr;
  const int V = pr.bf16 ? 8 : 4;
  const int64_t n = pr.B * ((pr.L + kRowsF - 1) / kRowsF) * (C / V);
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  return launch_conv_fwd_kernel(pr.bf16, a, grid, s);
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
