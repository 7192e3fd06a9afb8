// Forward pass of the mixer hot path on gfx950:
//   causal depthwise conv1d + SiLU (fused into the chunk loads)
//   -> chunked evaluation of the selective recurrence (Eq. (1) of the Video-Ma2mba
//      review, pith.science verdict for arXiv 2411.19460; selective form of the
//      Mamba-2 paper in that page's reference list)
//   -> SiLU(z) gate.
//
// Decomposition (obtained by unrolling the recurrence inside a chunk of Q steps,
// with cs_t the chunk-local cumulative sum of l = dt * A):
//   h_t = exp(cs_t) H_{c-1} + sum_{s <= t in chunk} exp(cs_t - cs_s) dt_s x_s B_s^T
//   y_t = sum_{s<=t} (C_t . B_s) exp(cs_t - cs_s) dt_s x_s      (intra-chunk, MFMA)
//       + exp(cs_t) H_{c-1} C_t                                  (carried state, MFMA)
//       + D x_t
//   H_c = exp(cs_{Q-1}) H_{c-1} + sum_s exp(cs_{Q-1} - cs_s) dt_s x_s B_s^T   (MFMA)
//
// Work split (the sequence is cut into sub-segments of `cps` chunks):
//   1. walk_kernel<STATE>: one workgroup per (batch, sub-segment, head) walks its
//      chunks from a zero state and writes the sub-segment's end state S_k and
//      its total log-decay.
//   2. scan_kernel: per state element, H_in(k+1) = exp(lsum_k) H_in(k) + S_k over
//      the sub-segments (a short sequential scan; 256 steps at L = 1M).
//   3. walk_kernel<OUT>: the same walk started from H_in(k), now producing y,
//      the gated output, the optional sequence checkpoints and h_final.
// The state stays in registers (MFMA accumulator layout) along each walk, so
// the only state traffic through memory is one state per sub-segment.
#include <type_traits>

#include "chunk_io.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace ssd {

namespace {

struct WalkArgs {
  Problem pr;
  int64_t cps, n_sub;
  float* ws_state;          // STATE: [B][n_sub][H][P][N] end states
  float* ws_lsum;           // STATE: [B][n_sub][H] total log-decay
  const float* init;        // OUT: initial states (null = zeros)
  int64_t init_sb, init_sk; // OUT: element strides of init per batch / sub-segment
  MView out;
  float* h_final;
  float* h_ckpt;
  int64_t ckpt_every;
};

constexpr int kModeState = 0;
constexpr int kModeOut = 1;

// Launch shape of the walks: two 4-wave workgroups per CU (2 waves per SIMD, up to
// 256 registers each; the output pass needs ~80 KB of LDS per workgroup).
// Independent workgroups on a CU overlap one's memory phase with the other's
// MFMA phase, which one larger workgroup cannot do across its own barriers.
template <int MODE>
struct WalkShape;
template <>
struct WalkShape<0> {
  static constexpr int waves = 4, waves_per_simd = 2;
};
template <>
struct WalkShape<1> {
  static constexpr int waves = 4, waves_per_simd = 2;
};

template <typename IO, int P, int N, int MODE>
__global__ void __launch_bounds__(WalkShape<MODE>::waves * 64)
    __attribute__((amdgpu_waves_per_eu(WalkShape<MODE>::waves_per_simd, WalkShape<MODE>::waves_per_simd)))
    walk_kernel(WalkArgs a) {
  constexpr int NW = WalkShape<MODE>::waves;
  constexpr int NTHR = NW * 64;
  using T = io_traits<IO>;
  using E = typename T::elem;
  using Lt = typename T::lds;
  constexpr bool OUT = MODE == kModeOut;
  constexpr int V = T::vec;
  constexpr int PADK = 16 / sizeof(Lt);
  constexpr int ldN = N + PADK, ldQ = kQ + PADK, ldP = P + PADK;
  // x and w o x are kept row-major ([s][p], 16-byte row stores); the products that
  // need them transposed read them with LDS transpose loads
  __shared__ __align__(16) Lt sB[kQ * ldN];
  __shared__ __align__(16) Lt sXw[kQ * ldP];
  // the C tile; in the output epilogue (C is dead by then) it holds y + D x as fp32
  constexpr int ldY = P + 4;
  constexpr size_t kCBytes = OUT ? kQ * ldN * sizeof(Lt) : 16;
  constexpr size_t kYBytes = OUT ? kQ * ldY * sizeof(float) : 16;
  __shared__ __align__(16) char sCY[kCBytes > kYBytes ? kCBytes : kYBytes];
  Lt* sC = reinterpret_cast<Lt*>(sCY);
  float* sY = reinterpret_cast<float*>(sCY);
  __shared__ __align__(16) Lt sX[OUT ? kQ * ldP : 8];
  __shared__ __align__(16) Lt sM[OUT ? kQ * ldQ : 8];
  __shared__ __align__(16) Lt sH[OUT ? P * ldN : 8];
  __shared__ __align__(16) float s_dt[kQ];
  __shared__ __align__(16) float s_cs[kQ];
  __shared__ float s_w[kQ];
  // state walk: w_s and the log-decay of every chunk of the sub-segment, computed
  // before the walk (one wave per chunk), so no chunk waits on a one-wave step
  constexpr int kMaxCps = 64;
  __shared__ float s_wall[OUT ? 1 : kMaxCps * kQ], s_lall[OUT ? 1 : kMaxCps];
  __shared__ float s_conv[P * 5];  // head h's conv taps (right-aligned on 4) and bias

  const Problem& pr = a.pr;
  const int64_t total = static_cast<int64_t>(pr.B) * a.n_sub * pr.H;
  const int64_t lid = xcd_remap(blockIdx.x, total);
  const int h = static_cast<int>(lid % pr.H);
  const int64_t k = (lid / pr.H) % a.n_sub;
  const int b = static_cast<int>(lid / (static_cast<int64_t>(pr.H) * a.n_sub));
  const int g = h / (pr.H / pr.G);
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const float Ah = pr.A[h];
  const float Dh = OUT && pr.D ? pr.D[h] : 0.f;
  const bool gate = OUT && pr.z.p != nullptr;

  // Output tiles (16x16) of the 64-row chunk products: row tile rt = wave % 4; with
  // 8 waves the columns are split in halves between waves w and w + 4.
  constexpr int HALVES = NW / 4;
  const int rt = wave % 4;
  const int m0 = rt * 16;
  const int half = wave / 4;
  constexpr int CBJ = 4 / HALVES;        // column tiles of C B^T per wave
  constexpr int YJ = (P / 16) / HALVES;  // column tiles of y per wave
  // State tiles (16x16 of the P x N state) owned by this wave
  constexpr int PT = P / 16, NT = N / 16, WPP = NW / PT, NJS = (NT + WPP - 1) / WPP;
  const int s_pi = wave % PT;
  const int s_nj0 = (wave / PT) * NJS;
  const bool s_owns = s_nj0 < NT;
  const int64_t PN = static_cast<int64_t>(P) * N;

  // the head's conv taps and bias, once per workgroup (read by every chunk's loads)
  if (pr.K > 0 && !(pr.xp.p && !OUT))
    for (int i = threadIdx.x; i < P * 5; i += NTHR) {
      const int cl = i / 5, j = i % 5, c = h * P + cl;
      const int kk = j - (4 - pr.K);
      s_conv[i] = j == 4 ? (pr.conv_b ? pr.conv_b[c] : 0.f) : (kk >= 0 ? pr.conv_w[c * pr.K + kk] : 0.f);
    }

  f32x4 accH[NJS];
  {
    const float* init = nullptr;
    if constexpr (OUT)
      if (a.init) init = a.init + b * a.init_sb + k * a.init_sk + h * PN;
#pragma unroll
    for (int j = 0; j < NJS; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = s_pi * 16 + acc_row(e);
        const int n = (s_nj0 + j) * 16 + acc_col();
        accH[j][e] = (init && s_owns) ? init[p * N + n] : 0.f;
      }
  }
  if constexpr (OUT) {
    if (s_owns)
#pragma unroll
      for (int j = 0; j < NJS; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sH[(s_pi * 16 + acc_row(e)) * ldN + (s_nj0 + j) * 16 + acc_col()] = T::to_lds(accH[j][e]);
  }

  // Everything a chunk reads from global memory (raw x rows, post-conv B/C rows,
  // dt) is prefetched into registers one chunk ahead, so those loads are in flight
  // while the previous chunk computes; z is loaded when the chunk is staged and used
  // in its epilogue.
  // dt of head h from the pre-pass table ([B][L][H] fp32, softplus applied)
  const float* dtp = pr.dtsp + b * pr.L * pr.H + h;
  const E* zp = OUT && gate ? static_cast<const E*>(pr.z.p) + b * pr.z.sb + h * P : nullptr;
  const int64_t tbeg = k * a.cps * kQ;
  // B/C rows per loader task: as many tasks as threads (every thread's loads are
  // issued, a task's or not)
  constexpr int RBL = (OUT ? 2 : 1) * (N / (16 / static_cast<int>(sizeof(E)))) * kQ / NTHR > 0
                          ? (OUT ? 2 : 1) * (N / (16 / static_cast<int>(sizeof(E)))) * kQ / NTHR
                          : 1;
  ChunkLoader<IO, P, N, false, true, OUT, NTHR, 1, RBL, false> ld;  // B (and C) rows
  // the state walk's second register set of B rows (it loads two chunks ahead)
  ChunkLoader<IO, P, N, false, true, OUT, NTHR, 1, RBL, false> ld2;
  // x rows: thread tid loads the XPT 16-byte vectors v = tid + NTHR i of the chunk's raw
  // 64 x P rows (row v / XV, columns V (v % XV)), one chunk ahead.  At the chunk they go
  // to LDS staging rows 3 .., behind the 3 rows before the chunk (the conv halo, kept
  // in registers since the previous chunk by the threads that loaded those rows), and
  // each conv task reads its rows from there: every x row is read from memory once.
  // (The forward has no post-conv x pre-pass: x is always raw here.)
  constexpr int XV = P / V;
  constexpr int XPT = kQ * XV / NTHR;
  static_assert(kQ * XV % NTHR == 0 && 3 * XV <= NTHR, "x vectors tile the threads");
  const E* xsrc = static_cast<const E*>(pr.xbc.p) + b * pr.xbc.sb + h * P;
  uint4 xr[XPT], xr2[XPT];  // xr2: the state walk's second set
  uint32_t xok = 0, xok2 = 0;
  uint4 xhalo = make_uint4(0u, 0u, 0u, 0u);
  const int vlast = static_cast<int>(threadIdx.x) + NTHR * (XPT - 1);
  const bool holds_halo = vlast >= (kQ - 3) * XV;  // rows kQ-3 .. kQ-1 of the chunk
  auto issue_x = [&](int64_t tn) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int v = static_cast<int>(threadIdx.x) + NTHR * i;
      const int64_t t = tn + v / XV;
      m |= (t < pr.L ? 1u : 0u) << i;
      xr[i] = *reinterpret_cast<const uint4*>(xsrc + (t < pr.L ? t : pr.L - 1) * pr.xbc.st + (v % XV) * V);
    }
    xok = m;
  };
  // the same into a given register set (the state walk's two sets)
  auto issue_x_into = [&](int64_t tn, uint4 (&xd)[XPT], uint32_t& okd) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int v = static_cast<int>(threadIdx.x) + NTHR * i;
      const int64_t t = tn + v / XV;
      m |= (t < pr.L ? 1u : 0u) << i;
      xd[i] = *reinterpret_cast<const uint4*>(xsrc + (t < pr.L ? t : pr.L - 1) * pr.xbc.st + (v % XV) * V);
    }
    okd = m;
  };
  // the halo of the walk's first chunk: rows tbeg-3 .. tbeg-1 of x, or of the carried
  // conv state before the sequence (zero before that, and without conv)
  if (holds_halo && pr.K > 0) {
    const int64_t t = k * a.cps * kQ - 3 + (vlast / XV - (kQ - 3));
    const int cv = (vlast % XV) * V;
    if (t >= 0) {
      xhalo = *reinterpret_cast<const uint4*>(xsrc + t * pr.xbc.st + cv);
    } else if (pr.cs_in.p && t >= -(pr.K - 1)) {
      const E* csi = static_cast<const E*>(pr.cs_in.p) + b * pr.cs_in.sb + h * P;
      xhalo = *reinterpret_cast<const uint4*>(csi + (t + pr.K - 1) * pr.cs_in.st + cv);
    }
  }
  // staging rows: the dead M tile (output walk) or a buffer of its own
  __shared__ __align__(16) uint4 sRawBuf[OUT ? 1 : (kQ + 3) * XV];
  static_assert(!OUT || (kQ + 3) * XV * 16 <= sizeof(Lt) * kQ * ldQ, "x staging fits the M tile");
  uint4* const sRaw = OUT ? reinterpret_cast<uint4*>(sM) : sRawBuf;
  float dt_pre = 0.f;
  // gate inputs of this thread's output vectors (row k / (P / V), columns
  // V (k % (P / V)) for k = tid + NTHR q), loaded one chunk phase ahead as 16-byte rows
  constexpr int NYV = (kQ * P / V + NTHR - 1) / NTHR;
  uint4 zr[OUT ? NYV : 1];
  // without a gate the (unused) loads read x rows, which are always valid
  const E* zsrc = zp ? zp : static_cast<const E*>(pr.xbc.p) + b * pr.xbc.sb;
  const int64_t zst = zp ? pr.z.st : pr.xbc.st;
  auto prefetch_z = [&](int64_t tn) {
    if constexpr (OUT) {
#pragma unroll
      for (int q = 0; q < NYV; ++q) {
        const int k = min(static_cast<int>(threadIdx.x) + NTHR * q, kQ * P / V - 1);
        const int r = k / (P / V), col = (k % (P / V)) * V;
        // rows past the end read row 0 and are never stored; no select after the
        // load, so it stays in flight until the epilogue
        const int64_t t = tn + r < pr.L ? tn + r : 0;
        zr[q] = *reinterpret_cast<const uint4*>(zsrc + t * zst + col);
      }
    }
  };
  // dt of the next chunk (unconditional, from a clamped row: a load under a branch
  // would be waited for at once, and with it every load still in flight; rows past
  // the end are masked in (1)).  Every wave loads it (no branch); wave 0 uses it.
  auto prefetch = [&](int64_t tn) {
    const uint32_t r = tn + lane < pr.L ? lane : static_cast<uint32_t>(pr.L - 1 - tn);
    dt_pre = *byte_off(dtp + tn * pr.H, r * static_cast<uint32_t>(pr.H) * sizeof(float));
  };
  if constexpr (OUT) {
    prefetch(tbeg);
  } else {
    // every chunk's dt (16 chunks per wave at most: all loads first, then the scans)
    constexpr int kPer = kMaxCps / NW;
    float dtr[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t t = tbeg + (wave + NW * i) * kQ + lane;
      dtr[i] = dtp[(t < pr.L ? t : pr.L - 1) * pr.H];
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ci = wave + NW * i;
      const int64_t t = tbeg + ci * kQ + lane;
      const float dtv = ci < a.cps && t < pr.L ? dtr[i] : 0.f;
      const float cs = wave_incl_scan(dtv * Ah);
      const float csl = lane_value(cs, kWave - 1);
      s_wall[ci * kQ + lane] = dtv * __expf(csl - cs);
      if (lane == 0) s_lall[ci] = csl;
    }
    __syncthreads();
  }
  // post-conv x (SiLU; taps right-aligned on 4 in s_conv) of XPT rows per task from
  // the staged raw rows of chunk c: sX = x (output walk), sXw = x * w_s; rows past the
  // end are zero
  auto conv_rows = [&](int64_t c, int64_t t0) __attribute__((always_inline)) {
    const int cg = static_cast<int>(threadIdx.x) % XV, r0 = (static_cast<int>(threadIdx.x) / XV) * XPT;
    const int cl = cg * V;
    uint4 raw[XPT + 3];
#pragma unroll
    for (int i = 0; i < XPT + 3; ++i) raw[i] = sRaw[(r0 + i) * XV + cg];
    // with or without conv as one uniform branch around the whole tile: a branch per
    // element would cut the tile into blocks, and with it the overlap of the
    // elements' exp / reciprocal latencies
    auto tile = [&](auto conv_tag) __attribute__((always_inline)) {
      constexpr bool CONV = decltype(conv_tag)::value;
      float w4[4][V], bias[V];
      if constexpr (CONV)
#pragma unroll
        for (int v = 0; v < V; ++v) {
#pragma unroll
          for (int j = 0; j < 4; ++j) w4[j][v] = s_conv[(cl + v) * 5 + j];
          bias[v] = s_conv[(cl + v) * 5 + 4];
        }
#pragma unroll
      for (int r = 0; r < XPT; ++r) {
        float o[V], ow[V];
        const bool live = t0 + r0 + r < pr.L;
        const float ws = live ? (OUT ? s_w[r0 + r] : s_wall[c * kQ + r0 + r]) : 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          float val;
          if constexpr (CONV) {
            float pre = bias[v];
#pragma unroll
            for (int j = 0; j < 4; ++j) pre = fmaf(w4[j][v], raw_elem<IO>(raw[r + j], v), pre);
            val = siluf_(pre);
          } else {
            val = raw_elem<IO>(raw[r + 3], v);
          }
          o[v] = live ? val : 0.f;
          ow[v] = o[v] * ws;
        }
        if constexpr (OUT) lds_put_row<IO>(sX + (r0 + r) * ldP + cl, o);
        lds_put_row<IO>(sXw + (r0 + r) * ldP + cl, ow);
      }
    };
    if (pr.K > 0)
      tile(std::true_type{});
    else
      tile(std::false_type{});
  };
  issue_x(tbeg);
  ld.issue_raw(pr, b, h, g, tbeg);

  float lsum = 0.f;
  if constexpr (OUT) {
    // the output walk: each chunk's rows loaded one chunk ahead (its registers hold one set)
    for (int64_t c = 0; c < a.cps; ++c) {
      const int64_t t0 = tbeg + c * kQ;
      if (t0 >= pr.L) break;
      if constexpr (OUT) {
        if (a.h_ckpt && t0 % a.ckpt_every == 0 && s_owns) {
          float* dst = a.h_ckpt + ((t0 / a.ckpt_every) * pr.B + b) * pr.H * PN + h * PN;
#pragma unroll
          for (int j = 0; j < NJS; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              dst[(s_pi * 16 + acc_row(e)) * N + (s_nj0 + j) * 16 + acc_col()] = accH[j][e];
        }
      }
      // (1) dt (softplus applied by the pre-pass), l = dt * A, chunk-local cumsum (wave 0)
      if (OUT && wave == 0) {
        const float dtv = t0 + lane < pr.L ? dt_pre : 0.f;
        const float cs = wave_incl_scan(dtv * Ah);
        const float csl = lane_value(cs, kWave - 1);
        s_dt[lane] = dtv;
        s_cs[lane] = cs;
        s_w[lane] = dtv * __expf(csl - cs);
      }
      // (2) conv + stores into LDS (the raw rows are staged while wave 0 finishes (1);
      // one barrier then covers both)
      //   sX[s][p] = x (OUT only), sXw[s][p] = x * w_s, sB[s][n], sC[s][n] (OUT only)
      // z first: the epilogue's wait for it then leaves the next chunk's loads, issued
      // after it, in flight
      prefetch_z(t0);
      // raw x rows (masked past the end) and the halo to the staging rows
#pragma unroll
      for (int i = 0; i < XPT; ++i) {
        const int v = static_cast<int>(threadIdx.x) + NTHR * i;
        sRaw[(3 + v / XV) * XV + v % XV] = keep_if((xok >> i) & 1u, xr[i]);
      }
      if (holds_halo) sRaw[(vlast / XV - (kQ - 3)) * XV + vlast % XV] = xhalo;
      xhalo = keep_if((xok >> (XPT - 1)) & 1u, xr[XPT - 1]);  // the next chunk's halo
      // B / C rows go to LDS as loaded (the tiles keep the I/O element type)
      static_assert(sizeof(Lt) == sizeof(E), "LDS tiles hold I/O elements");
      ld.consume_bc_raw([&](int seg, int s, int cl, const uint4& v) {
        *reinterpret_cast<uint4*>((seg == 1 ? sB : sC) + s * ldN + cl) = v;
      });
      __syncthreads();
      const float cs_last = s_cs[kQ - 1];
      lsum += cs_last;
      conv_rows(c, t0);
      // the next chunk's loads go in flight now, dt first (its wait in (1) then leaves
      // the row loads in flight); the last chunk reloads its own rows
      {
        const int64_t tn = c + 1 < a.cps && t0 + kQ < pr.L ? t0 + kQ : t0;
        if constexpr (OUT) prefetch(tn);
        issue_x(tn);
        ld.issue_raw(pr, b, h, g, tn);
      }
      __syncthreads();

      if constexpr (OUT) {
        // C B^T (-> masked, decayed, dt-scaled intra-chunk matrix Mt) and the carried-state
        // term C H_{c-1}^T in one pass over the C strip
        f32x4 yacc[YJ];
#pragma unroll
        for (int j = 0; j < YJ; ++j) yacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        float cst[4];
        {
          f32x4 cb[CBJ];
#pragma unroll
          for (int j = 0; j < CBJ; ++j) cb[j] = f32x4{0.f, 0.f, 0.f, 0.f};
          mma_strip_ab<Lt, true, true, CBJ, YJ>(cb, yacc, sC, ldN, m0, sB, ldN, 16 * CBJ * half, sH, ldN,
                                               16 * YJ * half, N);
          // cs at this lane's rows t = m0 + acc_row(e) (four consecutive) and cs, dt at its
          // columns s; the decay mask without a branch (exp(-inf) = 0 above the diagonal)
          const float4 c4 = *reinterpret_cast<const float4*>(s_cs + m0 + acc_row(0));
          cst[0] = c4.x; cst[1] = c4.y; cst[2] = c4.z; cst[3] = c4.w;
#pragma unroll
          for (int j = 0; j < CBJ; ++j) {
            const int s = 16 * CBJ * half + 16 * j + acc_col();
            const float css = s_cs[s], dts = s_dt[s];
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int t = m0 + acc_row(e);
              v[e] = cb[j][e] * __expf(s <= t ? cst[e] - css : -__builtin_inff()) * dts;
            }
            // Mt stored transposed, [s][t]: the lane's four rows are one packed piece
            lds_put4<IO>(sM + s * ldQ + m0 + acc_row(0), v[0], v[1], v[2], v[3]);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ecs = __expf(cst[e]);
#pragma unroll
          for (int j = 0; j < YJ; ++j) yacc[j][e] *= ecs;
        }
        // (3) H_c = exp(cs_last) H_{c-1} + (w o x)^T B in the registers now: the products
        // above took H_{c-1} from its LDS copy, which is replaced after the barrier, while
        // M X runs (one barrier per chunk fewer than replacing it at the chunk's end)
        if (s_owns) {
          const float decay = __expf(cs_last);
#pragma unroll
          for (int j = 0; j < NJS; ++j) accH[j] *= decay;
          mma_strip<Lt, false, false, NJS>(accH, sXw, ldP, s_pi * 16, sB, ldN, s_nj0 * 16, kQ);
        }
        __syncthreads();
        if (s_owns)
#pragma unroll
          for (int j = 0; j < NJS; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sH[(s_pi * 16 + acc_row(e)) * ldN + (s_nj0 + j) * 16 + acc_col()] = T::to_lds(accH[j][e]);
        mma_strip<Lt, false, false, YJ>(yacc, sM, ldQ, m0, sX, ldP, 16 * YJ * half, kQ);
        // y = Ydiag + exp(cs_t) Yoff + D x (fp32, through the dead C tile), then
        // out = y * silu(z) on 16-byte rows
        float xg[YJ][4];
#pragma unroll
        for (int j = 0; j < YJ; ++j) acc_gather(xg[j], sX, ldP, m0, 16 * (YJ * half + j));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = m0 + acc_row(e);
#pragma unroll
          for (int j = 0; j < YJ; ++j) {
            const int p = 16 * (YJ * half + j) + acc_col();
            sY[t * ldY + p] = yacc[j][e] + Dh * xg[j][e];
          }
        }
        __syncthreads();
        E* op = static_cast<E*>(a.out.p) + b * a.out.sb + h * P;
#pragma unroll
        for (int q = 0; q < NYV; ++q) {
          const int k = static_cast<int>(threadIdx.x) + NTHR * q;
          const int r = k / (P / V), col = (k % (P / V)) * V;
          if ((kQ * P / V) % NTHR == 0 || k < kQ * P / V) {
            float y[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
              y[v] = sY[r * ldY + col + v];
              if (gate) y[v] *= siluf_(raw_elem<IO>(zr[q], v));
            }
            if (t0 + r < pr.L) store_vec16<IO>(op + (t0 + r) * a.out.st + col, y);
          }
        }
      }
      __syncthreads();  // the next chunk's staging rewrites the tiles read above
    }
  } else {
    // The state walk: the rows of each chunk are loaded two chunks ahead, into two
    // register sets (it has the registers: under 200 of 256), set 1 for odd chunks.  The
    // chunks run in pairs with no branch between the two calls, so the compiler's load
    // counters see each set's loads in issue order and each chunk waits only for its
    // own set (a branch merging registers with loads in flight makes it wait for all).
    const int64_t nc = min(a.cps, (pr.L - tbeg + kQ - 1) / kQ);  // chunks of this walk
    {
      const int64_t t1 = nc > 1 ? tbeg + kQ : tbeg;  // (a one-chunk walk reloads its own)
      issue_x_into(t1, xr2, xok2);
      ld2.issue_raw(pr, b, h, g, t1);
    }
    auto step = [&](int64_t c, uint4 (&xd)[XPT], uint32_t& okd, auto& ldd) __attribute__((always_inline)) {
      const int64_t t0 = tbeg + c * kQ;
      // raw x rows (masked past the end) and the halo to the staging rows; B rows to LDS
#pragma unroll
      for (int i = 0; i < XPT; ++i) {
        const int v = static_cast<int>(threadIdx.x) + NTHR * i;
        sRaw[(3 + v / XV) * XV + v % XV] = keep_if((okd >> i) & 1u, xd[i]);
      }
      if (holds_halo) sRaw[(vlast / XV - (kQ - 3)) * XV + vlast % XV] = xhalo;
      xhalo = keep_if((okd >> (XPT - 1)) & 1u, xd[XPT - 1]);  // the next chunk's halo
      ldd.consume_bc_raw([&](int seg, int s, int cl, const uint4& v) {
        *reinterpret_cast<uint4*>(sB + s * ldN + cl) = v;
      });
      __syncthreads();
      const float cs_last = s_lall[c];
      lsum += cs_last;
      conv_rows(c, t0);
      // the rows two chunks ahead into the set just read (past the walk's last chunk
      // they reload this chunk's rows, which nothing reads)
      {
        const int64_t tn = c + 2 < nc ? t0 + 2 * kQ : t0;
        issue_x_into(tn, xd, okd);
        ldd.issue_raw(pr, b, h, g, tn);
      }
      __syncthreads();
      // (3) H_c = exp(cs_last) H_{c-1} + (w o x)^T B
      if (s_owns) {
        const float decay = __expf(cs_last);
#pragma unroll
        for (int j = 0; j < NJS; ++j) accH[j] *= decay;
        mma_strip<Lt, false, false, NJS>(accH, sXw, ldP, s_pi * 16, sB, ldN, s_nj0 * 16, kQ);
      }
      __syncthreads();  // the next chunk's staging rewrites the tiles read above
    };
    int64_t c = 0;
    for (; c + 1 < nc; c += 2) {
      step(c, xr, xok, ld);
      step(c + 1, xr2, xok2, ld2);
    }
    if (c < nc) step(c, xr, xok, ld);
  }

  if constexpr (!OUT) {
    float* dst = a.ws_state + ((b * a.n_sub + k) * pr.H + h) * PN;
    if (s_owns)
#pragma unroll
      for (int j = 0; j < NJS; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dst[(s_pi * 16 + acc_row(e)) * N + (s_nj0 + j) * 16 + acc_col()] = accH[j][e];
    if (threadIdx.x == 0) a.ws_lsum[(b * a.n_sub + k) * pr.H + h] = lsum;
  } else {
    if (a.h_final && k == a.n_sub - 1 && s_owns) {
      float* dst = a.h_final + (static_cast<int64_t>(b) * pr.H + h) * PN;
#pragma unroll
      for (int j = 0; j < NJS; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dst[(s_pi * 16 + acc_row(e)) * N + (s_nj0 + j) * 16 + acc_col()] = accH[j][e];
    }
  }
}

// Exclusive scan of the affine sub-segment maps: ws_state[k] <- H_in(k).  Each
// thread owns 4 consecutive state elements (one head: P*N is a multiple of 4) and
// keeps 8 steps of loads in flight.
__device__ __forceinline__ float4 axpy4(float a, const float4& x, const float4& y) {
  return make_float4(fmaf(a, x.x, y.x), fmaf(a, x.y, y.y), fmaf(a, x.z, y.z), fmaf(a, x.w, y.w));
}

__global__ void __launch_bounds__(256) scan_kernel(const float* h0, float* ws_state,
                                                   const float* ws_lsum, int64_t B, int H,
                                                   int64_t PN, int64_t n_sub) {
  const int64_t e4 = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  const int64_t per_b = H * PN;
  if (e4 * 4 >= B * per_b) return;
  const int64_t e = e4 * 4;
  const int64_t b = e / per_b, rem = e % per_b;
  const int h = static_cast<int>(rem / PN);
  float4 hc = h0 ? *reinterpret_cast<const float4*>(h0 + e) : make_float4(0.f, 0.f, 0.f, 0.f);
  float* base = ws_state + b * n_sub * per_b + rem;
  const float* lb = ws_lsum + b * n_sub * H + h;
  int64_t k = 0;
  for (; k + 8 <= n_sub; k += 8) {
    float4 sv[8];
    float l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sv[i] = *reinterpret_cast<const float4*>(base + (k + i) * per_b);
      l[i] = lb[(k + i) * H];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<float4*>(base + (k + i) * per_b) = hc;
      hc = axpy4(__expf(l[i]), hc, sv[i]);
    }
  }
  for (; k < n_sub; ++k) {
    const float4 sv = *reinterpret_cast<const float4*>(base + k * per_b);
    *reinterpret_cast<float4*>(base + k * per_b) = hc;
    hc = axpy4(__expf(lb[k * H]), hc, sv);
  }
}

template <typename IO>
__global__ void conv_state_out_kernel(Problem pr, MView dst) {
  using E = typename io_traits<IO>::elem;
  const int64_t km1 = pr.K - 1;
  const int64_t cd = static_cast<int64_t>(pr.H) * pr.P + 2LL * pr.G * pr.N;
  const int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (e >= pr.B * km1 * cd) return;
  const int64_t c = e % cd, j = (e / cd) % km1, b = e / (cd * km1);
  const int64_t tau = pr.L - km1 + j;
  E v;
  if (tau >= 0)
    v = static_cast<const E*>(pr.xbc.p)[b * pr.xbc.sb + tau * pr.xbc.st + c];
  else if (pr.cs_in.p)
    v = static_cast<const E*>(pr.cs_in.p)[b * pr.cs_in.sb + (tau + km1) * pr.cs_in.st + c];
  else
    v = E(0);
  static_cast<E*>(dst.p)[b * dst.sb + j * dst.st + c] = v;
}

// dt = softplus(dt_raw + dt_bias) (or the sum alone), once per (token, head) for both
// walks: fp32 [B][L][H], one element per thread.
template <typename IO>
__global__ void __launch_bounds__(256) dt_prepass_kernel(Problem pr, float* out) {
  using T = io_traits<IO>;
  using E = typename T::elem;
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= pr.B * pr.L * pr.H) return;
  const int h = static_cast<int>(i % pr.H);
  const int64_t t = (i / pr.H) % pr.L, b = i / (pr.H * pr.L);
  const float u = T::to_f(static_cast<const E*>(pr.dt.p)[b * pr.dt.sb + t * pr.dt.st + h]) +
                  (pr.dt_bias ? pr.dt_bias[h] : 0.f);
  out[i] = pr.softplus ? softplusf_(u) : u;
}

template <typename IO, int P, int N>
hipError_t run_walks(const Problem& pr, const FwdOut& o, const Plan& pl, float* ws_state,
                     float* ws_lsum, hipStream_t s) {
  WalkArgs a{};
  a.pr = pr;
  a.cps = pl.cps;
  a.n_sub = pl.n_sub;
  a.ws_state = ws_state;
  a.ws_lsum = ws_lsum;
  a.out = o.out;
  a.h_final = o.h_final;
  a.h_ckpt = o.h_ckpt;
  a.ckpt_every = o.ckpt_every > 0 ? o.ckpt_every : 1;
  const int64_t PN = static_cast<int64_t>(P) * N;
  const dim3 grid(static_cast<unsigned>(pr.B * pl.n_sub * pr.H));
  if (pl.n_sub > 1) {
    {
      TimingScope ts(kKWalkState, s);
      hipLaunchKernelGGL((walk_kernel<IO, P, N, kModeState>), grid,
                         dim3(WalkShape<kModeState>::waves * 64), 0, s, a);
    }
    const int64_t ne = pr.B * pr.H * PN;
    {
      TimingScope ts(kKScan, s);
      hipLaunchKernelGGL(scan_kernel, dim3(static_cast<unsigned>((ne / 4 + 255) / 256)), dim3(256), 0, s,
                         pr.h0, ws_state, ws_lsum, pr.B, pr.H, PN, pl.n_sub);
    }
    a.init = ws_state;
    a.init_sb = pl.n_sub * pr.H * PN;
    a.init_sk = pr.H * PN;
  } else {
    a.init = pr.h0;
    a.init_sb = pr.H * PN;
    a.init_sk = 0;
  }
  {
    TimingScope ts(kKWalkOut, s);
    hipLaunchKernelGGL((walk_kernel<IO, P, N, kModeOut>), grid, dim3(WalkShape<kModeOut>::waves * 64),
                       0, s, a);
  }
  return hipGetLastError();
}

template <typename IO>
hipError_t dispatch_pn(const Problem& pr, const FwdOut& o, const Plan& pl, float* st, float* ls,
                       hipStream_t s) {
#define SSD_CASE(PP, NN) \
  if (pr.P == PP && pr.N == NN) return run_walks<IO, PP, NN>(pr, o, pl, st, ls, s);
  SSD_CASE(64, 128)
  SSD_CASE(64, 64)
  SSD_CASE(64, 32)
  SSD_CASE(64, 16)
  SSD_CASE(32, 128)
  SSD_CASE(32, 64)
  SSD_CASE(32, 32)
  SSD_CASE(32, 16)
#undef SSD_CASE
  return hipErrorInvalidValue;
}

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

Plan make_plan(int64_t B, int64_t L, int H) {
  Plan pl{};
  pl.nchunks = (L + kQ - 1) / kQ;
  // workgroups: one round of resident walks (two per CU on 256 CUs).  More, shorter
  // sub-segments only add rounds, prologues and scan steps: at 8,192 tokens, 32 heads,
  // 2,048 walks of 2 chunks took 0.173 ms, 512 walks of 8 chunks 0.121 ms; at the
  // 80-head batch-16 shapes one walk per (batch, head) drops the state walk and the
  // scan (1.54 -> 1.12 ms at 4,096 tokens)
  const int64_t target = 512;
  int64_t want = (target + B * H - 1) / (B * H);
  if (want < 1) want = 1;
  int64_t cps = (pl.nchunks + want - 1) / want;
  if (cps < 1) cps = 1;
  if (cps > 64) cps = 64;
  pl.cps = cps;
  pl.n_sub = (pl.nchunks + cps - 1) / cps;
  return pl;
}

// Scratch layout: [B|C post-conv rows][dt table][sub-segment states][sub-segment log-decays]
size_t dt_table_bytes(const Problem& pr) {
  return align256(static_cast<size_t>(pr.B) * pr.L * pr.H * sizeof(float));
}

size_t fwd_workspace_bytes(const Problem& pr, const Plan& pl) {
  size_t n = bc_prepass_bytes(pr) + dt_table_bytes(pr);
  if (pl.n_sub > 1) {
    const size_t st = static_cast<size_t>(pr.B) * pl.n_sub * pr.H * pr.P * pr.N * sizeof(float);
    const size_t ls = static_cast<size_t>(pr.B) * pl.n_sub * pr.H * sizeof(float);
    n += align256(st) + align256(ls);
  }
  return n;
}

hipError_t launch_fwd(const Problem& pr_in, const FwdOut& o, const Plan& pl, void* ws,
                      hipStream_t s) {
  Problem pr = pr_in;
  char* w = static_cast<char*>(ws);
  hipError_t err = hipSuccess;
  if (pr.K > 0) {
    err = launch_bc_prepass(pr, w, nullptr, s);
    if (err != hipSuccess) return err;
    const int64_t gn2 = 2LL * pr.G * pr.N;
    pr.bc = View{w, pr.L * gn2, gn2};
    w += bc_prepass_bytes(pr);
  }
  {
    float* dts = reinterpret_cast<float*>(w);
    const int64_t n = pr.B * pr.L * pr.H;
    TimingScope ts(kKBcPrepass, s);
    if (pr.bf16)
      hipLaunchKernelGGL(dt_prepass_kernel<bf16_t>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                         s, pr, dts);
    else
      hipLaunchKernelGGL(dt_prepass_kernel<float>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                         s, pr, dts);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    pr.dtsp = dts;
    w += dt_table_bytes(pr);
  }
  float* st = reinterpret_cast<float*>(w);
  float* ls = nullptr;
  if (pl.n_sub > 1) {
    const size_t stb = static_cast<size_t>(pr.B) * pl.n_sub * pr.H * pr.P * pr.N * sizeof(float);
    ls = reinterpret_cast<float*>(w + align256(stb));
  }
  err = pr.bf16 ? dispatch_pn<bf16_t>(pr, o, pl, st, ls, s) : dispatch_pn<float>(pr, o, pl, st, ls, s);
  if (err != hipSuccess) return err;
  if (o.cs_out.p && pr.K > 1) err = launch_conv_state_out(pr, o.cs_out, s);
  return err;
}

// Chunk-group states for the backward pass: in-group prefix states P_c and group end
// states E_g (group_state_kernel), then the exclusive scan over groups from h0 turns
// E_g into H_in(g), the state entering group g, in place.
hipError_t launch_group_chunk_states(const Problem& pr, int64_t nch, void* Pst, float* Psc,
                                     float* Eg, float* lsum, float* glsum, MView xp_out,
                                     hipStream_t s) {
  const int64_t PN = static_cast<int64_t>(pr.P) * pr.N;
  hipError_t err = launch_group_local_states(pr, nch, Pst, Psc, Eg, lsum, glsum, xp_out, s);
  if (err != hipSuccess) return err;
  const int64_t ne = pr.B * pr.H * PN, ngr = (nch + kG - 1) / kG;
  {
    TimingScope ts(kKScanGroups, s);
    hipLaunchKernelGGL(scan_kernel, dim3(static_cast<unsigned>((ne / 4 + 255) / 256)), dim3(256), 0, s,
                       pr.h0, Eg, glsum, pr.B, pr.H, PN, ngr);
  }
  return hipGetLastError();
}

hipError_t launch_conv_state_out(const Problem& pr, MView dst, hipStream_t s) {
  const int64_t cd = static_cast<int64_t>(pr.H) * pr.P + 2LL * pr.G * pr.N;
  const int64_t ne = pr.B * (pr.K - 1) * cd;
  if (ne <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((ne + 255) / 256));
  TimingScope ts(kKConvStateOut, s);
  if (pr.bf16)
    hipLaunchKernelGGL(conv_state_out_kernel<bf16_t>, grid, dim3(256), 0, s, pr, dst);
  else
    hipLaunchKernelGGL(conv_state_out_kernel<float>, grid, dim3(256), 0, s, pr, dst);
  return hipGetLastError();
}

}  // namespace ssd
