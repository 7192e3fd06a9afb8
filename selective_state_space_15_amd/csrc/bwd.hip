// Backward pass of the mixer hot path on gfx950: gradients of
//   out_t = y_t * silu(z_t),   y_t = h_t C_t + D x_t,
//   h_t = exp(dt_t A) h_{t-1} + dt_t x_t B_t^T          (Eq. (1) of the Video-Ma2mba
//   review, pith.science verdict for arXiv 2411.19460, in its selective form)
// with respect to x, B, C, dt (raw), z, A, D, dt_bias and h0, recomputing the
// forward from (h0, conv state) -- one segment of sequence-axis checkpointing.
//
// Chunked form (chunks of Q = 64, cs_t the chunk-local cumsum of l = dt A,
// H_{c-1} the state entering chunk c, dH_c the gradient of the state leaving it):
//   dy    = dout silu(z),   dz = dout y silu'(z)
//   dH_{c-1} = exp(cs_Q) dH_c + sum_t exp(cs_t) dy_t C_t^T            (reverse scan)
//   Mt[t,s] = (C_t . B_s) exp(cs_t - cs_s) dt_s          (s <= t)
//   W[t,s]  = (dy_t . x_s) exp(cs_t - cs_s) dt_s          (s <= t)
//   dx_s  = sum_t Mt[t,s] dy_t + exp(cs_Q - cs_s) dt_s dH_c B_s + D dy_s
//   dB_s  = sum_t W[t,s] C_t + exp(cs_Q - cs_s) dt_s x_s dH_c          (summed over heads)
//   dC_t  = sum_s W[t,s] B_s + exp(cs_t) dy_t H_{c-1}                 (summed over heads)
//   d cs_t (as independent variables):
//       + sum_s (C_t.B_s) e^{cs_t-cs_s} dt_s (dy_t.x_s)   - [same, summed over t] at s
//       + dy_t . exp(cs_t) H_{c-1} C_t                     (carried-state term)
//       - exp(cs_Q - cs_s) dt_s x_s^T dH_c B_s             (chunk-state term)
//       + [at the last row] <dH_c, H_c> = exp(cs_Q) <dH_c, H_{c-1}> + sum_s (previous term)
//   dl_r  = sum_{t >= r} dcs_t,   ddt_s = (direct terms) + A dl_s,   dA = sum dt dl,
//   dD = sum dy . x,   ddt_raw = ddt sigmoid(dt_raw + dt_bias),  ddt_bias = sum ddt_raw.
//
// Kernels: the chunk states, walked in groups of kG chunks (in-group prefix states and
// the state entering each group, by a scan over groups), and the dy C^T terms walked
// the same way in reverse (both in chunk_states.hip); scan_rev_kernel (reverse scan
// over groups, dh0); bwd_main_kernel (per chunk and block of heads of one group: H and
// dH from the in-group and group terms, every gradient above, dB / dC summed over the
// block's heads in registers and written as one fp32 partial per block); then the
// conv backward (or the dB / dC finalize without conv) and ordered parameter
// reductions.
#include "chunk_io.hpp"
#include "common.hpp"
#include "launch.hpp"

#ifndef SSD_BWD_EARLY_UNROLL
#define SSD_BWD_EARLY_UNROLL 2
#endif

namespace ssd {

hipError_t launch_conv_bwd_fused(const Problem& pr, const void* dx_ws, const float* dbc_sum,
                                 int per_g, View dcs_out, MView dxbc, float* dconv_w, float* dconv_b,
                                 MView dcs_in, int accumulate, void* ws, hipStream_t s);
size_t conv_bwd_partials_bytes(int64_t B, int64_t L, int64_t C);

namespace {

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

constexpr int kMaxHeadBlock = 32;  // heads per bwd_main workgroup, at most
constexpr int kDtTab = 8;          // heads whose dt / cs tables are in LDS at a time

struct BwdArgs {
  Problem pr;
  int64_t nch;
  int hb_heads;            // heads per block (all in one group)
  int nhb;                 // blocks of heads
  // States in chunk groups of kG chunks (chunk_states.hip): for chunk c of group g,
  //   H_{c-1} = P_{c-1} + exp(l_{c0} + .. + l_{c-1}) H_in(g)   (no P term at c = c0)
  //   dH_c    = Q_c + exp(l_{c+1} + .. + l_{c1}) dH_out(g)      (no Q term at c = c1)
  // [B][nch][H][P][N] in-group prefix states P_c and suffix gradients Q_c: fp32 for
  // fp32 I/O; fp16 for bf16 I/O, restored by the factors Psc / Qsc
  // [B][nch][H][state_scale_blocks] (one per block of 16 rows x state_scale_cols)
  const void* Ps;
  const void* Qs;
  const float* Psc;
  const float* Qsc;
  const float* Hin;        // [B][ngr][H][P][N] state entering each group
  const float* dHout;      // [B][ngr][H][P][N] gradient leaving each group
  const float* lsum;       // [B][nch][H] chunk log-decay
  int64_t ngr;
  View dout;
  MView dx;                // x-channel gradients [B][L][H*P] (dxbc itself, or scratch)
  MView dz;
  MView ddt;
  float* dbc_part;         // [nhb][B][L][2N] fp32
  float* par_part;         // [B][nch][H][3]: dA, dD, ddt_bias partials
};

// ------------------------------------------------------------------ reverse scan
// dHs[c] <- gradient leaving step c (a group of chunks here); g runs
// dH_{c-1} = exp(lsum_c) dH_c + dS_c, with lsum_c and dS_c the step's total log-decay
// and its own gradient term.
// Each thread owns 4 consecutive state elements of one head, 8 chunks of loads in flight.
__device__ __forceinline__ float4 axpy4(float a, const float4& x, const float4& y) {
  return make_float4(fmaf(a, x.x, y.x), fmaf(a, x.y, y.y), fmaf(a, x.z, y.z), fmaf(a, x.w, y.w));
}

__global__ void __launch_bounds__(256) scan_rev_kernel(const float* dh_final, float* dHs,
                                                       const float* lsum, float* dh0, int64_t B,
                                                       int H, int64_t PN, int64_t nch) {
  const int64_t e4 = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  const int64_t per_b = H * PN;
  if (e4 * 4 >= B * per_b) return;
  const int64_t e = e4 * 4;
  const int64_t b = e / per_b, rem = e % per_b;
  const int h = static_cast<int>(rem / PN);
  float4 gcur = dh_final ? *reinterpret_cast<const float4*>(dh_final + e) : make_float4(0.f, 0.f, 0.f, 0.f);
  float* base = dHs + b * nch * per_b + rem;
  const float* lb = lsum + b * nch * H + h;
  int64_t c = nch - 1;
  for (; c >= 7; c -= 8) {
    float4 sv[8];
    float l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sv[i] = *reinterpret_cast<const float4*>(base + (c - i) * per_b);
      l[i] = lb[(c - i) * H];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<float4*>(base + (c - i) * per_b) = gcur;
      gcur = axpy4(__expf(l[i]), gcur, sv[i]);
    }
  }
  for (; c >= 0; --c) {
    const float4 sv = *reinterpret_cast<const float4*>(base + c * per_b);
    *reinterpret_cast<float4*>(base + c * per_b) = gcur;
    gcur = axpy4(__expf(lb[c * H]), gcur, sv);
  }
  if (dh0) *reinterpret_cast<float4*>(dh0 + e) = gcur;
}

// ------------------------------------------------------------------ main
// Launch shape: NW = 4 waves (one per SIMD; every wave computes a 16-row strip of
// each product across all of its columns) or NW = 8 (two per SIMD; waves w and w+4
// share strip w % 4 and take one half of the columns each, so each SIMD has a
// second instruction stream to issue while the other waits on LDS, MFMA or memory
// latency).  Row sums over columns are then kept per half and added in (f).
template <int NW>
struct MainShape {
  static constexpr int threads = NW * kWave;
  static constexpr int halves = NW / 4;
  // with one wave per SIMD there are registers to spare: unroll the MFMA K loops so
  // operand reads overlap the MFMAs
  static constexpr int unroll = NW == 4 ? 2 : 1;
};

template <typename IO, int P, int N, int NW>
__global__ void __launch_bounds__(NW * kWave) bwd_main_kernel(BwdArgs a) {
  using T = io_traits<IO>;
  using E = typename T::elem;
  using Lt = typename T::lds;
  constexpr int kThreads = MainShape<NW>::threads;
  constexpr int NHALF = MainShape<NW>::halves;
  constexpr int kMainUnroll = MainShape<NW>::unroll;
  // (a) and (b) run while no next-head prefetch is held in registers: their K loops are
  // unrolled so that the fragment reads of later K-steps issue ahead of the MFMAs
  constexpr int kEarlyUnroll = SSD_BWD_EARLY_UNROLL;
  constexpr int PADK = 16 / sizeof(Lt);
  constexpr int ldN = N + PADK, ldQ = kQ + PADK, ldP = P + PADK;
  constexpr int NTn = N / 16, PJ = P / 16;
  // 16-column tiles per wave: P columns, Q (= 64) columns, N columns
  constexpr int PJw = PJ / NHALF, QJw = 4 / NHALF, NTw = NTn / NHALF;
  static_assert(PJ % NHALF == 0 && NTn % NHALF == 0, "column halves must be whole tiles");
  __shared__ __align__(16) Lt sC[kQ * ldN];   // C rows [t][n]
  __shared__ __align__(16) Lt sB[kQ * ldN];   // B rows [s][n]
  __shared__ __align__(16) Lt sX[kQ * ldP];   // x [s][p]
  // Mt and W stored transposed, [s][t]: a lane's four accumulator rows t are then one
  // 8-byte (bf16) or 16-byte (fp32) piece of a row
  __shared__ __align__(16) Lt sM[kQ * ldQ];   // Mt [s][t]
  __shared__ __align__(16) Lt sW[kQ * ldQ];   // W  [s][t]
  __shared__ __align__(16) Lt sDY[kQ * ldP];  // dy [t][p]
  __shared__ __align__(16) Lt sH[P * ldN];    // H_{c-1} [p][n]
  __shared__ __align__(16) Lt sdH[P * ldN];   // dH_c [p][n]
  // bf16 I/O: dy and C also as low parts (v - bf16(v)), so the products that feed
  // the log-decay gradient most (dy x^T, C B^T, C H^T) run at about 16 bits
  constexpr bool SPLIT = sizeof(Lt) == 2;
  __shared__ __align__(16) Lt sDYlo[SPLIT ? kQ * ldP : 8];
  __shared__ __align__(16) Lt sClo[SPLIT ? kQ * ldN : 8];
  constexpr int ldG = P + 4;
  __shared__ __align__(16) float sG2[kQ * ldG];  // dout silu'(z) [t][p] (fp32)
  // per head of the block: dt and the chunk-local cumsum cs of dt A
  __shared__ __align__(16) float s_dtH[kDtTab][kQ];
  __shared__ __align__(16) float s_csH[kDtTab][kQ];
  // d dt / d dt_raw = sigmoid(dt_raw + dt_bias), tabulated with dt for bf16 I/O (the
  // fp32 tiles leave no LDS for it: there (f) computes it from dt)
  constexpr bool kSigTab = sizeof(Lt) == 2;
  __shared__ float s_sgH[kSigTab ? kDtTab : 1][kQ];
  __shared__ float s_row[NHALF][kQ], s_yo[NHALF][kQ], s_v[NHALF][kQ], s_col[4][kQ];
  // per-wave partials of <dH, H> and of dD, double-buffered by head parity: wave 0 reads
  // head h's in (f) while the other waves already stage head h + 1
  __shared__ float s_red[2][2][NW];
  __shared__ float s_par[2][kMaxHeadBlock];  // A, D of the block's heads
  // per head of the block: exp(l_{c0} + .. + l_{c-1}) and exp(l_{c+1} + .. + l_{c1})
  __shared__ float s_gdec[2][kMaxHeadBlock];

  const Problem& pr = a.pr;
  const int64_t total = static_cast<int64_t>(pr.B) * a.nch * a.nhb;
  const int64_t lid = xcd_remap(blockIdx.x, total);
  const int hb = static_cast<int>(lid % a.nhb);
  const int64_t c = (lid / a.nhb) % a.nch;
  const int b = static_cast<int>(lid / (static_cast<int64_t>(a.nhb) * a.nch));
  const int h_first = hb * a.hb_heads;
  const int g = h_first / (pr.H / pr.G);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int strip = wave % 4, hf = wave / 4;
  const int m0 = strip * 16;
  // first column of this wave's half: P, Q and N columns
  const int p0 = hf * PJw * 16, s0 = hf * QJw * 16, n0 = hf * NTw * 16;
  const int64_t t0 = c * kQ;
  const int64_t PN = static_cast<int64_t>(P) * N;
  // chunk group of c: chunks [c_lo, c_hi)
  const int64_t grp = c / kG, c_lo = grp * kG;
  const int64_t c_hi = c_lo + kG < a.nch ? c_lo + kG : a.nch;

  // Every global input of a head (dt, post-conv x rows, dout, z, H_{c-1}, dH_c) is
  // loaded into registers by prefetch(), issued for head h+1 in three parts while
  // head h runs its last three MFMA phases (dt / x / dout / z, then H, then dH: one
  // burst of all 23 loads per thread stalls the wave on the memory pipeline), and
  // moved into LDS at the start of head h+1, so the memory latency of a head hides
  // behind the previous head's compute.
  constexpr int V = T::vec;
  constexpr int NXV = P * kQ / (V * kThreads);  // 16-byte row vectors per thread
  static_assert(P * kQ % (V * kThreads) == 0, "the x / dout tiles must tile the block");
  constexpr int NH4 = (P * N + 4 * kThreads - 1) / (4 * kThreads);
  uint4 pf_x[NXV], pf_do[NXV], pf_z[NXV];
  // P_{c-1}, Q_c: 4 fp16 each (bf16 I/O, with their scale factors) or 4 fp32
  constexpr bool F16S = sizeof(E) == 2;
  using SV = std::conditional_t<F16S, uint2, uint4>;
  using SE = std::conditional_t<F16S, uint16_t, float>;
  SV hv[NH4], gv[NH4];
  float4 hg[NH4], gg[NH4];   // H_in, dH_out
  float hsc[NH4], gsc[NH4];  // the scale factors of hv, gv
  constexpr int SC = state_scale_cols(P, N), kSB = state_scale_blocks(P, N);
  // without conv, x is the raw xbc channels (fields selected one by one: a selected
  // struct copy of the kernel argument would go through scratch memory)
  const bool xpre = pr.xp.p != nullptr;
  const E* xs_p = static_cast<const E*>(xpre ? pr.xp.p : pr.xbc.p);
  const int64_t xs_sb = xpre ? pr.xp.sb : pr.xbc.sb, xs_st = xpre ? pr.xp.st : pr.xbc.st;
  // Every load is unconditional, from a clamped (valid) address, and nothing uses the
  // loaded values before stage(): rows past the end are zeroed there.  A select right
  // after a load would make the wave wait for it at the point of issue.
  const bool gate = pr.z.p != nullptr;
  // Global addresses are a uniform base (the chunk's first row; scalar registers)
  // plus a 32-bit per-thread offset (row strides are at most kMaxRowStride), which
  // keeps each address in one vector register.
  const E* xs_c = xs_p + b * xs_sb + t0 * xs_st;
  const E* dq_c = static_cast<const E*>(a.dout.p) + b * a.dout.sb + t0 * a.dout.st;
  // without a gate the z loads repeat the dout loads (and are not used)
  const E* zq_c = gate ? static_cast<const E*>(pr.z.p) + b * pr.z.sb + t0 * pr.z.st : dq_c;
  const int64_t zst = gate ? pr.z.st : a.dout.st;
  auto prefetch = [&](int h, int part) {
    if (part == 0)
#pragma unroll
    for (int q = 0; q < NXV; ++q) {
      const int i = threadIdx.x + q * kThreads;
      const uint32_t r = t0 + i / (P / V) < pr.L ? i / (P / V) : 0;
      const uint32_t cl = (i % (P / V)) * V;
      pf_x[q] = *byte_off(reinterpret_cast<const uint4*>(xs_c + h * P),
                          (r * static_cast<uint32_t>(xs_st) + cl) * sizeof(E));
      pf_do[q] = *byte_off(reinterpret_cast<const uint4*>(dq_c + h * P),
                           (r * static_cast<uint32_t>(a.dout.st) + cl) * sizeof(E));
      pf_z[q] = *byte_off(reinterpret_cast<const uint4*>(zq_c + h * P),
                          (r * static_cast<uint32_t>(zst) + cl) * sizeof(E));
    }
    // in-group terms P_{c-1} (c > c0) and Q_c (c < c1); where there is none, the
    // loads read a valid slot and are masked when staged
    const float* Hgg = a.Hin + ((b * a.ngr + grp) * pr.H + h) * PN;
    const float* dHgg = a.dHout + ((b * a.ngr + grp) * pr.H + h) * PN;
    const int64_t pslot = ((b * a.nch + (c > 0 ? c - 1 : 0)) * pr.H + h), qslot = (b * a.nch + c) * pr.H + h;
    const SE* Pg = static_cast<const SE*>(a.Ps) + pslot * PN;
    const SE* Qg = static_cast<const SE*>(a.Qs) + qslot * PN;
#pragma unroll
    for (int q = 0; q < NH4; ++q) {
      const uint32_t i = min((static_cast<int>(threadIdx.x) + q * kThreads) * 4, P * N - 4);
      // scale block of elements i .. i+3 (one row p, four columns n)
      const uint32_t blk = (i / N) / 16 * (N / SC) + (i % N) / SC;
      if (part == 1) {
        hv[q] = *reinterpret_cast<const SV*>(Pg + i);
        hg[q] = *reinterpret_cast<const float4*>(Hgg + i);
        if constexpr (F16S) hsc[q] = a.Psc[pslot * kSB + blk];
      }
      if (part == 2) {
        gv[q] = *reinterpret_cast<const SV*>(Qg + i);
        gg[q] = *reinterpret_cast<const float4*>(dHgg + i);
        if constexpr (F16S) gsc[q] = a.Qsc[qslot * kSB + blk];
      }
    }
  };
  prefetch(h_first, 0);
  prefetch(h_first, 1);
  prefetch(h_first, 2);
  // dt and cs of heads hh0 .. hh0 + kDtTab - 1 into the LDS tables: one wave per head,
  // one token per lane.  The raw dt, dt_bias and A of a group of heads are loaded one
  // group ahead (load_dt), unconditionally from clamped rows and heads, and used by
  // the next fill_dt: a use right after the loads would wait for them, and for every
  // store in flight.
  constexpr int DTW = (kDtTab + NW - 1) / NW;  // table rows per wave
  E dtn_raw[DTW];
  float dtn_bias[DTW], dtn_A[DTW];
  auto load_dt = [&](int hh0) {
    const uint32_t r = t0 + lane < pr.L ? lane : static_cast<uint32_t>(pr.L - 1 - t0);
#pragma unroll
    for (int k = 0; k < DTW; ++k) {
      const int i = wave + k * NW;
      const int hc = min(hh0 + i, a.hb_heads - 1);
      const int h = h_first + hc;
      dtn_raw[k] = *byte_off(static_cast<const E*>(pr.dt.p) + b * pr.dt.sb + t0 * pr.dt.st + h,
                             r * static_cast<uint32_t>(pr.dt.st) * sizeof(E));
      dtn_bias[k] = pr.dt_bias ? pr.dt_bias[h] : 0.f;
      dtn_A[k] = pr.A[h];
    }
  };
  auto fill_dt = [&]() {
    const bool live = t0 + lane < pr.L;
#pragma unroll
    for (int k = 0; k < DTW; ++k) {
      const int i = wave + k * NW;
      const float u = T::to_f(dtn_raw[k]) + dtn_bias[k];
      const float dtv = live ? (pr.softplus ? softplusf_(u) : u) : 0.f;
      const float cs = wave_incl_scan(dtv * dtn_A[k]);
      if (i < kDtTab) {
        s_dtH[i][lane] = dtv;
        s_csH[i][lane] = cs;
        if constexpr (kSigTab) s_sgH[i][lane] = pr.softplus ? 1.f / (1.f + __expf(-u)) : 1.f;
      }
    }
  };
  load_dt(0);
  fill_dt();
  load_dt(kDtTab);
  // the block's per-head parameters, read once (a load right where a head needs them
  // would stall that head on its latency)
  if (threadIdx.x < a.hb_heads) {
    const int h = h_first + threadIdx.x;
    float before = 0.f, after = 0.f;
    for (int64_t k = c_lo; k < c_hi; ++k) {
      const float l = a.lsum[(b * a.nch + k) * pr.H + h];
      if (k < c) before += l;
      if (k > c) after += l;
    }
    s_gdec[0][threadIdx.x] = __expf(before);
    s_gdec[1][threadIdx.x] = __expf(after);
    s_par[0][threadIdx.x] = pr.A[h];
    s_par[1][threadIdx.x] = pr.D ? pr.D[h] : 0.f;
  }

  // B and C rows of the group (post-conv), shared by every head of the block
  conv_rows<IO, P, N, false, true, true, kThreads>(pr, b, 0, g, t0, [&](int seg, int s, int cl, const float* o) {
    lds_put_row<IO>((seg == 1 ? sB : sC) + s * ldN + cl, o);
  });
  const bool clo = SPLIT && pr.bc_lo.p != nullptr;
  // B's low part too, where the dout silu'(z) tile (not yet in use) can hold a B tile:
  // C B^T, shared by every head of the block, is then (C + C_lo)(B + B_lo)^T less the
  // C_lo B_lo^T term, at about 16 bits
  constexpr bool kBlo = SPLIT && kQ * ldG * sizeof(float) >= kQ * ldN * sizeof(Lt);
  Lt* const sBlo = reinterpret_cast<Lt*>(sG2);
  if (clo) {
    Problem prl = pr;
    prl.bc = pr.bc_lo;
    conv_rows<IO, P, N, false, false, true, kThreads>(prl, b, 0, g, t0, [&](int, int s, int cl, const float* o) {
      lds_put_row<IO>(sClo + s * ldN + cl, o);
    });
    if constexpr (kBlo)
      conv_rows<IO, P, N, false, true, false, kThreads>(prl, b, 0, g, t0, [&](int, int s, int cl, const float* o) {
        lds_put_row<IO>(sBlo + s * ldN + cl, o);
      });
  }
  __syncthreads();
  f32x4 cb[QJw];  // (C B^T)[t in rows m0.., s in this wave's half]
#pragma unroll
  for (int j = 0; j < QJw; ++j) cb[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  mma_strip<Lt, true, true, QJw, kMainUnroll>(cb, sC, ldN, m0, sB, ldN, s0, N);
  if (clo) {
    mma_strip<Lt, true, true, QJw, kMainUnroll>(cb, sClo, ldN, m0, sB, ldN, s0, N);
    if constexpr (kBlo) mma_strip<Lt, true, true, QJw, kMainUnroll>(cb, sC, ldN, m0, sBlo, ldN, s0, N);
  }
  if constexpr (kBlo) __syncthreads();  // the first head's staging rewrites the B_lo tile

  f32x4 accdB[NTw], accdC[NTw];
#pragma unroll
  for (int j = 0; j < NTw; ++j) {
    accdB[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    accdC[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Head hs from the prefetch registers into LDS: x rows; dy = dout silu(z) (and its
  // low part); dout silu'(z); H_{c-1} and dH_c, with the wave's part of <dH, H>.
  // Masks are applied to the raw words and the gate is blended in arithmetically: a
  // per-element select around SiLU becomes a branch, and a branch here would make the
  // wave wait for every store in flight as well as for these loads.
  const float gw = gate ? 1.f : 0.f;
  auto stage_head = [&](int hs) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NXV; ++q) {
      const int i = threadIdx.x + q * kThreads;
      const int r = i / (P / V), cl = (i % (P / V)) * V;
      const bool ok = t0 + r < pr.L;  // rows past the end are zero
      *reinterpret_cast<uint4*>(sX + r * ldP + cl) = keep_if(ok, pf_x[q]);
      const uint4 dq = keep_if(ok, pf_do[q]);
      float dy[V], lo[V], g2[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const float dv = raw_elem<IO>(dq, v), zv = raw_elem<IO>(pf_z[q], v);
        dy[v] = dv * fmaf(gw, siluf_(zv), 1.f - gw);
        g2[v] = gw * dv * dsiluf_(zv);
        lo[v] = dy[v] - T::to_f(T::from_f(dy[v]));
      }
      lds_put_row<IO>(sDY + r * ldP + cl, dy);
      if constexpr (SPLIT) lds_put_row<IO>(sDYlo + r * ldP + cl, lo);
#pragma unroll
      for (int v = 0; v < V; v += 4)
        *reinterpret_cast<float4*>(sG2 + r * ldG + cl + v) = make_float4(g2[v], g2[v + 1], g2[v + 2], g2[v + 3]);
    }
    // H_{c-1} and dH_c from the in-group and group states (fp32, before rounding)
    const int hi = hs < a.hb_heads ? hs : a.hb_heads - 1;
    const float aH = s_gdec[0][hi], bD = s_gdec[1][hi];
    const bool useP = c > c_lo, useQ = c < c_hi - 1;
    float dot = 0.f;
#pragma unroll
    for (int q = 0; q < NH4; ++q) {
      const int i = (threadIdx.x + q * kThreads) * 4;
      if (NH4 * 4 * kThreads == P * N || i < P * N) {
        const int p = i / N, n = i % N;
        float4 pv, qv;
        if constexpr (F16S) {
          // A zero scale masks a slot (a slot without a term still holds finite values),
          // and the power-of-two scaling is exact; each fp16 -> fp32 conversion folds
          // into that fma (v_fma_mix_f32).
          const float ps = useP ? hsc[q] : 0.f, qs = useQ ? gsc[q] : 0.f;
          pv = make_float4(fmaf(h2f_lo(hv[q].x), ps, 0.f), fmaf(h2f_hi(hv[q].x), ps, 0.f),
                           fmaf(h2f_lo(hv[q].y), ps, 0.f), fmaf(h2f_hi(hv[q].y), ps, 0.f));
          qv = make_float4(fmaf(h2f_lo(gv[q].x), qs, 0.f), fmaf(h2f_hi(gv[q].x), qs, 0.f),
                           fmaf(h2f_lo(gv[q].y), qs, 0.f), fmaf(h2f_hi(gv[q].y), qs, 0.f));
        } else {
          const SV ph = keep_if(useP, hv[q]), qh = keep_if(useQ, gv[q]);
          pv = make_float4(__uint_as_float(ph.x), __uint_as_float(ph.y), __uint_as_float(ph.z), __uint_as_float(ph.w));
          qv = make_float4(__uint_as_float(qh.x), __uint_as_float(qh.y), __uint_as_float(qh.z), __uint_as_float(qh.w));
        }
        const float hf[4] = {fmaf(aH, hg[q].x, pv.x), fmaf(aH, hg[q].y, pv.y), fmaf(aH, hg[q].z, pv.z),
                             fmaf(aH, hg[q].w, pv.w)};
        const float df[4] = {fmaf(bD, gg[q].x, qv.x), fmaf(bD, gg[q].y, qv.y), fmaf(bD, gg[q].z, qv.z),
                             fmaf(bD, gg[q].w, qv.w)};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          sH[p * ldN + n + k] = T::to_lds(hf[k]);
          sdH[p * ldN + n + k] = T::to_lds(df[k]);
          dot += hf[k] * df[k];
        }
      }
    }
    dot = wave_sum(dot);
    if (lane == 0) s_red[hs & 1][0][wave] = dot;
  };
  stage_head(0);
  __syncthreads();

  // bf16 with two column tiles per wave: rows m0 .. m0 + 15, columns p0 .. p0 + 31 of a
  // [rows][cols] bf16 output from accumulator-layout values v[j][e] (tile j, row
  // 4 (lane / 16) + e).  For each pair of rows e, e + 1 the two tiles' packed pairs swap
  // odd and even 16-lane rows (v_permlane16_swap), so that each lane then holds two
  // rows of one column of 32 consecutive ones: every store writes 64-byte row pieces
  // (per-element stores write 32-byte ones).  Rows at or past L are skipped.
  constexpr bool kPairStore = sizeof(E) == 2 && PJw == 2;
  auto store_rows2 = [&](E* base, uint32_t st, const float (&v)[PJw][4]) __attribute__((always_inline)) {
    if constexpr (kPairStore)
#pragma unroll
    for (int ep = 0; ep < 4; ep += 2) {
      const uint32_t r0 = f2bf2(v[0][ep], v[0][ep + 1]), r1 = f2bf2(v[1][ep], v[1][ep + 1]);
      const auto y = __builtin_amdgcn_permlane16_swap(r0, r1, false, false);
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int row = m0 + 4 * (w + 2 * (lane >> 5)) + ep;
        const uint32_t col = p0 + (lane & 31);
        const uint32_t word = w == 0 ? y[0] : y[1];
        if (t0 + row < pr.L)
          *byte_off(base, (row * st + col) * static_cast<uint32_t>(sizeof(E))) =
              __builtin_bit_cast(E, static_cast<uint16_t>(word & 0xffffu));
        if (t0 + row + 1 < pr.L)
          *byte_off(base, ((row + 1) * st + col) * static_cast<uint32_t>(sizeof(E))) =
              __builtin_bit_cast(E, static_cast<uint16_t>(word >> 16));
      }
    }
  };

  for (int hh = 0; hh < a.hb_heads; ++hh) {
    const int h = h_first + hh;
    // the next head (the last head reloads and restages itself: no branch around the
    // prefetch or the staging)
    const int hn = hh + 1 < a.hb_heads ? hh + 1 : hh;
    const float Ah = s_par[0][hh];
    const float Dh = s_par[1][hh];
    if (hh > 0 && hh % kDtTab == 0) {
      // every wave, wave 0 with the previous head's (f) included, is past the barrier
      // that ends the previous iteration: the tables are free
      fill_dt();
      load_dt(hh + kDtTab);
      __syncthreads();
    }
    const float* s_dt = s_dtH[hh % kDtTab];
    const float* s_cs = s_csH[hh % kDtTab];
    // The head's per-lane scalars, read once: cs and dt at this lane's accumulator rows
    // t = m0 + acc_row(e) (four consecutive rows) and columns s = s0 + 16 j + acc_col().
    const float cs_last = s_cs[kQ - 1];
    float cst[4], dtt[4], css[QJw], dts[QJw];
    {
      const float4 c4 = *reinterpret_cast<const float4*>(s_cs + m0 + acc_row(0));
      const float4 d4 = *reinterpret_cast<const float4*>(s_dt + m0 + acc_row(0));
      cst[0] = c4.x; cst[1] = c4.y; cst[2] = c4.z; cst[3] = c4.w;
      dtt[0] = d4.x; dtt[1] = d4.y; dtt[2] = d4.z; dtt[3] = d4.w;
    }
#pragma unroll
    for (int j = 0; j < QJw; ++j) {
      css[j] = s_cs[s0 + 16 * j + acc_col()];
      dts[j] = s_dt[s0 + 16 * j + acc_col()];
    }
    // exp(cs_t) (carried-state terms) and, at rows s, the chunk-state decay
    // exp(cs_Q - cs_s) alone (dqe) and times dt_s (dqd)
    float ecs[4], dqe[4], dqd[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ecs[e] = __expf(cst[e]);
      dqe[e] = __expf(cs_last - cst[e]);
      dqd[e] = dqe[e] * dtt[e];
    }
    // dy (hi + lo) and dout silu'(z) at this lane's accumulator positions
    // (rows m0 + 4*(lane/16)+e, cols 16j + lane%16)
    float dyr[PJw][4], g2r[PJw][4];
#pragma unroll
    for (int j = 0; j < PJw; ++j) {
      acc_gather(dyr[j], sDY, ldP, m0, p0 + 16 * j);
      if constexpr (SPLIT) {
        float lo4[4];
        acc_gather(lo4, sDYlo, ldP, m0, p0 + 16 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) dyr[j][e] += lo4[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) g2r[j][e] = sG2[(m0 + acc_row(e)) * ldG + p0 + 16 * j + acc_col()];
    }

    // (a) Mt, y, dz, carried-state dcs term, dD
    // exp(cs_t - cs_s) masked, at the cb positions: no branch (exp(-inf) = 0 above the
    // diagonal, where the difference would also overflow)
    float lt[QJw][4];
#pragma unroll
    for (int j = 0; j < QJw; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = m0 + acc_row(e), s = s0 + 16 * j + acc_col();
        lt[j][e] = __expf(s <= t ? cst[e] - css[j] : -__builtin_inff());
      }
#pragma unroll
    for (int j = 0; j < QJw; ++j)
      lds_put4<IO>(sM + (s0 + 16 * j + acc_col()) * ldQ + m0 + acc_row(0), cb[j][0] * lt[j][0] * dts[j],
                   cb[j][1] * lt[j][1] * dts[j], cb[j][2] * lt[j][2] * dts[j], cb[j][3] * lt[j][3] * dts[j]);
    f32x4 yacc[PJw];
#pragma unroll
    for (int j = 0; j < PJw; ++j) yacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (clo)
      mma_strip2<Lt, true, true, PJw, kEarlyUnroll>(yacc, sC, sClo, ldN, m0, sH, ldN, p0, N);
    else
      mma_strip<Lt, true, true, PJw, kEarlyUnroll>(yacc, sC, ldN, m0, sH, ldN, p0, N);
    float yo_part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int j = 0; j < PJw; ++j) {
        yacc[j][e] *= ecs[e];
        yo_part[e] += dyr[j][e] * yacc[j][e];
      }
    }
    __syncthreads();
    mma_strip<Lt, false, false, PJw, kEarlyUnroll>(yacc, sM, ldQ, m0, sX, ldP, p0, kQ);
    float dD_part = 0.f;
    {
      E* dzp = a.dz.p ? static_cast<E*>(a.dz.p) + b * a.dz.sb + t0 * a.dz.st + h * P : nullptr;
      float dzv[PJw][4], xg[PJw][4];
#pragma unroll
      for (int j = 0; j < PJw; ++j) acc_gather(xg[j], sX, ldP, m0, p0 + 16 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = m0 + acc_row(e);
        E* dzr = dzp ? byte_off(dzp, (t * static_cast<uint32_t>(a.dz.st) + p0 + acc_col()) * sizeof(E)) : nullptr;
#pragma unroll
        for (int j = 0; j < PJw; ++j) {
          const float xv = xg[j][e];
          const float y = yacc[j][e] + Dh * xv;
          dD_part += dyr[j][e] * xv;
          dzv[j][e] = g2r[j][e] * y;
          if constexpr (!kPairStore)
            if (dzp && t0 + t < pr.L) dzr[16 * j] = T::from_f(dzv[j][e]);
        }
      }
      if constexpr (kPairStore)
        if (dzp) store_rows2(dzp, static_cast<uint32_t>(a.dz.st), dzv);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      yo_part[e] = row_sum16(yo_part[e]);
    if (acc_col() == 0)
#pragma unroll
      for (int e = 0; e < 4; ++e) s_yo[hf][m0 + acc_row(e)] = yo_part[e];
    dD_part = wave_sum(dD_part);
    if (lane == 0) s_red[hh & 1][1][wave] = dD_part;

    // (b) dYX = dY X^T, W, row / column sums of (C.B)(dy.x) e^{..} (dt)
    {
      f32x4 dyx[QJw];
#pragma unroll
      for (int j = 0; j < QJw; ++j) dyx[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (SPLIT)
        mma_strip2<Lt, true, true, QJw, kEarlyUnroll>(dyx, sDY, sDYlo, ldP, m0, sX, ldP, s0, P);
      else
        mma_strip<Lt, true, true, QJw, kEarlyUnroll>(dyx, sDY, ldP, m0, sX, ldP, s0, P);
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < QJw; ++j) {
        float csum = 0.f, wv[4];
        const int s = s0 + 16 * j + acc_col();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float wp = dyx[j][e] * lt[j][e];  // (dy_t.x_s) e^{cs_t-cs_s}, masked
          const float m2 = wp * cb[j][e];
          rs[e] += m2 * dts[j];
          csum += m2;
          wv[e] = wp * dts[j];
        }
        lds_put4<IO>(sW + s * ldQ + m0 + acc_row(0), wv[0], wv[1], wv[2], wv[3]);
        csum = col_sum4(csum);
        if (lane < 16) s_col[strip][s] = csum;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rs[e] = row_sum16(rs[e]);
      }
      if (acc_col() == 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) s_row[hf][m0 + acc_row(e)] = rs[e];
    }
    __syncthreads();

    // the next head's inputs go in flight now, behind the remaining MFMA work
    prefetch(h_first + hn, 0);
    // (c) dx rows s = m0..: Mt^T dY + exp(cs_Q - cs_s) dt_s B dH^T + D dy
    {
      f32x4 dxd[PJw], dxs[PJw];
#pragma unroll
      for (int j = 0; j < PJw; ++j) {
        dxd[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        dxs[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      mma_strip<Lt, true, false, PJw, kMainUnroll>(dxd, sM, ldQ, m0, sDY, ldP, p0, kQ);
      mma_strip<Lt, true, true, PJw, kMainUnroll>(dxs, sB, ldN, m0, sdH, ldN, p0, N);
      E* dxp = static_cast<E*>(a.dx.p) + b * a.dx.sb + t0 * a.dx.st + h * P;
      float dxv[PJw][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = m0 + acc_row(e);
        E* dxr = byte_off(dxp, (s * static_cast<uint32_t>(a.dx.st) + p0 + acc_col()) * sizeof(E));
#pragma unroll
        for (int j = 0; j < PJw; ++j) {
          dxv[j][e] = dxd[j][e] + dqd[e] * dxs[j][e] + Dh * dyr[j][e];
          if constexpr (!kPairStore)
            if (t0 + s < pr.L) dxr[16 * j] = T::from_f(dxv[j][e]);
        }
      }
      if constexpr (kPairStore) store_rows2(dxp, static_cast<uint32_t>(a.dx.st), dxv);
    }
    prefetch(h_first + hn, 1);
    // (d) dB rows s: W^T C + exp(cs_Q - cs_s) dt_s (X dH); chunk-state dcs term
    {
      f32x4 U[NTw];
#pragma unroll
      for (int j = 0; j < NTw; ++j) U[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      mma_strip<Lt, true, false, NTw, kMainUnroll>(U, sX, ldP, m0, sdH, ldN, n0, P);
      float vp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NTw; ++j) {
        float bg[4];
        acc_gather(bg, sB, ldN, m0, n0 + 16 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vp[e] += U[j][e] * bg[e];
          accdB[j][e] += dqd[e] * U[j][e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        vp[e] = row_sum16(vp[e]);
      if (acc_col() == 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) s_v[hf][m0 + acc_row(e)] = dqe[e] * vp[e];
      mma_strip<Lt, true, false, NTw, kMainUnroll>(accdB, sW, ldQ, m0, sC, ldN, n0, kQ);
    }
    prefetch(h_first + hn, 2);
    // (e) dC rows t: W B + exp(cs_t) dY H
    {
      mma_strip<Lt, false, false, NTw, kMainUnroll>(accdC, sW, ldQ, m0, sB, ldN, n0, kQ);
      f32x4 tmp[NTw];
#pragma unroll
      for (int j = 0; j < NTw; ++j) tmp[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      mma_strip<Lt, true, false, NTw, kMainUnroll>(tmp, sDY, ldP, m0, sH, ldN, n0, P);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < NTw; ++j) accdC[j][e] += ecs[e] * tmp[j][e];
    }
    __syncthreads();

    // (f) dcs -> dl (reverse cumsum) -> ddt, dA, ddt_bias (wave 0, one token per lane)
    if (wave == 0) {
      const int s = lane;
      const float dts = s_dt[s];
      const float colsum = s_col[0][s] + s_col[1][s] + s_col[2][s] + s_col[3][s];
      float vs = s_v[0][s], rsum = s_row[0][s], yo = s_yo[0][s];
#pragma unroll
      for (int k = 1; k < NHALF; ++k) {
        vs += s_v[k][s];
        rsum += s_row[k][s];
        yo += s_yo[k][s];
      }
      float dcs = rsum + yo - dts * colsum - dts * vs;
      float hdh = 0.f, dD_sum = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        hdh += s_red[hh & 1][0][w];
        dD_sum += s_red[hh & 1][1][w];
      }
      const float sum_dtv = wave_sum(dts * vs);
      if (s == kQ - 1) dcs += __expf(s_cs[kQ - 1]) * hdh + sum_dtv;
      // dl_s = sum_{t >= s} dcs_t = (sum of all) - (inclusive prefix at s) + dcs_s
      // (exact at the last lane, where the prefix is the sum itself)
      const float incl = wave_incl_scan(dcs);
      const float dl = (lane_value(incl, kWave - 1) - incl) + dcs;
      const float ddt = colsum + vs + Ah * dl;
      const bool valid = t0 + s < pr.L;
      // d softplus(u)/du = sigmoid(u) = 1 - exp(-softplus(u))
      float sig;
      if constexpr (kSigTab)
        sig = s_sgH[hh % kDtTab][s];
      else
        sig = pr.softplus ? -expm1f(-dts) : 1.f;
      const float ddt_raw = valid ? ddt * sig : 0.f;
      if (valid)
        *byte_off(static_cast<E*>(a.ddt.p) + b * a.ddt.sb + t0 * a.ddt.st + h,
                  s * static_cast<uint32_t>(a.ddt.st) * sizeof(E)) = T::from_f(ddt_raw);
      const float dA_part = wave_sum(dts * dl);
      const float db_part = wave_sum(ddt_raw);
      if (lane == 0) {
        float* pp = a.par_part + ((b * a.nch + c) * pr.H + h) * 3;
        pp[0] = dA_part;
        pp[1] = dD_sum;
        pp[2] = db_part;
      }
    }
    // The next head's staging writes none of what (f) reads (the per-wave partials are
    // double-buffered, the dt tables are refilled behind a barrier), so wave 0 finishes
    // (f) while the other waves stage; they meet at the barrier after the staging.
    stage_head(hh + 1);
    __syncthreads();
  }

  // dB (rows s) and dC (rows t) of the block's heads -> fp32 partial
  float* part = a.dbc_part + ((static_cast<int64_t>(hb) * pr.B + b) * pr.L + t0) * (2 * N);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t t = m0 + acc_row(e);
    if (t0 + t < pr.L)
#pragma unroll
      for (int j = 0; j < NTw; ++j) {
        part[t * (2 * N) + n0 + 16 * j + acc_col()] = accdB[j][e];
        part[t * (2 * N) + N + n0 + 16 * j + acc_col()] = accdC[j][e];
      }
  }
}

// dB / dC of each group = the sum of its head-block partials, in block order.
// Without conv the sums are the B / C channels of dxbc; with conv they are the
// post-conv gradient the conv backward reads, stored in place in the group's
// first slot.  One thread per 4 consecutive values.
template <typename IO, bool TO_DXBC>
__global__ void __launch_bounds__(256) dbc_reduce_kernel(Problem pr, float* part, int nhb,
                                                          MView dxbc) {
  using E = typename io_traits<IO>::elem;
  const int N = pr.N, G = pr.G;
  const int64_t q4 = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  const int64_t per_t = 2LL * G * N;  // B | C channels of one row
  if (q4 * 4 >= pr.B * pr.L * per_t) return;
  const int64_t e = q4 * 4;
  const int64_t ch = e % per_t, t = (e / per_t) % pr.L, b = e / (per_t * pr.L);
  const bool isC = ch >= static_cast<int64_t>(G) * N;
  const int g = static_cast<int>((isC ? ch - G * N : ch) / N);
  const int n = static_cast<int>((isC ? ch - G * N : ch) % N);
  const int per_g = nhb / G;
  const int64_t slot = static_cast<int64_t>(pr.B) * pr.L * (2 * N);
  float* p0 = part + (static_cast<int64_t>(g) * per_g) * slot + (b * pr.L + t) * (2 * N) +
              (isC ? N : 0) + n;
  float4 acc = *reinterpret_cast<const float4*>(p0);
  for (int q = 1; q < per_g; ++q) {
    const float4 v = *reinterpret_cast<const float4*>(p0 + q * slot);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  if constexpr (TO_DXBC) {
    const float f[4] = {acc.x, acc.y, acc.z, acc.w};
    E* dst = static_cast<E*>(dxbc.p) + b * dxbc.sb + t * dxbc.st + static_cast<int64_t>(pr.H) * pr.P + ch;
#pragma unroll
    for (int v = 0; v < 4; ++v) dst[v] = io_traits<IO>::from_f(f[v]);
  } else {
    *reinterpret_cast<float4*>(p0) = acc;
  }
}

// dA, dD, ddt_bias: ordered sums of the per-(batch, chunk) partials ([B*nch][H][3])
__global__ void __launch_bounds__(256) head_params_kernel(const float* par, int64_t B, int64_t nch,
                                                          int H, float* dA, float* dD,
                                                          float* ddt_bias, int accumulate) {
  const float acc = block_colsum(par, B * nch, 3LL * H);
  const int i = blockIdx.x * kWave + threadIdx.x;
  if (threadIdx.x >= kWave || i >= 3 * H) return;
  const int h = i / 3, k = i % 3;
  float* dst = k == 0 ? dA : (k == 1 ? dD : ddt_bias);
  if (!dst) return;
  dst[h] = accumulate ? dst[h] + acc : acc;
}

struct BwdLayout {
  size_t bc, bc_lo, xp, H, Hsc, lsum, dH, dHsc, Hg, dHg, glsum, dbc, par, dx, conv, total;
  int64_t nch, ngr;
  int hb_heads, nhb;
};

BwdLayout bwd_layout(const Problem& pr) {
  BwdLayout l{};
  l.nch = (pr.L + kQ - 1) / kQ;
  l.ngr = (l.nch + kG - 1) / kG;
  const int hpg = pr.H / pr.G;
  int hb = 1;
  for (int d = 1; d <= kMaxHeadBlock; ++d)
    if (hpg % d == 0) hb = d;
  l.hb_heads = hb;
  l.nhb = pr.H / hb;
  const size_t es = pr.bf16 ? 2 : 4;
  const size_t PN = static_cast<size_t>(pr.P) * pr.N;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  l.bc = take(bc_prepass_bytes(pr));
  l.bc_lo = take(pr.bf16 ? bc_prepass_bytes(pr) : 0);
  l.xp = take(x_prepass_bytes(pr));
  const size_t ss = pr.bf16 ? 2 : 4;  // slot state element: fp16 or fp32
  l.H = take(static_cast<size_t>(pr.B) * l.nch * pr.H * PN * ss);
  const size_t nsb = pr.bf16 ? state_scale_blocks(pr.P, pr.N) : 0;
  l.Hsc = take(static_cast<size_t>(pr.B) * l.nch * pr.H * nsb * 4);
  l.lsum = take(static_cast<size_t>(pr.B) * l.nch * pr.H * 4);
  l.dH = take(static_cast<size_t>(pr.B) * l.nch * pr.H * PN * ss);
  l.dHsc = take(static_cast<size_t>(pr.B) * l.nch * pr.H * nsb * 4);
  l.Hg = take(static_cast<size_t>(pr.B) * l.ngr * pr.H * PN * 4);
  l.dHg = take(static_cast<size_t>(pr.B) * l.ngr * pr.H * PN * 4);
  l.glsum = take(static_cast<size_t>(pr.B) * l.ngr * pr.H * 4);
  l.dbc = take(static_cast<size_t>(l.nhb) * pr.B * pr.L * 2 * pr.N * 4);
  l.par = take(static_cast<size_t>(pr.B) * l.nch * pr.H * 3 * 4);
  l.dx = take(pr.K > 0 ? static_cast<size_t>(pr.B) * pr.L * pr.H * pr.P * es : 0);
  const int64_t cd = static_cast<int64_t>(pr.H) * pr.P + 2LL * pr.G * pr.N;
  l.conv = take(pr.K > 0 ? conv_bwd_partials_bytes(pr.B, pr.L, cd) : 0);
  l.total = off;
  return l;
}

template <typename IO, int P, int N>
hipError_t run_bwd(const Problem& pr, const BwdIn& in, const BwdOut& o, char* ws,
                   const BwdLayout& l, hipStream_t s) {
  BwdArgs a{};
  a.pr = pr;
  a.nch = l.nch;
  a.hb_heads = l.hb_heads;
  a.nhb = l.nhb;
  void* Ps = ws + l.H;
  void* Qs = ws + l.dH;
  float* Psc = reinterpret_cast<float*>(ws + l.Hsc);
  float* Qsc = reinterpret_cast<float*>(ws + l.dHsc);
  float* Hg = reinterpret_cast<float*>(ws + l.Hg);
  float* dHg = reinterpret_cast<float*>(ws + l.dHg);
  float* lsum = reinterpret_cast<float*>(ws + l.lsum);
  float* glsum = reinterpret_cast<float*>(ws + l.glsum);
  a.Ps = Ps;
  a.Qs = Qs;
  a.Psc = Psc;
  a.Qsc = Qsc;
  a.Hin = Hg;
  a.dHout = dHg;
  a.lsum = lsum;
  a.ngr = l.ngr;
  a.dout = in.dout;
  a.dz = o.dz;
  a.ddt = o.ddt;
  a.dbc_part = reinterpret_cast<float*>(ws + l.dbc);
  a.par_part = reinterpret_cast<float*>(ws + l.par);
  const int64_t hp = static_cast<int64_t>(pr.H) * pr.P;
  if (pr.K > 0) {
    a.dx = MView{ws + l.dx, pr.L * hp, hp};
  } else {
    a.dx = o.dxbc;  // x channels come first in dxbc rows
  }
  const int64_t PN = static_cast<int64_t>(P) * N;
  const int64_t ne = pr.B * pr.H * PN;
  // 1. in-group prefix states and, by a scan over groups, the state entering each group;
  // with bf16 I/O and a conv the state walk also convolves x and writes the post-conv
  // rows that step 4 reads
  const MView xp_out = pr.bf16 && pr.K > 0 ? MView{ws + l.xp, pr.L * hp, hp} : MView{nullptr, 0, 0};
  hipError_t e = launch_group_chunk_states(pr, l.nch, Ps, Psc, Hg, lsum, glsum, xp_out, s);
  if (e != hipSuccess) return e;
  // 2. in-group suffix gradients, 3. reverse scan over groups -> gradient leaving each
  // group, dh0
  e = launch_group_dstates(pr, l.nch, in.dout, Qs, Qsc, dHg, s);
  if (e != hipSuccess) return e;
  {
    TimingScope ts(kKScanRev, s);
    hipLaunchKernelGGL(scan_rev_kernel, dim3(static_cast<unsigned>((ne / 4 + 255) / 256)), dim3(256), 0,
                       s, in.dh_final, dHg, glsum, o.dh0, pr.B, pr.H, PN, l.ngr);
  }
  // 4. main
  {
    TimingScope ts(kKBwdMain, s);
    // two waves per SIMD where the column halves are whole tiles and the x / dout
    // tiles split evenly over 512 threads (bf16, P = 64, N >= 32)
    constexpr int NW = (sizeof(IO) == 2 && P == 64 && N >= 32) ? 8 : 4;
    hipLaunchKernelGGL((bwd_main_kernel<IO, P, N, NW>), dim3(static_cast<unsigned>(pr.B * l.nch * l.nhb)),
                       dim3(MainShape<NW>::threads), 0, s, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 5. dB / dC: head-block sums (and the conv backward); with one head block per group
  // and a conv, the partials already are the sums
  if (pr.K == 0 || l.nhb != pr.G) {
    const int64_t n4 = pr.B * pr.L * 2LL * pr.G * pr.N / 4;
    const dim3 grid(static_cast<unsigned>((n4 + 255) / 256));
    TimingScope ts(kKDbcReduce, s);
    if (pr.K > 0)
      hipLaunchKernelGGL((dbc_reduce_kernel<IO, false>), grid, dim3(256), 0, s, pr, a.dbc_part,
                         l.nhb, o.dxbc);
    else
      hipLaunchKernelGGL((dbc_reduce_kernel<IO, true>), grid, dim3(256), 0, s, pr, a.dbc_part,
                         l.nhb, o.dxbc);
  }
  if (pr.K > 0) {
    e = launch_conv_bwd_fused(pr, ws + l.dx, a.dbc_part, l.nhb / pr.G, in.dcs_out, o.dxbc,
                              o.dconv_w, o.dconv_b, o.dcs_in, o.accumulate, ws + l.conv, s);
    if (e != hipSuccess) return e;
  }
  // 6. parameter reductions
  TimingScope ts(kKParams, s);
  hipLaunchKernelGGL(head_params_kernel, dim3(static_cast<unsigned>((3 * pr.H + kWave - 1) / kWave)),
                     dim3(256), 0, s, a.par_part, pr.B, l.nch, pr.H, o.dA, o.dD, o.ddt_bias,
                     o.accumulate);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(const Problem& pr) { return bwd_layout(pr).total; }

bool bwd_supported(const Problem& pr) {
  // fp32 operands of the P x N state tiles do not fit the LDS budget at N = 128
  return pr.bf16 || pr.N <= 64;
}

hipError_t launch_bwd(const Problem& pr_in, const BwdIn& in, const BwdOut& o, void* ws_v,
                      hipStream_t s) {
  Problem pr = pr_in;
  char* ws = static_cast<char*>(ws_v);
  const BwdLayout l = bwd_layout(pr);
  if (pr.K > 0) {
    // bf16 I/O: the pre-pass convolves B and C only (the state walk convolves x);
    // fp32 I/O: x, B and C
    const hipError_t e = pr.bf16 ? launch_bc_prepass(pr, ws + l.bc, ws + l.bc_lo, s, kKXbcPrepass)
                                 : launch_xbc_prepass(pr, ws + l.xp, ws + l.bc, ws + l.bc_lo, s);
    if (e != hipSuccess) return e;
    const int64_t gn2 = 2LL * pr.G * pr.N;
    pr.bc = View{ws + l.bc, pr.L * gn2, gn2};
    if (pr.bf16) pr.bc_lo = View{ws + l.bc_lo, pr.L * gn2, gn2};
    const int64_t hp = static_cast<int64_t>(pr.H) * pr.P;
    pr.xp = View{ws + l.xp, pr.L * hp, hp};
  }
#define SSD_CASE(IO, PP, NN) \
  if (pr.P == PP && pr.N == NN) return run_bwd<IO, PP, NN>(pr, in, o, ws, l, s);
  if (pr.bf16) {
    SSD_CASE(bf16_t, 64, 128)
    SSD_CASE(bf16_t, 64, 64)
    SSD_CASE(bf16_t, 64, 32)
    SSD_CASE(bf16_t, 64, 16)
    SSD_CASE(bf16_t, 32, 128)
    SSD_CASE(bf16_t, 32, 64)
    SSD_CASE(bf16_t, 32, 32)
    SSD_CASE(bf16_t, 32, 16)
  } else {
    SSD_CASE(float, 64, 64)
    SSD_CASE(float, 64, 32)
    SSD_CASE(float, 64, 16)
    SSD_CASE(float, 32, 64)
    SSD_CASE(float, 32, 32)
    SSD_CASE(float, 32, 16)
  }
#undef SSD_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
