// Per-chunk state contractions of the backward pass.
//
// Unrolling the selective recurrence (Eq. (1) of the Video-Ma2mba review,
// pith.science verdict for arXiv 2411.19460) over one chunk of Q tokens, with cs_t
// the chunk-local cumulative sum of dt * A, splits the state leaving chunk c and
// the gradient of the state entering it into a carried part and the chunk's own
// part:
//   H_c     = exp(cs_{Q-1}) H_{c-1} + S_c,   S_c[p][n]  = sum_s w_s x_s[p] B_s[n],
//             w_s = dt_s exp(cs_{Q-1} - cs_s);
//   dH_{c-1} = exp(cs_{Q-1}) dH_c   + dS_c,  dS_c[p][n] = sum_t exp(cs_t) dy_t[p] C_t[n],
//             dy = dout * silu(z) (dout alone without the gate).
// The chunk terms S_c and dS_c are independent across chunks.  Here they are summed
// along groups of kG consecutive chunks (one workgroup per group and block of heads,
// the walked state in MFMA accumulators), so that only one state per group goes
// through the scans; the per-chunk states inside a group are the in-group prefix
// (S) and suffix (dS) sums, completed with the group's carried state where the main
// backward kernel stages them.
//
// A workgroup takes one group of chunks and a block of heads of one group of B / C
// channels.  Each chunk's B rows (S) or C rows (dS) are staged in LDS once and reused
// by every head of the block; each (chunk, head) step's own rows (x, or dout and z)
// are loaded one step ahead, so they are in flight while the previous step's MFMA
// product is computed and stored.  With bf16 I/O and a conv, the S walk reads the raw
// x rows of all heads of its block a chunk ahead instead, convolves them (SiLU) at the
// chunk boundary and writes the post-conv rows for the main backward kernel, so the
// backward's pre-pass only convolves B and C.  bf16 I/O: dS is accumulated from split operands
// (dy_hi C_hi + dy_lo C_hi + dy_hi C_lo), since the state gradient feeds the
// log-decay gradient through an fp32 dot with H.
#include "chunk_io.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace ssd {

namespace {

constexpr int rows_per_task(int vec_per_row, int nthr) {
  return vec_per_row * kQ / nthr < 1 ? 1 : (vec_per_row * kQ / nthr > 8 ? 8 : vec_per_row * kQ / nthr);
}

// ------------------------------------------------------------------ chunk groups
// The contractions above, walked over a group of kG consecutive chunks per workgroup,
// so that the scans only see one state per group.  With l_c the log-decay of chunk c
// and groups [c0, c1]:
//   S walk (forward):   P_c = exp(l_c) P_{c-1} + S_c from P_{c0-1} = 0; P_c goes to
//                       slot c for c < c1 and E_g = P_{c1} to the group buffer;
//   dS walk (reverse):  Q_{c-1} = exp(l_c) Q_c + dS_c from Q_{c1} = 0; Q_c goes to
//                       slot c for c0 <= c < c1 and F_g = Q_{c0-1} to the group buffer.
// (Slot c1, read by no chunk, takes the slot-format copy of E_g / F_g.)  The group
// buffers are fp32; the slots are fp32 for fp32 I/O and, for bf16 I/O, fp16 with one
// power-of-two scale per block of 16 rows x state_scale_cols columns.
// The group scans then give H_in(g) (the state entering group g) and dH_out(g) (the
// gradient leaving it), and for chunk c of group g
//   H_{c-1} = P_{c-1} + exp(l_{c0} + .. + l_{c-1}) H_in(g)      (P_{c0-1} = 0)
//   dH_c    = Q_c + exp(l_{c+1} + .. + l_{c1}) dH_out(g)         (Q_{c1} = 0),
// which the main backward kernel forms when it stages H and dH.
struct GroupArgs {
  Problem pr;
  int64_t nch, ngr;
  int hb;         // heads per workgroup (divides H / G, at most GroupShape::max_heads)
  View dout;      // dS only
  void* out;      // [B][nch][H][P][N]: P_c (S) or Q_c (dS); bf16 I/O: fp16 times 2^k
  float* oscale;  // [B][nch][H][state_scale_blocks]: 2^-k, restoring a block (bf16 I/O)
  float* grp;     // [B][ngr][H][P][N]: E_g (S) or F_g (dS)
  float* lsum;    // S only: [B][nch][H] chunk log-decay
  float* glsum;   // S only: [B][ngr][H] group log-decay
  MView xp_out;   // S walk that convolves x itself: post-conv x rows [B][L][H*P] (bf16)
};

template <bool DS>
struct GroupShape {
  // the walked states of the block's heads stay in registers (16x16 fp32 tiles: 16 per
  // wave for 2 heads on 4 waves, 8 per wave for 2 heads on 8 waves); two waves per SIMD.
  // Two heads per workgroup keep enough workgroups for the 8-chunk groups.
  static constexpr int waves = DS ? 8 : 4;
  static constexpr int waves_per_simd = 2;
  static constexpr int max_heads = 2;
};

// HB heads per workgroup (a template parameter: the head loop is unrolled, so each
// head's state tiles are addressed statically, with no branch around the products)
// CX: the S walk reads raw x rows, convolves them (SiLU) itself and writes the
// post-conv rows to xp_out for the main backward kernel (bf16 I/O with a conv; the
// pre-pass then convolves only B and C).
template <typename IO, int P, int N, bool DS, int HB, bool CX = false>
__global__ void __launch_bounds__(GroupShape<DS>::waves * 64)
    __attribute__((amdgpu_waves_per_eu(GroupShape<DS>::waves_per_simd)))
    group_state_kernel(GroupArgs a) {
  constexpr int NW = GroupShape<DS>::waves;
  constexpr int NTHR = NW * 64;
  constexpr int HBM = HB;
  using T = io_traits<IO>;
  using E = typename T::elem;
  using Lt = typename T::lds;
  constexpr int V = T::vec;
  constexpr int PADK = 16 / sizeof(Lt);
  constexpr int ldN = N + PADK, ldP = P + PADK;
  constexpr bool SPLIT = DS && sizeof(Lt) == 2;
  // bf16 I/O keeps the slot states in fp16 (scaled); fp32 I/O keeps them in fp32
  constexpr bool F16S = sizeof(E) == 2;
  constexpr int SC = state_scale_cols(P, N), JB = SC / 16, kSB = state_scale_blocks(P, N);
  __shared__ __align__(16) Lt sK[kQ * ldN];                       // B or C rows [t][n]
  __shared__ __align__(16) Lt sKlo[SPLIT ? kQ * ldN : 8];         // C - bf16(C)
  __shared__ __align__(16) Lt sA[2][kQ * ldP];                    // w x or exp(cs) dy, [t][p]
  __shared__ __align__(16) Lt sAlo[SPLIT ? 2 : 1][SPLIT ? kQ * ldP : 8];
  __shared__ float s_w[HBM][kQ];                                  // w_s (S) or exp(cs_t) (dS)
  __shared__ float s_l[HBM];                                      // chunk log-decay per head
  // CX: a step's raw x rows behind the 3 rows before its chunk, and the block's conv
  // taps (right-aligned on 4) and biases
  constexpr int XVR = P / V;                    // 16-byte vectors per x row
  constexpr int CR = CX ? kQ * XVR / NTHR : 1;  // conv rows per task
  static_assert(!CX || (!DS && sizeof(E) == 2 && kQ * XVR % NTHR == 0 && 3 * XVR <= NTHR),
                "conv tasks tile the workgroup");
  __shared__ __align__(16) uint4 sRawG[CX ? HB : 1][CX ? (kQ + 3) * XVR : 1];
  __shared__ float s_cvw[CX ? HB * P * 5 : 1];

  const Problem& pr = a.pr;
  const int nhb = pr.H / HB;
  const int64_t total = pr.B * a.ngr * nhb;
  const int64_t lid = xcd_remap(blockIdx.x, total);
  const int hblk = static_cast<int>(lid % nhb);
  const int64_t grp = (lid / nhb) % a.ngr;
  const int b = static_cast<int>(lid / (static_cast<int64_t>(nhb) * a.ngr));
  const int hfirst = hblk * HB;
  const int g = hfirst / (pr.H / pr.G);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t c_lo = grp * kG;
  const int ng = static_cast<int>(min(static_cast<int64_t>(kG), a.nch - c_lo));  // chunks in the group
  const int nsteps = ng * HB;
  // walk order: step k = (chunk i, head hh), chunk c = c_lo + i (S) or c_lo + ng-1-i (dS)
  auto chunk_of = [&](int k) -> int64_t {
    const int i = k / HB;
    return DS ? c_lo + (ng - 1 - i) : c_lo + i;
  };

  const bool klo = SPLIT && pr.bc_lo.p != nullptr;

  constexpr int NDT = ((P / V) * kQ + NTHR - 1) / NTHR;
  uint4 dvr[NDT], zvr[DS ? NDT : 1];
  const View rows = DS ? a.dout : (pr.K > 0 && !CX ? pr.xp : pr.xbc);
  const E* dbase = static_cast<const E*>(rows.p) + b * rows.sb;
  const bool gate = DS && pr.z.p != nullptr;
  const float gw = gate ? 1.f : 0.f;
  const E* zbase = gate ? static_cast<const E*>(pr.z.p) + b * pr.z.sb : dbase;
  const int64_t zst = gate ? pr.z.st : rows.st;
  // rows of step k (unconditional loads from clamped rows; masked when staged)
  auto issue_step = [&](int k) {
    const int64_t c = chunk_of(k);
    const int h = hfirst + k % HB;
    const int64_t t0 = c * kQ;
#pragma unroll
    for (int q = 0; q < NDT; ++q) {
      const int task = min(static_cast<int>(threadIdx.x) + q * NTHR, (P / V) * kQ - 1);
      const int col = (task % (P / V)) * V, r = task / (P / V);
      const int64_t t = t0 + r < pr.L ? t0 + r : t0;
      dvr[q] = *reinterpret_cast<const uint4*>(dbase + t * rows.st + h * P + col);
      if constexpr (DS) zvr[q] = *reinterpret_cast<const uint4*>(zbase + t * zst + h * P + col);
    }
  };
  auto stage = [&](int k, int buf) __attribute__((always_inline)) {
    const int hh = k % HB;
    const int64_t t0 = chunk_of(k) * kQ;
    Lt* A = sA[buf];
    Lt* Alo = sAlo[SPLIT ? buf : 0];
#pragma unroll
    for (int q = 0; q < NDT; ++q) {
      const int task = threadIdx.x + q * NTHR;
      if ((P / V) * kQ % NTHR != 0 && task >= (P / V) * kQ) continue;
      const int col = (task % (P / V)) * V, r = task / (P / V);
      const bool ok = t0 + r < pr.L;
      const float sc = s_w[hh][r];
      const uint4 dq = keep_if(ok, dvr[q]);
      float o[V], lo[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        if constexpr (DS)
          o[v] = raw_elem<IO>(dq, v) * fmaf(gw, siluf_(raw_elem<IO>(zvr[q], v)), 1.f - gw) * sc;
        else
          o[v] = raw_elem<IO>(dq, v) * sc;
      }
      if constexpr (DS)
#pragma unroll
        for (int v = 0; v < V; ++v) lo[v] = o[v] - T::to_f(T::from_f(o[v]));
      lds_put_row<IO>(A + r * ldP + col, o);
      if constexpr (SPLIT) lds_put_row<IO>(Alo + r * ldP + col, lo);
    }
  };

  // A wave holds NJS 16 x 16 tiles of one 16-row strip of the P x N state.
  constexpr int PT = P / 16, NT = N / 16, WPP = NW / PT, NJS = (NT + WPP - 1) / WPP;
  static_assert(NW % PT == 0, "waves must cover the state rows");
  const int s_pi = wave % PT, s_nj0 = (wave / PT) * NJS;
  constexpr bool kAllOwn = NJS * WPP == NT;
  const bool owns = kAllOwn || s_nj0 < NT;
  static_assert(NJS % JB == 0, "a wave's state tiles cover whole scale blocks");
  // bf16 I/O, S walk: each wave's fp16 tiles go through a private LDS row buffer, so
  // that the global stores are 16-byte rows covering whole 128-byte lines (a store per
  // element writes 32-byte pieces, and the state stores are bound by their count).
  // The dS walk, whose LDS traffic per step is 2.4 times the S walk's, measured slower
  // with it and stores per element.
  // fp16 slot stores: 0 per element, 1 staged in LDS, 2 transposed across lanes
  constexpr int kStoreMode = !F16S ? 0 : (!DS ? 1 : (NJS % 4 == 0 ? 2 : 0));
  constexpr int ldO = 16 * NJS + 8;  // halves per staged row (16 bytes of padding)
  __shared__ __align__(16) uint16_t sOut[kStoreMode == 1 ? NW : 1][kStoreMode == 1 ? 16 * ldO : 8];
  const int64_t PN = static_cast<int64_t>(P) * N;
  f32x4 acc[HBM][NJS];
#pragma unroll
  for (int i = 0; i < HBM; ++i)
#pragma unroll
    for (int j = 0; j < NJS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float glsum = 0.f;  // S: group log-decay of head `wave` (its lane 0 writes it)

  // Group rows of a chunk (B for S; C and its low part for dS): unconditional loads of
  // clamped rows, masked when they go to LDS.
  constexpr int GV = N / V;                     // 16-byte vectors per row
  constexpr int GRB = rows_per_task(GV, NTHR);  // rows per task
  constexpr int GT = GV * (kQ / GRB);           // tasks
  constexpr int GQ = (GT + NTHR - 1) / NTHR;    // tasks per thread
  uint4 gr[GQ][GRB], grl[SPLIT ? GQ : 1][SPLIT ? GRB : 1];
  const bool bcpre = pr.bc.p != nullptr;
  const E* gsrc = static_cast<const E*>(bcpre ? pr.bc.p : pr.xbc.p) + b * (bcpre ? pr.bc.sb : pr.xbc.sb);
  const int64_t gst = bcpre ? pr.bc.st : pr.xbc.st;
  const int gcol = (bcpre ? 0 : pr.H * P) + (DS ? pr.G * N : 0) + g * N;
  const E* glsrc = klo ? static_cast<const E*>(pr.bc_lo.p) + b * pr.bc_lo.sb : gsrc;
  const int64_t glst = klo ? pr.bc_lo.st : gst;
  const int glcol = klo ? (DS ? pr.G * N : 0) + g * N : gcol;
  auto issue_rows = [&](int64_t c) {
    const int64_t t0 = c * kQ;
#pragma unroll
    for (int q = 0; q < GQ; ++q) {
      const int task = min(static_cast<int>(threadIdx.x) + q * NTHR, GT - 1);
      const int cv = (task % GV) * V, r0 = (task / GV) * GRB;
#pragma unroll
      for (int r = 0; r < GRB; ++r) {
        const int64_t t = t0 + r0 + r < pr.L ? t0 + r0 + r : pr.L - 1;
        gr[q][r] = *reinterpret_cast<const uint4*>(gsrc + t * gst + gcol + cv);
        if constexpr (SPLIT) grl[q][r] = *reinterpret_cast<const uint4*>(glsrc + t * glst + glcol + cv);
      }
    }
  };
  auto put_rows = [&](int64_t c) {
    const int64_t t0 = c * kQ;
#pragma unroll
    for (int q = 0; q < GQ; ++q) {
      const int task = threadIdx.x + q * NTHR;
      if (GT % NTHR != 0 && task >= GT) continue;
      const int cv = (task % GV) * V, r0 = (task / GV) * GRB;
#pragma unroll
      for (int r = 0; r < GRB; ++r) {
        const bool ok = t0 + r0 + r < pr.L;  // rows past the end are zero
        *reinterpret_cast<uint4*>(sK + (r0 + r) * ldN + cv) = keep_if(ok, gr[q][r]);
        if constexpr (SPLIT)
          *reinterpret_cast<uint4*>(sKlo + (r0 + r) * ldN + cv) = keep_if(ok && klo, grl[q][r]);
      }
    }
  };
  // dt of the block's heads (wave w: heads w, w + NW, ..), loaded one chunk ahead
  constexpr int DTK = (HB + NW - 1) / NW;
  E dtr[DTK];
  float hbias[DTK], hA[DTK];
#pragma unroll
  for (int k = 0; k < DTK; ++k) {
    const int h = hfirst + min(wave + k * NW, HB - 1);
    hbias[k] = pr.dt_bias ? pr.dt_bias[h] : 0.f;
    hA[k] = pr.A[h];
  }
  auto issue_dt = [&](int64_t c) {
    const int64_t t0 = c * kQ;
    const int64_t t = t0 + lane < pr.L ? t0 + lane : pr.L - 1;
#pragma unroll
    for (int k = 0; k < DTK; ++k) {
      const int h = hfirst + min(wave + k * NW, HB - 1);
      dtr[k] = static_cast<const E*>(pr.dt.p)[b * pr.dt.sb + t * pr.dt.st + h];
    }
  };
  // w_s (S) or exp(cs_t) (dS) and the chunk log-decay of each head; S also records
  // the chunk log-decays (and sums the group's, when count is set)
  auto put_dt = [&](int64_t c, bool count) {
    const int64_t t0 = c * kQ;
    const bool live = t0 + lane < pr.L;
#pragma unroll
    for (int k = 0; k < DTK; ++k) {
      const int hh = wave + k * NW;
      if (hh >= HB) continue;
      const float u = T::to_f(dtr[k]) + hbias[k];
      const float dtv = live ? (pr.softplus ? softplusf_(u) : u) : 0.f;
      const float cs = wave_incl_scan(dtv * hA[k]);
      const float csl = lane_value(cs, kWave - 1);
      if constexpr (DS) {
        s_w[hh][lane] = __expf(cs);
      } else {
        s_w[hh][lane] = dtv * __expf(csl - cs);
        if (lane == 0 && a.lsum) a.lsum[(b * a.nch + c) * pr.H + hfirst + hh] = csl;
        if (count) glsum += csl;  // wave hh's own lanes: lane 0 writes the sum
      }
      if (lane == 0) s_l[hh] = csl;
    }
  };

  // Per chunk: the HB head steps (unrolled); the last one (CX: the first) also issues
  // the next chunk's group rows and dt (CX: and x rows), and after its product they go
  // to LDS.  Every load is consumed in the iteration that issues it, so each wait counts
  // exactly the loads it needs and leaves the state stores in flight.  (The last chunk
  // reloads itself.)
  // CX: a chunk's raw x rows of every head of the block and each head's conv halo (the
  // 3 rows before the chunk: raw rows, or the carried conv state before the sequence,
  // zero before that), loaded a chunk ahead with the B rows; staged in LDS and convolved
  // for all heads at once, so a chunk needs one staging barrier and one conv barrier.
  uint4 cxr[CX ? HB : 1][CX ? NDT : 1], chv[CX ? HB : 1];
  bool chok[CX ? HB : 1];
  const E* csb = CX && pr.cs_in.p ? static_cast<const E*>(pr.cs_in.p) + b * pr.cs_in.sb : nullptr;
  auto issue_cx = [&](int64_t c) {
    const int64_t t0 = c * kQ;
#pragma unroll
    for (int hh = 0; hh < (CX ? HB : 0); ++hh) {
      const int h = hfirst + hh;
#pragma unroll
      for (int q = 0; q < NDT; ++q) {
        const int task = min(static_cast<int>(threadIdx.x) + q * NTHR, XVR * kQ - 1);
        const int r = task / XVR;
        const int64_t t = t0 + r < pr.L ? t0 + r : t0;
        cxr[hh][q] = *reinterpret_cast<const uint4*>(dbase + t * rows.st + h * P + (task % XVR) * V);
      }
      const int i = min(static_cast<int>(threadIdx.x), 3 * XVR - 1);
      const int64_t t = t0 - 3 + i / XVR;
      const int col = h * P + (i % XVR) * V;
      const bool from_state = t < 0 && csb && t >= -(pr.K - 1);
      // the address is chosen, not the loaded value (a select after the load would wait)
      const E* src = from_state ? csb + (t + pr.K - 1) * pr.cs_in.st + col
                                : dbase + (t >= 0 ? t : 0) * rows.st + col;
      chv[hh] = *reinterpret_cast<const uint4*>(src);
      chok[hh] = static_cast<int>(threadIdx.x) < 3 * XVR && (t >= 0 || from_state);
    }
  };
  // the loaded rows (zero past the end) and halos to LDS
  auto put_cx = [&](int64_t c) {
    const int64_t t0 = c * kQ;
#pragma unroll
    for (int hh = 0; hh < (CX ? HB : 0); ++hh) {
#pragma unroll
      for (int q = 0; q < NDT; ++q) {
        const int task = threadIdx.x + q * NTHR;
        if (XVR * kQ % NTHR != 0 && task >= XVR * kQ) continue;
        const int r = task / XVR;
        sRawG[hh][(3 + r) * XVR + task % XVR] = keep_if(t0 + r < pr.L, cxr[hh][q]);
      }
      if (static_cast<int>(threadIdx.x) < 3 * XVR) sRawG[hh][threadIdx.x] = keep_if(chok[hh], chv[hh]);
    }
  };
  // conv + SiLU of CR rows per task and head: w_s x to head hh's product tile sA[hh],
  // x to the post-conv rows
  auto conv_cx = [&](int64_t c) {
    const int64_t t0 = c * kQ;
    const int cg = static_cast<int>(threadIdx.x) % XVR, r0 = (static_cast<int>(threadIdx.x) / XVR) * CR;
    const int cl = cg * V;
#pragma unroll
    for (int hh = 0; hh < (CX ? HB : 0); ++hh) {
      uint4 raw[CR + 3];
#pragma unroll
      for (int i = 0; i < CR + 3; ++i) raw[i] = sRawG[hh][(r0 + i) * XVR + cg];
      float w4[4][V], bias[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
#pragma unroll
        for (int j = 0; j < 4; ++j) w4[j][v] = s_cvw[(hh * P + cl + v) * 5 + j];
        bias[v] = s_cvw[(hh * P + cl + v) * 5 + 4];
      }
      E* xo = static_cast<E*>(a.xp_out.p) + b * a.xp_out.sb + (hfirst + hh) * P + cl;
#pragma unroll
      for (int r = 0; r < CR; ++r) {
        const int row = r0 + r;
        const bool live = t0 + row < pr.L;
        const float sc = s_w[hh][row];
        float o[V], ow[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
          float pre = bias[v];
#pragma unroll
          for (int j = 0; j < 4; ++j) pre = fmaf(w4[j][v], raw_elem<IO>(raw[r + j], v), pre);
          o[v] = live ? siluf_(pre) : 0.f;
          ow[v] = o[v] * sc;
        }
        lds_put_row<IO>(sA[hh] + row * ldP + cl, ow);
        if (live) store_vec16<IO>(xo + (t0 + row) * a.xp_out.st, o);
      }
    }
  };

  if constexpr (CX)
    for (int i = threadIdx.x; i < HB * P * 5; i += NTHR) {
      const int hh = i / (P * 5), cl = (i / 5) % P, j = i % 5;
      const int c = (hfirst + hh) * P + cl;
      const int kk = j - (4 - pr.K);
      s_cvw[i] = j == 4 ? (pr.conv_b ? pr.conv_b[c] : 0.f) : (kk >= 0 ? pr.conv_w[c * pr.K + kk] : 0.f);
    }
  issue_rows(chunk_of(0));
  issue_dt(chunk_of(0));
  if constexpr (CX)
    issue_cx(chunk_of(0));
  else
    issue_step(0);
  put_rows(chunk_of(0));
  put_dt(chunk_of(0), true);
  if constexpr (CX) put_cx(chunk_of(0));
  __syncthreads();
  if constexpr (CX)
    conv_cx(chunk_of(0));
  else
    stage(0, 0);
  __syncthreads();
  for (int i = 0; i < ng; ++i) {
    const int64_t c = chunk_of(i * HB);
    const int64_t cn = chunk_of(min(i + 1, ng - 1) * HB);
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      const int k = i * HB + hh;
      const int h = hfirst + hh;
      if constexpr (CX) {
        // the next chunk's rows, a chunk ahead (the last chunk reloads its own)
        if (hh == 0) {
          issue_rows(cn);
          issue_dt(cn);
          issue_cx(cn);
        }
      } else {
        issue_step(k + 1 < nsteps ? k + 1 : k);
        if (hh == HB - 1) {
          issue_rows(cn);
          issue_dt(cn);
        }
      }
      if (owns) {
        const Lt* A = sA[CX ? hh : (k & 1)];
        const Lt* Alo = sAlo[SPLIT ? (k & 1) : 0];
        const float dec = __expf(s_l[hh]);
#pragma unroll
        for (int j = 0; j < NJS; ++j) acc[hh][j] *= dec;
        if constexpr (SPLIT) {
          mma_strip2<Lt, false, false, NJS>(acc[hh], A, Alo, ldP, s_pi * 16, sK, ldN, s_nj0 * 16, kQ);
          if (klo) mma_strip<Lt, false, false, NJS>(acc[hh], A, ldP, s_pi * 16, sKlo, ldN, s_nj0 * 16, kQ);
        } else {
          mma_strip<Lt, false, false, NJS>(acc[hh], A, ldP, s_pi * 16, sK, ldN, s_nj0 * 16, kQ);
        }
      }
      // S: P_c to slot c; dS: Q_{c-1} to slot c - 1.  The group's end state (S, last
      // chunk) and start gradient (dS, first chunk) go to the group buffer after the
      // walk; their slot copies land in slot c1, which no chunk reads (every step stores
      // the same way: no branch around the stores, whose waits would then take the
      // loads in flight with them).
      if (owns) {
        const int64_t c1 = c_lo + ng - 1;
        const int64_t slot = DS ? (c == c_lo ? c1 : c - 1) : c;
        const int64_t so = ((b * a.nch + slot) * pr.H + h) * PN;
        // a wave's stores cover whole rows of its columns: each cache line of the state
        // is written by one wave, within a few instructions
        if constexpr (!F16S) {
          float* dst = static_cast<float*>(a.out) + so;
#pragma unroll
          for (int j = 0; j < NJS; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              dst[(s_pi * 16 + acc_row(e)) * N + (s_nj0 + j) * 16 + acc_col()] = acc[hh][j][e];
        } else {
          // bf16 I/O: fp16 times 2^k per scale block, with k such that the block's
          // largest magnitude lands in [2^14, 2^15): every value keeps fp16's 11-bit
          // precision down to 2^-29 of that maximum, and none overflows.
          uint16_t* dst = static_cast<uint16_t*>(a.out) + so;
          float* sdst = a.oscale + ((b * a.nch + slot) * pr.H + h) * kSB;
          float upb[NJS / JB];
#pragma unroll
          for (int jb = 0; jb < NJS; jb += JB) {
            float m = 0.f;
#pragma unroll
            for (int j = jb; j < jb + JB; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(acc[hh][j][e]));
            const int ex = static_cast<int>((__float_as_uint(wave_max(m)) >> 23) & 0xffu);
            const int kx = min(141 - ex, 126);  // ex >= 15: 2^(ex-127) <= max < 2^(ex-126)
            upb[jb / JB] = __uint_as_float(static_cast<uint32_t>(kx + 127) << 23);
            // every lane stores the same value (a lane branch would be one around a store)
            sdst[s_pi * (N / SC) + (s_nj0 + jb) * 16 / SC] = __uint_as_float(static_cast<uint32_t>(127 - kx) << 23);
          }
          auto hval = [&](int j, int e) { return acc[hh][j][e] * upb[j / JB]; };
          if constexpr (kStoreMode == 2) {
            // Per group of 4 tiles and pair of accumulator rows e: the 4 tiles' packed
            // pairs, transposed between registers and 16-lane rows by two lane swaps,
            // leave register q holding rows 4q + e, e + 1 of tile g in lane row g: each
            // store then writes one row's 64 consecutive columns (128 bytes).
#pragma unroll
            for (int jg = 0; jg < NJS; jg += 4)
#pragma unroll
              for (int ep = 0; ep < 4; ep += 2) {
                uint32_t R[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) R[jj] = f2h2(hval(jg + jj, ep), hval(jg + jj, ep + 1));
                const auto x02 = __builtin_amdgcn_permlane32_swap(R[0], R[2], false, false);
                const auto x13 = __builtin_amdgcn_permlane32_swap(R[1], R[3], false, false);
                const auto y01 = __builtin_amdgcn_permlane16_swap(x02[0], x13[0], false, false);
                const auto y23 = __builtin_amdgcn_permlane16_swap(x02[1], x13[1], false, false);
                const uint32_t Q[4] = {y01[0], y01[1], y23[0], y23[1]};
                uint16_t* col = dst + s_pi * 16 * N + (s_nj0 + jg) * 16 + lane;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  col[(4 * q + ep) * N] = static_cast<uint16_t>(Q[q] & 0xffffu);
                  col[(4 * q + ep + 1) * N] = static_cast<uint16_t>(Q[q] >> 16);
                }
              }
          } else {
#pragma unroll
            for (int j = 0; j < NJS; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint16_t hv = __builtin_bit_cast(uint16_t, static_cast<_Float16>(hval(j, e)));
                if constexpr (kStoreMode == 1)
                  sOut[wave][acc_row(e) * ldO + j * 16 + acc_col()] = hv;
                else
                  dst[(s_pi * 16 + acc_row(e)) * N + (s_nj0 + j) * 16 + acc_col()] = hv;
              }
          }
          // staged: the wave's 16 rows x 16 NJS columns back as 16-byte row pieces (LDS
          // accesses of one wave complete in order: no barrier)
          constexpr int VPR = 16 * NJS / 8;  // 16-byte pieces per row
#pragma unroll
          for (int q = 0; q < (kStoreMode == 1 ? (16 * VPR + kWave - 1) / kWave : 0); ++q) {
            const int idx = lane + kWave * q, row = idx / VPR, cv = idx % VPR;
            if (16 * VPR % kWave == 0 || idx < 16 * VPR)
              *reinterpret_cast<uint4*>(dst + (s_pi * 16 + row) * N + s_nj0 * 16 + cv * 8) =
                  *reinterpret_cast<const uint4*>(&sOut[wave][row * ldO + cv * 8]);
          }
        }
      }
      if (hh == HB - 1) {
        __syncthreads();  // every product of chunk c is done with sK, s_w, s_l (and sA)
        put_rows(cn);
        put_dt(cn, i + 1 < ng);
        if constexpr (CX) put_cx(cn);
        __syncthreads();
      }
      if constexpr (CX) {
        if (hh == HB - 1) {
          conv_cx(cn);
          __syncthreads();
        }
      } else {
        stage(k + 1 < nsteps ? k + 1 : k, (k + 1) & 1);
        __syncthreads();
      }
    }
  }
  // E_g (S: the state after the group's last chunk) or F_g (dS: the gradient after its
  // first chunk), fp32
  if (owns) {
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      float* dst = a.grp + ((b * a.ngr + grp) * pr.H + hfirst + hh) * PN;
      if constexpr (NJS % 4 == 0) {
        // per group of 4 tiles and accumulator row e, transposed between registers and
        // 16-lane rows by two lane swaps: each store writes 64 columns of one row
#pragma unroll
        for (int jg = 0; jg < NJS; jg += 4)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const auto x02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[hh][jg][e]),
                                                              __float_as_uint(acc[hh][jg + 2][e]), false, false);
            const auto x13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[hh][jg + 1][e]),
                                                              __float_as_uint(acc[hh][jg + 3][e]), false, false);
            const auto y01 = __builtin_amdgcn_permlane16_swap(x02[0], x13[0], false, false);
            const auto y23 = __builtin_amdgcn_permlane16_swap(x02[1], x13[1], false, false);
            const uint32_t Q[4] = {y01[0], y01[1], y23[0], y23[1]};
#pragma unroll
            for (int q = 0; q < 4; ++q)
              dst[(s_pi * 16 + 4 * q + e) * N + (s_nj0 + jg) * 16 + lane] = __uint_as_float(Q[q]);
          }
      } else {
#pragma unroll
        for (int j = 0; j < NJS; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            dst[(s_pi * 16 + acc_row(e)) * N + (s_nj0 + j) * 16 + acc_col()] = acc[hh][j][e];
      }
    }
  }
  if constexpr (!DS)
    if (wave < HB && lane == 0 && a.glsum) a.glsum[(b * a.ngr + grp) * pr.H + hfirst + wave] = glsum;
}

int heads_per_group_block(const Problem& pr, int max_heads) {
  int hb = max_heads;
  while ((pr.H / pr.G) % hb) hb /= 2;
  return hb;
}

template <typename IO, int PP, int NN, bool DS, bool CX>
hipError_t launch_group_kernel(const GroupArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.hb == 2)
    hipLaunchKernelGGL((group_state_kernel<IO, PP, NN, DS, 2, CX>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((group_state_kernel<IO, PP, NN, DS, 1, CX>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <bool DS>
hipError_t launch_groups(const Problem& pr, int64_t nch, View dout, void* out, float* oscale,
                         float* grp, float* lsum, float* glsum, MView xp_out, hipStream_t s) {
  GroupArgs a{};
  a.pr = pr;
  a.nch = nch;
  a.ngr = (nch + kG - 1) / kG;
  a.hb = heads_per_group_block(pr, GroupShape<DS>::max_heads);
  a.dout = dout;
  a.out = out;
  a.oscale = oscale;
  a.grp = grp;
  a.lsum = lsum;
  a.glsum = glsum;
  a.xp_out = xp_out;
  static_assert(GroupShape<DS>::max_heads == 2, "head blocks of 2 or 1");
  const dim3 grid(static_cast<unsigned>(pr.B * a.ngr * (pr.H / a.hb)));
  const dim3 block(GroupShape<DS>::waves * 64);
  TimingScope ts(DS ? kKDstate : kKChunkStates, s);
  // the S walk convolves x itself where it is given the post-conv rows to write
  const bool cx = !DS && pr.bf16 && pr.K > 0 && xp_out.p != nullptr;
#define SSD_CASE(IO, PP, NN)                                                                     \
  if (pr.P == PP && pr.N == NN) {                                                                \
    if constexpr (!DS && sizeof(IO) == 2)                                                        \
      if (cx) return launch_group_kernel<IO, PP, NN, DS, true>(a, grid, block, s);               \
    return launch_group_kernel<IO, PP, NN, DS, false>(a, grid, block, s);                        \
  }
  if (pr.bf16) {
    SSD_CASE(bf16_t, 64, 128) SSD_CASE(bf16_t, 64, 64) SSD_CASE(bf16_t, 64, 32)
    SSD_CASE(bf16_t, 64, 16) SSD_CASE(bf16_t, 32, 128) SSD_CASE(bf16_t, 32, 64)
    SSD_CASE(bf16_t, 32, 32) SSD_CASE(bf16_t, 32, 16)
  } else {
    SSD_CASE(float, 64, 64) SSD_CASE(float, 64, 32) SSD_CASE(float, 64, 16)
    SSD_CASE(float, 32, 64) SSD_CASE(float, 32, 32) SSD_CASE(float, 32, 16)
  }
#undef SSD_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_group_local_states(const Problem& pr, int64_t nch, void* Pst, float* Psc,
                                     float* Eg, float* lsum, float* glsum, MView xp_out,
                                     hipStream_t s) {
  // post-conv x: written here from the raw rows (xp_out, bf16 I/O) or read from the
  // pre-pass's rows (pr.xp, fp32 I/O)
  if (pr.K > 0 && !pr.xp.p && !xp_out.p) return hipErrorInvalidValue;
  return launch_groups<false>(pr, nch, View{nullptr, 0, 0}, Pst, Psc, Eg, lsum, glsum, xp_out, s);
}

hipError_t launch_group_dstates(const Problem& pr, int64_t nch, View dout, void* Qst,
                                float* Qsc, float* Fg, hipStream_t s) {
  return launch_groups<true>(pr, nch, dout, Qst, Qsc, Fg, nullptr, nullptr, MView{nullptr, 0, 0}, s);
}

}  // namespace ssd
