// Internal host-side interface between the C ABI layer (api.hip) and the kernel
// translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

constexpr int kQ = 64;         // chunk length of the chunked evaluation
constexpr int kThreads = 256;  // threads per workgroup of the chunk kernels
// Largest row stride (elements) of an activation view: 64 rows of a chunk plus a
// row's channels then stay within a 32-bit element offset from the chunk's first row.
constexpr int64_t kMaxRowStride = int64_t(1) << 24;

// Kernel kinds of the timing instrumentation (ssd_timing_* in ssd.h).
enum KernelKind {
  kKBcPrepass, kKWalkState, kKScan, kKWalkOut, kKConvStateOut, kKConvFwd, kKChunkStates,
  kKDstate, kKScanRev, kKBwdMain, kKConvBwd, kKDbcReduce, kKParams, kKScanGroups, kKXbcPrepass,
  kKLinear, kKDecode, kKNorm, kKernelKinds
};

// Brackets the launches made during its lifetime with HIP events on stream `s`
// when timing is enabled (no-op otherwise).
class TimingScope {
 public:
  TimingScope(int kind, hipStream_t s);
  ~TimingScope();
  TimingScope(const TimingScope&) = delete;
  TimingScope& operator=(const TimingScope&) = delete;

 private:
  int kind_;
  hipStream_t s_;
  void* a_ = nullptr;
  void* b_ = nullptr;
};

struct View {
  const void* p;
  int64_t sb, st;  // element strides (batch, time)
};
struct MView {
  void* p;
  int64_t sb, st;
};

// Sub-segment plan of the forward pass: each workgroup walks `cps` chunks of one
// head; the states at sub-segment starts come from a scan over sub-segments.
struct Plan {
  int64_t nchunks;  // ceil(L / kQ)
  int64_t cps;      // chunks per sub-segment
  int64_t n_sub;    // sub-segments
};

struct Problem {
  int bf16;  // 1 = bf16 I/O, 0 = fp32 I/O
  int64_t B, L;
  int H, P, N, G, K;
  View xbc;
  const float* conv_w;
  const float* conv_b;
  View cs_in;  // conv state in (p may be null)
  View dt;
  const float* dt_bias;
  int softplus;
  const float* A;
  const float* D;
  View z;  // p may be null
  const float* h0;
  View bc;     // post-conv B|C rows [B][L][2*G*N] from the conv pre-pass (p null: read xbc)
  View bc_lo;  // bf16 I/O backward: post-conv B|C minus its bf16 rounding (p null: none)
  View xp;     // post-conv x rows [B][L][H*P] from a pre-pass or the backward's state
               // walk (p null: conv in the loaders)
  const float* dtsp;  // forward: dt = softplus(dt_raw + dt_bias) (or the sum alone without
                      // softplus) as fp32 [B][L][H], from the dt pre-pass
};

struct FwdOut {
  MView out;
  float* h_final;
  float* h_ckpt;
  int64_t ckpt_every;
  MView cs_out;  // p may be null
};

Plan make_plan(int64_t B, int64_t L, int H);
size_t fwd_workspace_bytes(const Problem& pr, const Plan& pl);
hipError_t launch_fwd(const Problem& pr, const FwdOut& o, const Plan& pl, void* ws,
                      hipStream_t s);

// conv-state copy: dst rows j < K-1 = conv inputs at t = L-(K-1)+j
hipError_t launch_conv_state_out(const Problem& pr, MView dst, hipStream_t s);

// Chunk groups of kG chunks: in-group prefix states P_c (slot c < the group's last
// chunk) and group end states E_g, with chunk and group log-decays; in-group suffix
// gradients Q_c and group start gradients F_g (dout / z and C rows as for the chunk
// form).  See chunk_states.hip for the recurrences.  The slot states are
// [B][nch][H][P][N]: fp32 for fp32 I/O; for bf16 I/O fp16, each block of 16 rows (p) x
// state_scale_cols columns (n) scaled by a power of two, with Psc / Qsc
// [B][nch][H][state_scale_blocks] holding the factors that restore them (block
// p / 16 * (N / state_scale_cols) + n / state_scale_cols).  E_g and F_g are fp32.
constexpr int kG = 8;
// the columns of one of 8 waves spread over the 16-row strips of a P x N state
constexpr int state_scale_cols(int P, int N) {
  return 16 * ((N / 16 + 8 / (P / 16) - 1) / (8 / (P / 16)));
}
constexpr int state_scale_blocks(int P, int N) { return (P / 16) * (N / state_scale_cols(P, N)); }
// xp_out (bf16 I/O with a conv): the S walk convolves the raw x rows itself and writes
// the post-conv rows there; otherwise (p null) it reads them from pr.xp.
hipError_t launch_group_local_states(const Problem& pr, int64_t nch, void* Pst, float* Psc,
                                     float* Eg, float* lsum, float* glsum, MView xp_out,
                                     hipStream_t s);
hipError_t launch_group_dstates(const Problem& pr, int64_t nch, View dout, void* Qst,
                                float* Qsc, float* Fg, hipStream_t s);
// group_local_states, then the scan over groups: Eg[b][g][h] <- H_in(g)
hipError_t launch_group_chunk_states(const Problem& pr, int64_t nch, void* Pst, float* Psc,
                                     float* Eg, float* lsum, float* glsum, MView xp_out,
                                     hipStream_t s);

// ---------------------------------------------------------------- backward
struct BwdIn {
  View dout;                // [B,L,H*P]
  const float* dh_final;    // [B,H,P,N] or null
  View dcs_out;             // [B,K-1,Cd] gradient of the returned conv state (p may be null)
};
struct BwdOut {
  MView dxbc;               // [B,L,Cd]
  MView ddt;                // [B,L,H]
  MView dz;                 // [B,L,H*P] (p null without gate)
  float *dA, *dD, *ddt_bias, *dconv_w, *dconv_b, *dh0;
  MView dcs_in;             // [B,K-1,Cd] (p may be null)
  int accumulate;
};
size_t bwd_workspace_bytes(const Problem& pr);
bool bwd_supported(const Problem& pr);
hipError_t launch_bwd(const Problem& pr, const BwdIn& in, const BwdOut& o, void* ws,
                      hipStream_t s);

// ---------------------------------------------------------------- standalone conv
struct ConvProblem {
  int bf16;
  int64_t B, L, C;
  int K, silu;
  View x;
  const float* w;
  const float* b;
  View state_in;
};
hipError_t launch_conv_fwd(const ConvProblem& cp, MView out, MView state_out, hipStream_t s);
hipError_t launch_conv_fwd_range(int bf16, int64_t B, int64_t L, int C, int K, int silu, View x,
                                 int x_c0, View st, int st_c0, const float* w, const float* bias,
                                 MView out, int o_c0, hipStream_t s, void* out_lo);
// B|C post-conv pre-pass of the SSD entry points: channels [H*P, Cd) of xbc -> dst,
// and (dst_lo != null, bf16 I/O) the rounding residual v - bf16(v) -> dst_lo; `kind`
// names it for the timing instrumentation (the forward's or the backward's pre-pass)
hipError_t launch_bc_prepass(const Problem& pr, void* dst, void* dst_lo, hipStream_t s,
                             int kind = kKBcPrepass);
size_t bc_prepass_bytes(const Problem& pr);
// Workgroups of `threads` threads of `kernel` resident on the current device at once
// (all CUs; cached per device and kernel); 0 if the runtime cannot tell.
int64_t resident_blocks(const void* kernel, int threads);
// Both pre-passes of the backward in one launch (fp32 I/O; with bf16 I/O the state
// group walk convolves x): post-conv x channels -> xp ([B][L][H*P]), post-conv B|C ->
// bc ([B][L][2GN]) and (bf16 I/O) its rounding residual -> bc_lo.
hipError_t launch_xbc_prepass(const Problem& pr, void* xp, void* bc, void* bc_lo, hipStream_t s);
size_t x_prepass_bytes(const Problem& pr);
size_t conv_bwd_workspace_bytes(int64_t B, int64_t L, int64_t C);
hipError_t launch_conv_bwd(const ConvProblem& cp, View dout, View dstate_out, MView dx, float* dw,
                           float* db, MView dstate_in, int accumulate, void* ws, hipStream_t s);

// ---------------------------------------------------------------- mixer projections
// y[M][N] = x[M][K] w[N][K]^T (bf16, fp32 accumulation), optionally with x's rows
// RMS-normalised over K and scaled by norm_w[K] first, and a residual r[M][N] added.
struct LinearProblem {
  int64_t M, N, K;
  const void* x;
  int64_t ldx;
  const void* w;
  int64_t ldw;
  const float* norm_w;
  float eps;
  const void* residual;
  int64_t ldr;
  void* y;
  int64_t ldy;
};
hipError_t launch_linear(const LinearProblem& lp, hipStream_t s);
// backward of y = x w^T: dx = dy w (bf16) and dw (+)= dy^T x (fp32)
hipError_t launch_linear_dgrad(int64_t M, int64_t N, int64_t K, const void* dy, int64_t lddy,
                               const void* w, int64_t ldw, void* dx, int64_t lddx, hipStream_t s);
hipError_t launch_linear_wgrad(int64_t M, int64_t N, int64_t K, const void* dy, int64_t lddy,
                               const void* x, int64_t ldx, float* dw, int64_t lddw, int accumulate,
                               hipStream_t s);

// ---------------------------------------------------------------- RMSNorm of the block
size_t rmsnorm_bwd_workspace_bytes(int64_t K);
int rmsnorm_max_k();
hipError_t launch_rmsnorm_fwd(int64_t M, int K, const void* x, int64_t ldx, const float* g, float eps,
                              void* y, int64_t ldy, float* rstd, hipStream_t s);
hipError_t launch_rmsnorm_bwd(int64_t M, int K, const void* x, int64_t ldx, const float* g, float eps,
                              const void* dy, int64_t lddy, const void* dres, int64_t ldres, void* dx,
                              int64_t lddx, float* dg, int accumulate, void* ws, hipStream_t s);

// ---------------------------------------------------------------- streaming decode
// pr.L tokens stepped one at a time from (pr.h0, pr.cs_in); state out to h_out (may
// equal pr.h0), conv state out to cs_out (distinct from pr.cs_in), outputs to out.
hipError_t launch_decode(const Problem& pr, float* h_out, MView out, MView cs_out, hipStream_t s);

}  // namespace ssd
