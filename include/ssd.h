/*
 * ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 mixer hot path:
 *
 *     causal depthwise conv1d + SiLU  ->  selective SSD recurrence  ->  SiLU(z) gate
 *
 * and its backward pass.
 *
 * What is computed (sources: the pith.science review of Video-Ma2mba, arXiv
 * 2411.19460 -- skeptic critique and referee report, Eq. (1) and the Conv1d-buffer
 * critique; the Mamba / Mamba-2 papers in the arXiv index page's reference list for
 * the selective form of Eq. (1)):
 *
 *   conv:  pre[t,c] = b[c] + sum_{k<K} w[c,k] * xin[t-K+1+k, c]      (xin[t<0] = carried state)
 *          xbc[t,c] = silu(pre[t,c]);   conv state out = the last K-1 rows of xin
 *   split: x[t,h,p] = xbc[t, h*P+p],  B[t,g,n] = xbc[t, H*P+g*N+n],
 *          C[t,g,n] = xbc[t, H*P+G*N+g*N+n],   head h uses group g = h / (H/G)
 *   dt:    dt[t,h] = softplus(dt_raw[t,h] + dt_bias[h])   (or dt_raw + dt_bias)
 *   Eq.(1) selective form, per head h:
 *          h_t = exp(dt_t * A_h) * h_{t-1} + dt_t * x_t B_t^T        (state P x N)
 *          y_t = h_t C_t + D_h x_t
 *   gate:  out_t = y_t * silu(z_t)
 *
 * The state needed to resume a sequence at step s is (h_s, the last K-1 conv
 * inputs) -- the review's point that checkpointing h alone is not exact when a
 * causal conv precedes the SSD.  Every entry point takes both in and returns both,
 * so a long sequence can be run and trained segment by segment (multi-axis
 * gradient checkpointing along the sequence axis).
 *
 * Conventions
 *   Pointers   All tensor pointers are caller-owned *device* pointers (hipMalloc /
 *              torch device memory).  The library allocates nothing, keeps no
 *              pointer after return, and never synchronises.  Scratch memory comes
 *              from the caller through (ws, ws_bytes), sized by the *_workspace
 *              queries; its contents need not be initialised.
 *   Streams    `stream` is a hipStream_t (NULL = the legacy default stream).  All
 *              work is enqueued asynchronously on it; results are valid once the
 *              stream has been synchronised.  Calls that overlap on one device and
 *              share a workspace race.
 *   Views      ssd_view = {ptr, stride_b, stride_t}: a [batch, time, channels]
 *              tensor whose channel dim is contiguous; strides are in *elements*.
 *              A view with ptr == NULL means "absent" where the argument is optional.
 *              Activations use the I/O dtype `io`; base pointers must be 16-byte
 *              aligned and stride_b, stride_t multiples of 16 bytes, except the dt /
 *              ddt views, which need only element alignment.  stride_t is at most
 *              2^24 elements (SSD_ERR_SHAPE otherwise).
 *   Dtypes     Activations, conv states and activation gradients: `io` (bf16 or
 *              fp32).  Parameters (A, D, dt_bias, conv w and b), SSD states (h0,
 *              h_final, checkpoints, dh) and parameter gradients: fp32.  All
 *              arithmetic accumulates in fp32; bf16 results are rounded to nearest
 *              even.
 *   Layouts    h0 / h_final / dh: [B][H][P][N] (n contiguous) fp32, base pointer
 *                                 16-byte aligned (SSD_ERR_ALIGN otherwise).
 *              conv state:        [B][K-1][Cd] rows, oldest first -- the same layout
 *                                 as xbc rows, so the previous segment's last K-1
 *                                 input rows can be passed as a view.
 *              conv weight:       [Cd][K]; w[c][K-1] multiplies the current token.
 *                                 Weight and bias base pointers 16-byte aligned
 *                                 (SSD_ERR_ALIGN otherwise).
 *   Errors     Every call returns ssd_status.  All validation happens before any
 *              launch; nothing is enqueued on error.  Launch failures return
 *              SSD_ERR_HIP with detail in ssd_last_error() (thread-local).
 *              Unsupported shapes return SSD_ERR_UNSUPPORTED; there is no fallback.
 *   Preconditions (documented, not checked on the device): A <= 0 and dt >= 0
 *              (always true with dt_softplus = 1).
 *   Supported  headdim P in {32, 64}; dstate N in {16, 32, 64, 128}; conv width
 *              K in {0 (no conv), 2, 3, 4}; chunk in {0, 64} (0 selects 64; the result
 *              does not depend on the chunk length up to rounding, and other lengths
 *              return SSD_ERR_UNSUPPORTED rather than being remapped); any seqlen >= 1,
 *              any batch >= 1, nheads % ngroups == 0.
 *   Entry points beyond the hot path: ssd_fwd_noalloc (no workspace), ssd_decode
 *              (streaming one-token steps), mixer_proj / mixer_proj_bwd (the block's
 *              projections), rmsnorm_fwd / rmsnorm_bwd (the block's norms).
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSD_OK = 0,
  SSD_ERR_NULL = -1,        /* a required pointer is NULL */
  SSD_ERR_SHAPE = -2,       /* a dimension is out of range or inconsistent */
  SSD_ERR_DTYPE = -3,       /* unknown dtype */
  SSD_ERR_ALIGN = -4,       /* a pointer or stride breaks the alignment rule */
  SSD_ERR_UNSUPPORTED = -5, /* valid but not implemented (P, N, K or chunk) */
  SSD_ERR_WORKSPACE = -6,   /* ws too small (or NULL with ws_bytes > 0 needed) */
  SSD_ERR_HIP = -7          /* a HIP call or kernel launch failed */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef struct {
  int64_t batch;      /* B */
  int64_t seqlen;     /* L, tokens in this call (a segment of a longer stream) */
  int64_t nheads;     /* H */
  int64_t headdim;    /* P */
  int64_t dstate;     /* N */
  int64_t ngroups;    /* G (B and C shared by the H/G heads of a group) */
  int64_t chunk;      /* Q, intra-chunk length of the chunked evaluation (0 = 64) */
  int64_t conv_width; /* K; 0 = no conv: xbc already holds x|B|C */
} ssd_dims;

typedef struct {
  void* ptr;
  int64_t stride_b; /* elements between batches */
  int64_t stride_t; /* elements between time steps */
} ssd_view;

/* ABI version of this header (bumped on any signature change). */
#define SSD_ABI_VERSION 1
int ssd_abi_version(void);

/* Static text of a status code. */
const char* ssd_status_string(int status);

/* Detail of the last error on this thread (empty string if none). */
const char* ssd_last_error(void);

/* Scratch bytes ssd_fwd / ssd_bwd need for these dims (0 is possible). */
ssd_status ssd_fwd_workspace(const ssd_dims* d, ssd_dtype io, size_t* bytes);
ssd_status ssd_bwd_workspace(const ssd_dims* d, ssd_dtype io, size_t* bytes);

/*
 * ssd_fwd -- conv1d+SiLU (when d->conv_width > 0), SSD recurrence, SiLU(z) gate.
 *
 *   xbc             [B,L,Cd], Cd = H*P + 2*G*N, channel order x | B | C.  Raw
 *                   (pre-conv) rows when conv_width > 0, else the SSD inputs.
 *   conv_w, conv_b  [Cd,K] and [Cd] (conv_b may be NULL); ignored without conv.
 *   conv_state_in   [B,K-1,Cd] carried conv inputs (ptr NULL = zeros).
 *   conv_state_out  [B,K-1,Cd] receives the last K-1 conv inputs (ptr NULL = skip).
 *                   May not alias xbc.
 *   dt              [B,L,H] raw dt;  dt_bias [H] or NULL;  dt_softplus 0/1.
 *   A               [H] (<= 0);  D [H] or NULL.
 *   z               [B,L,H*P] gate input (ptr NULL = no gate: out = y).
 *   h0              [B,H,P,N] initial state, NULL = zeros.
 *   out             [B,L,H*P] output; must not overlap any input.
 *   h_final         [B,H,P,N] state after the last token, NULL = skip.
 *   h_ckpt          optional sequence checkpoints: [ceil(L/ckpt_every),B,H,P,N];
 *                   entry j is the state before token j*ckpt_every (entry 0 = h0).
 *                   ckpt_every must be a positive multiple of 64 when h_ckpt != NULL.
 */
ssd_status ssd_fwd(const ssd_dims* d, ssd_dtype io, ssd_view xbc, const float* conv_w,
                   const float* conv_b, ssd_view conv_state_in, ssd_view conv_state_out,
                   ssd_view dt, const float* dt_bias, int dt_softplus, const float* A,
                   const float* D, ssd_view z, const float* h0, ssd_view out, float* h_final,
                   float* h_ckpt, int64_t ckpt_every, void* ws, size_t ws_bytes, void* stream);

/*
 * ssd_fwd_noalloc -- ssd_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments and results as ssd_fwd, without (ws, ws_bytes): its scratch is a
 * fixed array of SSD_FWD_NOALLOC_SCRATCH_BYTES in the library's device image, which
 * each GPU the library runs on holds until the process ends.  The call itself
 * allocates nothing.
 *
 *   Limit    dims whose ssd_fwd_workspace() exceeds SSD_FWD_NOALLOC_SCRATCH_BYTES
 *            return SSD_ERR_WORKSPACE before anything is enqueued (at d_model 1024
 *            shapes -- 32 heads x 64, d_state 128, batch 1 -- up to about 149K tokens
 *            per call; longer sequences run as several calls with carried state, or
 *            through ssd_fwd).
 *   Device   the scratch of the *current* device is used; `stream` must belong to it.
 *            The first call on a device looks up the array's address on that device.
 *   Races    every call on one GPU shares that GPU's array: calls that overlap on one
 *            device (other streams, other host threads) race.  Calls on one stream
 *            are ordered and safe.  The scratch needs no initialisation.
 */
#define SSD_FWD_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
ssd_status ssd_fwd_noalloc(const ssd_dims* d, ssd_dtype io, ssd_view xbc, const float* conv_w,
                           const float* conv_b, ssd_view conv_state_in, ssd_view conv_state_out,
                           ssd_view dt, const float* dt_bias, int dt_softplus, const float* A,
                           const float* D, ssd_view z, const float* h0, ssd_view out,
                           float* h_final, float* h_ckpt, int64_t ckpt_every, void* stream);

/*
 * ssd_bwd -- gradients of ssd_fwd (same inputs) given dout = dLoss/dout, the
 * gradient dh_final of the returned state and dconv_state_out of the returned conv
 * state (both optional: NULL / ptr NULL = zero).  Recomputes the forward from
 * (h0, conv_state_in): with these set to a segment checkpoint this is the
 * per-segment backward of sequence-axis gradient checkpointing.
 *
 *   dxbc            [B,L,Cd] gradient w.r.t. xbc (raw rows when conv_width > 0).
 *   ddt             [B,L,H] gradient w.r.t. dt_raw.
 *   dz              [B,L,H*P] (required iff z is given).
 *   dA, dD, ddt_bias [H]; dconv_w [Cd,K]; dconv_b [Cd]: parameter gradients, fp32,
 *                   overwritten (accumulate = 0) or added to (accumulate = 1).
 *                   dD, ddt_bias, dconv_w, dconv_b may be NULL (not computed).
 *   dh0             [B,H,P,N] gradient w.r.t. h0 (NULL = skip).
 *   dconv_state_in  [B,K-1,Cd] gradient w.r.t. conv_state_in (ptr NULL = skip).
 */
ssd_status ssd_bwd(const ssd_dims* d, ssd_dtype io, ssd_view xbc, const float* conv_w,
                   const float* conv_b, ssd_view conv_state_in, ssd_view dt, const float* dt_bias,
                   int dt_softplus, const float* A, const float* D, ssd_view z, const float* h0,
                   ssd_view dout, const float* dh_final, ssd_view dconv_state_out, ssd_view dxbc,
                   ssd_view ddt, ssd_view dz, float* dA, float* dD, float* ddt_bias,
                   float* dconv_w, float* dconv_b, float* dh0, ssd_view dconv_state_in,
                   int accumulate, void* ws, size_t ws_bytes, void* stream);

/*
 * conv1d_fwd -- causal depthwise conv of width K in [2,4] over [B,L,C] rows, plus
 * bias and optional SiLU (the first stage of the hot path, as a standalone call):
 *     pre[t,c] = b[c] + sum_{k<K} w[c,k] xin[t-K+1+k, c],  out = silu(pre) or pre,
 * xin[t < 0] = the carried state rows.  Source: the pith.science review of
 * Video-Ma2mba, skeptic critique ("load-bearing attack": the causal Conv1d of the
 * Mamba-2 block before the SSD, whose last K-1 inputs a sequence checkpoint must keep).
 *   x [B,L,C] -> out [B,L,C];  state_in / state_out [B,K-1,C] as in ssd_fwd.
 */
ssd_status conv1d_fwd(int64_t batch, int64_t seqlen, int64_t channels, int32_t width,
                      ssd_dtype io, ssd_view x, const float* w, const float* b, int silu,
                      ssd_view state_in, ssd_view out, ssd_view state_out, void* stream);

/* Scratch bytes conv1d_bwd needs (per-tile partial sums of dw and db). */
ssd_status conv1d_bwd_workspace(int64_t batch, int64_t seqlen, int64_t channels, int32_t width,
                                size_t* bytes);

/*
 * conv1d_bwd -- gradients of conv1d_fwd given dout [B,L,C] and the gradient
 * dstate_out of the returned state (ptr NULL = zero) -- the conv-buffer gradient that
 * crosses a segment boundary backwards (same review, skeptic critique, "concrete test":
 * segmented gradients equal full-storage backprop only with the conv buffer carried).
 *   dx [B,L,C]; dw [C,K] and db [C] (fp32, db may be NULL; overwritten or added to
 *   per `accumulate`); dstate_in [B,K-1,C] (ptr NULL = skip).
 */
ssd_status conv1d_bwd(int64_t batch, int64_t seqlen, int64_t channels, int32_t width,
                      ssd_dtype io, ssd_view x, const float* w, const float* b, int silu,
                      ssd_view state_in, ssd_view dout, ssd_view dstate_out, ssd_view dx,
                      float* dw, float* db, ssd_view dstate_in, int accumulate, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * ssd_decode -- streaming decode: d->seqlen new tokens (usually 1) stepped one at a
 * time from the carried state, for inference over streams longer than any single
 * forward call (the two-million-token inference mode of the pith.science review of
 * Video-Ma2mba, referee report summary).  The same function as ssd_fwd over these
 * tokens with (h0, conv_state_in) = (h_in, conv_state_in): conv1d + SiLU of the new
 * raw rows against the carried conv inputs, the recurrence of Eq. (1) in its selective
 * form one step per token, y + D x, SiLU(z) gate.
 *
 *   xbc, dt, z, out   [B,T,.] views as in ssd_fwd (element alignment suffices)
 *   conv_state_in     [B,K-1,Cd] carried raw rows (ptr NULL = zeros)
 *   conv_state_out    [B,K-1,Cd] required when conv_width > 1; must not alias
 *                     conv_state_in (callers ping-pong two buffers)
 *   h_in              [B,H,P,N] fp32 state in (NULL = zeros)
 *   h_out             [B,H,P,N] fp32 state out (required; may equal h_in)
 * The state is read once and written once per call; cost per call is latency-bound
 * (one workgroup per (batch, head)).  No workspace.
 */
ssd_status ssd_decode(const ssd_dims* d, ssd_dtype io, ssd_view xbc, const float* conv_w,
                      const float* conv_b, ssd_view conv_state_in, ssd_view conv_state_out,
                      ssd_view dt, const float* dt_bias, int dt_softplus, const float* A,
                      const float* D, ssd_view z, const float* h_in, float* h_out, ssd_view out,
                      void* stream);

/*
 * mixer_proj -- the mixer's linear layers (in_proj, out_proj) on MFMA:
 *
 *     y[m][n] = sum_k x'[m][k] * w[n][k]  (+ residual[m][n])
 *
 * with x' = x, or, when norm_w != NULL, each row RMS-normalised over its K entries
 * and scaled: x'[m][k] = x[m][k] * rsqrt(mean_k' x[m][k']^2 + norm_eps) * norm_w[k]
 * (the pre-norm before in_proj and the gated norm before out_proj of the Mamba-2
 * block; the gate itself is already applied by ssd_fwd's output).
 *   x         [M][ldx] bf16, row m = one token's input vector (K contiguous)
 *   w         [N][ldw] bf16, the nn.Linear weight layout [out][in]
 *   norm_w    [K] fp32 or NULL;  norm_eps >= 0
 *   residual  [M][ldr] bf16 or NULL, added in fp32 before the bf16 rounding of y
 *   y         [M][ldy] bf16 (may not overlap x or w; may equal residual)
 * fp32 accumulation; y rounded to nearest even.  Supported: io = SSD_BF16, K a
 * multiple of 64, N a multiple of 8; 16-byte aligned base pointers and leading
 * dimensions that are multiples of 8 elements.  Sources: the Video-Ma2mba model
 * card's architecture diagram and specification table (Mamba-2 LM, d_model 1024,
 * bf16) and the Mamba-2 block of the arXiv index page's "Builds on" list.
 */
ssd_status mixer_proj(int64_t M, int64_t N, int64_t K, ssd_dtype io, const void* x, int64_t ldx,
                      const void* w, int64_t ldw, const float* norm_w, float norm_eps,
                      const void* residual, int64_t ldr, void* y, int64_t ldy, void* stream);

/*
 * mixer_proj_bwd -- backward of y = x w^T (mixer_proj without its options):
 *     dx[m][k]  = sum_n dy[m][n] w[n][k]            (bf16; skipped when dx == NULL)
 *     dw[n][k] (+)= sum_m dy[m][n] x[m][k]          (fp32; added to when accumulate = 1;
 *                                                   skipped when dw == NULL)
 * dy [M][lddy], x [M][ldx], w [N][ldw], dx [M][lddx] bf16; dw [N][lddw] fp32.  The
 * norm and residual of a fused forward are differentiated by rmsnorm_bwd and by adding
 * dy itself, by the caller.  Supported: io = SSD_BF16, N and K multiples of 8, any M;
 * bf16 base pointers 16-byte aligned with leading dimensions that are multiples of 8.
 * MFMA products with both operands staged in LDS (transposed ones read with the gfx950
 * LDS transpose loads); deterministic.
 */
ssd_status mixer_proj_bwd(int64_t M, int64_t N, int64_t K, ssd_dtype io, const void* dy, int64_t lddy,
                          const void* x, int64_t ldx, const void* w, int64_t ldw, void* dx, int64_t lddx,
                          float* dw, int64_t lddw, int accumulate, void* stream);

/*
 * rmsnorm_fwd / rmsnorm_bwd -- the block's RMSNorm over rows of K bf16 entries (the
 * norm before in_proj, and the gated norm before out_proj applied to ssd_fwd's gated
 * output; Mamba-2 block of the arXiv index page's "Builds on" list):
 *     r[m] = (mean_k x[m][k]^2 + eps)^(-1/2),   y[m][k] = x[m][k] r[m] g[k]
 *     dx[m][k] = r g[k] dy[m][k] - x[m][k] r^3 / K sum_j g[j] dy[m][j] x[m][j]  (+ dres[m][k])
 *     dg[k] (+)= sum_m dy[m][k] x[m][k] r[m]       (ordered sum: deterministic)
 * x, y, dy, dres, dx bf16 [M][ld] (dx may equal dy or dres); g, dg fp32 [K], 16-byte
 * aligned; rstd fp32 [M] or NULL.  K a multiple of 8, at most 5120.  rmsnorm_bwd needs
 * rmsnorm_bwd_workspace(K) bytes of scratch (partial sums of dg).
 */
ssd_status rmsnorm_fwd(int64_t M, int64_t K, ssd_dtype io, const void* x, int64_t ldx, const float* g,
                       float eps, void* y, int64_t ldy, float* rstd, void* stream);
ssd_status rmsnorm_bwd_workspace(int64_t K, size_t* bytes);
ssd_status rmsnorm_bwd(int64_t M, int64_t K, ssd_dtype io, const void* x, int64_t ldx, const float* g,
                       float eps, const void* dy, int64_t lddy, const void* dres, int64_t ldres, void* dx,
                       int64_t lddx, float* dg, int accumulate, void* ws, size_t ws_bytes, void* stream);

/*
 * Timing instrumentation (off by default).  While enabled, every kernel the
 * library enqueues is bracketed by HIP events on the caller's stream.
 *   ssd_timing_enable(1) clears the totals and starts recording; (0) stops.
 *   ssd_timing_read(kind, ...) waits for the recorded events and returns the
 *     summed device time (ms) and launch count of kernel kind `kind`
 *     (0 .. ssd_timing_kinds()-1; ssd_timing_name gives its name).
 * Host-side state is process-wide; enable it only around work you measure.
 */
ssd_status ssd_timing_enable(int on);
ssd_status ssd_timing_read(int kind, double* total_ms, int64_t* launches);
const char* ssd_timing_name(int kind);
int ssd_timing_kinds(void);

#ifdef __cplusplus
}
#endif
#endif /* SSD_H */
