// C ABI of the mixer hot path (declarations and contract in include/ssd.h).
//
// This layer only validates arguments, sizes scratch memory and enqueues kernels on
// the caller's stream; it allocates nothing and never synchronises.  Every check
// runs before the first launch, so an error leaves the stream untouched.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/ssd.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

ssd_status fail(ssd_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ssd_status fail(ssd_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ssd_status hip_fail(hipError_t e, const char* where) {
  return fail(SSD_ERR_HIP, "%s: %s (%s)", where, hipGetErrorName(e), hipGetErrorString(e));
}

int esize(ssd_dtype io) { return io == SSD_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// fp32 state arrays are read and written as 16-byte vectors
ssd_status check_state(const void* p, const char* name) {
  if (p && !aligned16(p)) return fail(SSD_ERR_ALIGN, "%s: state pointer not 16-byte aligned", name);
  return SSD_OK;
}

// conv weights and bias are read as 16-byte vectors
ssd_status check_param16(const void* p, const char* name) {
  if (p && !aligned16(p)) return fail(SSD_ERR_ALIGN, "%s: pointer not 16-byte aligned", name);
  return SSD_OK;
}

// A [B, T, C] activation view.  vec: 16-byte rule (vector loads); else element rule.
ssd_status check_view(const ssd_view& v, const char* name, ssd_dtype io, bool required, bool vec,
                      int64_t T, int64_t C) {
  if (!v.ptr) {
    if (required) return fail(SSD_ERR_NULL, "%s: NULL pointer", name);
    return SSD_OK;
  }
  const int es = esize(io);
  if (v.stride_t < C && T > 1) return fail(SSD_ERR_SHAPE, "%s: stride_t %lld < channels %lld", name,
                                           (long long)v.stride_t, (long long)C);
  if (v.stride_b < 0 || v.stride_t < 0) return fail(SSD_ERR_SHAPE, "%s: negative stride", name);
  // kernels address a chunk's rows as a uniform base plus a 32-bit in-chunk offset
  if (v.stride_t > ssd::kMaxRowStride)
    return fail(SSD_ERR_SHAPE, "%s: stride_t %lld elements exceeds %lld", name, (long long)v.stride_t,
                (long long)ssd::kMaxRowStride);
  if (vec) {
    if (!aligned16(v.ptr)) return fail(SSD_ERR_ALIGN, "%s: base pointer not 16-byte aligned", name);
    if ((v.stride_b * es) % 16 || (v.stride_t * es) % 16)
      return fail(SSD_ERR_ALIGN, "%s: strides (%lld, %lld) elements are not multiples of 16 bytes",
                  name, (long long)v.stride_b, (long long)v.stride_t);
  } else if (reinterpret_cast<uintptr_t>(v.ptr) % es) {
    return fail(SSD_ERR_ALIGN, "%s: base pointer not element-aligned", name);
  }
  return SSD_OK;
}

#define TRY(x)                      \
  do {                              \
    ssd_status _st = (x);           \
    if (_st != SSD_OK) return _st;  \
  } while (0)

ssd_status check_dims(const ssd_dims* d, ssd_dtype io) {
  if (!d) return fail(SSD_ERR_NULL, "dims: NULL");
  if (io != SSD_F32 && io != SSD_BF16) return fail(SSD_ERR_DTYPE, "unknown dtype %d", (int)io);
  if (d->batch < 1 || d->seqlen < 1 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
      d->ngroups < 1)
    return fail(SSD_ERR_SHAPE, "dims must be >= 1 (B=%lld L=%lld H=%lld P=%lld N=%lld G=%lld)",
                (long long)d->batch, (long long)d->seqlen, (long long)d->nheads,
                (long long)d->headdim, (long long)d->dstate, (long long)d->ngroups);
  if (d->nheads % d->ngroups)
    return fail(SSD_ERR_SHAPE, "nheads %lld not a multiple of ngroups %lld", (long long)d->nheads,
                (long long)d->ngroups);
  if (d->batch > (1 << 20) || d->nheads > 4096 || d->seqlen > (int64_t(1) << 40))
    return fail(SSD_ERR_SHAPE, "dims out of range");
  if (d->headdim != 32 && d->headdim != 64)
    return fail(SSD_ERR_UNSUPPORTED, "headdim %lld (supported: 32, 64)", (long long)d->headdim);
  if (d->dstate != 16 && d->dstate != 32 && d->dstate != 64 && d->dstate != 128)
    return fail(SSD_ERR_UNSUPPORTED, "dstate %lld (supported: 16, 32, 64, 128)",
                (long long)d->dstate);
  if (d->chunk != 0 && d->chunk != ssd::kQ)
    return fail(SSD_ERR_UNSUPPORTED, "chunk %lld (supported: 0 or %d)", (long long)d->chunk, ssd::kQ);
  if (d->conv_width != 0 && (d->conv_width < 2 || d->conv_width > 4))
    return fail(SSD_ERR_UNSUPPORTED, "conv_width %lld (supported: 0, 2, 3, 4)",
                (long long)d->conv_width);
  return SSD_OK;
}

ssd::View cv(const ssd_view& v) { return ssd::View{v.ptr, v.stride_b, v.stride_t}; }
ssd::MView mv(const ssd_view& v) { return ssd::MView{v.ptr, v.stride_b, v.stride_t}; }

ssd::Problem make_problem(const ssd_dims* d, ssd_dtype io) {
  ssd::Problem pr{};
  pr.bf16 = io == SSD_BF16;
  pr.B = d->batch;
  pr.L = d->seqlen;
  pr.H = static_cast<int>(d->nheads);
  pr.P = static_cast<int>(d->headdim);
  pr.N = static_cast<int>(d->dstate);
  pr.G = static_cast<int>(d->ngroups);
  pr.K = static_cast<int>(d->conv_width);
  return pr;
}

int64_t cdim(const ssd_dims* d) { return d->nheads * d->headdim + 2 * d->ngroups * d->dstate; }

}  // namespace

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char* ssd_status_string(int status) {
  switch (status) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_NULL: return "SSD_ERR_NULL: a required pointer is NULL";
    case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE: a dimension is out of range or inconsistent";
    case SSD_ERR_DTYPE: return "SSD_ERR_DTYPE: unknown dtype";
    case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN: pointer or stride breaks the alignment rule";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: shape not implemented";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace too small";
    case SSD_ERR_HIP: return "SSD_ERR_HIP: HIP launch or runtime error";
    default: return "unknown ssd_status";
  }
}

const char* ssd_last_error(void) { return g_last_error.c_str(); }

ssd_status ssd_fwd_workspace(const ssd_dims* d, ssd_dtype io, size_t* bytes) {
  TRY(check_dims(d, io));
  if (!bytes) return fail(SSD_ERR_NULL, "bytes: NULL");
  const ssd::Problem pr = make_problem(d, io);
  *bytes = ssd::fwd_workspace_bytes(pr, ssd::make_plan(pr.B, pr.L, pr.H));
  return SSD_OK;
}

}  // extern "C"

namespace {

// ssd_fwd with its scratch given as (ws, ws_bytes).  When `scratch` is non-null it is
// called after validation, with the bytes needed, and returns the scratch to use (or
// an error status through *st): the no-alloc entry point supplies the per-device
// static array this way, so nothing device-side happens before every check passed.
using ScratchFn = void* (*)(size_t need, ssd_status* st);

ssd_status fwd_impl(const ssd_dims* d, ssd_dtype io, ssd_view xbc, const float* conv_w,
                    const float* conv_b, ssd_view conv_state_in, ssd_view conv_state_out,
                    ssd_view dt, const float* dt_bias, int dt_softplus, const float* A,
                    const float* D, ssd_view z, const float* h0, ssd_view out, float* h_final,
                    float* h_ckpt, int64_t ckpt_every, void* ws, size_t ws_bytes, void* stream,
                    ScratchFn scratch) {
  g_last_error.clear();
  TRY(check_dims(d, io));
  const int64_t L = d->seqlen, Cd = cdim(d), HP = d->nheads * d->headdim;
  const int64_t K = d->conv_width;
  TRY(check_view(xbc, "xbc", io, true, true, L, Cd));
  TRY(check_view(dt, "dt", io, true, false, L, d->nheads));
  TRY(check_view(z, "z", io, false, true, L, HP));
  TRY(check_view(out, "out", io, true, true, L, HP));
  if (!A) return fail(SSD_ERR_NULL, "A: NULL");
  if (K > 0) {
    if (!conv_w) return fail(SSD_ERR_NULL, "conv_w: NULL with conv_width %lld", (long long)K);
    TRY(check_param16(conv_w, "conv_w"));
    TRY(check_param16(conv_b, "conv_b"));
    TRY(check_view(conv_state_in, "conv_state_in", io, false, true, K - 1, Cd));
    TRY(check_view(conv_state_out, "conv_state_out", io, false, true, K - 1, Cd));
  }
  TRY(check_state(h0, "h0"));
  TRY(check_state(h_final, "h_final"));
  TRY(check_state(h_ckpt, "h_ckpt"));
  if (h_ckpt && (ckpt_every <= 0 || ckpt_every % ssd::kQ))
    return fail(SSD_ERR_SHAPE, "ckpt_every %lld must be a positive multiple of %d",
                (long long)ckpt_every, ssd::kQ);
  ssd::Problem pr = make_problem(d, io);
  const ssd::Plan pl = ssd::make_plan(pr.B, pr.L, pr.H);
  const size_t need = ssd::fwd_workspace_bytes(pr, pl);
  if (scratch) {
    ssd_status st = SSD_OK;
    ws = scratch(need, &st);
    if (st != SSD_OK) return st;
    ws_bytes = need;
  }
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(SSD_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  pr.xbc = cv(xbc);
  pr.conv_w = K > 0 ? conv_w : nullptr;
  pr.conv_b = K > 0 ? conv_b : nullptr;
  pr.cs_in = K > 0 ? cv(conv_state_in) : ssd::View{nullptr, 0, 0};
  pr.dt = cv(dt);
  pr.dt_bias = dt_bias;
  pr.softplus = dt_softplus ? 1 : 0;
  pr.A = A;
  pr.D = D;
  pr.z = cv(z);
  pr.h0 = h0;
  ssd::FwdOut o{};
  o.out = mv(out);
  o.h_final = h_final;
  o.h_ckpt = h_ckpt;
  o.ckpt_every = ckpt_every;
  o.cs_out = K > 0 ? mv(conv_state_out) : ssd::MView{nullptr, 0, 0};
  const hipError_t e = ssd::launch_fwd(pr, o, pl, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ssd_fwd launch");
  return SSD_OK;
}

// ---------------------------------------------------------------- no-alloc scratch
//
// Scratch of ssd_fwd_noalloc: one file-scope device array, which every GPU the
// library runs on holds (at its own address) until the process ends.  Host code never
// uses the array's name as an address: the per-device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kNoAllocScratchBytes = SSD_FWD_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

void* noalloc_scratch(size_t need, ssd_status* st) {
  if (need > kNoAllocScratchBytes) {
    *st = fail(SSD_ERR_WORKSPACE,
               "ssd_fwd_noalloc: these dims need %zu bytes of scratch, above its fixed %zu bytes "
               "(use ssd_fwd with a caller workspace)", need, kNoAllocScratchBytes);
    return nullptr;
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = hip_fail(e, "ssd_fwd_noalloc: hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = fail(SSD_ERR_UNSUPPORTED, "ssd_fwd_noalloc: device %d beyond %d", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *st = hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                     "ssd_fwd_noalloc: hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

ssd_status ssd_fwd(const ssd_dims* d, ssd_dtype io, ssd_view xbc, const float* conv_w,
                   const float* conv_b, ssd_view conv_state_in, ssd_view conv_state_out,
                   ssd_view dt, const float* dt_bias, int dt_softplus, const float* A,
                   const float* D, ssd_view z, const float* h0, ssd_view out, float* h_final,
                   float* h_ckpt, int64_t ckpt_every, void* ws, size_t ws_bytes, void* stream) {
  return fwd_impl(d, io, xbc, conv_w, conv_b, conv_state_in, conv_state_out, dt, dt_bias,
                  dt_softplus, A, D, z, h0, out, h_final, h_ckpt, ckpt_every, ws, ws_bytes, stream,
                  nullptr);
}

ssd_status ssd_fwd_noalloc(const ssd_dims* d, ssd_dtype io, ssd_view xbc, const float* conv_w,
                           const float* conv_b, ssd_view conv_state_in, ssd_view conv_state_out,
                           ssd_view dt, const float* dt_bias, int dt_softplus, const float* A,
                           const float* D, ssd_view z, const float* h0, ssd_view out,
                           float* h_final, float* h_ckpt, int64_t ckpt_every, void* stream) {
  return fwd_impl(d, io, xbc, conv_w, conv_b, conv_state_in, conv_state_out, dt, dt_bias,
                  dt_softplus, A, D, z, h0, out, h_final, h_ckpt, ckpt_every, nullptr, 0, stream,
                  noalloc_scratch);
}

ssd_status ssd_bwd_workspace(const ssd_dims* d, ssd_dtype io, size_t* bytes) {
  TRY(check_dims(d, io));
  if (!bytes) return fail(SSD_ERR_NULL, "bytes: NULL");
  const ssd::Problem pr = make_problem(d, io);
  if (!ssd::bwd_supported(pr))
    return fail(SSD_ERR_UNSUPPORTED, "ssd_bwd with fp32 I/O supports dstate <= 64");
  *bytes = ssd::bwd_workspace_bytes(pr);
  return SSD_OK;
}

ssd_status ssd_bwd(const ssd_dims* d, ssd_dtype io, ssd_view xbc, const float* conv_w,
                   const float* conv_b, ssd_view conv_state_in, ssd_view dt, const float* dt_bias,
                   int dt_softplus, const float* A, const float* D, ssd_view z, const float* h0,
                   ssd_view dout, const float* dh_final, ssd_view dconv_state_out, ssd_view dxbc,
                   ssd_view ddt, ssd_view dz, float* dA, float* dD, float* ddt_bias,
                   float* dconv_w, float* dconv_b, float* dh0, ssd_view dconv_state_in,
                   int accumulate, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  TRY(check_dims(d, io));
  const int64_t L = d->seqlen, Cd = cdim(d), HP = d->nheads * d->headdim;
  const int64_t K = d->conv_width;
  TRY(check_view(xbc, "xbc", io, true, true, L, Cd));
  TRY(check_view(dt, "dt", io, true, false, L, d->nheads));
  TRY(check_view(z, "z", io, false, true, L, HP));
  TRY(check_view(dout, "dout", io, true, true, L, HP));
  TRY(check_view(dxbc, "dxbc", io, true, true, L, Cd));
  TRY(check_view(ddt, "ddt", io, true, false, L, d->nheads));
  TRY(check_view(dz, "dz", io, z.ptr != nullptr, true, L, HP));
  if (!A) return fail(SSD_ERR_NULL, "A: NULL");
  if (!dA) return fail(SSD_ERR_NULL, "dA: NULL");
  TRY(check_state(h0, "h0"));
  TRY(check_state(dh_final, "dh_final"));
  TRY(check_state(dh0, "dh0"));
  if (K > 0) {
    if (!conv_w) return fail(SSD_ERR_NULL, "conv_w: NULL with conv_width %lld", (long long)K);
    TRY(check_param16(conv_w, "conv_w"));
    TRY(check_param16(conv_b, "conv_b"));
    TRY(check_view(conv_state_in, "conv_state_in", io, false, true, K - 1, Cd));
    TRY(check_view(dconv_state_out, "dconv_state_out", io, false, true, K - 1, Cd));
    TRY(check_view(dconv_state_in, "dconv_state_in", io, false, true, K - 1, Cd));
  }
  ssd::Problem pr = make_problem(d, io);
  if (!ssd::bwd_supported(pr))
    return fail(SSD_ERR_UNSUPPORTED, "ssd_bwd with fp32 I/O supports dstate <= 64");
  const size_t need = ssd::bwd_workspace_bytes(pr);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(SSD_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  pr.xbc = cv(xbc);
  pr.conv_w = K > 0 ? conv_w : nullptr;
  pr.conv_b = K > 0 ? conv_b : nullptr;
  pr.cs_in = K > 0 ? cv(conv_state_in) : ssd::View{nullptr, 0, 0};
  pr.dt = cv(dt);
  pr.dt_bias = dt_bias;
  pr.softplus = dt_softplus ? 1 : 0;
  pr.A = A;
  pr.D = D;
  pr.z = cv(z);
  pr.h0 = h0;
  ssd::BwdIn in{};
  in.dout = cv(dout);
  in.dh_final = dh_final;
  in.dcs_out = K > 0 ? cv(dconv_state_out) : ssd::View{nullptr, 0, 0};
  ssd::BwdOut o{};
  o.dxbc = mv(dxbc);
  o.ddt = mv(ddt);
  o.dz = z.ptr ? mv(dz) : ssd::MView{nullptr, 0, 0};
  o.dA = dA;
  o.dD = dD;
  o.ddt_bias = ddt_bias;
  o.dconv_w = K > 0 ? dconv_w : nullptr;
  o.dconv_b = K > 0 ? dconv_b : nullptr;
  o.dh0 = dh0;
  o.dcs_in = K > 0 ? mv(dconv_state_in) : ssd::MView{nullptr, 0, 0};
  o.accumulate = accumulate ? 1 : 0;
  const hipError_t e = ssd::launch_bwd(pr, in, o, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ssd_bwd launch");
  return SSD_OK;
}

namespace {
ssd_status check_conv(int64_t batch, int64_t seqlen, int64_t channels, int32_t width,
                      ssd_dtype io) {
  if (io != SSD_F32 && io != SSD_BF16) return fail(SSD_ERR_DTYPE, "unknown dtype %d", (int)io);
  if (batch < 1 || seqlen < 1 || channels < 1 || batch > (1 << 20) || seqlen > (int64_t(1) << 40) ||
      channels > (1 << 24))
    return fail(SSD_ERR_SHAPE, "conv dims out of range (B=%lld L=%lld C=%lld)", (long long)batch,
                (long long)seqlen, (long long)channels);
  if (width < 2 || width > 4)
    return fail(SSD_ERR_UNSUPPORTED, "conv width %d (supported: 2, 3, 4)", (int)width);
  const int vec = io == SSD_BF16 ? 8 : 4;
  if (channels % vec)
    return fail(SSD_ERR_UNSUPPORTED, "channels %lld not a multiple of %d", (long long)channels, vec);
  return SSD_OK;
}

ssd::ConvProblem make_conv(int64_t batch, int64_t seqlen, int64_t channels, int32_t width,
                           ssd_dtype io, ssd_view x, const float* w, const float* b, int silu,
                           ssd_view state_in) {
  ssd::ConvProblem cp{};
  cp.bf16 = io == SSD_BF16;
  cp.B = batch;
  cp.L = seqlen;
  cp.C = channels;
  cp.K = width;
  cp.silu = silu ? 1 : 0;
  cp.x = cv(x);
  cp.w = w;
  cp.b = b;
  cp.state_in = cv(state_in);
  return cp;
}
}  // namespace

ssd_status conv1d_fwd(int64_t batch, int64_t seqlen, int64_t channels, int32_t width,
                      ssd_dtype io, ssd_view x, const float* w, const float* b, int silu,
                      ssd_view state_in, ssd_view out, ssd_view state_out, void* stream) {
  g_last_error.clear();
  TRY(check_conv(batch, seqlen, channels, width, io));
  TRY(check_view(x, "x", io, true, true, seqlen, channels));
  TRY(check_view(out, "out", io, true, true, seqlen, channels));
  TRY(check_view(state_in, "state_in", io, false, true, width - 1, channels));
  TRY(check_view(state_out, "state_out", io, false, true, width - 1, channels));
  if (!w) return fail(SSD_ERR_NULL, "w: NULL");
  TRY(check_param16(w, "w"));
  TRY(check_param16(b, "b"));
  const ssd::ConvProblem cp = make_conv(batch, seqlen, channels, width, io, x, w, b, silu, state_in);
  const hipError_t e = ssd::launch_conv_fwd(cp, mv(out), mv(state_out), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "conv1d_fwd launch");
  return SSD_OK;
}

ssd_status conv1d_bwd_workspace(int64_t batch, int64_t seqlen, int64_t channels, int32_t width,
                                size_t* bytes) {
  TRY(check_conv(batch, seqlen, channels, width, SSD_F32));
  if (!bytes) return fail(SSD_ERR_NULL, "bytes: NULL");
  *bytes = ssd::conv_bwd_workspace_bytes(batch, seqlen, channels);
  return SSD_OK;
}

ssd_status conv1d_bwd(int64_t batch, int64_t seqlen, int64_t channels, int32_t width,
                      ssd_dtype io, ssd_view x, const float* w, const float* b, int silu,
                      ssd_view state_in, ssd_view dout, ssd_view dstate_out, ssd_view dx,
                      float* dw, float* db, ssd_view dstate_in, int accumulate, void* ws,
                      size_t ws_bytes, void* stream) {
  g_last_error.clear();
  TRY(check_conv(batch, seqlen, channels, width, io));
  TRY(check_view(x, "x", io, true, true, seqlen, channels));
  TRY(check_view(dout, "dout", io, true, true, seqlen, channels));
  TRY(check_view(dx, "dx", io, true, true, seqlen, channels));
  TRY(check_view(state_in, "state_in", io, false, true, width - 1, channels));
  TRY(check_view(dstate_out, "dstate_out", io, false, true, width - 1, channels));
  TRY(check_view(dstate_in, "dstate_in", io, false, true, width - 1, channels));
  if (!w) return fail(SSD_ERR_NULL, "w: NULL");
  if (!dw) return fail(SSD_ERR_NULL, "dw: NULL");
  TRY(check_param16(w, "w"));
  TRY(check_param16(b, "b"));
  const size_t need = ssd::conv_bwd_workspace_bytes(batch, seqlen, channels);
  if (!ws || ws_bytes < need)
    return fail(SSD_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  const ssd::ConvProblem cp = make_conv(batch, seqlen, channels, width, io, x, w, b, silu, state_in);
  const hipError_t e = ssd::launch_conv_bwd(cp, cv(dout), cv(dstate_out), mv(dx), dw, db,
                                            mv(dstate_in), accumulate ? 1 : 0, ws,
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "conv1d_bwd launch");
  return SSD_OK;
}

ssd_status mixer_proj(int64_t M, int64_t N, int64_t K, ssd_dtype io, const void* x, int64_t ldx,
                      const void* w, int64_t ldw, const float* norm_w, float norm_eps,
                      const void* residual, int64_t ldr, void* y, int64_t ldy, void* stream) {
  g_last_error.clear();
  if (io != SSD_BF16) return fail(SSD_ERR_UNSUPPORTED, "mixer_proj: bf16 I/O only");
  if (M < 1 || N < 1 || K < 1 || M > (int64_t(1) << 40) || N > (1 << 24) || K > (1 << 24))
    return fail(SSD_ERR_SHAPE, "mixer_proj: dims out of range (M=%lld N=%lld K=%lld)", (long long)M,
                (long long)N, (long long)K);
  if (K % 64) return fail(SSD_ERR_UNSUPPORTED, "mixer_proj: K=%lld not a multiple of 64", (long long)K);
  if (N % 8) return fail(SSD_ERR_UNSUPPORTED, "mixer_proj: N=%lld not a multiple of 8", (long long)N);
  if (!x || !w || !y) return fail(SSD_ERR_NULL, "mixer_proj: x, w and y are required");
  if (ldx < K || ldw < K || ldy < N || (residual && ldr < N))
    return fail(SSD_ERR_SHAPE, "mixer_proj: a leading dimension is below its row length");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (residual && !aligned16(residual)) ||
      (norm_w && !aligned16(norm_w)))
    return fail(SSD_ERR_ALIGN, "mixer_proj: base pointers must be 16-byte aligned");
  if (ldx % 8 || ldw % 8 || ldy % 8 || (residual && ldr % 8))
    return fail(SSD_ERR_ALIGN, "mixer_proj: leading dimensions must be multiples of 8 elements");
  if (norm_w && !(norm_eps >= 0.f))
    return fail(SSD_ERR_SHAPE, "mixer_proj: norm_eps must be >= 0");
  ssd::LinearProblem lp{M, N, K, x, ldx, w, ldw, norm_w, norm_eps, residual, ldr, y, ldy};
  const hipError_t e = ssd::launch_linear(lp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mixer_proj launch");
  return SSD_OK;
}

ssd_status ssd_decode(const ssd_dims* d, ssd_dtype io, ssd_view xbc, const float* conv_w,
                      const float* conv_b, ssd_view conv_state_in, ssd_view conv_state_out,
                      ssd_view dt, const float* dt_bias, int dt_softplus, const float* A,
                      const float* D, ssd_view z, const float* h_in, float* h_out, ssd_view out,
                      void* stream) {
  g_last_error.clear();
  TRY(check_dims(d, io));
  const int64_t T = d->seqlen, Cd = cdim(d), HP = d->nheads * d->headdim;
  const int64_t K = d->conv_width;
  // element-aligned views: the decode step reads single elements
  TRY(check_view(xbc, "xbc", io, true, false, T, Cd));
  TRY(check_view(dt, "dt", io, true, false, T, d->nheads));
  TRY(check_view(z, "z", io, false, false, T, HP));
  TRY(check_view(out, "out", io, true, false, T, HP));
  if (!A) return fail(SSD_ERR_NULL, "A: NULL");
  if (!h_out) return fail(SSD_ERR_NULL, "h_out: NULL (the decode state is always returned)");
  if (K > 1) {
    if (!conv_w) return fail(SSD_ERR_NULL, "conv_w: NULL with conv_width %lld", (long long)K);
    TRY(check_view(conv_state_in, "conv_state_in", io, false, false, K - 1, Cd));
    TRY(check_view(conv_state_out, "conv_state_out", io, true, false, K - 1, Cd));
    if (conv_state_in.ptr && conv_state_in.ptr == conv_state_out.ptr)
      return fail(SSD_ERR_SHAPE, "conv_state_out must not alias conv_state_in");
  } else if (K > 0 && !conv_w) {
    return fail(SSD_ERR_NULL, "conv_w: NULL with conv_width %lld", (long long)K);
  }
  ssd::Problem pr = make_problem(d, io);
  pr.xbc = cv(xbc);
  pr.conv_w = K > 0 ? conv_w : nullptr;
  pr.conv_b = K > 0 ? conv_b : nullptr;
  pr.cs_in = K > 1 ? cv(conv_state_in) : ssd::View{nullptr, 0, 0};
  pr.dt = cv(dt);
  pr.dt_bias = dt_bias;
  pr.softplus = dt_softplus ? 1 : 0;
  pr.A = A;
  pr.D = D;
  pr.z = cv(z);
  pr.h0 = h_in;
  const hipError_t e = ssd::launch_decode(pr, h_out, mv(out),
                                          K > 1 ? mv(conv_state_out) : ssd::MView{nullptr, 0, 0},
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ssd_decode launch");
  return SSD_OK;
}

namespace {
ssd_status check_mat(const void* p, int64_t ld, int64_t cols, const char* name) {
  if (!p) return fail(SSD_ERR_NULL, "%s: NULL", name);
  if (ld < cols) return fail(SSD_ERR_SHAPE, "%s: leading dimension %lld below its row length %lld", name,
                             (long long)ld, (long long)cols);
  if (!aligned16(p) || ld % 8)
    return fail(SSD_ERR_ALIGN, "%s: base 16-byte aligned and leading dimension a multiple of 8 required", name);
  return SSD_OK;
}
}  // namespace

ssd_status mixer_proj_bwd(int64_t M, int64_t N, int64_t K, ssd_dtype io, const void* dy, int64_t lddy,
                          const void* x, int64_t ldx, const void* w, int64_t ldw, void* dx, int64_t lddx,
                          float* dw, int64_t lddw, int accumulate, void* stream) {
  g_last_error.clear();
  if (io != SSD_BF16) return fail(SSD_ERR_UNSUPPORTED, "mixer_proj_bwd: bf16 I/O only");
  if (M < 1 || N < 1 || K < 1 || M > (int64_t(1) << 40) || N > (1 << 24) || K > (1 << 24))
    return fail(SSD_ERR_SHAPE, "mixer_proj_bwd: dims out of range (M=%lld N=%lld K=%lld)", (long long)M,
                (long long)N, (long long)K);
  if (N % 8 || K % 8)
    return fail(SSD_ERR_UNSUPPORTED, "mixer_proj_bwd: N=%lld and K=%lld must be multiples of 8", (long long)N,
                (long long)K);
  if (!dx && !dw) return fail(SSD_ERR_NULL, "mixer_proj_bwd: neither dx nor dw requested");
  TRY(check_mat(dy, lddy, N, "dy"));
  if (dx) {
    TRY(check_mat(w, ldw, K, "w"));
    TRY(check_mat(dx, lddx, K, "dx"));
  }
  if (dw) {
    TRY(check_mat(x, ldx, K, "x"));
    if (lddw < K) return fail(SSD_ERR_SHAPE, "dw: leading dimension below K");
    if (reinterpret_cast<uintptr_t>(dw) % 4) return fail(SSD_ERR_ALIGN, "dw: not 4-byte aligned");
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (dx) e = ssd::launch_linear_dgrad(M, N, K, dy, lddy, w, ldw, dx, lddx, s);
  if (e == hipSuccess && dw) e = ssd::launch_linear_wgrad(M, N, K, dy, lddy, x, ldx, dw, lddw, accumulate, s);
  if (e != hipSuccess) return hip_fail(e, "mixer_proj_bwd launch");
  return SSD_OK;
}

ssd_status rmsnorm_fwd(int64_t M, int64_t K, ssd_dtype io, const void* x, int64_t ldx, const float* g,
                       float eps, void* y, int64_t ldy, float* rstd, void* stream) {
  g_last_error.clear();
  if (io != SSD_BF16) return fail(SSD_ERR_UNSUPPORTED, "rmsnorm_fwd: bf16 I/O only");
  if (M < 1 || K < 8 || M > (int64_t(1) << 40)) return fail(SSD_ERR_SHAPE, "rmsnorm_fwd: dims out of range");
  if (K % 8 || K > ssd::rmsnorm_max_k())
    return fail(SSD_ERR_UNSUPPORTED, "rmsnorm_fwd: K=%lld (multiples of 8 up to %d)", (long long)K,
                ssd::rmsnorm_max_k());
  TRY(check_mat(x, ldx, K, "x"));
  TRY(check_mat(y, ldy, K, "y"));
  if (!g || !aligned16(g)) return fail(SSD_ERR_ALIGN, "rmsnorm_fwd: g NULL or not 16-byte aligned");
  if (!(eps >= 0.f)) return fail(SSD_ERR_SHAPE, "rmsnorm_fwd: eps must be >= 0");
  const hipError_t e = ssd::launch_rmsnorm_fwd(M, static_cast<int>(K), x, ldx, g, eps, y, ldy, rstd,
                                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rmsnorm_fwd launch");
  return SSD_OK;
}

ssd_status rmsnorm_bwd_workspace(int64_t K, size_t* bytes) {
  if (!bytes) return fail(SSD_ERR_NULL, "bytes: NULL");
  if (K < 8 || K % 8 || K > ssd::rmsnorm_max_k())
    return fail(SSD_ERR_UNSUPPORTED, "rmsnorm_bwd: K=%lld (multiples of 8 up to %d)", (long long)K,
                ssd::rmsnorm_max_k());
  *bytes = ssd::rmsnorm_bwd_workspace_bytes(K);
  return SSD_OK;
}

ssd_status rmsnorm_bwd(int64_t M, int64_t K, ssd_dtype io, const void* x, int64_t ldx, const float* g,
                       float eps, const void* dy, int64_t lddy, const void* dres, int64_t ldres, void* dx,
                       int64_t lddx, float* dg, int accumulate, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (io != SSD_BF16) return fail(SSD_ERR_UNSUPPORTED, "rmsnorm_bwd: bf16 I/O only");
  if (M < 1 || M > (int64_t(1) << 40)) return fail(SSD_ERR_SHAPE, "rmsnorm_bwd: dims out of range");
  size_t need = 0;
  TRY(rmsnorm_bwd_workspace(K, &need));
  TRY(check_mat(x, ldx, K, "x"));
  TRY(check_mat(dy, lddy, K, "dy"));
  TRY(check_mat(dx, lddx, K, "dx"));
  if (dres) TRY(check_mat(dres, ldres, K, "dres"));
  if (!g || !aligned16(g)) return fail(SSD_ERR_ALIGN, "rmsnorm_bwd: g NULL or not 16-byte aligned");
  if (dg && !aligned16(dg)) return fail(SSD_ERR_ALIGN, "rmsnorm_bwd: dg not 16-byte aligned");
  if (!(eps >= 0.f)) return fail(SSD_ERR_SHAPE, "rmsnorm_bwd: eps must be >= 0");
  if (!ws || ws_bytes < need)
    return fail(SSD_ERR_WORKSPACE, "rmsnorm_bwd: workspace %zu bytes < %zu needed", ws_bytes, need);
  const hipError_t e = ssd::launch_rmsnorm_bwd(M, static_cast<int>(K), x, ldx, g, eps, dy, lddy, dres, ldres,
                                               dx, lddx, dg, accumulate, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rmsnorm_bwd launch");
  return SSD_OK;
}

}  // extern "C"
