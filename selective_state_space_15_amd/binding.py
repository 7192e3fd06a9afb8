"""Thin ctypes binding of libssd.so (the C ABI in include/ssd.h).

Argument marshalling only: tensors are passed as device pointers and element
strides, the stream is torch's current HIP stream, and every status code other
than SSD_OK raises SsdError with the library's detail text.  All arithmetic of the
hot path runs in the HIP kernels behind these calls; nothing here computes.

Torch is used for device memory and streams only.  A missing or unloadable
library raises at import of the first call -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd.so")

SSD_OK, SSD_ERR_NULL, SSD_ERR_SHAPE, SSD_ERR_DTYPE = 0, -1, -2, -3
SSD_ERR_ALIGN, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP = -4, -5, -6, -7
SSD_F32, SSD_BF16 = 0, 1


class SsdError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class ssd_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "chunk", "conv_width")]


class ssd_view(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_t", ctypes.c_int64)]


_V = ssd_view
_F = ctypes.c_void_p          # float* (device)
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_D = ctypes.POINTER(ssd_dims)

_SIGS = {
    "ssd_abi_version": ([], _I),
    "ssd_status_string": ([_I], ctypes.c_char_p),
    "ssd_last_error": ([], ctypes.c_char_p),
    "ssd_fwd_workspace": ([_D, _I, ctypes.POINTER(_SZ)], _I),
    "ssd_bwd_workspace": ([_D, _I, ctypes.POINTER(_SZ)], _I),
    "ssd_fwd": ([_D, _I, _V, _F, _F, _V, _V, _V, _F, _I, _F, _F, _V, _F, _V, _F, _F, _I64, _P, _SZ, _P], _I),
    "ssd_fwd_noalloc": ([_D, _I, _V, _F, _F, _V, _V, _V, _F, _I, _F, _F, _V, _F, _V, _F, _F, _I64, _P], _I),
    "ssd_bwd": ([_D, _I, _V, _F, _F, _V, _V, _F, _I, _F, _F, _V, _F, _V, _F, _V, _V, _V, _V,
                 _F, _F, _F, _F, _F, _F, _V, _I, _P, _SZ, _P], _I),
    "conv1d_fwd": ([_I64, _I64, _I64, ctypes.c_int32, _I, _V, _F, _F, _I, _V, _V, _V, _P], _I),
    "conv1d_bwd_workspace": ([_I64, _I64, _I64, ctypes.c_int32, ctypes.POINTER(_SZ)], _I),
    "conv1d_bwd": ([_I64, _I64, _I64, ctypes.c_int32, _I, _V, _F, _F, _I, _V, _V, _V, _V, _F, _F, _V,
                    _I, _P, _SZ, _P], _I),
    "ssd_decode": ([_D, _I, _V, _F, _F, _V, _V, _V, _F, _I, _F, _F, _V, _F, _F, _V, _P], _I),
    "mixer_proj": ([_I64, _I64, _I64, _I, _P, _I64, _P, _I64, _F, ctypes.c_float, _P, _I64, _P, _I64,
                    _P], _I),
    "mixer_proj_bwd": ([_I64, _I64, _I64, _I, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _F, _I64, _I, _P], _I),
    "rmsnorm_fwd": ([_I64, _I64, _I, _P, _I64, _F, ctypes.c_float, _P, _I64, _F, _P], _I),
    "rmsnorm_bwd_workspace": ([_I64, ctypes.POINTER(_SZ)], _I),
    "rmsnorm_bwd": ([_I64, _I64, _I, _P, _I64, _F, ctypes.c_float, _P, _I64, _P, _I64, _P, _I64, _F, _I, _P,
                     _SZ, _P], _I),
    "ssd_timing_enable": ([_I], _I),
    "ssd_timing_read": ([_I, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64)], _I),
    "ssd_timing_name": ([_I], ctypes.c_char_p),
    "ssd_timing_kinds": ([], _I),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libssd.so (built by build.py).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() "
                               "(or python -m selective_state_space_15_amd.build)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = res
        _lib = l
    return _lib


def exported_symbols():
    return list(_SIGS)


def _check(st: int, where: str):
    if st != SSD_OK:
        raise SsdError(st, where, lib().ssd_last_error().decode())


# ------------------------------------------------------------------ marshalling

def io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    raise TypeError(f"unsupported I/O dtype {t.dtype}")


def view(t: torch.Tensor | None) -> ssd_view:
    """[B, T, C] tensor (channel dim contiguous) -> ssd_view; None -> absent."""
    if t is None:
        return ssd_view(None, 0, 0)
    if t.dim() != 3 or (t.shape[2] > 1 and t.stride(2) != 1):
        raise ValueError(f"expected a [B, T, C] view with contiguous channels, got {tuple(t.shape)} "
                         f"strides {t.stride()}")
    return ssd_view(t.data_ptr(), t.stride(0), t.stride(1))


def fptr(t: torch.Tensor | None):
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError("fp32 contiguous tensor expected")
    return t.data_ptr()


def stream_ptr(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_dims(batch, seqlen, nheads, headdim, dstate, ngroups=1, chunk=0, conv_width=0) -> ssd_dims:
    return ssd_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, conv_width)


# ------------------------------------------------------------------ argument checks
#
# The C ABI receives raw device pointers and cannot see sizes, so a short or
# mistyped tensor would turn into an out-of-bounds device access.  Every entry point
# below therefore checks, before the call, that each tensor is on the same CUDA
# device, has the dtype the call expects and at least the extent the kernels touch.

def _dev_of(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError(f"tensor on {t.device}: every argument must be a CUDA (HIP) tensor")
    return t.device


def _same_device(ts, where):
    devs = {_dev_of(t) for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"{where}: tensors on several devices {sorted(map(str, devs))}")


def _act(t, name, B, T, C, dtype, required=True):
    """[B, T, >=C] activation view in the I/O dtype."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.dim() != 3 or tuple(t.shape[:2]) != (B, T) or t.shape[2] != C:
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected ({B}, {T}, {C})")


def _f32(t, name, shape, required=False):
    """fp32 contiguous tensor of exactly `shape`."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if t.dtype != torch.float32:
        raise ValueError(f"{name}: dtype {t.dtype}, expected torch.float32")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _ws_ok(ws, need, where):
    if need == 0:
        return
    if ws is None or ws.numel() * ws.element_size() < need:
        have = 0 if ws is None else ws.numel() * ws.element_size()
        raise ValueError(f"{where}: workspace of {have} bytes < {need} needed")


def _ssd_common(d: ssd_dims, xbc, A, dt, conv_w, conv_b, conv_states, dt_bias, D, z, h0):
    B, L, H, P, N, G, K = d.batch, d.seqlen, d.nheads, d.headdim, d.dstate, d.ngroups, d.conv_width
    cd = H * P + 2 * G * N
    if xbc is None:
        raise ValueError("xbc is required")
    io = xbc.dtype
    _act(xbc, "xbc", B, L, cd, io)
    _act(dt, "dt", B, L, H, io)
    _act(z, "z", B, L, H * P, io, required=False)
    _f32(A, "A", (H,), required=True)
    _f32(D, "D", (H,))
    _f32(dt_bias, "dt_bias", (H,))
    _f32(h0, "h0", (B, H, P, N))
    if K > 0:
        _f32(conv_w, "conv_w", (cd, K), required=True)
        _f32(conv_b, "conv_b", (cd,))
        for name, t in conv_states.items():
            _act(t, name, B, K - 1, cd, io, required=False)
    return io, cd


# ------------------------------------------------------------------ entry points

def ssd_abi_version() -> int:
    return lib().ssd_abi_version()


def ssd_status_string(status: int) -> str:
    return lib().ssd_status_string(status).decode()


def ssd_fwd_workspace(d: ssd_dims, io: int) -> int:
    n = _SZ(0)
    _check(lib().ssd_fwd_workspace(ctypes.byref(d), io, ctypes.byref(n)), "ssd_fwd_workspace")
    return n.value


def ssd_bwd_workspace(d: ssd_dims, io: int) -> int:
    n = _SZ(0)
    _check(lib().ssd_bwd_workspace(ctypes.byref(d), io, ctypes.byref(n)), "ssd_bwd_workspace")
    return n.value


def conv1d_bwd_workspace(batch, seqlen, channels, width) -> int:
    n = _SZ(0)
    _check(lib().conv1d_bwd_workspace(batch, seqlen, channels, width, ctypes.byref(n)),
           "conv1d_bwd_workspace")
    return n.value


def _ws(t: torch.Tensor | None):
    return (None, 0) if t is None else (t.data_ptr(), t.numel() * t.element_size())


def ssd_fwd(d: ssd_dims, xbc, A, dt, out, *, conv_w=None, conv_b=None, conv_state_in=None,
            conv_state_out=None, dt_bias=None, dt_softplus=True, D=None, z=None, h0=None,
            h_final=None, h_ckpt=None, ckpt_every=0, ws=None, stream=None):
    """Enqueue ssd_fwd.  Tensor views: xbc [B,L,Cd], dt [B,L,H], z/out [B,L,H*P],
    conv states [B,K-1,Cd]; fp32 contiguous A, D, dt_bias, conv_w, conv_b, h0,
    h_final, h_ckpt; ws a byte tensor of ssd_fwd_workspace() bytes (or None)."""
    io, cd = _ssd_common(d, xbc, A, dt, conv_w, conv_b,
                         dict(conv_state_in=conv_state_in, conv_state_out=conv_state_out),
                         dt_bias, D, z, h0)
    B, L, H, P, N = d.batch, d.seqlen, d.nheads, d.headdim, d.dstate
    _act(out, "out", B, L, H * P, io)
    _f32(h_final, "h_final", (B, H, P, N))
    if h_ckpt is not None:
        if ckpt_every <= 0:
            raise ValueError("ckpt_every must be positive with h_ckpt")
        _f32(h_ckpt, "h_ckpt", ((L + ckpt_every - 1) // ckpt_every, B, H, P, N))
    _same_device([xbc, A, dt, out, conv_w, conv_b, conv_state_in, conv_state_out, dt_bias, D, z, h0,
                  h_final, h_ckpt, ws], "ssd_fwd")
    _ws_ok(ws, ssd_fwd_workspace(d, io_dtype(xbc)), "ssd_fwd")
    wsp, wsn = _ws(ws)
    st = lib().ssd_fwd(ctypes.byref(d), io_dtype(xbc), view(xbc), fptr(conv_w), fptr(conv_b),
                       view(conv_state_in), view(conv_state_out), view(dt), fptr(dt_bias),
                       int(bool(dt_softplus)), fptr(A), fptr(D), view(z), fptr(h0), view(out),
                       fptr(h_final), fptr(h_ckpt), int(ckpt_every), wsp, wsn, stream_ptr(stream))
    _check(st, "ssd_fwd")


NOALLOC_SCRATCH_BYTES = 128 << 20   # SSD_FWD_NOALLOC_SCRATCH_BYTES in include/ssd.h


def ssd_fwd_noalloc(d: ssd_dims, xbc, A, dt, out, *, conv_w=None, conv_b=None, conv_state_in=None,
                    conv_state_out=None, dt_bias=None, dt_softplus=True, D=None, z=None, h0=None,
                    h_final=None, h_ckpt=None, ckpt_every=0, stream=None):
    """Enqueue ssd_fwd_noalloc: ssd_fwd whose scratch is the library's fixed per-device
    array (no workspace argument, nothing allocated).  Same tensors as ssd_fwd."""
    io, cd = _ssd_common(d, xbc, A, dt, conv_w, conv_b,
                         dict(conv_state_in=conv_state_in, conv_state_out=conv_state_out),
                         dt_bias, D, z, h0)
    B, L, H, P, N = d.batch, d.seqlen, d.nheads, d.headdim, d.dstate
    _act(out, "out", B, L, H * P, io)
    _f32(h_final, "h_final", (B, H, P, N))
    if h_ckpt is not None:
        if ckpt_every <= 0:
            raise ValueError("ckpt_every must be positive with h_ckpt")
        _f32(h_ckpt, "h_ckpt", ((L + ckpt_every - 1) // ckpt_every, B, H, P, N))
    _same_device([xbc, A, dt, out, conv_w, conv_b, conv_state_in, conv_state_out, dt_bias, D, z, h0,
                  h_final, h_ckpt], "ssd_fwd_noalloc")
    st = lib().ssd_fwd_noalloc(ctypes.byref(d), io_dtype(xbc), view(xbc), fptr(conv_w), fptr(conv_b),
                               view(conv_state_in), view(conv_state_out), view(dt), fptr(dt_bias),
                               int(bool(dt_softplus)), fptr(A), fptr(D), view(z), fptr(h0), view(out),
                               fptr(h_final), fptr(h_ckpt), int(ckpt_every), stream_ptr(stream))
    _check(st, "ssd_fwd_noalloc")


def ssd_bwd(d: ssd_dims, xbc, A, dt, dout, dxbc, ddt, dA, *, conv_w=None, conv_b=None,
            conv_state_in=None, dt_bias=None, dt_softplus=True, D=None, z=None, h0=None,
            dh_final=None, dconv_state_out=None, dz=None, dD=None, ddt_bias=None, dconv_w=None,
            dconv_b=None, dh0=None, dconv_state_in=None, accumulate=False, ws=None, stream=None):
    """Enqueue ssd_bwd (gradients of ssd_fwd; see include/ssd.h)."""
    io, cd = _ssd_common(d, xbc, A, dt, conv_w, conv_b,
                         dict(conv_state_in=conv_state_in, dconv_state_out=dconv_state_out,
                              dconv_state_in=dconv_state_in), dt_bias, D, z, h0)
    B, L, H, P, N, K = d.batch, d.seqlen, d.nheads, d.headdim, d.dstate, d.conv_width
    _act(dout, "dout", B, L, H * P, io)
    _act(dxbc, "dxbc", B, L, cd, io)
    _act(ddt, "ddt", B, L, H, io)
    _act(dz, "dz", B, L, H * P, io, required=z is not None)
    for name, t in (("dA", dA), ("dD", dD), ("ddt_bias", ddt_bias)):
        _f32(t, name, (H,), required=name == "dA")
    _f32(dh_final, "dh_final", (B, H, P, N))
    _f32(dh0, "dh0", (B, H, P, N))
    if K > 0:
        _f32(dconv_w, "dconv_w", (cd, K))
        _f32(dconv_b, "dconv_b", (cd,))
    _same_device([xbc, A, dt, dout, dxbc, ddt, dA, conv_w, conv_b, conv_state_in, dt_bias, D, z, h0,
                  dh_final, dconv_state_out, dz, dD, ddt_bias, dconv_w, dconv_b, dh0, dconv_state_in,
                  ws], "ssd_bwd")
    _ws_ok(ws, ssd_bwd_workspace(d, io_dtype(xbc)), "ssd_bwd")
    wsp, wsn = _ws(ws)
    st = lib().ssd_bwd(ctypes.byref(d), io_dtype(xbc), view(xbc), fptr(conv_w), fptr(conv_b),
                       view(conv_state_in), view(dt), fptr(dt_bias), int(bool(dt_softplus)),
                       fptr(A), fptr(D), view(z), fptr(h0), view(dout), fptr(dh_final),
                       view(dconv_state_out), view(dxbc), view(ddt), view(dz), fptr(dA), fptr(dD),
                       fptr(ddt_bias), fptr(dconv_w), fptr(dconv_b), fptr(dh0), view(dconv_state_in),
                       int(bool(accumulate)), wsp, wsn, stream_ptr(stream))
    _check(st, "ssd_bwd")


def conv1d_fwd(x, w, out, *, b=None, silu=True, state_in=None, state_out=None, stream=None):
    B, L, C = x.shape
    K = w.shape[1] if w is not None and w.dim() == 2 else 0
    _act(x, "x", B, L, C, x.dtype)
    _act(out, "out", B, L, C, x.dtype)
    _f32(w, "w", (C, K), required=True)
    _f32(b, "b", (C,))
    _act(state_in, "state_in", B, K - 1, C, x.dtype, required=False)
    _act(state_out, "state_out", B, K - 1, C, x.dtype, required=False)
    _same_device([x, w, out, b, state_in, state_out], "conv1d_fwd")
    st = lib().conv1d_fwd(B, L, C, w.shape[1], io_dtype(x), view(x), fptr(w), fptr(b),
                          int(bool(silu)), view(state_in), view(out), view(state_out),
                          stream_ptr(stream))
    _check(st, "conv1d_fwd")


def conv1d_bwd(x, w, dout, dx, dw, *, b=None, silu=True, state_in=None, dstate_out=None, db=None,
               dstate_in=None, accumulate=False, ws=None, stream=None):
    B, L, C = x.shape
    K = w.shape[1] if w is not None and w.dim() == 2 else 0
    for name, t in (("x", x), ("dout", dout), ("dx", dx)):
        _act(t, name, B, L, C, x.dtype)
    _f32(w, "w", (C, K), required=True)
    _f32(dw, "dw", (C, K), required=True)
    _f32(b, "b", (C,))
    _f32(db, "db", (C,))
    for name, t in (("state_in", state_in), ("dstate_out", dstate_out), ("dstate_in", dstate_in)):
        _act(t, name, B, K - 1, C, x.dtype, required=False)
    _same_device([x, w, dout, dx, dw, b, state_in, dstate_out, db, dstate_in, ws], "conv1d_bwd")
    if K >= 2:
        _ws_ok(ws, conv1d_bwd_workspace(B, L, C, K), "conv1d_bwd")
    wsp, wsn = _ws(ws)
    st = lib().conv1d_bwd(B, L, C, w.shape[1], io_dtype(x), view(x), fptr(w), fptr(b),
                          int(bool(silu)), view(state_in), view(dout), view(dstate_out), view(dx),
                          fptr(dw), fptr(db), view(dstate_in), int(bool(accumulate)), wsp, wsn,
                          stream_ptr(stream))
    _check(st, "conv1d_bwd")


def ssd_decode(d: ssd_dims, xbc, A, dt, out, h_out, *, conv_w=None, conv_b=None, conv_state_in=None,
               conv_state_out=None, dt_bias=None, dt_softplus=True, D=None, z=None, h_in=None,
               stream=None):
    """Enqueue ssd_decode: d.seqlen new tokens stepped from (h_in, conv_state_in);
    h_out (may be h_in) and conv_state_out (not conv_state_in) receive the state."""
    io, cd = _ssd_common(d, xbc, A, dt, conv_w, conv_b,
                         dict(conv_state_in=conv_state_in, conv_state_out=conv_state_out),
                         dt_bias, D, z, h_in)
    B, L, H, P, N, K = d.batch, d.seqlen, d.nheads, d.headdim, d.dstate, d.conv_width
    _act(out, "out", B, L, H * P, io)
    _f32(h_out, "h_out", (B, H, P, N), required=True)
    if K > 1 and conv_state_out is None:
        raise ValueError("conv_state_out is required with a conv")
    _same_device([xbc, A, dt, out, h_out, conv_w, conv_b, conv_state_in, conv_state_out, dt_bias, D, z,
                  h_in], "ssd_decode")
    st = lib().ssd_decode(ctypes.byref(d), io_dtype(xbc), view(xbc), fptr(conv_w), fptr(conv_b),
                          view(conv_state_in), view(conv_state_out), view(dt), fptr(dt_bias),
                          int(bool(dt_softplus)), fptr(A), fptr(D), view(z), fptr(h_in), fptr(h_out),
                          view(out), stream_ptr(stream))
    _check(st, "ssd_decode")


def _mat(t, name, rows, cols):
    """[rows, >=cols] bf16 matrix with a contiguous last dim (a 2-D view of [.., C] rows)."""
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name}: dtype {t.dtype}, expected torch.bfloat16")
    if t.dim() != 2 or t.shape[0] != rows or t.shape[1] != cols or (cols > 1 and t.stride(1) != 1):
        raise ValueError(f"{name}: shape {tuple(t.shape)} strides {t.stride()}, expected ({rows}, {cols}) "
                         "with a contiguous last dim")
    return t.data_ptr(), t.stride(0)


def mixer_proj(x, w, y, *, norm_w=None, norm_eps=1e-5, residual=None, stream=None):
    """y = RMSNorm?(x) w^T (+ residual): x [M, K], w [N, K] (nn.Linear layout), y and
    residual [M, N]; bf16 2-D views with a contiguous last dim; norm_w [K] fp32."""
    M, K = x.shape
    N = w.shape[0]
    xp, ldx = _mat(x, "x", M, K)
    wp, ldw = _mat(w, "w", N, K)
    yp, ldy = _mat(y, "y", M, N)
    rp, ldr = _mat(residual, "residual", M, N) if residual is not None else (None, 0)
    _f32(norm_w, "norm_w", (K,))
    _same_device([x, w, y, residual, norm_w], "mixer_proj")
    st = lib().mixer_proj(M, N, K, SSD_BF16, xp, ldx, wp, ldw, fptr(norm_w), float(norm_eps), rp, ldr,
                          yp, ldy, stream_ptr(stream))
    _check(st, "mixer_proj")


def mixer_proj_bwd(dy, *, x=None, w=None, dx=None, dw=None, accumulate=False, stream=None):
    """dx = dy w (bf16) and/or dw (+)= dy^T x (fp32) for y = x w^T: dy [M, N], x [M, K],
    w [N, K], dx [M, K] bf16 2-D views; dw [N, K] fp32 contiguous."""
    M, N = dy.shape
    K = (w.shape[1] if w is not None else x.shape[1])
    dyp, lddy = _mat(dy, "dy", M, N)
    xp, ldx = _mat(x, "x", M, K) if x is not None else (None, 0)
    wp, ldw = _mat(w, "w", N, K) if w is not None else (None, 0)
    dxp, lddx = _mat(dx, "dx", M, K) if dx is not None else (None, 0)
    if dx is not None and w is None:
        raise ValueError("dx needs w")
    if dw is not None and x is None:
        raise ValueError("dw needs x")
    _f32(dw, "dw", (N, K))
    _same_device([dy, x, w, dx, dw], "mixer_proj_bwd")
    st = lib().mixer_proj_bwd(M, N, K, SSD_BF16, dyp, lddy, xp, ldx, wp, ldw, dxp, lddx, fptr(dw), K,
                              int(bool(accumulate)), stream_ptr(stream))
    _check(st, "mixer_proj_bwd")


def rmsnorm_fwd(x, g, y, *, eps=1e-5, rstd=None, stream=None):
    """y = RMSNorm(x) * g over the last dim of 2-D bf16 views x, y [M, K]; g [K] fp32."""
    M, K = x.shape
    xp, ldx = _mat(x, "x", M, K)
    yp, ldy = _mat(y, "y", M, K)
    _f32(g, "g", (K,), required=True)
    _f32(rstd, "rstd", (M,))
    _same_device([x, g, y, rstd], "rmsnorm_fwd")
    _check(lib().rmsnorm_fwd(M, K, SSD_BF16, xp, ldx, fptr(g), float(eps), yp, ldy, fptr(rstd),
                             stream_ptr(stream)), "rmsnorm_fwd")


def rmsnorm_bwd_workspace(K) -> int:
    n = _SZ(0)
    _check(lib().rmsnorm_bwd_workspace(K, ctypes.byref(n)), "rmsnorm_bwd_workspace")
    return n.value


def rmsnorm_bwd(x, g, dy, dx, *, eps=1e-5, dres=None, dg=None, accumulate=False, ws=None, stream=None):
    """dx = d RMSNorm(x)*g / dx . dy (+ dres); dg (+)= gradient of g.  2-D bf16 views."""
    M, K = x.shape
    xp, ldx = _mat(x, "x", M, K)
    dyp, lddy = _mat(dy, "dy", M, K)
    dxp, lddx = _mat(dx, "dx", M, K)
    rp, ldr = _mat(dres, "dres", M, K) if dres is not None else (None, 0)
    _f32(g, "g", (K,), required=True)
    _f32(dg, "dg", (K,))
    _same_device([x, g, dy, dx, dres, dg, ws], "rmsnorm_bwd")
    _ws_ok(ws, rmsnorm_bwd_workspace(K), "rmsnorm_bwd")
    wsp, wsn = _ws(ws)
    _check(lib().rmsnorm_bwd(M, K, SSD_BF16, xp, ldx, fptr(g), float(eps), dyp, lddy, rp, ldr, dxp, lddx,
                             fptr(dg), int(bool(accumulate)), wsp, wsn, stream_ptr(stream)), "rmsnorm_bwd")


# ------------------------------------------------------------------ timing instrumentation

def ssd_timing_enable(on: bool) -> None:
    _check(lib().ssd_timing_enable(int(bool(on))), "ssd_timing_enable")


def ssd_timing_read() -> dict:
    """{kernel name: (total_ms, launches)} for every kind recorded since enable."""
    out = {}
    for k in range(lib().ssd_timing_kinds()):
        ms, n = ctypes.c_double(0.0), _I64(0)
        _check(lib().ssd_timing_read(k, ctypes.byref(ms), ctypes.byref(n)), "ssd_timing_read")
        out[lib().ssd_timing_name(k).decode()] = (ms.value, n.value)
    return out
