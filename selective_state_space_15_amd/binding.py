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
    "ssd_bwd": ([_D, _I, _V, _F, _F, _V, _V, _F, _I, _F, _F, _V, _F, _V, _F, _V, _V, _V, _V,
                 _F, _F, _F, _F, _F, _F, _V, _I, _P, _SZ, _P], _I),
    "conv1d_fwd": ([_I64, _I64, _I64, ctypes.c_int32, _I, _V, _F, _F, _I, _V, _V, _V, _P], _I),
    "conv1d_bwd_workspace": ([_I64, _I64, _I64, ctypes.c_int32, ctypes.POINTER(_SZ)], _I),
    "conv1d_bwd": ([_I64, _I64, _I64, ctypes.c_int32, _I, _V, _F, _F, _I, _V, _V, _V, _V, _F, _F, _V,
                    _I, _P, _SZ, _P], _I),
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
    wsp, wsn = _ws(ws)
    st = lib().ssd_fwd(ctypes.byref(d), io_dtype(xbc), view(xbc), fptr(conv_w), fptr(conv_b),
                       view(conv_state_in), view(conv_state_out), view(dt), fptr(dt_bias),
                       int(bool(dt_softplus)), fptr(A), fptr(D), view(z), fptr(h0), view(out),
                       fptr(h_final), fptr(h_ckpt), int(ckpt_every), wsp, wsn, stream_ptr(stream))
    _check(st, "ssd_fwd")


def ssd_bwd(d: ssd_dims, xbc, A, dt, dout, dxbc, ddt, dA, *, conv_w=None, conv_b=None,
            conv_state_in=None, dt_bias=None, dt_softplus=True, D=None, z=None, h0=None,
            dh_final=None, dconv_state_out=None, dz=None, dD=None, ddt_bias=None, dconv_w=None,
            dconv_b=None, dh0=None, dconv_state_in=None, accumulate=False, ws=None, stream=None):
    """Enqueue ssd_bwd (gradients of ssd_fwd; see include/ssd.h)."""
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
    st = lib().conv1d_fwd(B, L, C, w.shape[1], io_dtype(x), view(x), fptr(w), fptr(b),
                          int(bool(silu)), view(state_in), view(out), view(state_out),
                          stream_ptr(stream))
    _check(st, "conv1d_fwd")


def conv1d_bwd(x, w, dout, dx, dw, *, b=None, silu=True, state_in=None, dstate_out=None, db=None,
               dstate_in=None, accumulate=False, ws=None, stream=None):
    B, L, C = x.shape
    wsp, wsn = _ws(ws)
    st = lib().conv1d_bwd(B, L, C, w.shape[1], io_dtype(x), view(x), fptr(w), fptr(b),
                          int(bool(silu)), view(state_in), view(dout), view(dstate_out), view(dx),
                          fptr(dw), fptr(db), view(dstate_in), int(bool(accumulate)), wsp, wsn,
                          stream_ptr(stream))
    _check(st, "conv1d_bwd")


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
