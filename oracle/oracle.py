"""ctypes wrapper around the fp64 CPU oracle (ssd_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU-baseline
leg may import this module; the GPU library and its Python binding never do.

Every array is converted to contiguous float64 before the call.  Shapes follow the
oracle's header comment:
    x, z        [B, L, H, P]      dt_raw      [B, L, H]
    Bm, Cm      [B, L, G, N]      h0          [B, H, P, N]
    conv input  [B, L, Cd]        conv state  [B, K-1, Cd]     conv weight [Cd, K]

The mixer helpers compose the conv and the SSD the way a Mamba-2 mixer wires
them: the conv output row is split into x (H*P channels), then B (G*N), then
C (G*N) -- the channel order of the Mamba-2 block that the Video-Ma2mba and
Vamba pages build on.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile ssd_oracle.c into liboracle.so (gcc, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = ctypes.CDLL(_LIB)
        for name in ("oracle_conv1d_fwd", "oracle_conv1d_bwd", "oracle_ssd_fwd", "oracle_ssd_bwd"):
            getattr(_lib, name).restype = None
        _lib.oracle_num_threads.restype = ctypes.c_int
    return _lib


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def _c(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


# --------------------------------------------------------------------------- conv

def conv1d_fwd(xraw, w, bias=None, state_in=None, silu=True):
    """Causal depthwise conv (+SiLU).  Returns (out [B,L,Cd], state_out [B,K-1,Cd])."""
    xraw, w, bias, state_in = _c(xraw), _c(w), _c(bias), _c(state_in)
    Bsz, L, Cd = xraw.shape
    K = w.shape[1]
    out = np.empty((Bsz, L, Cd))
    st = np.empty((Bsz, K - 1, Cd))
    lib().oracle_conv1d_fwd(_i64(Bsz), _i64(L), _i64(Cd), ctypes.c_int(K), _p(xraw),
                            _p(state_in), _p(w), _p(bias), ctypes.c_int(int(silu)),
                            _p(out), _p(st))
    return out, st


def conv1d_bwd(xraw, w, bias, state_in, silu, dout, dstate_out=None):
    """Returns (dxraw, dw, db, dstate_in)."""
    xraw, w, bias, state_in = _c(xraw), _c(w), _c(bias), _c(state_in)
    dout, dstate_out = _c(dout), _c(dstate_out)
    Bsz, L, Cd = xraw.shape
    K = w.shape[1]
    dx = np.empty((Bsz, L, Cd))
    dw = np.empty((Cd, K))
    db = np.empty((Cd,))
    dst = np.empty((Bsz, K - 1, Cd))
    lib().oracle_conv1d_bwd(_i64(Bsz), _i64(L), _i64(Cd), ctypes.c_int(K), _p(xraw),
                            _p(state_in), _p(w), _p(bias), ctypes.c_int(int(silu)), _p(dout),
                            _p(dstate_out), _p(dx), _p(dw), _p(db), _p(dst))
    return dx, dw, db, dst


# --------------------------------------------------------------------------- ssd

def _dims(x, Bm):
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    return Bsz, L, H, P, N, G


def ssd_fwd(x, dt_raw, A, Bm, Cm, dt_bias=None, softplus=True, D=None, z=None, h0=None):
    """Sequential recurrence.  Returns (out, y_pre_gate, h_final)."""
    x, dt_raw, A, Bm, Cm = _c(x), _c(dt_raw), _c(A), _c(Bm), _c(Cm)
    dt_bias, D, z, h0 = _c(dt_bias), _c(D), _c(z), _c(h0)
    Bsz, L, H, P, N, G = _dims(x, Bm)
    out = np.empty((Bsz, L, H, P))
    y = np.empty((Bsz, L, H, P))
    hf = np.empty((Bsz, H, P, N))
    lib().oracle_ssd_fwd(_i64(Bsz), _i64(L), _i64(H), _i64(P), _i64(N), _i64(G), _p(x),
                         _p(dt_raw), _p(dt_bias), ctypes.c_int(int(softplus)), _p(A), _p(Bm),
                         _p(Cm), _p(D), _p(z), _p(h0), _p(out), _p(y), _p(hf))
    return out, y, hf


def ssd_bwd(x, dt_raw, A, Bm, Cm, dout, dt_bias=None, softplus=True, D=None, z=None, h0=None,
            dh_final=None, block=4096):
    """Reverse sweep with time-blocked exact recompute (block=0: literal full storage).

    Returns a dict with dx, ddt (w.r.t. dt_raw), dB, dC, dz, dA, dD, ddt_bias, dh0."""
    x, dt_raw, A, Bm, Cm, dout = _c(x), _c(dt_raw), _c(A), _c(Bm), _c(Cm), _c(dout)
    dt_bias, D, z, h0, dh_final = _c(dt_bias), _c(D), _c(z), _c(h0), _c(dh_final)
    Bsz, L, H, P, N, G = _dims(x, Bm)
    r = dict(dx=np.empty((Bsz, L, H, P)), ddt=np.empty((Bsz, L, H)),
             dB=np.empty((Bsz, L, G, N)), dC=np.empty((Bsz, L, G, N)),
             dz=np.empty((Bsz, L, H, P)) if z is not None else None,
             dA=np.empty((H,)), dD=np.empty((H,)), ddt_bias=np.empty((H,)),
             dh0=np.empty((Bsz, H, P, N)))
    lib().oracle_ssd_bwd(_i64(Bsz), _i64(L), _i64(H), _i64(P), _i64(N), _i64(G), _p(x),
                         _p(dt_raw), _p(dt_bias), ctypes.c_int(int(softplus)), _p(A), _p(Bm),
                         _p(Cm), _p(D), _p(z), _p(h0), _p(dout), _p(dh_final), _p(r["dx"]),
                         _p(r["ddt"]), _p(r["dB"]), _p(r["dC"]), _p(r["dz"]), _p(r["dA"]),
                         _p(r["dD"]), _p(r["ddt_bias"]), _p(r["dh0"]), _i64(int(block)))
    if D is None:
        r["dD"] = None
    if dt_bias is None:
        r["ddt_bias"] = None
    return r


# --------------------------------------------------------------------------- mixer

def split_xbc(xbc, H, P, G, N):
    """[B, L, H*P + 2*G*N] -> x [B,L,H,P], B [B,L,G,N], C [B,L,G,N] (copies)."""
    Bsz, L, _ = xbc.shape
    hp, gn = H * P, G * N
    x = xbc[..., :hp].reshape(Bsz, L, H, P)
    Bm = xbc[..., hp:hp + gn].reshape(Bsz, L, G, N)
    Cm = xbc[..., hp + gn:hp + 2 * gn].reshape(Bsz, L, G, N)
    return x, Bm, Cm


def mixer_fwd(xbc_raw, conv_w, conv_b, dt_raw, A, H, P, G, N, dt_bias=None, D=None, z=None,
              h0=None, conv_state=None, softplus=True):
    """conv1d+SiLU -> SSD -> SiLU(z) gate.  Returns dict(out, y, h_final, conv_state_out, xbc)."""
    xbc, st_out = conv1d_fwd(xbc_raw, conv_w, conv_b, conv_state, silu=True)
    x, Bm, Cm = split_xbc(xbc, H, P, G, N)
    out, y, hf = ssd_fwd(x, dt_raw, A, Bm, Cm, dt_bias, softplus, D, z, h0)
    return dict(out=out, y=y, h_final=hf, conv_state_out=st_out, xbc=xbc)


def mixer_bwd(xbc_raw, conv_w, conv_b, dt_raw, A, H, P, G, N, dout, dt_bias=None, D=None, z=None,
              h0=None, conv_state=None, dh_final=None, dconv_state_out=None, softplus=True,
              block=4096):
    """Backward of mixer_fwd.  Returns the ssd_bwd dict plus dxbc_raw, dconv_w, dconv_b,
    dconv_state (w.r.t. the carried-in conv state) and dxbc (post-conv)."""
    xbc, _ = conv1d_fwd(xbc_raw, conv_w, conv_b, conv_state, silu=True)
    x, Bm, Cm = split_xbc(xbc, H, P, G, N)
    r = ssd_bwd(x, dt_raw, A, Bm, Cm, dout, dt_bias, softplus, D, z, h0, dh_final, block)
    Bsz, L = x.shape[:2]
    dxbc = np.concatenate([r["dx"].reshape(Bsz, L, H * P), r["dB"].reshape(Bsz, L, G * N),
                           r["dC"].reshape(Bsz, L, G * N)], axis=-1)
    dxr, dw, db, dst = conv1d_bwd(xbc_raw, conv_w, conv_b, conv_state, True, dxbc, dconv_state_out)
    r.update(dxbc=dxbc, dxbc_raw=dxr, dconv_w=dw, dconv_b=db, dconv_state=dst)
    return r


# --------------------------------------------------------------------------- projections, norms
#
# The mixer around the hot path (Video-Ma2mba model card, architecture diagram and
# specification table: a Mamba-2 LM with d_model 1024 in bf16; the Mamba-2 block of
# the arXiv index page's "Builds on" list):
#     zxbcdt = in_proj(u)            [z | xBC | dt_raw]
#     out    = hot path (conv1d + SiLU -> SSD -> SiLU(z) gate)
#     final  = out_proj(out)
# and the full block with its two RMSNorms and the residual:
#     final  = u + out_proj(RMSNorm(out) * g_out),   in_proj applied to RMSNorm(u) * g_in
# All in fp64 with numpy; the matrix products are numpy matmuls.

def rmsnorm(x, g, eps):
    """Root-mean-square norm over the last axis: x / sqrt(mean(x^2) + eps) * g."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def linear(x, w, norm_w=None, eps=1e-5, residual=None):
    """y = x' w^T (+ residual), w in the nn.Linear layout [out, in]; x' = x, or its
    RMSNorm times norm_w over the `in` axis when norm_w is given."""
    x = np.asarray(x, dtype=np.float64)
    if norm_w is not None:
        x = rmsnorm(x, norm_w, eps)
    y = x @ np.asarray(w, dtype=np.float64).T
    if residual is not None:
        y = y + np.asarray(residual, dtype=np.float64)
    return y


def mixer_full_fwd(u, w_in, conv_w, conv_b, A, H, P, G, N, w_out, dt_bias=None, D=None, h0=None,
                   conv_state=None, norm_in=None, norm_out=None, eps=1e-5, residual=False):
    """in_proj -> conv1d + SiLU -> SSD -> SiLU(z) gate -> out_proj over u [B, L, d_model].
    With norm_in / norm_out / residual: the full block (pre-norm, gated norm, skip).
    Returns dict(final, zxbcdt, out, h_final, conv_state_out)."""
    u = np.asarray(u, dtype=np.float64)
    Bsz, L, _ = u.shape
    hp, cd = H * P, H * P + 2 * G * N
    zx = linear(u, w_in, norm_in, eps)
    z, xbc, dt = zx[..., :hp], zx[..., hp:hp + cd], zx[..., hp + cd:hp + cd + H]
    r = mixer_fwd(xbc, conv_w, conv_b, dt, A, H, P, G, N, dt_bias=dt_bias, D=D,
                  z=z.reshape(Bsz, L, H, P), h0=h0, conv_state=conv_state)
    out = r["out"].reshape(Bsz, L, hp)
    final = linear(out, w_out, norm_out, eps, u if residual else None)
    return dict(final=final, zxbcdt=zx, out=out, h_final=r["h_final"],
                conv_state_out=r["conv_state_out"])


def rmsnorm_bwd(x, g, eps, dy):
    """Gradients of y = rmsnorm(x, g, eps) over the last axis: returns (dx, dg), dg summed
    over every leading axis.  With r = (mean(x^2) + eps)^(-1/2): y_j = g_j x_j r and
    dr/dx_k = -r^3 x_k / K, so dx_k = r g_k dy_k - (r^3 x_k / K) sum_j g_j dy_j x_j."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    K = x.shape[-1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    s = np.sum(g * dy * x, axis=-1, keepdims=True)
    dx = r * g * dy - x * (r ** 3) * s / K
    dg = np.sum((dy * x * r).reshape(-1, K), axis=0)
    return dx, dg


def block_bwd(u, w_in, conv_w, conv_b, A, H, P, G, N, w_out, dfinal, dt_bias=None, D=None,
              norm_in=None, norm_out=None, eps=1e-5, residual=True, h0=None, conv_state=None,
              dh_final=None, dconv_state_out=None):
    """Backward of mixer_full_fwd (the full block when norm_in, norm_out and residual are
    set) given dfinal = dLoss/dfinal.  Returns dict with du, dw_in, dw_out, dnorm_in,
    dnorm_out and the hot-path gradients (dconv_w, dconv_b, dA, dD, ddt_bias, dh0,
    dconv_state)."""
    u = np.asarray(u, dtype=np.float64)
    dF = np.asarray(dfinal, dtype=np.float64)
    w_in = np.asarray(w_in, dtype=np.float64)
    w_out = np.asarray(w_out, dtype=np.float64)
    Bsz, L, dm = u.shape
    hp, cd = H * P, H * P + 2 * G * N
    un = rmsnorm(u, norm_in, eps) if norm_in is not None else u
    zx = un @ w_in.T
    z, xbc, dt = zx[..., :hp], zx[..., hp:hp + cd], zx[..., hp + cd:hp + cd + H]
    f = mixer_fwd(xbc, conv_w, conv_b, dt, A, H, P, G, N, dt_bias=dt_bias, D=D,
                  z=z.reshape(Bsz, L, H, P), h0=h0, conv_state=conv_state)
    out = f["out"].reshape(Bsz, L, hp)
    on = rmsnorm(out, norm_out, eps) if norm_out is not None else out
    # out_proj
    d_on = dF @ w_out
    dw_out = dF.reshape(-1, dm).T @ on.reshape(-1, hp)
    if norm_out is not None:
        d_out, dnorm_out = rmsnorm_bwd(out, norm_out, eps, d_on)
    else:
        d_out, dnorm_out = d_on, None
    # hot path
    r = mixer_bwd(xbc, conv_w, conv_b, dt, A, H, P, G, N, d_out.reshape(Bsz, L, H, P),
                  dt_bias=dt_bias, D=D, z=z.reshape(Bsz, L, H, P), h0=h0, conv_state=conv_state,
                  dh_final=dh_final, dconv_state_out=dconv_state_out)
    dzx = np.concatenate([r["dz"].reshape(Bsz, L, hp), r["dxbc_raw"], r["ddt"]], axis=-1)
    # in_proj
    d_un = dzx @ w_in
    dw_in = dzx.reshape(-1, zx.shape[-1]).T @ un.reshape(-1, dm)
    if norm_in is not None:
        du, dnorm_in = rmsnorm_bwd(u, norm_in, eps, d_un)
    else:
        du, dnorm_in = d_un, None
    if residual:
        du = du + dF
    return dict(du=du, dw_in=dw_in, dw_out=dw_out, dnorm_in=dnorm_in, dnorm_out=dnorm_out,
                dconv_w=r["dconv_w"], dconv_b=r["dconv_b"], dA=r["dA"], dD=r["dD"],
                ddt_bias=r["ddt_bias"], dh0=r["dh0"], dconv_state=r["dconv_state"], dzx=dzx)


def stack_fwd_bwd(u, layers, H, P, G, N, dfinal, eps=1e-5):
    """A stack of full blocks (each layer a dict of w_in, conv_w, conv_b, A, w_out,
    dt_bias, D, norm_in, norm_out) over u [B, L, d_model], all states starting at zero:
    the forward through the layers, then the backward layer by layer from the top with
    block_bwd.  Returns (final, du, [per-layer gradient dicts])."""
    xs = [np.asarray(u, dtype=np.float64)]
    for p in layers:
        xs.append(mixer_full_fwd(xs[-1], p["w_in"], p["conv_w"], p["conv_b"], p["A"], H, P, G, N, p["w_out"],
                                 dt_bias=p["dt_bias"], D=p["D"], norm_in=p["norm_in"], norm_out=p["norm_out"],
                                 eps=eps, residual=True)["final"])
    g = np.asarray(dfinal, dtype=np.float64)
    grads = [None] * len(layers)
    for i in reversed(range(len(layers))):
        p = layers[i]
        r = block_bwd(xs[i], p["w_in"], p["conv_w"], p["conv_b"], p["A"], H, P, G, N, p["w_out"], g,
                      dt_bias=p["dt_bias"], D=p["D"], norm_in=p["norm_in"], norm_out=p["norm_out"], eps=eps,
                      residual=True)
        grads[i] = r
        g = r["du"]
    return xs[-1], g, grads
