"""The full Mamba-2 block over the C ABI, forward and backward.

    final = u + out_proj(RMSNorm(out) * g_out),   out = hot path(in_proj(RMSNorm(u) * g_in))

(the block of the Video-Ma2mba model card's architecture diagram: a Mamba-2 LM of such
blocks; the gated norm acts on ssd_fwd's SiLU(z)-gated output).  The hot path is
conv1d + SiLU -> SSD -> SiLU(z) gate (ssd_fwd / ssd_bwd), the projections are
mixer_proj / mixer_proj_bwd, the norms rmsnorm_fwd / rmsnorm_bwd.  Every call carries
the (h, conv buffer) state in and out, so a block can be run on any token range of a
longer sequence -- the cells of multi-axis gradient checkpointing (magc.py).

This module sequences library calls and slices views; every arithmetic step runs in
the HIP kernels behind the calls.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as bd

EPS = 1e-5

# A projection whose plain form (no norm prologue) runs on mixer_proj's 256 x 256 MFMA
# blocks -- at least 1,024 of them, both dimensions >= 256, K a multiple of 64 -- is
# faster as a norm pass of its own followed by the plain product than with the norm
# folded into the product (whose registers only fit the 128 x 128 blocks).
BIG_BLOCKS = 1024


def _big_blocks(M: int, N: int, K: int) -> bool:
    return M >= 256 and N >= 256 and K % 64 == 0 and -(-M // 256) * -(-N // 256) >= BIG_BLOCKS


def _overlap(a: torch.Tensor, b: torch.Tensor) -> bool:
    a0, b0 = a.data_ptr(), b.data_ptr()
    return a0 < b0 + b.numel() * b.element_size() and b0 < a0 + a.numel() * a.element_size()


@dataclass
class Shape:
    d_model: int
    H: int
    P: int
    N: int
    G: int = 1
    K: int = 4

    @property
    def hp(self):
        return self.H * self.P

    @property
    def cd(self):
        return self.H * self.P + 2 * self.G * self.N

    @property
    def dip(self):
        return 2 * self.H * self.P + 2 * self.G * self.N + self.H


@dataclass
class Weights:
    """One block's parameters on the device: w_in [dip, d_model], w_out [d_model, H*P]
    (bf16, nn.Linear layout), norm_in [d_model], norm_out [H*P], conv_w [Cd, K],
    conv_b [Cd], A, D, dt_bias [H] (fp32)."""
    w_in: torch.Tensor
    w_out: torch.Tensor
    norm_in: torch.Tensor
    norm_out: torch.Tensor
    conv_w: torch.Tensor
    conv_b: torch.Tensor
    A: torch.Tensor
    D: torch.Tensor
    dt_bias: torch.Tensor


GRAD_NAMES = ("w_in", "w_out", "norm_in", "norm_out", "conv_w", "conv_b", "A", "D", "dt_bias")


def zero_grads(w: Weights) -> dict:
    """fp32 gradient buffers shaped like the parameters."""
    return {k: torch.zeros(getattr(w, k).shape, dtype=torch.float32, device=getattr(w, k).device)
            for k in GRAD_NAMES}


class Scratch:
    """Device workspaces for blocks of shape `sh` over up to `T` tokens per call (batch B)."""

    def __init__(self, sh: Shape, B: int, T: int, device):
        self.sh, self.B, self.T = sh, B, T
        dims = bd.make_dims(B, T, sh.H, sh.P, sh.N, sh.G, 0, sh.K)
        by = lambda n: torch.empty(max(n, 1), dtype=torch.uint8, device=device)
        self.fws = by(bd.ssd_fwd_workspace(dims, bd.SSD_BF16))
        self.bws = by(bd.ssd_bwd_workspace(dims, bd.SSD_BF16))
        self.nws = by(max(bd.rmsnorm_bwd_workspace(sh.d_model), bd.rmsnorm_bwd_workspace(sh.hp)))
        e = lambda c: torch.empty(B * T, c, dtype=torch.bfloat16, device=device)
        self.un, self.zx, self.out, self.on = e(sh.d_model), e(sh.dip), e(sh.hp), e(sh.hp)
        self.d_on, self.d_out, self.dzx, self.d_un = e(sh.hp), e(sh.hp), e(sh.dip), e(sh.d_model)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("block activations must be contiguous [B, L, C] tensors")


def _dims(sh: Shape, B: int, L: int):
    return bd.make_dims(B, L, sh.H, sh.P, sh.N, sh.G, 0, sh.K)


def _hot_views(sh: Shape, zx: torch.Tensor, B: int, L: int):
    z3 = zx[:B * L].view(B, L, sh.dip)
    hp, cd = sh.hp, sh.cd
    return z3[..., :hp], z3[..., hp:hp + cd], z3[..., hp + cd:hp + cd + sh.H]


def block_fwd(sh: Shape, w: Weights, u: torch.Tensor, final: torch.Tensor, sc: Scratch, *, h0=None,
              conv_state=None, h_final=None, conv_state_out=None, eps=EPS):
    """final [B, L, d_model] = block(u [B, L, d_model]); the norm before in_proj is fused
    into the projection's operand load, the gated norm and the residual into out_proj --
    or, for projections large enough for the big MFMA blocks, each norm is a pass of its
    own: u's into final's buffer (unused until out_proj writes it; final must then not
    overlap u), the output's in place in the scratch."""
    B, L, dm = u.shape
    _contig(u, final)
    n = B * L
    if n > sc.B * sc.T:
        raise ValueError(f"{n} tokens exceed the scratch of {sc.B * sc.T}")
    zx = sc.zx[:n]
    u2, f2 = u.reshape(n, dm), final.reshape(n, dm)
    if _big_blocks(n, sh.dip, dm) and not _overlap(u, final):
        bd.rmsnorm_fwd(u2, w.norm_in, f2, eps=eps)
        bd.mixer_proj(f2, w.w_in, zx)
    else:
        bd.mixer_proj(u2, w.w_in, zx, norm_w=w.norm_in, norm_eps=eps)
    z, xbc, dt = _hot_views(sh, zx, B, L)
    out = sc.out[:n].view(B, L, sh.hp)
    bd.ssd_fwd(_dims(sh, B, L), xbc, w.A, dt, out, conv_w=w.conv_w, conv_b=w.conv_b, conv_state_in=conv_state,
               conv_state_out=conv_state_out, dt_bias=w.dt_bias, D=w.D, z=z, h0=h0, h_final=h_final, ws=sc.fws)
    o2 = out.view(n, sh.hp)
    if _big_blocks(n, dm, sh.hp):
        bd.rmsnorm_fwd(o2, w.norm_out, o2, eps=eps)
        bd.mixer_proj(o2, w.w_out, f2, residual=u2)
    else:
        bd.mixer_proj(o2, w.w_out, f2, norm_w=w.norm_out, norm_eps=eps, residual=u2)


def block_bwd(sh: Shape, w: Weights, u: torch.Tensor, dfinal: torch.Tensor, du: torch.Tensor, grads: dict,
              sc: Scratch, *, h0=None, conv_state=None, dh_final=None, dconv_state_out=None, dh0=None,
              dconv_state_in=None, accumulate=True, eps=EPS):
    """Gradients of block_fwd over u [B, L, d_model] given dfinal: du (may be dfinal
    itself), parameter gradients added into `grads` (overwritten when accumulate is
    False), dh0 / dconv_state_in of the carried states.  Recomputes the block's forward
    from (u, h0, conv_state)."""
    B, L, dm = u.shape
    _contig(u, dfinal, du)
    n = B * L
    if n > sc.B * sc.T:
        raise ValueError(f"{n} tokens exceed the scratch of {sc.B * sc.T}")
    hp = sh.hp
    u2, dF = u.reshape(n, dm), dfinal.reshape(n, dm)
    # recompute: the normalised input, the in_proj rows, the hot-path output, its norm
    un, zx = sc.un[:n], sc.zx[:n]
    bd.rmsnorm_fwd(u2, w.norm_in, un, eps=eps)
    bd.mixer_proj(un, w.w_in, zx)
    z, xbc, dt = _hot_views(sh, zx, B, L)
    out = sc.out[:n]
    dims = _dims(sh, B, L)
    bd.ssd_fwd(dims, xbc, w.A, dt, out.view(B, L, hp), conv_w=w.conv_w, conv_b=w.conv_b,
               conv_state_in=conv_state, dt_bias=w.dt_bias, D=w.D, z=z, h0=h0, ws=sc.fws)
    on = sc.on[:n]
    bd.rmsnorm_fwd(out, w.norm_out, on, eps=eps)
    # out_proj and the gated norm
    d_on, d_out = sc.d_on[:n], sc.d_out[:n]
    bd.mixer_proj_bwd(dF, x=on, w=w.w_out, dx=d_on, dw=grads["w_out"], accumulate=accumulate)
    bd.rmsnorm_bwd(out, w.norm_out, d_on, d_out, eps=eps, dg=grads["norm_out"], accumulate=accumulate,
                   ws=sc.nws)
    # hot path: its three input gradients land in one in_proj-row array [dz | dxBC | ddt]
    dzx = sc.dzx[:n]
    dz, dxbc, ddt = _hot_views(sh, dzx, B, L)
    bd.ssd_bwd(dims, xbc, w.A, dt, d_out.view(B, L, hp), dxbc, ddt, grads["A"], conv_w=w.conv_w,
               conv_b=w.conv_b, conv_state_in=conv_state, dt_bias=w.dt_bias, D=w.D, z=z, h0=h0,
               dh_final=dh_final, dconv_state_out=dconv_state_out, dz=dz, dD=grads["D"],
               ddt_bias=grads["dt_bias"], dconv_w=grads["conv_w"], dconv_b=grads["conv_b"], dh0=dh0,
               dconv_state_in=dconv_state_in, accumulate=accumulate, ws=sc.bws)
    # in_proj, the norm before it, and the residual
    d_un = sc.d_un[:n]
    bd.mixer_proj_bwd(dzx, x=un, w=w.w_in, dx=d_un, dw=grads["w_in"], accumulate=accumulate)
    bd.rmsnorm_bwd(u2, w.norm_in, d_un, du.reshape(n, dm), eps=eps, dres=dF, dg=grads["norm_in"],
                   accumulate=accumulate, ws=sc.nws)
