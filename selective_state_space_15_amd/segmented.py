"""Sequence-axis gradient checkpointing driver over the C ABI.

The multi-axis gradient checkpointing of Video-Ma2mba (pith.science review of arXiv
2411.19460, "key machinery") stores the recurrent state every s steps and rebuilds
each s-step cell in the backward pass.  Because a causal Conv1d precedes the SSD
(the same review's skeptic critique), an exact checkpoint is the pair
(h_s, the last K-1 conv inputs); both are carried here.

forward_segmented: one ssd_fwd call over the whole sequence that also writes the
    state at every segment start (h_ckpt); the conv-buffer checkpoint of segment k
    is a view of the K-1 raw rows before it, so nothing is copied.
backward_segmented: segments in reverse order, each one ssd_bwd call that
    recomputes its forward from (h_ckpt[k], conv rows) and receives the gradients
    of its end state (dh, dconv) from the segment after it; parameter gradients
    are accumulated across segments by the library (accumulate = 1).

This module only sequences library calls and slices views; every arithmetic step
runs in the HIP kernels behind the calls.
"""
from __future__ import annotations

import torch

from . import binding as bd


def _io(t: torch.Tensor) -> int:
    return bd.io_dtype(t)


def forward_segmented(dims: bd.ssd_dims, seg: int, xbc, A, dt, out, *, conv_w=None, conv_b=None,
                      conv_state_in=None, dt_bias=None, D=None, z=None, h0=None, h_final=None,
                      ws=None, stream=None):
    """Run the forward once and return h_ckpt [nseg, B, H, P, N] (entry k = state
    before token k*seg).  `seg` must be a positive multiple of 64."""
    L = dims.seqlen
    nseg = (L + seg - 1) // seg
    h_ckpt = torch.empty(nseg, dims.batch, dims.nheads, dims.headdim, dims.dstate,
                         dtype=torch.float32, device=xbc.device)
    bd.ssd_fwd(dims, xbc, A, dt, out, conv_w=conv_w, conv_b=conv_b, conv_state_in=conv_state_in,
               dt_bias=dt_bias, D=D, z=z, h0=h0, h_final=h_final, h_ckpt=h_ckpt, ckpt_every=seg,
               ws=ws, stream=stream)
    return h_ckpt


def conv_ckpt(xbc, conv_state_in, t0: int, K: int):
    """Conv-buffer checkpoint of the segment starting at token t0: the K-1 raw rows
    before it, as a view (rows from conv_state_in when t0 < K-1 need a join)."""
    if K <= 1:
        return None
    if t0 >= K - 1:
        return xbc[:, t0 - (K - 1):t0]
    if t0 == 0:
        return conv_state_in
    # a segment shorter than the conv buffer: join carried rows and new rows
    prev = conv_state_in if conv_state_in is not None else torch.zeros(
        xbc.shape[0], K - 1, xbc.shape[2], dtype=xbc.dtype, device=xbc.device)
    return torch.cat([prev[:, t0:], xbc[:, :t0]], dim=1).contiguous()


def backward_segmented(dims: bd.ssd_dims, seg: int, h_ckpt, xbc, A, dt, dout, dxbc, ddt, dA, *,
                       conv_w=None, conv_b=None, conv_state_in=None, dt_bias=None, D=None, z=None,
                       dz=None, dD=None, ddt_bias=None, dconv_w=None, dconv_b=None, dh_final=None,
                       dconv_state_out=None, dh0=None, dconv_state_in=None, ws=None, stream=None):
    """Reverse sweep over segments.  Parameter gradients are overwritten (the first
    call of the sweep overwrites, the others accumulate).  Returns nothing; dh0 and
    dconv_state_in (if given) receive the gradients of the initial states."""
    L, B, H, P, N, K = dims.seqlen, dims.batch, dims.nheads, dims.headdim, dims.dstate, dims.conv_width
    nseg = (L + seg - 1) // seg
    dev = xbc.device
    dh = dh_final
    dcs = dconv_state_out
    dh_buf = [torch.empty(B, H, P, N, dtype=torch.float32, device=dev) for _ in range(2)]
    cd = xbc.shape[2]
    dcs_buf = [torch.empty(B, max(K - 1, 1), cd, dtype=xbc.dtype, device=dev) for _ in range(2)] if K > 1 else None
    for i, k in enumerate(reversed(range(nseg))):
        t0, t1 = k * seg, min(L, (k + 1) * seg)
        d = bd.make_dims(B, t1 - t0, H, P, N, dims.ngroups, dims.chunk, K)
        last = k == 0
        dh_out = dh0 if last else dh_buf[i % 2]
        dcs_out = (dconv_state_in if last else dcs_buf[i % 2]) if K > 1 else None
        bd.ssd_bwd(d, xbc[:, t0:t1], A, dt[:, t0:t1], dout[:, t0:t1], dxbc[:, t0:t1], ddt[:, t0:t1], dA,
                   conv_w=conv_w, conv_b=conv_b, conv_state_in=conv_ckpt(xbc, conv_state_in, t0, K),
                   dt_bias=dt_bias, D=D, z=None if z is None else z[:, t0:t1],
                   h0=h_ckpt[k], dh_final=dh, dconv_state_out=dcs,
                   dz=None if dz is None else dz[:, t0:t1], dD=dD, ddt_bias=ddt_bias,
                   dconv_w=dconv_w, dconv_b=dconv_b, dh0=dh_out, dconv_state_in=dcs_out,
                   accumulate=i > 0, ws=ws, stream=stream)
        dh, dcs = dh_out, dcs_out
