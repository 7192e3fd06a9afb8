"""Multi-axis gradient checkpointing (MA-GC) of a stack of Mamba-2 blocks over one long
sequence, on the C ABI.

The pith.science review of Video-Ma2mba (arXiv 2411.19460; "key machinery") describes
the scheme: layer-wise checkpoints keep the input of every l-th layer, sequence-wise
checkpoints keep the recurrent state every s tokens, and the grid cells they bound
(l layers x s tokens) are recomputed forward and backpropagated through in the backward
pass.  The same review's skeptic critique points out that a causal conv precedes the
SSD, so a sequence checkpoint is the pair (h, the last K-1 conv inputs); both are kept
here, which makes the recompute exact.

Activation memory, in per-token-per-layer units, is M = L S / l + L S / s + l s (L
layers, S tokens), minimised at l = s = (L S)^(1/3) (same review, "key machinery").
Here the three terms have different sizes: a layer checkpoint is d_model bf16 values
per token, a sequence checkpoint is one fp32 state (H P N values) plus K-1 conv rows
per layer and segment, and a cell holds l layer inputs of s tokens plus one block's
working set of s tokens.  `model_bytes` evaluates the memory with those sizes.

stack_forward keeps the checkpoints; stack_backward walks the cells from the last
layer group and the last segment backwards:
  * recompute the cell: from the group's layer checkpoint (the segment's rows) and each
    layer's (h, conv) checkpoint at the segment start, run the group's layers forward
    over the segment, keeping each layer's input rows;
  * backpropagate through the cell, top layer first: block_bwd of each layer on the
    segment, given the gradient at its output rows and the (dh, dconv) carried in from
    the next segment of the same layer; it yields the gradient at its input rows and the
    (dh, dconv) to carry into the previous segment.
Parameter gradients accumulate over cells.  This module sequences library calls only.
"""
from __future__ import annotations

import torch

from . import binding as bd
from . import block


def model_bytes(sh: block.Shape, n_layers: int, S: int, l: int, s: int) -> dict:
    """Activation memory of MA-GC by term (bytes), batch 1, bf16 activations: the layer
    checkpoints (L S / l rows), the sequence checkpoints (L S / s states), the cell (l s
    rows plus one block's working set and workspaces over s tokens) and the sequence-long
    buffers every scheme holds (the running activation and two gradient rows)."""
    dm = sh.d_model
    state = sh.H * sh.P * sh.N * 4 + (sh.K - 1) * sh.cd * 2
    dims = bd.make_dims(1, s, sh.H, sh.P, sh.N, sh.G, 0, sh.K)
    work = s * 2 * (2 * dm + 2 * sh.dip + 4 * sh.hp)          # block.Scratch rows
    ws = (bd.ssd_fwd_workspace(dims, bd.SSD_BF16) + bd.ssd_bwd_workspace(dims, bd.SSD_BF16) +
          max(bd.rmsnorm_bwd_workspace(dm), bd.rmsnorm_bwd_workspace(sh.hp)))
    return {"layer_ckpt": ((n_layers + l - 1) // l) * S * dm * 2,
            "seq_ckpt": n_layers * ((S + s - 1) // s) * state,
            "cell": l * s * dm * 2 + work + ws,
            "sequence_buffers": 3 * S * dm * 2}


def best_intervals(sh: block.Shape, n_layers: int, S: int, ls=None, ss=None):
    """(l, s) minimising model_bytes over the given candidate intervals (defaults: the
    divisors-like powers of two up to L and S)."""
    ls = ls or [l for l in range(1, n_layers + 1) if n_layers % l == 0]
    ss = ss or [1 << k for k in range(6, S.bit_length()) if (1 << k) <= S]
    best = min(((sum(model_bytes(sh, n_layers, S, l, s).values()), l, s) for l in ls for s in ss))
    return best[1], best[2]


class Checkpoints:
    def __init__(self):
        self.layer = {}   # layer index -> [1, S, d_model] input of that layer
        self.h = []       # [layer][segment] -> fp32 state at the segment start
        self.conv = []    # [layer][segment] -> conv rows at the segment start


def _segments(S: int, s: int):
    return [(t0, min(S, t0 + s)) for t0 in range(0, S, s)]


def stack_forward(sh: block.Shape, layers, u: torch.Tensor, sc: block.Scratch, l: int, s: int):
    """Forward of the stack over u [1, S, d_model]; returns (final, Checkpoints)."""
    B, S, dm = u.shape
    if B != 1:
        raise ValueError("the stack runs one sequence (batch 1)")
    dev = u.device
    ck = Checkpoints()
    x = u
    segs = _segments(S, s)
    for i, w in enumerate(layers):
        if i % l == 0:
            ck.layer[i] = x
        y = torch.empty_like(x)
        hs, cs = [], []
        h = torch.zeros(1, sh.H, sh.P, sh.N, device=dev)
        c = torch.zeros(1, sh.K - 1, sh.cd, dtype=torch.bfloat16, device=dev)
        for t0, t1 in segs:
            hs.append(h)
            cs.append(c)
            h_next = torch.empty_like(h)
            c_next = torch.empty_like(c)
            block.block_fwd(sh, w, x[:, t0:t1], y[:, t0:t1], sc, h0=h, conv_state=c, h_final=h_next,
                            conv_state_out=c_next)
            h, c = h_next, c_next
        ck.h.append(hs)
        ck.conv.append(cs)
        x = y
    return x, ck


def stack_backward(sh: block.Shape, layers, ck: Checkpoints, dfinal: torch.Tensor, grads, sc: block.Scratch,
                   l: int, s: int) -> torch.Tensor:
    """Gradient of the stack's input given dfinal [1, S, d_model]; parameter gradients are
    added into grads[i] (dicts from block.zero_grads)."""
    n_layers = len(layers)
    _, S, dm = dfinal.shape
    dev = dfinal.device
    segs = _segments(S, s)
    dX = dfinal
    top = n_layers
    for g0 in reversed(range(0, n_layers, l)):
        group = list(range(g0, min(g0 + l, top)))
        dX_below = torch.empty_like(dX)
        dh = {i: torch.zeros(1, sh.H, sh.P, sh.N, device=dev) for i in group}
        dc = {i: torch.zeros(1, sh.K - 1, sh.cd, dtype=torch.bfloat16, device=dev) for i in group}
        for k in reversed(range(len(segs))):
            t0, t1 = segs[k]
            # recompute the cell: each layer's input rows of this segment
            xs = {group[0]: ck.layer[g0][:, t0:t1]}
            for i in group[:-1]:
                xn = torch.empty(1, t1 - t0, dm, dtype=torch.bfloat16, device=dev)
                block.block_fwd(sh, layers[i], xs[i], xn, sc, h0=ck.h[i][k], conv_state=ck.conv[i][k])
                xs[i + 1] = xn
            # backpropagate through the cell, top layer first; the bottom layer writes its
            # input gradient straight into the rows of the group below
            g = dX[:, t0:t1]
            for i in reversed(group):
                dh_in = torch.empty_like(dh[i])
                dc_in = torch.empty_like(dc[i])
                gi = dX_below[:, t0:t1] if i == group[0] else torch.empty_like(g)
                block.block_bwd(sh, layers[i], xs[i], g, gi, grads[i], sc, h0=ck.h[i][k],
                                conv_state=ck.conv[i][k], dh_final=dh[i], dconv_state_out=dc[i], dh0=dh_in,
                                dconv_state_in=dc_in, accumulate=True)
                dh[i], dc[i] = dh_in, dc_in
                g = gi
            del xs
        dX = dX_below
        top = g0
    return dX
