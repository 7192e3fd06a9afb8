"""The segmented training step captured once in a HIP graph and replayed.

The step is the one bench.py times: one ssd_fwd over the whole sequence that keeps the
(h) state every `seg` tokens, then ssd_bwd segment by segment in reverse, carrying
(dh, dconv) between segments.  Every library call enqueues its kernels on the stream it
is given and allocates, copies and clears nothing (its scratch is the caller's
workspace), so the whole step -- 1 + nseg calls and the driver's small carry buffers --
is captured by torch.cuda.CUDAGraph and replayed with no host work between kernels.

Each replay starts from new inputs (in_proj rows, upstream gradient, carried states)
written into the captured buffers by eager copies, and must equal the same step run
eagerly on those inputs, bitwise: the same kernels in the same order, and no atomics.
"""
import pytest
import torch

from selective_state_space_15_amd import binding as bd
from selective_state_space_15_amd import segmented, synth
from tests.gpu_cases import Case, _bwd_outputs, _dout, fdev, to_dev

pytestmark = pytest.mark.gpu

SEG = 1024


def _inputs(d, seed):
    """Device inputs of one replay: in_proj rows, dout and the four carried states."""
    c = Case(d, seed=seed, states=True)
    zx = c.dev_inputs()[0]
    st = c.st
    return dict(zx=zx, dout=to_dev(_dout(c, 0, d.L), d.dtype), h0=fdev(st["h0"]),
                cs_in=to_dev(st["conv_state"], d.dtype), dh_final=fdev(st["dh_final"]),
                dcs_out=to_dev(st["dconv_state"], d.dtype))


def _step(d, buf, p, fws, bws, o):
    """Forward with checkpoints, then the reverse segment sweep; returns h_ckpt."""
    hp, cd, H = d.hp, d.cd, d.H
    zx = buf["zx"]
    z, xbc, dt = zx[..., :hp], zx[..., hp:hp + cd], zx[..., hp + cd:hp + cd + H]
    dims = bd.make_dims(d.B, d.L, H, d.P, d.N, d.G, 0, d.K)
    h_ckpt = segmented.forward_segmented(dims, SEG, xbc, p["A"], dt, o["out"], conv_w=p["conv_w"],
                                         conv_b=p["conv_b"], conv_state_in=buf["cs_in"],
                                         dt_bias=p["dt_bias"], D=p["D"], z=z, h0=buf["h0"],
                                         h_final=o["h_final"], ws=fws)
    segmented.backward_segmented(dims, SEG, h_ckpt, xbc, p["A"], dt, buf["dout"], o["dxbc"], o["ddt"],
                                 o["dA"], conv_w=p["conv_w"], conv_b=p["conv_b"],
                                 conv_state_in=buf["cs_in"], dt_bias=p["dt_bias"], D=p["D"], z=z,
                                 dz=o["dz"], dD=o["dD"], ddt_bias=o["ddt_bias"], dconv_w=o["dconv_w"],
                                 dconv_b=o["dconv_b"], dh_final=buf["dh_final"],
                                 dconv_state_out=buf["dcs_out"], dh0=o["dh0"],
                                 dconv_state_in=o["dconv_state"], ws=bws)
    return h_ckpt


def _outputs(d):
    o = _bwd_outputs(d, d.L, torch.bfloat16)
    o["out"] = torch.empty(d.B, d.L, d.hp, dtype=torch.bfloat16, device="cuda")
    o["h_final"] = torch.empty(d.B, d.H, d.P, d.N, device="cuda")
    return o


@pytest.mark.parametrize("name", ["c1", "c4"])
def test_segmented_step_replayed_from_a_hip_graph(name):
    # d_model 1024 shapes over 5 segments (the last one ragged); and the 80-head shapes
    # at batch 2 over 3 segments
    d = (synth.CONFIGS["c1"].with_(L=4 * SEG + 333) if name == "c1"
         else synth.CONFIGS["c4"].with_(B=2, L=2 * SEG + 100))
    print(f"[graph] {name} B={d.B} L={d.L} H={d.H} seg={SEG}", flush=True)
    p = {k: fdev(v) for k, v in Case(d, seed=900).p.items()}
    dims = bd.make_dims(d.B, d.L, d.H, d.P, d.N, d.G, 0, d.K)
    fws = torch.empty(bd.ssd_fwd_workspace(dims, bd.SSD_BF16), dtype=torch.uint8, device="cuda")
    seg_dims = bd.make_dims(d.B, SEG, d.H, d.P, d.N, d.G, 0, d.K)
    bws = torch.empty(bd.ssd_bwd_workspace(seg_dims, bd.SSD_BF16), dtype=torch.uint8, device="cuda")

    buf = _inputs(d, 901)
    o = _outputs(d)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(d, buf, p, fws, bws, o)  # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        h_ckpt = _step(d, buf, p, fws, bws, o)

    for r in range(3):
        new = _inputs(d, 910 + r)
        for k, v in new.items():
            buf[k].copy_(v)
        graph.replay()
        torch.cuda.synchronize()
        # the same step, eagerly, on the same inputs (own outputs and workspaces)
        oe = _outputs(d)
        fe, be = torch.empty_like(fws), torch.empty_like(bws)
        he = _step(d, new, p, fe, be, oe)
        torch.cuda.synchronize()
        diff = [k for k in oe if oe[k] is not None and not torch.equal(o[k], oe[k])]
        if not torch.equal(h_ckpt, he):
            diff.append("h_ckpt")
        print(f"[graph] {name} replay {r}: outputs differing from the eager step: {diff or 'none'}",
              flush=True)
        assert not diff, (r, diff)
        assert torch.isfinite(o["out"].float()).all() and torch.isfinite(o["dxbc"].float()).all()
