"""GPU parity of the streaming decode (ssd_decode) against the fp64 oracle.

A stream of tokens is fed to ssd_decode one token per call (and in mixed multi-token
calls), carrying (h, conv buffer) from call to call; the concatenated outputs, the
final state and the final conv buffer must match the oracle's forward over the whole
stream from the same initial state.  The oracle's forward is the recurrence itself,
so this is the split-with-carried-state property at one-token splits, on the GPU.
Bar: relative L2 <= 1e-2 (bf16) / 1e-4 (fp32); the conv buffer (a copy of raw rows)
bitwise.
"""
import numpy as np
import pytest
import torch

from selective_state_space_15_amd import binding as bd
from selective_state_space_15_amd import synth
from tests.gpu_cases import TOL, Case, check_chunks, fdev, rel_l2, to_dev, to_host

pytestmark = pytest.mark.gpu


def decode_stream(case, splits):
    """Run the case's tokens through ssd_decode in calls of the given lengths."""
    d = case.d
    io = torch.bfloat16 if d.dtype == "bf16" else torch.float32
    zx, z, xbc, dt = case.dev_inputs()
    p = {k: fdev(v) for k, v in case.p.items()}
    st = case.st
    h = fdev(st["h0"]).clone() if "h0" in st else torch.zeros(d.B, d.H, d.P, d.N, device="cuda")
    K = d.K
    cs = [to_dev(st["conv_state"], d.dtype) if "conv_state" in st else
          torch.zeros(d.B, max(K - 1, 1), d.cd, dtype=io, device="cuda"),
          torch.empty(d.B, max(K - 1, 1), d.cd, dtype=io, device="cuda")]
    out = torch.empty(d.B, d.L, d.hp, dtype=io, device="cuda")
    t0, i = 0, 0
    for n in splits:
        t1 = t0 + n
        dims = bd.make_dims(d.B, n, d.H, d.P, d.N, d.G, 0, K)
        sl = slice(t0, t1)
        bd.ssd_decode(dims, xbc[:, sl], p["A"], dt[:, sl], out[:, sl], h,
                      conv_w=p.get("conv_w") if K else None, conv_b=p.get("conv_b") if K else None,
                      conv_state_in=cs[i % 2] if K > 1 else None,
                      conv_state_out=cs[(i + 1) % 2] if K > 1 else None,
                      dt_bias=p["dt_bias"], D=p["D"], z=z[:, sl] if z is not None else None, h_in=h)
        t0, i = t1, i + 1
    assert t0 == d.L
    torch.cuda.synchronize()
    return dict(out=out, h_final=h, conv_state_out=cs[i % 2] if K > 1 else None)


def check_decode(case, splits):
    d = case.d
    g = decode_stream(case, splits)
    st = case.st
    r = case.oracle_fwd(h0=st["h0"].astype(np.float64) if "h0" in st else None,
                        conv_state=st["conv_state"].astype(np.float64) if "conv_state" in st else None)
    tol = TOL[d.dtype]
    e_out = rel_l2(to_host(g["out"]), r["out"])
    e_h = rel_l2(to_host(g["h_final"]), r["h_final"])
    print(f"[decode] {d} calls={len(splits)} out={e_out:.2e} h_final={e_h:.2e}", flush=True)
    assert e_out <= tol and e_h <= tol, (e_out, e_h)
    check_chunks("out", to_host(g["out"]), r["out"], tol, "decode")
    if d.K > 1:
        assert np.array_equal(to_host(g["conv_state_out"]), r["conv_state_out"])


def test_decode_c1_shapes_one_token_per_call():
    """d_model 1024 shapes (32 heads x 64, d_state 128, conv 4), batch 2, from carried
    (h, conv) states, 300 tokens, one call per token."""
    d = synth.CONFIGS["c1"].with_(B=2, L=300)
    check_decode(Case(d, seed=80, states=True), [1] * 300)


def test_decode_mixed_call_lengths():
    """Calls of 1, 2 (shorter than the conv buffer), 77 and single tokens mixed."""
    d = synth.CONFIGS["c1"].with_(L=200)
    splits = [1, 2, 77, 1, 1, 3, 100, 15]
    check_decode(Case(d, seed=81, states=True), splits)


@pytest.mark.parametrize("P,N,G", [(32, 16, 2), (64, 64, 1), (32, 128, 1)])
def test_decode_other_shapes(P, N, G):
    d = synth.Dims(B=2, L=130, H=4, P=P, N=N, G=G, K=4, d_model=256)
    check_decode(Case(d, seed=82, states=True), [1] * 64 + [66])


def test_decode_whole_head_workgroups_p32():
    """512 (batch, head) pairs take one workgroup per head (16 P threads); here with
    P = 32, N = 64 and two groups, one token per call and a multi-token call."""
    d = synth.Dims(B=8, L=12, H=64, P=32, N=64, G=2, K=4, d_model=1024)
    check_decode(Case(d, seed=87, states=True), [1] * 8 + [4])


def test_decode_fp32_no_conv_no_gate():
    """The fp32 single-scan configuration (4 heads x 32, d_state 16, no conv, no gate)."""
    d = synth.CONFIGS["c0"].with_(L=96)
    check_decode(Case(d, seed=83), [1] * 96)


def test_decode_c4_shapes_batch16():
    """d_model 2560 shapes (80 heads), batch 16, 40 tokens one at a time."""
    d = synth.CONFIGS["c4"].with_(L=40)
    check_decode(Case(d, seed=84, states=True), [1] * 40)


@pytest.mark.parametrize("name", ["c1", "c4"])
def test_decode_steps_replayed_from_a_hip_graph(name):
    """A serving loop's form of decode: one-token ssd_decode calls captured once in a HIP
    graph (torch.cuda.CUDAGraph; the library launches on the stream it is given), then
    replayed from three different carried states, each written into the captured
    buffers by eager copies between replays.  Every replay must equal the same calls
    made eagerly from that state, bitwise: the same kernels on the same inputs.  c4
    (batch 16, 80 heads) takes the resident-workgroup kernel."""
    d = synth.CONFIGS["c1"].with_(B=2, L=16) if name == "c1" else synth.CONFIGS["c4"].with_(L=6)
    case = Case(d, seed=85, states=True)
    _, z, xbc, dt = case.dev_inputs()
    p = {k: fdev(v) for k, v in case.p.items()}
    dims = bd.make_dims(d.B, 1, d.H, d.P, d.N, d.G, 0, d.K)

    def steps(h, cs, out):
        for t in range(d.L):
            sl = slice(t, t + 1)
            bd.ssd_decode(dims, xbc[:, sl], p["A"], dt[:, sl], out[:, sl], h, conv_w=p["conv_w"],
                          conv_b=p["conv_b"], conv_state_in=cs[t % 2], conv_state_out=cs[(t + 1) % 2],
                          dt_bias=p["dt_bias"], D=p["D"], z=z[:, sl], h_in=h)

    def buffers():
        return (torch.zeros(d.B, d.H, d.P, d.N, device="cuda"),
                [torch.zeros(d.B, d.K - 1, d.cd, dtype=torch.bfloat16, device="cuda") for _ in range(2)],
                torch.zeros(d.B, d.L, d.hp, dtype=torch.bfloat16, device="cuda"))

    h, cs, out = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        steps(*buffers())  # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps(h, cs, out)
    gen = torch.Generator().manual_seed(86)
    for r in range(3):
        h0 = torch.randn(d.B, d.H, d.P, d.N, generator=gen).mul_(0.5 * (r + 1)).cuda()
        c0 = torch.randn(d.B, d.K - 1, d.cd, generator=gen).to(torch.bfloat16).cuda()
        h.copy_(h0)
        cs[0].copy_(c0)
        graph.replay()
        torch.cuda.synchronize()
        he, cse, oute = buffers()
        he.copy_(h0)
        cse[0].copy_(c0)
        steps(he, cse, oute)
        torch.cuda.synchronize()
        last = d.L % 2
        print(f"[decode graph] replay {r}: out max |diff| {(out.float() - oute.float()).abs().max().item():.3e}",
              flush=True)
        assert torch.equal(out, oute) and torch.equal(h, he) and torch.equal(cs[last], cse[last]), r
        assert torch.isfinite(out.float()).all()
