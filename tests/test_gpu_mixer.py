"""GPU parity of the mixer's projections (mixer_proj) and of the whole mixer against
the fp64 oracle.

* mixer_proj alone: y = x W^T on MFMA, plain, with the RMSNorm prologue, with the
  residual epilogue, at ragged M and N, against numpy fp64 products.
* The d_model 1024 mixer (32 heads x 64, d_state 128, conv 4, bf16), token
  embeddings u ~ N(0, 1) and weights ~ N(0, 0.02^2), L = 8192:
      in_proj (mixer_proj) -> ssd_fwd (conv1d + SiLU -> SSD -> SiLU(z) gate)
      -> out_proj (mixer_proj)
  against the oracle's fp64 in_proj, hot path and out_proj.  The GPU rounds the
  in_proj rows and the gated output to bf16 between the stages, as any bf16
  pipeline does; the oracle carries fp64 throughout.
* The full block: RMSNorm before in_proj, the gated RMSNorm before out_proj (over
  the SiLU(z)-gated output) and the residual, at the same shapes.
Bar: relative L2 <= 1e-2 (bf16 I/O) on every output, plus the per-chunk bar.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from selective_state_space_15_amd import binding as bd
from selective_state_space_15_amd import synth
from tests.gpu_cases import TOL, check_chunks, fdev, rel_l2, to_host

pytestmark = pytest.mark.gpu
EPS = 1e-5


def bits_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)


@pytest.mark.parametrize("M,N,K,norm,res", [(1000, 4384, 1024, False, False), (333, 1000, 2048, True, False),
                                            (257, 1024, 2048, False, True), (8192, 1024, 2048, True, True),
                                            (1, 8, 64, True, True)])
def test_mixer_proj(M, N, K, norm, res):
    r = np.random.default_rng(M + N + K)
    x = synth.bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    w = synth.bf16_bits((0.02 * r.standard_normal((N, K))).astype(np.float32))
    g = (1.0 + 0.1 * r.standard_normal(K)).astype(np.float32) if norm else None
    rr = synth.bf16_bits(r.standard_normal((M, N)).astype(np.float32)) if res else None
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    bd.mixer_proj(bits_dev(x), bits_dev(w), y, norm_w=fdev(g), norm_eps=EPS,
                  residual=None if rr is None else bits_dev(rr))
    torch.cuda.synchronize()
    ref = orc.linear(synth.bf16_to_f32(x), synth.bf16_to_f32(w), g, EPS,
                     None if rr is None else synth.bf16_to_f32(rr))
    e = rel_l2(to_host(y), ref)
    print(f"[proj] M={M} N={N} K={K} norm={norm} res={res} rel_l2={e:.2e}", flush=True)
    assert e <= TOL["bf16"]
    check_chunks("y", to_host(y)[None], ref[None], TOL["bf16"], "proj")


def run_mixer(d, seed, full_block):
    """GPU mixer over u; returns (final, zxbcdt, out) as host float64 plus the inputs."""
    B, L = d.B, d.L
    u = synth.tokens(d, seed)
    wts = synth.mixer_weights(d, seed)
    prm = synth.params(d, seed)
    ud = bits_dev(u)
    dip = d.d_in_proj
    zx = torch.empty(B, L, dip, dtype=torch.bfloat16, device="cuda")
    bd.mixer_proj(ud.view(B * L, d.d_model), bits_dev(wts["w_in"]), zx.view(B * L, dip),
                  norm_w=fdev(wts["norm_in"]) if full_block else None, norm_eps=EPS)
    hp, cd, H = d.hp, d.cd, d.H
    z, xbc, dt = zx[..., :hp], zx[..., hp:hp + cd], zx[..., hp + cd:hp + cd + H]
    dims = bd.make_dims(B, L, H, d.P, d.N, d.G, 0, d.K)
    out = torch.empty(B, L, hp, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(bd.ssd_fwd_workspace(dims, bd.SSD_BF16), 1), dtype=torch.uint8, device="cuda")
    p = {k: fdev(v) for k, v in prm.items()}
    bd.ssd_fwd(dims, xbc, p["A"], dt, out, conv_w=p["conv_w"], conv_b=p["conv_b"], dt_bias=p["dt_bias"],
               D=p["D"], z=z, ws=ws)
    final = torch.empty(B, L, d.d_model, dtype=torch.bfloat16, device="cuda")
    bd.mixer_proj(out.view(B * L, hp), bits_dev(wts["w_out"]), final.view(B * L, d.d_model),
                  norm_w=fdev(wts["norm_out"]) if full_block else None, norm_eps=EPS,
                  residual=ud.view(B * L, d.d_model) if full_block else None)
    torch.cuda.synchronize()
    return dict(final=to_host(final), zx=to_host(zx), out=to_host(out)), u, wts, prm


def oracle_mixer(d, u, wts, prm, full_block):
    f = lambda a: a.astype(np.float64)
    return orc.mixer_full_fwd(synth.bf16_to_f32(u), synth.bf16_to_f32(wts["w_in"]), f(prm["conv_w"]),
                              f(prm["conv_b"]), f(prm["A"]), d.H, d.P, d.G, d.N,
                              synth.bf16_to_f32(wts["w_out"]), dt_bias=f(prm["dt_bias"]), D=f(prm["D"]),
                              norm_in=f(wts["norm_in"]) if full_block else None,
                              norm_out=f(wts["norm_out"]) if full_block else None, eps=EPS,
                              residual=full_block)


@pytest.mark.parametrize("full_block", [False, True])
def test_c1_mixer_forward(full_block):
    """The d_model 1024 mixer at L = 8192 (and the full block around it) against the
    oracle, stage by stage: in_proj rows, gated hot-path output, final output."""
    d = synth.CONFIGS["c1"]
    g, u, wts, prm = run_mixer(d, 70 + int(full_block), full_block)
    r = oracle_mixer(d, u, wts, prm, full_block)
    tag = "block" if full_block else "mixer"
    errs = dict(zxbcdt=rel_l2(g["zx"], r["zxbcdt"]), out=rel_l2(g["out"], r["out"]),
                final=rel_l2(g["final"], r["final"]))
    print(f"[{tag}] L={d.L} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= TOL["bf16"] for v in errs.values()), errs
    check_chunks("final", g["final"], r["final"], TOL["bf16"], tag)
    check_chunks("out", g["out"], r["out"], TOL["bf16"], tag)


def test_mixer_batched_ragged():
    """Batch 3, ragged L = 777, a smaller mixer (d_model 256: 8 heads x 32, d_state 64;
    in_proj rows of 648 channels)."""
    d = synth.Dims(B=3, L=777, H=8, P=32, N=64, G=1, K=4, d_model=256)
    for full in (False, True):
        g, u, wts, prm = run_mixer(d, 72 + int(full), full)
        r = oracle_mixer(d, u, wts, prm, full)
        e = rel_l2(g["final"], r["final"])
        print(f"[mixer-small] full_block={full} final={e:.2e}", flush=True)
        assert e <= TOL["bf16"]
        check_chunks("final", g["final"], r["final"], TOL["bf16"], "small")
