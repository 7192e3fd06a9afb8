"""GPU parity of the full Mamba-2 block (RMSNorm -> in_proj -> hot path -> gated RMSNorm
-> out_proj -> residual), forward and backward, against the fp64 oracle.

Backward outputs compared: du, the projection weight gradients (fp32), both norm gains,
the conv weight and bias, A, D, dt_bias, and the gradients of both carried states (h and
the conv buffer).  Also the building blocks alone: mixer_proj_bwd (input and weight
gradients, ragged M and a reduction length that is not a multiple of 64) and rmsnorm
forward / backward.  Bar: relative L2 <= 1e-2 (bf16 I/O), plus the per-chunk bar on du.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from selective_state_space_15_amd import binding as bd
from selective_state_space_15_amd import block, synth
from tests.gpu_cases import TOL, check_chunks, fdev, rel_l2, to_dev, to_host

pytestmark = pytest.mark.gpu
EPS = block.EPS


def bits_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)


# the last two cases' weight gradients (K = 16,384 and a ragged 16,392 tokens, 17 x 9
# blocks of 256 with ragged edges) take the big 256 x 256 blocks of the long-K rule
@pytest.mark.parametrize("M,N,K", [(1000, 4384, 1024), (777, 1024, 2048), (333, 648, 256), (16384, 4104, 2104),
                                   (16392, 4104, 2104)])
def test_mixer_proj_bwd(M, N, K):
    r = np.random.default_rng(M + N)
    dy = synth.bf16_bits(r.standard_normal((M, N)).astype(np.float32))
    x = synth.bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    w = synth.bf16_bits((0.02 * r.standard_normal((N, K))).astype(np.float32))
    dw0 = r.standard_normal((N, K)).astype(np.float32)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dw = fdev(dw0)
    bd.mixer_proj_bwd(bits_dev(dy), x=bits_dev(x), w=bits_dev(w), dx=dx, dw=dw, accumulate=True)
    torch.cuda.synchronize()
    f = synth.bf16_to_f32
    rdx = f(dy).astype(np.float64) @ f(w).astype(np.float64)
    rdw = dw0 + f(dy).astype(np.float64).T @ f(x).astype(np.float64)
    e = dict(dx=rel_l2(to_host(dx), rdx), dw=rel_l2(to_host(dw), rdw))
    print(f"[proj_bwd] M={M} N={N} K={K} " + " ".join(f"{k}={v:.2e}" for k, v in e.items()), flush=True)
    assert all(v <= TOL["bf16"] for v in e.values()), e


@pytest.mark.parametrize("K", [8, 72, 200])
def test_mixer_proj_big_blocks_ragged_k(K):
    """dx = dy w with 8,192 x 8,192 outputs (1,024 blocks of 256 x 256: the big blocks) and
    a reduction (the projection's output width) that ends inside its last K-tile of 64:
    none, one or three whole tiles before it."""
    M = N = 8192
    r = np.random.default_rng(K)
    dy = synth.bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    w = synth.bf16_bits((0.1 * r.standard_normal((K, N))).astype(np.float32))
    dx = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    bd.mixer_proj_bwd(bits_dev(dy), w=bits_dev(w), dx=dx)
    torch.cuda.synchronize()
    f = lambda a: synth.bf16_to_f32(a).astype(np.float64)
    e = rel_l2(to_host(dx), f(dy) @ f(w))
    print(f"[proj ragged K] K={K} dx={e:.2e}", flush=True)
    assert e <= TOL["bf16"], e


def test_rmsnorm_fwd_bwd():
    r = np.random.default_rng(90)
    M, K = 999, 2048
    x = synth.bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    dy = synth.bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    dres = synth.bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    g = (1 + 0.1 * r.standard_normal(K)).astype(np.float32)
    y = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    rs = torch.empty(M, device="cuda")
    bd.rmsnorm_fwd(bits_dev(x), fdev(g), y, eps=EPS, rstd=rs)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dg = torch.zeros(K, device="cuda")
    ws = torch.empty(bd.rmsnorm_bwd_workspace(K), dtype=torch.uint8, device="cuda")
    bd.rmsnorm_bwd(bits_dev(x), fdev(g), bits_dev(dy), dx, eps=EPS, dres=bits_dev(dres), dg=dg, ws=ws)
    torch.cuda.synchronize()
    f = lambda a: synth.bf16_to_f32(a).astype(np.float64)
    ry = orc.rmsnorm(f(x), g, EPS)
    rdx, rdg = orc.rmsnorm_bwd(f(x), g, EPS, f(dy))
    e = dict(y=rel_l2(to_host(y), ry), dx=rel_l2(to_host(dx), rdx + f(dres)), dg=rel_l2(to_host(dg), rdg),
             rstd=rel_l2(to_host(rs), 1 / np.sqrt(np.mean(f(x) ** 2, axis=1) + EPS)))
    print("[rmsnorm] " + " ".join(f"{k}={v:.2e}" for k, v in e.items()), flush=True)
    assert all(v <= TOL["bf16"] for v in e.values()), e


def make_block(d: synth.Dims, seed: int):
    sh = block.Shape(d.d_model, d.H, d.P, d.N, d.G, d.K)
    wts = synth.mixer_weights(d, seed)
    prm = synth.params(d, seed)
    w = block.Weights(w_in=bits_dev(wts["w_in"]), w_out=bits_dev(wts["w_out"]), norm_in=fdev(wts["norm_in"]),
                      norm_out=fdev(wts["norm_out"]), conv_w=fdev(prm["conv_w"]), conv_b=fdev(prm["conv_b"]),
                      A=fdev(prm["A"]), D=fdev(prm["D"]), dt_bias=fdev(prm["dt_bias"]))
    return sh, w, wts, prm


def oracle_block_bwd(d, u, wts, prm, dF, st):
    f = lambda a: a.astype(np.float64)
    b = synth.bf16_to_f32
    return orc.block_bwd(b(u), b(wts["w_in"]), f(prm["conv_w"]), f(prm["conv_b"]), f(prm["A"]), d.H, d.P, d.G,
                         d.N, b(wts["w_out"]), b(dF), dt_bias=f(prm["dt_bias"]), D=f(prm["D"]),
                         norm_in=f(wts["norm_in"]), norm_out=f(wts["norm_out"]), eps=EPS, residual=True,
                         h0=f(st["h0"]), conv_state=f(st["conv_state"]), dh_final=f(st["dh_final"]),
                         dconv_state_out=f(st["dconv_state"]))


@pytest.mark.parametrize("name", ["small", "c1", "c4", "c1-prenorm"])
def test_block_fwd_bwd(name, monkeypatch):
    if name == "c1-prenorm":
        # the forward's norms as passes of their own (rmsnorm_fwd, then plain products),
        # the form large projections take
        monkeypatch.setattr(block, "BIG_BLOCKS", 1)
    if name == "small":
        d = synth.Dims(B=2, L=777, H=8, P=32, N=64, G=1, K=4, d_model=256)
    elif name in ("c1", "c1-prenorm"):
        d = synth.CONFIGS["c1"]
    else:  # the batched 2.7B-style shapes (d_model 2560, 80 heads) at batch 2, L = 1000
        d = synth.CONFIGS["c4"].with_(B=2, L=1000)
    seed = 91
    sh, w, wts, prm = make_block(d, seed)
    u = synth.tokens(d, seed)
    dF = synth.dfinal(d, seed)
    st = synth.states(d, seed)
    B, L = d.B, d.L
    sc = block.Scratch(sh, B, L, "cuda")
    ud = bits_dev(u)
    final = torch.empty(B, L, d.d_model, dtype=torch.bfloat16, device="cuda")
    block.block_fwd(sh, w, ud, final, sc, h0=fdev(st["h0"]), conv_state=to_dev(st["conv_state"], "bf16"))
    du = torch.empty_like(ud)
    grads = block.zero_grads(w)
    dh0 = torch.empty(B, d.H, d.P, d.N, device="cuda")
    dcs = torch.empty(B, d.K - 1, d.cd, dtype=torch.bfloat16, device="cuda")
    block.block_bwd(sh, w, ud, bits_dev(dF), du, grads, sc, h0=fdev(st["h0"]),
                    conv_state=to_dev(st["conv_state"], "bf16"), dh_final=fdev(st["dh_final"]),
                    dconv_state_out=to_dev(st["dconv_state"], "bf16"), dh0=dh0, dconv_state_in=dcs,
                    accumulate=False)
    torch.cuda.synchronize()
    f = lambda a: a.astype(np.float64)
    rf = orc.mixer_full_fwd(synth.bf16_to_f32(u), synth.bf16_to_f32(wts["w_in"]), f(prm["conv_w"]),
                            f(prm["conv_b"]), f(prm["A"]), d.H, d.P, d.G, d.N, synth.bf16_to_f32(wts["w_out"]),
                            dt_bias=f(prm["dt_bias"]), D=f(prm["D"]), h0=f(st["h0"]),
                            conv_state=f(st["conv_state"]), norm_in=f(wts["norm_in"]),
                            norm_out=f(wts["norm_out"]), eps=EPS, residual=True)
    r = oracle_block_bwd(d, u, wts, prm, dF, st)
    e = dict(final=rel_l2(to_host(final), rf["final"]), du=rel_l2(to_host(du), r["du"]),
             dw_in=rel_l2(to_host(grads["w_in"]), r["dw_in"]), dw_out=rel_l2(to_host(grads["w_out"]), r["dw_out"]),
             dnorm_in=rel_l2(to_host(grads["norm_in"]), r["dnorm_in"]),
             dnorm_out=rel_l2(to_host(grads["norm_out"]), r["dnorm_out"]),
             dconv_w=rel_l2(to_host(grads["conv_w"]), r["dconv_w"]), dconv_b=rel_l2(to_host(grads["conv_b"]), r["dconv_b"]),
             dA=rel_l2(to_host(grads["A"]), r["dA"]), dD=rel_l2(to_host(grads["D"]), r["dD"]),
             ddt_bias=rel_l2(to_host(grads["dt_bias"]), r["ddt_bias"]), dh0=rel_l2(to_host(dh0), r["dh0"]),
             dconv_state=rel_l2(to_host(dcs), r["dconv_state"]))
    print(f"[block] {name} L={L} " + " ".join(f"{k}={v:.2e}" for k, v in e.items()), flush=True)
    assert all(v <= TOL["bf16"] for v in e.values()), e
    check_chunks("du", to_host(du), r["du"], TOL["bf16"], name)
