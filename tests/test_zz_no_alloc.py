"""ssd_fwd_noalloc (scratch in the library's fixed per-device array) against ssd_fwd
(scratch from a caller workspace): the same kernels on the same inputs, so every
output must be bitwise equal.  Two calls in a row on one device, the second with a
smaller input, so the second reuses the array the first one wrote; and a size beyond
the array's limit is refused before anything is enqueued."""
import pytest
import torch

from selective_state_space_15_amd import binding as bd
from selective_state_space_15_amd import synth
from tests.gpu_cases import Case, TOL, fdev, rel_l2, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(case, noalloc, ckpt_every):
    d = case.d
    zx, z, xbc, dt = case.dev_inputs()
    st = case.st
    dims = case.dims()
    out = torch.empty(d.B, d.L, d.hp, dtype=torch.bfloat16, device="cuda")
    hf = torch.empty(d.B, d.H, d.P, d.N, device="cuda")
    cso = torch.empty(d.B, d.K - 1, d.cd, dtype=torch.bfloat16, device="cuda")
    nck = (d.L + ckpt_every - 1) // ckpt_every
    hck = torch.empty(nck, d.B, d.H, d.P, d.N, device="cuda")
    p = case.p
    kw = dict(conv_w=fdev(p["conv_w"]), conv_b=fdev(p["conv_b"]),
              conv_state_in=to_dev(st["conv_state"], "bf16"), conv_state_out=cso,
              dt_bias=fdev(p["dt_bias"]), D=fdev(p["D"]), z=z, h0=fdev(st["h0"]), h_final=hf,
              h_ckpt=hck, ckpt_every=ckpt_every)
    # poison the outputs so that anything left unwritten shows
    for t in (out, hf, cso, hck):
        t.fill_(float("nan"))
    if noalloc:
        bd.ssd_fwd_noalloc(dims, xbc, fdev(p["A"]), dt, out, **kw)
    else:
        ws = torch.empty(max(bd.ssd_fwd_workspace(dims, bd.SSD_BF16), 1), dtype=torch.uint8,
                         device="cuda")
        bd.ssd_fwd(dims, xbc, fdev(p["A"]), dt, out, ws=ws, **kw)
    torch.cuda.synchronize()
    return dict(out=out, h_final=hf, conv_state_out=cso, h_ckpt=hck)


@pytest.mark.parametrize("L,seed", [(5000, 60), (777, 61)])
def test_noalloc_equals_workspace_entry_point(L, seed):
    case = Case(synth.CONFIGS["c1"].with_(L=L), seed=seed, states=True)
    a = _run(case, True, 1024)
    b = _run(case, False, 1024)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    r = case.oracle_fwd(h0=case.st["h0"].astype("float64"),
                        conv_state=case.st["conv_state"].astype("float64"))
    e = rel_l2(to_host(a["out"]), r["out"])
    print(f"[noalloc] L={L} bitwise equal to ssd_fwd; out vs oracle {e:.2e}", flush=True)
    assert e <= TOL["bf16"]


def test_noalloc_two_calls_in_a_row_second_smaller():
    big = Case(synth.CONFIGS["c1"].with_(L=6000), seed=62, states=True)
    small = Case(synth.CONFIGS["c1"].with_(L=300), seed=63, states=True)
    a1 = _run(big, True, 1024)
    a2 = _run(small, True, 128)
    b1 = _run(big, False, 1024)
    b2 = _run(small, False, 128)
    for k in a1:
        assert torch.equal(a1[k], b1[k]), ("first", k)
        assert torch.equal(a2[k], b2[k]), ("second", k)


def test_noalloc_rejects_dims_beyond_its_scratch():
    d = bd.make_dims(1, 1 << 20, 32, 64, 128, 1, 0, 4)
    assert bd.ssd_fwd_workspace(d, bd.SSD_BF16) > bd.NOALLOC_SCRATCH_BYTES
    case = Case(synth.CONFIGS["c1"].with_(L=64), seed=64)
    zx, z, xbc, dt = case.dev_inputs()
    L = 1 << 20
    xbig = torch.zeros(1, L, case.d.cd, dtype=torch.bfloat16, device="cuda")
    dtbig = torch.zeros(1, L, 32, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(1, L, case.d.hp, dtype=torch.bfloat16, device="cuda")
    p = case.p
    with pytest.raises(bd.SsdError) as e:
        bd.ssd_fwd_noalloc(d, xbig, fdev(p["A"]), dtbig, out, conv_w=fdev(p["conv_w"]),
                           conv_b=fdev(p["conv_b"]), dt_bias=fdev(p["dt_bias"]), D=fdev(p["D"]))
    assert e.value.status == bd.SSD_ERR_WORKSPACE
