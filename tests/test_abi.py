"""CPU-side tests of the boundary and the host logic (no GPU, no kernel launch).

* libssd.so loads and exports every function include/ssd.h declares, and the
  binding marshals exactly those.
* Argument validation returns the documented status before anything is enqueued
  (these calls never reach a HIP API, so they run on a machine without a GPU).
* Workspace sizes scale as documented (O(L / 64) chunk states in the backward,
  O(L / sub-segment) states in the forward, nothing proportional to L * state).
* The seeded input generator is deterministic, window-independent and rounds to
  bf16 exactly like torch does.
* The segment driver's conv-buffer checkpoint views.
"""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from selective_state_space_15_amd import binding as bd
from selective_state_space_15_amd import segmented, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:ssd_status|int|const char\*)\s+([a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = bd.lib()
    names = header_functions()
    assert len(names) >= 14, names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(bd.exported_symbols()) == names


def test_abi_version_and_status_strings():
    assert bd.ssd_abi_version() == 1
    for st in range(-7, 1):
        assert bd.ssd_status_string(st).startswith("SSD_")
    assert "unknown" in bd.ssd_status_string(42)


def _err(fn, *a):
    with pytest.raises(bd.SsdError) as e:
        fn(*a)
    return e.value.status


def test_workspace_query_validation():
    ok = bd.make_dims(1, 1000, 32, 64, 128, 1, 0, 4)
    assert bd.ssd_fwd_workspace(ok, bd.SSD_BF16) > 0
    assert _err(bd.ssd_fwd_workspace, bd.make_dims(0, 10, 4, 64, 128), bd.SSD_BF16) == bd.SSD_ERR_SHAPE
    assert _err(bd.ssd_fwd_workspace, bd.make_dims(1, 10, 3, 64, 128, 2), bd.SSD_BF16) == bd.SSD_ERR_SHAPE
    assert _err(bd.ssd_fwd_workspace, bd.make_dims(1, 10, 4, 48, 128), bd.SSD_BF16) == bd.SSD_ERR_UNSUPPORTED
    assert _err(bd.ssd_fwd_workspace, bd.make_dims(1, 10, 4, 64, 96), bd.SSD_BF16) == bd.SSD_ERR_UNSUPPORTED
    assert _err(bd.ssd_fwd_workspace, bd.make_dims(1, 10, 4, 64, 128, 1, 256), bd.SSD_BF16) == bd.SSD_ERR_UNSUPPORTED
    assert _err(bd.ssd_fwd_workspace, bd.make_dims(1, 10, 4, 64, 128, 1, 0, 5), bd.SSD_BF16) == bd.SSD_ERR_UNSUPPORTED
    assert _err(bd.ssd_fwd_workspace, ok, 7) == bd.SSD_ERR_DTYPE
    assert _err(bd.ssd_bwd_workspace, bd.make_dims(1, 64, 2, 64, 128, 1, 0, 4), bd.SSD_F32) == bd.SSD_ERR_UNSUPPORTED


def test_entry_points_reject_bad_arguments_before_launch():
    lib = bd.lib()
    d = bd.make_dims(1, 100, 4, 64, 64, 1, 0, 4)
    nullv = bd.ssd_view(None, 0, 0)
    # xbc missing
    st = lib.ssd_fwd(ctypes.byref(d), bd.SSD_BF16, nullv, None, None, nullv, nullv, nullv, None, 1,
                     None, None, nullv, None, nullv, None, None, 0, None, 0, None)
    assert st == bd.SSD_ERR_NULL
    assert b"xbc" in lib.ssd_last_error()
    # misaligned base pointer (never dereferenced: validation fails first)
    cd = 4 * 64 + 2 * 64
    bad = bd.ssd_view(0x1002, 100 * cd, cd)
    st = lib.ssd_fwd(ctypes.byref(d), bd.SSD_BF16, bad, None, None, nullv, nullv, nullv, None, 1,
                     None, None, nullv, None, nullv, None, None, 0, None, 0, None)
    assert st == bd.SSD_ERR_ALIGN
    # stride not a multiple of 16 bytes
    bad = bd.ssd_view(0x1000, 100 * (cd + 1), cd + 1)
    st = lib.ssd_fwd(ctypes.byref(d), bd.SSD_BF16, bad, None, None, nullv, nullv, nullv, None, 1,
                     None, None, nullv, None, nullv, None, None, 0, None, 0, None)
    assert st == bd.SSD_ERR_ALIGN
    # fp32 state pointers must be 16-byte aligned
    st = lib.ssd_fwd(ctypes.byref(d), bd.SSD_BF16, bd.ssd_view(0x1000, 100 * cd, cd), 0x8000, None,
                     nullv, nullv, bd.ssd_view(0x2000, 400, 4), None, 1, 0x9000, None, nullv, 0x9004,
                     bd.ssd_view(0x4000, 100 * 256, 256), None, None, 0, None, 0, None)
    assert st == bd.SSD_ERR_ALIGN and b"h0" in lib.ssd_last_error()
    # checkpoint spacing must be a multiple of 64
    good = bd.ssd_view(0x1000, 100 * cd, cd)
    dtv = bd.ssd_view(0x2000, 400, 4)
    outv = bd.ssd_view(0x4000, 100 * 256, 256)
    st = lib.ssd_fwd(ctypes.byref(d), bd.SSD_BF16, good, 0x8000, None, nullv, nullv, dtv, None, 1,
                     0x9000, None, nullv, None, outv, None, 0xa000, 100, None, 0, None)
    assert st == bd.SSD_ERR_SHAPE
    # workspace too small
    st = lib.ssd_fwd(ctypes.byref(bd.make_dims(1, 100000, 4, 64, 64, 1, 0, 4)), bd.SSD_BF16,
                     bd.ssd_view(0x1000, 100000 * cd, cd), 0x8000, None, nullv, nullv,
                     bd.ssd_view(0x2000, 400000, 4), None, 1, 0x9000, None, nullv, None,
                     bd.ssd_view(0x4000, 100000 * 256, 256), None, None, 0, None, 0, None)
    assert st == bd.SSD_ERR_WORKSPACE
    # backward: dz required when z is given
    st = lib.ssd_bwd(ctypes.byref(d), bd.SSD_BF16, good, 0x8000, None, nullv, dtv, None, 1, 0x9000,
                     None, outv, None, outv, None, nullv, good, dtv, nullv, 0xb000, None, None, None,
                     None, None, nullv, 0, None, 0, None)
    assert st == bd.SSD_ERR_NULL
    # conv: width and channel multiple
    assert lib.conv1d_fwd(1, 10, 64, 5, bd.SSD_BF16, good, 0x8000, None, 1, nullv, good, nullv, None) \
        == bd.SSD_ERR_UNSUPPORTED
    assert lib.conv1d_fwd(1, 10, 60, 4, bd.SSD_BF16, good, 0x8000, None, 1, nullv, good, nullv, None) \
        == bd.SSD_ERR_UNSUPPORTED
    # conv weights and bias are read as 16-byte vectors
    assert lib.conv1d_fwd(1, 10, 64, 4, bd.SSD_BF16, good, 0x8004, None, 1, nullv, good, nullv, None) \
        == bd.SSD_ERR_ALIGN
    assert lib.conv1d_fwd(1, 10, 64, 4, bd.SSD_BF16, good, 0x8000, 0x9008, 1, nullv, good, nullv, None) \
        == bd.SSD_ERR_ALIGN
    st = lib.ssd_fwd(ctypes.byref(d), bd.SSD_BF16, good, 0x8004, None, nullv, nullv, dtv, None, 1,
                     0x9000, None, nullv, None, outv, None, None, 0, None, 0, None)
    assert st == bd.SSD_ERR_ALIGN and b"conv_w" in lib.ssd_last_error()


def test_workspace_scaling_is_linear_and_modest():
    f16k = bd.ssd_fwd_workspace(bd.make_dims(1, 16384, 32, 64, 128, 1, 0, 4), bd.SSD_BF16)
    f1m = bd.ssd_fwd_workspace(bd.make_dims(1, 1 << 20, 32, 64, 128, 1, 0, 4), bd.SSD_BF16)
    # post-conv B|C rows (512 B/token) + the fp32 dt table (4 B per token and head) + one
    # fp32 state per sub-segment of <= 4096 tokens
    assert f1m <= (1 << 20) * (512 + 32 * 4) + 256 * (1 << 20) + (1 << 22)
    b16k = bd.ssd_bwd_workspace(bd.make_dims(1, 16384, 32, 64, 128, 1, 0, 4), bd.SSD_BF16)
    b32k = bd.ssd_bwd_workspace(bd.make_dims(1, 32768, 32, 64, 128, 1, 0, 4), bd.SSD_BF16)
    assert abs(b32k - 2 * b16k) <= 8192       # linear in the segment length
    assert f16k < b16k


def test_generator_is_deterministic_and_window_independent():
    d = synth.CONFIGS["c2"].with_(L=9000)
    a = synth.zxbcdt(d, 3)
    b = synth.zxbcdt(d, 3, 4000, 8500)
    assert np.array_equal(a[:, 4000:8500], b)
    assert not np.array_equal(a, synth.zxbcdt(d, 4))
    f = synth.bf16_to_f32(a)
    assert abs(float(f.std()) - d.sigma) < 0.05 * d.sigma + 0.1 * d.sigma  # drift adds variance


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    v = (r.standard_normal(100000) * np.exp(r.uniform(-20, 20, 100000))).astype(np.float32)
    mine = synth.bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_params_follow_the_recipe():
    p = synth.params(synth.CONFIGS["c1"], 0)
    assert np.all(p["A"] <= -1.0) and np.all(p["A"] >= -16.0)
    dt0 = np.log1p(np.exp(p["dt_bias"].astype(np.float64)))
    assert np.all(dt0 > 0.99e-3) and np.all(dt0 < 1.01e-1)
    assert np.all(np.abs(p["conv_w"]) <= 0.5) and p["conv_w"].shape == (2304, 4)


def test_conv_checkpoint_views():
    x = torch.arange(2 * 10 * 8, dtype=torch.float32).reshape(2, 10, 8)
    st = torch.full((2, 3, 8), -1.0)
    assert segmented.conv_ckpt(x, st, 0, 4) is st
    v = segmented.conv_ckpt(x, st, 6, 4)
    assert v.data_ptr() == x[:, 3:6].data_ptr() and torch.equal(v, x[:, 3:6])
    j = segmented.conv_ckpt(x, st, 2, 4)          # shorter than the buffer: carried + new rows
    assert torch.equal(j, torch.cat([st[:, 2:], x[:, :2]], dim=1))
    assert segmented.conv_ckpt(x, st, 5, 0) is None


# ------------------------------------------------------------------ binding argument checks
def _cpu_fwd_args(L=100, H=4, P=64, N=64, K=4, dtype=torch.bfloat16):
    cd = H * P + 2 * N
    d = bd.make_dims(1, L, H, P, N, 1, 0, K)
    a = dict(xbc=torch.zeros(1, L, cd, dtype=dtype), A=torch.zeros(H), dt=torch.zeros(1, L, H, dtype=dtype),
             out=torch.zeros(1, L, H * P, dtype=dtype))
    kw = dict(conv_w=torch.zeros(cd, K), conv_b=torch.zeros(cd), dt_bias=torch.zeros(H), D=torch.zeros(H),
              z=torch.zeros(1, L, H * P, dtype=dtype))
    return d, a, kw


def test_binding_rejects_host_tensors_before_the_call():
    d, a, kw = _cpu_fwd_args()
    with pytest.raises(ValueError, match="CUDA"):
        bd.ssd_fwd(d, a["xbc"], a["A"], a["dt"], a["out"], **kw)


@pytest.mark.parametrize("bad", ["dt_dtype", "out_short", "z_channels", "A_len", "h0_shape",
                                 "conv_w_shape", "ckpt_rows", "ckpt_every"])
def test_binding_rejects_mismatched_shapes_and_dtypes(bad):
    d, a, kw = _cpu_fwd_args()
    if bad == "dt_dtype":
        a["dt"] = a["dt"].float()
    elif bad == "out_short":
        a["out"] = a["out"][:, :50]
    elif bad == "z_channels":
        kw["z"] = kw["z"][..., :128]
    elif bad == "A_len":
        a["A"] = torch.zeros(3)
    elif bad == "h0_shape":
        kw["h0"] = torch.zeros(1, 4, 64, 32)
    elif bad == "conv_w_shape":
        kw["conv_w"] = torch.zeros(10, 4)
    elif bad == "ckpt_rows":
        kw.update(h_ckpt=torch.zeros(1, 1, 4, 64, 64), ckpt_every=64)   # needs 2 rows at L=100
    elif bad == "ckpt_every":
        kw.update(h_ckpt=torch.zeros(1, 1, 4, 64, 64), ckpt_every=0)
    with pytest.raises(ValueError):
        bd.ssd_fwd(d, a["xbc"], a["A"], a["dt"], a["out"], **kw)


def test_binding_bwd_and_conv_checks():
    d, a, kw = _cpu_fwd_args(L=64)
    L, cd = 64, a["xbc"].shape[2]
    dout = torch.zeros(1, L, 256, dtype=torch.bfloat16)
    dxbc = torch.zeros(1, L, cd, dtype=torch.bfloat16)
    ddt = torch.zeros(1, L, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dz"):          # gate given, dz missing
        bd.ssd_bwd(d, a["xbc"], a["A"], a["dt"], dout, dxbc, ddt, torch.zeros(4), **kw)
    with pytest.raises(ValueError, match="dxbc"):
        bd.ssd_bwd(d, a["xbc"], a["A"], a["dt"], dout, dxbc[..., :cd - 8], ddt, torch.zeros(4),
                   dz=torch.zeros(1, L, 256, dtype=torch.bfloat16), **kw)
    x = torch.zeros(2, 10, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="w"):
        bd.conv1d_fwd(x, torch.zeros(32, 4), torch.zeros_like(x))
    with pytest.raises(ValueError, match="dw"):
        bd.conv1d_bwd(x, torch.zeros(64, 4), x, torch.zeros_like(x), torch.zeros(64, 3))


def test_noalloc_refuses_oversize_dims_before_any_device_call():
    """The scratch limit is checked after validation and before the device lookup:
    with dims beyond it the call returns SSD_ERR_WORKSPACE (no GPU needed; the
    pointers are never dereferenced)."""
    lib = bd.lib()
    L, H, P, N, K = 1 << 20, 32, 64, 128, 4
    cd = H * P + 2 * N
    d = bd.make_dims(1, L, H, P, N, 1, 0, K)
    assert bd.ssd_fwd_workspace(d, bd.SSD_BF16) > bd.NOALLOC_SCRATCH_BYTES
    base = 1 << 20                                   # a fake, aligned device address
    v = lambda c: bd.ssd_view(base, L * c, c)
    st = lib.ssd_fwd_noalloc(ctypes.byref(d), bd.SSD_BF16, v(cd), base, base, bd.ssd_view(None, 0, 0),
                             bd.ssd_view(None, 0, 0), bd.ssd_view(base, L * H, H), None, 1, base, None,
                             bd.ssd_view(None, 0, 0), None, v(H * P), None, None, 0, None)
    assert st == bd.SSD_ERR_WORKSPACE, st
    assert b"scratch" in lib.ssd_last_error()
