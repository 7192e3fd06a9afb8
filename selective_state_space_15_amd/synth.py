"""Seeded synthetic inputs for the mixer hot path.

This module only draws random numbers and rounds them to the I/O dtype; it holds
none of the method's arithmetic.  Both the GPU tests / bench and the fp64 oracle
take their inputs from here, so parity measures only the GPU arithmetic.

Workloads (shapes from the Video-Ma2mba model card: Mamba-2 LM, 48 layers,
d_model 1024, bf16; 2.7B-style variant from the same card's variant table):

  c0  single SSD scan, fp32: B=1, L=512, 4 heads x 32, d_state 16, no conv, no gate
  c1  one mixer, bf16: d_model 1024, 32 heads x 64, d_state 128, conv 4, B=1, L=8192
  c2  c1 shapes, L = 4096 frames x 256 tokens = 1,048,576, per-frame mean drift
  c3  c1 shapes, L = 262,144 as 16 segments of 16,384 (segmented fwd+bwd)
  c4  2.7B-style: d_model 2560, 80 heads x 64, d_state 128, conv 4, B=16, L=4096

Hot-path inputs of the mixer configs are the in_proj output row per token,
laid out [z (H*P) | xBC (H*P + 2*G*N) | dt_raw (H)].  With token embeddings
u ~ N(0, 1) and in_proj weights ~ N(0, 0.02^2), every in_proj output channel is
N(0, d_model * 0.02^2) and nearly independent of the others, so the generator
draws that row directly with sigma = 0.02 * sqrt(d_model).  For c2 the frame
drift u_t = mu_f + noise (mu a per-channel random walk over frames with step
std 0.1) maps through in_proj to a per-channel random-walk offset with step std
0.1 * sigma added to every token of the frame.

Parameters: A = -exp(U(0, ln 16)); D ~ N(0, 1); dt_bias = log(expm1(dt0)) with
dt0 log-uniform in [1e-3, 1e-1] (so softplus(dt_bias) = dt0); conv weight and
bias ~ U(-1/sqrt(K), 1/sqrt(K)).  Upstream gradient dout ~ N(0, 1).

Every tensor has its own stream; large tensors are drawn in blocks of
``BLOCK`` tokens, each from its own counter-derived stream
SeedSequence([seed, tensor_id, batch, block]), so any token window can be
regenerated on its own and blocks can be filled in parallel.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

BLOCK = 4096

# tensor ids for the counter-derived streams
_T_ZXBCDT, _T_DOUT, _T_X, _T_DT, _T_B, _T_C, _T_DRIFT = 1, 2, 3, 4, 5, 6, 7
_T_A, _T_D, _T_DTB, _T_CW, _T_CB, _T_H0, _T_CS, _T_DH, _T_DCS = 11, 12, 13, 14, 15, 16, 17, 18, 19
_T_U, _T_WIN, _T_WOUT, _T_NIN, _T_NOUT, _T_DFINAL = 21, 22, 23, 24, 25, 26


@dataclass(frozen=True)
class Dims:
    B: int
    L: int
    H: int
    P: int
    N: int
    G: int = 1
    K: int = 4            # conv width; 0 = no conv (plain SSD)
    Q: int = 256          # chunk length named by the workload
    d_model: int = 0      # 0 = no in_proj (plain SSD inputs)
    dtype: str = "bf16"   # I/O dtype: "bf16" or "f32"
    gate: bool = True
    seg: int = 0          # segment length of the segmented workloads (0 = none)
    drift: bool = False   # per-frame mean drift (c2)
    frame: int = 256

    @property
    def hp(self) -> int:
        return self.H * self.P

    @property
    def cd(self) -> int:
        return self.H * self.P + 2 * self.G * self.N

    @property
    def d_in_proj(self) -> int:
        return 2 * self.H * self.P + 2 * self.G * self.N + self.H

    @property
    def sigma(self) -> float:
        return 0.02 * math.sqrt(self.d_model) if self.d_model else 1.0

    def with_(self, **kw) -> "Dims":
        return replace(self, **kw)


CONFIGS = {
    "c0": Dims(B=1, L=512, H=4, P=32, N=16, G=1, K=0, Q=64, d_model=0, dtype="f32", gate=False),
    "c1": Dims(B=1, L=8192, H=32, P=64, N=128, G=1, K=4, Q=256, d_model=1024),
    "c2": Dims(B=1, L=1048576, H=32, P=64, N=128, G=1, K=4, Q=256, d_model=1024, drift=True),
    "c3": Dims(B=1, L=262144, H=32, P=64, N=128, G=1, K=4, Q=256, d_model=1024, seg=16384),
    "c4": Dims(B=16, L=4096, H=80, P=64, N=128, G=1, K=4, Q=256, d_model=2560),
}


# ----------------------------------------------------------------- bf16 helpers

def bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_io(a, dtype: str) -> np.ndarray:
    """Round float values to what the I/O dtype can hold (returned as float32)."""
    a = np.asarray(a, dtype=np.float32)
    return bf16_to_f32(bf16_bits(a)) if dtype == "bf16" else a


# ----------------------------------------------------------------- streams

def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed)] + [int(k) for k in key])))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def params(d: Dims, seed: int = 0) -> dict:
    """Per-head and per-channel parameters (float32; fp32 on both sides)."""
    H = d.H
    A = -np.exp(_rng(seed, _T_A).uniform(0.0, math.log(16.0), H))
    D = _rng(seed, _T_D).standard_normal(H)
    dt0 = np.exp(_rng(seed, _T_DTB).uniform(math.log(1e-3), math.log(1e-1), H))
    dt_bias = np.log(np.expm1(dt0))
    p = dict(A=A.astype(np.float32), D=D.astype(np.float32), dt_bias=dt_bias.astype(np.float32))
    if d.K:
        lim = 1.0 / math.sqrt(d.K)
        p["conv_w"] = _rng(seed, _T_CW).uniform(-lim, lim, (d.cd, d.K)).astype(np.float32)
        p["conv_b"] = _rng(seed, _T_CB).uniform(-lim, lim, d.cd).astype(np.float32)
    return p


def _drift_table(d: Dims, seed: int, b: int) -> np.ndarray:
    """Per-frame per-channel offsets: random walk with step std 0.1 * sigma."""
    nf = (d.L + d.frame - 1) // d.frame
    steps = _rng(seed, _T_DRIFT, b).standard_normal((nf, d.d_in_proj)) * (0.1 * d.sigma)
    return np.cumsum(steps, axis=0)


def _fill_rows(d: Dims, seed: int, tid: int, width: int, scale: float, out: np.ndarray,
               t0: int, t1: int, drift: bool) -> None:
    """Fill out[b, :, :] (float32 or bf16 bits) with tokens [t0, t1) of tensor tid."""
    bf = out.dtype == np.uint16

    def job(args):
        b, blk, table = args
        lo, hi = max(t0, blk * BLOCK), min(t1, (blk + 1) * BLOCK)
        r = _rng(seed, tid, b, blk)
        # always a full block, so a token's value does not depend on L or the window
        v = r.standard_normal((BLOCK, width), dtype=np.float32)[lo - blk * BLOCK:hi - blk * BLOCK]
        if scale != 1.0:
            v *= np.float32(scale)
        if table is not None:
            fr = np.arange(lo, hi) // d.frame
            v += table[fr].astype(np.float32)
        out[b, lo - t0:hi - t0] = bf16_bits(v) if bf else v

    jobs = []
    for b in range(out.shape[0]):
        table = _drift_table(d, seed, b) if drift else None
        for blk in range(t0 // BLOCK, (t1 + BLOCK - 1) // BLOCK):
            jobs.append((b, blk, table))
    if len(jobs) > 2:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(job, jobs))
    else:
        for j in jobs:
            job(j)


def zxbcdt(d: Dims, seed: int = 0, t0: int = 0, t1: int | None = None, bits: bool = None) -> np.ndarray:
    """In_proj output rows [B, t1-t0, d_in_proj] = [z | xBC_raw | dt_raw] for tokens [t0, t1).

    Returned as bf16 bit patterns (uint16) for bf16 workloads unless bits=False,
    else float32 (already rounded to the I/O dtype)."""
    t1 = d.L if t1 is None else t1
    if bits is None:
        bits = d.dtype == "bf16"
    out = np.empty((d.B, t1 - t0, d.d_in_proj), dtype=np.uint16 if bits else np.float32)
    _fill_rows(d, seed, _T_ZXBCDT, d.d_in_proj, d.sigma, out, t0, t1, d.drift)
    if not bits and d.dtype == "bf16":
        out = round_io(out, "bf16")
    return out


def dout(d: Dims, seed: int = 0, t0: int = 0, t1: int | None = None, bits: bool = None) -> np.ndarray:
    """Upstream gradient at the hot-path output [B, t1-t0, H*P], N(0, 1)."""
    t1 = d.L if t1 is None else t1
    if bits is None:
        bits = d.dtype == "bf16"
    out = np.empty((d.B, t1 - t0, d.hp), dtype=np.uint16 if bits else np.float32)
    _fill_rows(d, seed, _T_DOUT, d.hp, 1.0, out, t0, t1, False)
    if not bits and d.dtype == "bf16":
        out = round_io(out, "bf16")
    return out


def split_zxbcdt(d: Dims, a: np.ndarray):
    """Views (z, xbc_raw, dt_raw) of an in_proj row array [B, L, d_in_proj]."""
    hp, cd = d.hp, d.cd
    return a[..., :hp], a[..., hp:hp + cd], a[..., hp + cd:hp + cd + d.H]


def ssd_inputs(d: Dims, seed: int = 0) -> dict:
    """Plain SSD inputs (no conv, no in_proj): x [B,L,H,P], dt_raw [B,L,H], Bm, Cm [B,L,G,N],
    all float32 rounded to the I/O dtype.  x ~ N(0,1), dt_raw ~ N(0,1), B, C ~ N(0,1)/sqrt(N)."""
    B, L, H, P, N, G = d.B, d.L, d.H, d.P, d.N, d.G
    x = _rng(seed, _T_X).standard_normal((B, L, H, P))
    dt = _rng(seed, _T_DT).standard_normal((B, L, H))
    Bm = _rng(seed, _T_B).standard_normal((B, L, G, N)) / math.sqrt(N)
    Cm = _rng(seed, _T_C).standard_normal((B, L, G, N)) / math.sqrt(N)
    r = lambda a: round_io(a.astype(np.float32), d.dtype)
    return dict(x=r(x), dt_raw=r(dt), Bm=r(Bm), Cm=r(Cm))


def states(d: Dims, seed: int = 0, scale: float = 0.5) -> dict:
    """Non-zero carried states for state-carry tests: h0 [B,H,P,N] fp32 and conv_state
    [B,K-1,Cd] (I/O dtype), plus upstream state gradients dh_final and dconv_state."""
    B, H, P, N = d.B, d.H, d.P, d.N
    out = dict(h0=(_rng(seed, _T_H0).standard_normal((B, H, P, N)) * scale).astype(np.float32),
               dh_final=(_rng(seed, _T_DH).standard_normal((B, H, P, N)) * scale).astype(np.float32))
    if d.K:
        cs = _rng(seed, _T_CS).standard_normal((B, d.K - 1, d.cd)) * d.sigma
        dcs = _rng(seed, _T_DCS).standard_normal((B, d.K - 1, d.cd)) * scale
        out["conv_state"] = round_io(cs.astype(np.float32), d.dtype)
        out["dconv_state"] = round_io(dcs.astype(np.float32), d.dtype)
    return out


# ----------------------------------------------------------------- mixer projections

def tokens(d: Dims, seed: int = 0, t0: int = 0, t1: int | None = None) -> np.ndarray:
    """Token embeddings u [B, t1-t0, d_model] ~ N(0, 1) (plus the per-frame mean drift,
    a per-channel random walk over frames with step std 0.1, when d.drift), as bf16
    bit patterns."""
    t1 = d.L if t1 is None else t1
    out = np.empty((d.B, t1 - t0, d.d_model), dtype=np.uint16)
    if d.drift:
        # same drift construction as the in_proj rows, in token space (step std 0.1)
        def table(b):
            nf = (d.L + d.frame - 1) // d.frame
            return np.cumsum(_rng(seed, _T_DRIFT, b, 1).standard_normal((nf, d.d_model)) * 0.1, axis=0)
        _fill_rows_table(d, seed, _T_U, d.d_model, 1.0, out, t0, t1, table)
    else:
        _fill_rows(d, seed, _T_U, d.d_model, 1.0, out, t0, t1, False)
    return out


def _fill_rows_table(d, seed, tid, width, scale, out, t0, t1, table_of):
    bf = out.dtype == np.uint16
    for b in range(out.shape[0]):
        table = table_of(b)
        for blk in range(t0 // BLOCK, (t1 + BLOCK - 1) // BLOCK):
            lo, hi = max(t0, blk * BLOCK), min(t1, (blk + 1) * BLOCK)
            v = _rng(seed, tid, b, blk).standard_normal((BLOCK, width), dtype=np.float32)[lo - blk * BLOCK:hi - blk * BLOCK]
            v = v * np.float32(scale) + table[np.arange(lo, hi) // d.frame].astype(np.float32)
            out[b, lo - t0:hi - t0] = bf16_bits(v) if bf else v


def mixer_weights(d: Dims, seed: int = 0) -> dict:
    """Random-init projection weights of the mixer (nn.Linear layout [out, in]), as bf16
    bit patterns: W_in [d_in_proj, d_model] and W_out [d_model, H*P] ~ N(0, 0.02^2);
    RMSNorm gains (fp32) of the full block ~ 1 + N(0, 0.1^2): norm_in [d_model] before
    in_proj, norm_out [H*P] before out_proj."""
    w_in = _rng(seed, _T_WIN).standard_normal((d.d_in_proj, d.d_model), dtype=np.float32) * np.float32(0.02)
    w_out = _rng(seed, _T_WOUT).standard_normal((d.d_model, d.hp), dtype=np.float32) * np.float32(0.02)
    n_in = 1.0 + 0.1 * _rng(seed, _T_NIN).standard_normal(d.d_model)
    n_out = 1.0 + 0.1 * _rng(seed, _T_NOUT).standard_normal(d.hp)
    return dict(w_in=bf16_bits(w_in), w_out=bf16_bits(w_out), norm_in=n_in.astype(np.float32),
                norm_out=n_out.astype(np.float32))


def dfinal(d: Dims, seed: int = 0) -> np.ndarray:
    """Upstream gradient at the mixer's final output [B, L, d_model] ~ N(0, 1), bf16 bits."""
    out = np.empty((d.B, d.L, d.d_model), dtype=np.uint16)
    _fill_rows(d, seed, _T_DFINAL, d.d_model, 1.0, out, 0, d.L, False)
    return out
