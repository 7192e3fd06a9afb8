"""Benchmark of the Mamba-2 mixer hot path on one MI355X.

Step = one pass of the whole hot path over one batch: the forward over L tokens
(causal conv1d + SiLU -> chunked SSD -> SiLU(z) gate, keeping only the (h, conv
buffer) checkpoints every `seg` tokens), then the backward segment by segment in
reverse (recompute from the checkpoint, all gradients).  Workload: d_model 1024
shapes (32 heads x 64, d_state 128, conv 4), batch 1, L = 1,048,576 tokens as 64
segments of 16,384, bf16 I/O, seeded synthetic in_proj rows (see synth.py).

Prints one JSON line with tokens/s of the whole step, the forward alone, the
roofline of the dominant kernel (HIP events on the launch stream) and the fp64
oracle timed on a bounded prefix on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--L", type=int, default=1 << 20)
    ap.add_argument("--seg", type=int, default=16384)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample", type=int, default=49152, help="oracle prefix tokens (0 = skip)")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for counter runs: one 256 MiB device copy (byte-counter calibration), "
                         "then two fwd+bwd passes over a single segment; prints no JSON")
    return ap.parse_args()


COPY_BYTES = 256 << 20
# HBM bytes of the dominant kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of
# `bench.py --pmc-probe` (see the report for the commands and the copy calibration)
TRAFFIC_REPORT = os.path.join(ROOT, "profiles", "bwd_main_seg16k_hbm_bytes.md")
KERNEL_SYMBOL = {"bwd_main": "bwd_main_kernel", "walk_out": "walk_kernel", "walk_state": "walk_kernel",
                 "conv_bwd": "conv_bwd_kernel"}


def measured_traffic(kind: str):
    """HBM bytes per launch of kernel `kind` from the committed counter report, or None
    when there is none for it or its sources changed since the counters were taken."""
    from selective_state_space_15_amd import profiling
    rec = profiling.read_bytes_report(TRAFFIC_REPORT)
    sym = KERNEL_SYMBOL.get(kind)
    if not rec or rec.get("kernel") != sym:
        return None
    if rec.get("source_fingerprint") != profiling.source_fingerprint(sym):
        return None
    return rec["hbm_bytes_per_launch"]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "the path has no collectives and shards by sequence only in its design notes.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from selective_state_space_15_amd import binding as bd
    from selective_state_space_15_amd import segmented, synth

    if args.pmc_probe:
        args.L = args.seg
    d = synth.CONFIGS["c2"].with_(L=args.L, seg=args.seg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bd.lib()

    # ---------------------------------------------------------------- inputs (host, seeded)
    zx_bits = synth.zxbcdt(d, args.seed)
    zx = torch.from_numpy(zx_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    del zx_bits
    dout = torch.from_numpy(synth.dout(d, args.seed + 7).view(np.int16)).to(dev).view(torch.bfloat16)
    prm = {k: torch.from_numpy(v).to(dev) for k, v in synth.params(d, args.seed).items()}
    hp, cd, H = d.hp, d.cd, d.H
    z, xbc, dt = zx[..., :hp], zx[..., hp:hp + cd], zx[..., hp + cd:hp + cd + H]
    L, B = d.L, d.B
    dims = bd.make_dims(B, L, H, d.P, d.N, d.G, 0, d.K)
    seg_dims = bd.make_dims(B, args.seg, H, d.P, d.N, d.G, 0, d.K)
    out = torch.empty(B, L, hp, dtype=torch.bfloat16, device=dev)
    fws = torch.empty(max(bd.ssd_fwd_workspace(dims, bd.SSD_BF16), 1), dtype=torch.uint8, device=dev)
    bws = torch.empty(max(bd.ssd_bwd_workspace(seg_dims, bd.SSD_BF16), 1), dtype=torch.uint8, device=dev)
    g = dict(dxbc=torch.empty(B, L, cd, dtype=torch.bfloat16, device=dev),
             ddt=torch.empty(B, L, H, dtype=torch.bfloat16, device=dev),
             dz=torch.empty(B, L, hp, dtype=torch.bfloat16, device=dev),
             dA=torch.empty(H, device=dev), dD=torch.empty(H, device=dev),
             ddt_bias=torch.empty(H, device=dev), dconv_w=torch.empty(cd, d.K, device=dev),
             dconv_b=torch.empty(cd, device=dev))
    stream = torch.cuda.current_stream()

    def fwd():
        return segmented.forward_segmented(dims, args.seg, xbc, prm["A"], dt, out, conv_w=prm["conv_w"],
                                           conv_b=prm["conv_b"], dt_bias=prm["dt_bias"], D=prm["D"],
                                           z=z, ws=fws)

    def bwd(h_ckpt):
        segmented.backward_segmented(dims, args.seg, h_ckpt, xbc, prm["A"], dt, dout, g["dxbc"],
                                     g["ddt"], g["dA"], conv_w=prm["conv_w"], conv_b=prm["conv_b"],
                                     dt_bias=prm["dt_bias"], D=prm["D"], z=z, dz=g["dz"], dD=g["dD"],
                                     ddt_bias=g["ddt_bias"], dconv_w=g["dconv_w"],
                                     dconv_b=g["dconv_b"], ws=bws)

    def step():
        bwd(fwd())

    if args.pmc_probe:
        src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        print("pmc probe done", flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = e0.elapsed_time(e1) / args.steps

    # forward alone (same launches), for the forward-only rate
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for _ in range(args.steps):
        fwd()
    f1.record(stream)
    torch.cuda.synchronize()
    ms_fwd = f0.elapsed_time(f1) / args.steps

    # one more step with per-kernel HIP events (library instrumentation, same stream)
    bd.ssd_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ktimes = bd.ssd_timing_read()
    bd.ssd_timing_enable(False)

    tokens = B * L
    # algorithmic bytes per token (each input read once, each output written once)
    es = 2
    fwd_bytes = es * (cd + 2 * hp + H)                    # xBC raw, z, dt in; out
    bwd_bytes = es * (cd + 2 * hp + H) + es * (cd + hp + H)  # + dout in; dxBC, dz, ddt out
    step_bytes = fwd_bytes + bwd_bytes
    roof_tok_s = HBM_PEAK_GBS * 1e9 / step_bytes
    # dominant kernel: the largest summed device time; its algorithmic bytes per
    # launch = the per-token bytes of its pass x the tokens one launch covers
    fwd_kinds = {"walk_state", "scan", "walk_out", "conv_state_out"}
    dom = max(ktimes, key=lambda k: ktimes[k][0])
    dom_ms, dom_n = ktimes[dom]
    dom_avg_ms = dom_ms / max(dom_n, 1)
    if dom in fwd_kinds:
        per_tok, tok_per_launch = fwd_bytes, tokens
    else:
        per_tok, tok_per_launch = bwd_bytes, B * args.seg
    achieved = per_tok * tok_per_launch / (dom_avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(dom)

    res = {
        "metric": "SSD mixer fwd+bwd tokens/sec at d=1024, L=1M (segmented 64 x 16384)",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"mamba2 mixer hot path d_model=1024 (32x64 heads, d_state 128, "
                               f"conv 4), B={B}, L={L}, segments of {args.seg}, fwd+bwd",
                   "global_batch": B, "seq_len": L},
        "fwd_tokens_per_s": tokens / (ms_fwd * 1e-3),
        "ms_fwd": ms_fwd,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": dom,
                     "kernel_avg_ms": dom_avg_ms, "kernel_launches_per_step": dom_n / args.steps,
                     "alg_bytes_per_launch": per_tok * tok_per_launch},
        "path_roofline": {"alg_bytes_per_token": step_bytes, "roofline_tokens_per_s": roof_tok_s,
                          "frac": (tokens / (ms_step * 1e-3)) / roof_tok_s},
        "kernel_ms_per_step": {k: v[0] / args.steps for k, v in ktimes.items() if v[1]},
        "wall_s": wall,
    }

    # ---------------------------------------------------------------- CPU oracle baseline
    if args.cpu_sample > 0:
        from oracle import oracle as orc
        n = min(args.cpu_sample, L)
        f = synth.bf16_to_f32(synth.zxbcdt(d, args.seed, 0, n)).astype(np.float64)
        zz, xr, dtr = f[..., :hp], f[..., hp:hp + cd], f[..., hp + cd:hp + cd + H]
        p64 = {k: v.astype(np.float64) for k, v in synth.params(d, args.seed).items()}
        do = synth.bf16_to_f32(synth.dout(d, args.seed + 7, 0, n)).astype(np.float64)
        t = time.perf_counter()
        orc.mixer_fwd(xr, p64["conv_w"], p64["conv_b"], dtr, p64["A"], H, d.P, d.G, d.N,
                      dt_bias=p64["dt_bias"], D=p64["D"], z=zz.reshape(B, n, H, d.P))
        orc.mixer_bwd(xr, p64["conv_w"], p64["conv_b"], dtr, p64["A"], H, d.P, d.G, d.N,
                      do.reshape(B, n, H, d.P), dt_bias=p64["dt_bias"], D=p64["D"],
                      z=zz.reshape(B, n, H, d.P))
        sec = time.perf_counter() - t
        res["cpu_baseline"] = {"value": B * n / sec, "unit": "tokens/s", "cores": orc.num_threads(),
                               "kind": "oracle",
                               "sample": f"fwd+bwd over the first {n} tokens of the same workload "
                                         f"(fp64, {sec:.1f} s)"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
