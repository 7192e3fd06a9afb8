"""Benchmark of the Mamba-2 mixer hot path on one MI355X.

Headline step = one pass of the whole hot path over one batch: the forward over L
tokens (causal conv1d + SiLU -> chunked SSD -> SiLU(z) gate, keeping only the (h,
conv buffer) checkpoints every `seg` tokens), then the backward segment by segment in
reverse (recompute from the checkpoint, all gradients).  Workload: d_model 1024
shapes (32 heads x 64, d_state 128, conv 4), batch 1, L = 1,048,576 tokens as 64
segments of 16,384, bf16 I/O, seeded synthetic in_proj rows (see synth.py).

Prints one JSON line: tokens/s of that step (value), per-step median / min, the
forward alone with its own roofline, the per-kernel device times, the roofline of the
dominant kernel (HIP events on the launch stream), the path-level roofline, and extra
measurements that are not the headline:
  c4       the batched 2.7B-style shapes (B = 16, L = 4096, 80 heads), fwd + bwd
  c1_mixer in_proj -> hot path -> out_proj at L = 8192 (MFMA projections; the working
           set fits the 256 MB last-level cache)
  decode   one-token streaming decode latency at d_model 1024 and the 80-head shapes
           (per call from Python, and per step replayed from a HIP graph)
  magc     peak memory and training rate of a 48-block stack under multi-axis
           gradient checkpointing
  copy_ceiling  a plain 4 GiB device copy and fill, the practical HBM ceiling
and the fp64 oracle timed on a bounded prefix on the host cores (all of them, and one).
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--L", type=int, default=1 << 20)
    ap.add_argument("--seg", type=int, default=16384)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample", type=int, default=49152, help="oracle prefix tokens (0 = skip)")
    ap.add_argument("--cpu-sample-1t", type=int, default=4096,
                    help="oracle prefix tokens for the one-thread figure (0 = skip)")
    ap.add_argument("--extras", type=int, default=1, help="0 = headline step only")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for counter runs: one 256 MiB device copy (byte-counter calibration), "
                         "then two fwd+bwd passes over a single segment; prints no JSON")
    ap.add_argument("--oracle-only", type=int, default=0, help=argparse.SUPPRESS)
    return ap.parse_args()


COPY_BYTES = 256 << 20
# HBM bytes of the dominant kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of
# `bench.py --pmc-probe` (see the report for the commands and the copy calibration)
TRAFFIC_REPORT = os.path.join(ROOT, "profiles", "bwd_main_seg16k_hbm_bytes.md")
KERNEL_SYMBOL = {"bwd_main": "bwd_main_kernel", "walk_out": "walk_kernel", "walk_state": "walk_kernel",
                 "conv_bwd": "conv_bwd_kernel"}
FWD_KINDS = {"prepass", "walk_state", "scan", "walk_out", "conv_state_out"}


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


def hot_bytes(d):
    """Algorithmic bytes per token (each input read once, each output written once):
    forward = xBC raw + z + dt in, out; backward = the forward's inputs + dout in,
    dxBC + dz + ddt out."""
    es = 2
    fwd = es * (d.cd + 2 * d.hp + d.H)
    bwd = es * (d.cd + 2 * d.hp + d.H) + es * (d.cd + d.hp + d.H)
    return fwd, bwd


def timed(fn, steps, stream):
    """Per-call device times (ms) of `steps` back-to-back calls, HIP events on `stream`."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def oracle_sample(n: int, seed: int) -> dict:
    """fp64 oracle fwd + bwd over the first n tokens of the headline workload."""
    import numpy as np

    from oracle import oracle as orc
    from selective_state_space_15_amd import synth
    d = synth.CONFIGS["c2"]
    B, H, hp, cd = d.B, d.H, d.hp, d.cd
    f = synth.bf16_to_f32(synth.zxbcdt(d, seed, 0, n)).astype(np.float64)
    zz, xr, dtr = f[..., :hp], f[..., hp:hp + cd], f[..., hp + cd:hp + cd + H]
    p64 = {k: v.astype(np.float64) for k, v in synth.params(d, seed).items()}
    do = synth.bf16_to_f32(synth.dout(d, seed + 7, 0, n)).astype(np.float64)
    t = time.perf_counter()
    orc.mixer_fwd(xr, p64["conv_w"], p64["conv_b"], dtr, p64["A"], H, d.P, d.G, d.N,
                  dt_bias=p64["dt_bias"], D=p64["D"], z=zz.reshape(B, n, H, d.P))
    orc.mixer_bwd(xr, p64["conv_w"], p64["conv_b"], dtr, p64["A"], H, d.P, d.G, d.N,
                  do.reshape(B, n, H, d.P), dt_bias=p64["dt_bias"], D=p64["D"],
                  z=zz.reshape(B, n, H, d.P))
    sec = time.perf_counter() - t
    return {"value": B * n / sec, "unit": "tokens/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"fwd+bwd over the first {n} tokens of the same workload (fp64, {sec:.1f} s)"}


def main():
    args = parse()
    if args.oracle_only:
        print(json.dumps(oracle_sample(args.oracle_only, args.seed)), flush=True)
        return
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
        # the mixer projections at the d_model 1024 shapes (in_proj and out_proj, L = 8192)
        c1 = synth.CONFIGS["c1"]
        u = torch.randn(c1.L, c1.d_model, device=dev).to(torch.bfloat16)
        w_in = (0.02 * torch.randn(c1.d_in_proj, c1.d_model, device=dev)).to(torch.bfloat16)
        zxp = torch.empty(c1.L, c1.d_in_proj, dtype=torch.bfloat16, device=dev)
        w_out = (0.02 * torch.randn(c1.d_model, c1.hp, device=dev)).to(torch.bfloat16)
        fin = torch.empty(c1.L, c1.d_model, dtype=torch.bfloat16, device=dev)
        for _ in range(2):
            bd.mixer_proj(u, w_in, zxp)
            bd.mixer_proj(zxp[:, :c1.hp], w_out, fin)
        torch.cuda.synchronize()
        print("pmc probe done", flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed steps
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    per_step = timed(step, args.steps, stream)
    wall = time.perf_counter() - t_wall
    ms_step = sum(per_step) / args.steps
    print(f"[bench] headline: {ms_step:.2f} ms/step", file=sys.stderr, flush=True)

    # forward alone (same launches), for the forward-only rate
    ms_fwd = float(np.mean(timed(fwd, args.steps, stream)))

    # one more set of steps with per-kernel HIP events (library instrumentation, same stream)
    bd.ssd_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ktimes = bd.ssd_timing_read()
    bd.ssd_timing_enable(False)

    tokens = B * L
    fwd_bytes, bwd_bytes = hot_bytes(d)
    step_bytes = fwd_bytes + bwd_bytes
    roof_tok_s = HBM_PEAK_GBS * 1e9 / step_bytes
    # dominant kernel: the largest summed device time; its algorithmic bytes per
    # launch = the per-token bytes of its pass x the tokens one launch covers
    dom = max(ktimes, key=lambda k: ktimes[k][0])
    dom_ms, dom_n = ktimes[dom]
    dom_avg_ms = dom_ms / max(dom_n, 1)
    if dom in FWD_KINDS:
        per_tok, tok_per_launch = fwd_bytes, tokens
    else:
        per_tok, tok_per_launch = bwd_bytes, B * args.seg
    achieved = per_tok * tok_per_launch / (dom_avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(dom)
    fwd_gbs = fwd_bytes * tokens / (ms_fwd * 1e-3) / 1e9

    res = {
        "metric": "SSD mixer fwd+bwd tokens/sec at d=1024, L=1M (segmented 64 x 16384)",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": float(np.median(per_step)),
        "ms_per_step_min": float(np.min(per_step)),
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
        "fwd_roofline": {"bound": "hbm", "achieved": fwd_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": fwd_gbs / HBM_PEAK_GBS, "alg_bytes_per_token": fwd_bytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": dom,
                     "kernel_avg_ms": dom_avg_ms, "kernel_launches_per_step": dom_n / args.steps,
                     "alg_bytes_per_launch": per_tok * tok_per_launch},
        "path_roofline": {"alg_bytes_per_token": step_bytes, "roofline_tokens_per_s": roof_tok_s,
                          "frac": (tokens / (ms_step * 1e-3)) / roof_tok_s},
        "kernel_ms_per_step": {k: v[0] / args.steps for k, v in ktimes.items() if v[1]},
        "wall_s": wall,
    }
    del zx, dout, out, fws, bws, g
    torch.cuda.empty_cache()

    if args.extras:
        res["c4"] = bench_c4(args, stream)
        print("[bench] c4 done", file=sys.stderr, flush=True)
        res["c1_mixer"] = bench_c1_mixer(args, stream)
        print("[bench] c1 mixer done", file=sys.stderr, flush=True)
        res["decode"] = bench_decode(args, stream)
        print("[bench] decode done", file=sys.stderr, flush=True)
        res["magc"] = bench_magc(args, stream)
        print("[bench] magc done", file=sys.stderr, flush=True)
        res["copy_ceiling"] = bench_copy(stream)
        print("[bench] copy ceiling done", file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- CPU oracle baseline
    if args.cpu_sample > 0:
        res["cpu_baseline"] = oracle_sample(min(args.cpu_sample, L), args.seed)
    if args.cpu_sample_1t > 0:
        env = dict(os.environ, OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-only",
                            str(args.cpu_sample_1t), "--seed", str(args.seed)],
                           capture_output=True, text=True, env=env, timeout=600)
        if r.returncode == 0:
            res["cpu_baseline_1thread"] = json.loads(r.stdout.strip().splitlines()[-1])
    print(json.dumps(res), flush=True)


def bench_c4(args, stream):
    """Batched 2.7B-style hot path (B=16, L=4096, 80 heads x 64, d_state 128), one
    forward and one backward over the whole batch per step."""
    import numpy as np
    import torch

    from selective_state_space_15_amd import binding as bd
    from selective_state_space_15_amd import synth
    d = synth.CONFIGS["c4"]
    dev = stream.device
    B, L, H, hp, cd = d.B, d.L, d.H, d.hp, d.cd
    zx = torch.from_numpy(synth.zxbcdt(d, args.seed).view(np.int16)).to(dev).view(torch.bfloat16)
    dout = torch.from_numpy(synth.dout(d, args.seed + 7).view(np.int16)).to(dev).view(torch.bfloat16)
    p = {k: torch.from_numpy(v).to(dev) for k, v in synth.params(d, args.seed).items()}
    z, xbc, dt = zx[..., :hp], zx[..., hp:hp + cd], zx[..., hp + cd:hp + cd + H]
    dims = bd.make_dims(B, L, H, d.P, d.N, d.G, 0, d.K)
    out = torch.empty(B, L, hp, dtype=torch.bfloat16, device=dev)
    fws = torch.empty(max(bd.ssd_fwd_workspace(dims, bd.SSD_BF16), 1), dtype=torch.uint8, device=dev)
    bws = torch.empty(max(bd.ssd_bwd_workspace(dims, bd.SSD_BF16), 1), dtype=torch.uint8, device=dev)
    dxbc = torch.empty(B, L, cd, dtype=torch.bfloat16, device=dev)
    ddt = torch.empty(B, L, H, dtype=torch.bfloat16, device=dev)
    dz = torch.empty(B, L, hp, dtype=torch.bfloat16, device=dev)
    gp = {k: torch.empty(H, device=dev) for k in ("dA", "dD", "ddt_bias")}
    dcw, dcb = torch.empty(cd, d.K, device=dev), torch.empty(cd, device=dev)

    def fwd():
        bd.ssd_fwd(dims, xbc, p["A"], dt, out, conv_w=p["conv_w"], conv_b=p["conv_b"],
                   dt_bias=p["dt_bias"], D=p["D"], z=z, ws=fws)

    def step():
        fwd()
        bd.ssd_bwd(dims, xbc, p["A"], dt, dout, dxbc, ddt, gp["dA"], conv_w=p["conv_w"],
                   conv_b=p["conv_b"], dt_bias=p["dt_bias"], D=p["D"], z=z, dz=dz, dD=gp["dD"],
                   ddt_bias=gp["ddt_bias"], dconv_w=dcw, dconv_b=dcb, ws=bws)

    for _ in range(2):
        step()
    n = max(args.steps, 5)
    ms = timed(step, n, stream)
    msf = timed(fwd, n, stream)
    fb, bb = hot_bytes(d)
    tok = B * L
    med, medf = float(np.median(ms)), float(np.median(msf))
    gbs = (fb + bb) * tok / (med * 1e-3) / 1e9
    gbsf = fb * tok / (medf * 1e-3) / 1e9
    # the full block around it (RMSNorm, in_proj, hot path, gated RMSNorm, out_proj,
    # residual), forward + backward with every parameter gradient
    from selective_state_space_15_amd import block
    del zx, dout, out, fws, bws, dxbc, ddt, dz
    torch.cuda.empty_cache()
    sh = block.Shape(d.d_model, H, d.P, d.N, d.G, d.K)
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    wt = synth.mixer_weights(d, args.seed)
    w = block.Weights(w_in=bits(wt["w_in"]), w_out=bits(wt["w_out"]), norm_in=torch.from_numpy(wt["norm_in"]).to(dev),
                      norm_out=torch.from_numpy(wt["norm_out"]).to(dev), conv_w=p["conv_w"], conv_b=p["conv_b"],
                      A=p["A"], D=p["D"], dt_bias=p["dt_bias"])
    u = bits(synth.tokens(d, args.seed))
    dF = bits(synth.dfinal(d, args.seed))
    fin, du = torch.empty_like(u), torch.empty_like(u)
    sc = block.Scratch(sh, B, L, dev)
    grads = block.zero_grads(w)

    def blk():
        block.block_fwd(sh, w, u, fin, sc)
        block.block_bwd(sh, w, u, dF, du, grads, sc, accumulate=False)

    blk()
    msb = float(np.median(timed(blk, n, stream)))
    bd.ssd_timing_enable(True)
    blk()
    torch.cuda.synchronize()
    kt = bd.ssd_timing_read()
    bd.ssd_timing_enable(False)
    lin_ms = kt["linear"][0]
    gemm_flops = 3 * 2.0 * tok * d.d_model * (d.d_in_proj + hp)  # forward, input and weight gradients
    block_res = {"tokens_per_s": tok / (msb * 1e-3), "ms_per_step_median": msb,
                 "projection_ms": lin_ms, "projection_tflops": gemm_flops / (lin_ms * 1e-3) / 1e12,
                 "note": "forward + backward of the full block; the backward recomputes the block's forward"}
    return {"workload": f"hot path fwd+bwd, 2.7B-style shapes: B={B}, L={L}, {H}x{d.P} heads, "
                        f"d_state {d.N}, conv {d.K}, bf16",
            "tokens_per_s": tok / (med * 1e-3), "ms_per_step_median": med, "ms_per_step_min": min(ms),
            "fwd_tokens_per_s": tok / (medf * 1e-3), "ms_fwd_median": medf,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "alg_bytes_per_token": fb + bb},
            "fwd_roofline": {"bound": "hbm", "achieved": gbsf, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": gbsf / HBM_PEAK_GBS, "alg_bytes_per_token": fb},
            "full_block": block_res}


def bench_c1_mixer(args, stream):
    """in_proj (mixer_proj) -> ssd_fwd -> out_proj (mixer_proj) at the d_model 1024
    shapes, L = 8192; the projections' flops against the bf16 MFMA peak."""
    import numpy as np
    import torch

    from selective_state_space_15_amd import binding as bd
    from selective_state_space_15_amd import synth
    d = synth.CONFIGS["c1"]
    dev = stream.device
    B, L, H, hp, cd, dm, dip = d.B, d.L, d.H, d.hp, d.cd, d.d_model, d.d_in_proj
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    u = bits(synth.tokens(d, args.seed)).view(B * L, dm)
    w = synth.mixer_weights(d, args.seed)
    w_in, w_out = bits(w["w_in"]), bits(w["w_out"])
    p = {k: torch.from_numpy(v).to(dev) for k, v in synth.params(d, args.seed).items()}
    zx = torch.empty(B, L, dip, dtype=torch.bfloat16, device=dev)
    z, xbc, dt = zx[..., :hp], zx[..., hp:hp + cd], zx[..., hp + cd:hp + cd + H]
    out = torch.empty(B, L, hp, dtype=torch.bfloat16, device=dev)
    final = torch.empty(B * L, dm, dtype=torch.bfloat16, device=dev)
    dims = bd.make_dims(B, L, H, d.P, d.N, d.G, 0, d.K)
    fws = torch.empty(max(bd.ssd_fwd_workspace(dims, bd.SSD_BF16), 1), dtype=torch.uint8, device=dev)

    def in_proj():
        bd.mixer_proj(u, w_in, zx.view(B * L, dip))

    def hot():
        bd.ssd_fwd(dims, xbc, p["A"], dt, out, conv_w=p["conv_w"], conv_b=p["conv_b"],
                   dt_bias=p["dt_bias"], D=p["D"], z=z, ws=fws)

    def out_proj():
        bd.mixer_proj(out.view(B * L, hp), w_out, final)

    def mixer():
        in_proj()
        hot()
        out_proj()

    for _ in range(3):
        mixer()
    n = max(args.steps, 20)
    t_mix = float(np.median(timed(mixer, n, stream)))
    t_in = float(np.median(timed(in_proj, n, stream)))
    t_out = float(np.median(timed(out_proj, n, stream)))
    t_hot = float(np.median(timed(hot, n, stream)))
    # context: the vendor library (torch.matmul -> hipBLASLt) on the same two products
    # (plain products, no fused epilogue; the weights pre-transposed once)
    w_in_t, w_out_t = w_in.t().contiguous(), w_out.t().contiguous()
    out2 = out.view(B * L, hp)
    t_in_lib = float(np.median(timed(lambda: torch.matmul(u, w_in_t, out=zx.view(B * L, dip)), n, stream)))
    t_out_lib = float(np.median(timed(lambda: torch.matmul(out2, w_out_t, out=final), n, stream)))
    tok = B * L
    hot_fwd_bytes = hot_bytes(d)[0]
    hot_gbs = hot_fwd_bytes * tok / (t_hot * 1e-3) / 1e9
    f_in, f_out = 2.0 * tok * dm * dip, 2.0 * tok * hp * dm
    tf_in, tf_out = f_in / (t_in * 1e-3) / 1e12, f_out / (t_out * 1e-3) / 1e12
    tf = (f_in + f_out) / ((t_in + t_out) * 1e-3) / 1e12
    return {"workload": f"mixer forward in_proj -> hot path -> out_proj, d_model {dm}, B={B}, L={L}, bf16 "
                        "(working set cache-resident)",
            "tokens_per_s": tok / (t_mix * 1e-3), "ms_median": t_mix,
            "in_proj_ms": t_in, "out_proj_ms": t_out,
            "hot_path_fwd": {"tokens_per_s": tok / (t_hot * 1e-3), "ms_median": t_hot,
                             "roofline": {"bound": "hbm", "achieved": hot_gbs, "peak": HBM_PEAK_GBS,
                                          "unit": "GB/s", "frac": hot_gbs / HBM_PEAK_GBS,
                                          "alg_bytes_per_token": hot_fwd_bytes},
                             "note": "ssd_fwd alone (B/C conv and dt pre-passes, both walks, the "
                                     "sub-segment scan) on the in_proj rows above, back to back; "
                                     "the 105 MB working set stays in the 256 MB MALL"},
            "gemm_roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                              "frac": tf / MFMA_BF16_PEAK_TFS, "in_proj_tflops": tf_in,
                              "out_proj_tflops": tf_out, "flops_per_token": (f_in + f_out) / tok,
                              "hipblaslt_in_proj_tflops": f_in / (t_in_lib * 1e-3) / 1e12,
                              "hipblaslt_out_proj_tflops": f_out / (t_out_lib * 1e-3) / 1e12}}


def bench_decode(args, stream):
    """One-token streaming decode (ssd_decode, T = 1 per call, carried state), at the
    d_model 1024 shapes (B = 1) and the 80-head shapes (B = 16)."""
    import numpy as np
    import torch

    from selective_state_space_15_amd import binding as bd
    from selective_state_space_15_amd import synth
    dev = stream.device
    res = {}
    for name, d in (("d1024_b1", synth.CONFIGS["c1"].with_(L=256)), ("d2560_b16", synth.CONFIGS["c4"].with_(L=64))):
        B, T, H, hp, cd = d.B, d.L, d.H, d.hp, d.cd
        zx = torch.from_numpy(synth.zxbcdt(d, args.seed).view(np.int16)).to(dev).view(torch.bfloat16)
        p = {k: torch.from_numpy(v).to(dev) for k, v in synth.params(d, args.seed).items()}
        z, xbc, dt = zx[..., :hp], zx[..., hp:hp + cd], zx[..., hp + cd:hp + cd + H]
        h = torch.zeros(B, H, d.P, d.N, device=dev)
        cs = [torch.zeros(B, d.K - 1, cd, dtype=torch.bfloat16, device=dev) for _ in range(2)]
        out = torch.empty(B, T, hp, dtype=torch.bfloat16, device=dev)
        dims = bd.make_dims(B, 1, H, d.P, d.N, d.G, 0, d.K)
        state = {"t": 0}

        def one():
            t = state["t"] % T
            i = state["t"] % 2
            bd.ssd_decode(dims, xbc[:, t:t + 1], p["A"], dt[:, t:t + 1], out[:, t:t + 1], h,
                          conv_w=p["conv_w"], conv_b=p["conv_b"], conv_state_in=cs[i],
                          conv_state_out=cs[1 - i], dt_bias=p["dt_bias"], D=p["D"], z=z[:, t:t + 1],
                          h_in=h)
            state["t"] += 1

        for _ in range(10):
            one()
        ms = timed(one, 200, stream)
        med = float(np.median(ms))
        bd.ssd_timing_enable(True)
        for _ in range(200):
            one()
        torch.cuda.synchronize()
        kt = bd.ssd_timing_read()["decode"]
        bd.ssd_timing_enable(False)
        # the serving-loop form: S one-token steps captured once in a HIP graph and
        # replayed (no Python or per-call host work between the steps)
        S = 32
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            one()
        stream.wait_stream(side)
        state["t"] = 0
        with torch.cuda.graph(graph):
            for _ in range(S):
                one()
        graph.replay()
        g_ms = timed(graph.replay, 20, torch.cuda.current_stream())
        g_us = float(np.median(g_ms)) * 1e3 / S
        state_bytes = 2 * B * H * d.P * d.N * 4
        k_us = kt[0] / max(kt[1], 1) * 1e3
        res[name] = {"batch": B, "heads": H, "us_per_call_median": med * 1e3,
                     "kernel_us_avg": k_us, "tokens_per_s": B / (med * 1e-3),
                     "us_per_token_graph": g_us, "tokens_per_s_graph": B / (g_us * 1e-6),
                     "state_bytes_per_call": state_bytes,
                     "kernel_state_gbs": state_bytes / (k_us * 1e-6) / 1e9,
                     "note": "one call per token step from Python (host launch overhead included in "
                             "us_per_call); us_per_token_graph: 32 such steps captured in a HIP graph "
                             "and replayed; the kernel reads and writes the state once per call"}
    return res


def bench_copy(stream):
    """The practical HBM ceiling: a plain device copy of 4 GiB (reads plus writes) and a
    4 GiB fill, median of 5 (torch's own copy and fill kernels)."""
    import numpy as np
    import torch
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device=stream.device)
    dst = torch.empty_like(src)
    src.fill_(1)
    cp = timed(lambda: dst.copy_(src), 5, stream)
    fl = timed(lambda: dst.fill_(2), 5, stream)
    del src, dst
    torch.cuda.empty_cache()
    c_ms, f_ms = float(np.median(cp)), float(np.median(fl))
    return {"copy_bytes": n, "copy_GBs": 2 * n / (c_ms * 1e-3) / 1e9, "fill_GBs": n / (f_ms * 1e-3) / 1e9,
            "peak_GBs": 8000.0, "note": "reads plus writes of a 4 GiB device copy; a context ceiling, "
                                         "the rooflines use the published 8 TB/s"}


def bench_magc(args, stream):
    """Multi-axis gradient checkpointing of a 48-layer stack of full blocks at d_model 1024
    (random weights): for S = 16K .. 128K tokens, the intervals (l, s) minimising the
    memory model, the measured peak activation memory of one training pass (forward,
    backward, all parameter gradients) next to the model, and the pass's time."""
    import numpy as np
    import torch

    from selective_state_space_15_amd import block, magc, synth
    dev = stream.device
    d = synth.CONFIGS["c1"]
    n_layers = 48
    sh = block.Shape(d.d_model, d.H, d.P, d.N, d.G, d.K)
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    layers = []
    for i in range(n_layers):
        w, p = synth.mixer_weights(d, args.seed + i), synth.params(d, args.seed + i)
        layers.append(block.Weights(w_in=bits(w["w_in"]), w_out=bits(w["w_out"]), norm_in=f32(w["norm_in"]),
                                    norm_out=f32(w["norm_out"]), conv_w=f32(p["conv_w"]), conv_b=f32(p["conv_b"]),
                                    A=f32(p["A"]), D=f32(p["D"]), dt_bias=f32(p["dt_bias"])))
    grads = [block.zero_grads(w) for w in layers]
    rows = []
    for S in (16384, 32768, 65536, 131072):
        l, s = magc.best_intervals(sh, n_layers, S)
        dS = d.with_(L=S)
        u, dF = bits(synth.tokens(dS, args.seed)), bits(synth.dfinal(dS, args.seed))
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        t = time.perf_counter()
        sc = block.Scratch(sh, 1, s, dev)
        _, ck = magc.stack_forward(sh, layers, u, sc, l, s)
        magc.stack_backward(sh, layers, ck, dF, grads, sc, l, s)
        torch.cuda.synchronize()
        sec = time.perf_counter() - t
        peak = torch.cuda.max_memory_allocated() - base
        model = sum(magc.model_bytes(sh, n_layers, S, l, s).values())
        rows.append({"S": S, "l": l, "s": s, "peak_MiB": peak / 2**20, "model_MiB": model / 2**20,
                     "train_pass_s": sec, "tokens_per_s": S / sec})
        del u, dF, sc, ck
    ratios = [rows[i + 1]["peak_MiB"] / rows[i]["peak_MiB"] for i in range(len(rows) - 1)]
    return {"workload": f"{n_layers}-layer stack of full Mamba-2 blocks, d_model 1024 (32x64 heads, d_state 128), "
                        "batch 1, bf16, forward + backward with multi-axis gradient checkpointing",
            "rows": rows, "peak_ratio_per_doubling": ratios}


if __name__ == "__main__":
    main()
