#!/usr/bin/env python3
"""One training step of one tensor-parallel shard of the parallel transformer
block with sliding-window attention, on one MI355X:

    ptb_forward + ptb_backward + lamb_step (over the shard's six parameter
    tensors, refreshing the bf16 weights the next forward reads)

timed with HIP events on the stream the library launches on.  The timed
steps call ptb_forward / ptb_backward / lamb_step whole, with events only at
their boundaries; a second set of K forward + backward passes goes through
the stage entry points (exactly what the whole calls execute) with an event
before each stage, which gives the per-stage times and the dominant kernel's
launch time for the roofline.

Prints ONE JSON line.  `value` is the block's model TFLOP/s, 6 * N * T FLOP
(N = matrix parameters of the shard, T = tokens; the 6N-per-token estimate of
the MegaScale study guide, ch.2 §2.1) over the measured fwd+bwd time; `mfu`
divides it by the bf16 dense MFMA peak; `lamb_gbps` is the LAMB step's
algorithmic bytes over its time.  `roofline` describes the dominant kernel
stage; `cpu_baseline` times the fp64 CPU oracle on one full step's forward and
backward of the same workload; `serial` times the serial pre-LN block (two
LayerNorms, four separate projections) on the same workload and weights, the
arrangement the PTB replaces.

    python bench.py [--steps K] [--warmup W] [--config 175b_w512]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "PTB+SWA layer fwd+bwd TFLOP/s & MFU at 175B TP=8 shard; LAMB step GB/s"
PEAK_BF16 = 2.5e15       # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12        # MI355X HBM3E, bytes/s
ROOT = os.path.dirname(os.path.abspath(__file__))


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", default="175b_w512")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip timing the fp64 CPU oracle")
    p.add_argument("--no-serial", action="store_true",
                   help="skip timing the serial pre-LN block on the same workload")
    p.add_argument("--no-lamb-shard", action="store_true",
                   help="skip timing one data-parallel rank's sharded LAMB")
    p.add_argument("--cpu-baseline-all", action="store_true",
                   help="also time the fp64 CPU oracle's forward + backward on every other "
                        "workload (minutes of host time; off by default)")
    p.add_argument("--no-extra-configs", action="store_true",
                   help="skip the forward + backward timings of the other workloads "
                        "(175b_w2048, small, 530b_w512)")
    p.add_argument("--out", default=None, help="also write the JSON line to this file")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run one plain device-to-device copy of MIB MiB and exit (the "
                        "reference kernel for scaling HBM byte counters)")
    return p.parse_args()


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4}))


def matrix_params(cfg):
    """Matrix parameters of the shard: w_in [3A + F, h] plus w_out [A + F, h]."""
    A, F = cfg.attn_width, cfg.ffn
    return (3 * A + F) * cfg.hidden + (A + F) * cfg.hidden


def model_flops(cfg):
    """6 * N * T: the model FLOPs of one forward + backward (2N + 4N per token)."""
    return 6.0 * matrix_params(cfg) * cfg.tokens


def stage_flops(cfg):
    """Algorithmic FLOPs of each stage (GEMMs 2*M*N*K; attention over the band)."""
    T, h, A, F = cfg.tokens, cfg.hidden, cfg.attn_width, cfg.ffn
    N1, K2 = 3 * A + F, A + F
    w = min(cfg.window, cfg.seq)
    pairs = (w * (w + 1) // 2 + (cfg.seq - w) * w) * cfg.batch * cfg.n_heads
    att_fwd = 4.0 * cfg.head_dim * pairs          # QK^T and PV
    return {
        "fwd.layernorm": 0.0,
        "fwd.gemm_in": 2.0 * T * N1 * h,
        "fwd.attention": att_fwd,
        "fwd.gemm_out": 2.0 * T * K2 * h,
        "bwd.gemm_dcat": 2.0 * T * K2 * h,
        "bwd.gemm_dw_out": 2.0 * K2 * h * T,
        "bwd.attention": 2.0 * att_fwd,           # dV, dP, dQ, dK (recompute not counted)
        "bwd.gemm_dw_in": 2.0 * N1 * h * T,
        "bwd.gemm_dxn": 2.0 * T * h * N1,
        "bwd.layernorm": 0.0,
    }


def lamb_bytes(params):
    """Algorithmic HBM bytes of one lamb_step: pass A reads w, g, m, v and
    writes m, v; pass B reads w, m, v, writes w (and the bf16 copy)."""
    total = 0
    for p in params:
        n = p["w"].numel()
        g = p["g"].element_size()
        total += n * (4 + g + 4 + 4 + 4 + 4)            # pass A
        total += n * (12 + 4 + (2 if p.get("w_bf16") is not None else 0))  # pass B
    return total


def lamb_bytes_headline(params):
    """The two-pass exact minimum of the step without the bf16 weight copy:
    38 B/param with bf16 gradients (pass A 22 B, pass B 16 B)."""
    total = 0
    for p in params:
        n = p["w"].numel()
        total += n * (4 + p["g"].element_size() + 4 + 4 + 4 + 4) + n * (12 + 4)
    return total


def ln_bytes(cfg):
    """HBM bytes the two LayerNorm stages must move (activations in the layer
    dtype, statistics and LN parameters in fp32).
    forward : read x; write xn, and for bf16 the residual xn - bf16(xn) that
              the compensated q/k pass reads; write mean, rstd
    backward: read x, dxn (and dy when the residual is on), mean, rstd,
              gamma; write dx, dgamma, dbeta
    The backward's per-workgroup partial column sums (written, then read by
    the fixed-order reduction) are extra traffic, reported separately."""
    T, h = cfg.tokens, cfg.hidden
    e = 2 if cfg.dtype == "bf16" else 4
    fwd = T * h * e + T * h * e + (T * h * 2 if e == 2 else 0) + 8 * T + 8 * h
    bwd = T * h * e * (3 if cfg.add_residual else 2) + T * h * e + 8 * T + 4 * h + 8 * h
    rows_per_block = 8
    nblk = -(-T // rows_per_block)
    partials = 2 * (2 * nblk * h * 4)
    return {"fwd": fwd, "bwd": bwd, "bwd_partials": partials}


def time_stages(shard, nfwd, nbwd, steps):
    """Mean milliseconds of each stage over `steps` forward + backward passes
    through the stage entry points, with a HIP event before each stage on the
    stream the library launches on (torch's current stream)."""
    import numpy as np
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nfwd + nbwd + 1)]
          for _ in range(steps)]
    for k in range(steps):
        i = 0
        for s in range(nfwd):
            ev[k][i].record(); i += 1
            shard.forward_stage(s)
        for s in range(nbwd):
            ev[k][i].record(); i += 1
            shard.backward_stage(s)
        ev[k][i].record()
    torch.cuda.synchronize()
    return [float(np.mean([ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(steps)]))
            for i in range(nfwd + nbwd)]


def roofline_for(cfg, per_stage):
    """The dominant stage (a GEMM) against the dense bf16 MFMA peak."""
    flops = stage_flops(cfg)
    dom = max((n for n in per_stage if n in flops and n != "lamb"), key=lambda n: per_stage[n])
    achieved = flops[dom] / (per_stage[dom] * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
            "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
            "frac": round(achieved / (PEAK_BF16 / 1e12), 4),
            "traffic": traffic_for(dom) if cfg.name == "175b_w512" else None,
            "flop_per_launch": flops[dom], "ms_per_launch": round(per_stage[dom], 4)}


def ln_rates(cfg, per_stage):
    lb = ln_bytes(cfg)
    f = lb["fwd"] / (per_stage["fwd.layernorm"] * 1e-3)
    b = lb["bwd"] / (per_stage["bwd.layernorm"] * 1e-3)
    m = (lb["bwd"] + lb["bwd_partials"]) / (per_stage["bwd.layernorm"] * 1e-3)
    return {"fwd_bytes": lb["fwd"], "fwd_gbps": round(f / 1e9, 1),
            "fwd_hbm_frac": round(f / PEAK_HBM, 4),
            "bwd_bytes": lb["bwd"], "bwd_gbps": round(b / 1e9, 1),
            "bwd_hbm_frac": round(b / PEAK_HBM, 4),
            "bwd_with_partials_gbps": round(m / 1e9, 1)}


def time_config(name, args):
    """Forward + backward of another workload: whole calls timed with events,
    then the per-stage breakdown, the dominant stage's roofline and the
    LayerNorm rates."""
    import numpy as np
    import torch
    from transformer_block_lamb_amd import binding as B
    from transformer_block_lamb_amd.device import PtbShard
    from transformer_block_lamb_amd.synth import CONFIGS, ptb_inputs
    cfg = CONFIGS[name]
    shard = PtbShard(cfg, ptb_inputs(cfg))
    for _ in range(args.warmup):
        shard.forward()
        shard.backward()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record()
        shard.forward()
        ev[k][1].record()
        shard.backward()
        ev[k][2].record()
    torch.cuda.synchronize()
    f = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    b = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    st = time_stages(shard, len(B.FWD_STAGES), len(B.BWD_STAGES), args.steps)
    names = [f"fwd.{n}" for n in B.FWD_STAGES] + [f"bwd.{n}" for n in B.BWD_STAGES]
    per_stage = dict(zip(names, st))
    mf = model_flops(cfg)
    ex = sum(stage_flops(cfg).values())
    out = {"workload": f"{cfg.name}: batch {cfg.batch}, seq {cfg.seq}, hidden {cfg.hidden}, "
                       f"{cfg.n_heads} heads x {cfg.head_dim}, ffn {cfg.ffn}, window "
                       f"{cfg.window}, {cfg.dtype}",
           "fwd_ms": round(f, 4), "bwd_ms": round(b, 4),
           "model_tflops": round(mf / ((f + b) * 1e-3) / 1e12, 2),
           "mfu": round(mf / ((f + b) * 1e-3) / PEAK_BF16, 4),
           "executed_tflops": round(ex / ((f + b) * 1e-3) / 1e12, 2),
           "stages_ms": {n: round(v, 4) for n, v in per_stage.items()},
           "roofline": roofline_for(cfg, per_stage),
           "layernorm": ln_rates(cfg, per_stage)}
    del shard
    torch.cuda.empty_cache()
    return out


def time_serial(cfg, inputs, args, ptb_ms):
    """Forward and backward of the serial pre-LN block on the same inputs and
    weights (LN2 with unit gamma, zero beta), timed like the PTB step."""
    import numpy as np
    import torch
    from transformer_block_lamb_amd.device import SerialShard
    from transformer_block_lamb_amd.synth import second_ln_params
    g2, b2 = second_ln_params(cfg)
    ser = SerialShard(cfg, inputs, g2, b2)
    for _ in range(args.warmup):
        ser.forward()
        ser.backward()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record()
        ser.forward()
        ev[k][1].record()
        ser.backward()
        ev[k][2].record()
    torch.cuda.synchronize()
    f = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    b = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    del ser
    return {"fwd_ms": round(f, 4), "bwd_ms": round(b, 4),
            "ptb_speedup": round((f + b) / ptb_ms, 4)}


def time_lamb_shard(params, args, dp=8):
    """One data-parallel rank's half-steps of ZeRO-2 sharded LAMB (rank 0 of
    `dp`, its 1/dp range of every tensor): lamb_shard_norms then
    lamb_shard_apply, called directly on the rank's descriptors.  The
    all-reduce of the 12 norms between them is a collective across ranks and
    is not part of the timed kernels (the rank's own norms stand in for the
    sum)."""
    import numpy as np
    import torch
    from transformer_block_lamb_amd import binding as B
    from transformer_block_lamb_amd.device import ShardedLamb
    from transformer_block_lamb_amd.synth import LAMB_HPARAMS
    hp = LAMB_HPARAMS
    sh = ShardedLamb(params, dp)
    R = sh.ranks[0]
    assert len(R["keep"]) == len(params)  # every tensor reaches rank 0
    norms = torch.empty(2 * len(params), dtype=torch.float64, device="cuda")
    ratios = torch.empty(len(params), dtype=torch.float32, device="cuda")

    def half_steps(it):
        B.lamb_shard_norms(R["desc"], hp["beta1"], hp["beta2"], hp["eps"], it, norms, R["scratch"])
        B.lamb_shard_apply(R["desc"], hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], it, norms,
                           ratios, R["scratch"])

    for it in range(1, args.warmup + 1):
        half_steps(it)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record()
        half_steps(args.warmup + 1 + k)
        ev[k][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    nb = lamb_bytes(R["params"])
    return {"dp": dp, "rank_params": int(sum(p["w"].numel() for p in R["params"])),
            "ms": round(ms, 4), "gbps": round(nb / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nb / (ms * 1e-3) / PEAK_HBM, 4)}


def cpu_baseline(cfg, inputs, mflops):
    """The fp64 oracle's forward + backward of one full step of the workload."""
    from oracle import ptb as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    d = O.dims_of(cfg)
    t0 = time.perf_counter()
    y, saved = O.ptb_forward(d, inputs["x"], inputs["gamma"], inputs["beta"], inputs["w_in"],
                             inputs["w_out"])
    O.ptb_backward(d, inputs["x"], inputs["gamma"], inputs["w_in"], inputs["w_out"], saved,
                   inputs["dy"])
    dt = time.perf_counter() - t0
    return {"value": round(mflops / dt / 1e12, 4), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"one full forward+backward of the {cfg.name} shard ({cfg.tokens} tokens) "
                      f"in fp64 numpy, model FLOPs 6*N*T over its wall time"}


# The sources the GEMM kernels are compiled from: counters taken from any
# other version of them no longer describe the kernels that run.
GEMM_SOURCES = ("gemm.hip", "common.h", "kernels.h")


def gemm_source_digest():
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, "transformer_block_lamb_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def traffic_for(kernel_stage):
    """HBM bytes per launch of the dominant stage from the committed counter
    summary, or None when absent or taken from a different kernel source."""
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("gemm_sources_sha256") != gemm_source_digest():
        return None
    return rec.get("stages", {}).get(kernel_stage)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's shard only: the tensor-parallel collectives are not "
              "part of this library, so --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch
    from transformer_block_lamb_amd import binding as B
    from transformer_block_lamb_amd.device import PtbShard
    from transformer_block_lamb_amd.synth import CONFIGS, LAMB_HPARAMS, ptb_inputs

    cfg = CONFIGS[args.config]
    inputs = ptb_inputs(cfg)
    shard = PtbShard(cfg, inputs)
    A, F = cfg.attn_width, cfg.ffn
    dev = "cuda"
    w_in_m = torch.from_numpy(inputs["w_in"]).to(dev)     # fp32 masters
    w_out_m = torch.from_numpy(inputs["w_out"]).to(dev)
    hp = LAMB_HPARAMS
    wd = hp["weight_decay"]

    def tensor(w, g, copy=None):
        return dict(w=w, g=g, m=torch.zeros_like(w), v=torch.zeros_like(w), w_bf16=copy,
                    weight_decay=wd)

    params = [tensor(w_in_m[:3 * A], shard.dw_in[:3 * A], shard.w_in[:3 * A]),     # W_qkv
              tensor(w_in_m[3 * A:], shard.dw_in[3 * A:], shard.w_in[3 * A:]),     # W_fc1
              tensor(w_out_m[:A], shard.dw_out[:A], shard.w_out[:A]),              # W_o
              tensor(w_out_m[A:], shard.dw_out[A:], shard.w_out[A:]),              # W_fc2
              tensor(shard.gamma, shard.dgamma), tensor(shard.beta, shard.dbeta)]
    desc = B.lamb_tensors(params)
    lscratch = torch.empty(B.lamb_scratch_bytes(desc), dtype=torch.uint8, device=dev)
    ratios = torch.empty(len(params), dtype=torch.float32, device=dev)

    names = [f"fwd.{n}" for n in B.FWD_STAGES] + [f"bwd.{n}" for n in B.BWD_STAGES] + ["lamb"]

    def step(it, events=None):
        """One training step through the library's whole calls."""
        if events is not None:
            events[0].record()
        shard.forward()
        if events is not None:
            events[1].record()
        shard.backward()
        if events is not None:
            events[2].record()
        B.lamb_step(desc, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], it, ratios, lscratch)
        if events is not None:
            events[3].record()

    for it in range(1, args.warmup + 1):
        step(it)
    torch.cuda.synchronize()

    # the timed region: K whole steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_wall = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + 1 + k, ev[k])
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    lamb_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    step_ms = float(np.mean([e[0].elapsed_time(e[3]) for e in ev]))
    fb_each = [e[0].elapsed_time(e[2]) for e in ev]

    # per-stage breakdown: K more forward + backward passes through the
    # stage entry points (the events between stages add about 1.5 us each,
    # so these stages sum to slightly more than fwd_ms + bwd_ms)
    nfb = len(B.FWD_STAGES) + len(B.BWD_STAGES)
    per_stage = dict(zip(names[:nfb], time_stages(shard, len(B.FWD_STAGES), len(B.BWD_STAGES),
                                                  args.steps)))
    per_stage["lamb"] = lamb_ms

    print(f"{cfg.name}: fwd+bwd {fwd_ms + bwd_ms:.4f} ms, lamb {lamb_ms:.4f} ms", file=sys.stderr,
          flush=True)
    serial = None
    if not args.no_serial:
        serial = time_serial(cfg, inputs, args, fwd_ms + bwd_ms)
    lamb_shard = None if args.no_lamb_shard else time_lamb_shard(params, args)

    flops = stage_flops(cfg)
    mflops = model_flops(cfg)
    value = mflops / ((fwd_ms + bwd_ms) * 1e-3) / 1e12
    executed = sum(flops.values()) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12
    lb = lamb_bytes(params)
    lb38 = lamb_bytes_headline(params)
    roofline = roofline_for(cfg, {n: v for n, v in per_stage.items() if n != "lamb"})
    extra = {}
    if not args.no_extra_configs:
        for name in ("175b_w2048", "small", "530b_w512"):
            if name != cfg.name:
                print(f"timing {name}", file=sys.stderr, flush=True)
                extra[name] = time_config(name, args)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, random init)",
        "config": {"workload": f"{cfg.name}: one TP=8 shard, batch {cfg.batch}, seq {cfg.seq}, "
                               f"hidden {cfg.hidden}, {cfg.n_heads} heads x {cfg.head_dim}, "
                               f"ffn {cfg.ffn}, window {cfg.window}; LAMB over its 6 tensors",
                   "global_batch": cfg.batch, "seq_len": cfg.seq, "parallelism": "tp8-shard"},
        "mfu": round(value / (PEAK_BF16 / 1e12), 4),
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4), "lamb_ms": round(lamb_ms, 4),
        "fwd_bwd_ms_median": round(float(np.median(fb_each)), 4),
        "fwd_bwd_ms_min": round(float(np.min(fb_each)), 4),
        # headline accounting: 38 B/param (two-pass exact minimum, bf16 g)
        "lamb_gbps": round(lb38 / (lamb_ms * 1e-3) / 1e9, 1),
        "lamb_hbm_frac": round(lb38 / (lamb_ms * 1e-3) / PEAK_HBM, 4),
        "lamb_bytes": lb38,
        # including the bf16 weight copy pass B also writes (40 B/param)
        "lamb_with_copy_gbps": round(lb / (lamb_ms * 1e-3) / 1e9, 1),
        "lamb_with_copy_hbm_frac": round(lb / (lamb_ms * 1e-3) / PEAK_HBM, 4),
        "lamb_with_copy_bytes": lb,
        "layernorm": ln_rates(cfg, per_stage),
        "executed_tflops": round(executed, 2),
        "wall_ms_per_step": round(t_wall * 1e3 / args.steps, 4),
        "stages_ms": {n: round(v, 4) for n, v in per_stage.items()},
        "roofline": roofline,
    }
    if extra:
        out["configs"] = extra
    if lamb_shard is not None:
        out["lamb_zero2_rank"] = lamb_shard
    if serial is not None:
        serial["model_tflops"] = round(mflops / ((serial["fwd_ms"] + serial["bwd_ms"]) * 1e-3)
                                       / 1e12, 2)
        out["serial"] = serial
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inputs, mflops)
        if args.cpu_baseline_all:
            from transformer_block_lamb_amd.synth import ptb_inputs as _inputs
            per = {}
            for name in ("tiny", "small", "175b_w2048", "530b_w512"):
                c = CONFIGS[name]
                per[name] = cpu_baseline(c, _inputs(c), model_flops(c))
                print(f"cpu baseline {name}: {per[name]['seconds']} s", file=sys.stderr, flush=True)
            out["cpu_baseline"]["per_config"] = per
    line = json.dumps(out)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
