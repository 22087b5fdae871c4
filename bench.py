#!/usr/bin/env python3
"""Benchmark of the fused weight-gradient + optimizer step (FORGE) on one MI355X.

A step is one pass of the hot path for each layer of the workload, on inputs
already resident in device memory: the input gradient dX = dY W (old weights),
then the fused dW = dY^T X + optimizer update of W and its moments. The default
workload is the q_proj-shaped layer (W 4096x4096 bf16, fp32 AdamW moments,
8192 tokens, stochastic rounding). `value` counts the algorithmic FLOPs of both
GEMMs of every step (4 * T * out * in per layer) over the timed wall time.
With --inputs fp8 the fused step reads X as E4M3 and dY as E5M2 codes, each with
one float32 scale (dgrad keeps bf16), and its roofline peak is the FP8 one.

Besides the JSON line's contract fields it reports:
  roofline      the fused kernel's achieved TFLOP/s (2*T*out*in per launch over its
                mean launch time, HIP events on the launch stream) against the MI355X
                dense peak of its input dtype;
  cpu_baseline  the float64 oracle timed on the host on a bounded sample;
  unfused       the two-phase baseline (dW stored as fp32, separate optimizer pass),
                its time, the fused speedup and the transient memory each needs.
"""
from __future__ import annotations

import argparse
import functools
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused wgrad+AdamW TFLOP/s & ms/layer (Llama-8B shapes), % MFMA peak, dW HBM bytes"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "fp8": 5000.0}   # MI355X dense MFMA peaks
HBM_GBS = 8000.0


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "optimizer_gemm_amd", "csrc")
    names = ["forge_internal.h", "forge_gemm_kernel.h", "forge_wgrad.hip"]
    names += sorted(f for f in os.listdir(csrc) if f.startswith("forge_gemm") and f.endswith(".hip"))
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="q_proj_8192",
                   help="q_proj_8192 | llama8b_layer_8192 | llama8b_tp8_8192 | down_q8_16384 | qwen14b_mlp_4096 | "
                        "fp32_256 | stack | llama8b_mlp_train_8192 (training steps through autograd)")
    p.add_argument("--blocks", type=int, default=4,
                   help="llama8b_mlp_train_8192: number of SwiGLU MLP blocks in the model")
    p.add_argument("--cold-calls", type=int, default=10,
                   help="fused calls of the first layer timed after a 1 GiB write that evicts the memory-side cache")
    p.add_argument("--group", action="store_true",
                   help="decoder-layer workloads (llama8b_layer_8192, llama8b_tp8_8192, stack) and "
                        "llama8b_mlp_train_8192: the layers that share an input (q, k, v; gate, up) take one "
                        "grouped fused step (forge_linear_wgrad_step_group) on one X")
    p.add_argument("--opt", default="adamw")
    p.add_argument("--states", default=None, choices=("f32", "bf16", "q8", "q8dyn"),
                   help="moment storage format (default: the workload's)")
    p.add_argument("--inputs", default="native", choices=("native", "fp8"),
                   help="fp8: the fused step reads X as E4M3 and dY as E5M2 codes with per-tensor scales "
                        "(W and dgrad stay bf16)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-unfused", action="store_true")
    p.add_argument("--no-mfma-peak", action="store_true",
                   help="skip the MFMA-throughput microbenchmark (achieved bf16 peak beside the data-sheet one)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain 1 GiB device copy (3 times) to calibrate HBM byte counters")
    p.add_argument("--record-traffic", nargs=4, metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB"),
                   help="no GPU work: turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE databases of this bench (and of "
                        "--calibrate-copy) into profiles/traffic_<workload>.json for the current kernel source")
    return p.parse_args()


def _counter_means(db: str, counter: str) -> dict:
    """Mean per dispatch of one counter, per kernel name, from a rocprofv3 results database."""
    import sqlite3
    con = sqlite3.connect(db)
    cols = [d[1] for d in con.execute("pragma table_info(counters_collection)")]
    acc = {}
    for row in con.execute("select * from counters_collection"):
        d = dict(zip(cols, row))
        if d["counter_name"] == counter:
            acc.setdefault(d["kernel_name"], []).append(float(d["value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _traffic_name(args) -> str:
    return args.workload + ("_fp8" if args.inputs == "fp8" else "") + (f"_{args.states}" if args.states else "")


def record_traffic(args) -> int:
    """HBM bytes per launch of the fused kernel: counters in KiB, scaled by what the same
    counters read for a copy of known size."""
    fetch_db, write_db, cfetch_db, cwrite_db = args.record_traffic
    copy_bytes = 4 * (1 << 28)
    cf = [v for k, v in _counter_means(cfetch_db, "FETCH_SIZE").items() if "copyBuffer" in k]
    cw = [v for k, v in _counter_means(cwrite_db, "WRITE_SIZE").items() if "copyBuffer" in k]
    if not cf or not cw:
        print("no copy kernel in the calibration databases", file=sys.stderr)
        return 1
    f_scale, w_scale = copy_bytes / (cf[0] * 1024), copy_bytes / (cw[0] * 1024)

    def fused(means):
        # the optimizer epilogue is template argument EPI = 1 of gemm_kernel
        hits = [v for k, v in means.items() if "gemm_kernel<" in k and ">, 1, " in k]
        if len(hits) != 1:
            raise SystemExit(f"expected one fused kernel in the counters, found {len(hits)}")
        return hits[0] * 1024

    fetch = fused(_counter_means(fetch_db, "FETCH_SIZE")) * f_scale
    write = fused(_counter_means(write_db, "WRITE_SIZE")) * w_scale
    rec = {"workload": args.workload, "opt": args.opt, "kernel_source_hash": kernel_source_hash(),
           "bytes_per_launch": int(round(fetch + write)), "fetch_bytes": int(round(fetch)),
           "write_bytes": int(round(write)), "fetch_scale": f_scale, "write_scale": w_scale,
           "inputs": args.inputs, "source": f"profiles/wgrad_fused_{_traffic_name(args)}.md"}
    out = os.path.join(ROOT, "profiles", f"traffic_{_traffic_name(args)}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return 0


def calibrate_copy() -> int:
    """A plain copy of known size: 1 GiB read + 1 GiB written per dispatch."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_dispatch": 4 * n, "bytes_written_per_dispatch": 4 * n}))
    return 0


def cpu_baseline(spec, wl_config, opt, io, sr, fp8):
    """The float64 oracle (dgrad + fused step) timed on the host on a bounded sample of one layer."""
    import numpy as np
    from oracle import gemm, optim, step as ostep
    from synth import draw_layer_batch, draw_layer_batch_fp8, draw_layer_init, f32_from_bf16_bits
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:
        cores = os.cpu_count() or 1
    X, dY = draw_layer_batch(wl_config, 0, 1, spec)
    W0 = draw_layer_init(wl_config, 0, spec)
    n_rows = spec.out if spec.P <= 32 * 1024 * 1024 else 1024
    rows = np.arange(n_rows)
    hp = optim.hyper(opt)
    slots = optim.SLOTS[opt]
    z = np.zeros((n_rows, spec.inn), np.float32)
    dYw = f32_from_bf16_bits(dY) if io == "bf16" else dY
    Ww = f32_from_bf16_bits(W0[rows]) if io == "bf16" else W0[rows]
    fkw, Xs, dYs = {}, X, dY
    if fp8:
        Xs, dYs, sx, sd = draw_layer_batch_fp8(wl_config, 0, 1, spec, "e4m3", "e5m2")
        fkw = dict(x_fmt="e4m3", dy_fmt="e5m2", x_scale=sx, dy_scale=sd)
    reps, times = 4, []  # about 10 s of host work on the q_proj layer
    for _ in range(reps):
        c0 = time.perf_counter()
        gemm.dgrad(dYw[:, rows], Ww)  # dX contribution of the sampled rows of W
        ostep.wgrad_step(opt, Xs, dYs, W0[rows], z if "m" in slots else None, z if "v" in slots else None,
                         hp, 1, 1, io=io, sr=sr, rows=rows, **fkw)
        times.append(time.perf_counter() - c0)
    tcpu = float(np.median(times))
    flops = 4.0 * spec.T * n_rows * spec.inn
    return {"value": round(flops / tcpu / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{spec.name} {n_rows} of {spec.out} output rows x {spec.inn}, T={spec.T}: float64 "
                      f"dgrad + fused-step oracle, median of {reps} ({tcpu:.2f} s each)"}


TRAIN_WORKLOAD = "llama8b_mlp_train_8192"


def train_main(args) -> int:
    """Training steps through autograd: a model of SwiGLU MLP blocks of Llama-3.1-8B
    shape (d 4096, hidden 14336; gate, up and down are ForgeLinear layers), 8192 tokens,
    AdamW with stochastic rounding and float32 moments. One step = forward, backward
    (dgrad and the fused step per layer) for the fused schedule; forward, backward with
    the float32 dW stored per layer, then the optimizer pass over every layer for the
    two-phase schedule. Each schedule runs with and without activation checkpointing
    (per block); each reports its step time and its peak memory above what the model,
    its moments and the batch hold."""
    import numpy as np
    import torch

    from optimizer_gemm_amd.nn import ForgeLinear, SwiGLUBlock, step_all
    from synth import LayerSpec

    d, hidden, T, blocks = 4096, 14336, 8192, args.blocks
    if blocks < 1:
        print("--blocks must be at least 1", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    opt = args.opt
    state = args.states or "f32"
    P = hidden * d                          # weights per linear (all three have hidden x d)
    n_lin = 3 * blocks
    step_flops = n_lin * 6.0 * T * P        # forward, dgrad and wgrad GEMMs of every linear
    gen = torch.Generator(device=dev)
    gen.manual_seed(0x5EED_7000)
    x = torch.randn(T, d, device=dev, generator=gen).to(torch.bfloat16)
    G = (torch.randn(T, d, device=dev, generator=gen) * 1e-3).to(torch.bfloat16)

    def run(fused: bool, ckpt: bool):
        torch.manual_seed(0x5EED_7001)   # same initial weights in every schedule
        model = torch.nn.Sequential(*[
            SwiGLUBlock(d, hidden, checkpoint=ckpt, seed=b, fused=fused, device=dev, opt=opt, states=state,
                        hyper={"stochastic_round": 1}, grouped=args.group) for b in range(blocks)])
        xin = x.clone().requires_grad_(True)
        lins = [m for m in model.modules() if isinstance(m, ForgeLinear)]

        def step():
            xin.grad = None
            model(xin).backward(G)
            if not fused:
                step_all(model)

        for _ in range(args.warmup):
            step()
        xin.grad = None
        torch.cuda.synchronize()
        resident = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        if fused:
            for m in lins:
                m.timing = []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - resident
        ms = e0.elapsed_time(e1) / args.steps
        calls = [a.elapsed_time(b) for m in lins for (a, b) in (m.timing or [])]
        for m in lins:
            m.timing = None
        # what the training state itself holds: weights, moments (and scales), batch and output gradient
        state_bytes = sum(t.numel() * t.element_size() for t in list(model.parameters()) + list(model.buffers()))
        state_bytes += sum(t.numel() * t.element_size() for t in (x, G))
        out = {"ms_per_step": round(ms, 3), "tflops": round(step_flops / (ms * 1e-3) / 1e12, 2),
               "peak_above_resident_bytes": int(peak), "model_state_bytes": int(state_bytes),
               "process_resident_bytes": int(resident)}
        del model, xin, lins
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        return out, calls

    res = {}
    fused_calls = []
    for fused in (True, False):
        for ckpt in (False, True):
            name = ("fused" if fused else "two_phase") + ("_ckpt" if ckpt else "")
            print(f"[bench] training schedule {name}: {blocks} block(s), T={T}", file=sys.stderr, flush=True)
            r, calls = run(fused, ckpt)
            res[name] = r
            if fused and not ckpt:
                fused_calls = calls
            print(f"[bench]   {r}", file=sys.stderr, flush=True)
    floor = n_lin * 4 * P
    for sfx in ("", "_ckpt"):
        f, t = res["fused" + sfx], res["two_phase" + sfx]
        res["speedup" + sfx] = round(t["ms_per_step"] / f["ms_per_step"], 3)
        # peak = model state + the step's transient peak; the state is the same in both schedules
        res["peak_reduction" + sfx] = round(1.0 - (f["model_state_bytes"] + f["peak_above_resident_bytes"]) /
                                            (t["model_state_bytes"] + t["peak_above_resident_bytes"]), 4)
        res["transient_reduction" + sfx] = round(1.0 - f["peak_above_resident_bytes"] /
                                                 t["peak_above_resident_bytes"], 4)
    res["gradient_floor_bytes"] = int(floor)

    # every layer's fused step of the timed steps (a grouped launch of gate and up is one
    # timed call covering both layers)
    fused_ms = float(np.sum(fused_calls)) if fused_calls else float("nan")
    fused_tflops = n_lin * args.steps * 2.0 * T * P / (fused_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["bf16"]
    fz = res["fused"]
    spec = LayerSpec("gate_proj", hidden, d, T)
    cpu = None if args.no_cpu_baseline else cpu_baseline(spec, 2, opt, "bf16", True, False)
    rec = {
        "metric": METRIC,
        "value": fz["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fz["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian batch and output gradient; random-init weights)",
        "config": {"workload": TRAIN_WORKLOAD, "blocks": blocks, "shapes": [f"{hidden}x{d}", f"{d}x{hidden}"],
                   "tokens": T, "optimizer": opt, "states": state, "stochastic_round": True,
                   "step": ("forward, then backward: dgrad(old W) and the fused wgrad+optimizer per layer, gate and "
                            "up as one grouped launch" if args.group else
                            "forward, then backward: dgrad(old W) and the fused wgrad+optimizer per layer")
                           + " (value counts 6*T*out*in per linear: forward, dgrad, wgrad)"},
        "fused_tflops": round(fused_tflops, 2),
        "pct_mfma_peak": round(100.0 * fused_tflops / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(fused_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(fused_tflops / peak, 4), "traffic": None},
        "cpu_baseline": cpu,
        "train_step": res,
    }
    print(json.dumps(rec))
    return 0


def main() -> int:
    args = parse()
    if args.calibrate_copy:
        return calibrate_copy()
    if args.record_traffic:
        return record_traffic(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(tensor-parallel shards run the same kernel on each GPU's share)", file=sys.stderr)
        return 2
    if args.workload == TRAIN_WORKLOAD:
        return train_main(args)
    import numpy as np
    import torch

    import optimizer_gemm_amd as forge
    from synth import WORKLOADS, draw_layer_batch, draw_layer_batch_fp8, draw_layer_init, llama8b_stack

    if args.workload == "stack":
        layers = llama8b_stack(8192, 32)
        wl_config, state, sr = 5, "f32", True
    else:
        wl = WORKLOADS[args.workload]
        layers, wl_config, state, sr = wl.layers, wl.config, wl.state, wl.stochastic_round
    if args.states:
        state = args.states
    opt = args.opt
    # int8 moments: linear codes ("q8") or the dynamic 8-bit code ("q8dyn")
    code = "dynamic" if state == "q8dyn" else "linear"
    wstep = functools.partial(forge.wgrad_step, code=code)
    wunfused = functools.partial(forge.wgrad_unfused, code=code)
    optstep = functools.partial(forge.optimizer_step, code=code)
    dev = torch.device("cuda:0")
    io = layers[0].io
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    fp8 = args.inputs == "fp8"
    if fp8 and io != "bf16":
        print("FP8 inputs need bf16 weights", file=sys.stderr)
        return 2

    def to_dev(a):
        if io == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # one (X, dY, dX) buffer set per distinct shape; W and its moments per layer
    # (in the 224-layer stack, layers of one shape start from that shape's initial W)
    shape_bufs = {}
    shape_w0 = {}
    per_layer = []
    t0 = time.perf_counter()
    for li, spec in enumerate(layers):
        key = (spec.out, spec.inn, spec.T)
        if key not in shape_bufs:
            X, dY = draw_layer_batch(wl_config, li, 1, spec)
            bufs = [to_dev(X), to_dev(dY), torch.empty((spec.T, spec.inn), dtype=tdt, device=dev), None, None]
            if fp8:
                # the fused step reads FP8 codes; dgrad keeps the bf16 dY
                Xq, dYq, sx, sd = draw_layer_batch_fp8(wl_config, li, 1, spec, "e4m3", "e5m2")
                bufs[0] = torch.from_numpy(Xq).to(dev).view(torch.float8_e4m3fn)
                bufs.append(torch.from_numpy(dYq).to(dev).view(torch.float8_e5m2))
                bufs[3] = torch.tensor([sx], dtype=torch.float32, device=dev)
                bufs[4] = torch.tensor([sd], dtype=torch.float32, device=dev)
            else:
                bufs.append(bufs[1])
            shape_bufs[key] = tuple(bufs)
        if args.workload == "stack":
            if key not in shape_w0:
                shape_w0[key] = to_dev(draw_layer_init(wl_config, li, spec))
            W = shape_w0[key].clone()
        else:
            W = to_dev(draw_layer_init(wl_config, li, spec))
        m, v, ms, vs = forge.new_states(W, opt, state)
        per_layer.append((spec, W, m, v, ms, vs, ((0x5EED0000 + wl_config) ^ li)))
    shape_w0.clear()
    torch.cuda.synchronize()
    resident = torch.cuda.memory_allocated()
    print(f"[bench] setup {time.perf_counter() - t0:.1f}s: {len(layers)} layer(s), workload {args.workload}, "
          f"opt {opt}, states {state}, inputs {args.inputs}, resident {resident / 2**30:.2f} GiB",
          file=sys.stderr, flush=True)
    hyper = forge.make_hyper(opt, stochastic_round=int(sr))

    step_counter = [0]

    # units of the step: one layer each, or (--group) the layers of a decoder layer that share an
    # input (q, k, v and gate, up, in the order q, k, v, o, gate, up, down) as one grouped step
    units = [[k] for k in range(len(per_layer))]
    if args.group:
        if args.workload not in ("llama8b_layer_8192", "llama8b_tp8_8192", "stack"):
            print("--group needs a decoder-layer workload", file=sys.stderr)
            return 2
        units = []
        for b in range(0, len(per_layer), 7):
            units += [[b, b + 1, b + 2], [b + 3], [b + 4, b + 5], [b + 6]]

    def one_step(fused_events=None):
        step_counter[0] += 1
        t = step_counter[0]
        for unit in units:
            for k in unit:
                spec, W = per_layer[k][0], per_layer[k][1]
                X, dY, dX, xs, ds, dYf = shape_bufs[(spec.out, spec.inn, spec.T)]
                forge.dgrad(dY, W, dX)
            k0 = unit[0]
            if fused_events is not None:
                fused_events[k0][0].record()
            if len(unit) == 1:
                spec, W, m, v, ms, vs, seed = per_layer[k0]
                X, dY, dX, xs, ds, dYf = shape_bufs[(spec.out, spec.inn, spec.T)]
                wstep(X, dYf, W, m, v, opt, hyper, t, seed, ms, vs, x_scale=xs, dy_scale=ds)
            else:
                mem = [per_layer[k] for k in unit]
                bufs = [shape_bufs[(L[0].out, L[0].inn, L[0].T)] for L in mem]
                forge.wgrad_step_group(bufs[0][0], [b[5] for b in bufs], [L[1] for L in mem], [L[2] for L in mem],
                                       [L[3] for L in mem], opt, hyper, t, [L[6] for L in mem],
                                       [L[4] for L in mem], [L[5] for L in mem], code=code,
                                       x_scale=bufs[0][3], dy_scales=[b[4] for b in bufs])
            if fused_events is not None:
                fused_events[k0][1].record()
                for k in unit[1:]:  # the group's time is the first member's
                    fused_events[k][0].record()
                    fused_events[k][1].record()

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    flops_gemm = [2.0 * s.T * s.out * s.inn for (s, *_rest) in per_layer]
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in per_layer]
          for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    wall0 = time.perf_counter()
    start.record()
    for k in range(args.steps):
        one_step(ev[k])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    peak_transient = torch.cuda.max_memory_allocated() - resident
    elapsed_ms = start.elapsed_time(end)
    ms_per_step = elapsed_ms / args.steps
    total_flops = 2.0 * sum(flops_gemm) * args.steps  # dgrad + wgrad per layer per step
    value = total_flops / (elapsed_ms * 1e-3) / 1e12
    fused_ms = [[ev[k][j][0].elapsed_time(ev[k][j][1]) for j in range(len(per_layer))] for k in range(args.steps)]
    fused_ms_layer = np.mean(np.array(fused_ms), axis=0)           # mean per layer
    fused_total = float(np.sum(fused_ms_layer))
    fused_tflops = sum(flops_gemm) / (fused_total * 1e-3) / 1e12
    peak = PEAK_TFLOPS["fp8" if fp8 else io]
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step, fused {fused_total:.3f} ms/step "
          f"({fused_tflops:.1f} TFLOP/s), wall {wall:.2f}s", file=sys.stderr, flush=True)

    # --- per-call statistics of the first layer's fused kernel: warm (the timed loop's
    # calls) and cold (each call after a 1 GiB write, larger than the 256 MB memory-side
    # cache, so X, dY, W and the moments come from HBM) ---
    def pct(xs):
        a = np.sort(np.asarray(xs, dtype=np.float64))
        return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
                "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}

    call_stats = {"layer": f"{per_layer[0][0].name} {per_layer[0][0].out}x{per_layer[0][0].inn} T={per_layer[0][0].T}",
                  "unit": "us", "warm": pct([fused_ms[k][0] * 1e3 for k in range(args.steps)])}
    if args.cold_calls > 0:
        spec0, W0d, m0, v0, ms0, vs0, seed0 = per_layer[0]
        X0, _, _, xs0, ds0, dY0 = shape_bufs[(spec0.out, spec0.inn, spec0.T)]
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cold = []
        for r in range(args.cold_calls):
            flush.fill_(float(r))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            wstep(X0, dY0, W0d, m0, v0, opt, hyper, 30_000 + r, seed0, ms0, vs0, x_scale=xs0,
                             dy_scale=ds0)
            e1.record()
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1) * 1e3)
        del flush
        call_stats["cold"] = pct(cold)

    # --- traffic from committed rocprofv3 counters (only if taken on this kernel source) ---
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_{_traffic_name(args)}.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("opt", "adamw") == opt:
            traffic = tr.get("bytes_per_launch")

    # --- unfused baseline (separate timed region) ---
    unfused = None
    if not args.no_unfused and args.workload != "stack":
        spec, W, m, v, ms, vs, seed = per_layer[0]
        X, _, dX, xs, ds, dY = shape_bufs[(spec.out, spec.inn, spec.T)]
        sc = dict(x_scale=xs, dy_scale=ds)
        n_rep = max(3, min(args.steps, 20))
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        wstep(X, dY, W, m, v, opt, hyper, 10_000, seed, ms, vs, **sc)
        torch.cuda.synchronize()
        fused_transient = torch.cuda.max_memory_allocated() - base
        torch.cuda.reset_peak_memory_stats()
        dW = torch.empty((spec.out, spec.inn), dtype=torch.float32, device=dev)
        wunfused(X, dY, W, m, v, opt, hyper, 10_001, seed, ms, vs, dW_workspace=dW, **sc)
        torch.cuda.synchronize()
        unfused_transient = torch.cuda.max_memory_allocated() - base
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
              torch.cuda.Event(enable_timing=True)) for _ in range(n_rep)]
        f_e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_rep)]
        # a spin kernel keeps the GPU busy while the host enqueues each repetition, so the
        # event pairs time the kernels and not the host's launch latency (which dominates
        # on launch-bound layers)
        hold = getattr(torch.cuda, "_sleep", None)
        for r in range(n_rep):
            if hold is not None:
                hold(1_000_000)
            f_e[r][0].record()
            wstep(X, dY, W, m, v, opt, hyper, 10_002 + r, seed, ms, vs, **sc)
            f_e[r][1].record()
            e[r][0].record()
            forge.wgrad(X, dY, dW, **sc)
            e[r][1].record()
            optstep(dW, W, m, v, opt, hyper, 10_002 + r, seed, ms, vs)
            e[r][2].record()
        torch.cuda.synchronize()
        gemm_ms = float(np.median([a.elapsed_time(b) for a, b, _ in e]))
        opt_ms = float(np.median([b.elapsed_time(c) for _, b, c in e]))
        fused_med = float(np.median([a.elapsed_time(b) for a, b in f_e]))
        del dW
        unfused = {"gemm_store_ms": round(gemm_ms, 4), "optimizer_ms": round(opt_ms, 4),
                   "total_ms": round(gemm_ms + opt_ms, 4), "fused_ms": round(fused_med, 4),
                   "speedup_vs_unfused": round((gemm_ms + opt_ms) / fused_med, 3),
                   "dW_hbm_bytes_algorithmic": {"fused": 0, "unfused": 8 * spec.out * spec.inn},
                   "peak_transient_bytes": {"fused": int(fused_transient), "unfused": int(unfused_transient)},
                   "layer": f"{spec.name} {spec.out}x{spec.inn} T={spec.T}"}

    # --- the stack under the two-phase schedule: every layer's fp32 dW resident before the update ---
    stack_two_phase = None
    if args.workload == "stack" and not args.no_unfused:
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dWs = []
        for (spec, W, m, v, ms, vs, seed) in per_layer:
            X, dY, dX, xs, ds, dYf = shape_bufs[(spec.out, spec.inn, spec.T)]
            forge.dgrad(dY, W, dX)
            dWs.append(forge.wgrad(X, dYf, x_scale=xs, dy_scale=ds))
        for (spec, W, m, v, ms, vs, seed), dW in zip(per_layer, dWs):
            optstep(dW, W, m, v, opt, hyper, 20_000, seed, ms, vs)
        e1.record()
        torch.cuda.synchronize()
        floor = torch.cuda.max_memory_allocated() - base
        del dWs
        stack_two_phase = {"ms_per_pass": round(e0.elapsed_time(e1), 3), "peak_transient_bytes": int(floor),
                           "largest_layer_dW_bytes": int(max(4 * s.out * s.inn for s, *_ in per_layer))}

    cpu = None if args.no_cpu_baseline else cpu_baseline(layers[0], wl_config, opt, io, sr, fp8)

    # achieved bf16 MFMA rate of this device under full load (outside the timed region)
    mfma = None
    if not args.no_mfma_peak and io == "bf16" and not fp8:
        pk = forge.mfma_peak()
        mfma = {"tflops": round(pk["tflops"], 1), "unit": "TFLOP/s",
                "kernel": "back-to-back v_mfma_f32_32x32x16_bf16, register operands, all CUs",
                "fused_frac": round(fused_tflops / pk["tflops"], 4)}

    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 (e4m3 x e5m2) wgrad, bf16 dgrad" if fp8 else io,
        "data": "synthetic (seeded Gaussian inputs of the layer shapes; random-init weights)",
        "config": {"workload": args.workload, "layers": len(layers),
                   "shapes": sorted({f"{s.out}x{s.inn}" for s in layers}), "tokens": layers[0].T,
                   "optimizer": opt, "states": state, "stochastic_round": bool(sr), "inputs": args.inputs,
                   "step": ("dgrad(old W) of each layer, then its fused wgrad+optimizer step; q,k,v and gate,up "
                            "each take one grouped fused step after their dgrads" if args.group else
                            "dgrad(old W) then fused wgrad+optimizer, per layer")},
        "fused_ms_per_layer": [round(float(x), 4) for x in fused_ms_layer][:8],
        "fused_tflops": round(fused_tflops, 2),
        "fused_call_us": call_stats,
        "pct_mfma_peak": round(100.0 * fused_tflops / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(fused_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(fused_tflops / peak, 4), "traffic": traffic},
        "mfma_peak_measured": mfma,
        "cpu_baseline": cpu,
        "unfused": unfused,
        "resident_bytes": int(resident),
        "peak_transient_bytes": int(peak_transient),
        "wall_s": round(wall, 3),
    }
    if stack_two_phase is not None:
        rec["two_phase_schedule"] = stack_two_phase
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
