#!/usr/bin/env python3
"""Benchmark of the attention forward on one MI355X.

One step = one call of the whole path (validate/plan on the host, sequence
metadata, Q load, K/V staging + present write, QK^T, score epilogue, online
softmax, PV, finalize) on the bf16 GQA causal prefill workload
(B=4, S=2048, 32 query / 8 KV heads, head size 128), inputs resident in HBM.

Prints one JSON line: the headline TFLOP/s (algorithmic FLOPs: 4*D per
unmasked (query, key) pair, i.e. QK^T + PV), the roofline of the dominant
kernel (the step is one launch of it, timed with HIP events on the stream it
runs on), the oracle's CPU
throughput on a bounded sample, and secondary figures for the other workloads
(decode as KV GB/s).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}  # dense, MI355X
HBM_PEAK_GBS = 8000.0
HEADLINE = "gqa_prefill_causal_bf16"
# prefill workloads also timed cache-cold (inputs rotated over several copies)
ROTATED = ("gqa_prefill_causal_bf16", "gqa_prefill_window_sink_bf16", "mha_cross_f16")
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
NOMINAL_CLOCK_GHZ = 2.4
# the kernel a step's roofline is about, by the path the library reports
DOMINANT = {"olk_tiled_fwd": ("flash_fwd_kernel", "flash_fwd_kernel"),
            "olk_rope+olk_tiled_fwd": ("flash_fwd_kernel", "rope_vec2_kernel + flash_fwd_kernel"),
            "olk_decode_split+combine": ("decode_mfma_kernel",
                                         "decode_mfma_kernel + combine_kernel")}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-secondary", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the GroupQueryAttention backward line (for profiling)")
    ap.add_argument("--settle-seconds", type=float, default=0.4,
                    help="after the timed steps, launch for this long and time the steps again "
                         "at the settled clock (reported as `steady`; 0: skip)")
    ap.add_argument("--rotate-buffers", type=int, default=4,
                    help="input/output sets cycled for the cache-cold prefill figures "
                         "(0: skip them)")
    return ap.parse_args()


# ---- algorithmic work (bookkeeping of the definition's masks) ---------------

def allowed_pairs(p, inputs) -> np.ndarray:
    """Number of attended keys per (b, i) row (same for every head)."""
    from transformer_attention_fwd_amd.workloads import valid_lengths
    tot = valid_lengths(p, inputs)
    out = np.zeros((p.B, p.S), dtype=np.int64)
    for b in range(p.B):
        if p.op == "gqa":
            total = int(tot[b])
            qoff = total - p.S
            valid = total
        else:
            total = p.T
            qoff = p.P
            valid = int(tot[b]) if (p.op == "attention" or p.mask_filter_value <= -5000) else total
            if p.op == "mha" and valid == 0:
                valid = total
        pos = qoff + np.arange(p.S)
        hi = np.full(p.S, valid)
        if p.causal:
            hi = np.minimum(hi, pos + 1)
        lo = np.zeros(p.S, dtype=np.int64)
        if p.window > 0:
            lo = np.maximum(0, pos - p.window + 1)
        if p.bias_bh is not None and p.bias_cols > 0:
            hi = np.minimum(hi, p.bias_cols)
        if p.mask_kind == "bool":
            # attended keys of each row under a head-broadcast BOOL mask
            m = inputs["mask"].numpy().astype(bool)
            assert m.shape[1] == 1, "head-broadcast masks only"
            mb = m[b if m.shape[0] > 1 else 0, 0]
            cols = mb.shape[-1]
            for i in range(p.S):
                row = mb[i if mb.shape[0] > 1 else 0]
                h_i = min(int(hi[i]), cols)
                out[b, i] = int(row[int(lo[i]):h_i].sum()) if h_i > lo[i] else 0
            continue
        out[b] = np.maximum(0, hi - lo)
    return out


def flops(p, inputs) -> float:
    return 2.0 * (p.D + p.Dv) * float(allowed_pairs(p, inputs).sum()) * p.Hq


def prefill_bytes(p, inputs) -> float:
    """Least HBM traffic of a prefill call: Q and Y once, every K/V row some
    query attends once, bias and mask once, present written once
    (GroupQueryAttention)."""
    from transformer_attention_fwd_amd.workloads import valid_lengths
    es = 2 if p.dtype != "f32" else 4
    qy = p.B * p.S * p.Hq * (p.D + p.Dv) * es
    tot = valid_lengths(p, inputs)
    rows = 0.0
    for b in range(p.B):
        if p.op == "gqa":
            rows += float(tot[b])
        else:
            valid = int(tot[b]) if (p.op == "attention" or p.mask_filter_value <= -5000) else p.T
            valid = valid or p.T
            rows += float(min(valid, p.P + p.S) if p.causal else valid)
    kv = rows * p.Hkv * (p.D + p.Dv) * es
    bias = float(inputs["bias"].numel() * es) if "bias" in inputs else 0.0
    mask = float(inputs["mask"].numel() * inputs["mask"].element_size()) if "mask" in inputs else 0.0
    present = kv if p.op == "gqa" else 0.0
    return qy + kv + bias + mask + present


def decode_bytes(p, inputs, inplace: bool) -> float:
    """KV bytes read + Q/Y + new K/V + present append (or full copy)."""
    from transformer_attention_fwd_amd.workloads import valid_lengths
    es = 2 if p.dtype != "f32" else 4
    tot = valid_lengths(p, inputs).astype(np.float64)
    kv = float((tot - p.S).sum()) * p.Hkv * (p.D + p.Dv) * es          # past rows read
    new = p.B * p.S * p.Hkv * (p.D + p.Dv) * es                         # new K/V read
    qy = p.B * p.S * p.Hq * (p.D + p.Dv) * es
    append = new if inplace else float(tot.sum()) * p.Hkv * (p.D + p.Dv) * es
    return kv + new + qy + append


# ---- timing ---------------------------------------------------------------------

def time_launches(call, steps: int, warmup: int):
    import torch
    for _ in range(warmup):
        call.launch()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        call.launch()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def time_steady(call, steps: int, settle_s: float):
    """Step time once the shader clock has settled: launches back to back for
    at least settle_s seconds of wall time (the clock rises over the first
    ~30 ms of sustained work after an idle spell), then `steps` timed launches.
    Returns (ms per step, seconds spent settling)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(20):
            call.launch()
        torch.cuda.synchronize()
    settled = time.perf_counter() - t0
    ms, _ = time_launches(call, steps, 0)
    return ms, settled


def _profile_record(path: str, workload: str, kernel: str):
    """The committed rocprofv3 record of `kernel` on `workload`, if it was taken
    on the kernel's current source (else None)."""
    from transformer_attention_fwd_amd.prof import kernel_source_sha
    try:
        with open(path) as f:
            ent = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if ent and ent.get("kernel") == kernel and ent.get("kernel_sha256") == kernel_source_sha(kernel):
        return ent
    return None


def traffic_for(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE
    counters, or None when they were taken on another version of its source."""
    ent = _profile_record(PROFILE_TRAFFIC, workload, kernel)
    return None if ent is None else float(ent["fetch_bytes"]) + float(ent["write_bytes"])


def roofline(name, p, res, work: float, bound: str, kernel: str, step_kernels: str):
    """Roofline of the step's dominant kernel: algorithmic work / the measured
    step time, against MI355X's published peak; the committed counters add the
    HBM traffic, the shader clock the kernel ran at and the matrix / vector
    busy fractions."""
    ms = res["ms_per_step"]
    if bound == "mfma":
        achieved, peak, unit = work / (ms * 1e-3) / 1e12, MFMA_PEAK_TFLOPS[p.dtype], "TFLOP/s"
    else:
        achieved, peak, unit = work / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    r = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 5), "traffic": traffic_for(name, kernel),
         "kernel": kernel, "step_kernels": step_kernels, "step_ms": round(ms, 5),
         ("flops_per_launch" if bound == "mfma" else "bytes_per_launch"): work}
    c = _profile_record(PROFILE_COUNTERS, name, kernel)
    if c is not None:
        r["counters"] = {"clock_ghz": round(c["clock_ghz"], 3),
                         "mfma_busy": round(c["mfma_busy"], 4),
                         "valu_busy": round(c["valu_busy"], 4),
                         "valu_per_mfma": round(c["valu_per_mfma"], 3),
                         "profiled_kernel_us": round(c["mean_duration_us"], 2)}
        if bound == "mfma":
            # the same figure against the peak at the clock the kernel ran at
            r["frac_at_measured_clock"] = round(
                achieved / (peak * c["clock_ghz"] / NOMINAL_CLOCK_GHZ), 5)
    return r


def cpu_baseline(p, inputs, kind: str, target_s: float):
    """Oracle throughput on a bounded random sample of rows."""
    from oracle import olk_ref
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(7)
    pairs = allowed_pairs(p, inputs)
    # calibrate on a small sample, then size the sample to ~target_s
    n = 64
    rows = None
    spent = 0.0
    work = 0.0
    n_rows = 0
    for _ in range(3):
        rows = np.stack([rng.integers(0, p.B, n), rng.integers(0, p.Hq, n),
                         rng.integers(0, p.S, n)], axis=1).astype(np.int32)
        t0 = time.perf_counter()
        olk_ref.attention_rows(p, inputs, rows, threads=cores)
        dt = time.perf_counter() - t0
        spent += dt
        n_rows += len(rows)
        npairs = float(pairs[rows[:, 0], rows[:, 2]].sum())
        if kind == "flops":
            work += 2.0 * (p.D + p.Dv) * npairs
        else:
            es = 2 if p.dtype != "f32" else 4
            work += npairs * (p.D + p.Dv) * es
        if spent >= target_s:
            break
        n = int(min(200000, max(n * 2, n * (target_s - spent) / max(dt, 1e-3))))
    value = work / spent / (1e12 if kind == "flops" else 1e9)
    return {"value": round(value, 6), "unit": "TFLOP/s" if kind == "flops" else "GB/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{n_rows} random (b, h, i) query rows of {p.B}x{p.Hq}x{p.S} "
                      f"({spent:.1f} s of float64 oracle time)"}


def check_rows(p, inputs, y, n=48):
    """Sampled-row parity against the oracle before timing."""
    import torch
    from oracle import olk_ref
    rng = np.random.default_rng(3)
    rows = np.stack([rng.integers(0, p.B, n), rng.integers(0, p.Hq, n),
                     rng.integers(0, p.S, n)], axis=1).astype(np.int32)
    want = olk_ref.attention_rows(p, inputs, rows)
    yl = y.detach().to("cpu").to(torch.float64)
    yl = yl.view(p.B, p.S, p.Hq, p.Dv) if p.q_rank == 3 else yl.permute(0, 2, 1, 3)
    got = yl.numpy()[rows[:, 0], rows[:, 2], rows[:, 1]]
    return float(np.abs(got - want).max())


def time_rotating(p, dev, inputs, sets: int, steps: int, warmup: int, decode: bool):
    """Cache-cold step time: `sets` copies of the inputs and outputs (a working
    set beyond the 256 MB MALL) used in turn, so no step finds its data in the
    caches the previous one filled."""
    import torch
    from transformer_attention_fwd_amd import olk
    calls = []
    for _ in range(sets):
        d = {k: v.clone() for k, v in dev.items()}
        calls.append(olk.Call(p, d, mode="fwd", want_present=(p.op == "gqa")))
    for i in range(warmup):
        calls[i % sets].launch()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        calls[i % sets].launch()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del calls
    return ms


def run_workload(name, steps, warmup, with_cpu, cpu_s, is_headline, rotate=0, settle_s=0.0):
    import torch
    from transformer_attention_fwd_amd import olk
    from transformer_attention_fwd_amd.workloads import workload
    p, inputs = workload(name)
    dev = {k: v.to("cuda") for k, v in inputs.items()}
    decode = p.S == 1
    res = {"workload": name}
    if decode:
        # KV-cache decode: present already holds the past (in-place append)
        pk = torch.empty((p.B, p.Hkv, p.P + p.L, p.D), dtype=p.torch_dtype, device="cuda")
        pv = torch.empty((p.B, p.Hkv, p.P + p.L, p.Dv), dtype=p.torch_dtype, device="cuda")
        pk[:, :, : p.P] = dev.pop("past_k")
        pv[:, :, : p.P] = dev.pop("past_v")
        call = olk.Call(p, dev, mode="decode", kv_inplace=True, present_k=pk, present_v=pv)
    else:
        call = olk.Call(p, dev, mode="fwd", want_present=(p.op == "gqa"))
    call.launch()
    torch.cuda.synchronize()
    res["kernel"] = olk.olk_last_kernel_name()
    res["max_abs_err_sampled"] = check_rows(p, inputs, call.y)
    ms, wall = time_launches(call, steps, warmup)
    res["ms_per_step"] = ms
    res["wall_s"] = wall
    steady = time_steady(call, max(steps, 50), settle_s) if settle_s > 0 else None
    dom = DOMINANT.get(res["kernel"])
    if decode:
        by = decode_bytes(p, inputs, inplace=True)
        res["value"] = by / (ms * 1e-3) / 1e9
        res["unit"] = "GB/s"
        res["frac_of_peak"] = res["value"] / HBM_PEAK_GBS
        res["bytes_per_step"] = by
        if dom:
            res["roofline"] = roofline(name, p, res, by, "hbm", dom[0], dom[1])
        if steady:
            v = by / (steady[0] * 1e-3) / 1e9
            res["steady"] = {"settle_s": round(steady[1], 3), "steps": max(steps, 50),
                             "ms_per_step": round(steady[0], 5), "value": round(v, 3),
                             "frac_of_peak": round(v / HBM_PEAK_GBS, 5)}
    else:
        fl = flops(p, inputs)
        res["value"] = fl / (ms * 1e-3) / 1e12
        res["unit"] = "TFLOP/s"
        res["frac_of_peak"] = res["value"] / MFMA_PEAK_TFLOPS[p.dtype]
        res["flops_per_step"] = fl
        by = prefill_bytes(p, inputs)
        res["hbm_bytes_algorithmic"] = by
        res["hbm_frac"] = round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 5)
        if dom:
            # With present written by the prefill kernel itself the step is one
            # launch of it, so the HIP-event step time is its launch duration.
            res["roofline"] = roofline(name, p, res, fl, "mfma", dom[0], dom[1])
        if steady:
            v = fl / (steady[0] * 1e-3) / 1e12
            res["steady"] = {"settle_s": round(steady[1], 3), "steps": max(steps, 50),
                             "ms_per_step": round(steady[0], 5), "value": round(v, 3),
                             "frac_of_peak": round(v / MFMA_PEAK_TFLOPS[p.dtype], 5)}
        if rotate > 1:
            cold = time_rotating(p, dev, inputs, rotate, steps, warmup, decode)
            res["cold"] = {"sets": rotate, "ms_per_step": round(cold, 5),
                           "value": round(fl / (cold * 1e-3) / 1e12, 3),
                           "frac_of_peak": round(fl / (cold * 1e-3) / 1e12 /
                                                 MFMA_PEAK_TFLOPS[p.dtype], 5)}
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(p, inputs, "bytes" if decode else "flops", cpu_s)
    del call, dev
    torch.cuda.empty_cache()
    return p, res


def run_backward(steps: int, warmup: int):
    """GroupQueryAttention backward on the headline shape: dQ, dK, dV from Q, K,
    V and a seeded dY.  Algorithmic FLOPs: 2*(3*D + 2*Dv) per unmasked (query,
    key) pair (S recomputed, dP, dV, dK, dQ)."""
    import torch
    from transformer_attention_fwd_amd import olk
    from transformer_attention_fwd_amd.workloads import workload
    p, inputs = workload(HEADLINE)
    dev = {k: v.to("cuda") for k, v in inputs.items()}
    g = torch.Generator().manual_seed(5)
    dy = torch.randn(p.B, p.S, p.Hq * p.Dv, generator=g).to(p.torch_dtype).cuda()
    call = olk.BwdCall(p, dev, dy)
    ms, _ = time_launches(call, steps, warmup)
    fl = 2.0 * (3 * p.D + 2 * p.Dv) * float(allowed_pairs(p, inputs).sum()) * p.Hq
    res = {"value": fl / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "ms_per_step": ms,
           "kernel": olk.olk_last_kernel_name(), "flops_per_step": fl}
    res["frac_of_peak"] = res["value"] / MFMA_PEAK_TFLOPS[p.dtype]
    del call, dev
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the attention path runs one GPU per process and has no multi-GPU path; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    torch.cuda.set_device(0)
    if args.backward_only:
        r = run_backward(args.steps, args.warmup)
        print(json.dumps({"workload": "gqa_backward_bf16", **r}), flush=True)
        return
    t_start = time.perf_counter()
    p, head = run_workload(args.workload, args.steps, args.warmup, not args.no_cpu,
                           args.cpu_seconds, True, args.rotate_buffers, args.settle_seconds)
    print(f"[bench] {args.workload}: {head['value']:.1f} {head['unit']} "
          f"({head['ms_per_step']:.3f} ms/step) err={head['max_abs_err_sampled']:.2e}",
          file=sys.stderr, flush=True)
    secondary = {}
    if not args.no_secondary:
        from transformer_attention_fwd_amd.workloads import WORKLOAD_ORDER
        for name in WORKLOAD_ORDER:
            if name == args.workload:
                continue
            rot = args.rotate_buffers if name in ROTATED else 0
            _, r = run_workload(name, max(10, args.steps // 2), max(3, args.warmup // 2), False,
                                0, False, rot, args.settle_seconds)
            print(f"[bench] {name}: {r['value']:.1f} {r['unit']} ({r['ms_per_step']:.4f} ms) "
                  f"err={r['max_abs_err_sampled']:.2e}", file=sys.stderr, flush=True)
            secondary[name] = {k: r[k] for k in ("value", "unit", "frac_of_peak", "ms_per_step",
                                                 "kernel", "max_abs_err_sampled", "roofline",
                                                 "hbm_frac", "cold", "steady") if k in r}
    if not args.no_secondary:
        r = run_backward(max(3, args.steps // 10), 1)
        print(f"[bench] gqa_backward_bf16: {r['value']:.1f} {r['unit']} ({r['ms_per_step']:.3f} ms)",
              file=sys.stderr, flush=True)
        secondary["gqa_backward_bf16"] = r
    line = {
        "metric": "attention TFLOP/s (prefill) + KV GB/s (decode), % of MI355X MFMA/HBM peak",
        "value": round(head["value"], 3),
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic (seeded N(0,1) inputs; no dataset)",
        "config": {"workload": args.workload, "op": p.op, "batch": p.B, "seq_len": p.S,
                   "q_heads": p.Hq, "kv_heads": p.Hkv, "head_size": p.D,
                   "causal": p.causal, "local_window_size": p.window,
                   "outputs": "Y + present_key/present_value"},
        "frac_of_peak": round(head["frac_of_peak"], 5),
        "kernel": head["kernel"],
        "max_abs_err_sampled": head["max_abs_err_sampled"],
        "roofline": head.get("roofline"),
        "hbm_frac": head.get("hbm_frac"),
        "cold": head.get("cold"),
        "steady": head.get("steady"),
        "cpu_baseline": head.get("cpu_baseline"),
        "secondary": secondary,
        "bench_wall_s": round(time.perf_counter() - t_start, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
