"""rocprofv3 helpers: a calibration copy kernel and summaries of profiler output.

    python -m transformer_attention_fwd_amd.prof copy [MiB]
        runs a plain elementwise copy (torch.neg) of a known size five times,
        the reference for scaling the FETCH_SIZE / WRITE_SIZE counters.
    python -m transformer_attention_fwd_amd.prof stats DIR OUT.md "COMMAND"
        writes the per-kernel table of a `rocprofv3 --kernel-trace --stats` run.
    python -m transformer_attention_fwd_amd.prof traffic WORKLOAD KERNEL \\
            FETCH_DIR WRITE_DIR CAL_FETCH_DIR CAL_WRITE_DIR MIB OUT.md "COMMANDS"
        turns the four `--pmc` runs into HBM bytes per launch of KERNEL and
        records them in profiles/traffic.json under WORKLOAD, keyed by the
        sha256 of the kernel's source file and the shared internal header
        (bench.py reports them only while those are unchanged).
    python -m transformer_attention_fwd_amd.prof sq WORKLOAD KERNEL RUN_DIR OUT.md "COMMAND"
        summarises one `rocprofv3 --kernel-trace --pmc` run of the SQ / GRBM
        counters below: matrix-core and VALU busy fractions, VALU and MFMA
        instruction counts per launch, and the shader clock the launches ran
        at (GRBM_GUI_ACTIVE cycles over the traced duration); recorded in
        profiles/counters.json under WORKLOAD, keyed like the traffic.

Nothing here runs on the attention path; it only reads profiler CSV files.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
COUNTERS_JSON = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "transformer_attention_fwd_amd", "csrc")
COPY_KERNEL = "neg"  # substring of the calibration kernel's name

# source file of each kernel (by a substring of its name)
KERNEL_SOURCES = {
    "flash_fwd_kernel": "olk_flash.hip",
    "decode_mfma_kernel": "olk_decode.hip",
    "decode_kernel": "olk_decode.hip",
    "combine_kernel": "olk_generic.hip",
    "generic_kernel": "olk_generic.hip",
    "tiled_kernel": "olk_tiled.hip",
    "rope": "olk_rope.hip",
    "present_kernel": "olk_present.hip",
    "bwd_": "olk_backward_mfma.hip",
}

# SQ / GRBM counters of one `sq` pass (at most 8 SQ and 2 GRBM counters per run)
SQ_COUNTERS = ["GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU",
               "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_TRANS_F32", "SQ_WAVE_CYCLES",
               "SQ_WAIT_INST_ANY", "SQ_BUSY_CYCLES"]
CU_NUM, SIMD_NUM, XCC_NUM = 256, 1024, 8


def kernel_source_sha(kernel: str):
    """sha256 over the kernel's source file and olk_internal.h (None if unknown)."""
    for key, src in KERNEL_SOURCES.items():
        if key in kernel:
            h = hashlib.sha256()
            for name in (src, "olk_internal.h"):
                with open(os.path.join(CSRC, name), "rb") as f:
                    h.update(f.read())
            return h.hexdigest()
    return None


def _one(pattern: str) -> str:
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def counter_per_dispatch(run_dir: str, kernel: str, counter: str) -> tuple[float, int]:
    """Mean of `counter` over the dispatches whose kernel name contains `kernel`."""
    path = _one(os.path.join(run_dir, "**", "*counter_collection.csv"))
    per = defaultdict(float)
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
                per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"{counter}: no dispatch of a kernel named *{kernel}* in {path}")
    return sum(per.values()) / len(per), len(per)


def counters_per_dispatch(run_dir: str, kernel: str) -> tuple[dict, list]:
    """{counter: mean over the dispatches of `kernel` of the counter summed over
    its instances}, and the dispatch ids."""
    path = _one(os.path.join(run_dir, "**", "*counter_collection.csv"))
    per = defaultdict(lambda: defaultdict(float))
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"]:
                per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatch of a kernel named *{kernel}* in {path}")
    names = set().union(*[set(v) for v in per.values()])
    return {n: sum(v.get(n, 0.0) for v in per.values()) / len(per) for n in names}, list(per)


def durations_ns(run_dir: str, kernel: str) -> list[float]:
    path = _one(os.path.join(run_dir, "**", "*kernel_trace.csv"))
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"]:
                out.append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    return out


def write_sq(workload: str, kernel: str, run_dir: str, out: str, command: str) -> None:
    c, ids = counters_per_dispatch(run_dir, kernel)
    dur = durations_ns(run_dir, kernel)
    # GRBM_GUI_ACTIVE counts per XCC; the sum over the 8 XCCs is 8x the cycles
    gui = c["GRBM_GUI_ACTIVE"] / XCC_NUM
    mean_ns = sum(dur) / len(dur) if dur else float("nan")
    rec = {
        "kernel": kernel, "kernel_sha256": kernel_source_sha(kernel), "dispatches": len(ids),
        "mean_duration_us": mean_ns / 1e3,
        "clock_ghz": gui / mean_ns if dur else None,
        "mfma_busy": c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMD_NUM),
        "valu_busy": c["SQ_ACTIVE_INST_VALU"] / (gui * CU_NUM),
        "insts_valu": c["SQ_INSTS_VALU"], "insts_mfma": c["SQ_INSTS_MFMA"],
        "insts_trans_f32": c["SQ_INSTS_VALU_TRANS_F32"],
        "valu_per_mfma": (c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"]) / max(c["SQ_INSTS_MFMA"], 1.0),
        "wave_cycles": c["SQ_WAVE_CYCLES"], "wait_inst_any": c["SQ_WAIT_INST_ANY"],
        "busy_cycles": c["SQ_BUSY_CYCLES"], "gui_active_cycles": gui,
    }
    allrec = {}
    if os.path.exists(COUNTERS_JSON):
        with open(COUNTERS_JSON) as f:
            allrec = json.load(f)
    allrec[workload] = rec
    with open(COUNTERS_JSON, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
    lines = [f"# SQ counters of `{kernel}` on {workload}", "",
             "Command (from the repository root):", "", "```", command, "```", "",
             "| quantity | value |", "|---|---:|",
             f"| dispatches | {len(ids)} |",
             f"| mean duration (kernel trace) | {mean_ns / 1e3:.2f} us |",
             f"| GRBM_GUI_ACTIVE per XCC | {gui:.0f} cycles |",
             f"| shader clock = cycles / duration | {rec['clock_ghz']:.3f} GHz |",
             f"| MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {SIMD_NUM} SIMDs) | {100 * rec['mfma_busy']:.1f} % |",
             f"| VALU busy = SQ_ACTIVE_INST_VALU / (cycles x {CU_NUM} CUs) | {100 * rec['valu_busy']:.1f} % |",
             f"| SQ_INSTS_VALU per launch (MFMA included) | {c['SQ_INSTS_VALU']:.4g} |",
             f"| SQ_INSTS_MFMA per launch | {c['SQ_INSTS_MFMA']:.4g} |",
             f"| non-MFMA VALU instructions per MFMA | {rec['valu_per_mfma']:.2f} |",
             f"| SQ_INSTS_VALU_TRANS_F32 per launch | {c['SQ_INSTS_VALU_TRANS_F32']:.4g} |",
             f"| SQ_WAVE_CYCLES | {c['SQ_WAVE_CYCLES']:.4g} |",
             f"| SQ_WAIT_INST_ANY (share of wave cycles) | {c['SQ_WAIT_INST_ANY']:.4g} ({100 * c['SQ_WAIT_INST_ANY'] / max(c['SQ_WAVE_CYCLES'], 1):.1f} %) |",
             f"| SQ_BUSY_CYCLES | {c['SQ_BUSY_CYCLES']:.4g} |"]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(rec))


def stats_table(run_dir: str) -> list[dict]:
    path = _one(os.path.join(run_dir, "**", "*kernel_stats.csv"))
    with open(path) as f:
        return list(csv.DictReader(f))


def write_stats(run_dir: str, out: str, command: str) -> None:
    rows = stats_table(run_dir)
    lines = ["# rocprofv3 kernel statistics", "", "Command (from the repository root):", "",
             "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | share % |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"]
        short = name if len(name) < 110 else name[:107] + "..."
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_traffic(workload: str, kernel: str, fetch_dir: str, write_dir: str, cal_fetch: str,
                  cal_write: str, mib: float, out: str, commands: str) -> None:
    nbytes = mib * 2**20
    f_k, nf = counter_per_dispatch(fetch_dir, kernel, "FETCH_SIZE")
    w_k, nw = counter_per_dispatch(write_dir, kernel, "WRITE_SIZE")
    f_c, _ = counter_per_dispatch(cal_fetch, COPY_KERNEL, "FETCH_SIZE")
    w_c, _ = counter_per_dispatch(cal_write, COPY_KERNEL, "WRITE_SIZE")
    f_scale, w_scale = nbytes / f_c, nbytes / w_c  # bytes per counter unit
    fetch_b, write_b = f_k * f_scale, w_k * w_scale
    rec = {}
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as f:
            rec = json.load(f)
    rec[workload] = {
        "kernel": kernel,
        "kernel_sha256": kernel_source_sha(kernel),
        "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
        "fetch_counter_per_dispatch": f_k, "write_counter_per_dispatch": w_k,
        "copy_bytes": nbytes, "copy_fetch_counter": f_c, "copy_write_counter": w_c,
        "fetch_scale": f_scale, "write_scale": w_scale,
    }
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    lines = [f"# HBM traffic of `{kernel}` on {workload}", "",
             "Commands (from the repository root, one rocprofv3 run per counter):", "",
             "```", commands, "```", "",
             f"| quantity | value |", "|---|---:|",
             f"| FETCH_SIZE per dispatch ({nf} dispatches) | {f_k:.1f} |",
             f"| WRITE_SIZE per dispatch ({nw} dispatches) | {w_k:.1f} |",
             f"| copy kernel ({mib:.0f} MiB read + written): FETCH_SIZE | {f_c:.1f} |",
             f"| copy kernel: WRITE_SIZE | {w_c:.1f} |",
             f"| bytes per FETCH_SIZE unit (copy calibration) | {f_scale:.2f} |",
             f"| bytes per WRITE_SIZE unit (copy calibration) | {w_scale:.2f} |",
             f"| HBM bytes read per launch | {fetch_b / 1e6:.2f} MB |",
             f"| HBM bytes written per launch | {write_b / 1e6:.2f} MB |",
             f"| total per launch | {(fetch_b + write_b) / 1e6:.2f} MB |"]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(rec[workload]))


def copy(mib: float) -> None:
    import torch
    n = int(mib * 2**20) // 2
    a = torch.randn(n, dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x5", flush=True)


def main(argv: list[str]) -> None:
    cmd = argv[0] if argv else ""
    if cmd == "copy":
        copy(float(argv[1]) if len(argv) > 1 else 512.0)
    elif cmd == "stats":
        write_stats(argv[1], argv[2], argv[3])
    elif cmd == "sq":
        write_sq(argv[1], argv[2], argv[3], argv[4], argv[5])
    elif cmd == "traffic":
        write_traffic(argv[1], argv[2], argv[3], argv[4], argv[5], argv[6], float(argv[7]),
                      argv[8], argv[9])
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
