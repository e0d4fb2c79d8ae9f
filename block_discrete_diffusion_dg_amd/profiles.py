"""Summaries of rocprofv3 output for the repository's profiles/ folder.

  python -m block_discrete_diffusion_dg_amd.profiles stats <kernel_stats.csv> <out.md> --command "<cmd>"
  python -m block_discrete_diffusion_dg_amd.profiles traffic <fetch_csv> <write_csv> <out_stem>
      --kernel <name regex> --copy-bytes N --command-fetch "<cmd>" --command-write "<cmd>"
  python -m block_discrete_diffusion_dg_amd.profiles mfma <counter_csv> <out.md> --command "<cmd>"
      (counters MfmaUtil, MfmaFlopsBF16, GRBM_GUI_ACTIVE per dispatch)

`traffic` turns FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) into HBM
bytes per launch of one kernel, scaled by what the same counter reads for a
plain device copy of known size, and records a hash of the kernel's sources:
bench.py reports the figure only while the sources still hash the same.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PROFILES = os.path.join(ROOT, "profiles")

# Sources that define each profiled kernel (hashed into the traffic record).
KERNEL_SOURCES = {
    "moe_experts": ["csrc/k_moe.hip", "csrc/stream.h", "csrc/common.h"],
    "lmhead": ["csrc/k_lmhead.hip", "csrc/common.h"],
    "attn": ["csrc/k_attn.hip", "csrc/common.h"],
}

# Kernel classes of the matrix-core summary: (label, name pattern).
MFMA_CLASSES = [("attention (attn_kernel)", r"attn_kernel"), ("LM head (lmhead_kernel)", r"lmhead_kernel"),
                ("experts (moe_experts_kernel)", r"moe_experts_kernel"), ("QKV (qkv_sk_kernel)", r"qkv_sk_kernel"),
                ("O-proj (resid_sk_kernel)", r"resid_sk_kernel"), ("router (router_kernel)", r"router_kernel")]
GPU_CLOCK_HZ = 2.4e9  # MI355X peak engine clock, for cycles -> time


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", name)


def summarize_stats(csv_path: str, out_md: str, command: str) -> None:
    """Library kernels first (per-call time), then one line for everything the
    host framework launched (weight generation, copies) outside the step."""
    rows = list(csv.DictReader(open(csv_path)))
    ours = [r for r in rows if "at::native" not in r["Name"] and "rocclr" not in r["Name"]]
    other = [r for r in rows if r not in ours]
    lines = ["# Kernel time summary (rocprofv3 --kernel-trace --stats)", "",
             f"Command: `{command}`", "",
             "Library kernels (the denoising path):", "",
             "| kernel | calls | avg us | total ms |", "|---|---:|---:|---:|"]
    for r in ours:
        lines.append(f"| {_short(r['Name'])[:60]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.2f} |")
    tot = sum(float(r["TotalDurationNs"]) for r in other) / 1e6
    calls = sum(int(r["Calls"]) for r in other)
    lines += ["", f"Other kernels (PyTorch weight generation and runtime copies before the timed "
                  f"steps): {calls} calls, {tot:.1f} ms in total."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_dispatch(csv_path: str, counter: str):
    per = defaultdict(list)
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter:
            per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def summarize_traffic(fetch_csv: str, write_csv: str, out_stem: str, kernel: str, kernel_regex: str,
                      copy_bytes: int, command_fetch: str, command_write: str) -> dict:
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    pat = re.compile(kernel_regex)

    def pick(per):
        vals = [v for name, vs in per.items() if pat.search(name) for v in vs]
        return sum(vals) / len(vals) if vals else None, len(vals)

    def copy_kib(per):
        # the copy probe is the largest dispatch of the runtime's buffer copy
        vals = [v for name, vs in per.items() if "copyBuffer" in name for v in vs]
        return max(vals) if vals else None

    f_kib, nf = pick(fetch)
    w_kib, nw = pick(write)
    cf, cw = copy_kib(fetch), copy_kib(write)
    fetch_factor = (copy_bytes / 1024) / cf if cf else None
    write_factor = (copy_bytes / 1024) / cw if cw else None
    rec = {
        "kernel": kernel,
        "kernel_regex": kernel_regex,
        "dispatches": {"fetch": nf, "write": nw},
        "fetch_kib_per_dispatch": f_kib,
        "write_kib_per_dispatch": w_kib,
        "copy_probe_bytes": copy_bytes,
        "copy_probe_fetch_kib": cf,
        "copy_probe_write_kib": cw,
        "fetch_scale": fetch_factor,
        "write_scale": write_factor,
        "hbm_bytes_per_launch": (f_kib * 1024 * (fetch_factor or 1.0) + w_kib * 1024 * (write_factor or 1.0))
        if f_kib is not None and w_kib is not None else None,
        "source_hash": source_hash(kernel),
        "command_fetch": command_fetch,
        "command_write": command_write,
    }
    with open(out_stem + ".json", "w") as f:
        json.dump(rec, f, indent=1)
    md = [f"# HBM traffic of {kernel} (rocprofv3 --pmc)", "",
          f"FETCH_SIZE command: `{command_fetch}`", "",
          f"WRITE_SIZE command: `{command_write}`", "",
          f"- dispatches: {nf} (fetch run), {nw} (write run)",
          f"- FETCH_SIZE: {f_kib:.0f} KiB per dispatch" if f_kib is not None else "- FETCH_SIZE: n/a",
          f"- WRITE_SIZE: {w_kib:.0f} KiB per dispatch" if w_kib is not None else "- WRITE_SIZE: n/a",
          f"- copy probe ({copy_bytes} B device copy): FETCH {cf} KiB, WRITE {cw} KiB -> "
          f"scales {fetch_factor}, {write_factor}",
          f"- HBM bytes per launch (scaled): {rec['hbm_bytes_per_launch']}",
          f"- source hash: {rec['source_hash']}"]
    with open(out_stem + ".md", "w") as f:
        f.write("\n".join(md) + "\n")
    return rec


def summarize_mfma(csv_path: str, out_md: str, command: str) -> dict:
    """Per kernel class: mean MfmaUtil (percent of SIMD cycles with the matrix
    core busy while the dispatch ran), bf16 MFMA flops per dispatch, and the
    GPU-active cycles per dispatch (time at the peak clock)."""
    per = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(csv_path)):
        per[r["Counter_Name"]][r["Kernel_Name"]].append(float(r["Counter_Value"]))
    out = {}
    lines = ["# Matrix-core use per kernel (rocprofv3 --pmc)", "", f"Command: `{command}`", "",
             "MfmaUtil is rocprofv3's derived metric: SQ_VALU_MFMA_BUSY_CYCLES summed over the SIMDs over "
             "GRBM_GUI_ACTIVE times the SIMD count, during each dispatch (counters serialise the dispatches). "
             "MfmaFlopsBF16 = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512. Rate = flops / (active cycles / 2.4 GHz); "
             "the dense bf16 peak is 2.5 PFLOP/s.", "",
             "| kernel | dispatches | MfmaUtil % | bf16 GFLOP per dispatch | active us per dispatch | TFLOP/s | of peak |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for label, pat in MFMA_CLASSES:
        rx = re.compile(pat)
        util = [v for k, vs in per["MfmaUtil"].items() if rx.search(k) for v in vs]
        flops = [v for k, vs in per["MfmaFlopsBF16"].items() if rx.search(k) for v in vs]
        act = [v for k, vs in per["GRBM_GUI_ACTIVE"].items() if rx.search(k) for v in vs]
        if not util:
            continue
        u, f, a = sum(util) / len(util), sum(flops) / max(1, len(flops)), sum(act) / max(1, len(act))
        t = a / GPU_CLOCK_HZ
        rate = f / t / 1e12 if t > 0 else 0.0
        out[label] = {"dispatches": len(util), "mfma_util_pct": u, "gflop": f / 1e9, "active_us": t * 1e6,
                      "tflops": rate}
        lines.append(f"| {label} | {len(util)} | {u:.1f} | {f / 1e9:.3f} | {t * 1e6:.1f} | {rate:.0f} | "
                     f"{rate / 2500:.3f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return out


def traffic_for(kernel: str, stem: str):
    """HBM bytes per launch recorded for `kernel`, or None when no record
    exists or the kernel's sources changed since it was taken."""
    path = os.path.join(PROFILES, stem + ".json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel") != kernel or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("out_stem")
    t.add_argument("--kernel", required=True)
    t.add_argument("--kernel-regex", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    m.add_argument("out")
    m.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.cmd == "stats":
        summarize_stats(a.csv, a.out, a.command)
    elif a.cmd == "mfma":
        print(json.dumps(summarize_mfma(a.csv, a.out, a.command), indent=1))
    else:
        print(json.dumps(summarize_traffic(a.fetch_csv, a.write_csv, a.out_stem, a.kernel, a.kernel_regex,
                                           a.copy_bytes, a.command_fetch, a.command_write), indent=1))


if __name__ == "__main__":
    main()
