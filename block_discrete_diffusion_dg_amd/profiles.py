"""Summaries of rocprofv3 output for the repository's profiles/ folder.

  python -m block_discrete_diffusion_dg_amd.profiles stats <kernel_trace.csv> <out.md> --command "<cmd>"
  python -m block_discrete_diffusion_dg_amd.profiles traffic <fetch_csv> <write_csv> <out_stem>
      --kernel <name regex> --copy-bytes N --command-fetch "<cmd>" --command-write "<cmd>"
  python -m block_discrete_diffusion_dg_amd.profiles mfma <counter_csv> <out.md> --command "<cmd>"
      (counters MfmaUtil, MfmaFlopsBF16, GRBM_GUI_ACTIVE per dispatch)
  python -m block_discrete_diffusion_dg_amd.profiles counters <counter_csv> <out.md> --kernel-regex R --command "<cmd>"
      (any counters of the kernels matching R, with the wave-state ratios of SQ_RATIOS)

`traffic` turns FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) into HBM
bytes per launch of one kernel, scaled by what the same counter reads for a
plain device copy of known size, and records a hash of the kernel's sources:
bench.py reports the figure only while the sources still hash the same.

Every summary counts only the dispatches issued after the first dispatch of
the marker kernel (--after, default init_canvas_kernel): in `bench.py
--profile` the prefill runs before the canvas is set up, and everything after
it is denoising steps, so the prefill's launches of the same kernels (2,048
causal rows) do not enter the per-step averages.
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
N_XCD = 8  # accelerator complex dies; GRBM_GUI_ACTIVE is summed over them


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", name)


MARKER = "init_canvas_kernel"


def _dispatch_order(r) -> int:
    for key in ("Dispatch_Id", "Correlation_Id", "Start_Timestamp"):
        if r.get(key) not in (None, ""):
            return int(r[key])
    raise KeyError("no dispatch id or timestamp column")


def after_marker(rows, marker: str = MARKER):
    """The rows (one per dispatch, or per dispatch and counter) issued after
    the first dispatch of `marker`, and whether the marker was found (if not,
    every row is kept)."""
    marks = [_dispatch_order(r) for r in rows if marker and marker in r["Kernel_Name"]]
    if not marks:
        return list(rows), False
    first = min(marks)
    return [r for r in rows if _dispatch_order(r) > first], True


def _scope_line(found: bool, marker: str) -> str:
    return (f"Counted: dispatches after the first `{marker}` (the denoising steps; the prefill's launches "
            "come before it)." if found else f"Counted: every dispatch (no `{marker}` dispatch in the trace).")


def summarize_stats(csv_path: str, out_md: str, command: str, marker: str = MARKER) -> dict:
    """Per-dispatch kernel trace -> per-kernel calls and mean duration: library
    kernels first, then one line for everything the host framework launched
    (weight generation, copies)."""
    rows, found = after_marker(list(csv.DictReader(open(csv_path))), marker)
    per = defaultdict(list)
    for r in rows:
        per[_short(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    ours = {k: v for k, v in per.items() if "at::native" not in k and "rocclr" not in k and "__amd" not in k}
    other = [d for k, v in per.items() if k not in ours for d in v]
    lines = ["# Kernel time summary (rocprofv3 --kernel-trace --stats)", "",
             f"Command: `{command}`", "", _scope_line(found, marker), "",
             "Library kernels (the denoising path):", "",
             "| kernel | calls | avg us | total ms |", "|---|---:|---:|---:|"]
    out = {}
    for k, v in sorted(ours.items(), key=lambda kv: -sum(kv[1])):
        out[k] = {"calls": len(v), "avg_us": sum(v) / len(v)}
        lines.append(f"| {k[:60]} | {len(v)} | {sum(v) / len(v):.2f} | {sum(v) / 1e3:.2f} |")
    lines += ["", f"Other kernels in the same span (runtime copies and PyTorch): {len(other)} calls, "
                  f"{sum(other) / 1e3:.1f} ms in total."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out


def _per_dispatch(csv_path: str, counter: str, marker: str = MARKER):
    """Counter values per kernel name, for the dispatches after the marker
    (the copy probe runs after the timed steps, so it is among them)."""
    rows, found = after_marker(list(csv.DictReader(open(csv_path))), marker)
    per = defaultdict(list)
    for r in rows:
        if r["Counter_Name"] == counter:
            per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per, found


def summarize_traffic(fetch_csv: str, write_csv: str, out_stem: str, kernel: str, kernel_regex: str,
                      copy_bytes: int, command_fetch: str, command_write: str, marker: str = MARKER) -> dict:
    fetch, found_f = _per_dispatch(fetch_csv, "FETCH_SIZE", marker)
    write, found_w = _per_dispatch(write_csv, "WRITE_SIZE", marker)
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
        "after_marker": marker if found_f and found_w else None,
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
          f"WRITE_SIZE command: `{command_write}`", "", _scope_line(found_f and found_w, marker), "",
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


def summarize_mfma(csv_path: str, out_md: str, command: str, marker: str = MARKER) -> dict:
    """Per kernel class: mean MfmaUtil (percent of SIMD cycles with the matrix
    core busy while the dispatch ran), bf16 MFMA flops per dispatch, and the
    GPU-active cycles per dispatch. GRBM_GUI_ACTIVE counts busy cycles of each
    of the 8 XCDs and rocprofv3 sums them, so the dispatch's active time is
    the sum / 8 at the 2.4 GHz peak clock."""
    per = defaultdict(lambda: defaultdict(list))
    rows, found = after_marker(list(csv.DictReader(open(csv_path))), marker)
    for r in rows:
        per[r["Counter_Name"]][r["Kernel_Name"]].append(float(r["Counter_Value"]))
    out = {}
    lines = ["# Matrix-core use per kernel (rocprofv3 --pmc)", "", f"Command: `{command}`", "",
             "MfmaUtil is rocprofv3's derived metric: SQ_VALU_MFMA_BUSY_CYCLES summed over the SIMDs over "
             "GRBM_GUI_ACTIVE times the SIMD count, during each dispatch (counters serialise the dispatches). "
             "MfmaFlopsBF16 = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512. GRBM_GUI_ACTIVE is summed over the 8 XCDs, "
             "so active time = GRBM_GUI_ACTIVE / 8 / 2.4 GHz, and rate = flops / active time; the dense bf16 "
             "peak is 2.5 PFLOP/s. Collecting counters lengthens short dispatches, so active times run above "
             "the kernel-trace durations.", "", _scope_line(found, marker), "",
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
        t = a / N_XCD / GPU_CLOCK_HZ
        rate = f / t / 1e12 if t > 0 else 0.0
        out[label] = {"dispatches": len(util), "mfma_util_pct": u, "gflop": f / 1e9, "active_us": t * 1e6,
                      "tflops": rate}
        lines.append(f"| {label} | {len(util)} | {u:.1f} | {f / 1e9:.3f} | {t * 1e6:.1f} | {rate:.0f} | "
                     f"{rate / 2500:.3f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return out


# Wave-state counters of the shader sequencer and their ratios: wave-cycle
# counters share one unit, so their ratios to SQ_WAVE_CYCLES are fractions of
# the time waves were resident; bank conflicts are per LDS instruction cycle.
SQ_RATIOS = [("waiting (any)", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
             ("waiting for an instruction to issue", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
             ("issuing (any)", "SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES"),
             ("issuing LDS instructions", "SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES"),
             ("waiting to issue an LDS instruction", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"),
             ("LDS bank-conflict cycles per LDS issue cycle", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS")]


def summarize_counters(csv_path: str, out_md: str, kernel_regex: str, command: str,
                       marker: str = MARKER) -> dict:
    """Mean per dispatch of every counter in the file for the kernels matching
    kernel_regex (after the marker), and the SQ_RATIOS that the file holds."""
    rows, found = after_marker(list(csv.DictReader(open(csv_path))), marker)
    rx = re.compile(kernel_regex)
    per = defaultdict(list)
    for r in rows:
        if rx.search(r["Kernel_Name"]):
            per[r["Counter_Name"]].append(float(r["Counter_Value"]))
    means = {k: sum(v) / len(v) for k, v in sorted(per.items())}
    ratios = {label: means[a] / means[b] for label, a, b in SQ_RATIOS
              if a in means and b in means and means[b] > 0}
    lines = [f"# Counters of `{kernel_regex}` (rocprofv3 --pmc)", "", f"Command: `{command}`", "",
             _scope_line(found, marker), "",
             "| counter | dispatches | mean per dispatch |", "|---|---:|---:|"]
    lines += [f"| {k} | {len(per[k])} | {v:.6g} |" for k, v in means.items()]
    if ratios:
        lines += ["", "| ratio | value |", "|---|---:|"]
        lines += [f"| {label} | {v:.3f} |" for label, v in ratios.items()]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return {"means": means, "ratios": ratios}


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
    s.add_argument("--after", default=MARKER)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("out_stem")
    t.add_argument("--kernel", required=True)
    t.add_argument("--kernel-regex", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--after", default=MARKER)
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    m.add_argument("out")
    m.add_argument("--command", required=True)
    m.add_argument("--after", default=MARKER)
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("out")
    c.add_argument("--kernel-regex", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--after", default=MARKER)
    a = ap.parse_args()
    if a.cmd == "stats":
        print(json.dumps(summarize_stats(a.csv, a.out, a.command, a.after), indent=1))
    elif a.cmd == "mfma":
        print(json.dumps(summarize_mfma(a.csv, a.out, a.command, a.after), indent=1))
    elif a.cmd == "counters":
        print(json.dumps(summarize_counters(a.csv, a.out, a.kernel_regex, a.command, a.after), indent=1))
    else:
        print(json.dumps(summarize_traffic(a.fetch_csv, a.write_csv, a.out_stem, a.kernel, a.kernel_regex,
                                           a.copy_bytes, a.command_fetch, a.command_write, a.after), indent=1))


if __name__ == "__main__":
    main()
