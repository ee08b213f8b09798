"""Turns rocprofv3 output into the short text summaries kept under profiles/.

    python -m quantized_grouped_gemm_amd.profiling copy [--mib 1024] [--reps 5]
        Runs a plain device copy of known size (torch elementwise kernel, MiB
        read + MiB written per launch): the calibration kernel for the HBM
        byte counters FETCH_SIZE and WRITE_SIZE.

    python -m quantized_grouped_gemm_amd.profiling stats STATS_CSV --cmd CMD --out FILE.md
        Renders a `rocprofv3 --kernel-trace --stats` kernel_stats.csv as a
        markdown table headed by the command that produced it.

    python -m quantized_grouped_gemm_amd.profiling traffic --kernel REGEX --workload NAME
            --fetch CSV --write CSV --copy-fetch CSV --copy-write CSV --copy-mib M
            [--per-step N] --cmd CMD --out profiles/traffic.json
        Averages FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the kernels
        matching REGEX, scales each by (known bytes / counted bytes) of the
        copy kernel, and records the HBM bytes per launch (times N when one
        step is N dispatches of the matching kernels, each once per step)
        together with a hash of the kernel sources, so that a later change to
        a kernel makes the figure stale.

This module only reads CSV files and launches one torch copy; it is not on
the compute path.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys

_PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("gemm_q4.hip", "common.h", "ffn.hip", "decode.hip", "gemv.h")


def _code_only(text: str) -> str:
    """The source without its comments and blank space: what the compiler sees
    (string literals in these files hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(files=KERNEL_SOURCES, root=None) -> str:
    """Hash of the kernels' code (comments and spacing ignored): counters taken
    on one hash stay valid while the code they measured is unchanged."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(root or os.path.join(_PKG, "csrc"), f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _copy(mib: int, reps: int) -> None:
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)   # reads mib MiB, writes mib MiB
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": mib, "reps": reps}), flush=True)


def counter_per_dispatch(path: str, counter: str, kernel_regex: str) -> tuple[float, int]:
    """Mean of `counter` over the dispatches whose kernel name matches."""
    rx = re.compile(kernel_regex)
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or not rx.search(r["Kernel_Name"]):
                continue
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for /{kernel_regex}/ in {path}")
    return sum(per.values()) / len(per), len(per)


def _stats(path: str, cmd: str, out: str, top: int) -> None:
    with open(path) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# rocprofv3 kernel statistics", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in rows[:top]:
        name = r["Name"]
        short = re.sub(r"\(.*$", "", name) if "moeq4" in name else name[:60]
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def _traffic(a) -> None:
    copy_bytes = a.copy_mib * (1 << 20)
    cf, _ = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_regex)
    cw, _ = counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_regex)
    kf, n1 = counter_per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    kw, n2 = counter_per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    f_fac = copy_bytes / (cf * 1024.0)
    w_fac = copy_bytes / (cw * 1024.0)
    ent = {
        "source_hash": kernel_source_hash(),
        "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw, "dispatches": [n1, n2],
        "copy_mib": a.copy_mib, "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": f_fac, "write_scale": w_fac,
        "dispatches_per_step": a.per_step,
        "bytes_per_launch": a.per_step * (kf * 1024.0 * f_fac + kw * 1024.0 * w_fac),
        "command": a.cmd,
    }
    d = {}
    if os.path.exists(a.out):
        with open(a.out) as f:
            d = json.load(f)
    d.setdefault(a.name, {})[a.workload] = ent
    with open(a.out, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({a.name: {a.workload: ent}}))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=5)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--top", type=int, default=12)
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True, help="regex over kernel names")
    t.add_argument("--name", required=True, help="key under which the figure is stored")
    t.add_argument("--workload", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    # the copy is torch.mul(src, 1.0, out=dst); the fill that creates src reads nothing
    t.add_argument("--copy-regex", default="MulFunctor")
    t.add_argument("--per-step", type=int, default=1, help="dispatches of the matching kernels per step")
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd_name == "copy":
        _copy(a.mib, a.reps)
    elif a.cmd_name == "stats":
        _stats(a.csv, a.cmd, a.out, a.top)
    else:
        _traffic(a)


if __name__ == "__main__":
    sys.exit(main())
