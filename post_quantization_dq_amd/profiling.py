"""Summaries of rocprofv3 output for the solver kernels (kernel-trace statistics and the
FETCH_SIZE / WRITE_SIZE counter passes), written as short markdown files.

  python -m post_quantization_dq_amd.profiling stats TRACE_DIR OUT.md --command "..."
  python -m post_quantization_dq_amd.profiling counters FETCH_DIR WRITE_DIR CFETCH_DIR \\
      CWRITE_DIR OUT.md --kernel k_rowpass --copy-bytes 1073741824 --command "..."

The counter summary scales each kernel's FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by
what the same counter reads for a plain device-to-device copy of known size, and records
the hash of the kernel sources it was taken on; bench.py only uses a traffic figure whose
hash matches the current sources.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics
from pathlib import Path

HERE = Path(__file__).resolve().parent


def kernel_source_hash() -> str:
    """Hash of everything that decides the device code: every source under csrc/ (kernels,
    launch code) and the compiler flags of the build."""
    from .build import FLAGS

    h = hashlib.sha256()
    for f in sorted((HERE / "csrc").iterdir()):
        if f.suffix in (".hip", ".hpp", ".h"):
            h.update(f.name.encode())
            h.update(f.read_bytes())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    base = name.split("(")[0].replace("void ", "")
    return base.replace("dqk::", "")


def _find(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def stats_summary(trace_dir: str, command: str) -> str:
    rows = list(csv.DictReader(open(_find(trace_dir, "kernel_stats.csv"))))
    lines = ["# Kernel trace statistics", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share (%) |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    lines += ["", f"kernel_source_sha256: {kernel_source_hash()}", ""]
    return "\n".join(lines)


def _counter_means(d: str, counter: str) -> dict:
    per = {}
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def counters_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, kernel, copy_bytes,
                     alg_bytes, command) -> str:
    fe, wr = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    cf, cw = _counter_means(cfetch_dir, "FETCH_SIZE"), _counter_means(cwrite_dir, "WRITE_SIZE")

    def copy_kib(d):
        vals = [v for k, vs in d.items() if "copy" in k.lower() for v in vs]
        return statistics.median(vals)

    fk, wk = copy_kib(cf), copy_kib(cw)
    f_scale, w_scale = copy_bytes / (fk * 1024.0), copy_bytes / (wk * 1024.0)
    lines = ["# HBM traffic counters", "", "Command (one rocprofv3 --pmc pass per counter):", "",
             "```", command, "```", "",
             f"Plain copy of {copy_bytes} bytes: FETCH_SIZE {fk:.1f} KiB, WRITE_SIZE {wk:.1f} KiB per "
             f"dispatch -> scale factors {f_scale:.4f} (fetch), {w_scale:.4f} (write).", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |",
             "|---|---|---|---|---|---|"]
    target = None
    for name in sorted(set(fe) | set(wr)):
        if "dqk" not in name:
            continue
        f = statistics.mean(fe.get(name, [0.0]))
        w = statistics.mean(wr.get(name, [0.0]))
        rb, wb = f * 1024.0 * f_scale, w * 1024.0 * w_scale
        lines.append(f"| `{_short(name)}` | {len(fe.get(name, []))} | {f:.1f} | {w:.1f} | {rb / 1e6:.2f} | {wb / 1e6:.2f} |")
        if _short(name).startswith(kernel + "<"):
            target = (rb, wb)
    if target is None:
        raise ValueError(f"kernel {kernel} not in the counter output")
    lines += ["", f"Kernel: `{kernel}`; algorithmic bytes per launch {alg_bytes}; measured "
              f"{target[0] + target[1]:.0f} bytes per launch "
              f"({(target[0] + target[1]) / alg_bytes:.3f} x algorithmic).", "",
              f"kernel_source_sha256: {kernel_source_hash()}",
              f"traffic_bytes_per_launch: {target[0] + target[1]:.0f}", ""]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("trace_dir")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("fetch_dir")
    c.add_argument("write_dir")
    c.add_argument("cfetch_dir")
    c.add_argument("cwrite_dir")
    c.add_argument("out")
    c.add_argument("--kernel", required=True)
    c.add_argument("--copy-bytes", type=int, default=1 << 30)
    c.add_argument("--alg-bytes", type=int, required=True)
    c.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.what == "stats":
        text = stats_summary(a.trace_dir, a.command)
    else:
        text = counters_summary(a.fetch_dir, a.write_dir, a.cfetch_dir, a.cwrite_dir, a.kernel,
                                a.copy_bytes, a.alg_bytes, a.command)
    Path(a.out).write_text(text)
    print(text)


if __name__ == "__main__":
    main()
