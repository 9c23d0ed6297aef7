"""Summaries of rocprofv3 output for the solver kernels (kernel-trace statistics and the
FETCH_SIZE / WRITE_SIZE counter passes), written as short markdown files.

  python -m post_quantization_dq_amd.profiling stats TRACE_DIR OUT.md --command "..."
  python -m post_quantization_dq_amd.profiling counters FETCH_DIR WRITE_DIR CFETCH_DIR \\
      CWRITE_DIR OUT.md --kernel k_rowpass --kernel k_colpass --kernel k_finalize \\
      --alg-bytes N --copy-bytes 1073741824 --command "..."
  python -m post_quantization_dq_amd.profiling sq OUT.md DIR [DIR ...] --kernel k_rowpass \\
      --command "..."

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
    """rocprofv3's per-kernel statistics, plus the mean over the launches that did work: a
    solve queues sweeps that exit at once once it has finished, and those launches (shorter
    than 20% of the kernel's longest) are left out of the 'working' columns."""
    rows = list(csv.DictReader(open(_find(trace_dir, "kernel_stats.csv"))))
    durs = {}
    for r in csv.DictReader(open(_find(trace_dir, "kernel_trace.csv"))):
        durs.setdefault(_short(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# Kernel trace statistics", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share (%) | working calls | working average (us) |",
             "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        k = _short(r["Name"])
        d = durs.get(k, [])
        w = [x for x in d if x >= 0.2 * max(d)] if d else []
        wa = f"{statistics.mean(w):.2f}" if w else ""
        lines.append(f"| `{k}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} | {len(w)} | {wa} |")
    lines += ["", f"kernel_source_sha256: {kernel_source_hash()}", ""]
    return "\n".join(lines)


def _counter_means(d: str, counter: str) -> dict:
    """Per kernel: the counter's values over the dispatches that did work.  A solve queues
    sweeps that exit at once when the solve is already finished; their dispatches read next to
    nothing and are left out (values below 5% of the kernel's largest)."""
    per = {}
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: [x for x in v if x >= 0.05 * max(v)] or v for k, v in per.items()}


def counters_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, kernels, copy_bytes,
                     alg_bytes, command) -> str:
    """`kernels`: names whose per-launch traffic is recorded (their sum is the traffic of one
    solver iteration when they are the row pass, column pass and finalize); `alg_bytes`:
    algorithmic bytes of one launch of the first of them."""
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
             "Means over the dispatches that did work (queued sweeps that found the solve "
             "finished are left out).", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |",
             "|---|---|---|---|---|---|"]
    per = {}
    for name in sorted(set(fe) | set(wr)):
        if "dqk" not in name:
            continue
        f = statistics.mean(fe.get(name, [0.0]))
        w = statistics.mean(wr.get(name, [0.0]))
        rb, wb = f * 1024.0 * f_scale, w * 1024.0 * w_scale
        lines.append(f"| `{_short(name)}` | {len(fe.get(name, []))} | {f:.1f} | {w:.1f} | {rb / 1e6:.2f} | {wb / 1e6:.2f} |")
        for k in kernels:
            if _short(name).startswith(k + "<"):
                per[k] = (rb, wb)
    missing = [k for k in kernels if k not in per]
    if missing:
        raise ValueError(f"kernels {missing} not in the counter output")
    tot = sum(rb + wb for rb, wb in per.values())
    k0 = kernels[0]
    lines += ["", f"Kernel `{k0}`: algorithmic bytes per launch {alg_bytes}; measured "
              f"{sum(per[k0]):.0f} bytes per launch ({sum(per[k0]) / alg_bytes:.3f} x algorithmic).",
              f"Sum over {', '.join('`' + k + '`' for k in kernels)}: {tot:.0f} bytes "
              f"({tot / alg_bytes:.3f} x the algorithmic bytes of one launch of `{k0}`).", "",
              f"kernel_source_sha256: {kernel_source_hash()}"]
    lines += [f"traffic_bytes_per_launch[{k}]: {sum(per[k]):.0f}" for k in kernels]
    lines += [f"traffic_bytes_per_iteration: {tot:.0f}", ""]
    return "\n".join(lines)


def totals_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, kernels, per, alg_bytes,
                   copy_bytes, command) -> str:
    """Traffic summed over every dispatch of each listed kernel, divided by `per` (e.g. the
    iterations of the profiled solves), for batched solves whose launch groups differ in
    shape; `alg_bytes`: algorithmic bytes of one iteration (one read of every weight)."""
    def sums(d, counter):
        out = {}
        for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
            if r["Counter_Name"] == counter:
                k = _short(r["Kernel_Name"])
                out[k] = out.get(k, 0.0) + float(r["Counter_Value"])
        return out

    def copy_kib(d, counter):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(_find(d, "counter_collection.csv")))
                if r["Counter_Name"] == counter and "copy" in r["Kernel_Name"].lower()]
        return statistics.median(vals)

    f_scale = copy_bytes / (copy_kib(cfetch_dir, "FETCH_SIZE") * 1024.0)
    w_scale = copy_bytes / (copy_kib(cwrite_dir, "WRITE_SIZE") * 1024.0)
    fe, wr = sums(fetch_dir, "FETCH_SIZE"), sums(write_dir, "WRITE_SIZE")
    lines = ["# HBM traffic counters, summed per iteration", "",
             "Command (one rocprofv3 --pmc pass per counter):", "", "```", command, "```", "",
             f"Scale factors from a plain copy: {f_scale:.4f} (fetch), {w_scale:.4f} (write).  "
             f"Every dispatch of a kernel summed, divided by {per}.", "",
             "| kernel | read GB per iteration | write GB per iteration |", "|---|---|---|"]
    tot = 0.0
    for k in sorted(set(fe) | set(wr)):
        if not any(k.startswith(x + "<") for x in kernels):
            continue
        rb = fe.get(k, 0.0) * 1024.0 * f_scale / per
        wb = wr.get(k, 0.0) * 1024.0 * w_scale / per
        tot += rb + wb
        lines.append(f"| `{k}` | {rb / 1e9:.3f} | {wb / 1e9:.3f} |")
    lines += ["", f"Per iteration: {tot / 1e9:.3f} GB measured against {alg_bytes / 1e9:.3f} GB "
              f"algorithmic ({tot / alg_bytes:.3f} x).", "",
              f"kernel_source_sha256: {kernel_source_hash()}",
              f"traffic_bytes_per_iteration: {tot:.0f}", ""]
    return "\n".join(lines)


def sq_summary(dirs, kernels, command) -> str:
    """Mean per dispatch of every counter in the given --pmc output directories, for the
    listed kernels (one row per kernel, one column per counter)."""
    vals = {}
    for d in dirs:
        for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
            k = _short(r["Kernel_Name"])
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    # as for the traffic counters: dispatches of queued sweeps that found the solve finished
    # are left out (values below 5% of the kernel's largest)
    vals = {k: {c: [x for x in v if x >= 0.05 * max(v)] or v for c, v in cs.items()}
            for k, cs in vals.items()}
    names = sorted({c for k in vals for c in vals[k]})
    lines = ["# Shader counters", "", "Command (one rocprofv3 --pmc pass per directory):", "", "```",
             command, "```", "",
             "Mean per dispatch, over the dispatches that did work.  VALUBusy: percent of the "
             "kernel's GPU time in which the vector ALUs issue (SQ_ACTIVE_INST_VALU per CU over "
             "GRBM_GUI_ACTIVE); MemUnitStalled: percent of it in which the memory unit is stalled.", "",
             "| kernel | " + " | ".join(names) + " |", "|---" * (len(names) + 1) + "|"]
    for k in sorted(vals):
        if not any(k.startswith(x + "<") for x in kernels):
            continue
        row = [f"{statistics.mean(vals[k][c]):.4g}" if c in vals[k] else "" for c in names]
        lines.append(f"| `{k}` | " + " | ".join(row) + " |")
    lines += ["", f"kernel_source_sha256: {kernel_source_hash()}", ""]
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
    c.add_argument("--kernel", action="append", required=True)
    c.add_argument("--copy-bytes", type=int, default=1 << 30)
    c.add_argument("--alg-bytes", type=int, required=True)
    c.add_argument("--command", required=True)
    t = sub.add_parser("totals")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("cfetch_dir")
    t.add_argument("cwrite_dir")
    t.add_argument("out")
    t.add_argument("--kernel", action="append", required=True)
    t.add_argument("--per", type=float, required=True)
    t.add_argument("--alg-bytes", type=int, required=True)
    t.add_argument("--copy-bytes", type=int, default=1 << 30)
    t.add_argument("--command", required=True)
    q = sub.add_parser("sq")
    q.add_argument("out")
    q.add_argument("dirs", nargs="+")
    q.add_argument("--kernel", action="append", required=True)
    q.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.what == "stats":
        text = stats_summary(a.trace_dir, a.command)
    elif a.what == "counters":
        text = counters_summary(a.fetch_dir, a.write_dir, a.cfetch_dir, a.cwrite_dir, a.kernel,
                                a.copy_bytes, a.alg_bytes, a.command)
    elif a.what == "totals":
        text = totals_summary(a.fetch_dir, a.write_dir, a.cfetch_dir, a.cwrite_dir, a.kernel,
                              a.per, a.alg_bytes, a.copy_bytes, a.command)
    else:
        text = sq_summary(a.dirs, a.kernel, a.command)
    Path(a.out).write_text(text)
    print(text)


if __name__ == "__main__":
    main()
