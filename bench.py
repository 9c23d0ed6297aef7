"""Benchmark of the DualQuant dual-scale BCD solver on one MI355X.

One step = the whole hot path over one synthetic input: a dual-scale solve of a
down_proj-shaped 4096x14336 bf16 weight to NVFP4 (16 BCD iterations: init, sweeps,
finalizes, output pack), then the activation rescale-and-quantize of a 2048-token bf16
batch with the column scales the solve produced.  Inputs are resident in HBM before the
timed region.

Printed (one JSON line): whole-job throughput in Gelem/s per iteration (rows*cols*T /
step time); the roofline of the dominant kernel -- whichever of the row pass and the column
pass takes longer per step -- as algorithmic bytes (one read of W plus the scale vectors)
over its average launch duration from HIP event pairs attached to its launches in the timed
region, against the 8 TB/s HBM peak, with the counter-measured traffic recorded under
profiles/ when the kernel source is unchanged; and the CPU oracle timed on a bounded sample
on this host.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
  python bench.py --copy-calibration     # plain copy of known size, for counter scaling
  python bench.py --workload llama31_8b_nvfp4 --steps 3 --warmup 1   # the batched 224-matrix set
  python bench.py --workload linear_w4a4_mxfp4   # the quantised linear layer on solved codes
  python bench.py --workload linear_w4a4_nvfp4   # the same layer in NVFP4 (f16 cores)
  python bench.py --workload qkv_acts_nvfp4      # fused q/k/v activation quantise
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0
WORKLOAD = "down4096x14336_nvfp4"
ACT_TOKENS = 2048
METRIC = "BCD solver Gelem/s per iteration + achieved HBM GB/s vs peak (4096×14336 NVFP4)"


KERNELS = ("k_rowpass", "k_colpass", "k_finalize")
# The row pass is bound by VALU issue: 377 VALU instructions per 16-element chunk in a normal
# sweep (NVFP4 codes, bf16 weight; counted in the gfx950 assembly) against 256 CUs x 64 lanes
# x 2.4 GHz = 39.3 T lane-operations/s (unpacked fp32).
ROWPASS_VALU_PER_ELEM = {("NVFP4", 2): 377 / 16}
VALU_PEAK_LANE_OPS = 256 * 64 * 2.4e9


def recorded_traffic(kernel: str, workload: str):
    """Counter-measured HBM bytes per launch of `kernel` from profiles/, if the counters were
    taken on the current kernel source."""
    f = ROOT / "profiles" / f"{kernel}_{workload}_counters.md"
    if not f.exists():
        return None
    text = f.read_text()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    from post_quantization_dq_amd.profiling import kernel_source_hash

    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def copy_calibration():
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)


def cpu_baseline(W, X, fmt, iters):
    """The oracle on this host's cores, timed on one whole step of the same workload (the
    T-iteration solve of W, then the activation rescale-and-quantise of X)."""
    import oracle

    cores = min(16, os.cpu_count() or 1)
    oracle.set_threads(cores)
    steps, t0 = 0, time.perf_counter()
    while steps < 3 and (steps == 0 or time.perf_counter() - t0 < 10.0):   # 10 s of work or more
        res = oracle.solve(W, fmt, iters)
        oracle.rescale_quantize_acts(X, res["c"], fmt)
        steps += 1
    dt = (time.perf_counter() - t0) / steps
    m, n = W.shape
    return {"value": m * n * iters / dt / 1e9, "unit": "Gelem/s", "cores": cores, "kind": "oracle",
            "sample": f"{steps} whole steps: {m}x{n} bf16 {fmt} solve with {iters} BCD iterations "
                      f"plus the {X.shape[0]}x{n} activation quantise ({dt:.1f} s per step on "
                      f"{cores} threads)"}


def bench_llama_set(args):
    """The batched synthetic Llama-3.1-8B projection set (224 matrices, NVFP4, T = 20) as one
    dq_solve call; weights drawn on the GPU (the set is 14 GB)."""
    import torch

    import post_quantization_dq_amd as dq
    import synth

    dev = torch.device("cuda:0")
    T = 20
    probs = []
    for layer in range(synth.LLAMA31_8B_LAYERS):
        for pi in range(len(synth.LLAMA31_8B_PROJ)):
            W = synth.matrix_device(synth.llama_projection_spec(layer, pi), 0, dev)
            probs.append(dq.make_problem(W, "NVFP4", T))
    elems = sum(p.W.numel() for p in probs)
    print(f"[bench] llama31_8b_nvfp4: {len(probs)} matrices, {elems / 1e9:.2f} G bf16 weights, T={T}", flush=True)
    spec = dq.spec_of("NVFP4", None)
    ws = torch.empty(dq.dq_workspace_bytes(probs, spec, dq.dq_solve_opts(T, 0.0, None, 0, 0)),
                     dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        dq.solve_many(probs, "NVFP4", T, workspace=ws)
    torch.cuda.synchronize()
    passes = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(args.steps):
        dq.solve_many(probs, "NVFP4", T, workspace=ws, pass_ms=passes if k == args.steps - 1 else None)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    per_all = np.asarray(passes, dtype=np.float64).reshape(-1, 3)
    # Sweeps 1..T run every matrix.  The INIT sweep is lighter, and the re-solve sweeps after
    # rejections only run the matrices that rejected, so both stay out of the per-pass figures.
    per = per_all[1:T + 1]
    avg = {k: float(per[:, q].mean()) for q, k in enumerate(KERNELS)}
    dom = max(KERNELS[:2], key=lambda k: float(per[:, KERNELS.index(k)].sum()))
    alg_bytes = elems * 2 + 8 * sum(p.W.shape[0] + p.W.shape[1] for p in probs)
    achieved = alg_bytes / (avg[dom] * 1e-3) / 1e9
    out = {
        "metric": "BCD solver Gelem/s per iteration (batched Llama-3.1-8B projection set, NVFP4)",
        "value": round(elems * T / (ms_step * 1e-3) / 1e9, 3), "unit": "Gelem/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "224 Llama-3.1-8B-shaped projections (32 layers x q,k,v,o,gate,up,down), "
                               "bf16 Student-t nu=4 std 0.02, 1% outlier columns x15, NVFP4, 20 BCD "
                               "iterations, one batched dq_solve", "elements": elems, "iters": T},
        "roofline": {"bound": "hbm", "kernel": dom + " (all groups of one pass)", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "alg_bytes_per_launch": alg_bytes, "avg_launch_ms": round(avg[dom], 4),
                     "launches": int(per.shape[0])},
        "kernel_avg_us": {k: round(avg[k] * 1e3, 1) for k in KERNELS},
        "sweeps_per_solve": int(per_all.shape[0]),
    }
    print(json.dumps(out), flush=True)


FP4_MFMA_PEAK_TFLOPS = 10100.0   # MI355X dense FP4 matrix-core peak
F16_MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 / bf16 matrix-core peak


def bench_linear(args, fmt):
    """The quantised linear layer on codes the solver and the activation quantiser made:
    the q_proj-shaped 4096x4096 weight solved to `fmt` (MXFP4 or NVFP4, T = 16), 2048 tokens
    of activations rescaled by the solved c and quantised to the same format,
    Y = Aq Q^T diag(r) in bf16.  MXFP4 runs on the FP4 block-scaled matrix cores, NVFP4 on
    the f16 cores after an exact dequantisation in the kernel."""
    import torch

    import post_quantization_dq_amd as dq
    import synth

    dev = torch.device("cuda:0")
    W, _, _, _, T = synth.workload("q4096x4096_mxfp4")
    N, K = W.shape
    M = ACT_TOKENS
    X = synth.matrix(synth.WORKLOADS["k1024x4096_mxint4"]["X"].scaled(M, K), 0)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    res = dq.solve(to_dev(W), fmt, T)
    ac, asc, ats = dq.rescale_quantize_acts(to_dev(X), res["c"], fmt)
    nv = fmt == "NVFP4"
    bts = res["tscale"] if nv else None
    ats = ats if nv else None
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    spec = dq.spec_of(fmt)
    call = lambda: dq.dq_quantized_linear(spec, ac, asc, ats, M, res["codes"], res["scales"], bts, N, K,
                                          res["r"], y)
    print(f"[bench] quantised linear {fmt}: Y[{M}x{N}] = A[{M}x{K}] Q^T diag(r), bf16 out", flush=True)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flops = 2.0 * M * N * K
    tflops = flops / (ms * 1e-3) / 1e12
    peak = F16_MFMA_PEAK_TFLOPS if nv else FP4_MFMA_PEAK_TFLOPS
    out = {
        "metric": f"quantised linear layer TFLOP/s (W4A4 {fmt} codes from the solver)",
        "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": fmt.lower(), "data": "synthetic",
        "config": {"workload": f"q_proj-shaped {N}x{K} weight solved to {fmt} (T={T}); {M} tokens of "
                               f"activations rescaled by the solved c and quantised to {fmt}; bf16 output",
                   "M": M, "N": N, "K": K},
        "roofline": {"bound": "mfma", "kernel": "k_linear_nv_dma" if nv else "k_linear_dma",
                     "achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None,
                     "alg_flops_per_launch": flops, "avg_launch_ms": round(ms, 4),
                     "cores": "f16 (exact e2m1 x e4m3 elements)" if nv else "fp4 block-scaled"},
        "wall_ms_per_call": round(wall * 1e3, 4),
    }
    print(json.dumps(out), flush=True)


def bench_qkv_acts(args):
    """The fused multi-projection activation quantiser: 2048 tokens x 4096 bf16 activations
    quantised to NVFP4 for three projections (q, k, v), each with its own column scales, in
    one dq_rescale_quantize_acts_multi call; three single calls are timed beside it."""
    import torch

    import post_quantization_dq_amd as dq
    import synth

    dev = torch.device("cuda:0")
    fmt, M, K, n_out = "NVFP4", ACT_TOKENS, 4096, 3
    X = synth.matrix(synth.WORKLOADS["k1024x4096_mxint4"]["X"].scaled(M, K), 0)
    Xd = torch.from_numpy(np.ascontiguousarray(X).view(np.int16)).view(torch.bfloat16).to(dev)
    rng = np.random.default_rng(5)
    cs = [torch.from_numpy(np.exp2(rng.integers(-3, 4, K)).astype(np.float32)).to(dev) for _ in range(n_out)]
    spec = dq.spec_of(fmt)
    outs = [dq._outputs(M, K, fmt, dq.DEFAULT_GROUP[fmt], dev) for _ in cs]
    ws = torch.empty(dq.dq_quantize_multi_workspace_bytes(M, K, n_out, spec), dtype=torch.uint8, device=dev)
    multi = lambda: dq.dq_rescale_quantize_acts_multi(Xd, cs, spec, [o[0] for o in outs],
                                                      [o[1] for o in outs], [o[2] for o in outs], ws)

    def singles():
        for c, o in zip(cs, outs):
            dq.dq_rescale_quantize_acts(Xd, c, spec, o[0], o[1], o[2], ws)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    ms_multi, ms_single = timed(multi), timed(singles)
    # algorithmic bytes: X read twice (amax pre-pass, quantise), codes + block scales written
    alg = 2 * M * K * 2 + n_out * (M * K // 2 + M * K // 16)
    gbs = alg / (ms_multi * 1e-3) / 1e9
    out = {
        "metric": "fused q/k/v activation quantise (NVFP4), tokens per second",
        "value": round(M / (ms_multi * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_multi, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{M}x{K} bf16 activations, {n_out} outputs with their own column "
                               f"scales, NVFP4", "tokens": M, "cols": K, "outputs": n_out},
        "roofline": {"bound": "hbm", "kernel": "k_qamax_multi + k_quant_multi", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None, "alg_bytes_per_call": alg},
        "three_single_calls_ms": round(ms_single, 4),
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # default: 200 steps of a single-matrix workload, so that the one timed step that also
    # carries per-launch events (for the roofline) adds under 0.5% to the mean; 5 steps of
    # the 224-matrix set; 20 of the layer and activation benchmarks
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--format", default=None,
                    help="solve the workload's weight in another format (e.g. INT8, MXINT8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = {"llama31_8b_nvfp4": 5, "linear_w4a4_mxfp4": 20, "linear_w4a4_nvfp4": 20,
                      "qkv_acts_nvfp4": 20}.get(args.workload, 200)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the solve runs on a single MI355X and the library "
              "has no multi-GPU path (pass --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.workload == "llama31_8b_nvfp4":
        bench_llama_set(args)
        return
    if args.workload in ("linear_w4a4_mxfp4", "linear_w4a4_nvfp4"):
        bench_linear(args, args.workload.rsplit("_", 1)[1].upper())
        return
    if args.workload == "qkv_acts_nvfp4":
        bench_qkv_acts(args)
        return

    import torch

    import post_quantization_dq_amd as dq
    import synth

    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    fmt, group, T = wl["fmt"], wl["group"], wl["iters"]
    if args.format:
        fmt, group = args.format, None
    W_np = synth.matrix(wl["W"], 0)
    m, n = W_np.shape
    xspec = synth.MatrixSpec(ACT_TOKENS, n, "normal", 1.0, outliers=synth.outlier_count(n, 0.01),
                             outlier_scale=50.0, stream=9)
    X_np = synth.matrix(xspec, 0)
    W = torch.from_numpy(W_np.view(np.int16)).view(torch.bfloat16).to(dev)
    X = torch.from_numpy(X_np.view(np.int16)).view(torch.bfloat16).to(dev)
    print(f"[bench] workload {args.workload}: W {m}x{n} bf16, {fmt}, T={T}; acts {ACT_TOKENS}x{n}", flush=True)

    prob = dq.make_problem(W, fmt, T, group)
    spec = dq.spec_of(fmt, group)
    ws = torch.empty(dq.dq_workspace_bytes([prob], spec, dq.dq_solve_opts(T, 0.0, None, 0, 0)),
                     dtype=torch.uint8, device=dev)
    a_codes, a_scales, a_ts = dq._outputs(ACT_TOKENS, n, fmt, group or dq.DEFAULT_GROUP[fmt], dev)
    a_ws = torch.empty(max(1, dq.dq_quantize_workspace_bytes(ACT_TOKENS, n, spec)), dtype=torch.uint8, device=dev)

    def step(passes=None):
        rep = dq.solve_many([prob], fmt, T, group, workspace=ws, pass_ms=passes)[0]
        dq.dq_rescale_quantize_acts(X, prob.c, spec, a_codes, a_scales, a_ts, a_ws)
        return rep

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    passes = []
    reps = []
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for k in range(args.steps):
        # the last timed step also records a begin/end event pair on each solver kernel launch
        reps.append(step(passes if k == args.steps - 1 else None))
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f} ms)", flush=True)

    # per-kernel launch durations from the sampled step (event pairs attached to the launches)
    per = np.asarray(passes, dtype=np.float64).reshape(-1, 3)
    avg = {k: float(per[:, q].mean()) for q, k in enumerate(KERNELS)}
    per_step = {k: float(per[:, q].sum()) for q, k in enumerate(KERNELS)}
    dom = max(KERNELS[:2], key=lambda k: per_step[k])
    print("[bench] per-launch ms: " + ", ".join(f"{k} {avg[k] * 1e3:.1f} us" for k in KERNELS), flush=True)
    # algorithmic bytes of one pass over W: one read of W plus the r and c vectors
    alg_bytes = m * n * W.element_size() + 8 * (m + n)
    achieved = alg_bytes / (avg[dom] * 1e-3) / 1e9
    t_iter_ms = float(per.sum(axis=1).mean())
    traffic = recorded_traffic(dom, args.workload)
    nm = prob.nmse_hist.cpu().numpy()
    value = m * n * T / (ms_step * 1e-3) / 1e9

    out = {
        "metric": METRIC if (m, n, fmt) == (4096, 14336, "NVFP4")
                  else METRIC.replace("(4096×14336 NVFP4)", f"({m}×{n} {fmt})"),
        "value": round(value, 3),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {m}x{n} bf16 weight ({wl['W'].dist}, std {wl['W'].std}, "
                        f"{wl['W'].outliers} outlier columns x{wl['W'].outlier_scale:g}), {fmt} "
                        f"g={group or dq.DEFAULT_GROUP[fmt]}, {T} BCD iterations; then "
                        f"{ACT_TOKENS}x{n} bf16 activations rescaled by c and {fmt}-quantised",
            "rows": m, "cols": n, "format": fmt, "iters": T, "act_tokens": ACT_TOKENS,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": alg_bytes,
            "avg_launch_ms": round(avg[dom], 5),
            "launches": int(per.shape[0]),
        },
        "kernel_avg_us": {k: round(avg[k] * 1e3, 2) for k in KERNELS},
        "iteration_us": round(t_iter_ms * 1e3, 2),
        "iteration_hbm_frac": round(alg_bytes / (t_iter_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "sweeps_per_step": int(reps[-1].sweeps),
        "rejected_steps": int(reps[-1].rejected_steps),
        "nmse_first_last": [float(nm[0]), float(nm[-1])],
    }
    vpe = ROWPASS_VALU_PER_ELEM.get((fmt, W.element_size()))
    if dom == "k_rowpass" and vpe is not None:
        # the roof that binds the row pass: VALU lane-operations per second
        lane_ops = m * n * vpe / (avg[dom] * 1e-3)
        out["roofline"]["valu"] = {"instr_per_elem": round(vpe, 3),
                                   "achieved_lane_ops": round(lane_ops / 1e12, 2),
                                   "peak_lane_ops": round(VALU_PEAK_LANE_OPS / 1e12, 2),
                                   "unit": "T lane-ops/s",
                                   "frac": round(lane_ops / VALU_PEAK_LANE_OPS, 4)}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample ...", flush=True)
        out["cpu_baseline"] = cpu_baseline(W_np, X_np, fmt, T)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
