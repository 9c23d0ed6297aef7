"""dq_solve against the oracle.

  * end to end on every workload (full sizes and reduced ones with ragged shapes):
    nmse/relchg histories within 1e-5 relative, final scales within 1e-5 relative,
    at most 1e-4 of the codes different, same tensor scale;
  * teacher-forced single iterations from realistic states: unprojected closed forms
    within 1e-5 relative, projected scales equal except where the oracle's value sits
    within 1e-5 of a projection boundary, Qhat^0 codes bit-exact;
  * determinism (bitwise repeatable), batching (a batch equals its members solved
    alone), the rejection / re-solve path, early stop, empty and degenerate inputs.
"""

import numpy as np
import pytest
import torch

import post_quantization_dq_amd as dq
import synth
from gpu_util import (ALL_FORMATS, DEV, FORMATS, GROUPS, elements, near_projection_boundary, rel_err,
                      scales_np, to_dev)

pytestmark = pytest.mark.gpu


def _gpu_solve(W, fmt, iters, **kw):
    out = dq.solve(to_dev(W), fmt, iters, **kw)
    torch.cuda.synchronize()
    res = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}
    res["scales"] = scales_np(out["scales"], fmt)
    res["tscale"] = float(out["tscale"].item())
    return res


def _first_divergence(oracle, fmt, ref, got, T):
    """First iteration at which a projected scale differs between the two trajectories.
    Up to there every unprojected closed form must agree within 1e-5 relative, and each
    difference at that iteration must be an oracle-flagged boundary case (the oracle's value
    within 1e-6 of a projection boundary), where both neighbours are equally valid."""
    for t in range(1, T + 1):
        for key in ("r_trace", "c_trace"):
            a, b = ref[key][t - 1], got[key][t - 1]
            assert np.array_equal(np.isnan(a), np.isnan(b)), (key, t)
            ok = ~np.isnan(a)
            assert np.all(rel_err(b[ok], a[ok]) <= 1e-5), (key, t, rel_err(b[ok], a[ok]).max())
            pa, pb = oracle.project(fmt, a[ok]), oracle.project(fmt, b[ok])
            diff = pa != pb
            if diff.any():
                flagged = near_projection_boundary(oracle, fmt, a[ok][diff], 1e-6)
                assert np.all(flagged), (key, t, a[ok][diff][~flagged], b[ok][diff][~flagged])
                return t
    return T + 1


def _compare_e2e(oracle, ref, got, fmt, what, T):
    assert got["iters_run"] == ref["iters_run"] == T
    t_div = _first_divergence(oracle, fmt, ref, got, T)
    k = min(t_div, T + 1)
    assert np.all(rel_err(got["nmse"][:k], ref["nmse"][:k], 1e-30) <= 1e-5), (what, got["nmse"], ref["nmse"])
    d = np.abs(got["relchg"][:k] - ref["relchg"][:k])
    assert np.all(d <= 1e-5 * np.abs(ref["relchg"][:k]) + 1e-9), (what, got["relchg"], ref["relchg"])
    assert np.all(np.diff(got["nmse"]) <= 0.0), what
    if t_div > T:
        assert np.all(rel_err(got["r"], ref["r"]) <= 1e-5), what
        assert np.all(rel_err(got["c"], ref["c"]) <= 1e-5), what
        nb = elements(got["codes"], fmt) != elements(ref["codes"], fmt)
        assert nb.mean() <= 1e-4, (what, nb.sum())
        assert (got["scales"] != ref["scales"]).mean() <= 1e-4, what
        if fmt == "NVFP4":
            assert rel_err(got["tscale"], ref["tscale"]) <= 1e-5, what
        assert got["rejected"] == ref["rejected"], what
    else:
        # after a flagged boundary flip the two trajectories are different valid descents
        assert np.all(rel_err(got["nmse"], ref["nmse"], 1e-30) <= 2e-3), (what, t_div, got["nmse"], ref["nmse"])
        print(f"[e2e] {what}: flagged boundary divergence at iteration {t_div}", flush=True)
    return t_div


E2E_SMALL = [
    ("w256x512_int4", 256, 512, 16),
    ("q4096x4096_mxfp4", 301, 1024, 12),
    ("down4096x14336_nvfp4", 197, 9216, 16),     # two chunks per lane, ragged strips
    ("down4096x14336_nvfp4", 64, 1792, 20),
    ("k1024x4096_mxint4", 129, 2048, 16),
]


@pytest.mark.parametrize("name,rows,cols,iters", E2E_SMALL)
def test_end_to_end_reduced(oracle_lib, name, rows, cols, iters):
    w = synth.WORKLOADS[name]
    W = synth.matrix(w["W"].scaled(rows, cols), 0)
    ref = oracle_lib.solve(W, w["fmt"], iters)
    got = _gpu_solve(W, w["fmt"], iters, trace=True)
    _compare_e2e(oracle_lib, ref, got, w["fmt"], name, iters)


# the 8-bit formats on the same recipes (INT8 with both groups, fp32 and bf16 inputs)
E2E_8BIT = [
    ("INT8", 128, "w256x512_int4", 256, 512, 16),
    ("INT8", 64, "down4096x14336_nvfp4", 197, 9216, 12),
    ("MXINT8", 32, "k1024x4096_mxint4", 129, 2048, 12),
    ("MXINT8", 32, "q4096x4096_mxfp4", 256, 4096, 8),
]


@pytest.mark.parametrize("fmt,group,name,rows,cols,iters", E2E_8BIT)
def test_end_to_end_8bit(oracle_lib, fmt, group, name, rows, cols, iters):
    W = synth.matrix(synth.WORKLOADS[name]["W"].scaled(rows, cols), 0)
    ref = oracle_lib.solve(W, fmt, iters, group=group)
    got = _gpu_solve(W, fmt, iters, group=group, trace=True)
    assert got["codes"].size == rows * cols
    _compare_e2e(oracle_lib, ref, got, fmt, f"{fmt} g{group} {name}", iters)


E2E_MX_MINI = [
    ("MXFP8_E4M3", "q4096x4096_mxfp4", 256, 4096, 10),
    ("MXFP8_E5M2", "k1024x4096_mxint4", 129, 2048, 10),
    ("MXFP6_E2M3", "down4096x14336_nvfp4", 197, 9216, 10),
    ("MXFP6_E3M2", "q4096x4096_mxfp4", 256, 4096, 10),
    ("MXFP6_E2M3", "w256x512_int4", 256, 512, 16),
]


@pytest.mark.parametrize("fmt,name,rows,cols,iters", E2E_MX_MINI)
def test_end_to_end_mx_minifloat(oracle_lib, fmt, name, rows, cols, iters):
    W = synth.matrix(synth.WORKLOADS[name]["W"].scaled(rows, cols), 0)
    ref = oracle_lib.solve(W, fmt, iters)
    got = _gpu_solve(W, fmt, iters, trace=True)
    assert got["codes"].size == rows * cols * dq.CODE_BITS[fmt] // 8
    _compare_e2e(oracle_lib, ref, got, fmt, f"{fmt} {name}", iters)


# rows wider than 16384 columns: the row pass reads c and 1/c from global memory (the
# down projections of 18944 and 17408 columns, a 28672-column ragged one, and the maximum)
E2E_WIDE = [
    ("NVFP4", "down4096x14336_nvfp4", 96, 18944, 10),
    ("MXFP4", "down4096x14336_nvfp4", 64, 28672, 8),
    ("INT4", "down4096x14336_nvfp4", 37, 17408, 8),
    ("MXFP6_E2M3", "down4096x14336_nvfp4", 24, 65536, 6),
]


# fp32 weights: 24576 and 20480 columns (NVFP4: past the LDS limit by its tables) read c
# from L2; INT8 at 18432 keeps 144 KiB of column scales in LDS
E2E_WIDE_F32 = [
    ("MXFP4", "q4096x4096_mxfp4", 40, 24576, 8),
    ("NVFP4", "down4096x14336_nvfp4", 33, 20480, 8),
    ("INT8", "w256x512_int4", 33, 18432, 8),
]


@pytest.mark.parametrize("fmt,name,rows,cols,iters,dtype",
                         [c + ("bf16",) for c in E2E_WIDE] + [c + ("f32",) for c in E2E_WIDE_F32])
def test_end_to_end_wide(oracle_lib, fmt, name, rows, cols, iters, dtype):
    from dataclasses import replace

    W = synth.matrix(replace(synth.WORKLOADS[name]["W"].scaled(rows, cols), dtype=dtype), 0)
    print(f"[e2e] wide {fmt} {dtype} {rows}x{cols} T={iters}", flush=True)
    ref = oracle_lib.solve(W, fmt, iters)
    got = _gpu_solve(W, fmt, iters, trace=True)
    _compare_e2e(oracle_lib, ref, got, fmt, f"wide {fmt} {rows}x{cols}", iters)


# more rows than 16 per row-pass workgroup (one wave takes two rows, its neighbours one) and
# larger column-pass row ranges: 5120 rows -> blocks of 20, 9000 rows -> blocks of 36
E2E_TALL = [
    ("NVFP4", "down4096x14336_nvfp4", 5120, 1024, 8),
    ("MXFP4", "q4096x4096_mxfp4", 9000, 512, 8),
    ("INT4", "w256x512_int4", 4500, 512, 10),
]


@pytest.mark.parametrize("fmt,name,rows,cols,iters", E2E_TALL)
def test_end_to_end_tall(oracle_lib, fmt, name, rows, cols, iters):
    W = synth.matrix(synth.WORKLOADS[name]["W"].scaled(rows, cols), 0)
    print(f"[e2e] tall {fmt} {rows}x{cols} T={iters}", flush=True)
    ref = oracle_lib.solve(W, fmt, iters)
    got = _gpu_solve(W, fmt, iters, trace=True)
    _compare_e2e(oracle_lib, ref, got, fmt, f"tall {fmt} {rows}x{cols}", iters)


@pytest.mark.parametrize("name", ["w256x512_int4", "k1024x4096_mxint4", "q4096x4096_mxfp4",
                                  "down4096x14336_nvfp4"])
def test_end_to_end_full_size(oracle_lib, name):
    W, X, fmt, g, T = synth.workload(name)
    print(f"[e2e] {name} {W.shape} {fmt} T={T}", flush=True)
    got = _gpu_solve(W, fmt, T, trace=True)
    ref = oracle_lib.solve(W, fmt, T)
    _compare_e2e(oracle_lib, ref, got, fmt, name, T)
    print(f"[e2e] {name}: nmse {got['nmse'][0]:.6g} -> {got['nmse'][-1]:.6g}, rejected {got['rejected']}"
          f" (oracle {ref['rejected']})", flush=True)


def test_rejections_and_resolve_path(oracle_lib):
    # INT4 on the 256x512 workload keeps rejecting candidates once Qhat has settled
    W, _, fmt, g, _ = synth.workload("w256x512_int4")
    ref = oracle_lib.solve(W, fmt, 40)
    assert ref["rejected"] > 5
    got = _gpu_solve(W, fmt, 40, trace=True)
    t_div = _compare_e2e(oracle_lib, ref, got, fmt, "int4-40", 40)
    assert got["sweeps"] >= 41 + got["rejected"] - 1   # a re-solve sweep after each rejection
    assert t_div > 40, "INT4 accumulates in fp64: no boundary divergence expected"


@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_teacher_forced_step(oracle_lib, fmt):
    name = {"INT4": "w256x512_int4", "MXINT4": "k1024x4096_mxint4", "MXFP4": "q4096x4096_mxfp4",
            "NVFP4": "down4096x14336_nvfp4", "INT8": "w256x512_int4",
            "MXINT8": "k1024x4096_mxint4", "MXFP8_E4M3": "q4096x4096_mxfp4",
            "MXFP8_E5M2": "k1024x4096_mxint4", "MXFP6_E2M3": "q4096x4096_mxfp4",
            "MXFP6_E3M2": "down4096x14336_nvfp4"}[fmt]
    W = synth.matrix(synth.WORKLOADS[name]["W"].scaled(256, 512 if name == "w256x512_int4" else 4096), 0)
    rng = np.random.default_rng(5)
    states = [oracle_lib.solve(W, fmt, k) for k in (0, 3)]
    starts = [(s["r"], s["c"]) for s in states]
    starts.append((oracle_lib.project(fmt, np.exp2(rng.uniform(-1, 1, W.shape[0])).astype(np.float32)),
                   oracle_lib.project(fmt, np.exp2(rng.uniform(-1, 1, W.shape[1])).astype(np.float32))))
    for r0, c0 in starts:
        ref = oracle_lib.solve(W, fmt, 1, r_init=r0, c_init=c0)
        got = _gpu_solve(W, fmt, 1, r_init=to_dev(r0), c_init=to_dev(c0), trace=True)
        got["r_pre"], got["c_pre"] = got["r_trace"][0], got["c_trace"][0]
        ok = ~np.isnan(ref["r_pre"])
        assert np.array_equal(np.isnan(got["r_pre"]), ~ok)
        assert np.all(rel_err(got["r_pre"][ok], ref["r_pre"][ok]) <= 1e-5)
        flag = near_projection_boundary(oracle_lib, fmt, ref["r_pre"][ok])
        assert np.all((got["r"][ok] == ref["r"][ok]) | flag)
        okc = ~np.isnan(ref["c_pre"])
        assert np.all(rel_err(got["c_pre"][okc], ref["c_pre"][okc]) <= 1e-5)
        if np.array_equal(got["r"], ref["r"]):
            flagc = near_projection_boundary(oracle_lib, fmt, ref["c_pre"][okc])
            assert np.all((got["c"][okc] == ref["c"][okc]) | flagc)
        assert rel_err(got["nmse"][0], ref["nmse"][0]) <= 1e-6


@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_iteration_zero_is_bit_exact(oracle_lib, fmt):
    W = synth.matrix(synth.WORKLOADS["down4096x14336_nvfp4"]["W"].scaled(77, 2048), 1)
    rng = np.random.default_rng(6)
    r0 = oracle_lib.project(fmt, np.exp2(rng.uniform(-1, 1, 77)).astype(np.float32))
    c0 = oracle_lib.project(fmt, np.exp2(rng.uniform(-1, 1, 2048)).astype(np.float32))
    codes, scales, ts, _ = oracle_lib.quantize_weights(W, r0, c0, fmt)
    got = _gpu_solve(W, fmt, 0, r_init=to_dev(r0), c_init=to_dev(c0))
    assert np.array_equal(got["codes"], codes) and np.array_equal(got["scales"], scales)
    assert np.array_equal(got["r"], r0) and np.array_equal(got["c"], c0)
    if fmt == "NVFP4":
        assert got["tscale"] == np.float32(ts)


def test_deterministic(oracle_lib):
    W = synth.matrix(synth.WORKLOADS["down4096x14336_nvfp4"]["W"].scaled(512, 4096), 2)
    a = _gpu_solve(W, "NVFP4", 8)
    b = _gpu_solve(W, "NVFP4", 8)
    for k in ("r", "c", "codes", "scales", "nmse", "relchg"):
        assert np.array_equal(a[k], b[k]), k


def test_batch_equals_single():
    specs = [synth.WORKLOADS["down4096x14336_nvfp4"]["W"].scaled(200, 4096),
             synth.WORKLOADS["down4096x14336_nvfp4"]["W"].scaled(64, 14336),
             synth.WORKLOADS["k1024x4096_mxint4"]["W"].scaled(96, 4096)]
    Ws = [synth.matrix(s, 3) for s in specs]
    probs = [dq.make_problem(to_dev(W), "NVFP4", 6) for W in Ws]
    reps = dq.solve_many(probs, "NVFP4", 6)
    torch.cuda.synchronize()
    for W, p, rep in zip(Ws, probs, reps):
        one = _gpu_solve(W, "NVFP4", 6)
        assert np.array_equal(p.codes.cpu().numpy(), one["codes"])
        assert np.array_equal(p.r.cpu().numpy(), one["r"]) and np.array_equal(p.c.cpu().numpy(), one["c"])
        assert np.array_equal(p.nmse_hist.cpu().numpy(), one["nmse"])
        assert rep.rejected_steps == one["rejected"]


def test_early_stop_and_degenerate(oracle_lib):
    W, _, fmt, g, _ = synth.workload("w256x512_int4")
    got = _gpu_solve(W, fmt, 40, tol=1e9)
    assert got["iters_run"] == 1
    Z = np.zeros((64, 256), np.float32)
    got = _gpu_solve(Z, "NVFP4", 3)
    assert np.all(got["nmse"] == 0) and np.all(got["codes"] == 0) and got["tscale"] == 0.0
    assert np.all(got["r"] == 1) and np.all(got["c"] == 1)
    assert got["flags"] & 2 and got["flags"] & 4
    e = dq.solve(torch.empty(0, 256, dtype=torch.bfloat16, device=DEV), "NVFP4", 3)
    torch.cuda.synchronize()
    assert e["iters_run"] == 3
    Wn = synth.matrix(synth.WORKLOADS["down4096x14336_nvfp4"]["W"].scaled(8, 256), 0)
    Wf = synth.bf16_bits_to_f32(Wn).copy()
    Wf[3, 5] = np.nan
    got = _gpu_solve(Wf, "NVFP4", 1)
    assert got["flags"] & 1


@pytest.mark.parametrize("steps", [1, 2])
@pytest.mark.parametrize("name,rows,cols,iters", [("w256x512_int4", 256, 512, 16),
                                                  ("down4096x14336_nvfp4", 197, 9216, 12),
                                                  ("k1024x4096_mxint4", 129, 2048, 8)])
def test_scale_step_ablation(oracle_lib, steps, name, rows, cols, iters):
    """Row scales only / column scales only, against the oracle."""
    w = synth.WORKLOADS[name]
    W = synth.matrix(w["W"].scaled(rows, cols), 0)
    ref = oracle_lib.solve(W, w["fmt"], iters, steps=steps)
    got = _gpu_solve(W, w["fmt"], iters, trace=True, steps=steps)
    _compare_e2e(oracle_lib, ref, got, w["fmt"], f"{name} steps={steps}", iters)
    frozen = {1: ["c"], 2: ["r"]}[steps]
    for v in frozen:
        assert np.all(got[v] == 1.0), v


def test_batch_across_rounds_of_sweeps():
    """A batch whose members finish in different rounds of sweeps (INT4 rejections add
    re-solve sweeps for some matrices only) plus an empty problem: every member equals its
    own solve (codes, scales, r, c, histories, report), whichever code buffer its kept Qhat
    ended in."""
    base = synth.WORKLOADS["w256x512_int4"]["W"]
    Ws = [synth.workload("w256x512_int4")[0],
          synth.matrix(base.scaled(96, 512), 7),
          synth.matrix(synth.WORKLOADS["k1024x4096_mxint4"]["W"].scaled(130, 1024), 8)]
    iters = 40
    probs = [dq.make_problem(to_dev(W), "INT4", iters) for W in Ws]
    probs.insert(1, dq.make_problem(torch.empty(0, 512, dtype=torch.float32, device=DEV), "INT4", iters))
    reps = dq.solve_many(probs, "INT4", iters)
    torch.cuda.synchronize()
    assert reps[1].iters_run == iters and reps[1].rejected_steps == 0
    solo = [_gpu_solve(W, "INT4", iters) for W in Ws]
    print("[batch] rejected per member:", [one["rejected"] for one in solo],
          "sweeps:", [one["sweeps"] for one in solo], flush=True)
    assert max(one["rejected"] for one in solo) > 5
    for p, rep, one in zip([probs[0]] + probs[2:], [reps[0]] + reps[2:], solo):
        assert np.array_equal(p.codes.cpu().numpy(), one["codes"])
        assert np.array_equal(p.block_scales.cpu().numpy().view(np.uint16), one["scales"].view(np.uint16))
        assert np.array_equal(p.r.cpu().numpy(), one["r"]) and np.array_equal(p.c.cpu().numpy(), one["c"])
        assert np.array_equal(p.nmse_hist.cpu().numpy(), one["nmse"])
        assert rep.rejected_steps == one["rejected"] and rep.iters_run == one["iters_run"]
        assert rep.sweeps == one["sweeps"]
