"""dq_solve against the oracle.

  * end to end on every workload (full sizes and reduced ones with ragged shapes):
    nmse/relchg histories within 1e-5 relative, final scales within 1e-5 relative,
    at most 1e-4 of the codes different, same tensor scale;
  * teacher-forced single iterations from realistic states: unprojected closed forms
    within 1e-5 relative, projected scales equal except where the oracle's value sits
    within 1e-5 of a projection boundary, Qhat^0 codes bit-exact;
  * determinism (bitwise repeatable), batching (a batch equals its members solved
    alone), rejected steps, early stop, empty and degenerate inputs.
"""

import json
import os
import warnings

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


# Every oracle-flagged boundary flip seen by the end-to-end comparisons of this session:
# (case, iteration, vector, elements).  Written to $DQ_PARITY_RECORD (JSON) when set.
FLIP_RECORD = []
# Formats whose GPU sums use exact products in fp64: no projection flip is expected.
FP64_SUMS = ("INT4", "INT8")
MAX_RESYNCS = 6


def _record_flip(what, t, key, n):
    FLIP_RECORD.append({"case": what, "iteration": int(t), "vector": key, "elements": int(n)})
    warnings.warn(f"{what}: oracle-flagged projection flip of {n} {key} value(s) at iteration {t}; "
                  f"oracle resumed from the GPU's state")
    path = os.environ.get("DQ_PARITY_RECORD")
    if path:
        with open(path, "w") as f:
            json.dump(FLIP_RECORD, f, indent=1)


def _replay_scales(oracle, fmt, trace, init, t):
    """The scale vector after iteration t, rebuilt from the unprojected closed forms: each
    iteration projects its value, a NaN (D = 0, or a frozen step) keeps the previous one."""
    v = np.array(init, dtype=np.float32, copy=True)
    for s in range(t):
        x = trace[s]
        ok = ~np.isnan(x)
        if ok.any():
            v[ok] = oracle.project(fmt, x[ok])
    return v


def _compare_e2e(oracle, W, fmt, T, got, what, group=None, steps=3, r_init=None, c_init=None):
    """Strict end-to-end parity of a GPU solve (run with traces) against the oracle.

    Up to the first projection flip, every iteration's unprojected r and c must agree
    within 1e-5 relative and nmse / relchg within 1e-5.  A flip -- the two projected values
    of one scale differ -- is accepted only where the oracle's own unprojected value lies
    within 1e-6 of a projection boundary, where both neighbours are valid.  The oracle is
    then resumed from the GPU's exact state after that iteration (scales replayed from the
    GPU's traces through the oracle's projection, kept Qhat from the oracle's quantiser at
    the GPU's scales) and the comparison continues at the same tolerances.  At the end the
    GPU's r and c equal the replayed ones exactly, its codes, block scales and tensor scale
    are bit-exact with the oracle's quantiser at the scales of its last kept step, and the
    rejected-step count matches."""
    assert got["iters_run"] == T, what
    rows, cols = W.shape
    r_tr, c_tr = got["r_trace"], got["c_trace"]
    r0 = np.ones(rows, np.float32) if r_init is None else np.asarray(r_init, np.float32)
    c0 = np.ones(cols, np.float32) if c_init is None else np.asarray(c_init, np.float32)
    nm, rc = np.asarray(got["nmse"]), np.asarray(got["relchg"])
    assert np.all(np.diff(nm) <= 0.0), (what, nm)
    seg_t, seg_state, rejected, resyncs = 0, dict(r_init=r_init, c_init=c_init), 0, 0
    while True:
        ref = oracle.solve(W, fmt, T - seg_t, group, steps=steps, **seg_state)
        assert abs(nm[seg_t] - ref["nmse"][0]) <= 1e-5 * ref["nmse"][0] + 1e-30, (what, seg_t)
        flip = None
        for k in range(1, T - seg_t + 1):
            t = seg_t + k
            for key, tr in (("r", r_tr), ("c", c_tr)):
                a, b = ref[key + "_trace"][k - 1], tr[t - 1]
                assert np.array_equal(np.isnan(a), np.isnan(b)), (what, key, t)
                ok = ~np.isnan(a)
                err = rel_err(b[ok], a[ok])
                assert np.all(err <= 1e-5), (what, key, t, err.max())
                diff = oracle.project(fmt, a[ok]) != oracle.project(fmt, b[ok])
                if diff.any():
                    flagged = near_projection_boundary(oracle, fmt, a[ok][diff], 1e-6)
                    assert np.all(flagged), (what, key, t, a[ok][diff][~flagged], b[ok][diff][~flagged])
                    flip = (t, key, int(diff.sum()))
                    break
            if flip:
                break
            assert abs(nm[t] - ref["nmse"][k]) <= 1e-5 * ref["nmse"][k] + 1e-30, (what, t, nm[t], ref["nmse"][k])
            assert abs(rc[t] - ref["relchg"][k]) <= 1e-5 * ref["relchg"][k] + 1e-9, (what, t, rc[t], ref["relchg"][k])
        if flip is None:
            rejected += ref["rejected"]
            break
        t, key, n = flip
        assert fmt not in FP64_SUMS, f"{what}: projection flip with exact fp64 sums"
        _record_flip(what, t, key, n)
        resyncs += 1
        assert resyncs <= MAX_RESYNCS, f"{what}: more than {MAX_RESYNCS} flips"
        k = t - seg_t
        # oracle state before iteration t (equal on both sides up to there)
        before = oracle.solve(W, fmt, k - 1, group, steps=steps, **seg_state)
        rejected += before["rejected"]
        r_t = _replay_scales(oracle, fmt, r_tr, r0, t)
        c_t = _replay_scales(oracle, fmt, c_tr, c0, t)
        cand = oracle.quantize_weights(W, r_t, c_t, fmt, group)
        kept = (before["codes"], before["scales"], before["tscale"])
        prev_q = oracle.dequantize(*kept, fmt, rows, cols, group)
        same = np.array_equal(cand[3], prev_q)
        if rc[t] > 0.0:
            q_t = cand[:3]
        else:
            q_t = kept
            rejected += 0 if same else 1   # the GPU rejected a candidate that moved Qhat
        seg_t, seg_state = t, dict(r_init=r_t, c_init=c_t, q_init=q_t)
    # final state
    r_fin = _replay_scales(oracle, fmt, r_tr, r0, T)
    c_fin = _replay_scales(oracle, fmt, c_tr, c0, T)
    assert np.array_equal(got["r"], r_fin) and np.array_equal(got["c"], c_fin), what
    moved = [t for t in range(1, T + 1) if rc[t] > 0.0]
    s_last = moved[-1] if moved else 0
    r_s = _replay_scales(oracle, fmt, r_tr, r0, s_last)
    c_s = _replay_scales(oracle, fmt, c_tr, c0, s_last)
    codes, scales, ts, _ = oracle.quantize_weights(W, r_s, c_s, fmt, group)
    assert np.array_equal(got["codes"], codes), (what, "codes", int((elements(got["codes"], fmt) != elements(codes, fmt)).sum()))
    assert np.array_equal(got["scales"], scales), (what, "block scales")
    if fmt == "NVFP4":
        assert got["tscale"] == np.float32(ts), what
    assert got["rejected"] == rejected, (what, got["rejected"], rejected)
    return resyncs


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
    got = _gpu_solve(W, w["fmt"], iters, trace=True)
    _compare_e2e(oracle_lib, W, w["fmt"], iters, got, name)


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
    got = _gpu_solve(W, fmt, iters, group=group, trace=True)
    assert got["codes"].size == rows * cols
    _compare_e2e(oracle_lib, W, fmt, iters, got, f"{fmt} g{group} {name}", group=group)


# INT4 with 64-element groups, the listing page's setting (Tables 1, 6, 10-12): the
# 256x512 fp32 workload's shape and a bf16 q_proj-shaped 4096x4096 weight
E2E_INT4_G64 = [
    ("w256x512_int4", 256, 512, 16),
    ("q4096x4096_mxfp4", 4096, 4096, 16),
    ("down4096x14336_nvfp4", 197, 9216, 12),
]


@pytest.mark.parametrize("name,rows,cols,iters", E2E_INT4_G64)
def test_end_to_end_int4_group64(oracle_lib, name, rows, cols, iters):
    W = synth.matrix(synth.WORKLOADS[name]["W"].scaled(rows, cols), 0)
    print(f"[e2e] INT4 g64 {name} {rows}x{cols} T={iters}", flush=True)
    got = _gpu_solve(W, "INT4", iters, group=64, trace=True)
    assert got["scales"].size == rows * cols // 64
    assert _compare_e2e(oracle_lib, W, "INT4", iters, got, f"INT4 g64 {name}", group=64) == 0
    assert got["nmse"][-1] < got["nmse"][0]


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
    got = _gpu_solve(W, fmt, iters, trace=True)
    assert got["codes"].size == rows * cols * dq.CODE_BITS[fmt] // 8
    _compare_e2e(oracle_lib, W, fmt, iters, got, f"{fmt} {name}")


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
    got = _gpu_solve(W, fmt, iters, trace=True)
    _compare_e2e(oracle_lib, W, fmt, iters, got, f"wide {fmt} {rows}x{cols}")


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
    got = _gpu_solve(W, fmt, iters, trace=True)
    _compare_e2e(oracle_lib, W, fmt, iters, got, f"tall {fmt} {rows}x{cols}")


@pytest.mark.parametrize("name", ["w256x512_int4", "k1024x4096_mxint4", "q4096x4096_mxfp4",
                                  "down4096x14336_nvfp4"])
def test_end_to_end_full_size(oracle_lib, name):
    W, X, fmt, g, T = synth.workload(name)
    print(f"[e2e] {name} {W.shape} {fmt} T={T}", flush=True)
    got = _gpu_solve(W, fmt, T, trace=True)
    n = _compare_e2e(oracle_lib, W, fmt, T, got, name)
    print(f"[e2e] {name}: nmse {got['nmse'][0]:.6g} -> {got['nmse'][-1]:.6g}, rejected {got['rejected']},"
          f" oracle resumed {n} times", flush=True)


def test_rejections_and_resolve_path(oracle_lib):
    # INT4 on the 256x512 workload keeps rejecting candidates once Qhat has settled
    W, _, fmt, g, _ = synth.workload("w256x512_int4")
    ref = oracle_lib.solve(W, fmt, 40)
    assert ref["rejected"] > 5
    got = _gpu_solve(W, fmt, 40, trace=True)
    assert _compare_e2e(oracle_lib, W, fmt, 40, got, "int4-40") == 0
    # every sweep computes the r/c steps of both outcomes of its safeguard: T + 1 sweeps
    assert got["sweeps"] == 41 and got["rejected"] > 5


@pytest.mark.parametrize("fmt", ALL_FORMATS + ["INT4_G64"])
def test_teacher_forced_step(oracle_lib, fmt):
    group = None
    if fmt == "INT4_G64":
        fmt, group = "INT4", 64
    name = {"INT4": "w256x512_int4", "MXINT4": "k1024x4096_mxint4", "MXFP4": "q4096x4096_mxfp4",
            "NVFP4": "down4096x14336_nvfp4", "INT8": "w256x512_int4",
            "MXINT8": "k1024x4096_mxint4", "MXFP8_E4M3": "q4096x4096_mxfp4",
            "MXFP8_E5M2": "k1024x4096_mxint4", "MXFP6_E2M3": "q4096x4096_mxfp4",
            "MXFP6_E3M2": "down4096x14336_nvfp4"}[fmt]
    W = synth.matrix(synth.WORKLOADS[name]["W"].scaled(256, 512 if name == "w256x512_int4" else 4096), 0)
    rng = np.random.default_rng(5)
    states = [oracle_lib.solve(W, fmt, k, group) for k in (0, 3)]
    starts = [(s["r"], s["c"]) for s in states]
    starts.append((oracle_lib.project(fmt, np.exp2(rng.uniform(-1, 1, W.shape[0])).astype(np.float32)),
                   oracle_lib.project(fmt, np.exp2(rng.uniform(-1, 1, W.shape[1])).astype(np.float32))))
    for r0, c0 in starts:
        ref = oracle_lib.solve(W, fmt, 1, group, r_init=r0, c_init=c0)
        got = _gpu_solve(W, fmt, 1, group=group, r_init=to_dev(r0), c_init=to_dev(c0), trace=True)
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


@pytest.mark.parametrize("fmt,group,name,rows,cols", [("NVFP4", None, "down4096x14336_nvfp4", 96, 2048),
                                                    ("MXFP4", None, "q4096x4096_mxfp4", 130, 1024),
                                                    ("INT4", 64, "w256x512_int4", 256, 512)])
def test_end_to_end_from_given_scales(oracle_lib, fmt, group, name, rows, cols):
    """A whole solve started from caller-given admissible scales (r_init, c_init), strict
    parity with the oracle started from the same scales."""
    W = synth.matrix(synth.WORKLOADS[name]["W"].scaled(rows, cols), 2)
    rng = np.random.default_rng(rows + cols)
    r0 = oracle_lib.project(fmt, np.exp2(rng.uniform(-1, 1, rows)).astype(np.float32))
    c0 = oracle_lib.project(fmt, np.exp2(rng.uniform(-1, 1, cols)).astype(np.float32))
    T = 8
    got = _gpu_solve(W, fmt, T, group=group, r_init=to_dev(r0), c_init=to_dev(c0), trace=True)
    _compare_e2e(oracle_lib, W, fmt, T, got, f"{name} {fmt} from given scales", group=group,
                 r_init=r0, c_init=c0)


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
@pytest.mark.parametrize("name,rows,cols,iters,group", [("w256x512_int4", 256, 512, 16, None),
                                                        ("w256x512_int4", 256, 512, 16, 64),
                                                        ("down4096x14336_nvfp4", 197, 9216, 12, None),
                                                        ("k1024x4096_mxint4", 129, 2048, 8, None),
                                                        ("q4096x4096_mxfp4", 130, 2048, 8, None)])
def test_scale_step_ablation(oracle_lib, steps, name, rows, cols, iters, group):
    """Row scales only / column scales only, against the oracle."""
    w = synth.WORKLOADS[name]
    W = synth.matrix(w["W"].scaled(rows, cols), 0)
    got = _gpu_solve(W, w["fmt"], iters, trace=True, steps=steps, group=group)
    _compare_e2e(oracle_lib, W, w["fmt"], iters, got, f"{name} g{group} steps={steps}", group=group,
                 steps=steps)
    frozen = {1: ["c"], 2: ["r"]}[steps]
    for v in frozen:
        assert np.all(got[v] == 1.0), v


@pytest.mark.parametrize("tol", [0.0, 2e-3])
def test_batch_members_finishing_at_different_sweeps(tol):
    """A batch of INT4 members with different rejected steps plus an empty problem; with a
    relchg tolerance the members also stop after different numbers of sweeps (a rejected step
    reports relchg 0 and ends the solve).  Every member equals its own solve (codes, scales, r,
    c, histories, report), whichever code buffer its kept Qhat ended in."""
    base = synth.WORKLOADS["w256x512_int4"]["W"]
    Ws = [synth.workload("w256x512_int4")[0],
          synth.matrix(base.scaled(96, 512), 7),
          synth.matrix(synth.WORKLOADS["k1024x4096_mxint4"]["W"].scaled(130, 1024), 8)]
    iters = 40
    probs = [dq.make_problem(to_dev(W), "INT4", iters) for W in Ws]
    probs.insert(1, dq.make_problem(torch.empty(0, 512, dtype=torch.float32, device=DEV), "INT4", iters))
    reps = dq.solve_many(probs, "INT4", iters, tol=tol)
    torch.cuda.synchronize()
    assert reps[1].iters_run == iters and reps[1].rejected_steps == 0
    solo = [_gpu_solve(W, "INT4", iters, tol=tol) for W in Ws]
    print("[batch] rejected per member:", [one["rejected"] for one in solo],
          "sweeps:", [one["sweeps"] for one in solo], flush=True)
    if tol == 0.0:
        assert max(one["rejected"] for one in solo) > 5
        assert all(one["sweeps"] == iters + 1 for one in solo)
    else:
        assert len({one["sweeps"] for one in solo}) > 1
    for p, rep, one in zip([probs[0]] + probs[2:], [reps[0]] + reps[2:], solo):
        assert np.array_equal(p.codes.cpu().numpy(), one["codes"])
        assert np.array_equal(p.block_scales.cpu().numpy().view(np.uint16), one["scales"].view(np.uint16))
        assert np.array_equal(p.r.cpu().numpy(), one["r"]) and np.array_equal(p.c.cpu().numpy(), one["c"])
        assert rep.rejected_steps == one["rejected"] and rep.iters_run == one["iters_run"]
        k = rep.iters_run + 1   # history entries past an early stop are not written
        assert np.array_equal(p.nmse_hist.cpu().numpy()[:k], one["nmse"][:k])
        assert rep.sweeps == one["sweeps"]


def test_stream_ordered_on_a_side_stream():
    """dq_solve only enqueues: run it on a side stream, join that stream with an event, and the
    results (codes, scales, r, c, histories, device report) equal a solve on the default
    stream bit for bit.  Work queued on the side stream after the solve sees its outputs."""
    W = synth.matrix(synth.WORKLOADS["down4096x14336_nvfp4"]["W"].scaled(300, 4096), 4)
    Wd = to_dev(W)
    ref = dq.solve(Wd, "NVFP4", 8)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    p = dq.make_problem(Wd, "NVFP4", 8)
    done = torch.cuda.Event()
    with torch.cuda.stream(side):
        assert dq.solve_many([p], "NVFP4", 8, stream=side, read_reports=False) is None
        c_copy = p.c.clone()          # stream-ordered after the solve
        done.record(side)
    torch.cuda.current_stream().wait_event(done)
    rep = dq.read_report(p)
    assert torch.equal(p.codes, ref["codes"]) and torch.equal(p.block_scales, ref["scales"])
    assert torch.equal(p.r, ref["r"]) and torch.equal(p.c, ref["c"]) and torch.equal(c_copy, ref["c"])
    assert torch.equal(p.nmse_hist, ref["nmse"]) and torch.equal(p.relchg_hist, ref["relchg"])
    assert rep.iters_run == ref["iters_run"] == 8 and rep.rejected_steps == ref["rejected"]
    assert rep.sweeps == ref["sweeps"] and rep.flags == ref["flags"]
    assert (rep.flags & 32) == 0


def test_timed_solves_match_the_plain_solve():
    """The diagnostic timed solves (synchronous, and enqueue + read after the caller's wait)
    attach events and change nothing else: outputs and reports equal dq_solve's bit for bit,
    both report one positive duration triple per sweep that did work, and a second timed
    enqueue of a smaller problem replaces the first one's durations."""
    iters = 40
    W = synth.workload("w256x512_int4")[0]
    ref = _gpu_solve(W, "INT4", iters)
    assert ref["rejected"] > 0          # sweeps whose column pass takes the kept Qhat
    for mode in ("sync", "enqueue"):
        p = dq.make_problem(to_dev(W), "INT4", iters)
        if mode == "sync":
            per = []
            rep = dq.solve_many([p], "INT4", iters, pass_ms=per)[0]
        else:
            assert dq.solve_many([p], "INT4", iters, timed_sweeps=2 * iters, read_reports=False) is None
            torch.cuda.synchronize()
            per = dq.timed_passes([p], iters)
            rep = dq.read_report(p)
        assert np.array_equal(p.codes.cpu().numpy(), ref["codes"]), mode
        assert np.array_equal(p.block_scales.cpu().numpy().view(np.uint16), ref["scales"].view(np.uint16))
        assert np.array_equal(p.r.cpu().numpy(), ref["r"]) and np.array_equal(p.c.cpu().numpy(), ref["c"])
        assert np.array_equal(p.nmse_hist.cpu().numpy(), ref["nmse"])
        assert rep.sweeps == ref["sweeps"] and rep.rejected_steps == ref["rejected"]
        assert len(per) == ref["sweeps"], mode
        assert all(t > 0.0 for trip in per for t in trip), mode
    small = dq.make_problem(to_dev(synth.matrix(synth.WORKLOADS["w256x512_int4"]["W"].scaled(64, 512), 1)),
                            "MXFP4", 3)
    dq.solve_many([small], "MXFP4", 3, timed_sweeps=100, read_reports=False)
    torch.cuda.synchronize()
    per = dq.dq_solve_timed_read(2 * iters + 2)
    assert len(per) == 3 + 1          # the smaller solve's T + 1 queued sweeps, not the earlier 41
    assert len(dq.timed_passes([small], 3)) == dq.read_report(small).sweeps
    # timing only the first sweeps leaves the outputs alone
    again = dq.make_problem(small.W, "MXFP4", 3)
    dq.solve_many([again], "MXFP4", 3, timed_sweeps=2, read_reports=False)
    torch.cuda.synchronize()
    assert len(dq.dq_solve_timed_read(10)) == 2
    assert torch.equal(again.codes, small.codes) and torch.equal(again.r, small.r)
    assert torch.equal(again.c, small.c) and torch.equal(again.nmse_hist, small.nmse_hist)


def test_device_reports_of_a_batch_with_an_empty_problem():
    probs = [dq.make_problem(to_dev(synth.matrix(synth.WORKLOADS["w256x512_int4"]["W"].scaled(64, 512), 1)),
                             "MXFP4", 5),
             dq.make_problem(torch.empty(0, 512, dtype=torch.float32, device=DEV), "MXFP4", 5)]
    for p in probs:
        p.report.fill_(-1)
    reps = dq.solve_many(probs, "MXFP4", 5)
    assert reps[0].iters_run == 5 and reps[0].sweeps == 6 and (reps[0].flags & 32) == 0
    assert (reps[1].iters_run, reps[1].rejected_steps, reps[1].flags, reps[1].sweeps) == (5, 0, 0, 0)
