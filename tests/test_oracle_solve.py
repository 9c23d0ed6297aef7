"""Pins for the oracle's BCD solve and activation path.

What fixes them, independently of the oracle's code:
  * brute force: each scale step must attain the minimum of its row/column objective
    over the whole admissible set, and the unprojected value must match a golden-section
    line search (the closed form is the exact minimiser of a 1-D quadratic);
  * invariants: normalised MSE never increases (Theorem 1(i) on the DualQuant listing
    page, Fig. 2b / Fig. 3b captions); the dual-scale result is no worse than the
    single-scale start (Fig. 1); a planted exact factorisation is a fixed point; results
    do not depend on the thread count;
  * recomputation from outputs: nmse and relchg histories recomputed from the codes
    the solve returns after t and t-1 iterations, with numpy;
  * closed forms for the activation SQNR on planted inputs.
"""

import numpy as np
import pytest
import torch

import synth

FORMATS = ["INT4", "MXINT4", "MXFP4", "NVFP4"]
GROUPS = {"INT4": 128, "MXINT4": 32, "MXFP4": 32, "NVFP4": 16}


def _admissible(fmt):
    """Every admissible dual scale: positive E4M3 values (NVFP4), else positive normal
    finite bf16 values (INT4 and the MX formats)."""
    if fmt == "NVFP4":
        return torch.arange(1, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    bits = np.arange(0x0080, 0x7F80, dtype=np.uint32) << 16   # positive normal finite bf16
    return bits.view(np.float32).astype(np.float64)


def _golden(f, lo, hi, iters=200):
    g = (np.sqrt(5) - 1) / 2
    a, b = lo, hi
    c, d = b - g * (b - a), a + g * (b - a)
    for _ in range(iters):
        if f(c) < f(d):
            b = d
        else:
            a = c
        c, d = b - g * (b - a), a + g * (b - a)
    return (a + b) / 2


def _w(rows, cols, seed):
    spec = synth.MatrixSpec(rows, cols, "student_t", 0.02, nu=4, outliers=max(1, cols // 40),
                            outlier_scale=15.0, stream=77)
    return synth.matrix(spec, seed)


@pytest.mark.parametrize("fmt,g", [("INT4", 128), ("INT4", 64), ("MXINT4", 32), ("MXFP4", 32),
                                   ("NVFP4", 16)])
def test_scale_steps_are_constrained_minimisers(oracle_lib, fmt, g):
    rows, cols = 6, g * 4
    W = _w(rows, cols, 1)
    Wf = synth.bf16_bits_to_f32(W).astype(np.float64)
    rng = np.random.default_rng(2)
    r0 = oracle_lib.project(fmt, np.exp2(rng.uniform(-0.7, 0.7, rows)).astype(np.float32))
    c0 = oracle_lib.project(fmt, np.exp2(rng.uniform(-0.7, 0.7, cols)).astype(np.float32))
    _, _, _, Q0 = oracle_lib.quantize_weights(W, r0, c0, fmt, g)
    Q0 = Q0.astype(np.float64)
    res = oracle_lib.solve(W, fmt, 1, g, r_init=r0, c_init=c0)
    adm = _admissible(fmt)
    for i in range(rows):
        u = Q0[i] * c0
        f = lambda s: float(np.sum((Wf[i] - s * u) ** 2))
        x = _golden(f, 0.0, 8.0 * max(1.0, np.abs(Wf[i]).max() / max(np.abs(u).max(), 1e-30)))
        assert abs(res["r_pre"][i] - x) <= 1e-6 * x
        vals = ((Wf[i][None, :] - adm[:, None] * u[None, :]) ** 2).sum(axis=1)
        assert f(float(res["r"][i])) <= vals.min() * (1 + 1e-12) + 1e-300
    r1 = res["r"].astype(np.float64)
    for j in range(cols):
        u = r1 * Q0[:, j]
        if not np.any(u):
            assert np.isnan(res["c_pre"][j]) and res["c"][j] == c0[j]
            continue
        f = lambda s: float(np.sum((Wf[:, j] - s * u) ** 2))
        x = _golden(f, 0.0, 8.0 * max(1.0, np.abs(Wf[:, j]).max() / np.abs(u).max()))
        assert abs(res["c_pre"][j] - x) <= 1e-6 * x
        vals = ((Wf[:, j][None, :] - adm[:, None] * u[None, :]) ** 2).sum(axis=1)
        assert f(float(res["c"][j])) <= vals.min() * (1 + 1e-12) + 1e-300


def _workload_small(name, rows, cols):
    w = synth.WORKLOADS[name]
    return synth.matrix(w["W"].scaled(rows, cols), 0), w["fmt"]


SMALL = [("w256x512_int4", 256, 512), ("q4096x4096_mxfp4", 256, 1024),
         ("down4096x14336_nvfp4", 256, 1792), ("k1024x4096_mxint4", 256, 1024)]


@pytest.mark.parametrize("name,rows,cols,g", [s + (None,) for s in SMALL] + [("w256x512_int4", 256, 512, 64)])
def test_monotone_and_no_worse_than_single_scale(oracle_lib, name, rows, cols, g):
    W, fmt = _workload_small(name, rows, cols)
    res = oracle_lib.solve(W, fmt, 24, g)
    nm = res["nmse"]
    assert np.all(np.diff(nm) <= 0.0)
    assert nm[-1] <= nm[0]
    # single-scale start: nmse[0] is FQ(W) with r = c = 1
    codes, scales, ts, Q = oracle_lib.quantize_weights(W, None, None, fmt, g)
    Wf = (synth.bf16_bits_to_f32(W) if W.dtype == np.uint16 else W).astype(np.float64)
    assert np.isclose(nm[0], np.sum((Wf - Q) ** 2) / np.sum(Wf ** 2), rtol=1e-12)
    # the dual-scale fit improves on the single-scale start (strictly, on these weights)
    assert nm[-1] < nm[0]


@pytest.mark.parametrize("name,rows,cols", SMALL[:3])
def test_scale_step_ablation(oracle_lib, name, rows, cols):
    """Row scales only / column scales only (the news summary's ablation).  With no scale
    step the solve is the single-scale quantisation, repeated: every candidate equals the
    start.  With one step the other scale vector never moves, the history is still
    monotone and no worse than the start, and the running step is still the exact
    constrained minimiser of its objective (the frozen one is not)."""
    W, fmt = _workload_small(name, rows, cols)
    base = oracle_lib.solve(W, fmt, 0)
    none = oracle_lib.solve(W, fmt, 6, steps=0)
    assert np.all(none["nmse"] == none["nmse"][0]) and none["nmse"][0] == base["nmse"][0]
    assert np.array_equal(none["codes"], base["codes"]) and none["rejected"] == 0
    assert np.all(none["r"] == 1) and np.all(none["c"] == 1)
    assert np.all(np.isnan(none["r_trace"])) and np.all(np.isnan(none["c_trace"]))
    for steps, moving, frozen in ((1, "r", "c"), (2, "c", "r")):
        res = oracle_lib.solve(W, fmt, 12, steps=steps)
        assert np.all(res[frozen] == 1), (steps, frozen)
        assert np.all(np.isnan(res[frozen + "_trace"]))
        assert not np.all(np.isnan(res[moving + "_trace"]))
        assert np.all(np.diff(res["nmse"]) <= 0.0)
        assert res["nmse"][-1] <= res["nmse"][0]
    # the first row-only iteration equals the first dual iteration's r-step
    one_r = oracle_lib.solve(W, fmt, 1, steps=1)
    one = oracle_lib.solve(W, fmt, 1)
    assert np.array_equal(one_r["r"], one["r"]) and np.array_equal(
        one_r["r_trace"], one["r_trace"], equal_nan=True)


def test_history_recomputed_from_outputs(oracle_lib):
    W, fmt = _workload_small("down4096x14336_nvfp4", 64, 512)
    Wf = synth.bf16_bits_to_f32(W).astype(np.float64)
    T = 5
    full = oracle_lib.solve(W, fmt, T)
    prev = None
    for t in range(T + 1):
        res = oracle_lib.solve(W, fmt, t)
        Q = oracle_lib.dequantize(res["codes"], res["scales"], res["tscale"], fmt, *W.shape).astype(np.float64)
        F = np.sum((Wf - res["r"][:, None].astype(np.float64) * Q * res["c"][None, :].astype(np.float64)) ** 2)
        assert np.isclose(full["nmse"][t], F / np.sum(Wf ** 2), rtol=1e-10)
        if prev is not None:
            den = np.linalg.norm(prev)
            want = np.linalg.norm(Q - prev) / den if den > 0 else 0.0
            assert np.isclose(full["relchg"][t], want, rtol=1e-9, atol=1e-15)
        prev = Q


def _planted(fmt, rows, cols, seed, g=None):
    """W = diag(r0) Q0 diag(c0), Q0 exactly on the format's grid with every block's largest
    element at the top of its binade, so FQ(Q0) = Q0."""
    g = g or GROUPS[fmt]
    rng = np.random.default_rng(seed)
    nb = cols // g
    if fmt == "MXFP4":
        grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
        q = grid[rng.integers(0, 8, (rows, nb, g))] * rng.choice([-1, 1], (rows, nb, g))
        q[:, :, 0] = 6.0 * rng.choice([-1, 1], (rows, nb))
        e = rng.integers(-8, -3, (rows, nb, 1))
        Q0 = np.ldexp(q, e)
    elif fmt == "MXINT4":
        q = rng.integers(-7, 8, (rows, nb, g)).astype(np.float64)
        q[:, :, 0] = 7.0
        e = rng.integers(-8, -3, (rows, nb, 1))
        Q0 = np.ldexp(q, e - 2)
    else:  # INT4 with bf16 block scales
        q = rng.integers(-7, 8, (rows, nb, g)).astype(np.float64)
        q[:, :, 0] = -7.0
        s = torch.from_numpy(np.exp2(rng.uniform(-9, -4, (rows, nb, 1))).astype(np.float32)).to(
            torch.bfloat16).float().double().numpy()
        Q0 = q * s
    Q0 = Q0.reshape(rows, cols)
    if fmt == "INT4":
        r0 = _bf16_values(np.exp2(rng.uniform(-1, 1, rows)))
        c0 = np.ones(cols)
    else:
        r0 = np.ldexp(1.0, rng.integers(-2, 3, rows))
        c0 = np.ldexp(1.0, rng.integers(-2, 3, cols))
    W = (r0[:, None] * Q0 * c0[None, :]).astype(np.float32)
    return W, r0.astype(np.float32), c0.astype(np.float32)


def _bf16_values(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().double().numpy()


@pytest.mark.parametrize("fmt,g", [("MXFP4", 32), ("MXINT4", 32), ("INT4", 128), ("INT4", 64)])
def test_planted_factorisation_is_fixed_point(oracle_lib, fmt, g):
    W, r0, c0 = _planted(fmt, 8, g * 4, 3, g)
    if fmt != "INT4":   # MX products have few significant bits: exact in bf16
        assert np.array_equal(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(W)), W)
        W = synth.f32_to_bf16_bits(W)
    res = oracle_lib.solve(W, fmt, 4, g, r_init=r0, c_init=c0)
    assert np.all(res["nmse"] == 0.0)
    assert np.array_equal(res["r"], r0) and np.array_equal(res["c"], c0)
    assert res["rejected"] == 0


def test_thread_count_invariance(oracle_lib):
    W, fmt = _workload_small("down4096x14336_nvfp4", 128, 512)
    oracle_lib.set_threads(1)
    a = oracle_lib.solve(W, fmt, 6)
    oracle_lib.set_threads(7)
    b = oracle_lib.solve(W, fmt, 6)
    oracle_lib.set_threads(16)
    for k in ("r", "c", "codes", "scales", "nmse", "relchg"):
        assert np.array_equal(a[k], b[k]), k


def test_degenerate_inputs(oracle_lib):
    W = np.zeros((4, 64), np.float32)
    res = oracle_lib.solve(W, "NVFP4", 3)
    assert np.all(res["nmse"] == 0) and np.all(res["codes"] == 0) and res["tscale"] == 0
    assert np.all(res["r"] == 1) and np.all(res["c"] == 1)
    W = _w(4, 128, 9)
    W[2] = 0   # an all-zero row keeps its scale (D = 0)
    res = oracle_lib.solve(W, "MXFP4", 2, r_init=np.full(4, 2.0, np.float32))
    assert res["r"][2] == 2.0 and np.isnan(res["r_pre"][2])
    Wbad = synth.bf16_bits_to_f32(_w(4, 64, 9)).copy()
    Wbad[1, 3] = np.inf
    with pytest.raises(ValueError):
        oracle_lib.solve(Wbad, "NVFP4", 1)
    with pytest.raises(ValueError):
        oracle_lib.solve(_w(4, 48, 9), "MXFP4", 1)   # 48 columns is not a whole number of blocks


# ------------------------------------------------------------------ activation path
@pytest.mark.parametrize("fmt", FORMATS)
def test_rescale_is_exact_for_admissible_scales(oracle_lib, fmt):
    rng = np.random.default_rng(10)
    x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal(200_000).astype(np.float32) * 30))
    c = oracle_lib.project(fmt, np.exp2(rng.uniform(-6, 6, 200_000)).astype(np.float32))
    prod32 = (x * c).astype(np.float32).astype(np.float64)
    assert np.array_equal(prod32, x.astype(np.float64) * c.astype(np.float64))


@pytest.mark.parametrize("fmt", FORMATS)
def test_rescale_quantize_is_fq_of_rescaled(oracle_lib, fmt):
    rng = np.random.default_rng(11)
    X = synth.f32_to_bf16_bits(rng.standard_normal((32, 256)).astype(np.float32))
    c = oracle_lib.project(fmt, np.exp2(rng.uniform(-2, 2, 256)).astype(np.float32))
    codes, scales, ts, xq = oracle_lib.rescale_quantize_acts(X, c, fmt)
    V = (synth.bf16_bits_to_f32(X) * c[None, :]).astype(np.float32)
    c2, s2, t2, q2, _ = oracle_lib.fq(V, fmt)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2) and ts == t2
    codes1, scales1, ts1, _ = oracle_lib.rescale_quantize_acts(X, None, fmt)
    c3, s3, t3, _, _ = oracle_lib.fq(synth.bf16_bits_to_f32(X), fmt)
    assert np.array_equal(codes1, c3) and np.array_equal(scales1, s3) and ts1 == t3


def test_sqnr_closed_forms(oracle_lib):
    # MXINT4 block of 32 whose values are exactly representable: zero error
    q = np.arange(-7, 8, dtype=np.float64)
    row = np.concatenate([q, q, [7.0, -7.0]]) * 0.25        # scale 2^(e-2) with e = 0
    X = synth.f32_to_bf16_bits(row.astype(np.float32)[None, :])
    codes, scales, ts, _ = oracle_lib.rescale_quantize_acts(X, None, "MXINT4")
    assert oracle_lib.act_sqnr(X, None, codes, scales, ts, "MXINT4") == np.inf
    # move one element off the grid by delta < half a step: it rounds back, error = delta
    row2 = row.copy()
    row2[3] += 0.0625
    X2 = synth.f32_to_bf16_bits(row2.astype(np.float32)[None, :])
    codes, scales, ts, _ = oracle_lib.rescale_quantize_acts(X2, None, "MXINT4")
    want = 10 * np.log10(np.sum(row2 ** 2) / 0.0625 ** 2)
    assert np.isclose(oracle_lib.act_sqnr(X2, None, codes, scales, ts, "MXINT4"), want, rtol=1e-12)
    # with a column scale c = 2 on that element the rescaled value is on the grid again
    # only if the block scale is unchanged; the SQNR is then measured after dividing by c
    c = np.ones(32, np.float32)
    c[5] = 2.0
    codes, scales, ts, xq = oracle_lib.rescale_quantize_acts(X, c, "MXINT4")
    deq = oracle_lib.dequantize(codes, scales, ts, "MXINT4", 1, 32).astype(np.float64)[0]
    xhat = deq / c
    x = synth.bf16_bits_to_f32(X)[0].astype(np.float64)
    want = 10 * np.log10(np.sum(x ** 2) / np.sum((x - xhat) ** 2)) if np.any(x != xhat) else np.inf
    got = oracle_lib.act_sqnr(X, c, codes, scales, ts, "MXINT4")
    assert (got == want) or np.isclose(got, want, rtol=1e-12)
