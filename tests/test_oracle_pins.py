"""More pins for the oracle's solve, each fixed by something other than the oracle's code.

  * MX dual scales: a power-of-two row scale is absorbed exactly by every block's E8M0
    exponent (same codes, same reconstruction), a bf16 row scale is not, and row scales
    alone improve an MX fit.  This is the fact behind the bf16 admissible set of the MX
    dual scales (the conference entry's abstract: the method formally supports MX; the
    news summary: row scales alone already help).
  * NVFP4 planted fixed point: W = diag(r0) Q0 diag(c0) with Q0 on the NVFP4 grid, its
    block maxima at the top of E2M1 and one block at the top of E4M3, is reproduced
    exactly (power-of-two scales) or within rounding (E4M3 scales).
  * The reconstruction error through the column sums of the c-step:
    F = ||W||^2 - 2 sum_j c_j N_j + sum_j c_j^2 D_j, with N_j, D_j summed by numpy.
  * Convergence against the thresholds proposed for the listing page's Fig. 2 / Fig. 3
    captions (relative change near zero by t ~ 16, NMSE plateau within ~10 iterations),
    recorded per workload as the facts they are.
  * The NVFP4 tensor-scale limit derived from fp32 arithmetic, at its boundary.
  * Resuming a solve from its state (r, c, kept Qhat) is exact, also after a rejected step.
"""

import numpy as np
import pytest
import torch

import synth

MX = ["MXINT4", "MXFP4", "MXINT8", "MXFP8_E4M3", "MXFP6_E2M3"]


def _f64(W):
    return (synth.bf16_bits_to_f32(W) if W.dtype == np.uint16 else W).astype(np.float64)


# ------------------------------------------------------------------ MX dual scales
@pytest.mark.parametrize("fmt", MX)
def test_mx_power_of_two_row_scale_is_absorbed(oracle_lib, fmt):
    rng = np.random.default_rng(1)
    W = synth.matrix(synth.WORKLOADS["q4096x4096_mxfp4"]["W"].scaled(32, 512), 0)
    c0, s0, _, q0 = oracle_lib.quantize_weights(W, None, None, fmt)
    k = rng.integers(-3, 4, 32)
    r2 = np.ldexp(np.float32(1), k).astype(np.float32)
    c1, s1, _, q1 = oracle_lib.quantize_weights(W, r2, None, fmt)
    # codes unchanged, every block exponent shifted by -k, reconstruction r * Qhat unchanged
    assert np.array_equal(c0, c1)
    nz = s0.reshape(32, -1) > 0
    assert np.array_equal((s1.reshape(32, -1).astype(int) + k[:, None])[nz], s0.reshape(32, -1).astype(int)[nz])
    assert np.array_equal(q1.astype(np.float64) * r2[:, None], q0.astype(np.float64))
    # a bf16 row scale that is not a power of two changes codes
    rb = oracle_lib.project(fmt, np.full(32, 1.1, np.float32))
    c2, _, _, _ = oracle_lib.quantize_weights(W, rb, None, fmt)
    assert not np.array_equal(c0, c2)


@pytest.mark.parametrize("fmt", ["MXFP4", "MXINT4"])
def test_mx_row_scales_alone_improve_the_fit(oracle_lib, fmt):
    name = "q4096x4096_mxfp4" if fmt == "MXFP4" else "k1024x4096_mxint4"
    W = synth.matrix(synth.WORKLOADS[name]["W"].scaled(128, 1024), 0)
    res = oracle_lib.solve(W, fmt, 8, steps=1)
    assert np.all(res["c"] == 1.0)
    assert res["nmse"][-1] < res["nmse"][0]
    assert np.any(np.frexp(res["r"])[0] != 0.5)   # not powers of two
    both = oracle_lib.solve(W, fmt, 8)
    assert both["nmse"][-1] < res["nmse"][-1]


# ------------------------------------------------------------------ NVFP4 planted point
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def _nvfp4_planted(rows, cols, seed, st_exp=-14):
    """Q0 on the NVFP4 grid: s_t = 2^st_exp, block scales random E4M3 values, every block's
    largest element +-6, and one block at the top scale 448 (so the matrix amax is
    6 * 448 * s_t and the tensor scale is recovered exactly)."""
    rng = np.random.default_rng(seed)
    nb = cols // 16
    q = E2M1[rng.integers(0, 8, (rows, nb, 16))] * rng.choice([-1, 1], (rows, nb, 16))
    q[:, :, 3] = 6.0 * rng.choice([-1, 1], (rows, nb))
    sb = torch.from_numpy(rng.integers(0x20, 0x7F, (rows, nb, 1)).astype(np.uint8)).view(
        torch.float8_e4m3fn).double().numpy()
    sb[0, 0, 0] = 448.0
    Q0 = (q * sb * np.ldexp(1.0, st_exp)).reshape(rows, cols)
    return Q0


def test_nvfp4_planted_fixed_point_exact(oracle_lib):
    rows, cols = 8, 64
    Q0 = _nvfp4_planted(rows, cols, 4)
    rng = np.random.default_rng(5)
    r0 = np.ldexp(1.0, rng.integers(-2, 3, rows))
    c0 = np.ldexp(1.0, rng.integers(-2, 3, cols))
    W = (r0[:, None] * Q0 * c0[None, :]).astype(np.float32)
    assert np.array_equal(W.astype(np.float64), r0[:, None] * Q0 * c0[None, :])   # exact
    _, _, ts, q = oracle_lib.quantize_weights(W, r0.astype(np.float32), c0.astype(np.float32), "NVFP4")
    assert ts == np.ldexp(1.0, -14) and np.array_equal(q.astype(np.float64), Q0)
    res = oracle_lib.solve(W, "NVFP4", 4, r_init=r0.astype(np.float32), c_init=c0.astype(np.float32))
    assert np.all(res["nmse"] == 0.0) and np.all(res["relchg"] == 0.0)
    assert np.array_equal(res["r"], r0) and np.array_equal(res["c"], c0)
    assert res["rejected"] == 0 and res["tscale"] == np.ldexp(1.0, -14)


def test_nvfp4_planted_fixed_point_e4m3_scales(oracle_lib):
    """With scales that are not powers of two, 1/r is rounded, so the normalised matrix is
    Q0 up to fp32 rounding: the codes, block scales and dual scales are reproduced and the
    error stays at rounding level."""
    rows, cols = 8, 64
    Q0 = _nvfp4_planted(rows, cols, 6)
    rng = np.random.default_rng(7)
    e4m3 = lambda n: torch.from_numpy(rng.integers(0x30, 0x48, n).astype(np.uint8)).view(
        torch.float8_e4m3fn).double().numpy()
    r0, c0 = e4m3(rows), e4m3(cols)
    W = (r0[:, None] * Q0 * c0[None, :]).astype(np.float32)
    assert np.array_equal(W.astype(np.float64), r0[:, None] * Q0 * c0[None, :])
    codes0, scales0, _, _ = oracle_lib.quantize_weights(W, r0.astype(np.float32), c0.astype(np.float32), "NVFP4")
    res = oracle_lib.solve(W, "NVFP4", 4, r_init=r0.astype(np.float32), c_init=c0.astype(np.float32))
    assert np.array_equal(res["r"], r0.astype(np.float32)) and np.array_equal(res["c"], c0.astype(np.float32))
    assert np.array_equal(res["codes"], codes0) and np.array_equal(res["scales"], scales0)
    assert np.all(res["nmse"] <= 1e-12)


# ------------------------------------------------------------------ F through the c-step sums
@pytest.mark.parametrize("fmt,name", [("NVFP4", "down4096x14336_nvfp4"), ("MXINT4", "k1024x4096_mxint4"),
                                      ("INT4", "w256x512_int4"), ("MXFP4", "q4096x4096_mxfp4")])
def test_error_identity_through_column_sums(oracle_lib, fmt, name):
    """For the c-step of iteration t (new r^t, kept Qhat^{t-1}): numpy's N_j, D_j give the
    oracle's unprojected c^t, and ||W||^2 - 2 sum c_j N_j + sum c_j^2 D_j at the projected
    c^t equals the direct reconstruction error at (r^t, c^t, Qhat^{t-1})."""
    W = synth.matrix(synth.WORKLOADS[name]["W"].scaled(96, 512), 0)
    Wf = _f64(W)
    nW = np.sum(Wf ** 2)
    for t in (1, 3):
        prev = oracle_lib.solve(W, fmt, t - 1)
        cur = oracle_lib.solve(W, fmt, t)
        Q = oracle_lib.dequantize(prev["codes"], prev["scales"], prev["tscale"], fmt, *W.shape).astype(np.float64)
        r = cur["r"].astype(np.float64)
        N = np.sum(r[:, None] * Wf * Q, axis=0)
        D = np.sum((r[:, None] * Q) ** 2, axis=0)
        ok = D > 0
        x = cur["c_trace"][t - 1]
        assert np.array_equal(np.isnan(x), ~ok)
        assert np.all(np.abs(x[ok] - N[ok] / D[ok]) <= 2.0 ** -23 * np.abs(N[ok] / D[ok]))
        c = cur["c"].astype(np.float64)
        F_id = nW - 2.0 * np.sum(c * N) + np.sum(c * c * D)
        F_direct = np.sum((Wf - r[:, None] * Q * c[None, :]) ** 2)
        assert abs(F_id - F_direct) <= 1e-9 * F_direct
        if cur["relchg"][t] == 0.0:   # the candidate was rejected or equal: nmse[t] is F(Qhat^{t-1})
            assert abs(cur["nmse"][t] * nW - F_id) <= 1e-9 * F_id


# ------------------------------------------------------------------ convergence facts
# The thresholds proposed for the pages' qualitative captions: relchg[t] <= 1e-3 for some
# t <= 16, and the NMSE moving by less than 1% after t = 10.  On these synthetic weights
# the oracle meets them as recorded here.  INT4 and MXINT4 are still improving at t = 16
# (NMSE down 27% and 13% after t = 10); their relchg reaches 0 only at a rejected step
# (t = 15), where Qhat does not move.  Every MXFP4 candidate is rejected, so Qhat never
# moves and the NMSE is flat after the first scale steps.  NVFP4's change is 0.005 at
# t = 16 and its NMSE moves 0.9% after t = 10.
C8 = {"w256x512_int4": (True, False), "k1024x4096_mxint4": (True, False),
      "q4096x4096_mxfp4": (True, True), "down4096x14336_nvfp4": (False, True)}


@pytest.mark.slow
@pytest.mark.parametrize("name", list(C8))
def test_convergence_thresholds(oracle_lib, name):
    W, _, fmt, _, _ = synth.workload(name)
    res = oracle_lib.solve(W, fmt, 16)
    rc, nm = res["relchg"], res["nmse"]
    assert np.all(np.diff(nm) <= 0.0) and nm[-1] <= nm[0]
    relchg_ok = bool(np.any(rc[1:17] <= 1e-3))
    plateau_ok = bool(np.max(np.abs(nm[10:] - nm[10])) < 0.01 * nm[10])
    print(f"[c8] {name}: relchg {np.array2string(rc[1:], precision=4)}, nmse {nm[0]:.5g} -> {nm[-1]:.5g}, "
          f"rejected {res['rejected']}")
    assert (relchg_ok, plateau_ok) == C8[name]


# ------------------------------------------------------------------ NVFP4 tensor-scale limit
def _predict_tiny(A: np.float32) -> bool:
    """The limit derived from fp32 arithmetic: s_t = fl(A / 2688); every block factor
    d = e4m3(sb) s_t (smallest sb = 2^-9) and 6 s_t must have finite fp32 reciprocals."""
    with np.errstate(over="ignore", divide="ignore"):
        st = np.float32(A) / np.float32(2688)
        k6 = np.float32(1) / (np.float32(6) * st)
        idm = np.float32(1) / (np.float32(2.0 ** -9) * st)
    return not (st > 0 and np.isfinite(k6) and np.isfinite(idm))


def test_nvfp4_tensor_scale_limit(oracle_lib):
    rng = np.random.default_rng(8)
    base = (rng.standard_normal((4, 64)) * 0.25).astype(np.float32)
    # the boundary: fl(2^-9 s_t) <= 2^-128, i.e. s_t just above 2^-119
    edge = np.float32(2.0 ** -119) * np.float32(2688)
    As = [np.nextafter(edge, np.float32(0)), edge, np.nextafter(edge, np.float32(1)),
          np.float32(edge * 1.001), np.float32(edge * 0.999), np.float32(2.0 ** -100),
          np.float32(2.0 ** -140), np.float32(1e-44)]
    seen = set()
    for A in As:
        V = (base / np.abs(base).max() * A).astype(np.float32)
        V[0, 0] = A
        codes, scales, ts, q, flags = oracle_lib.fq(V, "NVFP4")
        tiny = _predict_tiny(A)
        seen.add(tiny)
        assert bool(flags & 16) == tiny, A
        if tiny:
            assert ts == 0.0 and np.all(codes == 0) and np.all(scales == 0) and np.all(q == 0)
        else:
            assert ts == np.float32(A) / np.float32(2688) and np.all(np.isfinite(q))
            assert np.any(codes != 0) and np.abs(q).max() > 0
    assert seen == {True, False}
    # in a solve the flag reaches the report and the codes are zero
    V = (base / np.abs(base).max() * np.float32(2.0 ** -112)).astype(np.float32)
    res = oracle_lib.solve(V, "NVFP4", 2)
    assert res["flags"] & 16 and np.all(res["codes"] == 0) and res["tscale"] == 0.0


# ------------------------------------------------------------------ resume
@pytest.mark.parametrize("fmt,name,split", [("INT4", "w256x512_int4", None), ("NVFP4", "down4096x14336_nvfp4", 5)])
def test_resume_is_exact(oracle_lib, fmt, name, split):
    """solve(T) equals solve(t) followed by a solve resumed from its outputs; for INT4 the
    split sits after a rejected step, where the kept Qhat is not FQ(W ./ r c^T)."""
    W = synth.matrix(synth.WORKLOADS[name]["W"].scaled(256, 512), 0)
    T = 20
    full = oracle_lib.solve(W, fmt, T)
    if split is None:
        rej = [t for t in range(1, T + 1) if full["relchg"][t] == 0.0]
        assert rej, "expected a rejected step"
        split = rej[0]
    a = oracle_lib.solve(W, fmt, split)
    b = oracle_lib.solve(W, fmt, T - split, r_init=a["r"], c_init=a["c"],
                         q_init=(a["codes"], a["scales"], a["tscale"]))
    assert np.array_equal(full["nmse"][split:], b["nmse"])
    assert np.array_equal(full["relchg"][split + 1:], b["relchg"][1:])
    for k in ("r", "c", "codes", "scales"):
        assert np.array_equal(full[k], b[k]), k
    assert full["tscale"] == b["tscale"]
    assert full["rejected"] == a["rejected"] + b["rejected"]
    if fmt == "INT4":   # the scales alone do not resume a rejected state
        c_only = oracle_lib.solve(W, fmt, 1, r_init=a["r"], c_init=a["c"])
        assert c_only["nmse"][0] != b["nmse"][0]
