"""The full synthetic Llama-3.1-8B projection set (32 layers x q, k, v, o, gate, up, down;
6.98 G weights, 14 GB bf16), NVFP4, 20 BCD iterations, solved as ONE batch on the GPU.

Five members (the two 14336-long shapes among them) are drawn with the numpy generator the
oracle shares and compared with the oracle end to end; one of them is also solved alone and must equal its batched result
bit for bit.  Every member is checked for the properties that hold at any size: all 20
iterations run, the normalised MSE never increases and ends no worse than the start, the
scales are finite and admissible.
"""

import numpy as np
import pytest
import torch

import post_quantization_dq_amd as dq
import synth
from gpu_util import DEV, scales_np, to_dev
from test_gpu_solve import _compare_e2e

pytestmark = pytest.mark.gpu

T = 20
# (layer, projection): k and v of layer 0, k of layer 31, gate of layer 17 (14336 rows) and
# down of layer 5 (14336 columns)
SAMPLED = {(0, 1), (0, 2), (31, 1), (17, 4), (5, 6)}


def test_llama31_8b_set_batched(oracle_lib):
    probs, meta = [], []
    for layer in range(synth.LLAMA31_8B_LAYERS):
        for pi, (name, rows, cols) in enumerate(synth.LLAMA31_8B_PROJ):
            spec = synth.llama_projection_spec(layer, pi)
            if (layer, pi) in SAMPLED:
                Wn = synth.matrix(spec, 0)
                W = to_dev(Wn)
            else:
                Wn, W = None, synth.matrix_device(spec, 0, DEV)
            probs.append(dq.make_problem(W, "NVFP4", T, trace=Wn is not None))
            meta.append((layer, name, Wn))
    total = sum(p.W.numel() for p in probs)
    print(f"[llama] {len(probs)} matrices, {total / 1e9:.2f} G weights", flush=True)
    assert len(probs) == 224 and total == 6_979_321_856
    reps = dq.solve_many(probs, "NVFP4", T)
    torch.cuda.synchronize()
    print("[llama] batched solve done", flush=True)

    for p, rep, (layer, name, Wn) in zip(probs, reps, meta):
        nm = p.nmse_hist.cpu().numpy()
        assert rep.iters_run == T, (layer, name)
        assert np.all(np.diff(nm) <= 0.0) and nm[-1] <= nm[0], (layer, name, nm)
        for v in (p.r, p.c):
            x = v.cpu().numpy()
            assert np.all(np.isfinite(x)) and np.all(x >= 2.0 ** -9) and np.all(x <= 448.0)
        assert (rep.flags & 1) == 0   # no non-finite input

    for p, rep, (layer, name, Wn) in zip(probs, reps, meta):
        if Wn is None:
            continue
        print(f"[llama] oracle check layer {layer} {name} {Wn.shape}", flush=True)
        got = {"r": p.r.cpu().numpy(), "c": p.c.cpu().numpy(),
               "codes": p.codes.cpu().numpy(),
               "scales": scales_np(p.block_scales, "NVFP4"),
               "tscale": float(p.tensor_scale.item()),
               "nmse": p.nmse_hist.cpu().numpy(), "relchg": p.relchg_hist.cpu().numpy(),
               "r_trace": p.r_trace.cpu().numpy(), "c_trace": p.c_trace.cpu().numpy(),
               "iters_run": rep.iters_run, "rejected": rep.rejected_steps}
        _compare_e2e(oracle_lib, Wn, "NVFP4", T, got, f"llama L{layer} {name}")

    # batch == alone, bit for bit
    k = next(i for i, m in enumerate(meta) if m[2] is not None)
    one = dq.solve(to_dev(meta[k][2]), "NVFP4", T)
    torch.cuda.synchronize()
    assert torch.equal(one["codes"], probs[k].codes) and torch.equal(one["r"], probs[k].r)
    assert torch.equal(one["c"], probs[k].c) and torch.equal(one["nmse"], probs[k].nmse_hist)
