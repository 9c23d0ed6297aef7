"""The quantiser and layer calls recorded in a HIP graph.

dq_rescale_quantize_acts (NVFP4: amax partials in the workspace), its multi-output (INT4
g64) and no-allocation forms, dq_quantize_weights, dq_quantized_linear_ws (INT4 with K split
over a workspace; NVFP4), dq_recode_mxint4_to_mxfp6 and dq_dequantize enqueue kernels only:
no allocation, no memset, no host wait, and every workspace byte a kernel reads was written
earlier in the same call.  So a forward made of them can be captured once and replayed.
Each replay here runs on new inputs, with eager work and host synchronisations between
replays, and must equal the eager calls on the same inputs bit for bit (codes, scales,
tensor scales, dequantised values and layer outputs)."""

import pytest
import torch

import post_quantization_dq_amd as dq
from gpu_util import DEV

pytestmark = pytest.mark.gpu

M, K, NQ, NN = 16, 4096, 1024, 512


def _randn(rows, cols, seed, std, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(rows, cols, generator=g) * std).to(dtype).to(DEV)


def _col_scales(cols, seed):
    g = torch.Generator().manual_seed(seed)
    c = torch.exp2(torch.rand(cols, generator=g) * 2.0 - 1.0)
    return c.to(torch.bfloat16).float().to(DEV)   # bf16 values, as the solver's c are


class _Fwd:
    """Buffers and workspaces of one mini forward: q/k/v-like INT4 g64 layers fed by one
    fused activation quantise, and an NVFP4 layer fed by the single-output quantise."""

    def __init__(self, w):
        self.w = w
        si, sn = dq.spec_of("INT4", 64), dq.spec_of("NVFP4")
        self.si, self.sn = si, sn
        self.acts = [dq._outputs(M, K, "INT4", 64, DEV) for _ in range(3)]
        self.qws = torch.empty(max(1, dq.dq_quantize_multi_workspace_bytes(M, K, 3, si)),
                               dtype=torch.uint8, device=DEV)
        nb = dq.dq_quantized_linear_workspace_bytes(si, M, NQ, K)
        assert nb > 0   # few tokens: K is split
        self.lws = torch.empty(nb, dtype=torch.uint8, device=DEV)
        self.ys = [torch.empty(M, NQ, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
        self.nact = dq._outputs(M, K, "NVFP4", 16, DEV)
        self.nws = torch.empty(max(1, dq.dq_quantize_workspace_bytes(M, K, sn)), dtype=torch.uint8,
                               device=DEV)
        self.yn = torch.empty(M, NN, dtype=torch.float32, device=DEV)
        # weight-side calls on a small weight that changes between replays
        self.wq = dq._outputs(NN, K, "NVFP4", 16, DEV)
        self.wws = torch.empty(max(1, dq.dq_quantize_workspace_bytes(NN, K, sn)), dtype=torch.uint8,
                               device=DEV)
        self.wdeq = torch.empty(NN, K, dtype=torch.float32, device=DEV)
        self.na = dq._outputs(M, K, "NVFP4", 16, DEV)
        self.mx = dq._outputs(M, K, "MXINT4", 32, DEV)
        self.mxws = torch.empty(max(1, dq.dq_quantize_workspace_bytes(M, K, dq.spec_of("MXINT4"))),
                                dtype=torch.uint8, device=DEV)
        self.rc = (torch.empty(M * K * 3 // 4, dtype=torch.uint8, device=DEV),
                   torch.empty(M * K // 32, dtype=torch.uint8, device=DEV))

    def run(self, X, X2):
        w = self.w
        dq.dq_rescale_quantize_acts_multi(X, w["c"], self.si, [a[0] for a in self.acts],
                                          [a[1] for a in self.acts], [a[2] for a in self.acts],
                                          self.qws)
        for o in range(3):
            codes, scales, _ = w["q"][o]
            dq.dq_quantized_linear_ws(self.si, self.acts[o][0], self.acts[o][1], None, M, codes,
                                      scales, None, NQ, K, w["r"][o], self.ys[o], self.lws)
        dq.dq_rescale_quantize_acts(X2, w["cn"], self.sn, *self.nact, self.nws)
        codes, scales, ts = w["n"]
        dq.dq_quantized_linear_ws(self.sn, self.nact[0], self.nact[1], self.nact[2], M, codes,
                                  scales, ts, NN, K, w["rn"], self.yn, None)
        dq.dq_quantize_weights(w["W"], w["rn"], w["cn"], self.sn, *self.wq, self.wws)
        dq.dq_dequantize(self.sn, *self.wq, NN, K, w["rn"], w["cn"], self.wdeq)
        dq.dq_rescale_quantize_acts_noalloc(X2, w["cn"], self.sn, *self.na)
        dq.dq_rescale_quantize_acts(X, None, dq.spec_of("MXINT4"), *self.mx, self.mxws)
        dq.dq_recode_mxint4_to_mxfp6(self.mx[0], self.mx[1], M, K, *self.rc)

    def outputs(self):
        out = ([t for a in self.acts for t in a] + self.ys + list(self.nact) + [self.yn] +
               list(self.wq) + [self.wdeq] + list(self.na) + list(self.mx[:2]) + list(self.rc))
        return [t.clone() for t in out]


def test_captured_forward_replays_equal_eager():
    w = {"c": [_col_scales(K, 10 + o) for o in range(3)], "cn": _col_scales(K, 20)}
    w["q"] = [dq.quantize_weights(_randn(NQ, K, 30 + o, 0.02), fmt="INT4", group=64)
              for o in range(3)]
    w["r"] = [_col_scales(NQ, 40 + o) for o in range(3)]
    w["n"] = dq.quantize_weights(_randn(NN, K, 50, 0.02), fmt="NVFP4")
    w["rn"] = _col_scales(NN, 51)
    w["W"] = _randn(NN, K, 52, 0.02)
    X = _randn(M, K, 1, 1.0)
    X2 = _randn(M, K, 2, 1.0)
    eager, graphed = _Fwd(w), _Fwd(w)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graphed.run(X, X2)   # a first run outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run(X, X2)
    torch.cuda.synchronize()

    for rep in range(4):
        # new inputs in place (eager work between replays), then eager calls and the replay
        X.copy_(_randn(M, K, 100 + rep, 1.0 + rep))
        X2.copy_(_randn(M, K, 200 + rep, 0.5 + rep))
        w["W"].copy_(_randn(NN, K, 300 + rep, 0.01 * (rep + 1)))
        torch.cuda.synchronize()
        eager.run(X, X2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(eager.outputs(), graphed.outputs())):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b), (rep, k)
        assert torch.count_nonzero(eager.ys[0]) > 0 and torch.count_nonzero(eager.yn) > 0
        assert torch.count_nonzero(eager.wdeq) > 0 and torch.equal(eager.na[0], eager.nact[0])


def test_captured_side_streams_equal_serial():
    """The independent layers of a group recorded on side streams (each with its own split
    workspace, joined back before the next call) replay to the same bits as the same calls
    issued one after another on one stream."""
    si = dq.spec_of("INT4", 64)
    w = [dq.quantize_weights(_randn(NQ, K, 60 + o, 0.02), fmt="INT4", group=64) for o in range(3)]
    r = [_col_scales(NQ, 70 + o) for o in range(3)]
    acts = dq.quantize_weights(_randn(M, K, 80, 1.0), fmt="INT4", group=64)   # M x K codes
    nb = dq.dq_quantized_linear_workspace_bytes(si, M, NQ, K)
    wss = [torch.empty(nb, dtype=torch.uint8, device=DEV) for _ in range(3)]
    ys_serial = [torch.empty(M, NQ, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    ys_graph = [torch.empty(M, NQ, dtype=torch.bfloat16, device=DEV) for _ in range(3)]

    def layer(o, y, ws):
        dq.dq_quantized_linear_ws(si, acts[0], acts[1], None, M, w[o][0], w[o][1], None, NQ, K,
                                  r[o], y, ws)

    side = [torch.cuda.Stream() for _ in range(3)]

    def branches():
        main = torch.cuda.current_stream()
        for o in range(3):
            side[o].wait_stream(main)
            with torch.cuda.stream(side[o]):
                layer(o, ys_graph[o], wss[o])
        for o in range(3):
            main.wait_stream(side[o])

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        branches()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        branches()
    torch.cuda.synchronize()
    for rep in range(3):
        new = dq.quantize_weights(_randn(M, K, 90 + rep, 1.0 + rep), fmt="INT4", group=64)
        acts[0].copy_(new[0])
        acts[1].copy_(new[1])
        for y in ys_graph:
            y.zero_()
        torch.cuda.synchronize()
        for o in range(3):
            layer(o, ys_serial[o], wss[0])   # one stream, one workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o in range(3):
            assert torch.equal(ys_serial[o].view(torch.uint8), ys_graph[o].view(torch.uint8)), (rep, o)
            assert torch.count_nonzero(ys_graph[o]) > 0
