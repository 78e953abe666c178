"""The whole training step (route, dispatch, forward, combine, [compaction],
dx, dg, dW) captured as one HIP graph with torch.cuda.graph: the library makes
no allocation, memset or host synchronization inside its calls, so a caller
can capture the step and replay it.  Every replay must be bitwise the eager
step; the replays run with eager steps and synchronizations between them, and
the outputs are poisoned before each replay so that a replay that wrote
nothing cannot pass.
"""
import numpy as np
import pytest
import torch

from expert_grouped_gemm_top_amd import workloads as W
from expert_grouped_gemm_top_amd.layer import MoeLayerBuffers
from moe_cases import logits_of, note, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # experts past 256 rows, 128-row tiles and the streaming path; both dW kernels
    (W.custom("graph_big", T=700, H=256, F=256, E=4, k=2, dtype="bf16", skew=True, dw=True), {}),
    (W.custom("graph_gather", T=300, H=256, F=128, E=16, k=4, dtype="bf16", skew=True, dw=True),
     {"gather_rows": True}),
    (W.custom("graph_compact", T=300, H=256, F=256, E=8, k=4, dtype="bf16", skew=True, dw=True, rho=0.6), {}),
    (W.custom("graph_recompute", T=300, H=256, F=256, E=8, k=4, dtype="bf16", skew=True, dw=True),
     {"keep_graph": False}),
    (W.custom("graph_fp32", T=90, H=64, F=40, E=6, k=3, dtype="f32", skew=True, dw=True), {}),
    # dW on a second stream, forked and joined inside the capture through an event
    (W.custom("graph_overlap", T=700, H=256, F=256, E=4, k=2, dtype="bf16", skew=True, dw=True),
     {"overlap_dw": True}),
]


@pytest.mark.parametrize("wl,opts", CASES, ids=[c[0].name for c in CASES])
def test_captured_step_replays_bitwise(wl, opts):
    note(f"graph capture {wl.name} T={wl.T} H={wl.H} F={wl.F} E={wl.E} k={wl.k} {wl.dtype} rho={wl.rho} {opts}")
    d = W.generate(wl, seed=0)
    t = to_dev(wl, d)
    logits = torch.from_numpy(np.ascontiguousarray(logits_of(wl, d))).cuda()
    L = MoeLayerBuffers(wl.T, wl.H, wl.F, wl.E, wl.k, t["x"].dtype, "cuda", rho=wl.rho, dw=wl.dw, dg=True, **opts)

    def step(stream):
        L.forward(logits, t["x"], t["W_gate"], t["W_up"], t["W_down"], stream)
        L.backward(t["dy"], t["W_gate"], t["W_up"], t["W_down"], stream=stream)

    outs = [L.y, L.dx, L.dg, L.dw_gate, L.dw_up, L.dw_down]
    # warm up on a side stream (capture requires it), then the eager reference
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step(side)
    torch.cuda.current_stream().wait_stream(side)
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()

    for replay in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for name, o, r in zip(("y", "dx", "dg", "dw_gate", "dw_up", "dw_down"), outs, ref):
            assert torch.equal(o, r), f"replay {replay}: {name} differs from the eager step"
        step(torch.cuda.current_stream())  # eager work between replays
        torch.cuda.synchronize()
