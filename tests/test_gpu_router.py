"""GPU parity of the router: moe_router_fwd (logits = x W_r) and moe_router_bwd
(dlogits, dW_r and the router's share of dx, with the top-k selection fixed),
against the CPU oracle on the same seeded inputs.

Inputs of both sides come from the seeded generator and the oracle only: the
selection and weights are the oracle's routing of the oracle's logits (rounded
to fp32), and dg is a seeded fp32 draw.
"""
import numpy as np
import pytest
import torch

import oracle
from expert_grouped_gemm_top_amd import moe
from moe_cases import assert_close, note, np32

pytestmark = pytest.mark.gpu

# fp32 outputs are sums of products that are exact in fp32 (bf16 inputs) or
# rounded once (fp32 inputs); bf16 outputs carry one rounding (2^-9 relative).
TOL_F32 = 1e-5
TOL_OUT = {"f32": 1e-5, "bf16": 1e-2}


def _round_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).bfloat16().float().numpy().astype(np.float64)


def _case(T, H, E, k, dtype, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (0.02 * rng.standard_normal((H, E))).astype(np.float32)
    dg = rng.standard_normal((T, k)).astype(np.float32)
    dx0 = rng.standard_normal((T, H)).astype(np.float32)
    if dtype == "bf16":
        x, wr, dx0 = _round_bf16(x), _round_bf16(wr), _round_bf16(dx0)
    x, wr, dx0 = (a.astype(np.float64) for a in (x, wr, dx0))
    logits = oracle.router_logits(x, wr).astype(np.float32)
    idx, w = oracle.route_topk(logits, k)
    return x, wr, dg.astype(np.float64), dx0, logits, idx, w.astype(np.float32)


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    return t.bfloat16() if dtype == "bf16" else t


SHAPES = [
    (64, 128, 8, 2, "f32"),
    (100, 256, 37, 5, "bf16"),
    (300, 384, 128, 8, "bf16"),
    (70, 136, 256, 16, "f32"),
    (1, 128, 1, 1, "bf16"),
    (33, 104, 20, 3, "bf16"),  # rows of W_r at alternating 16-byte alignment, a ragged reduction tail
    (4096, 2048, 128, 8, "bf16"),  # the Qwen3-30B-A3B router at 4096 tokens
]


@pytest.mark.parametrize("T,H,E,k,dtype", SHAPES)
def test_router_forward_and_backward(T, H, E, k, dtype):
    note(f"router T={T} H={H} E={E} k={k} {dtype}")
    x, wr, dg, dx0, logits_ref32, idx, w32 = _case(T, H, E, k, dtype, seed=T * 7 + E)
    xd, wrd = _dev(x, dtype), _dev(wr, dtype)
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, moe.moe_router_workspace_bytes(T, H, E)), dtype=torch.uint8, device="cuda")
    moe.moe_router_fwd(xd, wrd, logits, ws)
    ref_logits = oracle.router_logits(x, wr)
    assert_close("logits", np32(logits), ref_logits, TOL_F32)

    dl_ref, dwr_ref, dxr_ref = oracle.router_backward(x, wr, idx, w32.astype(np.float64), dg)
    idx_d = torch.from_numpy(idx).cuda()
    w_d = torch.from_numpy(w32).cuda()
    dg_d = torch.from_numpy(dg.astype(np.float32)).cuda()
    dl = torch.empty(T, E, dtype=torch.float32, device="cuda")
    dwr = torch.empty_like(wrd)
    for accumulate in (False, True):
        dx = _dev(dx0, dtype)
        moe.moe_router_bwd(xd, wrd, idx_d, w_d, dg_d, dl, dwr, dx, accumulate, ws)
        torch.cuda.synchronize()
        assert_close("dlogits", np32(dl), dl_ref, TOL_F32)
        # unselected experts get exact zeros
        mask = np.ones((T, E), bool)
        np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
        assert not np32(dl)[mask].any()
        assert_close("dW_r", np32(dwr), dwr_ref, TOL_OUT[dtype])
        assert_close("dx", np32(dx), dxr_ref + (dx0 if accumulate else 0), TOL_OUT[dtype])


def test_router_backward_k1_is_zero():
    T, H, E, k = 50, 128, 16, 1
    x, wr, dg, dx0, _, idx, w32 = _case(T, H, E, k, "bf16", seed=3)
    xd, wrd = _dev(x, "bf16"), _dev(wr, "bf16")
    dl = torch.full((T, E), 7.0, device="cuda")
    dwr = torch.full_like(wrd, 7.0)
    dx = _dev(dx0, "bf16")
    ws = torch.empty(max(16, moe.moe_router_workspace_bytes(T, H, E)), dtype=torch.uint8, device="cuda")
    moe.moe_router_bwd(xd, wrd, torch.from_numpy(idx).cuda(), torch.from_numpy(w32).cuda(),
                       torch.from_numpy(dg.astype(np.float32)).cuda(), dl, dwr, dx, True, ws)
    torch.cuda.synchronize()
    assert not dl.any() and not dwr.float().any()
    assert torch.equal(dx, _dev(dx0, "bf16"))  # adding exact zeros leaves dx unchanged


def test_layer_with_router_matches_oracle():
    """Router in front of a small bf16 layer: logits from x W_r, the expert path,
    then the router's backward added to dx -- the full-layer input gradient."""
    from expert_grouped_gemm_top_amd import workloads as W
    from expert_grouped_gemm_top_amd.layer import MoeLayerBuffers
    wl = W.custom("bf16_router_layer", T=96, H=256, F=128, E=16, k=4, dtype="bf16", router="wr", dw=False)
    d = W.generate(wl, seed=2)
    note(f"layer with router {wl}")
    x, wr, dy = (d[n].astype(np.float64) for n in ("x", "W_r", "dy"))
    Wg, Wu, Wd = (d[n].astype(np.float64) for n in ("W_gate", "W_up", "W_down"))
    logits = oracle.router_logits(x, wr).astype(np.float32)
    idx, w = oracle.route_topk(logits, wl.k)
    y_ref = oracle.forward(x, idx, w, Wg, Wu, Wd)
    dx_ref, dg_ref = oracle.backward(x, idx, w, Wg, Wu, Wd, dy)
    _, dwr_ref, dxr_ref = oracle.router_backward(x, wr, idx, w, dg_ref)

    dev = {n: torch.from_numpy(d[n]).cuda().bfloat16() for n in ("x", "W_r", "W_gate", "W_up", "W_down", "dy")}
    L = MoeLayerBuffers(wl.T, wl.H, wl.F, wl.E, wl.k, torch.bfloat16, "cuda", dw=False, dg=True, router=True)
    L.forward(None, dev["x"], dev["W_gate"], dev["W_up"], dev["W_down"], w_r=dev["W_r"])
    L.backward(dev["dy"], dev["W_gate"], dev["W_up"], dev["W_down"], w_r=dev["W_r"])
    torch.cuda.synchronize()
    assert np.array_equal(L.topk_idx.cpu().numpy(), idx)
    assert_close("y", np32(L.y), y_ref, 1e-2)
    assert_close("dg", np32(L.dg), dg_ref, 1e-2)
    assert_close("dW_r", np32(L.dw_r), dwr_ref, 1e-2)
    assert_close("dx (experts + router)", np32(L.dx), dx_ref + dxr_ref, 1e-2)
