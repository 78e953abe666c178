"""moe_dispatch_noalloc (the dispatch entry point that allocates nothing: its
workspace is a library-held device array) against moe_dispatch with a caller
workspace, through the C ABI: counts, offsets, perm, inv_perm and the sorted
rows bit for bit, on two calls in a row, the second smaller than the first
(the array keeps the first call's contents, which must not leak into the
second)."""
import numpy as np
import pytest
import torch

from expert_grouped_gemm_top_amd import moe
from expert_grouped_gemm_top_amd import workloads as W

pytestmark = pytest.mark.gpu


def _route(T, E, k, seed, skew):
    wl = W.custom("noalloc", T=T, H=64, F=64, E=E, k=k, dtype="bf16", skew=skew)
    logits = torch.from_numpy(W.generate(wl, seed=seed, weights=False)["logits"]).cuda()
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    moe.moe_route_topk(logits, idx, w, k)
    return idx


def _outputs(T, E, k, H):
    N = T * k
    z = lambda *s, dt=torch.int32: torch.full(s, -7, dtype=dt, device="cuda")  # noqa: E731
    return dict(counts=z(E), offsets=z(E + 1), perm=z(N), inv_perm=z(N),
                x_sorted=torch.zeros(N, H, dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("first,second", [((4096, 2048, 128, 8), (1000, 512, 64, 4)),
                                          ((16384, 256, 256, 8), (600, 128, 8, 2))])
def test_noalloc_dispatch_matches_workspace_dispatch(first, second):
    for call, (T, H, E, k) in enumerate((first, second)):
        print(f"noalloc dispatch call {call}: T={T} H={H} E={E} k={k}", flush=True)
        idx = _route(T, E, k, seed=call, skew=True)
        x = torch.from_numpy(W.round_bf16(np.random.default_rng([7, call]).standard_normal((T, H), np.float32)))
        x = x.to(torch.bfloat16).cuda()
        ref, got = _outputs(T, E, k, H), _outputs(T, E, k, H)
        ws = torch.empty(max(moe.moe_dispatch_workspace_bytes(T, E, k), 16), dtype=torch.uint8, device="cuda")
        assert moe.moe_dispatch_workspace_bytes(T, E, k) > 0  # the scratch array is in use
        moe.moe_dispatch(idx, x, ref["counts"], ref["offsets"], ref["perm"], ref["inv_perm"], ref["x_sorted"], ws, E)
        moe.moe_dispatch_noalloc(idx, x, got["counts"], got["offsets"], got["perm"], got["inv_perm"],
                                 got["x_sorted"], E)
        torch.cuda.synchronize()
        for n in ref:
            assert torch.equal(ref[n], got[n]), f"call {call}: {n} differs"
        # index-only form as well
        got2 = _outputs(T, E, k, H)
        moe.moe_dispatch_noalloc(idx, None, got2["counts"], got2["offsets"], got2["perm"], got2["inv_perm"], None, E)
        torch.cuda.synchronize()
        for n in ("counts", "offsets", "perm", "inv_perm"):
            assert torch.equal(ref[n], got2[n]), f"call {call} (index-only): {n} differs"
