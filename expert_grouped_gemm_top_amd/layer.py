"""One MoE layer's expert computation in training, driven through the C ABI.

``MoeLayerBuffers`` owns every device buffer of the path (torch allocations,
sized once from the host capacities) and ``forward`` / ``backward`` enqueue the
library calls in order on one stream -- (router logits,) route, dispatch,
grouped SwiGLU forward, combine; then optionally compaction, backward dx (+ dg),
dW and the router's backward.  No step here computes anything itself: every
value comes from libmoe's kernels.
"""
from __future__ import annotations

import torch

from . import moe


class MoeLayerBuffers:
    def __init__(self, T, H, F, E, k, dtype=torch.bfloat16, device="cuda", rho=None, dw=True, dg=True,
                 router=False, keep_graph=True, quota_cap=None, gather_rows=None, overlap_dw=False):
        """rho: quota ratio of the compacted backward (None: no compaction);
        quota_cap: the per-expert quota directly (e.g. from
        moe.moe_quota_cap_for_budget), instead of rho.  keep_graph=False: the
        forward keeps no pre-activations [hg|hu]; the backward recomputes them
        from the token rows (the recompute path that pull request #44 keeps
        behind keep_graph=False).  gather_rows: every GEMM reads the token
        rows x and the saved activations through the pair / row indices
        (perm, kept_perm, kept_src), so neither x_sorted nor the compacted
        copies are materialized; False materializes them (moe_dispatch's row
        copy, moe_compact_pairs' row gathers).  Results are the same bit for
        bit.  None picks gathering unless dW runs over all pairs: there the
        weight-gradient GEMM streams each expert's x rows many times, and
        contiguous rows serve it better than one copy costs.  overlap_dw: the
        weight gradients run on a second stream (default priority) alongside
        the dX GEMM and the dx sum, from the point where the dx call signals dO
        and dh complete (moe_signal_dh_ready); the caller's stream then waits
        for them.  Results are the same bit for bit."""
        self.T, self.H, self.F, self.E, self.k = T, H, F, E, k
        self.keep_graph = keep_graph
        self.N = N = T * k
        self.dtype, self.rho, self.dw, self.want_dg = dtype, rho, dw, dg
        dev = torch.device(device)
        self.device = dev
        self.overlap_dw = bool(overlap_dw) and dw
        if self.overlap_dw:
            self._dw_stream = torch.cuda.Stream(device=dev)  # default priority
            self._dh_ready = torch.cuda.Event()
            self._dh_ready.record(torch.cuda.current_stream(dev))  # creates the underlying hipEvent
        i32, f32 = torch.int32, torch.float32
        em = lambda *s, dt=dtype: torch.empty(*s, dtype=dt, device=dev)  # noqa: E731
        self.topk_idx = em(T, k, dt=i32)
        self.topk_w = em(T, k, dt=f32)
        self.counts = em(E, dt=i32)
        self.offsets = em(E + 1, dt=i32)
        self.perm = em(N, dt=i32)
        self.inv_perm = em(N, dt=i32)
        ws = moe.moe_dispatch_workspace_bytes(T, E, k)
        self.ws = em(max(ws, 16), dt=torch.uint8)
        compacted = rho is not None or quota_cap is not None
        self.gather_rows = (compacted or not dw) if gather_rows is None else bool(gather_rows)
        self.x_sorted = None if self.gather_rows else em(N, H)
        self.h_save = em(N, 2 * F)
        self.a_save = em(N, F)
        self.o_sorted = em(N, H)
        self.y = em(T, H)
        self.quota_cap = quota_cap
        self.compacted = rho is not None or quota_cap is not None
        if self.compacted:
            cap = moe.moe_quota_cap(T, E, k, rho) if quota_cap is None else quota_cap
            self.R = min(N, E * cap)
            self.kept_counts = em(E, dt=i32)
            self.kept_offsets = em(E + 1, dt=i32)
            self.kept_perm = em(self.R, dt=i32)
            self.kept_src = em(self.R, dt=i32)
            self.kept_inv = em(N, dt=i32)
            g = self.gather_rows
            self.x_kept = None if g else em(self.R, H)
            self.a_kept = None if g or not dw else em(self.R, F)
            # pre-activations of the kept rows: recomputed into it, or (materialized) gathered
            self.h_kept = em(self.R, 2 * F) if (not keep_graph or not g) else None
            self.score = em(N, dt=f32)
        else:
            self.R = N
        R = self.R
        self.dO = em(R, H)
        self.dh = em(R, 2 * F)
        self.dX = em(R, H)
        self.dx = em(T, H)
        self.dg = em(T, k, dt=f32) if dg else None
        if dw:
            self.dw_gate = em(E, H, F)
            self.dw_up = em(E, H, F)
            self.dw_down = em(E, F, H)
        self.router = router
        if router:  # logits = x W_r in front of routing; its backward needs dg
            assert dg, "the router backward needs dg"
            self.logits = em(T, E, dt=f32)
            self.dlogits = em(T, E, dt=f32)
            self.dw_r = em(H, E)
            self.router_ws = em(max(moe.moe_router_workspace_bytes(T, H, E), 16), dt=torch.uint8)

    # ------------------------------------------------------------------ forward
    def forward(self, logits, x, w_gate, w_up, w_down, stream=None, w_r=None, wq=None, wt=None):
        """With w_r (a layer built with router=True) the logits are x W_r and
        the `logits` argument is ignored.  With wq (moe.Fp8Weights of the same
        frozen weights) the expert GEMMs read the fp8 copy.  With wt
        (moe.Fp8KMajorWeights) both expert GEMMs run on the fp8 matrix cores:
        the token rows are quantized per row, then gathered on load."""
        self._x = x  # the backward reads token rows through the pair ids
        if w_r is not None:
            moe.moe_router_fwd(x, w_r, self.logits, self.router_ws, stream)
            logits = self.logits
        moe.moe_route_topk(logits, self.topk_idx, self.topk_w, self.k, stream)
        g = self.gather_rows or wt is not None  # index-only dispatch: the forward gathers x rows itself
        moe.moe_dispatch(self.topk_idx, None if g else x, self.counts, self.offsets, self.perm, self.inv_perm,
                         None if g else self.x_sorted, self.ws, self.E, stream)
        if wt is not None:
            if not hasattr(self, "xq"):
                dev, u8, f32 = self.device, torch.uint8, torch.float32
                self.xq = torch.empty(self.T, self.H, dtype=u8, device=dev)
                self.x_scale = torch.empty(self.T, dtype=f32, device=dev)
                self.aq = torch.empty(self.N, self.F, dtype=u8, device=dev)
                self.a_scale = torch.empty(self.N, dtype=f32, device=dev)
            moe.moe_quantize_rows_fp8(x, self.xq, self.x_scale, stream)
            moe.moe_grouped_swiglu_fwd_fp8(self.offsets, self.xq, self.x_scale, wt,
                                           self.h_save if self.keep_graph else None, self.a_save, self.aq,
                                           self.a_scale, self.o_sorted, self.N, perm=self.perm, k=self.k,
                                           stream=stream)
        elif wq is not None:
            assert self.keep_graph, "the fp8 path keeps the pre-activations"
            moe.moe_grouped_swiglu_fwd_fp8w(self.offsets, x if g else self.x_sorted, wq, self.h_save, self.a_save,
                                            self.o_sorted, self.N, perm=self.perm if g else None, k=self.k,
                                            stream=stream)
        elif self.gather_rows:
            moe.moe_grouped_swiglu_fwd_gather(self.offsets, x, self.perm, w_gate, w_up, w_down,
                                              self.h_save if self.keep_graph else None, self.a_save, self.o_sorted,
                                              self.k, self.N, max_expert_rows=self.T, stream=stream)
        else:
            moe.moe_grouped_swiglu_fwd(self.offsets, self.x_sorted, w_gate, w_up, w_down,
                                       self.h_save if self.keep_graph else None, self.a_save, self.o_sorted, self.N,
                                       max_expert_rows=self.T, stream=stream)
        moe.moe_combine(self.o_sorted, self.inv_perm, self.topk_w, self.y, self.k, stream)
        return self.y

    # ----------------------------------------------------------------- backward
    def compact(self, score, stream=None):
        """Selection within the quotas; index-only when rows are gathered on load."""
        kg, g = self.keep_graph, self.gather_rows
        moe.moe_compact_pairs(self.counts, self.offsets, self.perm, score, self.rho or 1.0, self.kept_counts,
                              self.kept_offsets, self.kept_perm, self.kept_src, self.kept_inv, self.T, self.k,
                              None if g else self.x_sorted, None if g or not self.dw else self.a_save,
                              None if g or not kg else self.h_save, None if g else self.x_kept,
                              None if g or not self.dw else self.a_kept, None if g or not kg else self.h_kept, stream,
                              cap=self.quota_cap)

    def backward(self, dy, w_gate, w_up, w_down, score=None, stream=None, w_r=None, wq=None):
        """dx (+ dg) and, for full fine-tuning, dW.  With a quota the backward
        runs on the compacted retained pairs; score: a pair-indexed fp32 tensor,
        None (the routing weights) or "metric" (moe_pair_scores: the norm of
        each pair's rank-one dW_down term).  With w_r, the router's backward
        follows: dlogits, dw_r, and its share added to dx."""
        g, k = self.gather_rows, self.k
        if self.compacted:
            if isinstance(score, str):
                assert score == "metric", score
                moe.moe_pair_scores(self.inv_perm, self.topk_w, self.a_save, dy, self.score, stream)
                score = self.score
            self.compact(self.topk_w.view(-1) if score is None else score, stream)
            offsets, inv, pairs, src = self.kept_offsets, self.kept_inv, self.kept_perm, self.kept_src
        else:
            offsets, inv, pairs, src = self.offsets, self.inv_perm, self.perm, None
        # rows of the backward: x, a and the pre-activations h, each either a
        # contiguous buffer or a source buffer read through a row map
        if g:
            x_rows, x_src, a_rows, a_src = self._x, pairs, self.a_save, src
        else:
            x_rows, x_src = (self.x_kept if self.compacted else self.x_sorted), None
            a_rows, a_src = (self.a_kept if self.compacted else self.a_save), None
        if not self.keep_graph:  # recompute [hg | hu] of the backward's rows
            h_rows, h_src = (self.h_kept if self.compacted else self.h_save), None
            moe.moe_grouped_swiglu_recompute(offsets, x_rows, w_gate, w_up, h_rows, None, self.R,
                                             max_expert_rows=self.T, stream=stream, x_src=x_src, x_div=k)
        elif self.compacted and not g:
            h_rows, h_src = self.h_kept, None
        else:
            h_rows, h_src = self.h_save, src
        extra = dict(inv_all=self.inv_perm if self.want_dg else None, o_sorted=self.o_sorted if self.want_dg else None,
                     dg=self.dg, stream=stream, h_src=h_src)
        if self.dw and self.overlap_dw:
            moe.moe_signal_dh_ready(self._dh_ready)
        if wq is not None:  # frozen fp8 weights: no weight gradient
            assert not self.dw, "fp8 weights are frozen: no dW"
            moe.moe_grouped_bwd_dx_fp8w(offsets, inv, dy, self.topk_w, h_rows, wq, self.dO, self.dh, self.dX,
                                        self.dx, self.R, **extra)
        else:
            moe.moe_grouped_bwd_dx(offsets, inv, dy, self.topk_w, h_rows, w_gate, w_up, w_down, self.dO, self.dh,
                                   self.dX, self.dx, self.R, **extra)
        if self.dw:
            # dW reads dO and dh only: on the side stream it runs alongside dX
            # and the dx sum, from the moment the dx call signals them complete
            s_main = stream if stream is not None else torch.cuda.current_stream(self.device)
            s_dw = self._dw_stream if self.overlap_dw else s_main
            if self.overlap_dw:
                s_dw.wait_event(self._dh_ready)
            moe.moe_grouped_bwd_dw(offsets, x_rows, a_rows, self.dO, self.dh, self.dw_gate, self.dw_up,
                                   self.dw_down, self.R, s_dw, x_src=x_src, x_div=k, a_src=a_src)
            if self.overlap_dw:
                s_main.wait_stream(s_dw)
        if w_r is not None:
            moe.moe_router_bwd(self._x, w_r, self.topk_idx, self.topk_w, self.dg, self.dlogits, self.dw_r, self.dx,
                               True, self.router_ws, stream)
        return self.dx
