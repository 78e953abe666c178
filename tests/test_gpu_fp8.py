"""GPU parity of the fp8 (OCP E4M3) frozen-weight path against the CPU oracle.

Bit-exact: the fp8 codes and per-expert scales written by
moe_quantize_weights_fp8 against the oracle's quantization of the same bf16
weights.  Within the bf16 tolerance (max|err|/max|ref| <= 1e-2): y, dx, dg and
the saved intermediates of a LoRA step (forward + dx) whose GEMMs read the fp8
copy, against the oracle run on the decoded weights decode(code) * scale --
the values the kernels multiply, exactly (an E4M3 value is exact in bf16 and
the scales are powers of two).
"""
import numpy as np
import pytest
import torch

import oracle
from expert_grouped_gemm_top_amd import moe
from expert_grouped_gemm_top_amd import workloads as W
from expert_grouped_gemm_top_amd.layer import MoeLayerBuffers
from moe_cases import assert_close, logits_of, note, np32, oracle_tokens, to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _oracle_fp8(d):
    """The oracle's fp8 storage of the bf16 weights, and the decoded weights."""
    qg, qu, sgu = oracle.quantize_fp8(d["W_gate"], d["W_up"])
    qd, _, sd = oracle.quantize_fp8(d["W_down"])
    dec = dict(d)
    dec["W_gate"] = oracle.dequantize_fp8(qg, sgu)
    dec["W_up"] = oracle.dequantize_fp8(qu, sgu)
    dec["W_down"] = oracle.dequantize_fp8(qd, sd)
    return (qg, qu, qd, sgu, sd), dec


def _check_codes(wq, ref):
    qg, qu, qd, sgu, sd = ref
    for name, got, want in (("q_gate", wq.q_gate, qg), ("q_up", wq.q_up, qu), ("q_down", wq.q_down, qd)):
        g = got.cpu().numpy()
        if not np.array_equal(g, want):
            bad = np.argwhere(g != want)[:5]
            raise AssertionError(f"{name}: {len(np.argwhere(g != want))} codes differ, e.g. at {bad.tolist()}")
    assert np.array_equal(wq.s_gu.cpu().numpy(), sgu.astype(np.float32)), "s_gu"
    assert np.array_equal(wq.s_down.cpu().numpy(), sd.astype(np.float32)), "s_down"


def test_quantize_special_values():
    """Zeros, negative zero, exact grid values, ties between grid values, a
    subnormal range and experts whose scale differs by many binades."""
    E, H, F = 6, 128, 64
    rng = np.random.default_rng(11)
    w = (0.02 * rng.standard_normal((E, H, F))).astype(np.float32)
    w[0] = 0.0                                           # an all-zero expert: scale 1, codes 0
    w[1].flat[:8] = [-0.0, 448.0, -448.0, 1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 15 * 2.0 ** -10]
    w[2] *= 2.0 ** 12                                    # a large scale
    w[3] *= 2.0 ** -30                                   # a tiny one
    w[4].flat[::7] = 0.0
    w = W.round_bf16(w)
    u = (0.03 * rng.standard_normal((E, H, F))).astype(np.float32)
    u[0] = 0.0
    u = W.round_bf16(u)
    ref = oracle.quantize_fp8(w, u)
    tw, tu = (torch.from_numpy(a).cuda().bfloat16() for a in (w, u))
    q0 = torch.empty(E, H, F, dtype=torch.uint8, device="cuda")
    q1 = torch.empty_like(q0)
    s = torch.empty(E, dtype=torch.float32, device="cuda")
    moe.moe_quantize_weights_fp8(tw, tu, q0, q1, s)
    torch.cuda.synchronize()
    assert np.array_equal(q0.cpu().numpy(), ref[0]) and np.array_equal(q1.cpu().numpy(), ref[1])
    assert np.array_equal(s.cpu().numpy(), ref[2].astype(np.float32))
    assert ref[2][0] == 1.0 and not ref[0][0].any()


def _run_fp8_layer(wl, d, gather):
    t = to_dev(wl, d)
    wq = moe.Fp8Weights(t["W_gate"], t["W_up"], t["W_down"])
    L = MoeLayerBuffers(wl.T, wl.H, wl.F, wl.E, wl.k, torch.bfloat16, "cuda", dw=False, dg=True,
                        gather_rows=gather)
    L.forward(torch.from_numpy(np.ascontiguousarray(logits_of(wl, d))).cuda(), t["x"], None, None, None, wq=wq)
    L.backward(t["dy"], None, None, None, wq=wq)
    torch.cuda.synchronize()
    return L, wq


SMALL = [
    W.custom("fp8_skew_e8", T=160, H=256, F=128, E=8, k=2, dtype="bf16", skew=True, dw=False),   # experts of 48+ rows too
    W.custom("fp8_e16_k4", T=96, H=384, F=256, E=16, k=4, dtype="bf16", skew=True, dw=False),
    W.custom("fp8_single_token", T=1, H=128, F=128, E=4, k=4, dtype="bf16", skew=False, dw=False),
    W.custom("fp8_big_expert", T=400, H=256, F=128, E=2, k=1, dtype="bf16", skew=True, dw=False),
    # widths that are multiples of 8 but not of the kernels' column blocks:
    # partial column blocks and reduction tails with fp8 weights
    W.custom("fp8_h200_f136", T=300, H=200, F=136, E=8, k=2, dtype="bf16", skew=True, dw=False),
    W.custom("fp8_h136_f200", T=160, H=136, F=200, E=16, k=4, dtype="bf16", skew=True, dw=False),
    # fewer features than one gate/up column block of 128 (one partial block)
    W.custom("fp8_h64_f40", T=120, H=64, F=40, E=4, k=2, dtype="bf16", skew=True, dw=False),
    W.custom("fp8_h104_f72", T=200, H=104, F=72, E=8, k=2, dtype="bf16", skew=True, dw=False),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("gather", [False, True])
def test_fp8_lora_step_matches_oracle(wl, gather):
    d = W.generate(wl, seed=4)
    note(f"fp8 layer {wl.name} gather={gather}")
    ref_q, dec = _oracle_fp8(d)
    L, wq = _run_fp8_layer(wl, d, gather)
    _check_codes(wq, ref_q)
    idx, w = oracle.route_topk(logits_of(wl, d), wl.k)
    counts, offsets, perm, inv = oracle.dispatch(idx, wl.E)
    assert np.array_equal(L.topk_idx.cpu().numpy(), idx)
    y, it = oracle.forward(dec["x"], idx, w, dec["W_gate"], dec["W_up"], dec["W_down"], intermediates=True)
    dx, dg = oracle.backward(dec["x"], idx, w, dec["W_gate"], dec["W_up"], dec["W_down"], dec["dy"])
    assert_close("h_save", np32(L.h_save), np.concatenate([it["hg"], it["hu"]], 1)[perm], TOL)
    assert_close("a_save", np32(L.a_save), it["a"][perm], TOL)
    assert_close("y", np32(L.y), y, TOL)
    assert_close("dx", np32(L.dx), dx, TOL)
    assert_close("dg", L.dg.cpu().numpy(), dg, TOL)


def test_fp8_full_size_lora_step():
    """The Qwen3-30B-A3B LoRA shape at 128 tokens (the weight-streaming case)
    with the frozen weights in fp8: all codes bit-exact, sampled tokens within
    tolerance."""
    wl = W.WORKLOADS["qwen3_lora_t128"]
    d = W.generate(wl, seed=0)
    note("fp8 full size: oracle quantization")
    ref_q, dec = _oracle_fp8(d)
    L, wq = _run_fp8_layer(wl, d, gather=True)
    _check_codes(wq, ref_q)
    idx, w = oracle.route_topk(logits_of(wl, d), wl.k)
    tokens = np.array([0, 1, 37, 64, 90, wl.T - 1], np.int32)
    note(f"oracle on {len(tokens)} sampled tokens")
    y, dx, dg, _, _ = oracle_tokens(wl, dec, idx, w, tokens)
    tt = torch.from_numpy(tokens).long().cuda()
    assert_close("y", np32(L.y[tt]), y[tokens], TOL)
    assert_close("dx", np32(L.dx[tt]), dx[tokens], TOL)
    assert_close("dg", L.dg[tt].cpu().numpy(), dg[tokens], TOL)
