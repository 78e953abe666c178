"""CPU oracle for one MoE layer's expert computation -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  It wraps ``moe_oracle.c`` (plain C, IEEE double, built
with gcc) through ctypes and shares no code with the HIP library.

Every function takes numpy arrays of any float dtype (fp32, bf16 values held in
fp32, or fp64); they are upcast exactly to float64 before the C code sees them.
Pair ids are ``p = t*k + j``.  Citations of the pages are in ``moe_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE-exact flags, OpenMP).  Returns the path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = ctypes.CDLL(_LIB)
        _lib.oracle_quota_cap.restype = ctypes.c_int64
        _lib.oracle_quota_cap_for_budget.restype = ctypes.c_int64
        _lib.oracle_quota_cap_for_budget.argtypes = [ctypes.c_int] * 8 + [ctypes.c_double]
        _lib.oracle_compact.restype = ctypes.c_int64
        _lib.oracle_dispatch.restype = ctypes.c_int
        _lib.oracle_num_threads.restype = ctypes.c_int
        _lib.oracle_e4m3_decode.restype = ctypes.c_double
        _lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        _lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        _lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        _lib.oracle_fp8_scale_exp.restype = ctypes.c_int
        _lib.oracle_fp8_scale_exp.argtypes = [ctypes.c_double]
        _lib.oracle_quantize_fp8.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def router_logits(x, Wr):
    """l[t,e] = sum_h x[t,h] Wr[h,e] in double."""
    x, Wr = _f64(x), _f64(Wr)
    T, H = x.shape
    E = Wr.shape[1]
    out = np.empty((T, E), np.float64)
    _load().oracle_router_logits(T, H, E, _p(x), _p(Wr), _p(out))
    return out


def router_backward(x, Wr, idx, w, dg):
    """Router backward with the selection fixed: dlogits [T,E], dWr [H,E] and
    the router's share of dx [T,H], from dg = dL/dw [T,k]."""
    x, Wr, w, dg = _f64(x), _f64(Wr), _f64(w), _f64(dg)
    idx = _i32(idx)
    T, H = x.shape
    E = Wr.shape[1]
    k = idx.shape[1]
    dl = np.empty((T, E), np.float64)
    dWr = np.empty((H, E), np.float64)
    dxr = np.empty((T, H), np.float64)
    _load().oracle_router_backward(T, H, E, k, _p(x), _p(Wr), _p(idx), _p(w), _p(dg), _p(dl), _p(dWr), _p(dxr))
    return dl, dWr, dxr


def route_topk(logits, k):
    """Top-k by (logit desc, index asc); softmax over the selected logits."""
    logits = _f64(logits)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _load().oracle_route_topk(T, E, k, _p(logits), _p(idx), _p(w))
    return idx, w


def dispatch(idx, E):
    """Stable per-expert grouping of pairs: counts, offsets, perm, inv_perm."""
    idx = _i32(idx)
    T, k = idx.shape
    N = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(N, np.int32)
    inv = np.empty(N, np.int32)
    rc = _load().oracle_dispatch(T, E, k, _p(idx), _p(counts), _p(offsets), _p(perm), _p(inv))
    if rc != 0:
        raise ValueError("expert index out of range")
    return counts, offsets, perm, inv


def quota_cap(T, E, k, rho):
    return int(_load().oracle_quota_cap(T, E, k, ctypes.c_double(rho)))


def pair_scores(a_pairs, dy, w):
    """score[p] = w[p] * ||a_p|| * ||dy_t||: the Frobenius norm of pair p's
    rank-one term in dW_down.  a_pairs [N, F] pair-indexed, dy [T, H], w [T, k]."""
    a_pairs, dy, w = _f64(a_pairs), _f64(dy), _f64(w)
    T, H = dy.shape
    k = w.shape[1]
    F = a_pairs.shape[1]
    out = np.empty(T * k, np.float64)
    _load().oracle_pair_scores(T, H, F, k, _p(a_pairs), _p(dy), _p(w), _p(out))
    return out


def quota_cap_for_budget(T, H, F, E, k, elem_bytes, with_dw, keep_graph, budget_bytes):
    return int(_load().oracle_quota_cap_for_budget(T, H, F, E, k, elem_bytes, int(bool(with_dw)),
                                                   int(bool(keep_graph)), float(budget_bytes)))


def compact(T, E, k, counts, offsets, perm, score, rho):
    """Per-expert top-q_e selection by (score desc, p asc) and compaction."""
    counts, offsets, perm = _i32(counts), _i32(offsets), _i32(perm)
    score = _f64(score).reshape(-1)
    N = T * k
    kc = np.empty(E, np.int32)
    ko = np.empty(E + 1, np.int32)
    kperm = np.empty(N, np.int32)
    ksrc = np.empty(N, np.int32)
    kinv = np.empty(N, np.int32)
    ret = np.empty(N, np.uint8)
    R = _load().oracle_compact(T, E, k, _p(counts), _p(offsets), _p(perm), _p(score),
                               ctypes.c_double(rho), _p(kc), _p(ko), _p(kperm), _p(ksrc),
                               _p(kinv), _p(ret))
    return dict(counts=kc, offsets=ko, perm=kperm[:R].copy(), src=ksrc[:R].copy(), inv=kinv,
                retained=ret, R=int(R))


def _tok_args(tokens):
    if tokens is None:
        return 0, None, None
    toks = _i32(tokens).reshape(-1)
    return len(toks), toks, _p(toks)


def forward(x, idx, w, Wg, Wu, Wd, tokens=None, intermediates=False):
    """y[t] = sum_j w[t,j] * SwiGLU_{idx[t,j]}(x[t]).

    With ``tokens`` only those rows of y (and those pairs' intermediates) are
    computed; the other rows are zero.  With ``intermediates`` also returns the
    pair-indexed hg, hu, a [N,F] and o [N,H]."""
    x, w, Wg, Wu, Wd = _f64(x), _f64(w), _f64(Wg), _f64(Wu), _f64(Wd)
    idx = _i32(idx)
    T, H = x.shape
    E, _, F = Wg.shape
    k = idx.shape[1]
    N = T * k
    y = np.zeros((T, H), np.float64)
    hg = hu = a = o = None
    if intermediates:
        hg = np.zeros((N, F)); hu = np.zeros((N, F)); a = np.zeros((N, F)); o = np.zeros((N, H))
    nt, _toks, tp = _tok_args(tokens)
    _load().oracle_forward(T, H, F, E, k, _p(x), _p(idx), _p(w), _p(Wg), _p(Wu), _p(Wd), nt, tp,
                           _p(y), _p(hg), _p(hu), _p(a), _p(o))
    if intermediates:
        return y, dict(hg=hg, hu=hu, a=a, o=o)
    return y


def backward(x, idx, w, Wg, Wu, Wd, dy, retained=None, tokens=None, intermediates=False):
    """dx (sum over retained pairs) and dg (every pair) for the given tokens.

    With ``intermediates`` also returns pair-indexed dO [N,H], dh [N,2F] =
    [dHg | dHu] and dX [N,H] (zero rows for dropped or uncomputed pairs)."""
    x, w, Wg, Wu, Wd, dy = _f64(x), _f64(w), _f64(Wg), _f64(Wu), _f64(Wd), _f64(dy)
    idx = _i32(idx)
    T, H = x.shape
    E, _, F = Wg.shape
    k = idx.shape[1]
    N = T * k
    ret = None if retained is None else np.ascontiguousarray(np.asarray(retained, np.uint8))
    dx = np.zeros((T, H))
    dg = np.zeros((T, k))
    dO = dh = dX = None
    if intermediates:
        dO = np.zeros((N, H)); dh = np.zeros((N, 2 * F)); dX = np.zeros((N, H))
    nt, _toks, tp = _tok_args(tokens)
    _load().oracle_backward(T, H, F, E, k, _p(x), _p(idx), _p(w), _p(Wg), _p(Wu), _p(Wd), _p(dy),
                            _p(ret), nt, tp, _p(dx), _p(dg), _p(dO), _p(dh), _p(dX))
    if intermediates:
        return dx, dg, dict(dO=dO, dh=dh, dX=dX)
    return dx, dg


def backward_dw(x, idx, w, Wg, Wu, Wd, dy, retained=None):
    """Full dW_gate, dW_up [E,H,F] and dW_down [E,F,H] over retained pairs."""
    x, w, Wg, Wu, Wd, dy = _f64(x), _f64(w), _f64(Wg), _f64(Wu), _f64(Wd), _f64(dy)
    idx = _i32(idx)
    T, H = x.shape
    E, _, F = Wg.shape
    k = idx.shape[1]
    ret = None if retained is None else np.ascontiguousarray(np.asarray(retained, np.uint8))
    dWg = np.empty((E, H, F)); dWu = np.empty((E, H, F)); dWd = np.empty((E, F, H))
    _load().oracle_backward_dw(T, H, F, E, k, _p(x), _p(idx), _p(w), _p(Wg), _p(Wu), _p(Wd),
                               _p(dy), _p(ret), _p(dWg), _p(dWu), _p(dWd))
    return dWg, dWu, dWd


def dw_entries(x, idx, w, Wg, Wu, Wd, dy, q_e, q_mat, q_r, q_c, retained=None):
    """Single weight-gradient entries; q_mat 0/1/2 = gate[e,h,f] / up[e,h,f] / down[e,f,h]."""
    x, w, Wg, Wu, Wd, dy = _f64(x), _f64(w), _f64(Wg), _f64(Wu), _f64(Wd), _f64(dy)
    idx = _i32(idx)
    T, H = x.shape
    E, _, F = Wg.shape
    k = idx.shape[1]
    ret = None if retained is None else np.ascontiguousarray(np.asarray(retained, np.uint8))
    q_e, q_mat, q_r, q_c = _i32(q_e), _i32(q_mat), _i32(q_r), _i32(q_c)
    out = np.empty(len(q_e))
    _load().oracle_dw_entries(T, H, F, E, k, _p(x), _p(idx), _p(w), _p(Wg), _p(Wu), _p(Wd), _p(dy),
                              _p(ret), len(q_e), _p(q_e), _p(q_mat), _p(q_r), _p(q_c), _p(out))
    return out


def e4m3_decode(codes):
    """Values of OCP E4M3 codes (uint8 array) as float64."""
    c = np.asarray(codes, dtype=np.uint8)
    L = _load()
    return np.array([L.oracle_e4m3_decode(int(v)) for v in c.reshape(-1)], dtype=np.float64).reshape(c.shape)


def e4m3_encode(values):
    """OCP E4M3 codes of float64 values (round to nearest even, saturating)."""
    v = _f64(values)
    L = _load()
    return np.array([L.oracle_e4m3_encode(float(x)) for x in v.reshape(-1)], dtype=np.uint8).reshape(v.shape)


def fp8_scale_exp(amax: float) -> int:
    """log2 of the smallest power-of-two scale s with amax <= 448 s."""
    return int(_load().oracle_fp8_scale_exp(float(amax)))


def quantize_fp8(w0, w1=None):
    """Per-expert fp8 storage of w0 [E, ...] (and w1 of the same E, sharing the
    scale): returns (q0, q1 or None, scale [E])."""
    a0 = _f64(w0)
    E = a0.shape[0]
    n0 = a0.size // E
    a1 = None if w1 is None else _f64(w1)
    n1 = 0 if a1 is None else a1.size // E
    q0 = np.empty(a0.shape, np.uint8)
    q1 = None if a1 is None else np.empty(a1.shape, np.uint8)
    scale = np.empty(E, np.float64)
    _load().oracle_quantize_fp8(E, n0, _p(a0), n1, _p(a1), _p(q0), _p(q1), _p(scale))
    return q0, q1, scale


def dequantize_fp8(q, scale):
    """w = E4M3 value x scale[e] (exact in float64)."""
    table = e4m3_decode(np.arange(256, dtype=np.uint8))
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(scale, dtype=np.float64).reshape((-1,) + (1,) * (q.ndim - 1))
    return table[q] * s


def quantize_rows_fp8(x):
    """Per-row fp8 storage of activations x [rows, n]: codes [rows, n] and one
    power-of-two scale per row (the rule of quantize_fp8, rows as experts)."""
    q, _, scale = quantize_fp8(x)
    return q, scale


def forward_fp8(x, idx, w, Wg, Wu, Wd):
    """The expert forward on E4M3 operands (oracle_forward_fp8): x quantized
    per token row, the weights per expert (W_gate and W_up sharing a scale),
    the SwiGLU output rounded to bf16 and quantized per pair row before the
    down product.  Returns y [T,H] and a dict of the pair-indexed hg, hu, a
    (bf16-rounded), aq codes, ascale, o, and the x codes / scales."""
    x = _f64(x)
    T, H = x.shape
    Wg, Wu, Wd = _f64(Wg), _f64(Wu), _f64(Wd)
    E, _, F = Wg.shape
    idx = _i32(idx)
    k = idx.shape[1]
    N = T * k
    w = _f64(w)
    qx, sx = quantize_rows_fp8(x)
    qg, qu, sgu = quantize_fp8(Wg, Wu)
    qd, _, sd = quantize_fp8(Wd)
    xd = np.ascontiguousarray(dequantize_fp8(qx, sx))
    Wgd = np.ascontiguousarray(dequantize_fp8(qg, sgu))
    Wud = np.ascontiguousarray(dequantize_fp8(qu, sgu))
    Wdd = np.ascontiguousarray(dequantize_fp8(qd, sd))
    y = np.zeros((T, H))
    hg = np.zeros((N, F)); hu = np.zeros((N, F)); a = np.zeros((N, F)); o = np.zeros((N, H))
    aq = np.zeros((N, F), np.uint8)
    ascale = np.zeros(N)
    _load().oracle_forward_fp8(T, H, F, E, k, _p(xd), _p(idx), _p(w), _p(Wgd), _p(Wud), _p(Wdd), _p(y), _p(hg), _p(hu),
                               _p(a), _p(aq), _p(ascale), _p(o))
    return y, dict(hg=hg, hu=hu, a=a, aq=aq, ascale=ascale, o=o, qx=qx, sx=sx)

