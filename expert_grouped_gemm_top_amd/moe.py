"""Thin ctypes binding of libmoe (C ABI in include/moe.h), one function per
entry point with the same name.

Arguments are torch tensors on the GPU (device memory only -- torch is used for
allocation and streams, never for the computation).  Each wrapper checks device,
dtype, contiguity and sizes before handing raw pointers to the library, so a
wrong tensor raises here instead of reaching a kernel.  Every call enqueues on
``stream`` (default: torch's current stream) and returns without synchronising.
The library is loaded on first use; if it has not been built the call fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
_STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED",
           3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP"}

_lib = None
_vp, _i, _sz, _d, _i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_double, ctypes.c_int64

_SIGS = {
    "moe_status_string": ([_i], ctypes.c_char_p),
    "moe_last_error": ([], ctypes.c_char_p),
    "moe_abi_version": ([], _i),
    "moe_launch_count": ([], _i64),
    "moe_signal_dh_ready": ([_vp], _i),
    "moe_router_workspace_bytes": ([_i, _i, _i], _sz),
    "moe_router_fwd": ([_i, _i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp], _i),
    "moe_route_topk": ([_i, _i, _i, _vp, _vp, _vp, _vp], _i),
    "moe_router_bwd": ([_i, _i, _i, _i, _i] + [_vp] * 8 + [_i, _vp, _sz, _vp], _i),
    "moe_dispatch_workspace_bytes": ([_i, _i, _i], _sz),
    "moe_dispatch": ([_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i),
    "moe_dispatch_noalloc": ([_i, _i, _i, _i, _i] + [_vp] * 8, _i),
    "moe_dispatch_noalloc_max_workspace": ([], _sz),
    "moe_grouped_swiglu_fwd": ([_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp], _i),
    "moe_grouped_swiglu_fwd_gather": ([_i] * 7 + [_vp] * 10, _i),
    "moe_grouped_swiglu_recompute": ([_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _i] + [_vp] * 5, _i),
    "moe_combine": ([_i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp], _i),
    "moe_grouped_bwd_dx": ([_i, _i, _i, _i, _i, _i, _i] + [_vp] * 17, _i),
    "moe_grouped_bwd_dw": ([_i, _i, _i, _i, _i, _vp, _vp, _vp, _i] + [_vp] * 8, _i),
    "moe_quota_cap": ([_i, _i, _i, _d], _i64),
    "moe_compact_pairs": ([_i, _i, _i, _i, _i, _i, _d] + [_vp] * 16, _i),
    "moe_compact_pairs_cap": ([_i, _i, _i, _i, _i, _i, _i] + [_vp] * 16, _i),
    "moe_quota_cap_for_budget": ([_i, _i, _i, _i, _i, _i, _i, _i, _sz], _i64),
    "moe_pair_scores": ([_i, _i, _i, _i, _i] + [_vp] * 6, _i),
    "moe_quantize_weights_fp8": ([_i, _i64, _i64] + [_vp] * 6, _i),
    "moe_grouped_swiglu_fwd_fp8w": ([_i] * 5 + [_vp] * 12, _i),
    "moe_grouped_bwd_dx_fp8w": ([_i] * 6 + [_vp] * 19, _i),
    "moe_quantize_rows_fp8": ([_i, _i, _vp, _vp, _vp, _vp], _i),
    "moe_transpose_fp8": ([_i, _i, _i, _vp, _vp, _vp], _i),
    "moe_grouped_swiglu_fwd_fp8": ([_i] * 5 + [_vp] * 15, _i),
}


class MoeError(RuntimeError):
    pass


def lib():
    """Load libmoe.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        L = lib()
        raise MoeError(f"{L.moe_status_string(rc).decode()}: {L.moe_last_error().decode()}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dt(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return MOE_F32
    if x.dtype == torch.bfloat16:
        return MOE_BF16
    raise MoeError(f"unsupported dtype {x.dtype}")


def _ptr(t, name, dtype=None, numel=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise MoeError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise MoeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise MoeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise MoeError(f"{name} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


I32, F32 = torch.int32, torch.float32


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_launch_count() -> int:
    """Kernel launches made so far by library calls from this thread."""
    return int(lib().moe_launch_count())


def moe_dispatch_workspace_bytes(T: int, E: int, k: int) -> int:
    return int(lib().moe_dispatch_workspace_bytes(T, E, k))


def moe_quota_cap(T: int, E: int, k: int, rho: float) -> int:
    return int(lib().moe_quota_cap(T, E, k, float(rho)))


def moe_router_workspace_bytes(T: int, H: int, E: int) -> int:
    return int(lib().moe_router_workspace_bytes(T, H, E))


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()


def moe_router_fwd(x, w_r, logits, workspace=None, stream=None):
    T, H = x.shape
    E = w_r.shape[1]
    d = x.dtype
    ws, ws_bytes = _ws(workspace)
    _check(lib().moe_router_fwd(T, H, E, _dt(x), _ptr(x, "x", d, T * H), _ptr(w_r, "w_r", d, H * E),
                                _ptr(logits, "logits", F32, T * E), ws, ws_bytes, _stream(stream)))


def moe_router_bwd(x, w_r, topk_idx, topk_w, dg, dlogits, dw_r, dx, accumulate: bool, workspace=None, stream=None):
    T, H = x.shape
    E = w_r.shape[1]
    k = topk_idx.shape[1]
    d = x.dtype
    ws, ws_bytes = _ws(workspace)
    _check(lib().moe_router_bwd(T, H, E, k, _dt(x), _ptr(x, "x", d, T * H), _ptr(w_r, "w_r", d, H * E),
                                _ptr(topk_idx, "topk_idx", I32, T * k), _ptr(topk_w, "topk_w", F32, T * k),
                                _ptr(dg, "dg", F32, T * k), _ptr(dlogits, "dlogits", F32, T * E),
                                _ptr(dw_r, "dw_r", d, H * E), _ptr(dx, "dx", d, T * H), 1 if accumulate else 0,
                                ws, ws_bytes, _stream(stream)))


def moe_route_topk(logits, topk_idx, topk_w, k: int, stream=None):
    T, E = logits.shape
    _check(lib().moe_route_topk(T, E, k, _ptr(logits, "logits", F32, T * E),
                                _ptr(topk_idx, "topk_idx", I32, T * k), _ptr(topk_w, "topk_w", F32, T * k),
                                _stream(stream)))


def moe_dispatch(topk_idx, x, counts, offsets, perm, inv_perm, x_sorted, workspace, E: int, stream=None):
    T, k = topk_idx.shape
    H = x.shape[1] if x is not None else 8
    dt = _dt(x) if x is not None else MOE_BF16
    N = T * k
    ws_need = moe_dispatch_workspace_bytes(T, E, k)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moe_dispatch(T, H, E, k, dt, _ptr(topk_idx, "topk_idx", I32, N),
                              _ptr(x, "x", None, T * H, allow_none=True), _ptr(counts, "counts", I32, E),
                              _ptr(offsets, "offsets", I32, E + 1), _ptr(perm, "perm", I32, N),
                              _ptr(inv_perm, "inv_perm", I32, N),
                              _ptr(x_sorted, "x_sorted", x.dtype if x is not None else None, N * H, allow_none=True),
                              _ptr(workspace, "workspace", None, None, allow_none=ws_need == 0), ws_bytes,
                              _stream(stream)))


def moe_dispatch_noalloc(topk_idx, x, counts, offsets, perm, inv_perm, x_sorted, E: int, stream=None):
    """moe_dispatch with the library-held workspace (no allocation anywhere)."""
    T, k = topk_idx.shape
    H = x.shape[1] if x is not None else 8
    dt = _dt(x) if x is not None else MOE_BF16
    N = T * k
    _check(lib().moe_dispatch_noalloc(T, H, E, k, dt, _ptr(topk_idx, "topk_idx", I32, N),
                                      _ptr(x, "x", None, T * H, allow_none=True), _ptr(counts, "counts", I32, E),
                                      _ptr(offsets, "offsets", I32, E + 1), _ptr(perm, "perm", I32, N),
                                      _ptr(inv_perm, "inv_perm", I32, N),
                                      _ptr(x_sorted, "x_sorted", x.dtype if x is not None else None, N * H,
                                           allow_none=True),
                                      _stream(stream)))


def moe_dispatch_noalloc_max_workspace() -> int:
    return int(lib().moe_dispatch_noalloc_max_workspace())


def moe_grouped_swiglu_fwd(offsets, x_sorted, w_gate, w_up, w_down, h_save, a_save, o_sorted, max_rows: int,
                           max_expert_rows: int | None = None, stream=None):
    E, H, F = w_gate.shape
    dt, d = _dt(w_gate), w_gate.dtype
    R = max_rows
    _check(lib().moe_grouped_swiglu_fwd(
        H, F, E, R, R if max_expert_rows is None else max_expert_rows, dt, _ptr(offsets, "offsets", I32, E + 1), _ptr(x_sorted, "x_sorted", d, R * H),
        _ptr(w_gate, "w_gate", d, E * H * F), _ptr(w_up, "w_up", d, E * H * F), _ptr(w_down, "w_down", d, E * F * H),
        _ptr(h_save, "h_save", d, R * 2 * F, allow_none=True), _ptr(a_save, "a_save", d, R * F),
        _ptr(o_sorted, "o_sorted", d, R * H), _stream(stream)))


class Fp8Weights:
    """Frozen expert weights stored once in fp8 (E4M3) by moe_quantize_weights_fp8:
    codes q_gate/q_up [E,H,F], q_down [E,F,H] (uint8) and per-expert fp32 scales
    s_gu (shared by W_gate and W_up) and s_down [E]."""

    def __init__(self, w_gate, w_up, w_down, stream=None):
        E, H, F = w_gate.shape
        if w_gate.dtype != torch.bfloat16:
            raise MoeError("fp8 storage is made from bf16 weights")
        dev = w_gate.device
        self.E, self.H, self.F = E, H, F
        self.q_gate = torch.empty(E, H, F, dtype=torch.uint8, device=dev)
        self.q_up = torch.empty(E, H, F, dtype=torch.uint8, device=dev)
        self.q_down = torch.empty(E, F, H, dtype=torch.uint8, device=dev)
        self.s_gu = torch.empty(E, dtype=F32, device=dev)
        self.s_down = torch.empty(E, dtype=F32, device=dev)
        moe_quantize_weights_fp8(w_gate, w_up, self.q_gate, self.q_up, self.s_gu, stream)
        moe_quantize_weights_fp8(w_down, None, self.q_down, None, self.s_down, stream)


class Fp8KMajorWeights:
    """fp8 (E4M3) weight codes in the K-major layout of the fp8 matrix-core
    forward (moe_grouped_swiglu_fwd_fp8): W_gate^T, W_up^T [E,F,H] and
    W_down^T [E,H,F] codes, transposed once from Fp8Weights' codes, with the
    same per-expert scales."""

    def __init__(self, wq: "Fp8Weights", stream=None):
        E, H, F = wq.E, wq.H, wq.F
        dev = wq.q_gate.device
        self.E, self.H, self.F = E, H, F
        self.t_gate = torch.empty(E, F, H, dtype=torch.uint8, device=dev)
        self.t_up = torch.empty(E, F, H, dtype=torch.uint8, device=dev)
        self.t_down = torch.empty(E, H, F, dtype=torch.uint8, device=dev)
        self.s_gu, self.s_down = wq.s_gu, wq.s_down
        moe_transpose_fp8(wq.q_gate, self.t_gate, stream)
        moe_transpose_fp8(wq.q_up, self.t_up, stream)
        moe_transpose_fp8(wq.q_down, self.t_down, stream)


def moe_transpose_fp8(q_in, q_out, stream=None):
    E, rows, cols = q_in.shape
    U8 = torch.uint8
    _check(lib().moe_transpose_fp8(E, rows, cols, _ptr(q_in, "in", U8, E * rows * cols),
                                   _ptr(q_out, "out", U8, E * rows * cols), _stream(stream)))


def moe_quantize_rows_fp8(x, q, scale, stream=None):
    rows, cols = x.shape
    _check(lib().moe_quantize_rows_fp8(rows, cols, _ptr(x, "x", torch.bfloat16, rows * cols),
                                       _ptr(q, "q", torch.uint8, rows * cols), _ptr(scale, "scale", F32, rows),
                                       _stream(stream)))


def moe_grouped_swiglu_fwd_fp8(offsets, xq, x_scale, wt: Fp8KMajorWeights, h_save, a_save, aq, a_scale, o_sorted,
                               max_rows: int, perm=None, k: int = 1, stream=None):
    """xq / x_scale: quantized rows of x_sorted, or with perm the quantized token
    rows (gathered on load)."""
    E, H, F = wt.E, wt.H, wt.F
    d, U8, R = torch.bfloat16, torch.uint8, max_rows
    nx = (R // k) if perm is not None else R
    _check(lib().moe_grouped_swiglu_fwd_fp8(
        H, F, E, k, R, _ptr(offsets, "offsets", I32, E + 1), _ptr(xq, "xq", U8, nx * H),
        _ptr(x_scale, "x_scale", F32, nx), _ptr(perm, "perm", I32, R, allow_none=True),
        _ptr(wt.t_gate, "t_gate", U8, E * F * H), _ptr(wt.t_up, "t_up", U8, E * F * H),
        _ptr(wt.t_down, "t_down", U8, E * H * F), _ptr(wt.s_gu, "s_gu", F32, E), _ptr(wt.s_down, "s_down", F32, E),
        _ptr(h_save, "h_save", d, R * 2 * F, allow_none=True), _ptr(a_save, "a_save", d, R * F),
        _ptr(aq, "aq", U8, R * F), _ptr(a_scale, "a_scale", F32, R), _ptr(o_sorted, "o_sorted", d, R * H),
        _stream(stream)))


def moe_quantize_weights_fp8(w0, w1, q0, q1, scale, stream=None):
    E = w0.shape[0]
    n0 = w0.numel() // E
    n1 = 0 if w1 is None else w1.numel() // E
    U8 = torch.uint8
    _check(lib().moe_quantize_weights_fp8(
        E, n0, n1, _ptr(w0, "w0", torch.bfloat16, E * n0), _ptr(w1, "w1", torch.bfloat16, E * n1, allow_none=True),
        _ptr(q0, "q0", U8, E * n0), _ptr(q1, "q1", U8, E * n1, allow_none=w1 is None), _ptr(scale, "scale", F32, E),
        _stream(stream)))


def moe_grouped_swiglu_fwd_fp8w(offsets, x_rows, wq: Fp8Weights, h_save, a_save, o_sorted, max_rows: int,
                                perm=None, k: int = 1, stream=None):
    """x_rows: x_sorted, or with perm the token matrix x [T, H] (rows gathered on load)."""
    E, H, F = wq.E, wq.H, wq.F
    d, U8, R = torch.bfloat16, torch.uint8, max_rows
    _check(lib().moe_grouped_swiglu_fwd_fp8w(
        H, F, E, k, R, _ptr(offsets, "offsets", I32, E + 1),
        _ptr(x_rows, "x_rows", d, (R // k) * H if perm is not None else R * H),
        _ptr(perm, "perm", I32, R, allow_none=True),
        _ptr(wq.q_gate, "q_gate", U8, E * H * F), _ptr(wq.q_up, "q_up", U8, E * H * F),
        _ptr(wq.q_down, "q_down", U8, E * F * H), _ptr(wq.s_gu, "s_gu", F32, E), _ptr(wq.s_down, "s_down", F32, E),
        _ptr(h_save, "h_save", d, R * 2 * F, allow_none=True), _ptr(a_save, "a_save", d, R * F),
        _ptr(o_sorted, "o_sorted", d, R * H), _stream(stream)))


def moe_grouped_bwd_dx_fp8w(offsets, inv, dy, topk_w, h_rows, wq: Fp8Weights, dO_rows, dh_rows, dX_rows, dx,
                            max_rows: int, inv_all=None, o_sorted=None, dg=None, stream=None, h_src=None):
    T, H = dy.shape
    E, F = wq.E, wq.F
    k = topk_w.shape[1]
    d, U8, R, N = torch.bfloat16, torch.uint8, max_rows, T * k
    _check(lib().moe_grouped_bwd_dx_fp8w(
        T, H, F, E, k, R, _ptr(offsets, "offsets", I32, E + 1), _ptr(inv, "inv", I32, N),
        _ptr(dy, "dy", d, T * H), _ptr(topk_w, "topk_w", F32, N),
        _ptr(h_rows, "h_rows", d, 2 * F if h_src is not None else R * 2 * F),
        _ptr(h_src, "h_src", I32, R, allow_none=True),
        _ptr(wq.q_gate, "q_gate", U8, E * H * F), _ptr(wq.q_up, "q_up", U8, E * H * F),
        _ptr(wq.q_down, "q_down", U8, E * F * H), _ptr(wq.s_gu, "s_gu", F32, E), _ptr(wq.s_down, "s_down", F32, E),
        _ptr(inv_all, "inv_all", I32, N, allow_none=dg is None),
        _ptr(o_sorted, "o_sorted", d, N * H, allow_none=dg is None), _ptr(dg, "dg", F32, N, allow_none=True),
        _ptr(dO_rows, "dO_rows", d, R * H), _ptr(dh_rows, "dh_rows", d, R * 2 * F), _ptr(dX_rows, "dX_rows", d, R * H),
        _ptr(dx, "dx", d, T * H), _stream(stream)))


def moe_grouped_swiglu_fwd_gather(offsets, x, perm, w_gate, w_up, w_down, h_save, a_save, o_sorted, k: int,
                                  max_rows: int, max_expert_rows: int | None = None, stream=None):
    E, H, F = w_gate.shape
    dt, d = _dt(w_gate), w_gate.dtype
    R = max_rows
    T = x.shape[0]
    _check(lib().moe_grouped_swiglu_fwd_gather(
        H, F, E, k, R, R if max_expert_rows is None else max_expert_rows, dt, _ptr(offsets, "offsets", I32, E + 1),
        _ptr(x, "x", d, T * H), _ptr(perm, "perm", I32, R), _ptr(w_gate, "w_gate", d, E * H * F),
        _ptr(w_up, "w_up", d, E * H * F), _ptr(w_down, "w_down", d, E * F * H),
        _ptr(h_save, "h_save", d, R * 2 * F, allow_none=True), _ptr(a_save, "a_save", d, R * F),
        _ptr(o_sorted, "o_sorted", d, R * H), _stream(stream)))


def moe_grouped_swiglu_recompute(offsets, x_rows, w_gate, w_up, h_rows, a_rows, max_rows: int,
                                 max_expert_rows: int | None = None, stream=None, x_src=None, x_div: int = 1):
    """x_src: row s of x is x_rows[x_src[s] / x_div] (rows gathered on load)."""
    E, H, F = w_gate.shape
    dt, d = _dt(w_gate), w_gate.dtype
    R = max_rows
    _check(lib().moe_grouped_swiglu_recompute(
        H, F, E, R, R if max_expert_rows is None else max_expert_rows, dt, _ptr(offsets, "offsets", I32, E + 1),
        _ptr(x_rows, "x_rows", d, H if x_src is not None else R * H), _ptr(x_src, "x_src", I32, R, allow_none=True),
        x_div, _ptr(w_gate, "w_gate", d, E * H * F), _ptr(w_up, "w_up", d, E * H * F),
        _ptr(h_rows, "h_rows", d, R * 2 * F), _ptr(a_rows, "a_rows", d, R * F, allow_none=True), _stream(stream)))


def moe_combine(rows, inv, topk_w, out, k: int, stream=None):
    T, H = out.shape
    d = out.dtype
    rows_needed = int(rows.shape[0])
    _check(lib().moe_combine(T, H, k, _dt(out), _ptr(rows, "rows", d, rows_needed * H), _ptr(inv, "inv", I32, T * k),
                             _ptr(topk_w, "topk_w", F32, T * k, allow_none=True), _ptr(out, "out", d, T * H),
                             _stream(stream)))


def moe_grouped_bwd_dx(offsets, inv, dy, topk_w, h_rows, w_gate, w_up, w_down, dO_rows, dh_rows, dX_rows, dx,
                       max_rows: int, inv_all=None, o_sorted=None, dg=None, stream=None, h_src=None):
    """h_src: row r's pre-activations are h_rows[h_src[r]] (e.g. h_save with kept_src)."""
    T, H = dy.shape
    E, _, F = w_gate.shape
    k = topk_w.shape[1]
    d = dy.dtype
    R = max_rows
    N = T * k
    _check(lib().moe_grouped_bwd_dx(
        T, H, F, E, k, R, _dt(dy), _ptr(offsets, "offsets", I32, E + 1), _ptr(inv, "inv", I32, N), _ptr(dy, "dy", d, T * H), _ptr(topk_w, "topk_w", F32, N),
        _ptr(h_rows, "h_rows", d, 2 * F if h_src is not None else R * 2 * F),
        _ptr(h_src, "h_src", I32, R, allow_none=True),
        _ptr(w_gate, "w_gate", d, E * H * F), _ptr(w_up, "w_up", d, E * H * F),
        _ptr(w_down, "w_down", d, E * F * H), _ptr(inv_all, "inv_all", I32, N, allow_none=dg is None),
        _ptr(o_sorted, "o_sorted", d, N * H, allow_none=dg is None), _ptr(dg, "dg", F32, N, allow_none=True),
        _ptr(dO_rows, "dO_rows", d, R * H), _ptr(dh_rows, "dh_rows", d, R * 2 * F), _ptr(dX_rows, "dX_rows", d, R * H),
        _ptr(dx, "dx", d, T * H), _stream(stream)))


def moe_signal_dh_ready(event):
    """Arm the next moe_grouped_bwd_dx* call of this thread to record `event`
    (a torch.cuda.Event, already created) once dO and dh are written."""
    _check(lib().moe_signal_dh_ready(ctypes.c_void_p(event.cuda_event if event is not None else None)))


def moe_grouped_bwd_dw(offsets, x_rows, a_rows, dO_rows, dh_rows, dw_gate, dw_up, dw_down, max_rows: int, stream=None,
                       x_src=None, x_div: int = 1, a_src=None):
    """x_src / a_src: rows gathered on load (row r of x is x_rows[x_src[r] / x_div],
    row r of a is a_rows[a_src[r]])."""
    E, H, F = dw_gate.shape
    d = dw_gate.dtype
    R = max_rows
    _check(lib().moe_grouped_bwd_dw(
        H, F, E, R, _dt(dw_gate), _ptr(offsets, "offsets", I32, E + 1),
        _ptr(x_rows, "x_rows", d, H if x_src is not None else R * H), _ptr(x_src, "x_src", I32, R, allow_none=True),
        x_div, _ptr(a_rows, "a_rows", d, F if a_src is not None else R * F),
        _ptr(a_src, "a_src", I32, R, allow_none=True),
        _ptr(dO_rows, "dO_rows", d, R * H), _ptr(dh_rows, "dh_rows", d, R * 2 * F),
        _ptr(dw_gate, "dw_gate", d, E * H * F), _ptr(dw_up, "dw_up", d, E * H * F),
        _ptr(dw_down, "dw_down", d, E * F * H), _stream(stream)))


def moe_quota_cap_for_budget(T: int, H: int, F: int, E: int, k: int, dtype, with_dw: bool, keep_graph: bool,
                             budget_bytes: int) -> int:
    dt = MOE_F32 if dtype == torch.float32 else MOE_BF16
    return int(lib().moe_quota_cap_for_budget(T, H, F, E, k, dt, int(bool(with_dw)), int(bool(keep_graph)),
                                              int(budget_bytes)))


def moe_pair_scores(inv_perm, topk_w, a_save, dy, score, stream=None):
    T, H = dy.shape
    k = topk_w.shape[1]
    F = a_save.shape[1]
    d = dy.dtype
    _check(lib().moe_pair_scores(T, H, F, k, _dt(dy), _ptr(inv_perm, "inv_perm", I32, T * k),
                                 _ptr(topk_w, "topk_w", F32, T * k), _ptr(a_save, "a_save", d, None),
                                 _ptr(dy, "dy", d, T * H), _ptr(score, "score", F32, T * k), _stream(stream)))


def moe_compact_pairs(counts, offsets, perm, score, rho, kept_counts, kept_offsets, kept_perm, kept_src,
                      kept_inv, T: int, k: int, x_sorted=None, a_save=None, h_save=None, x_kept=None, a_kept=None,
                      h_kept=None, stream=None, cap=None):
    """Quota from rho (moe_compact_pairs) or, when cap is given, that quota
    directly (moe_compact_pairs_cap; rho is then ignored)."""
    E = counts.shape[0]
    N = T * k
    ref = next((t for t in (x_sorted, a_save, h_save) if t is not None), None)
    d = ref.dtype if ref is not None else torch.bfloat16
    H = x_sorted.shape[1] if x_sorted is not None else 8
    F = a_save.shape[1] if a_save is not None else (h_save.shape[1] // 2 if h_save is not None else 8)
    q = moe_quota_cap(T, E, k, rho) if cap is None else int(cap)
    R = min(N, E * q) if q > 0 else 0
    call = lib().moe_compact_pairs if cap is None else lib().moe_compact_pairs_cap
    _check(call(
        T, H, F, E, k, MOE_F32 if d == torch.float32 else MOE_BF16, float(rho) if cap is None else q,
        _ptr(counts, "counts", I32, E),
        _ptr(offsets, "offsets", I32, E + 1), _ptr(perm, "perm", I32, N), _ptr(score, "score", F32, N),
        _ptr(kept_counts, "kept_counts", I32, E), _ptr(kept_offsets, "kept_offsets", I32, E + 1),
        _ptr(kept_perm, "kept_perm", I32, R), _ptr(kept_src, "kept_src", I32, R), _ptr(kept_inv, "kept_inv", I32, N),
        _ptr(x_sorted, "x_sorted", d, N * H, allow_none=True), _ptr(a_save, "a_save", d, N * F, allow_none=True),
        _ptr(h_save, "h_save", d, N * 2 * F, allow_none=True),
        _ptr(x_kept, "x_kept", d, R * H, allow_none=x_sorted is None),
        _ptr(a_kept, "a_kept", d, R * F, allow_none=a_save is None),
        _ptr(h_kept, "h_kept", d, R * 2 * F, allow_none=h_save is None), _stream(stream)))
