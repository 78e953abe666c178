"""Benchmark of one MoE layer's expert computation in training on one MI355X.

One step = the whole path on one batch: route -> dispatch -> grouped SwiGLU
forward -> combine -> backward dx (+ dg), plus compaction and dW for the
workloads that train experts.  Inputs are seeded synthetic tensors already
resident in HBM when timing starts.  Default workload: the Qwen3-30B-A3B
expert shape in a LoRA step (T=128 tokens, H=2048, F=768, E=128, top-8, bf16,
experts frozen: forward + dx).

Prints ONE JSON line: tokens/s over K timed steps, the roofline of the
dominant kernel (its duration from HIP events on its own stream, inside the
timed steps), and the CPU oracle timed on the host cores.  By default the line
also carries one record per other workload under "configs" (the tiny fp32
layer, full fine-tuning at the Qwen3 and GLM-Air shapes, the compacted
backward): step time, tokens/s, TFLOPS against the matrix-core peak, the
dominant kernel's roofline, the row kernels against HBM and a per-phase oracle
baseline on a token prefix.  Between the warmup
and the timed steps, a few untimed steps with every GEMM bracketed by events
give the per-kernel durations and pick the dominant kernel; inside the timed
steps only that kernel is bracketed (each event costs stream time).  After the
timed steps (untimed, --no-probes skips them): the per-step time distribution
(median, p10, p90; back to back and with the last-level cache flushed before
every step) and probes of plain read / write / copy bandwidth and of a bf16
library matmul on the same GPU, as context for the roofline fractions.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd+bwd tokens/sec and TFLOPS (% bf16 MFMA peak), Qwen3-30B-A3B shape"
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_F32_TFLOPS = 157.3
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published

# kernel ids of include/moe.h (moe_kernel)
K_GATEUP, K_DOWN, K_COMBINE, K_GRAD_ROWS, K_DA, K_DX, K_DW, K_DISPATCH_ROWS = 2, 3, 4, 5, 6, 7, 8, 1
K_ROUTER_FWD, K_ROUTER_DW = 10, 11
# Phases bracketed by moe_profile_kernel; a GEMM phase is every kernel one
# call launches (bf16: experts below 256 rows on row_gemm_bf16_kernel, larger
# ones on big_gemm_bf16_kernel; dW: dw_small_bf16_kernel then dw_bf16_kernel;
# fp32: row_gemm_f32_kernel, dw_f32_kernel), timed as one.
KERNEL_NAMES = {K_GATEUP: "gate/up GEMM + SwiGLU", K_DOWN: "down GEMM", K_DA: "dA GEMM + SwiGLU backward",
                K_DX: "dX GEMM", K_DW: "dW GEMMs",
                K_DISPATCH_ROWS: "dispatch_rows_kernel", K_GRAD_ROWS: "grad_rows_kernel",
                K_COMBINE: "combine_kernel", K_ROUTER_FWD: "router logits (x W_r)",
                K_ROUTER_DW: "router_bwd (dlogits, dW_r, dx)"}


def _parser():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="qwen3_lora_t128")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    p.add_argument("--cpu-tokens", type=int, default=0, help="tokens of the CPU-oracle sample (0: auto)")
    p.add_argument("--router", action="store_true",
                   help="run the router in front of the path (logits = x W_r, drawn W_r) and its backward after dx")
    p.add_argument("--gather-rows", choices=("auto", "on", "off"), default="auto",
                   help="GEMMs read token rows through the pair indices (on) or from the materialized x_sorted "
                        "(off); auto: the layer's choice (gathered unless dW runs over all pairs)")
    p.add_argument("--overlap-dw", action="store_true",
                   help="full fine-tuning: weight gradients on a second stream alongside the dX GEMM and the dx sum")
    p.add_argument("--no-keep-graph", action="store_true",
                   help="recompute path: the forward keeps no pre-activations, the backward recomputes them")
    p.add_argument("--forward-only", action="store_true",
                   help="time the forward alone (route, dispatch, expert GEMMs, combine), e.g. for decode batches")
    p.add_argument("--metric-score", action="store_true",
                   help="compacted workloads: rank pairs by the norm of their rank-one dW_down term instead of the "
                        "routing weight")
    p.add_argument("--budget-mib", type=int, default=0,
                   help="compacted workloads: quota from this memory budget for the backward's rows instead of rho")
    p.add_argument("--fp8-weights", action="store_true",
                   help="frozen expert weights stored once in fp8 (E4M3, one power-of-two scale per expert) and read "
                        "by the GEMMs (LoRA and forward-only workloads; not the headline configuration)")
    p.add_argument("--fp8-mma", action="store_true",
                   help="forward only, both expert GEMMs on the fp8 matrix cores (E4M3 operands: token rows and the "
                        "SwiGLU output quantized per row, weights per expert); peak: the fp8 one")
    p.add_argument("--no-probes", action="store_true",
                   help="skip the per-step distribution pass and the bandwidth / matrix-core probes")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="after the timed steps, run one plain elementwise copy of this many MiB (read and write "
                        "each) so that HBM byte counters can be calibrated against a kernel of known traffic")
    p.add_argument("--no-configs", action="store_true",
                   help="measure only the chosen workload (by default the tiny fp32 layer, full fine-tuning at the "
                        "Qwen3 and GLM-Air shapes and the compacted backward follow, one record each under "
                        "\"configs\")")
    return p


def parse():
    return _parser().parse_args()


def parse_defaults():
    """The default path options (no flags)."""
    return _parser().parse_args([])


# Sources whose code decides the HBM traffic of each kernel; a stored counter
# reading only counts while these files are unchanged.
KERNEL_SOURCES = {
    K_GATEUP: ("moe_gemm_bf16.hip", "moe_gemm_big.hip", "moe_lds32.h", "moe_common.h", "moe_launch.h"),
    K_DOWN: ("moe_gemm_bf16.hip", "moe_gemm_big.hip", "moe_lds32.h", "moe_common.h", "moe_launch.h"),
    K_DA: ("moe_gemm_bf16.hip", "moe_gemm_big.hip", "moe_lds32.h", "moe_common.h", "moe_launch.h"),
    K_DX: ("moe_gemm_bf16.hip", "moe_gemm_big.hip", "moe_lds32.h", "moe_common.h", "moe_launch.h"),
    K_DW: ("moe_gemm_dw.hip", "moe_lds32.h", "moe_common.h", "moe_launch.h"),
}
TRAFFIC_FILE = {K_GATEUP: "gemm_gateup", K_DOWN: "gemm_down", K_DA: "gemm_da", K_DX: "gemm_dx", K_DW: "gemm_dw"}


def sources_digest(kernel):
    """sha256 of the kernel's sources with comments and blank space removed
    (an edit of a comment does not change the kernel)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "expert_grouped_gemm_top_amd", "csrc", name)) as f:
            code = re.sub(r"/\*.*?\*/", " ", f.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        code = " ".join(code.split())
        h.update(name.encode() + b"\0" + code.encode())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary of this kernel
    and workload (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or
    None when there is none or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{TRAFFIC_FILE[kernel]}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    m_h = re.search(r"^sources_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not (m_b and m_h) or m_h.group(1) != sources_digest(kernel):
        return None
    return int(m_b.group(1))


def algorithmic(wl, counts, kept_counts=None, gathered=False, weight_bytes=None, fp8_inputs=False):
    """Per-kernel algorithmic bytes and flops (real rows only, no padding).
    gathered: the gate/up product reads token rows [T,H] through perm instead of
    the materialized x_sorted [N,H].  weight_bytes: bytes per expert-weight
    element when it differs from the activations' (1 for fp8 weights).
    fp8_inputs: the forward products read their activation rows as fp8 codes
    (1 byte) with one fp32 scale per row."""
    b = 2 if wl.dtype == "bf16" else 4
    wb = b if weight_bytes is None else weight_bytes
    ab = 1 if fp8_inputs else b  # bytes per activation element read by the forward products
    H, F, T, k = wl.H, wl.F, wl.T, wl.k
    N = wl.N
    Ea = int((counts > 0).sum())
    R = int(kept_counts.sum()) if kept_counts is not None else N
    Ea_b = int((kept_counts > 0).sum()) if kept_counts is not None else Ea
    sx = 4 * T if fp8_inputs else 0  # row scales
    return {
        K_DISPATCH_ROWS: (T * H * b + N * H * b + 4 * N, 0.0),
        K_GATEUP: (2 * H * F * wb * Ea + (T * H * ab + 4 * N if gathered else N * H * ab) + sx + N * 2 * F * b
                   + N * F * b, 4.0 * H * F * N),
        K_DOWN: (H * F * wb * Ea + N * F * ab + (4 * N if fp8_inputs else 0) + N * H * b, 2.0 * H * F * N),
        K_COMBINE: (N * H * b + 8 * N + T * H * b, 0.0),
        K_GRAD_ROWS: (T * H * b + R * H * b + 8 * N + N * H * b, 0.0),
        K_DA: (H * F * wb * Ea_b + R * H * b + 2 * R * 2 * F * b, 2.0 * H * F * R),
        K_DX: (2 * H * F * wb * Ea_b + R * 2 * F * b + R * H * b, 4.0 * H * F * R),
        K_DW: (R * (2 * H + 3 * F) * b + 3 * H * F * wl.E * b, 6.0 * H * F * R),
        # router: x and W_r in, fp32 logits out; backward reads x, W_r, dx and
        # writes dlogits, dW_r, dx
        K_ROUTER_FWD: (T * H * b + H * wl.E * b + 4 * T * wl.E, 2.0 * T * H * wl.E),
        K_ROUTER_DW: (2 * T * H * b + H * wl.E * b + 8 * T * wl.E + H * wl.E * b + T * H * b + 12 * T * k,
                      4.0 * T * H * wl.E),
    }


def environment(dev, read_clocks=True):
    """GPU, software versions and the host CPU the oracle baseline runs on.
    read_clocks: ask rocm-smi for the current clocks (a child process; skipped
    for profiled runs, which pass --no-probes)."""
    import torch
    p = torch.cuda.get_device_properties(dev)
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    clocks = None
    try:  # current shader / memory clocks as the driver reports them (best effort)
        import subprocess
        if not read_clocks:
            raise OSError("not asked for")
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
        found = {key: m.group(1) for key in ("sclk", "mclk")
                 for m in [re.search(rf"{key} clock level: [^:]+: \((\d+\s*Mhz)\)", r.stdout)] if m}
        clocks = found or None
    except (OSError, subprocess.SubprocessError):
        pass
    return {"gpu": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "clocks": clocks, "hip": torch.version.hip, "torch": torch.__version__, "host_cpu": cpu,
            "host_threads": os.cpu_count()}


def step_distribution(step, stream, dev, n):
    """Untimed pass after the timed steps: every step bracketed by HIP events on
    the layer's stream; median / p10 / p90 in ms, once back to back and once
    with a 512 MiB buffer read before every step, so that nothing the previous
    step left in the 256 MB last-level cache is reused (a read evicts with
    clean lines: a fill would leave dirty lines whose write-back then competes
    with the step)."""
    import numpy as np
    import torch
    flush = torch.ones(256 << 20, dtype=torch.float16, device=dev)  # 512 MiB

    def run(flushed):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in ev:  # no host sync between steps: the stream stays fed
            if flushed:
                flush.sum(dtype=torch.float32)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        q = np.percentile([a.elapsed_time(b) for a, b in ev], [10, 50, 90])
        return {"p10": float(q[0]), "median": float(q[1]), "p90": float(q[2])}

    out = {"steps": n, "back_to_back": run(False), "cache_flushed": run(True)}
    del flush
    return out


def probes(dev):
    """What this GPU reaches on plain work, as context for the roofline
    fractions (torch's own kernels): a write (fill) and a copy (read + write,
    both counted) over 1 GiB, and a bf16 8192^3 matmul (hipBLASLt).  No read
    probe: torch's reductions do not stream at HBM speed."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)

    def best_ms(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best

    res = {"write_GBs": n / best_ms(lambda: dst.fill_(2.0)) / 1e6,
           "copy_GBs": 2 * n / best_ms(lambda: dst.copy_(src)) / 1e6,
           "bf16_matmul_8192_TFLOPs": 2 * 8192 ** 3 / best_ms(lambda: torch.mm(a, b)) / 1e9}
    del src, dst, a, b
    # the library GEMM on one expert's gate/up product (M rows x K = H, N = 2F)
    # at the GLM-Air and Qwen3 shapes, beside the grouped kernels' per-phase rates
    res["bf16_matmul_expert_TFLOPs"] = {}
    for M, K, N in ((4096, 4096, 2816), (2048, 4096, 2816), (4096, 2048, 1536), (2048, 2048, 1536)):
        a = torch.randn(M, K, dtype=torch.bfloat16, device=dev)
        b = torch.randn(K, N, dtype=torch.bfloat16, device=dev)
        res["bf16_matmul_expert_TFLOPs"][f"{M}x{K}x{N}"] = 2 * M * K * N / best_ms(lambda: torch.mm(a, b), reps=10) / 1e9
        del a, b
    return res


def cpu_baseline(wl, d, logits, sample_tokens, min_seconds=10.0):
    """The oracle (as it stands, IEEE double) on a token prefix of the same
    workload, phase by phase: route -> dispatch -> forward (with the combine)
    -> [compaction] -> backward dx, dg -> [dW].  The whole sample is repeated
    until about ``min_seconds`` of host work has been timed."""
    import numpy as np

    import oracle
    T = sample_tokens
    # inputs upcast to float64 once, outside the timed region (input marshalling)
    sub = {n: np.ascontiguousarray(d[n][:T], dtype=np.float64) for n in ("x", "dy")}
    W64 = {n: np.ascontiguousarray(d[n], dtype=np.float64) for n in ("W_gate", "W_up", "W_down")}
    lg = np.ascontiguousarray(logits[:T], dtype=np.float64)
    Wg, Wu, Wd = W64["W_gate"], W64["W_up"], W64["W_down"]
    phases = {"route": 0.0, "dispatch": 0.0, "forward+combine": 0.0}
    if wl.rho is not None:
        phases["compact"] = 0.0
    phases["backward dx+dg"] = 0.0
    if wl.dw:
        phases["dW"] = 0.0
    reps, dt = 0, 0.0
    while dt < min_seconds and reps < 20:
        def timed(name, fn, *a, **kw):
            t0 = time.perf_counter()
            r = fn(*a, **kw)
            phases[name] += time.perf_counter() - t0
            return r
        idx, w = timed("route", oracle.route_topk, lg, wl.k)
        counts, offsets, perm, _ = timed("dispatch", oracle.dispatch, idx, wl.E)
        timed("forward+combine", oracle.forward, sub["x"], idx, w, Wg, Wu, Wd)
        retained = None
        if wl.rho is not None:
            retained = timed("compact", oracle.compact, T, wl.E, wl.k, counts, offsets, perm, w, wl.rho)["retained"]
        timed("backward dx+dg", oracle.backward, sub["x"], idx, w, Wg, Wu, Wd, sub["dy"], retained=retained)
        if wl.dw:
            timed("dW", oracle.backward_dw, sub["x"], idx, w, Wg, Wu, Wd, sub["dy"], retained=retained)
        dt = sum(phases.values())
        reps += 1
    steps = "route+dispatch+forward+combine" + ("+compact" if wl.rho is not None else "") + "+dx+dg" + \
            ("+dW" if wl.dw else "")
    return {"value": T * reps / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "precision": "fp64",
            "sample": f"{T} of {wl.T} tokens of {wl.name}, {reps} repetitions (fp64 oracle, {steps}), {dt:.2f} s wall",
            "phase_s_per_rep": {n: v / reps for n, v in phases.items()}}


def measure(wl, args, steps, warmup, cpu_tokens, cpu_seconds, dist_and_probes=False, timers=None):
    """One workload on the GPU: warmup, an untimed pass with every kernel
    bracketed (per-kernel durations, the dominant kernel), then ``steps`` timed
    steps with only the dominant kernel bracketed.  Returns the record.  With
    a dict ``timers``, the layer stays resident and timers[wl.name] = f(n)
    times n more steps (ms per step) for the interleaved rounds."""
    import numpy as np
    import torch

    from expert_grouped_gemm_top_amd import moe
    from expert_grouped_gemm_top_amd import workloads as W
    from expert_grouped_gemm_top_amd.layer import MoeLayerBuffers

    f32 = wl.dtype == "f32"
    tdt = torch.float32 if f32 else torch.bfloat16
    d = W.generate(wl, seed=0)
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(d[n]).to(dev).to(tdt) for n in ("x", "W_gate", "W_up", "W_down", "dy")}
    if wl.router == "wr":
        # router-weight workloads: the logits x W_r are an input of the step,
        # computed once here with the library's router kernel
        w_r_in = torch.from_numpy(d["W_r"]).to(dev).to(tdt)
        logits = torch.empty(wl.T, wl.E, dtype=torch.float32, device=dev)
        rws = torch.empty(max(moe.moe_router_workspace_bytes(wl.T, wl.H, wl.E), 16), dtype=torch.uint8, device=dev)
        moe.moe_router_fwd(t["x"], w_r_in, logits, rws)
        torch.cuda.synchronize()
        logits_host = None
    else:
        logits = torch.from_numpy(d["logits"]).to(dev)
        logits_host = d["logits"]
    quota_cap = None
    if args.budget_mib > 0 and wl.rho is not None:
        quota_cap = moe.moe_quota_cap_for_budget(wl.T, wl.H, wl.F, wl.E, wl.k, tdt, wl.dw,
                                                 not args.no_keep_graph, args.budget_mib << 20)
        assert quota_cap >= 1, "the budget does not hold one row per expert"
    L = MoeLayerBuffers(wl.T, wl.H, wl.F, wl.E, wl.k, tdt, dev, rho=wl.rho if quota_cap is None else None,
                        dw=wl.dw, dg=True, router=args.router, keep_graph=not args.no_keep_graph, quota_cap=quota_cap,
                        overlap_dw=args.overlap_dw,
                        gather_rows=None if args.gather_rows == "auto" else args.gather_rows == "on")
    score = "metric" if args.metric_score else None
    wq = wt = None
    if args.fp8_mma:
        assert not f32, "the fp8 matrix-core forward takes bf16 inputs"
        wt = moe.Fp8KMajorWeights(moe.Fp8Weights(t["W_gate"], t["W_up"], t["W_down"]))  # once, before any timing
        args = argparse.Namespace(**{**vars(args), "forward_only": True})
    if args.fp8_weights:
        assert not wl.dw and wl.rho is None and not args.no_keep_graph and not f32, \
            "fp8 weights are frozen: bf16 LoRA or forward-only workloads, pre-activations kept"
        wq = moe.Fp8Weights(t["W_gate"], t["W_up"], t["W_down"])  # once, before any timing
    w_r = torch.from_numpy(W.router_weights(wl, seed=0)).to(dev).to(tdt) if args.router else None
    stream = torch.cuda.current_stream()

    def step():
        L.forward(logits, t["x"], t["W_gate"], t["W_up"], t["W_down"], stream, w_r=w_r, wq=wq, wt=wt)
        if not args.forward_only:
            L.backward(t["dy"], t["W_gate"], t["W_up"], t["W_down"], stream=stream, w_r=w_r, score=score, wq=wq)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    gemm_kernels = [K_GATEUP, K_DOWN] + ([] if args.forward_only else [K_DA, K_DX] + ([K_DW] if wl.dw else []))
    router_kernels = ([K_ROUTER_FWD] + ([] if args.forward_only else [K_ROUTER_DW])) if args.router else []
    # HBM-bound row kernels launched once per step (the first combine of a step
    # is the forward's); the row copy of dispatch only when rows are materialized
    hbm_kernels = ([] if L.gather_rows or wt is not None else [K_DISPATCH_ROWS]) + [K_COMBINE] + \
                  ([] if args.forward_only else [K_GRAD_ROWS])
    profiled = gemm_kernels + router_kernels + hbm_kernels
    lib = moe.lib()
    lib.moe_profile_kernel.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]

    def event_pairs(n):
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in pairs:  # torch creates the underlying hipEvent at the first record
            a.record(stream)
            b.record(stream)
        return pairs

    def run_steps(n, kinds):
        """n steps; every launch of the given kernel kinds is bracketed by HIP
        events recorded on the stream it runs on (an event costs a few
        microseconds of stream time, so only the kinds asked for are armed)."""
        ev = {kk: event_pairs(n) for kk in kinds}
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(n):
            for kk in kinds:
                a, b = ev[kk][s]
                lib.moe_profile_kernel(kk, ctypes.c_void_p(a.cuda_event), ctypes.c_void_p(b.cuda_event))
            step()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        return dt, {kk: float(np.mean([a.elapsed_time(b) for a, b in ev[kk]])) for kk in kinds}

    # untimed pass: every GEMM's duration, to find the dominant kernel
    _, kernel_ms = run_steps(max(3, min(steps, 10)), profiled)
    dom = max(gemm_kernels, key=lambda kk: kernel_ms[kk])
    # timed steps: only the dominant kernel is bracketed by events
    elapsed, dom_ms = run_steps(steps, [dom])
    ms_per_step = elapsed * 1e3 / steps
    tokens_per_s = wl.T * steps / elapsed

    counts = L.counts.cpu().numpy()
    kept = L.kept_counts.cpu().numpy() if L.compacted else None
    alg = algorithmic(wl, counts, kept, gathered=L.gather_rows or wt is not None,
                      weight_bytes=1 if (wq is not None or wt is not None) else None, fp8_inputs=wt is not None)
    step_flops = sum(alg[kk][1] for kk in gemm_kernels)
    peak_flops = PEAK_F32_TFLOPS if f32 else (PEAK_FP8_TFLOPS if wt is not None else PEAK_BF16_TFLOPS)
    byts, flops = alg[dom]
    compute_bound = flops / byts > peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    sec = dom_ms[dom] * 1e-3
    if compute_bound:
        # fp32 layers run on plain fp32 FMAs (vector ALU), bf16 on the matrix cores
        roof = {"bound": "alu" if f32 else "mfma", "achieved": flops / sec / 1e12, "peak": peak_flops,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": byts / sec / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # the stored counter readings are of the bf16-weight kernels
    roof["traffic"] = None if (wq is not None or wt is not None) else measured_traffic(dom, wl.name)
    roof["kernel"] = KERNEL_NAMES[dom]
    roof["kernel_us"] = dom_ms[dom] * 1e3
    roof["algorithmic_bytes"] = byts
    roof["algorithmic_flops"] = flops
    roof["mfma_frac"] = flops / sec / 1e12 / peak_flops  # the phase's flops against the matrix-core peak
    roof["hbm_frac"] = byts / sec / 1e9 / PEAK_HBM_GBS

    rec = {
        "workload": wl.name, "T": wl.T, "H": wl.H, "F": wl.F, "E": wl.E, "k": wl.k, "dtype": "f32" if f32 else "bf16",
        "pass": ("router+" if args.router else "") + ("fwd" if args.forward_only else "fwd+dx+dg")
                + ("+dW" if wl.dw and not args.forward_only else "")
                + (f"+compact(rho={wl.rho})" if wl.rho and not quota_cap else "")
                + ("+router_bwd" if args.router else "")
                + ("+recompute_h" if args.no_keep_graph else "")
                + ("+dW_overlapped" if args.overlap_dw and wl.dw and not args.forward_only else "")
                + ("" if args.gather_rows == "auto" else f"+gather_rows={args.gather_rows}")
                + ("+metric_score" if args.metric_score else "")
                + (f"+budget({args.budget_mib} MiB: cap {quota_cap})" if quota_cap else "")
                + ("+fp8_weights" if wq is not None else "")
                + ("+fp8_matrix_cores" if wt is not None else ""),
        "weights": "fp8 E4M3 (per-expert power-of-two scale), widened to bf16" if wq is not None
                   else ("fp8 E4M3 codes, K-major (per-expert power-of-two scale)" if wt is not None
                         else ("fp32" if f32 else "bf16")),
        "gemm_operands": "fp8 E4M3 x E4M3 (rows and experts scaled by powers of two), fp32 accumulate"
                         if wt is not None else ("fp32" if f32 else "bf16, fp32 accumulate"),
        "experts_with_rows": int((counts > 0).sum()), "max_rows_per_expert": int(counts.max()),
        "retained_pairs": int(kept.sum()) if kept is not None else wl.N,
        "steps": steps, "warmup": warmup, "ms_per_step": ms_per_step, "tokens_per_s": tokens_per_s,
        "tflops": step_flops / (ms_per_step * 1e-3) / 1e12,
        "mfma_frac_of_step": step_flops / (ms_per_step * 1e-3) / 1e12 / peak_flops,
        "peak_tflops": peak_flops,
        "kernel_us": {KERNEL_NAMES[kk]: kernel_ms[kk] * 1e3 for kk in gemm_kernels + router_kernels},
        "gemm_tflops": {KERNEL_NAMES[kk]: alg[kk][1] / (kernel_ms[kk] * 1e-3) / 1e12 for kk in gemm_kernels},
        "roofline": roof,
        # dispatch / combine / dO rows against the HBM peak (algorithmic bytes)
        "hbm_kernels": {KERNEL_NAMES[kk]: {"us": kernel_ms[kk] * 1e3,
                                           "GB/s": alg[kk][0] / (kernel_ms[kk] * 1e-3) / 1e9,
                                           "frac": alg[kk][0] / (kernel_ms[kk] * 1e-3) / 1e9 / PEAK_HBM_GBS}
                        for kk in hbm_kernels},
    }
    if args.router:
        # bf16 router products run on the bf16 matrix cores (roofline: bf16 MFMA peak)
        rec["router"] = {KERNEL_NAMES[kk]: {"us": kernel_ms[kk] * 1e3,
                                            "TFLOP/s": alg[kk][1] / (kernel_ms[kk] * 1e-3) / 1e12,
                                            "frac_bf16_mfma": alg[kk][1] / (kernel_ms[kk] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                            "GB/s": alg[kk][0] / (kernel_ms[kk] * 1e-3) / 1e9}
                         for kk in router_kernels}
    if dist_and_probes:
        rec["step_ms"] = step_distribution(step, stream, dev, n=max(10, min(steps, 20)))
    if args.copy_probe_mib > 0:
        # one read + one write of copy_probe_mib MiB each, outside the timed steps
        src = torch.ones(args.copy_probe_mib << 19, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if timers is not None:
        def timer(n):
            for _ in range(2):  # untimed, as before the first measurement
                step()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                step()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) * 1e3 / n
        timers[wl.name] = timer
    else:
        del L, t, logits, wq, wt
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if cpu_tokens > 0:
        if logits_host is None:  # logits of a router-weight workload: x W_r by the oracle, in fp32
            import oracle
            logits_host = oracle.router_logits(d["x"], d["W_r"]).astype(np.float32)
        rec["cpu_baseline"] = cpu_baseline(wl, d, logits_host, min(cpu_tokens, wl.T), cpu_seconds)
    return rec


# Every default run also measures these workloads (one record each under
# "configs"): the tiny fp32 layer, full fine-tuning at the Qwen3 and GLM-Air
# shapes and the compacted backward, each with a shorter run and an oracle
# sample of a token prefix (tokens, seconds of host work).
SUB_CONFIGS = {"tiny_fp32": (64, 3.0), "qwen3_ft_t4096": (64, 5.0), "glm45air_t8192": (32, 5.0),
               "qwen3_compact_t16384": (64, 5.0)}


# Their forward on the fp8 matrix cores as well (no oracle sample: the fp8
# oracle is the bf16 one's loops on decoded operands).
FP8_CONFIGS = ("glm45air_t8192", "qwen3_compact_t16384")


ROUNDS = 2  # interleaved rounds after the first measurement of every workload


def round_orders(names, rounds):
    """Workload order of each round after the first (forward) measurement:
    reversed, forward, reversed, ..."""
    return [list(reversed(names)) if r % 2 == 0 else list(names) for r in range(rounds)]


def interleaved_rounds(names, timers, steps, rounds):
    """ms per step of every workload in every round, in round_orders' order."""
    out = {n: [] for n in names}
    for order in round_orders(names, rounds):
        for n in order:
            print(f"bench: round timing {n}", file=sys.stderr, flush=True)
            out[n].append(timers[n](steps[n]))
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(no sharding, no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    from expert_grouped_gemm_top_amd import workloads as W

    wl = W.WORKLOADS[args.workload]
    assert wl.dtype == "bf16", "the headline runs a bf16 workload"
    cpu_tokens = 0 if args.no_cpu_baseline else (args.cpu_tokens or min(wl.T, 128))
    timers = {} if not args.no_configs else None
    rec = measure(wl, args, args.steps, args.warmup, cpu_tokens, 10.0, dist_and_probes=not args.no_probes,
                  timers=timers)
    out = {
        "metric": METRIC, "value": rec["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {k: rec[k] for k in ("workload", "T", "H", "F", "E", "k", "pass", "weights", "experts_with_rows",
                                       "max_rows_per_expert")},
    }
    for key in ("tflops", "mfma_frac_of_step", "kernel_us", "gemm_tflops", "roofline", "hbm_kernels", "router",
                "step_ms"):
        if key in rec:
            out[key] = rec[key]
    dev = torch.device("cuda:0")
    out["env"] = environment(dev, read_clocks=not args.no_probes)
    if not args.no_probes:
        out["probes"] = probes(dev)
    if "cpu_baseline" in rec:
        out["cpu_baseline"] = rec["cpu_baseline"]
    if not args.no_configs:
        # the other workloads, each on the default path options
        base = parse_defaults()
        out["configs"] = {}
        for name, (toks, secs) in SUB_CONFIGS.items():
            if name == wl.name:
                continue
            print(f"bench: measuring {name}", file=sys.stderr, flush=True)
            out["configs"][name] = measure(W.WORKLOADS[name], base, 10, 3, 0 if args.no_cpu_baseline else toks, secs,
                                           timers=timers)
        # the forward of the matrix-core-bound layers on the fp8 matrix cores
        fp8 = argparse.Namespace(**{**vars(base), "fp8_mma": True})
        for name in FP8_CONFIGS:
            print(f"bench: measuring {name} forward on fp8", file=sys.stderr, flush=True)
            out["configs"][name + "_fp8_fwd"] = measure(W.WORKLOADS[name], fp8, 10, 3, 0, 0.0)
        # The bf16 workloads again, interleaved: each round times every one of
        # them in turn, the order reversed every other round (the first
        # measurement above is round 0, in forward order), so that a drift of
        # the box over the run shows up as a spread across rounds instead of
        # as a difference between workloads.
        import numpy as np
        recs = {wl.name: out, **{n: out["configs"][n] for n in timers if n != wl.name}}
        first = {n: r["ms_per_step"] for n, r in recs.items()}
        rounds = interleaved_rounds(list(recs), timers, {n: (args.steps if n == wl.name else 10) for n in recs},
                                    ROUNDS)
        for n, r in recs.items():
            seq = [first[n]] + rounds[n]
            r["rounds_ms_per_step"] = seq
            r["ms_per_step_median_of_rounds"] = float(np.median(seq))
        timers.clear()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
