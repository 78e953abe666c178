"""CPU checks of bench.py's bookkeeping: the algorithmic bytes and flops that
every roofline fraction divides by, written out here term by term for the
Qwen3-30B-A3B LoRA step, and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from expert_grouped_gemm_top_amd import workloads as W  # noqa: E402


def test_algorithmic_bytes_and_flops_of_the_lora_step():
    wl = W.WORKLOADS["qwen3_lora_t128"]
    T, H, F, E, k = 128, 2048, 768, 128, 8
    assert (wl.T, wl.H, wl.F, wl.E, wl.k) == (T, H, F, E, k)
    N, b = T * k, 2
    counts = np.full(E, N // E)  # every expert with rows
    alg = bench.algorithmic(wl, counts, gathered=True)
    # gate/up: both weight matrices of every expert once, the token rows once
    # (gathered on load) plus the pair indices, h = [hg|hu] and a out
    assert alg[bench.K_GATEUP] == (2 * H * F * b * E + (T * H * b + 4 * N) + N * 2 * F * b + N * F * b,
                                   4.0 * H * F * N)
    assert alg[bench.K_GATEUP][0] == 810553344  # the figure the profiles quote
    # down: W_down once, a in, o out
    assert alg[bench.K_DOWN] == (H * F * b * E + N * F * b + N * H * b, 2.0 * H * F * N)
    # dA: W_down once, dO in, h in and dh out
    assert alg[bench.K_DA] == (H * F * b * E + N * H * b + 2 * N * 2 * F * b, 2.0 * H * F * N)
    # dX: W_gate and W_up once, dh in, dX out
    assert alg[bench.K_DX] == (2 * H * F * b * E + N * 2 * F * b + N * H * b, 4.0 * H * F * N)
    # combine: rows in, indices and weights, y out
    assert alg[bench.K_COMBINE][0] == N * H * b + 8 * N + T * H * b
    # materialized rows: x_sorted [N, H] read instead of the gathered token rows
    alg_m = bench.algorithmic(wl, counts, gathered=False)
    assert alg_m[bench.K_GATEUP][0] - alg[bench.K_GATEUP][0] == N * H * b - (T * H * b + 4 * N)


def test_algorithmic_counts_only_experts_with_rows_and_retained_rows():
    wl = W.WORKLOADS["qwen3_ft_t4096"]
    H, F, E, b = wl.H, wl.F, wl.E, 2
    counts = np.zeros(E, dtype=np.int64)
    counts[:3] = [1000, 24, 8]
    counts[3] = wl.N - counts[:3].sum()
    kept = np.minimum(counts, 256)
    R = int(kept.sum())
    alg = bench.algorithmic(wl, counts, kept)
    assert alg[bench.K_GATEUP][0] == 2 * H * F * b * 4 + wl.N * H * b + wl.N * 3 * F * b  # 4 experts with rows
    assert alg[bench.K_DX] == (2 * H * F * b * 4 + R * 2 * F * b + R * H * b, 4.0 * H * F * R)
    # dW writes every expert's gradient, with rows or not
    assert alg[bench.K_DW] == (R * (2 * H + 3 * F) * b + 3 * H * F * E * b, 6.0 * H * F * R)


def test_fp8_weights_count_one_byte_per_weight():
    wl = W.WORKLOADS["qwen3_lora_t128"]
    counts = np.full(wl.E, wl.N // wl.E)
    a16 = bench.algorithmic(wl, counts, gathered=True)
    a8 = bench.algorithmic(wl, counts, gathered=True, weight_bytes=1)
    H, F, E = wl.H, wl.F, wl.E
    assert a16[bench.K_GATEUP][0] - a8[bench.K_GATEUP][0] == 2 * H * F * E
    assert a16[bench.K_DA][0] - a8[bench.K_DA][0] == H * F * E
    assert a16[bench.K_GATEUP][1] == a8[bench.K_GATEUP][1]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_fp8_matrix_core_forward_counts_one_byte_per_operand_element():
    wl = W.WORKLOADS["glm45air_t8192"]
    H, F, T, N, E = wl.H, wl.F, wl.T, wl.N, wl.E
    counts = np.full(E, N // E)
    a = bench.algorithmic(wl, counts, gathered=True, weight_bytes=1, fp8_inputs=True)
    # gate/up: fp8 weights of every expert, fp8 token rows + pair ids + row scales, bf16 h and a out
    assert a[bench.K_GATEUP] == (2 * H * F * E + T * H + 4 * N + 4 * T + N * 2 * F * 2 + N * F * 2, 4.0 * H * F * N)
    # down: fp8 weights, fp8 a rows + their scales, bf16 o out
    assert a[bench.K_DOWN] == (H * F * E + N * F + 4 * N + N * H * 2, 2.0 * H * F * N)



def test_interleaved_rounds_reverse_the_order_every_other_round():
    """After the first measurement of every workload (forward order), the
    rounds alternate reversed / forward, and every workload is timed once per
    round with its own step count."""
    names = ["a", "b", "c"]
    assert bench.round_orders(names, 3) == [["c", "b", "a"], ["a", "b", "c"], ["c", "b", "a"]]
    calls = []
    timers = {n: (lambda m: (lambda steps: calls.append((m, steps)) or float(len(calls))))(n) for n in names}
    out = bench.interleaved_rounds(names, timers, {"a": 20, "b": 10, "c": 10}, 2)
    assert calls == [("c", 10), ("b", 10), ("a", 20), ("a", 20), ("b", 10), ("c", 10)]
    assert out == {"a": [3.0, 4.0], "b": [2.0, 5.0], "c": [1.0, 6.0]}
