"""Seeded synthetic inputs for the MoE expert layer, shared by the HIP path's
tests and benchmark and by the CPU oracle's checks.

This module holds the workload recipes only -- shapes, value distributions and
the draw order -- and none of the layer's arithmetic.  Every tensor is drawn in
float32 from its own ``numpy.random.default_rng`` stream keyed by
``[seed, tensor_tag]`` (expert weights: ``[seed, tensor_tag, e]`` per expert),
so any one expert's weights can be regenerated alone.  bf16 workloads round
every drawn tensor except the router logits to bf16 (round to nearest even)
and keep them as bf16-exact float32 arrays.

Workloads (expert shapes of Qwen3-30B-A3B and of a GLM-4.5-Air-style layer; the
pages train Qwen3-30B-A3B and name GLM4.5-106B-A12B in the LRMoE abstract):
  tiny_fp32            T=64,    H=128,  F=64,   E=8,   k=2, fp32, router W_r
  qwen3_lora_t128      T=128,   H=2048, F=768,  E=128, k=8, bf16, N(0,1) logits
  qwen3_ft_t4096       T=4096,  H=2048, F=768,  E=128, k=8, bf16, skewed logits
  glm45air_t8192       T=8192,  H=4096, F=1408, E=128, k=8, bf16, skewed logits
  qwen3_compact_t16384 T=16384, H=2048, F=768,  E=128, k=8, bf16, skewed, quota rho=1
  qwen3_decode_t1/_t8  T=1 / 8, H=2048, F=768,  E=128, k=8, bf16, N(0,1) logits
Skew: logits += b_e with b_e = 1.2*ln(1/rank_e), rank_e = e+1 (expert 0 is the
hottest), added in float32.  "N(0, s)" means standard deviation s.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    F: int
    E: int
    k: int
    dtype: str            # "f32" or "bf16": activations and weights
    router: str           # "wr": logits come from x @ W_r; "logits": drawn directly
    skew: bool            # add the per-expert bias b_e to the logits
    dw: bool              # full fine-tune (weight gradients) or LoRA (dx only)
    rho: float | None     # retention quota ratio for the compacted backward, or None

    @property
    def N(self) -> int:
        return self.T * self.k


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 64, 128, 64, 8, 2, "f32", "wr", False, True, None),
    "qwen3_lora_t128": Workload("qwen3_lora_t128", 128, 2048, 768, 128, 8, "bf16", "logits", False, False, None),
    "qwen3_ft_t4096": Workload("qwen3_ft_t4096", 4096, 2048, 768, 128, 8, "bf16", "logits", True, True, None),
    "glm45air_t8192": Workload("glm45air_t8192", 8192, 4096, 1408, 128, 8, "bf16", "logits", True, True, None),
    "qwen3_compact_t16384": Workload("qwen3_compact_t16384", 16384, 2048, 768, 128, 8, "bf16", "logits", True, True, 1.0),
    # decode-sized batches: every routed expert has one or a few rows, so the
    # layer streams k (or up to T*k) experts' weights per step
    "qwen3_decode_t1": Workload("qwen3_decode_t1", 1, 2048, 768, 128, 8, "bf16", "logits", False, False, None),
    "qwen3_decode_t8": Workload("qwen3_decode_t8", 8, 2048, 768, 128, 8, "bf16", "logits", False, False, None),
}


def custom(name="custom", T=64, H=128, F=64, E=8, k=2, dtype="bf16", router="logits", skew=False,
           dw=True, rho=None) -> Workload:
    return Workload(name, T, H, F, E, k, dtype, router, skew, dw, rho)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), kept as float32."""
    import torch  # plumbing only: its CPU cast is a round-to-nearest-even
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def skew_bias(E: int) -> np.ndarray:
    """b_e = 1.2 * ln(1 / rank_e) with rank_e = e + 1, as float32."""
    return np.array([1.2 * math.log(1.0 / (e + 1)) for e in range(E)], dtype=np.float32)


_TAGS = {"x": 0, "W_r": 1, "logits": 2, "W_gate": 3, "W_up": 4, "W_down": 5, "dy": 6}


def _normal(shape, seed, *key):
    out = np.empty(shape, np.float32)
    np.random.default_rng([seed, *key]).standard_normal(out=out, dtype=np.float32)
    return out


def expert_weights(wl: Workload, name: str, experts=None, seed: int = 0) -> np.ndarray:
    """W_gate / W_up [len(experts),H,F] or W_down [len(experts),F,H] = 0.02 N(0,1)."""
    from concurrent.futures import ThreadPoolExecutor
    experts = list(range(wl.E)) if experts is None else [int(e) for e in experts]
    shape = (wl.H, wl.F) if name in ("W_gate", "W_up") else (wl.F, wl.H)
    out = np.empty((len(experts),) + shape, np.float32)
    tag = _TAGS[name]

    def fill(i):
        g = np.random.default_rng([seed, tag, experts[i]])
        g.standard_normal(out=out[i], dtype=np.float32)
        out[i] *= np.float32(0.02)

    with ThreadPoolExecutor(8) as ex:
        list(ex.map(fill, range(len(experts))))
    return round_bf16(out) if wl.dtype == "bf16" else out


def router_weights(wl: Workload, seed: int = 0) -> np.ndarray:
    """W_r [H,E] = 0.02 N(0,1), the same draw as a "wr" workload's router (for
    running the router in front of a workload whose logits are drawn)."""
    rnd = round_bf16 if wl.dtype == "bf16" else (lambda a: a)
    return rnd(np.float32(0.02) * _normal((wl.H, wl.E), seed, _TAGS["W_r"]))


def generate(wl: Workload, seed: int = 0, weights: bool = True) -> dict:
    """Draw the workload's tensors: x [T,H], W_r [H,E] (router "wr") or logits
    [T,E], W_gate, W_up [E,H,F], W_down [E,F,H] (unless ``weights`` is False),
    dy [T,H].  float32 numpy arrays, bf16-exact for bf16 workloads."""
    T, H, E = wl.T, wl.H, wl.E
    rnd = round_bf16 if wl.dtype == "bf16" else (lambda a: a)
    out = {"x": rnd(_normal((T, H), seed, _TAGS["x"]))}
    if wl.router == "wr":
        out["W_r"] = rnd(np.float32(0.02) * _normal((H, E), seed, _TAGS["W_r"]))
    else:
        logits = _normal((T, E), seed, _TAGS["logits"])
        if wl.skew:
            logits = (logits + skew_bias(E)[None, :]).astype(np.float32)
        out["logits"] = logits
    if weights:
        for name in ("W_gate", "W_up", "W_down"):
            out[name] = expert_weights(wl, name, None, seed)
    out["dy"] = rnd(_normal((T, H), seed, _TAGS["dy"]))
    return out
