"""Seeded synthetic inputs for the W4A8 GEMM workloads.

This module draws random FP16 activations and weights with the shapes and
value distributions of the workloads; it holds none of the quantization or
GEMM arithmetic.  Both the CPU oracle checks and the GPU library runs take
their inputs from here.

Recipe (seed 0 unless stated):
  * three independent streams from ``np.random.SeedSequence(seed).spawn(3)``:
    activations, outlier-channel choice, weights;
  * X = standard normal FP32 [M, K]; a set of outlier input channels is scaled
    by 20 (channels {3, 77} for the tiny and attention-projection shapes,
    otherwise ceil(0.5% of K) channels drawn without replacement); then cast
    to FP16;
  * W = 0.02 * standard normal FP32 [N, K], cast to FP16;
  * gamma (the weight of the normalization before a quantized layer)
    = 1 + 0.1 * standard normal FP32 [K], cast to FP16, from a fourth stream.
The weight stream does not depend on M, so workloads that share (N, K) share
W, and a smaller M takes the first rows of the largest M's draw.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get_workload", "make_x", "make_w", "make_gamma", "make_inputs"]


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    group_size: int  # 128 = g128 progressive, 0 = per-channel W4
    outliers: str    # "fixed" -> channels {3, 77}; "frac" -> ceil(0.5% K) random
    desc: str

    @property
    def ops(self) -> int:
        return 2 * self.M * self.N * self.K


# Shapes follow the LLM layers the pages evaluate (Llama-2-7B, Llama-3-8B,
# Llama-2-70B-like, Qwen1.5-72B); the values are synthetic.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 16, 256, 256, 128, "fixed", "tiny W4A8 GEMM M16 K256 N256 g128"),
        Workload("attn_proj", 256, 4096, 4096, 128, "fixed",
                 "Llama-2-7B attention projection M256 K4096 N4096 g128"),
        Workload("attn_qkv", 256, 4096, 12288, 128, "fixed",
                 "Llama-2-7B fused QKV projection M256 K4096 N12288 g128"),
        Workload("ffn_gateup_prefill", 1024, 4096, 28672, 128, "frac",
                 "Llama-3-8B FFN gate+up at prefill M1024 K4096 N28672 g128"),
        Workload("ffn_down_prefill", 1024, 14336, 4096, 128, "frac",
                 "Llama-3-8B FFN down at prefill M1024 K14336 N4096 g128"),
        Workload("decode_m1", 1, 8192, 28672, 128, "frac",
                 "Llama-70B-like FFN decode M1 K8192 N28672 g128"),
        Workload("decode_m16", 16, 8192, 28672, 128, "frac",
                 "Llama-70B-like FFN decode M16 K8192 N28672 g128"),
        Workload("decode_m64", 64, 8192, 28672, 128, "frac",
                 "Llama-70B-like FFN decode M64 K8192 N28672 g128"),
        Workload("ffn_large_g128", 4096, 8192, 24576, 128, "frac",
                 "Qwen1.5-72B-like FFN large batch M4096 K8192 N24576 g128"),
        Workload("ffn_large_perchannel", 4096, 8192, 24576, 0, "frac",
                 "Qwen1.5-72B-like FFN large batch M4096 K8192 N24576 per-channel W4"),
    ]
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.default_rng(s) for s in ss.spawn(3)]


def outlier_channels(K: int, mode: str, seed: int = 0) -> np.ndarray:
    """Input channels whose activations are scaled by 20."""
    if mode == "fixed":
        return np.array([c for c in (3, 77) if c < K], dtype=np.int64)
    _, ro, _ = _streams(seed)
    cnt = min(K, math.ceil(0.005 * K))
    return np.sort(ro.choice(K, cnt, replace=False)).astype(np.int64)


def make_x(M: int, K: int, mode: str = "frac", seed: int = 0) -> np.ndarray:
    """FP16 activations [M, K]: N(0,1) with outlier channels x20."""
    rx, _, _ = _streams(seed)
    X32 = rx.standard_normal((M, K), dtype=np.float32)
    cols = outlier_channels(K, mode, seed)
    if cols.size:
        X32[:, cols] *= np.float32(20.0)
    return X32.astype(np.float16)


def make_w(N: int, K: int, seed: int = 0) -> np.ndarray:
    """FP16 weights [N, K]: N(0, 0.02)."""
    _, _, rw = _streams(seed)
    W32 = rw.standard_normal((N, K), dtype=np.float32)
    W32 *= np.float32(0.02)
    return W32.astype(np.float16)


def make_gamma(K: int, seed: int = 0) -> np.ndarray:
    """FP16 normalization weight [K]: 1 + 0.1 N(0, 1) (a fourth stream; the
    first three are those of ``_streams``)."""
    rg = np.random.default_rng(np.random.SeedSequence(seed).spawn(4)[3])
    g32 = np.float32(1.0) + np.float32(0.1) * rg.standard_normal(K, dtype=np.float32)
    return g32.astype(np.float16)


def make_inputs(w: Workload | str, seed: int = 0, M: int | None = None):
    """(X fp16 [M,K], W fp16 [N,K]) for a workload; ``M`` may override the row count."""
    if isinstance(w, str):
        w = get_workload(w)
    m = w.M if M is None else M
    return make_x(m, w.K, w.outliers, seed), make_w(w.N, w.K, seed)
