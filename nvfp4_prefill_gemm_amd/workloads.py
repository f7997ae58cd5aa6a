"""Seeded synthetic workloads: shapes and input generators.

This module is shared by the oracle side (tests, CPU baseline) and the HIP
side (tests, benchmark).  It holds no arithmetic of the NVFP4 method: it only
draws random numbers, rounds them to BF16 storage, and names shapes.

Shapes are Qwen3-style transformer linear layers, the models whose prefill
the Mix-Quant page speeds up (Section 4.1 "Models", Section 4.2 "Prefilling
Stage Speedup", Figure 4).  The page measures on real prompts and trained
weights; these seeded tensors stand in for them: activations N(0, 1) with a
few outlier channels scaled x20 (or Student-t with nu = 4 for the long
agentic prefill), weights N(0, 0.02).

Seeds follow numpy ``PCG64([config_id, layer_id, tensor_id])`` with
tensor_id 0 for activations and 1 for weights.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# (name, K = in_features, N = out_features);  y[M, N] = x[M, K] @ W[N, K]^T
QWEN3_8B_LINEARS = (("qkv", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 24576), ("down", 12288, 4096))
QWEN3_32B_LINEARS = (("qkv", 5120, 10240), ("o", 8192, 5120), ("gate_up", 5120, 51200), ("down", 25600, 5120))


@dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    M: int
    linears: tuple  # of (name, K, N)
    act_dist: str = "normal_outliers"  # or "student_t4"
    outlier_channels: int | None = None  # None: round(0.005 * K)
    out_dtype: str = "bf16"
    fused: bool = False
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # 128x256 activations with 4 outlier channels, 256x256 weights, FP32 output.
    "tiny": Workload("tiny_nvfp4_linear_128x256x256", 0, 128, (("linear", 256, 256),),
                     outlier_channels=4, out_dtype="f32"),
    # Qwen3-8B prefill linears at 8192 tokens.
    "qwen3_8b_m8192": Workload("qwen3_8b_prefill_m8192", 1, 8192, QWEN3_8B_LINEARS),
    # Same shapes, long agentic prefill at 32768 tokens, heavy-tailed activations,
    # also through the fused quantize-in-prologue GEMM.
    "qwen3_8b_m32768_t4": Workload("qwen3_8b_prefill_m32768_student_t4", 2, 32768, QWEN3_8B_LINEARS,
                                   act_dist="student_t4", fused=True),
    # Qwen3-32B prefill linears at 16384 tokens.
    "qwen3_32b_m16384": Workload("qwen3_32b_prefill_m16384", 3, 16384, QWEN3_32B_LINEARS),
}

# Phase split: NVFP4 prefill at these token counts vs BF16 decode at these batch sizes.
PHASE_SPLIT_PREFILL_M = (512, 2048, 8192, 32768)
PHASE_SPLIT_DECODE_M = (1, 8, 64)
PHASE_SPLIT_CONFIG_ID = 4


def rng(config_id: int, layer_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([config_id, layer_id, tensor_id]))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 samples to BF16 storage (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def activations(M: int, K: int, g: np.random.Generator, dist: str = "normal_outliers",
                outlier_channels: int | None = None) -> np.ndarray:
    """BF16 bits [M, K]: N(0,1) with outlier columns x20, or Student-t(4)."""
    if dist == "normal_outliers":
        x = g.standard_normal((M, K), dtype=np.float32)
        n_out = int(round(0.005 * K)) if outlier_channels is None else int(outlier_channels)
        if n_out > 0:
            cols = g.choice(K, size=n_out, replace=False)
            x[:, cols] *= np.float32(20.0)
    elif dist == "student_t4":
        x = np.empty((M, K), dtype=np.float32)
        step = max(1, (1 << 24) // max(K, 1))
        for r0 in range(0, M, step):  # chunked: standard_t draws float64
            r1 = min(M, r0 + step)
            x[r0:r1] = g.standard_t(4.0, size=(r1 - r0, K)).astype(np.float32)
    else:
        raise ValueError(dist)
    return to_bf16_bits(x)


def weights(N: int, K: int, g: np.random.Generator, std: float = 0.02) -> np.ndarray:
    """BF16 bits [N, K] ~ N(0, std^2)."""
    return to_bf16_bits(g.standard_normal((N, K), dtype=np.float32) * np.float32(std))


def layer_inputs(w: Workload, layer_id: int, M: int | None = None):
    """(A bits [M, K], W bits [N, K]) for one linear layer of a workload."""
    _, K, N = w.linears[layer_id]
    M = w.M if M is None else M
    a = activations(M, K, rng(w.config_id, layer_id, 0), w.act_dist, w.outlier_channels)
    wt = weights(N, K, rng(w.config_id, layer_id, 1))
    return a, wt


def flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K
