"""Seeded synthetic inputs shared by the CPU oracle's tests and the HIP path.

This module only draws random numbers and lays them out; it holds none of the
FP8 method's arithmetic (no scaling, no FP8 rounding, no GEMM).  Both sides of
every parity check take their inputs from here, so neither side ever produces
the other's inputs.

Every tensor has its own PCG64 stream, ``numpy.random.default_rng([seed,
workload_id, tensor_id])``, so a tensor does not depend on which other tensors
were drawn before it.  Normal draws are made in float32 (``standard_normal(...,
dtype=float32)``) and then multiplied by the standard deviation in float32.
Tensors that the workload states as bf16 are rounded from those float32 values
to bf16 by round-to-nearest-even on the bit pattern, and are returned as their
uint16 bit patterns.

The shapes and value distributions follow the workloads of the FP8 pages: a
Llama-3-8B-class geometry (hidden 4096, MLP 14336, 8 KV heads of dimension 128),
N(0, 1) activations with a few outlier channels, N(0, 0.02) weights, and a
heavy-tailed Student-t(3) activation for the static-scale comparison.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "normal_f32",
    "outlier_channels",
    "tiny_w8a8",
    "decode_inputs",
    "prefill_inputs",
    "large_layer_inputs",
    "kv_inputs",
    "kv_append_inputs",
    "attention_queries",
    "STATIC_SCALE_NUM",
    "STATIC_SCALE_DEN",
]

# The static per-tensor activation scale of the large-layer workload is the
# float32 quotient of these two numbers (a calibration maximum of 120 mapped
# onto the E4M3 maximum 448, as in the static-scale example of the
# "Quantization: FP8 inference and KV-cache quantization" page).
STATIC_SCALE_NUM = 120.0
STATIC_SCALE_DEN = 448.0


def _rng(seed: int, workload: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(workload), int(tensor)])


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Input preparation only.  The draws here are finite, so no NaN handling.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    z = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    return z


def outlier_channels(rng: np.random.Generator, n_channels: int, count: int) -> np.ndarray:
    """``count`` distinct channel indices, drawn without replacement, sorted."""
    return np.sort(rng.choice(n_channels, size=count, replace=False))


def tiny_w8a8(seed: int = 0):
    """Tiny W8A8 case: X fp32 [16, 256] ~ N(0,1) with channels 3 and 77 scaled by
    50; W fp32 [512, 256] ~ N(0, 0.02)."""
    x = normal_f32(_rng(seed, 1, 0), (16, 256))
    x[:, [3, 77]] *= np.float32(50.0)
    w = normal_f32(_rng(seed, 1, 1), (512, 256), 0.02)
    return x, w


def _activation_bf16(seed: int, workload: int, m: int, k: int, n_out: int, gain: float):
    rng = _rng(seed, workload, 0)
    ch = outlier_channels(rng, k, n_out)
    x = normal_f32(rng, (m, k))
    x[:, ch] *= np.float32(gain)
    return bf16_bits_from_f32(x), ch


def decode_inputs(m: int, seed: int = 0, n: int = 14336, k: int = 4096, with_weight: bool = True):
    """Decode-shaped GEMM: X bf16 [m, k] ~ N(0,1) with 0.1% of channels
    (round(0.001 k) = 4 for k = 4096) scaled by 40; W fp32 [n, k] ~ N(0, 0.02),
    the same W for every m."""
    n_out = max(1, int(round(0.001 * k)))
    xb, ch = _activation_bf16(seed + 1000 * m, 2, m, k, n_out, 40.0)
    w = normal_f32(_rng(seed, 2, 1), (n, k), 0.02) if with_weight else None
    return xb, w, ch


def prefill_inputs(k: int, seed: int = 0, m: int = 8192, n: int = 4096, with_weight: bool = True):
    """Prefill-shaped GEMM: X bf16 [m, k] ~ N(0,1) with round(0.001 k) outlier
    channels scaled by 40; W fp32 [n, k] ~ N(0, 0.02)."""
    n_out = max(1, int(round(0.001 * k)))
    xb, ch = _activation_bf16(seed + k, 3, m, k, n_out, 40.0)
    w = normal_f32(_rng(seed + k, 3, 1), (n, k), 0.02) if with_weight else None
    return xb, w, ch


def large_layer_inputs(seed: int = 0, m: int = 4096, n: int = 28672, k: int = 8192, with_weight: bool = True):
    """Large-layer static-scale case: X bf16 [m, k] ~ Student-t(nu=3);
    W fp32 [n, k] ~ N(0, 0.02)."""
    rng = _rng(seed, 4, 0)
    x = rng.standard_t(3.0, size=(m, k)).astype(np.float32)
    w = normal_f32(_rng(seed, 4, 1), (n, k), 0.02) if with_weight else None
    return bf16_bits_from_f32(x), w


def kv_inputs(seed: int = 0, b: int = 8, s: int = 32768, h: int = 8, d: int = 128, n_out: int | None = None):
    """FP8 KV-cache case: K, V bf16 [b, s, h, d] ~ N(0,1), with 1% of the h*d
    (head, dim) channels (10 of 1024 at h=8, d=128) scaled by 20, chosen
    independently for K and V.  Returns (k_bits, v_bits, k_channels, v_channels)
    where channels are flat indices into h*d."""
    if n_out is None:
        n_out = max(1, int(round(0.01 * h * d)))
    out = []
    chans = []
    for t in (0, 1):
        rng = _rng(seed, 5, t)
        ch = outlier_channels(rng, h * d, n_out)
        x = normal_f32(rng, (b, s, h * d))
        x[:, :, ch] *= np.float32(20.0)
        out.append(bf16_bits_from_f32(x).reshape(b, s, h, d))
        chans.append(ch)
    return out[0], out[1], chans[0], chans[1]


def kv_append_inputs(k_channels, v_channels, seed: int = 0, b: int = 8, h: int = 8, d: int = 128):
    """One new token per sequence for the append path: K, V bf16 [b, h, d] with
    the same outlier channels as the cache they are appended to."""
    out = []
    for t, ch in ((2, k_channels), (3, v_channels)):
        x = normal_f32(_rng(seed, 5, t), (b, h * d))
        x[:, ch] *= np.float32(20.0)
        out.append(bf16_bits_from_f32(x).reshape(b, h, d))
    return out[0], out[1]


def attention_queries(seed: int = 0, b: int = 8, hq: int = 32, d: int = 128):
    """Decode-attention queries: q bf16 [b, hq, d] ~ N(0, 1), one new token per
    sequence and query head (hq = 32 query heads over the 8 kv heads of the
    KV-cache case: groups of 4, the Llama-3-8B-class geometry)."""
    return bf16_bits_from_f32(normal_f32(_rng(seed, 6, 0), (b, hq * d)).reshape(b, hq, d))
