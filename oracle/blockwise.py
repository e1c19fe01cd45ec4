"""Block-wise scaled FP8 quantization and GEMM, written out from the pages (CPU oracle).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module;
only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.

What is computed
----------------
Granularity (FP8 Quantization notebook, "Granularity": per-tensor, per-channel,
and per-block -- one scale per 128 x 128 tile of W, from the tile's absolute
maximum; FP8 Inference Explained, in depth -- "Scales and their granularity":
finer granularity contains outliers to fewer values).

* Weights: one scale per 128 x 128 block of W [N, K]:
  s_w[b, g] = RN32(amax(W[128 b : 128 b + 128, 128 g : 128 g + 128]) / 448).
  The last row block is shorter when N % 128 != 0.
* Activations: one scale per token and 128-element group along k,
  s_a[m, g] = RN32(amax(X[m, 128 g : 128 g + 128]) / 448) (reading: the
  per-token rule of "Inside a quantized linear layer" applied to each 128-deep
  block of the reduction, the block the weight scales and the FP32 promotion use).
* Codes: q = E4M3(RN32(x / s)) with the scale of the element's group, the
  same rounding and saturation as the per-token and per-channel quantizers
  (oracle/w8a8.py), and the same reading for an all-zero group (scale 1.0).
* GEMM: block-wise scales vary along k, so each 128-deep partial sum is
  multiplied by its own scales before the partials are added ("Inside a
  quantized linear layer", the paragraph on why per-token / per-channel scales
  are cheap and block-wise ones need purpose-built GEMMs; "Quantization: FP8
  inference and KV-cache quantization", on moving each 128-element partial sum
  to FP32):
      y[m, n] = sum_g s_a[m, g] * s_w[n // 128, g] * P_g[m, n],
      P_g[m, n] = sum_{k in group g} dec(a_q[m, k]) * dec(w_q[n, k]).

Exactness of the reference: every E4M3 x E4M3 product is a multiple of 2^-18
below 2^18 in magnitude, so P_g (128 products) is exact in float64; the scale
product s_a * s_w of two float32 values is exact in float64 (48 significant
bits); the remaining multiply and the sum over groups are float64 roundings,
(G + 1) * 2^-53 relative to the sum of absolute terms at worst -- far below the
float32 accumulator tolerance and a bf16 ulp.  The bf16 output is that value
rounded once to bf16.
"""

from __future__ import annotations

import numpy as np

from .fp8 import E4M3, bf16_round_bits, decode, encode
from .w8a8 import f32_div

__all__ = ["GROUP", "act_group_scales", "quant_act_blockwise", "weight_block_scales", "quant_weight_blockwise",
           "blockwise_partials", "gemm_blockwise_exact", "gemm_blockwise_abs", "gemm_blockwise_bf16"]

GROUP = 128


def _scale_from_amax(amax: np.ndarray) -> np.ndarray:
    s = f32_div(np.asarray(amax, np.float32), np.float32(E4M3.max_finite))
    return np.where(s == 0, np.float32(1.0), s).astype(np.float32)


def act_group_scales(x: np.ndarray) -> np.ndarray:
    """s_a [M, K / 128] from X [M, K] (float32 values)."""
    x = np.asarray(x, np.float32)
    M, K = x.shape
    assert K % GROUP == 0
    return _scale_from_amax(np.abs(x).reshape(M, K // GROUP, GROUP).max(axis=-1))


def quant_act_blockwise(x: np.ndarray):
    """Dynamic 1 x 128 activation quantization: returns (codes uint8 [M, K], s_a float32 [M, K / 128])."""
    x = np.asarray(x, np.float32)
    M, K = x.shape
    s = act_group_scales(x)
    t = f32_div(x, np.repeat(s, GROUP, axis=1))
    return encode(t, E4M3), s


def weight_block_scales(w: np.ndarray) -> np.ndarray:
    """s_w [ceil(N / 128), K / 128] from W [N, K] (float32 values)."""
    w = np.asarray(w, np.float32)
    N, K = w.shape
    assert K % GROUP == 0
    nb = -(-N // GROUP)
    a = np.zeros((nb * GROUP, K), np.float32)
    a[:N] = np.abs(w)  # padding rows are 0 and never raise a block maximum
    return _scale_from_amax(a.reshape(nb, GROUP, K // GROUP, GROUP).max(axis=(1, 3)))


def quant_weight_blockwise(w: np.ndarray):
    """128 x 128 block weight quantization: returns (codes uint8 [N, K], s_w float32 [ceil(N/128), K/128])."""
    w = np.asarray(w, np.float32)
    N, K = w.shape
    s = weight_block_scales(w)
    per_elem = np.repeat(np.repeat(s, GROUP, axis=0)[:N], GROUP, axis=1)
    return encode(f32_div(w, per_elem), E4M3), s


def blockwise_partials(a_q: np.ndarray, w_q: np.ndarray) -> np.ndarray:
    """P [G, M, N]: the exact 128-deep partial dot products (float64)."""
    a = decode(a_q, E4M3)
    w = decode(w_q, E4M3)
    M, K = a.shape
    G = K // GROUP
    return np.stack([a[:, g * GROUP:(g + 1) * GROUP] @ w[:, g * GROUP:(g + 1) * GROUP].T for g in range(G)])


def _scale_grid(s_a: np.ndarray, s_w: np.ndarray, N: int) -> np.ndarray:
    """[G, M, N] products s_a[m, g] * s_w[n // 128, g] (float64, exact)."""
    sa = np.asarray(s_a, np.float64)            # [M, G]
    sw = np.asarray(s_w, np.float64)            # [NB, G]
    sw_n = np.repeat(sw, GROUP, axis=0)[:N]     # [N, G]
    return sa.T[:, :, None] * sw_n.T[:, None, :]


def gemm_blockwise_exact(a_q, s_a, w_q, s_w) -> np.ndarray:
    """y [M, N] = sum_g s_a[m, g] s_w[n // 128, g] P_g[m, n] (float64)."""
    P = blockwise_partials(a_q, w_q)
    return (_scale_grid(s_a, s_w, w_q.shape[0]) * P).sum(axis=0)


def gemm_blockwise_abs(a_q, s_a, w_q, s_w) -> np.ndarray:
    """sum_g |s_a s_w| sum_k |a w| -- the scale of the accumulator tolerance."""
    a = np.abs(decode(a_q, E4M3))
    w = np.abs(decode(w_q, E4M3))
    G = a.shape[1] // GROUP
    P = np.stack([a[:, g * GROUP:(g + 1) * GROUP] @ w[:, g * GROUP:(g + 1) * GROUP].T for g in range(G)])
    return (np.abs(_scale_grid(s_a, s_w, w_q.shape[0])) * P).sum(axis=0)


def gemm_blockwise_bf16(a_q, s_a, w_q, s_w):
    """Y = bf16(y_exact); returns (y_bits uint16 [M, N], y_exact float64)."""
    y = gemm_blockwise_exact(a_q, s_a, w_q, s_w)
    return bf16_round_bits(y), y
