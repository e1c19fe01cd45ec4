"""FP8 W8A8 quantizers and scaled GEMM, written out from the pages (CPU oracle).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module;
only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.

What is computed
----------------
Scale convention (FP8 Inference Explained, in depth -- "Scales and their
granularity"; the "Quantization: FP8 inference and KV-cache quantization" page,
"Dynamic scales or static scales"): the stored scale is the *dequantization*
factor s = amax / 448, a value is encoded as round(x / s) and reads back as
s * code.  Scales are float32 ("Inside a quantized linear layer": one FP32
scale per output channel; the FP8 Quantization notebook's scaled-matmul call
takes float32 scales).

Reading of the arithmetic: every intermediate is one IEEE-754 binary32
operation rounded to nearest even, with no fused multiply-add and no flush to
zero; so s = RN32(amax / 448) and the value handed to the FP8 encoder is the
float32 quotient RN32(x / s).  numpy's float32 division is that operation.

* Dynamic per-token activation quantization: one scale per row of X from the
  row's absolute maximum, so the row maximum lands on 448 ("Dynamic scales or
  static scales"; "Inside a quantized linear layer": a small kernel finds each
  token's amax, divides and casts to E4M3).
* Static per-tensor quantization: a given scale s; values beyond 448 s saturate
  ("Dynamic scales or static scales": 180 / s = 672 is clamped to 448).
* Per-output-channel weight quantization: the dynamic row rule applied to the
  rows of W [N, K], done once offline (symmetric round-to-nearest, no
  calibration data).
* Scaled GEMM: both scale vectors are constant along k, so
  y_ij = s_a,i * s_w,j * sum_k a_q,ik * w_q,jk ("Inside a quantized linear
  layer", the paragraph on why the scales are cheap), with the FP8 x FP8
  products accumulated in FP32 and the result written as BF16 (FP8
  Quantization notebook, "How FP8 Matmul Works at the Hardware Level").

The oracle's accumulator is the *exact* sum: every E4M3 x E4M3 product is an
integer multiple of 2^-18 of magnitude below 2^18, so float64 sums of up to
2^17 such products are exact in any order, and a float64 matrix product of the
decoded values is the exact dot product.  The BF16 output is the exact
accumulator times both scales, evaluated in float64, rounded once to BF16.

Readings where the pages are silent: a row whose amax is 0 (or whose amax/448
underflows to 0 in float32) gets the scale 1.0 (the unit-scale default of the
KV-cache documentation summarised on the "Quantization: FP8 inference and
KV-cache quantization" page), so its codes are signed zeros.
"""

from __future__ import annotations

import numpy as np

from .fp8 import E4M3, Fp8Format, bf16_round_bits, decode, encode

__all__ = ["f32_div", "row_scales", "quant_rows_dynamic", "quant_per_token", "quant_weight_per_channel",
           "quant_static", "gemm_acc_exact", "gemm_abs_sum", "scaled_gemm_bf16", "scaled_gemm_f64",
           "relative_frobenius"]


def f32_div(a, b) -> np.ndarray:
    """IEEE binary32 quotient RN32(a / b) of float32 operands."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore", under="ignore"):
        return np.divide(a, b, dtype=np.float32)


def row_scales(x: np.ndarray, fmt: Fp8Format = E4M3) -> np.ndarray:
    """s_i = RN32(max_k |x_ik| / FMAX) per row, 1.0 where that is 0."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    s = f32_div(amax, np.float32(fmt.max_finite))
    return np.where(s == 0, np.float32(1.0), s).astype(np.float32)


def quant_rows_dynamic(x: np.ndarray, fmt: Fp8Format = E4M3):
    """Row-wise dynamic quantization: returns (codes uint8 [R, C], scales float32 [R])."""
    x = np.asarray(x, dtype=np.float32)
    s = row_scales(x, fmt)
    t = f32_div(x, s[..., None])
    return encode(t, fmt), s


def quant_per_token(x: np.ndarray):
    """Dynamic per-token E4M3 quantization of activations X [M, K] (float32 values)."""
    return quant_rows_dynamic(x, E4M3)


def quant_weight_per_channel(w: np.ndarray):
    """Offline per-output-channel E4M3 quantization of W [N, K] (float32 values)."""
    return quant_rows_dynamic(w, E4M3)


def quant_static(x: np.ndarray, scale, fmt: Fp8Format = E4M3) -> np.ndarray:
    """Given-scale quantization: code = FMT(RN32(x / s)), saturating."""
    t = f32_div(np.asarray(x, dtype=np.float32), np.float32(scale))
    return encode(t, fmt)


def gemm_acc_exact(a_q: np.ndarray, w_q: np.ndarray) -> np.ndarray:
    """Exact accumulator acc_ij = sum_k dec(a_ik) dec(w_jk), float64 [M, N]."""
    a = decode(a_q, E4M3)
    w = decode(w_q, E4M3)
    assert a_q.shape[1] < (1 << 17), "float64 exactness bound"
    return a @ w.T


def gemm_abs_sum(a_q: np.ndarray, w_q: np.ndarray) -> np.ndarray:
    """sum_k |dec(a_ik) dec(w_jk)| (exact, float64 [M, N]); the tolerance scale."""
    return np.abs(decode(a_q, E4M3)) @ np.abs(decode(w_q, E4M3)).T


def scaled_gemm_f64(acc: np.ndarray, s_a, s_w) -> np.ndarray:
    """acc * s_a,i * s_w,j in float64 (exact for these magnitudes up to one rounding)."""
    s_a = np.asarray(s_a, dtype=np.float64)
    s_w = np.asarray(s_w, dtype=np.float64)
    if s_a.ndim == 0 or s_a.size == 1:
        s_a = np.full(acc.shape[0], float(np.ravel(s_a)[0]))
    return acc * s_a[:, None] * s_w[None, :]


def scaled_gemm_bf16(a_q, s_a, w_q, s_w):
    """Y = bf16(diag(s_a) (A_q W_q^T) diag(s_w)); returns (y_bits uint16, acc float64)."""
    acc = gemm_acc_exact(a_q, w_q)
    return bf16_round_bits(scaled_gemm_f64(acc, s_a, s_w)), acc


def relative_frobenius(approx: np.ndarray, ref: np.ndarray) -> float:
    """||approx - ref||_F / ||ref||_F (FP8 Quantization notebook, the error metric of
    its quantize/restore example)."""
    approx = np.asarray(approx, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(approx - ref) / np.linalg.norm(ref))
