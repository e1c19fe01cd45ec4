"""FP8 KV-cache calibrate / quantize / dequantize / append (CPU oracle).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module;
only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.

The cache stores K and V in E4M3 or E5M2 with one float32 scale per attention
head (per-head scales "require calibration"; without calibration every scale
is 1.0) -- FP8 Inference Explained, in depth, "FP8 KV cache"; "Quantization:
FP8 inference and KV-cache quantization", "Turning it on in an engine".

Layout: a cache tensor is [B, S, H, D] (batch, sequence, kv head, head dim),
dense, head dim contiguous.

* calibrate: s_h = RN32(amax_h / FMAX), amax_h over all (b, s, d) of head h,
  FMAX = 448 (E4M3) or 57,344 (E5M2); a head whose amax is 0 (or whose quotient
  underflows to 0) gets 1.0.
* quantize:  code = FMT(RN32(x / s_h)), saturating.
* dequantize: bf16(RN32(dec(code) * s_h)): the float32 product of the decoded
  value and the scale, rounded to bf16 by round-to-nearest-even.
* append: quantize one new token per sequence [B, H, D] with the existing
  scales and write it at cache[b, pos_b, :, :]; nothing else changes.
"""

from __future__ import annotations

import numpy as np

from .fp8 import Fp8Format, bf16_round_bits, decode, encode, f32_from_bf16_bits
from .w8a8 import f32_div

__all__ = ["kv_calibrate", "kv_quant", "kv_dequant", "kv_append"]


def _as_f32(kv_bits: np.ndarray) -> np.ndarray:
    return f32_from_bf16_bits(kv_bits)


def kv_calibrate(kv_bits: np.ndarray, fmt: Fp8Format) -> np.ndarray:
    """Per-head scales [H] float32 of a bf16 tensor [B, S, H, D] (uint16 bits)."""
    b, s, h, d = kv_bits.shape
    x = _as_f32(kv_bits)
    amax = np.abs(x).max(axis=(0, 1, 3))
    sc = f32_div(amax, np.float32(fmt.max_finite))
    return np.where(sc == 0, np.float32(1.0), sc).astype(np.float32)


def kv_quant(kv_bits: np.ndarray, head_scales: np.ndarray, fmt: Fp8Format) -> np.ndarray:
    """bf16 [B, S, H, D] -> codes uint8 [B, S, H, D]."""
    x = _as_f32(kv_bits)
    s = np.asarray(head_scales, dtype=np.float32).reshape(1, 1, -1, 1)
    return encode(f32_div(x, s), fmt)


def kv_dequant(codes: np.ndarray, head_scales: np.ndarray, fmt: Fp8Format) -> np.ndarray:
    """codes uint8 [B, S, H, D] -> bf16 bits uint16 [B, S, H, D]."""
    v = decode(codes, fmt).astype(np.float32)          # exact: FP8 values fit float32
    s = np.asarray(head_scales, dtype=np.float32).reshape(1, 1, -1, 1)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = np.multiply(v, s, dtype=np.float32)     # RN32(dec * s)
    return bf16_round_bits(prod)


def kv_append(cache: np.ndarray, kv_new_bits: np.ndarray, pos: np.ndarray, head_scales: np.ndarray,
              fmt: Fp8Format) -> np.ndarray:
    """Returns a copy of cache [B, S_cap, H, D] with token b written at pos[b]."""
    out = np.array(cache, copy=True)
    codes = kv_quant(kv_new_bits[:, None], head_scales, fmt)[:, 0]
    for b, p in enumerate(np.asarray(pos)):
        out[b, int(p)] = codes[b]
    return out
