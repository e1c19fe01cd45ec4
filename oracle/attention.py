"""Decode attention over an FP8 KV cache, written out from the pages (CPU oracle).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module;
only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.

What is computed
----------------
One decode step: every sequence b has one new query token q[b, h, :] per query
head h and attends over the first L[b] positions of its cached keys and values.

* The cache holds FP8 codes with one scale per kv head, and a backend that does
  not compute in FP8 reads it back as code value times scale and computes in
  higher precision (FP8 Inference Explained, in depth -- "FP8 KV cache": per-
  tensor or per-attention-head scales; other backends store FP8 and compute in
  higher precision).  Here: K[t, g, :] = dec(kq[b, t, g, :]) * s_K[g], and the
  same for V, exactly (a code value has at most 4 significant bits and the scale
  24, so the float64 product is exact).
* Grouped query heads: query head h reads kv head h // (Hq / Hkv).
* Attention is the standard softmax attention ("FlashAttention v1/v2/v3/v4"
  post, blog.lo0.es -- "The trick that made it all possible: online softmax":
  the softmax of x is exp(x_i - m) / sum_j exp(x_j - m) with m the maximum):
      s_t = scale * sum_d q[d] K[t, d],   p_t = softmax(s)_t,   o = sum_t p_t V[t, :],
  with scale = 1 / sqrt(D) unless given.  An empty sequence (L[b] == 0) has no
  softmax; its output is 0 (reading).
* The same post states that the online recurrence (running maximum and running
  sum, partial outputs rescaled by exp(m_old - m_new)) gives exactly the standard
  result; `attention_online` takes that recurrence block by block, in the post's
  order and notation, so that the statement itself is pinned by the tests.

Everything is float64 from exact inputs (bf16 queries, exact dequantized K/V);
the bf16 output is that value rounded once.
"""

from __future__ import annotations

import numpy as np

from .fp8 import E4M3, Fp8Format, bf16_round_bits, decode

__all__ = ["attention_decode", "attention_decode_bf16", "attention_abs_weight", "attention_online"]


def _slices(q, kq, vq, s_k, s_v, lengths, fmt, scale, heads=None):
    """Yield (b, h, s, V) per requested (b, h): the scaled scores s [L] and the
    dequantized values V [L, D] of query head h's kv head, one slice at a time
    (so that long caches are never dequantized whole)."""
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    Hkv = kq.shape[2]
    assert Hq % Hkv == 0 and kq.shape[3] == D and vq.shape == kq.shape
    G = Hq // Hkv
    sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
    pairs = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    for b, h in pairs:
        L = int(lengths[b])
        if L == 0:
            yield b, h, None, None
            continue
        g = h // G
        K = decode(kq[b, :L, g, :], fmt) * np.float64(s_k[g])
        V = decode(vq[b, :L, g, :], fmt) * np.float64(s_v[g])
        yield b, h, sc * (K @ q[b, h]), V


def attention_decode(q, kq, vq, s_k, s_v, lengths, fmt: Fp8Format = E4M3, scale=None, heads=None) -> np.ndarray:
    """o [B, Hq, D] float64: softmax attention of each query head over the first
    lengths[b] cached positions of its kv head (only the (b, h) pairs in
    `heads`, if given; the rest stay 0)."""
    out = np.zeros(np.shape(q))
    for b, h, s, V in _slices(q, kq, vq, s_k, s_v, lengths, fmt, scale, heads):
        if s is None:
            continue
        e = np.exp(s - s.max())
        out[b, h] = (e / e.sum()) @ V
    return out


def attention_abs_weight(q, kq, vq, s_k, s_v, lengths, fmt: Fp8Format = E4M3, scale=None, heads=None) -> np.ndarray:
    """sum_t p_t |V[t, d]| per output (float64 [B, Hq, D]): the magnitude the
    output tolerance is relative to."""
    out = np.zeros(np.shape(q))
    for b, h, s, V in _slices(q, kq, vq, s_k, s_v, lengths, fmt, scale, heads):
        if s is None:
            continue
        e = np.exp(s - s.max())
        out[b, h] = (e / e.sum()) @ np.abs(V)
    return out


def attention_decode_bf16(q, kq, vq, s_k, s_v, lengths, fmt: Fp8Format = E4M3, scale=None, heads=None):
    """(bf16 bit patterns [B, Hq, D], float64 values) of the exact output rounded once."""
    o = attention_decode(q, kq, vq, s_k, s_v, lengths, fmt, scale, heads)
    return bf16_round_bits(o), o


def attention_online(q, kq, vq, s_k, s_v, lengths, block: int, fmt: Fp8Format = E4M3, scale=None) -> np.ndarray:
    """The same attention by the online recurrence over blocks of `block`
    positions: m^(t+1) = max(m^(t), m_new), l^(t+1) = exp(m^(t) - m^(t+1)) l^(t)
    + sum_new exp(x_j - m^(t+1)), accumulated outputs rescaled by the same
    factor, divided by the final l at the end."""
    out = np.zeros(np.shape(q))
    for b, h, s, V in _slices(q, kq, vq, s_k, s_v, lengths, fmt, scale):
        if s is None:
            continue
        m, l, acc = -np.inf, 0.0, np.zeros(V.shape[1])
        for t0 in range(0, len(s), block):
            x = s[t0:t0 + block]
            m_new = max(m, x.max())
            alpha = np.exp(m - m_new) if np.isfinite(m) else 0.0
            e = np.exp(x - m_new)
            l = alpha * l + e.sum()
            acc = alpha * acc + e @ V[t0:t0 + block]
            m = m_new
        out[b, h] = acc / l
    return out
