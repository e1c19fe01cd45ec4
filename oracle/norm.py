"""RMS normalisation, the producer the per-token quantization is fused into (CPU oracle).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module;
only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.

The pages say that engines fuse the per-token amax reduction into the kernel
that produces the activations ("FP8 Inference Explained, in depth" --
"Scales and their granularity").  Reading: that producer is the RMS
normalisation in front of the linear layers of the decoder-only transformers
the pages discuss.  The pages do not define it; this is the standard
definition (root mean square layer normalisation):

    y_k = x_k / sqrt(mean_k(x_k^2) + eps) * g_k

evaluated in float64 from the exact inputs.  Its fp32 evaluation on the GPU
differs from this by a few float32 roundings (a tolerance in the tests); the
quantization of the normalised rows is the per-token rule of oracle/w8a8.py.
"""

from __future__ import annotations

import numpy as np

__all__ = ["rmsnorm"]


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """y [M, K] float64: each row divided by its root mean square (plus eps) times g."""
    x = np.asarray(x, np.float64)
    g = np.asarray(g, np.float64)
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(np.float32(eps))) * g
