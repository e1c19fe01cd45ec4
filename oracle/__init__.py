"""CPU oracle for the FP8 W8A8 scaled GEMM, its quantizers and the FP8 KV cache.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow reference that the
HIP path is checked against.  It shares no code with the HIP library and does
not import it.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import, call, link or run anything here; the
product path never does, and must fail loudly rather than fall back to it.

Modules:
  fp8    -- E4M3 / E5M2 formats, saturating round-to-nearest-even encoder,
            bf16 rounding
  w8a8   -- per-token, per-tensor and per-channel quantizers; exact GEMM
            accumulator and scaled bf16 output
  kv     -- KV-cache calibrate / quantize / dequantize / append
  blockwise -- 1 x 128 activation groups, 128 x 128 weight blocks, and the
            GEMM that scales each 128-deep partial sum by its own scales
  mx     -- MXFP8: 32-element blocks along k with power-of-two (E8M0)
            scales; the GEMM that scales each 32-deep partial sum
  norm   -- RMS normalisation (the producer the per-token quantization is
            fused into)
  attention -- decode attention over an FP8 KV cache with per-head scales
            (standard softmax; the online recurrence, as a pinned statement)
  native -- the same encoder in plain C (oracle/c/fp8_oracle.c) for sweeps
            over every float32 bit pattern; loaded from its built library
"""

from . import attention, blockwise, fp8, kv, mx, norm, w8a8  # noqa: F401
