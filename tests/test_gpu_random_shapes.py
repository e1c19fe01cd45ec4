"""Seeded random shapes through the GEMM paths whose tiling changed most often:
fp8_scaled_gemm on bf16 (every fourth case fp32) activations quantized inside the call (per token: the
16-row-tile quantizer into the fragment order above 32 rows; per tensor: the
fragment-order static quantizer) and the block-wise GEMM in both accumulation
modes.  Every output is compared with the oracle by the checkers of the
per-shape tests (test_gpu_gemm.gemm_case, test_gpu_blockwise.run_case), with the
same tolerances; outputs start as NaN, so a tile left unwritten fails."""

import numpy as np
import pytest

from gpu_util import require_gpu
from workloads import bf16_bits_from_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _shape(rng):
    m = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 300)), int(rng.integers(300, 700))]))
    n = int(rng.integers(1, 700))
    k = 128 * int(rng.integers(1, 17))
    return m, n, k


def _inputs(rng, m, n, k, fp32=False):
    x = (rng.standard_t(4, (m, k)) * rng.uniform(0.5, 4)).astype(np.float32)
    x[:, rng.integers(0, k, 2)] *= 25
    w = (rng.standard_normal((n, k)) * 0.03).astype(np.float32)
    return (x if fp32 else bf16_bits_from_f32(x)), w


@pytest.mark.parametrize("seed", range(32))
def test_scaled_gemm_random_shapes(seed):
    from test_gpu_gemm import gemm_case
    rng = np.random.default_rng(1000 + seed)
    m, n, k = _shape(rng)
    xb, w = _inputs(rng, m, n, k, fp32=(seed % 4 == 1))   # fp32 activations every fourth case
    accum = ("exact", "mfma_fp8")[seed % 2]
    layout = ("packed", "row_major")[(seed // 2) % 2]
    static = np.float32(rng.uniform(0.005, 0.05)) if seed % 3 == 0 else None
    gemm_case(xb, w, accum=accum, static=static, layout=layout,
              what=f"random {m}x{n}x{k} {accum} {layout} {'static' if static is not None else 'per-token'}")


@pytest.mark.parametrize("seed", range(16))
def test_blockwise_random_shapes(seed):
    from test_gpu_blockwise import run_case
    rng = np.random.default_rng(2000 + seed)
    m, n, k = _shape(rng)
    xb, w = _inputs(rng, m, n, k)
    layout = ("packed", "row_major")[seed % 2]
    kmajor = seed % 4 >= 2
    for accum in ("exact", "mfma_fp8"):
        run_case(xb, w, accum=accum, w_layout=layout, a_layout=layout, kmajor=kmajor,
                 what=f"random block-wise {m}x{n}x{k} {accum} {layout} kmajor={kmajor}")
