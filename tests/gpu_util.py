"""Helpers shared by the GPU parity tests (test code only)."""

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_codes_equal(got: np.ndarray, want: np.ndarray, what: str, nan_ok_mask=None):
    """Bit-exact comparison of FP8 codes.  Where nan_ok_mask is set the input was
    NaN: any NaN code of the format is a correct encoding (the pages fix no NaN
    sign), so only NaN-ness is compared there."""
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    diff = got != want
    if nan_ok_mask is not None:
        diff &= ~nan_ok_mask
    if diff.any():
        idx = np.argwhere(diff)[:8]
        detail = ", ".join(f"{tuple(i)}: got {got[tuple(i)]:#04x} want {want[tuple(i)]:#04x}" for i in idx)
        raise AssertionError(f"{what}: {int(diff.sum())} of {diff.size} codes differ; first: {detail}")
