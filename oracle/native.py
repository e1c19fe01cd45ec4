"""Loader and build step for the plain-C FP8 encoder (oracle/c/fp8_oracle.c).

TEST INFRASTRUCTURE ONLY (CPU oracle).  The C encoder follows the same
definition as ``oracle.fp8.encode`` and exists only to make sweeps over every
float32 bit pattern affordable.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "c", "fp8_oracle.c")
LIB = os.path.join(_HERE, "c", "libfp8_oracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(LIB)
    lib.fp8o_init.restype = ctypes.c_int
    lib.fp8o_encode_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.fp8o_encode_bit_patterns.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.fp8o_quant_given_scale_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                                               ctypes.c_void_p]
    lib.fp8o_quant_grouped_scale_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                                 ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.fp8o_num_threads.restype = ctypes.c_int
    lib.fp8o_init()
    _lib = lib
    return lib


def _fmt_id(fmt) -> int:
    name = fmt if isinstance(fmt, str) else fmt.name
    return 1 if name.startswith("e5m2") else 0


def encode_f32(t: np.ndarray, fmt="e4m3") -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, dtype=np.uint8)
    load().fp8o_encode_f32(t.ctypes.data, t.size, _fmt_id(fmt), out.ctypes.data)
    return out


def encode_bit_patterns(start: int, n: int, fmt="e4m3") -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    load().fp8o_encode_bit_patterns(ctypes.c_uint32(start), n, _fmt_id(fmt), out.ctypes.data)
    return out


def quant_given_scale_f32(x: np.ndarray, s: float, fmt="e4m3") -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    load().fp8o_quant_given_scale_f32(x.ctypes.data, x.size, ctypes.c_float(s), _fmt_id(fmt), out.ctypes.data)
    return out


def quant_grouped_scale_f32(x: np.ndarray, scales: np.ndarray, inner: int, fmt="e4m3") -> np.ndarray:
    """code[i] = FMT(RN32(x[i] / scales[(i // inner) % len(scales)])) over the flat array."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    sc = np.ascontiguousarray(scales, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    load().fp8o_quant_grouped_scale_f32(x.ctypes.data, x.size, sc.ctypes.data, inner, sc.size, _fmt_id(fmt),
                                        out.ctypes.data)
    return out


def num_threads() -> int:
    return int(load().fp8o_num_threads())
