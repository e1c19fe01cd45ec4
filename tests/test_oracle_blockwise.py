"""Pins of the block-wise oracle (oracle/blockwise.py) to facts that do not come
from the oracle itself: the pages' worked outlier row, the reduction to the
per-token / per-channel GEMM when all group scales of a row (block) coincide,
exact rational arithmetic on a tiny case, and the placement of every scale."""

from fractions import Fraction

import numpy as np

from conftest import parse_num, read_golden
from oracle import blockwise as bw
from oracle import fp8, w8a8


def _golden_dict(name):
    return {r[0]: [parse_num(v) for v in r[1:]] for r in read_golden(name)}


def test_outlier_row_inside_one_group():
    """The pages' one-scale row (FP8 Inference Explained, in depth -- "The numbers
    in one byte") placed in group 1 of a 3-group row reads back as printed; the
    other groups keep scales of their own."""
    g = _golden_dict("row_outlier_example.txt")
    vals = np.float32(g["input"])
    x = np.zeros((1, 3 * 128), np.float32)
    x[0, 128:128 + len(vals)] = vals
    x[0, 5] = 3.0          # group 0: amax 3
    x[0, 300] = -0.75      # group 2: amax 0.75
    q, s = bw.quant_act_blockwise(x)
    assert s.shape == (1, 3)
    assert s[0, 1] == np.float32(400.0) / np.float32(448.0)
    assert s[0, 0] == np.float32(3.0) / np.float32(448.0)
    assert s[0, 2] == np.float32(0.75) / np.float32(448.0)
    readback = fp8.decode(q[0, 128:128 + len(vals)]) * np.float64(s[0, 1])
    assert np.round(readback, 4).tolist() == g["readback"]
    # each group's maximum lands on the top code
    assert q[0, 5] == 0x7E and q[0, 128 + len(vals) - 1] == 0x7E and q[0, 300] == 0xFE


def test_all_zero_group_has_unit_scale():
    x = np.zeros((2, 256), np.float32)
    x[1, 200] = 1.0
    q, s = bw.quant_act_blockwise(x)
    assert s[0].tolist() == [1.0, 1.0] and s[1, 0] == 1.0
    assert (q[0] == 0).all()


def test_weight_block_maxima_and_ragged_last_block():
    """Each 128 x 128 block's maximum is a power-of-two multiple of 448, so each
    block scale is that power of two exactly and the maximum encodes as 448; the
    last row block (N = 300) has 44 rows."""
    N, K = 300, 256
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((N, K)) * 1e-3).astype(np.float32)
    expo = {}
    for b in range(3):
        for gk in range(2):
            e = int(rng.integers(-8, 4))
            expo[(b, gk)] = e
            r = min(128 * b + int(rng.integers(0, 44)), N - 1)
            c = 128 * gk + int(rng.integers(0, 128))
            w[r, c] = np.float32(448.0 * 2.0 ** e)
    q, s = bw.quant_weight_blockwise(w)
    assert s.shape == (3, 2)
    for (b, gk), e in expo.items():
        assert s[b, gk] == np.float32(2.0 ** e), (b, gk)
    assert (q == 0x7E).sum() == 6
    # every code reads back within half a code spacing of its value (relative 2^-4)
    per = np.repeat(np.repeat(s, 128, axis=0)[:N], 128, axis=1).astype(np.float64)
    back = fp8.decode(q) * per
    big = np.abs(w) > per * 2.0 ** -6           # normal E4M3 range of the code
    assert (np.abs(back - w)[big] <= np.abs(w[big]) * 2.0 ** -4 + 1e-30).all()


def test_reduces_to_per_token_per_channel_gemm():
    """When every group of a row has the same maximum and every block column of a
    weight row block shares one scale, the block-wise GEMM is the per-token /
    per-channel GEMM: y = s_a s_w sum_k a w."""
    rng = np.random.default_rng(5)
    M, N, K = 5, 128, 512
    x = rng.standard_normal((M, K)).astype(np.float32)
    amax_rows = np.float32(rng.uniform(4, 9, M))
    for g in range(K // 128):
        x[:, g * 128] = amax_rows            # the same maximum in every group
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[0, ::128] = np.float32(0.3)            # one block row, one maximum per group
    qa, sa = bw.quant_act_blockwise(x)
    qw, sw = bw.quant_weight_blockwise(w)
    qa_t, sa_t = w8a8.quant_per_token(x)
    assert (sa == sa_t[:, None]).all() and np.array_equal(qa, qa_t)
    assert (sw == sw[0, 0]).all()
    y_bw = bw.gemm_blockwise_exact(qa, sa, qw, sw)
    acc = w8a8.gemm_acc_exact(qa, qw)
    y_pt = acc * sa_t.astype(np.float64)[:, None] * np.float64(sw[0, 0])
    # equal up to float64 rounding, measured against the sum of absolute terms
    scale = bw.gemm_blockwise_abs(qa, sa, qw, sw)
    assert (np.abs(y_bw - y_pt) <= 1e-14 * scale).all()


def test_tiny_case_in_exact_rationals():
    """M=2, N=3, K=256: the sum over groups of s_a s_w times the exact partial dot
    product, evaluated in Fractions, equals the float64 reference (to its own
    rounding) and gives the same bf16 bits."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((2, 256)) * np.float32([[1.0], [30.0]])).astype(np.float32)
    x[0, 131] = 200.0
    w = (rng.standard_normal((3, 256)) * 0.05).astype(np.float32)
    qa, sa = bw.quant_act_blockwise(x)
    qw, sw = bw.quant_weight_blockwise(w)
    bits, y = bw.gemm_blockwise_bf16(qa, sa, qw, sw)
    a = fp8.decode(qa)
    wv = fp8.decode(qw)
    for m in range(2):
        for n in range(3):
            tot = Fraction(0)
            for g in range(2):
                p = sum(Fraction(float(a[m, k])) * Fraction(float(wv[n, k])) for k in range(128 * g, 128 * g + 128))
                tot += Fraction(float(sa[m, g])) * Fraction(float(sw[0, g])) * p
            assert abs(Fraction(float(y[m, n])) - tot) <= abs(tot) * Fraction(1, 2 ** 50)
            assert fp8.bf16_round_bits(np.float64([float(tot)]))[0] == bits[m, n]


def test_each_scale_multiplies_its_own_group_and_block():
    """Only group g0 of A and W is nonzero: y uses s_a[m, g0] and s_w[n // 128, g0]
    and no other scale; rows n >= 128 take the second weight block's scale."""
    rng = np.random.default_rng(7)
    M, N, K, g0 = 3, 200, 384, 1
    x = np.zeros((M, K), np.float32)
    x[:, 128 * g0:128 * g0 + 128] = rng.standard_normal((M, 128)).astype(np.float32)
    x[:, 0] = np.float32([1.0, 2.0, 4.0])        # other groups: other scales, no products
    w = np.zeros((N, K), np.float32)
    w[:, 128 * g0:128 * g0 + 128] = (rng.standard_normal((N, 128)) * 0.02).astype(np.float32)
    w[:128, 128 * g0 + 3] *= 4.0                 # the two row blocks get different maxima
    w[5, 300] = 9.0
    qa, sa = bw.quant_act_blockwise(x)
    qw, sw = bw.quant_weight_blockwise(w)
    assert sw[0, g0] != sw[1, g0]
    y = bw.gemm_blockwise_exact(qa, sa, qw, sw)
    p = fp8.decode(qa)[:, 128 * g0:128 * g0 + 128] @ fp8.decode(qw)[:, 128 * g0:128 * g0 + 128].T
    want = p * sa[:, g0].astype(np.float64)[:, None]
    want[:, :128] *= np.float64(sw[0, g0])
    want[:, 128:] *= np.float64(sw[1, g0])
    assert np.allclose(y, want, rtol=1e-15, atol=0)


def test_abs_sum_bounds_the_value():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    w = (rng.standard_normal((130, 256)) * 0.02).astype(np.float32)
    qa, sa = bw.quant_act_blockwise(x)
    qw, sw = bw.quant_weight_blockwise(w)
    y = bw.gemm_blockwise_exact(qa, sa, qw, sw)
    s = bw.gemm_blockwise_abs(qa, sa, qw, sw)
    assert (np.abs(y) <= s * (1 + 1e-15)).all() and (s > 0).all()
    # flipping the sign of one activation row flips that output row exactly
    y2 = bw.gemm_blockwise_exact(qa ^ np.uint8(0x80) * (np.arange(4) == 2)[:, None].astype(np.uint8), sa, qw, sw)
    assert np.array_equal(y2[2], -y[2]) and np.array_equal(np.delete(y2, 2, 0), np.delete(y, 2, 0))


def test_abs_sum_in_exact_rationals_and_its_equality_case():
    """sum_g |s_a[m, g] s_w[n / 128, g]| sum_{k in g} |a_k w_k| (the scale of the
    block-wise accumulator tolerance) against exact rationals on a tiny case with a
    ragged last weight block, and its equality with the block-wise value itself
    when every code and scale is non-negative."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((2, 256)) * np.float32([[1.0], [30.0]])).astype(np.float32)
    w = (rng.standard_normal((130, 256)) * 0.05).astype(np.float32)
    w[129, 7] = 3.0
    qa, sa = bw.quant_act_blockwise(x)
    qw, sw = bw.quant_weight_blockwise(w)
    s = bw.gemm_blockwise_abs(qa, sa, qw, sw)
    a = fp8.decode(qa)
    wv = fp8.decode(qw)
    for m in range(2):
        for n in (0, 1, 127, 128, 129):
            tot = Fraction(0)
            for g in range(2):
                p = sum(abs(Fraction(float(a[m, k])) * Fraction(float(wv[n, k]))) for k in range(128 * g, 128 * g + 128))
                tot += abs(Fraction(float(sa[m, g])) * Fraction(float(sw[n // 128, g]))) * p
            assert abs(Fraction(float(s[m, n])) - tot) <= tot * Fraction(1, 2 ** 50)
    a_pos, w_pos = qa & np.uint8(0x7F), qw & np.uint8(0x7F)
    assert np.array_equal(bw.gemm_blockwise_abs(a_pos, sa, w_pos, sw), bw.gemm_blockwise_exact(a_pos, sa, w_pos, sw))
    # the signs of the codes do not change it
    assert np.array_equal(bw.gemm_blockwise_abs(a_pos, sa, w_pos, sw), s)
