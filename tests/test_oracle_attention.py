"""Pins of the decode-attention oracle (oracle/attention.py) to facts that do
not come from the oracle itself: PyTorch's own scaled-dot-product attention on
the same (independently dequantized) data, closed forms, the grouped-head
mapping, and the online recurrence the FlashAttention post states to be exact."""

import numpy as np
import pytest
import torch

from oracle import attention as at
from oracle.fp8 import E4M3, E5M2


def _case(seed, B=2, S=96, Hkv=2, G=4, D=128, fmt_max=0x7E):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float32)
    kq = rng.integers(0, fmt_max, (B, S, Hkv, D), dtype=np.uint8) ^ (rng.integers(0, 2, (B, S, Hkv, D), dtype=np.uint8) << 7)
    vq = rng.integers(0, fmt_max, (B, S, Hkv, D), dtype=np.uint8) ^ (rng.integers(0, 2, (B, S, Hkv, D), dtype=np.uint8) << 7)
    sk = (rng.random(Hkv) * 0.02 + 0.001).astype(np.float32)
    sv = (rng.random(Hkv) * 0.5 + 0.01).astype(np.float32)
    return q, kq, vq, sk, sv


@pytest.mark.parametrize("fmt,tdt,mx", [(E4M3, torch.float8_e4m3fn, 0x7E), (E5M2, torch.float8_e5m2, 0x7B)])
def test_matches_torch_sdpa_on_library_dequantized_cache(fmt, tdt, mx):
    q, kq, vq, sk, sv = _case(1, fmt_max=mx)
    L = np.array([96, 41])
    got = at.attention_decode(q, kq, vq, sk, sv, L, fmt)
    B, Hq, D = q.shape
    G = Hq // kq.shape[2]
    for b in range(B):
        n = int(L[b])
        K = torch.from_numpy(kq[b, :n]).view(tdt).to(torch.float64) * torch.from_numpy(sk.astype(np.float64))[None, :, None]
        V = torch.from_numpy(vq[b, :n]).view(tdt).to(torch.float64) * torch.from_numpy(sv.astype(np.float64))[None, :, None]
        Kh = K.permute(1, 0, 2).repeat_interleave(G, dim=0)          # [Hq, n, D]
        Vh = V.permute(1, 0, 2).repeat_interleave(G, dim=0)
        Q = torch.from_numpy(q[b].astype(np.float64))[:, None, :]    # [Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kh, Vh)[:, 0, :].numpy()
        np.testing.assert_allclose(got[b], ref, rtol=1e-10, atol=1e-12)


def test_online_recurrence_is_exact():
    q, kq, vq, sk, sv = _case(2, S=300)
    L = np.array([300, 129])
    ref = at.attention_decode(q, kq, vq, sk, sv, L)
    for block in (1, 7, 64, 128, 1000):
        np.testing.assert_allclose(at.attention_online(q, kq, vq, sk, sv, L, block), ref, rtol=1e-12, atol=1e-14)


def test_equal_keys_give_the_mean_of_the_values():
    q, kq, vq, sk, sv = _case(3)
    kq[:] = kq[:, :1]                      # every position has the same key
    L = np.array([96, 50])
    o = at.attention_decode(q, kq, vq, sk, sv, L)
    from oracle.fp8 import decode
    for b in range(2):
        for h in range(8):
            g = h // 4
            mean = decode(vq[b, :L[b], g, :]).mean(axis=0) * np.float64(sv[g])
            np.testing.assert_allclose(o[b, h], mean, rtol=1e-12, atol=1e-15)


def test_single_position_and_empty_sequence():
    q, kq, vq, sk, sv = _case(4)
    o = at.attention_decode(q, kq, vq, sk, sv, np.array([1, 0]))
    from oracle.fp8 import decode
    for h in range(8):
        assert np.array_equal(o[0, h], decode(vq[0, 0, h // 4, :]) * np.float64(sv[h // 4]))
    assert (o[1] == 0).all()


def test_dominant_key_selects_its_value():
    q, kq, vq, sk, sv = _case(5)
    q[:] = 0.0
    q[:, :, 0] = 1.0                        # scores follow key dimension 0
    kq[:, :, :, 0] = 0x00                   # all zero ...
    kq[:, 17, :, 0] = 0x7E                  # ... except position 17: 448 * s_k
    sk[:] = 1.0                             # score of position 17: 448 / sqrt(128) ~ 39.6
    o = at.attention_decode(q, kq, vq, sk, sv, np.array([96, 96]))
    from oracle.fp8 import decode
    for b in range(2):
        for h in range(8):
            v17 = decode(vq[b, 17, h // 4, :]) * np.float64(sv[h // 4])
            np.testing.assert_allclose(o[b, h], v17, rtol=1e-14, atol=1e-14 + np.abs(v17).max() * 1e-15 * 96)


def test_grouped_heads_read_their_kv_head():
    q, kq, vq, sk, sv = _case(6)
    vq[:, :, 0, :] = 0x38                   # kv head 0: every value +1
    vq[:, :, 1, :] = 0xB8                   # kv head 1: every value -1
    sv[:] = 1.0
    o = at.attention_decode(q, kq, vq, sk, sv, np.array([96, 20]))
    assert np.allclose(o[:, :4, :], 1.0, rtol=0, atol=1e-14) and np.allclose(o[:, 4:, :], -1.0, rtol=0, atol=1e-14)


def test_default_scale_is_inverse_sqrt_head_dim():
    q, kq, vq, sk, sv = _case(7, D=64)
    L = np.array([96, 96])
    assert np.array_equal(at.attention_decode(q, kq, vq, sk, sv, L),
                          at.attention_decode(q, kq, vq, sk, sv, L, scale=1.0 / 8.0))
    assert not np.allclose(at.attention_decode(q, kq, vq, sk, sv, L),
                           at.attention_decode(q, kq, vq, sk, sv, L, scale=1.0))


def test_abs_weight_bounds_the_output():
    q, kq, vq, sk, sv = _case(8)
    L = np.array([96, 77])
    o = at.attention_decode(q, kq, vq, sk, sv, L)
    w = at.attention_abs_weight(q, kq, vq, sk, sv, L)
    assert (np.abs(o) <= w * (1 + 1e-12)).all()


def test_abs_weight_is_the_output_of_the_absolute_values():
    """sum_t p_t |V[t, d]| two-sided: with non-negative value codes it equals the
    attention output itself (pinned against PyTorch's SDPA above), flipping value
    signs leaves it unchanged, and it matches p @ |V| with p from PyTorch's own
    float64 softmax of the scaled scores."""
    q, kq, vq, sk, sv = _case(8)
    L = np.array([96, 77])
    v_pos = vq & np.uint8(0x7F)
    w_pos = at.attention_abs_weight(q, kq, v_pos, sk, sv, L)
    assert np.array_equal(w_pos, at.attention_decode(q, kq, v_pos, sk, sv, L))
    w = at.attention_abs_weight(q, kq, vq, sk, sv, L)
    assert np.array_equal(w, w_pos)
    B, Hq, D = q.shape
    G = Hq // kq.shape[2]
    for b in range(B):
        n = int(L[b])
        K = torch.from_numpy(kq[b, :n]).view(torch.float8_e4m3fn).to(torch.float64) * \
            torch.from_numpy(sk.astype(np.float64))[None, :, None]
        V = torch.from_numpy(vq[b, :n]).view(torch.float8_e4m3fn).to(torch.float64).abs() * \
            torch.from_numpy(sv.astype(np.float64))[None, :, None]
        Kh = K.permute(1, 0, 2).repeat_interleave(G, dim=0)          # [Hq, n, D]
        Vh = V.permute(1, 0, 2).repeat_interleave(G, dim=0)
        Q = torch.from_numpy(q[b].astype(np.float64))[:, :, None]    # [Hq, D, 1]
        p = torch.softmax((Kh @ Q)[:, :, 0] / np.sqrt(D), dim=-1)    # [Hq, n]
        ref = (p[:, None, :] @ Vh)[:, 0, :].numpy()
        np.testing.assert_allclose(w[b], ref, rtol=1e-12, atol=0)
