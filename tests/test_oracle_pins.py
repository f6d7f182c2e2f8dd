"""The CPU oracle against its pins (brute force, worked examples, closed forms, invariants)."""

import numpy as np
import pytest

from oracle import attention_bwd, attention_fwd, bf16_bits_to_f64

from oracle_pins import ALL_PINS, BWD_PINS, FP8_PINS, WINDOW_PINS


def oracle_impl(q, k, v, scale, causal=False, kv_seqlens=None, return_p=False, window=None):
    return attention_fwd(q, k, v, scale, causal=causal, kv_seqlens=kv_seqlens, return_p=return_p,
                         window=window)


@pytest.mark.parametrize("pin", ALL_PINS + WINDOW_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle_impl)


def oracle_bwd(q, k, v, do, scale, causal=False, kv_seqlens=None, window=None):
    return attention_bwd(q, k, v, do, scale, causal=causal, kv_seqlens=kv_seqlens, window=window)


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda f: f.__name__)
def test_oracle_backward_pin(pin):
    pin(oracle_bwd, oracle_impl)


def fp8_namespace():
    import types

    from oracle import fp8
    return types.SimpleNamespace(decode=fp8.e4m3_decode, round=fp8.e4m3_round,
                                 quantize=fp8.quantize_e4m3, attention=fp8.attention_fwd_fp8,
                                 bound=fp8.p_rounding_bound)


@pytest.mark.parametrize("pin", FP8_PINS, ids=lambda f: f.__name__)
def test_oracle_fp8_pin(pin):
    pin(fp8_namespace())


def test_rows_subset_equals_full():
    r = np.random.default_rng(3)
    q = r.standard_normal((2, 2, 40, 8))
    k = r.standard_normal((2, 2, 40, 8))
    v = r.standard_normal((2, 2, 40, 8))
    rows = np.array([0, 5, 17, 39])
    for causal, lens in ((True, None), (False, [33, 7])):
        o, lse = attention_fwd(q, k, v, 0.4, causal, lens)
        o2, lse2 = attention_fwd(q, k, v, 0.4, causal, lens, rows=rows)
        assert np.array_equal(o[:, :, rows], o2)
        assert np.array_equal(lse[:, :, rows], lse2)


def test_empty_rows_and_empty_batch():
    r = np.random.default_rng(4)
    q = r.standard_normal((2, 1, 3, 4))
    k = r.standard_normal((2, 1, 5, 4))
    v = r.standard_normal((2, 1, 5, 4))
    o, lse = attention_fwd(q, k, v, 1.0, False, [0, 5])
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))
    o, lse = attention_fwd(np.zeros((0, 2, 3, 4)), np.zeros((0, 2, 5, 4)), np.zeros((0, 2, 5, 4)), 1.0)
    assert o.shape == (0, 2, 3, 4) and lse.shape == (0, 2, 3)


def test_bf16_bits_exact():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x3E00, 0x4049], dtype=np.uint16)
    want = np.array([1.0, -2.0, np.inf, -np.inf, 2.0 ** -133, -0.0, 0.125, 3.140625])
    got = bf16_bits_to_f64(bits)
    assert np.array_equal(got, want)
    assert np.signbit(got[5])
