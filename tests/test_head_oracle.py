"""Pins of the draft-head oracle (oracle/head.py) by values fixed outside it:
Python integer arithmetic on integer-valued inputs, one-hot rows, the IEEE
classes of non-finite sums, and hand-made bound cases."""

import numpy as np
import pytest

from oracle.head import bf16_to_f64, check_head_logits, head_logit_bound, head_logits_exact


def f32_to_bf16_bits(x):
    """Exact for the small integers and powers of two used here."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def test_widening_of_known_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x4049], dtype=np.uint16)
    got = bf16_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -1.0 and got[2] == 0.0 and np.signbit(got[3])
    assert got[4] == np.inf and got[5] == -np.inf
    assert got[6] == 2.0 ** -133          # the smallest bf16 subnormal
    assert got[7] == 3.140625             # 0x4049: 1.5703125 * 2


@pytest.mark.parametrize("rows,hidden,vocab", [(1, 32, 1), (3, 64, 17), (15, 96, 40), (64, 32, 5)])
def test_integer_inputs_match_python_integers(rows, hidden, vocab):
    rng = np.random.default_rng(rows * 100 + hidden)
    hi = rng.integers(-8, 9, size=(rows, hidden))
    wi = rng.integers(-8, 9, size=(vocab, hidden))
    got = head_logits_exact(f32_to_bf16_bits(hi), f32_to_bf16_bits(wi))
    for r in range(rows):
        for n in range(vocab):
            assert got[r, n] == sum(int(hi[r, i]) * int(wi[n, i]) for i in range(hidden))


def test_one_hot_rows_select_weight_columns():
    rng = np.random.default_rng(3)
    w = f32_to_bf16_bits(rng.integers(-100, 101, size=(50, 32)).astype(np.float32) / 64)
    h = np.zeros((32, 32), dtype=np.uint16)
    h[np.arange(32), np.arange(32)] = 0x3F80
    got = head_logits_exact(h, w)
    assert np.array_equal(got, bf16_to_f64(w).T)


def test_non_finite_classes():
    h = f32_to_bf16_bits([[1.0, 0.0], [np.inf, 1.0], [np.inf, -np.inf]])
    w = f32_to_bf16_bits([[2.0, 3.0], [0.0, 1.0], [-1.0, 0.0]])
    got = head_logits_exact(h, w)
    assert got[0, 0] == 2.0 and got[0, 1] == 0.0 and got[0, 2] == -1.0
    assert got[1, 0] == np.inf and np.isnan(got[1, 1]) and got[1, 2] == -np.inf  # inf * 0 is NaN
    assert np.isnan(got[2, 0])                                                    # inf - inf


def test_bound_cases():
    # exact sums: the bound is the bf16 half ulp plus the float32 summation term
    h = f32_to_bf16_bits([[1.0] * 32])
    w = f32_to_bf16_bits([[1.0] * 32])
    b = head_logit_bound(h, w)[0, 0]
    assert b == pytest.approx(2.0 ** -8 * 32 + (1 + 2.0 ** -8) * 2 * 32 * 2.0 ** -24 * 32 + 2.0 ** -125)
    ok, _ = check_head_logits(f32_to_bf16_bits([[32.0]]), h, w)
    assert ok
    # a logit one bf16 ulp away from 1.0 (2^-7) is outside the bound of an exact 1.0
    h1 = f32_to_bf16_bits([[1.0] + [0.0] * 31])
    w1 = f32_to_bf16_bits([[1.0] + [0.0] * 31])
    assert check_head_logits(np.array([[0x3F81]], dtype=np.uint16), h1, w1)[0] is False
    assert check_head_logits(np.array([[0x3F80]], dtype=np.uint16), h1, w1)[0] is True
    # a NaN where the exact sum is +inf is a class error
    hn = f32_to_bf16_bits([[np.inf] + [0.0] * 31])
    assert check_head_logits(np.array([[0x7FC0]], dtype=np.uint16), hn, w1)[0] is False
    assert check_head_logits(np.array([[0x7F80]], dtype=np.uint16), hn, w1)[0] is True


def test_rounding_of_a_sum_between_bf16_values_is_inside_the_bound():
    # S = 1 + 2^-9 lies between the bf16 values 1 (2^-9 away) and 1 + 2^-7
    # (3 * 2^-9 away): only the nearer one is within half an ulp
    h = f32_to_bf16_bits([[1.0, 2.0 ** -9] + [0.0] * 30])
    w = f32_to_bf16_bits([[1.0, 1.0] + [0.0] * 30])
    assert check_head_logits(np.array([[0x3F80]], dtype=np.uint16), h, w)[0] is True
    assert check_head_logits(np.array([[0x3F81]], dtype=np.uint16), h, w)[0] is False
