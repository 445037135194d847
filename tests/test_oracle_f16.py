"""Pins of the oracle's fp16 path (tko_topk_f16) against references that do
not share its method: the widening against numpy's float16 for every bit
pattern, and the top-k against the O(n^2) rank definition, numpy's lexsort
and Python's sorted, with fp16 values, on exhaustive tiny rows, on the
synthetic families re-encoded as fp16, and against the invariants."""

import itertools

import numpy as np
import pytest

import oracle
from oracle_pins import check_invariants, lexsort_reference, python_sorted_reference, rank_definition
from synth import FAMILIES, family_rows


def widen_f16(bits):
    with np.errstate(invalid="ignore"):
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# Ten fp16 symbols, one per class.
ALPHABET_F16 = np.array([0x7E00, 0xFC01, 0xFC00, 0xBC00, 0x8001, 0x8000, 0x0000, 0x0001, 0x3C00, 0x7C00],
                        dtype=np.uint16)


def test_widening_matches_numpy_for_every_pattern():
    lib = oracle.load()
    bits = np.arange(65536, dtype=np.uint16)
    ref = widen_f16(bits)
    got = np.array([lib.tko_f16_value(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_exhaustive_tiny_rows():
    for length in range(1, 5):
        rows = np.array(list(itertools.product(ALPHABET_F16, repeat=length)), dtype=np.uint16)
        for k in (1, 2, 3, 5):
            got = oracle.topk_f16(rows, length, k, threads=4)
            want = rank_definition(rows, k, widen_f16)
            for g, w in zip(got, want):
                assert np.array_equal(g, w), (length, k)


@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_families_against_library_sorts(family):
    for width, k in ((1, 1), (7, 5), (65, 64), (300, 20)):
        m = family_rows(family, 3, width, width + 2, seed=width, fmt="f16")
        idx, val, cnt, mask = oracle.topk_f16(m, width, k)
        for r in range(3):
            row = m[r, :width]
            for ref in (lexsort_reference(row, k, widen_f16), python_sorted_reference(row, k, widen_f16)):
                assert np.array_equal(idx[r], ref[0]) and np.array_equal(val[r], ref[1])
                assert cnt[r] == ref[2] and mask[r] == ref[3]
        check_invariants(m, width, k, idx, val, cnt, mask, widen_f16)


def test_wide_rows_invariants():
    for family in ("normal", "mixed_nonfinite", "uniform_bits", "levels64"):
        m = family_rows(family, 2, 9000, 9003, seed=3, fmt="f16")
        for k in (1, 64):
            check_invariants(m, 9000, k, *oracle.topk_f16(m, 9000, k), widen_f16)


def test_the_pins_tell_the_formats_apart():
    """Ranking fp16 rows as bf16 disagrees with the fp16 rank definition, so a
    widening mix-up in the oracle cannot pass these pins."""
    m = family_rows("uniform_bits", 8, 40, 40, seed=1, fmt="f16")
    wrong = oracle.topk_bf16(m, 40, 8)
    right = rank_definition(m, 8, widen_f16)
    assert not all(np.array_equal(a, b) for a, b in zip(wrong, right))
    assert all(np.array_equal(a, b) for a, b in zip(oracle.topk_f16(m, 40, 8), right))
