"""Pins of the oracle's fp32 path (tko_topk_f32): the O(n^2) rank
definition with float32 values on exhaustive tiny rows; numpy's lexsort and
Python's sorted on every family in fp32 form (random low fraction bits break
the ties the bf16 grid makes); the bf16 oracle on rows of bf16 values held
in fp32 (the same answer must come out); invariants on wide rows."""

import itertools

import numpy as np
import pytest

import oracle
from oracle_pins import check_invariants, lexsort_reference, python_sorted_reference, rank_definition
from synth import FAMILIES, bf16_to_f32_bits, family_rows

FILL32 = 0x7FC00000


def widen_f32(bits):
    with np.errstate(invalid="ignore"):  # signalling-NaN payloads raise the invalid flag
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


# Ten fp32 symbols, one per class.
ALPHABET_F32 = np.array([0x7FC00000, 0xFF800001, 0xFF800000, 0xBF800000, 0x80000001, 0x80000000, 0x00000000,
                         0x00000001, 0x3F800000, 0x7F800000], dtype=np.uint32)


def test_exhaustive_tiny_rows():
    for length in range(1, 5):
        rows = np.array(list(itertools.product(ALPHABET_F32, repeat=length)), dtype=np.uint32)
        for k in (1, 2, 3, 5):
            got = oracle.topk_f32(rows, length, k, threads=4)
            want = rank_definition(rows, k, widen_f32, word=np.uint32, fill=FILL32)
            for g, w in zip(got, want):
                assert np.array_equal(g, w), (length, k)


@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_families_against_library_sorts(family):
    for width, k in ((1, 1), (7, 5), (65, 64), (300, 20)):
        m = family_rows(family, 3, width, width + 2, seed=width, fmt="f32")
        idx, val, cnt, mask = oracle.topk_f32(m, width, k)
        want = rank_definition(m[:, :width], k, widen_f32, word=np.uint32, fill=FILL32)
        for g, w in zip((idx, val, cnt, mask), want):
            assert np.array_equal(g, w), (family, width, k)
        for r in range(3):
            row = m[r, :width]
            for ref in (lexsort_reference(row, k, widen_f32), python_sorted_reference(row, k, widen_f32)):
                assert np.array_equal(idx[r], ref[0]) and cnt[r] == ref[2] and mask[r] == ref[3]
        check_invariants(m, width, k, idx, val, cnt, mask, widen_f32, fill=FILL32)


@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_bf16_values_held_in_fp32_give_the_bf16_answer(family):
    m = family_rows(family, 4, 2000, 2003, seed=9)
    m32 = bf16_to_f32_bits(m)
    for k in (1, 17, 64):
        i16, v16, c16, k16 = oracle.topk_bf16(m, 2000, k)
        i32, v32, c32, k32 = oracle.topk_f32(m32, 2000, k)
        assert np.array_equal(i16, i32) and np.array_equal(c16, c32) and np.array_equal(k16, k32)
        assert np.array_equal(v16.astype(np.uint32) << 16, v32)


def test_wide_rows_invariants():
    for family in ("normal", "mixed_nonfinite", "uniform_bits", "levels64"):
        m = family_rows(family, 2, 9000, 9003, seed=3, fmt="f32")
        for k in (1, 64):
            check_invariants(m, 9000, k, *oracle.topk_f32(m, 9000, k), widen_f32, fill=FILL32)
