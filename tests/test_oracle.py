"""The CPU oracle against its pins (CPU only)."""

import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle_pins import (
    ALL_PINS,
    check_invariants,
    pin_closed_forms,
    pin_exhaustive,
    pin_golden,
    pin_invariants,
    pin_library_sorts,
    pin_padding,
    run,
)
from synth import family_rows


def test_exhaustive_tiny_rows(oracle_lib):
    pin_exhaustive(oracle_lib, max_len=5, ks=range(1, 7))


def test_golden_worked_examples(oracle_lib):
    pin_golden(oracle_lib)


def test_library_sorts(oracle_lib):
    pin_library_sorts(oracle_lib)


def test_library_sorts_large_k(oracle_lib):
    # k beyond one wavefront (65..256): the same definition, pinned the same way
    pin_library_sorts(oracle_lib, widths=(1, 64, 65, 257, 300, 1000), ks=(65, 128, 200, 256), seed=5)


def test_invariants_large_k(oracle_lib):
    pin_invariants(oracle_lib, widths=(4096, 9000), ks=(65, 129, 256), seed=9)


def test_padding_never_read(oracle_lib):
    pin_padding(oracle_lib)


def test_closed_forms(oracle_lib):
    pin_closed_forms(oracle_lib)


def test_invariants_wide_rows(oracle_lib):
    pin_invariants(oracle_lib)


def test_thread_count_does_not_change_results(oracle_lib):
    m = family_rows("uniform_bits", 37, 5000, 5003, seed=3)
    base = run(oracle_lib, m, 5000, 64, threads=1)
    for t in (2, 5, 37, 64):
        got = run(oracle_lib, m, 5000, 64, threads=t)
        for a, b in zip(base, got):
            assert np.array_equal(a, b)


def test_rejects_invalid_arguments(oracle_lib):
    m = np.zeros((2, 4), dtype=np.uint16)
    with pytest.raises(RuntimeError):
        oracle.topk_bf16(m, 4, 0, lib=oracle_lib)


# ---------------------------------------------------------------------------
# Planted mistakes: each edit below is a plausible bug in the oracle.  The pins
# must reject every one of them, or they are not pinning anything.
# ---------------------------------------------------------------------------

MUTANTS = {
    "ascending_order": ("if (a->value > b->value) return -1;\n  if (a->value < b->value) return 1;",
                        "if (a->value < b->value) return -1;\n  if (a->value > b->value) return 1;"),
    "ties_to_higher_index": ("if (a->col < b->col) return -1;\n  if (a->col > b->col) return 1;",
                             "if (a->col > b->col) return -1;\n  if (a->col < b->col) return 1;"),
    "nan_kept": ("mask |= 1u;\n        continue;", "mask |= 1u;"),
    "zeros_told_apart": ("memcpy(&f, &u, sizeof f);\n  return (double)f;",
                         "memcpy(&f, &u, sizeof f);\n  return (f == 0.0f && signbit(f)) ? -1e-300 : (double)f;"),
    "subnormals_flushed": ("memcpy(&f, &u, sizeof f);\n  return (double)f;",
                           "memcpy(&f, &u, sizeof f);\n  return fpclassify(f) == FP_SUBNORMAL ? 0.0 : (double)f;"),
    "fill_value": ("put_word(job->out_val, o, job->fill, job->word);", "put_word(job->out_val, o, 0, job->word);"),
    "fill_index": ("job->out_idx[o] = -1;", "job->out_idx[o] = 0;"),
    "mask_bits_swapped": ("(v > 0) ? 2u : 4u", "(v > 0) ? 4u : 2u"),
    "neginf_not_flagged": ("if (isinf(v)) mask |= (v > 0) ? 2u : 4u;", "if (isinf(v) && v > 0) mask |= 2u;"),
    "count_off_by_one": ("int64_t count = n < job->k ? n : job->k;", "int64_t count = n < job->k ? n : job->k - 1;"),
    "stride_ignored": ("const int64_t row = r * job->row_stride;", "const int64_t row = r * job->cols;"),
    "padding_read": [("for (int64_t c = 0; c < job->cols; ++c)",
                      "for (int64_t c = 0; c < job->row_stride; ++c)"),
                     ("(size_t)(job->cols > 0 ? job->cols : 1)", "(size_t)(job->row_stride > 0 ? job->row_stride : 1)")],
    "value_from_entry_slot": ("word_at(job->in, row + list[j].col, job->word)", "word_at(job->in, row + j, job->word)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_oracle_mutants_are_caught(name, tmp_path):
    with open(oracle.SOURCE) as f:
        src = f.read()
    edits = MUTANTS[name]
    for old, new in edits if isinstance(edits, list) else [edits]:
        assert src.count(old) == 1, f"mutation {name} no longer applies to the oracle source"
        src = src.replace(old, new)
    path = tmp_path / f"mut_{name}.c"
    path.write_text(src)
    so = str(tmp_path / f"libmut_{name}.so")
    subprocess.run(oracle.build_command(str(path), so), check=True)
    lib = oracle.load(so)
    caught = []
    for pin in ALL_PINS:
        try:
            if pin is pin_exhaustive:
                pin(lib, max_len=4, ks=range(1, 6))
            else:
                pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake '{name}'"
