"""The seeded input generators (CPU only)."""

import numpy as np
import pytest

from synth import CONFIGS, FAMILIES, f32_to_bf16_bits, family_rows, make_config_input, sha256_of
from synth.gen import BF16_NEG_INF, BF16_POS_INF, NAN_PAYLOADS, POISON


def test_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.0, 0.0, -0.0, 3.0e38, 1e-40], dtype=np.float32)
    got = f32_to_bf16_bits(x).tolist()
    # 1+2^-8 is halfway between 0x3F80 and 0x3F81 -> even 0x3F80; 1+3*2^-8 -> even 0x3F82
    assert got[:6] == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x0000, 0x8000]
    assert got[6] == 0x7F62  # 3e38 rounds to the nearest bf16, still finite
    assert got[7] == 0x0001  # 1e-40 = float32 bits 0x000116C2 -> bf16 subnormal 0x0001


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_configs_are_seeded_and_shaped(name):
    cfg = CONFIGS[name]
    a = make_config_input(name)
    b = make_config_input(name)
    assert a.shape == (cfg.rows, cfg.stride) and a.dtype == np.uint16 and a.flags.c_contiguous
    assert sha256_of(a) == sha256_of(b)
    if cfg.stride > cfg.cols:
        pad = a[:, cfg.cols:]
        assert set(np.unique(pad).tolist()) <= set(POISON)


def test_c3_fractions():
    cfg = CONFIGS["c3"]
    m = make_config_input("c3")[:, : cfg.cols]
    for r in range(cfg.rows):
        row = m[r]
        assert (row == BF16_POS_INF).sum() == 124
        assert (row == BF16_NEG_INF).sum() == 124
        assert np.isin(row, np.array(NAN_PAYLOADS, dtype=np.uint16)).sum() == 248
        assert ((row == 0x8000) | (row == 0)).sum() >= 2483  # forced zeros plus the zero level
        assert (row == 0x8000).sum() > 1000  # both signs of zero present


def test_c4_neginf_rows():
    cfg = CONFIGS["c4"]
    m = make_config_input("c4")[:, : cfg.cols]
    ninf_rows = [(m[r] == BF16_NEG_INF).sum() for r in range(cfg.rows)]
    assert sum(1 for n in ninf_rows if n == cfg.cols - 1) == 10


def test_families_deterministic_and_padded():
    for name in FAMILIES:
        a = family_rows(name, 3, 50, 53, seed=9)
        b = family_rows(name, 3, 50, 53, seed=9)
        assert np.array_equal(a, b), name
        assert set(np.unique(a[:, 50:]).tolist()) <= set(POISON), name
