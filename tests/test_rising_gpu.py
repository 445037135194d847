"""Rows that rise along a wave's share: the bf16/fp16 scan then takes a floor
from the end of the share (the k-th largest lane maximum of the share's last
chunk) before scanning it.  Parity with the oracle, byte for byte, where that
floor is taken (ascending rows of at least six chunks per wave), where it is
taken but useless (rows that rise and then fall), where it lands on ties
(a plateau at the top), with non-finite values sprinkled in, at forced span
counts, with the speculative floor and in the exact mode.
"""

import numpy as np
import pytest

import oracle
from gpu_util import assert_same, gpu_topk, log, need_gpu, upload
from synth import family_rows

pytestmark = pytest.mark.gpu

# 49152 columns give each wave of a single-span row exactly six chunks of 2048
WIDTHS = [49152, 49161, 98592, 151936, 248320]
KS = [1, 9, 32, 64]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _check(m, cols, k, spans, what, fmt="bf16", x=None):
    want = (oracle.topk_bf16 if fmt == "bf16" else oracle.topk_f16)(m, cols, k)
    log(f"rising {what} cols={cols} k={k} spans={spans}")
    assert_same(gpu_topk(m, cols, k, spans=spans, x=x, fmt=fmt), want, f"{what} cols={cols} k={k} spans={spans}")


@pytest.mark.parametrize("cols", WIDTHS)
def test_ascending_rows(cols):
    m = family_rows("ascending", 3, cols, cols, seed=cols)
    x = upload(m)
    for k in KS:
        for spans in (1, 0, 2):
            _check(m, cols, k, spans, "ascending", x=x)


def test_ascending_exact_mode():
    import wide_row_bf16_amd as tk
    from gpu_util import to_numpy

    cols = 151936
    m = family_rows("ascending", 3, cols, cols, seed=3)
    x = upload(m)
    for k in KS:
        log(f"rising exact k={k}")
        got = to_numpy(tk.topk_bf16(x, k, cols=cols, spans=1, exact=True))
        assert_same(got, oracle.topk_bf16(m, cols, k), f"ascending exact k={k}")


@pytest.mark.parametrize("cols", [98592, 151936])
def test_rise_then_fall(cols):
    """The first chunk rises (the floor from the share's end is taken) but the
    row falls again, so the last chunk holds small values: a low floor."""
    m = family_rows("ascending", 3, cols, cols, seed=11)
    half = cols // 2
    m[:, half:] = m[:, :cols - half][:, ::-1]
    x = upload(m)
    for k in KS:
        _check(m, cols, k, 1, "rise-fall", x=x)


@pytest.mark.parametrize("cols", [98592, 151936])
def test_plateau_ties_at_the_floor(cols):
    """A ramp that reaches its top value early and stays there: the top k are
    the first k columns of the plateau, all tied with the last chunk's keys."""
    ramp = family_rows("ascending", 2, cols, cols, seed=13)
    for r in range(ramp.shape[0]):
        top = ramp[r, -1]
        start = cols // 3 + 1000 * r
        ramp[r, start:] = top
    x = upload(ramp)
    for k in KS:
        for spans in (1, 0):
            _check(ramp, cols, k, spans, "plateau", x=x)


def test_ascending_with_nonfinite_values():
    cols = 151936
    m = family_rows("ascending", 4, cols, cols, seed=17)
    rng = np.random.default_rng(17)
    specials = np.array([0x7FC0, 0xFFC1, 0x7F80, 0xFF80, 0x8000, 0x0000], dtype=np.uint16)
    for r in range(m.shape[0]):
        pos = rng.choice(cols, size=40, replace=False)
        m[r, pos] = specials[rng.integers(0, len(specials), size=40)]
    # one row with +inf only near its start: kept ahead of the rising values
    m[3, 5] = 0x7F80
    x = upload(m)
    for k in KS:
        for spans in (1, 0):
            _check(m, cols, k, spans, "ascending+nonfinite", x=x)


def test_ascending_rows_fp16():
    cols = 151936
    m = family_rows("ascending", 3, cols, cols, seed=19, fmt="f16")
    x = upload(m)
    for k in KS:
        _check(m, cols, k, 1, "ascending fp16", fmt="f16", x=x)


# The same floor in the k > 64 scans (from each lane's two or four largest
# keys of the last chunk) and in the fp32 scans.
WIDE_KS = [65, 128, 129, 200, 256]


@pytest.mark.parametrize("cols", [98592, 151936])
def test_ascending_rows_wide_k(cols):
    m = family_rows("ascending", 3, cols, cols, seed=cols + 1)
    x = upload(m)
    for k in WIDE_KS:
        for spans in (1, 0):
            _check(m, cols, k, spans, "ascending wide", x=x)


def test_rise_fall_and_plateau_wide_k():
    cols = 151936
    m = family_rows("ascending", 3, cols, cols, seed=23)
    half = cols // 2
    m[0, half:] = m[0, :cols - half][::-1]
    m[1, cols // 3:] = m[1, -1]
    x = upload(m)
    for k in WIDE_KS:
        _check(m, cols, k, 1, "rise-fall/plateau wide", x=x)


def _check32(m, cols, k, spans, what, x):
    want = oracle.topk_f32(m, cols, k)
    log(f"rising f32 {what} cols={cols} k={k} spans={spans}")
    assert_same(gpu_topk(m, cols, k, spans=spans, x=x, fmt="f32"), want, f"f32 {what} cols={cols} k={k} spans={spans}")


@pytest.mark.parametrize("cols", [49152, 151936])
def test_ascending_rows_fp32(cols):
    m = family_rows("ascending", 3, cols, cols, seed=cols + 2, fmt="f32")
    x = upload(m)
    for k in KS + WIDE_KS:
        for spans in (1, 0):
            _check32(m, cols, k, spans, "ascending", x)


def test_rise_fall_and_plateau_fp32():
    cols = 151936
    m = family_rows("ascending", 3, cols, cols, seed=29, fmt="f32")
    half = cols // 2
    m[0, half:] = m[0, :cols - half][::-1]
    m[1, cols // 3:] = m[1, -1]
    x = upload(m)
    for k in (1, 32, 64, 128, 256):
        _check32(m, cols, k, 1, "rise-fall/plateau", x)
