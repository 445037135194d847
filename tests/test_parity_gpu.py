"""Parity of the HIP top-k with the CPU oracle, byte for byte in all four
outputs (idx, val, count, nonfinite).

Case structure follows the exactness suite of TensorFold PR #713 (widths from
4096 to 248320 with ties, both zeros, NaN and infinities, padded strides; the
split path equal to the single-group control), extended to small and odd
widths, misaligned rows, every k, forced span counts and the five workload
configurations at full size.
"""

import numpy as np
import pytest

import oracle
from gpu_util import assert_same, check_case, gpu_topk, log, need_gpu, upload
from synth import CONFIGS, FAMILIES, family_rows, make_config_input

pytestmark = pytest.mark.gpu

WIDTHS = [1, 7, 8, 9, 64, 65, 513, 1000, 4095, 4096, 4103, 8191, 32768, 65537, 98592, 151936, 248320]
KS = [1, 8, 16, 20, 32, 63, 64]
SPANS = [0, 1, 2, 3, 16, 64]


def stride_for(w, i):
    return [w, w + 1, w + 3, w + 128, -(-w // 64) * 64][i % 5]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_family_widths(family):
    fi = sorted(FAMILIES).index(family)
    for i, w in enumerate(WIDTHS):
        stride = stride_for(w, i + fi)
        k = KS[(i + fi) % len(KS)]
        spans = SPANS[(i + 2 * fi) % len(SPANS)]
        if spans > w:
            spans = 0
        offset = (i + fi) % 8
        rows = 3 if w < 100000 else 2
        m = family_rows(family, rows, w, stride, seed=1000 * fi + i)
        what = f"family={family} rows={rows} cols={w} stride={stride} k={k} spans={spans} offset={offset}"
        log(what)
        check_case(m, w, k, spans=spans, offset=offset, what=what)


@pytest.mark.parametrize("family", ["normal", "levels64", "mixed_nonfinite", "uniform_bits", "neginf_one_finite",
                                    "zeros_straddle", "ascending", "descending"])
@pytest.mark.parametrize("cols", [98592, 248320])
def test_split_equals_single_group(family, cols):
    """Every span count gives the oracle's bytes (the page's split == control check)."""
    m = family_rows(family, 3, cols, cols + 64, seed=cols)
    want = oracle.topk_bf16(m, cols, 20)
    x = upload(m)
    for spans in (1, 2, 3, 5, 16, 31, 64):
        log(f"split family={family} cols={cols} spans={spans}")
        assert_same(gpu_topk(m, cols, 20, spans=spans, x=x), want, f"{family} cols={cols} spans={spans}")


def test_every_k():
    m = family_rows("logit", 5, 20000, 20003, seed=5)
    x = upload(m)
    for k in range(1, 65):
        want = oracle.topk_bf16(m, 20000, k)
        for spans in (0, 1, 4):
            log(f"every_k k={k} spans={spans}")
            assert_same(gpu_topk(m, 20000, k, spans=spans, x=x), want, f"k={k} spans={spans}")


@pytest.mark.parametrize("offset", range(8))
def test_misaligned_rows(offset):
    for w in (5, 17, 100, 4103, 70001):
        for stride in (w, w + 1, w + 5):
            m = family_rows("uniform_bits", 4, w, stride, seed=w + offset)
            log(f"misaligned offset={offset} cols={w} stride={stride}")
            check_case(m, w, 64, offset=offset, what=f"offset={offset} cols={w} stride={stride}")
            check_case(m, w, 7, spans=2 if w > 8 else 1, offset=offset, what=f"offset={offset} cols={w} s=2")


def test_tiny_rows_all_k():
    for w in range(1, 40):
        m = family_rows("uniform_bits", 2, w, w, seed=w)
        for k in (1, 3, 8, 64):
            log(f"tiny cols={w} k={k}")
            check_case(m, w, k, what=f"tiny cols={w} k={k}")


def test_merge_dispatch_levels():
    """Forced span counts above the fused limit (64 spans) go through the merge
    dispatch, levels of up to 64 lists per workgroup: one full and one ragged
    group (65, 100), exact multiples (128), a group of one list (129), many
    groups (1000), and three levels (5000 spans of ~20 columns) -- for k from
    1 to 64, on ties, non-finite values and plain logits."""
    cases = [
        ("logit", 3, 98592, 20, 65),
        ("mixed_nonfinite", 2, 98592, 64, 100),
        ("levels64", 2, 98592, 1, 128),
        ("few_levels", 2, 98592, 33, 129),
        ("zeros_straddle", 2, 151936, 16, 1000),
        ("normal", 2, 100000, 64, 5000),
    ]
    for family, rows, cols, k, spans in cases:
        m = family_rows(family, rows, cols, cols + 5, seed=spans)
        log(f"merge levels family={family} rows={rows} cols={cols} k={k} spans={spans}")
        check_case(m, cols, k, spans=spans, what=f"merge levels {family} k={k} spans={spans}")


def test_wide_rows_need_several_spans():
    """Rows wider than one workgroup's span limit, and a two-level merge."""
    for family in ("normal", "uniform_bits", "levels64"):
        m = family_rows(family, 2, 600000, 600003, seed=6)
        for spans in (0, 3, 100):
            log(f"wide family={family} spans={spans}")
            check_case(m, 600000, 33, spans=spans, what=f"wide {family} spans={spans}")


def test_edge_cases():
    import torch

    import wide_row_bf16_amd as tk

    # rows == 0
    x = torch.empty((0, 10), dtype=torch.bfloat16, device="cuda")
    out = tk.topk_bf16(x, 5)
    assert out.idx.shape == (0, 5)
    # cols == 0
    m = np.zeros((3, 0), dtype=np.uint16)
    check_case(m, 0, 4, what="cols=0")
    # all NaN, all -inf, all +inf, single columns
    for fam in ("all_nan", "neginf_all"):
        for w in (1, 63, 64, 4097):
            check_case(family_rows(fam, 2, w, w, seed=w), w, 64, what=f"{fam} {w}")
    pinf = np.full((2, 5000), 0x7F80, dtype=np.uint16)
    check_case(pinf, 5000, 64, what="all +inf")
    check_case(pinf, 5000, 64, spans=3, what="all +inf split")
    # k larger than the non-NaN count, rows of zeros of both signs
    check_case(family_rows("zeros", 3, 50, 50, seed=1), 50, 64, what="zeros k>cols")
    check_case(family_rows("nan_sprinkled", 3, 40, 41, seed=2), 40, 64, what="nan k>count")


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_configs_full_size(name):
    """The workload configurations at full size, automatic plan and the
    single-group control, against the oracle on every row."""
    cfg = CONFIGS[name]
    m = make_config_input(name)
    log(f"config {name}: oracle on {cfg.rows} rows")
    want = oracle.topk_bf16(m, cfg.cols, cfg.k)
    x = upload(m)
    for spans in (0, 1):
        log(f"config {name} spans={spans}")
        assert_same(gpu_topk(m, cfg.cols, cfg.k, spans=spans, x=x), want, f"{name} spans={spans}")


@pytest.mark.parametrize("family", ["normal", "logit", "levels64", "mixed_nonfinite", "uniform_bits", "ascending",
                                    "descending", "zeros_straddle", "all_equal", "neginf_one_finite"])
def test_speculative_floor_and_exact_mode(family):
    """Wide single-span rows take the speculative floor; the exact mode and the
    floor must give the oracle's bytes alike."""
    cols = 248320
    m = family_rows(family, 3, cols, cols, seed=77)
    x = upload(m)
    for k in (1, 9, 64):
        want = oracle.topk_bf16(m, cols, k)
        for exact in (False, True):
            log(f"speculative family={family} k={k} exact={exact}")
            got = gpu_topk(m, cols, k, spans=1, x=x) if not exact else _exact(x, cols, k)
            assert_same(got, want, f"{family} k={k} exact={exact}")


def _exact(x, cols, k):
    import wide_row_bf16_amd as tk
    from gpu_util import to_numpy

    return to_numpy(tk.topk_bf16(x, k, cols=cols, spans=1, exact=True))


def test_speculation_falls_back_when_floor_is_too_high():
    """Large values in the first vectors of 15 lanes of each wave (60 in all)
    fill the top of the floor's sample, so the speculative floor lands on them
    whenever its rank is at most 60: k = 61 and k = 64 must scan again, k = 8
    and k = 60 verify.  (Each wave of a single-span 151936-column row starts at
    a multiple of 37984 columns for 16-byte aligned rows, and lane i's first
    vector starts 8 i columns in.)"""
    cols = 151936
    m = family_rows("normal", 4, cols, cols, seed=5)
    for w in range(4):
        for i in range(15):
            m[:, 37984 * w + 8 * i] = 0x42C8  # 100.0
    x = upload(m)
    for k in (8, 60, 61, 64):
        log(f"fallback k={k}")
        assert_same(gpu_topk(m, cols, k, spans=1, x=x), oracle.topk_bf16(m, cols, k), f"fallback k={k}")
