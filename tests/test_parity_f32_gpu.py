"""Parity of the HIP top-k on IEEE fp32 rows (tk_topk_f32) with the
oracle's fp32 path, byte for byte: every family in fp32 form (random low
fraction bits on the continuous families, exact ties on the others) over
widths, strides, k, forced spans and misaligned rows; split counts equal
the single-group control; the exact mode; the workload shapes at full size
in fp32 form; rows wider than the bf16 span limit in one span."""

import numpy as np
import pytest

import oracle
from gpu_util import assert_same, check_case, gpu_topk, log, need_gpu, upload
from synth import CONFIGS, FAMILIES, bf16_to_f32_bits, family_rows, make_config_input

pytestmark = pytest.mark.gpu

WIDTHS = [1, 3, 4, 5, 65, 1000, 4099, 32768, 98592, 151936]
KS = [1, 8, 20, 33, 64]
SPANS = [0, 1, 3, 16]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_family_widths_f32(family):
    fi = sorted(FAMILIES).index(family)
    for i, w in enumerate(WIDTHS):
        stride = [w, w + 1, w + 3, -(-w // 64) * 64][(i + fi) % 4]
        k = KS[(i + fi) % len(KS)]
        spans = SPANS[(i + 2 * fi) % len(SPANS)]
        if spans > w:
            spans = 0
        offset = (i + fi) % 4
        m = family_rows(family, 3, w, stride, seed=700 + 10 * fi + i, fmt="f32")
        what = f"f32 family={family} cols={w} stride={stride} k={k} spans={spans} offset={offset}"
        log(what)
        check_case(m, w, k, spans=spans, offset=offset, what=what, fmt="f32")


@pytest.mark.parametrize("family", ["normal", "levels64", "mixed_nonfinite", "uniform_bits", "zeros_straddle",
                                    "all_equal"])
def test_split_and_exact_f32(family):
    cols = 248320
    m = family_rows(family, 3, cols, cols, seed=23, fmt="f32")
    x = upload(m)
    for k in (1, 20, 64):
        want = oracle.topk_f32(m, cols, k)
        for spans in (1, 2, 7, 12, 64):
            log(f"f32 split family={family} k={k} spans={spans}")
            assert_same(gpu_topk(m, cols, k, spans=spans, x=x, fmt="f32"), want, f"{family} k={k} spans={spans}")
        assert_same(gpu_topk(m, cols, k, spans=1, x=x, fmt="f32", exact=True), want, f"{family} k={k} exact")


def test_one_span_wider_than_the_bf16_limit():
    cols = 600000
    m = family_rows("normal", 2, cols, cols + 1, seed=4, fmt="f32")
    for spans in (1, 0):
        log(f"f32 wide spans={spans}")
        check_case(m, cols, 40, spans=spans, what=f"f32 600000 spans={spans}", fmt="f32")


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
def test_configs_full_size_f32(name):
    cfg = CONFIGS[name]
    m = bf16_to_f32_bits(make_config_input(name), np.random.default_rng(31))
    log(f"f32 config {name}")
    want = oracle.topk_f32(m, cfg.cols, cfg.k)
    x = upload(m)
    for spans in (0, 1):
        assert_same(gpu_topk(m, cfg.cols, cfg.k, spans=spans, x=x, fmt="f32"), want, f"f32 {name} spans={spans}")


def test_equal_negative_rows_with_partial_waves():
    """Rows of one negative value whose waves hold fewer vectors than lanes:
    the zeros that out-of-range lanes read must never enter a batch (0.0
    would outrank every entry)."""
    for cols in (300, 1000, 4099):
        for v in (-1.0, -3.5e-30):
            m = np.full((2, cols), np.float32(v)).view(np.uint32)
            for k in (1, 5, 64):
                log(f"f32 equal negative cols={cols} v={v} k={k}")
                check_case(m, cols, k, spans=1, what=f"f32 equal {v} cols={cols} k={k}", fmt="f32")
                check_case(m, cols, k, what=f"f32 equal {v} cols={cols} k={k} auto", fmt="f32")


def test_split_rows_beyond_one_batch_and_state_f32():
    """4100 split fp32 rows: two launches of the fused fold share the arrival
    counters (zero again after every row), then other split shapes on the
    same stream."""
    cols = 2112
    m = family_rows("logit", 4100, cols, cols, seed=17, fmt="f32")
    want = oracle.topk_f32(m, cols, 24)
    x = upload(m)
    for spans in (2, 1, 3, 2):
        log(f"f32 4100 rows spans={spans}")
        assert_same(gpu_topk(m, cols, 24, spans=spans, x=x, fmt="f32"), want, f"f32 4100 rows spans={spans}")
    for rows, c, k, spans in ((15, 98592, 32, 0), (3, 70000, 64, 64), (40, 9000, 8, 4)):
        mm = family_rows("mixed_nonfinite", rows, c, c, seed=rows, fmt="f32")
        log(f"f32 state rows={rows} cols={c} k={k} spans={spans}")
        check_case(mm, c, k, spans=spans, what=f"f32 {rows}x{c} spans={spans}", fmt="f32")


@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_argmax_f32(family):
    """k = 1 on fp32 rows runs the argmax scan: the oracle's bytes, and the
    same as the general scan (tk_options.general) over widths, strides,
    misaligned rows and span counts."""
    import wide_row_bf16_amd as tk
    from gpu_util import to_numpy

    fi = sorted(FAMILIES).index(family)
    for i, w in enumerate([1, 3, 4, 5, 63, 1000, 4099, 16384, 98592, 151936]):
        stride = [w, w + 1, w + 3][(i + fi) % 3]
        spans = [0, 1, 2, 7, 64][(i + fi) % 5]
        if spans > w:
            spans = 0
        offset = (i + fi) % 4
        m = family_rows(family, 3, w, stride, seed=900 + 13 * fi + i, fmt="f32")
        what = f"f32 k=1 family={family} cols={w} stride={stride} spans={spans} offset={offset}"
        log(what)
        want = oracle.topk_f32(m, w, 1)
        x = upload(m, offset)
        assert_same(to_numpy(tk.topk_f32(x, 1, cols=w, spans=spans)), want, what)
        assert_same(to_numpy(tk.topk_f32(x, 1, cols=w, spans=spans, general=True)), want, what + " (general)")


def test_argmax_f32_batches():
    import wide_row_bf16_amd as tk
    from gpu_util import to_numpy

    cols = 4100
    m = family_rows("normal", 4100, cols, cols, seed=23, fmt="f32")
    want = oracle.topk_f32(m, cols, 1)
    x = upload(m)
    for spans in (2, 0, 1, 4):
        log(f"f32 k=1 4100 rows spans={spans}")
        assert_same(to_numpy(tk.topk_f32(x, 1, cols=cols, spans=spans)), want, f"f32 k=1 4100 rows spans={spans}")


@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_wide_k_f32(family):
    """64 < k <= 256 on fp32 rows (the multi-register scan): the oracle's
    bytes over widths, strides, misaligned rows and span counts."""
    fi = sorted(FAMILIES).index(family)
    for i, w in enumerate([1, 9, 65, 257, 1000, 4103, 70000, 151936]):
        stride = [w, w + 1, w + 3][(i + fi) % 3]
        k = [65, 100, 128, 129, 200, 256][(i + 2 * fi) % 6]
        spans = [0, 1, 2, 8, 64][(i + fi) % 5]
        if spans > w:
            spans = 0
        offset = (i + fi) % 4
        m = family_rows(family, 2, w, stride, seed=4000 + 7 * fi + i, fmt="f32")
        what = f"f32 wide family={family} cols={w} stride={stride} k={k} spans={spans} offset={offset}"
        log(what)
        check_case(m, w, k, spans=spans, offset=offset, what=what, fmt="f32")


@pytest.mark.parametrize("family", ["ascending", "normal", "few_levels", "posinf_many"])
def test_wide_k_f32_speculation_and_batches(family):
    cols = 151936
    m = family_rows(family, 3, cols, cols, seed=len(family), fmt="f32")
    x = upload(m)
    for k in (65, 200):
        want = oracle.topk_f32(m, cols, k)
        for exact in (False, True):
            log(f"f32 wide speculate family={family} k={k} exact={exact}")
            assert_same(gpu_topk(m, cols, k, x=x, fmt="f32", exact=exact), want, f"{family} k={k} exact={exact}")
    if family == "normal":
        mm = family_rows("logit", 4100, 1100, 1100, seed=5, fmt="f32")
        want = oracle.topk_f32(mm, 1100, 128)
        xx = upload(mm)
        for spans in (2, 1, 2):
            log(f"f32 wide 4100 rows spans={spans}")
            assert_same(gpu_topk(mm, 1100, 128, spans=spans, x=xx, fmt="f32"), want, f"f32 wide 4100 spans={spans}")


@pytest.mark.parametrize("name", ["c2", "c5"])
def test_wide_k_f32_configs(name):
    cfg = CONFIGS[name]
    m = bf16_to_f32_bits(make_config_input(name), np.random.default_rng(3))
    x = upload(m)
    for k in (128, 256):
        log(f"f32 wide {name} k={k}")
        assert_same(gpu_topk(m, cfg.cols, k, x=x, fmt="f32"), oracle.topk_f32(m, cfg.cols, k), f"f32 {name} k={k}")
