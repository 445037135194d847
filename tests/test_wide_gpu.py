"""64 < k <= 256 (the multi-register scan) against the CPU oracle, byte for
byte in all four outputs, over the exactness cases of TensorFold PR #713
(ties, both zeros, NaN, infinities, padded strides, split == single group),
the workload shapes at full size, k beyond the row width, batches of split
rows, and state kept across calls.
"""

import numpy as np
import pytest

import oracle
from gpu_util import assert_same, gpu_topk, log, need_gpu, to_numpy, upload
from synth import CONFIGS, FAMILIES, family_rows, make_config_input

pytestmark = pytest.mark.gpu

WIDTHS = [1, 9, 64, 65, 200, 257, 1000, 4096, 4103, 9000, 65537, 98592, 151936, 248320]
KS = [65, 100, 128, 129, 200, 255, 256]
SPANS = [0, 1, 2, 3, 8, 16, 64]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_family_widths(family, fmt):
    fi = sorted(FAMILIES).index(family)
    for i, w in enumerate(WIDTHS):
        stride = [w, w + 1, w + 3, w + 128][(i + fi) % 4]
        k = KS[(i + 2 * fi) % len(KS)]
        spans = SPANS[(i + fi) % len(SPANS)]
        if spans > w:
            spans = 0
        offset = (5 * i + fi) % 8
        rows = 3 if w < 100000 else 2
        m = family_rows(family, rows, w, stride, seed=7000 + 31 * fi + i, fmt=fmt)
        what = f"{fmt} family={family} rows={rows} cols={w} stride={stride} k={k} spans={spans} offset={offset}"
        log(what)
        want = (oracle.topk_bf16 if fmt == "bf16" else oracle.topk_f16)(m, w, k)
        assert_same(gpu_topk(m, w, k, spans=spans, offset=offset, fmt=fmt), want, what)


@pytest.mark.parametrize("k", [65, 128, 256])
@pytest.mark.parametrize("family", ["normal", "levels64", "all_equal", "zeros_straddle", "mixed_nonfinite",
                                    "posinf_many", "neginf_one_finite", "ascending", "uniform_bits"])
def test_split_equals_single_group(family, k):
    cols = 98592
    m = family_rows(family, 3, cols, cols + 8, seed=len(family) + k)
    want = oracle.topk_bf16(m, cols, k)
    x = upload(m, 3)
    for spans in (1, 2, 3, 5, 8, 13, 32, 64):
        log(f"wide family={family} k={k} spans={spans}")
        assert_same(gpu_topk(m, cols, k, spans=spans, x=x), want, f"{family} k={k} spans={spans}")


def test_every_k_on_one_row_set():
    cols = 20000
    m = family_rows("few_levels", 4, cols, cols, seed=3)
    x = upload(m)
    for k in range(65, 257, 7):
        log(f"wide k={k}")
        assert_same(gpu_topk(m, cols, k, x=x), oracle.topk_bf16(m, cols, k), f"k={k}")
        assert_same(gpu_topk(m, cols, k, spans=4, x=x), oracle.topk_bf16(m, cols, k), f"k={k} spans=4")


def test_rows_beyond_one_batch_and_state():
    """4100 split rows (two launches of the fused fold), then other shapes on
    the same stream: the arrival counters return to zero after every row."""
    cols = 4160
    m = family_rows("logit", 4100, cols, cols, seed=13)
    want = oracle.topk_bf16(m, cols, 100)
    x = upload(m)
    for spans in (2, 1, 2):
        log(f"wide 4100 rows spans={spans}")
        assert_same(gpu_topk(m, cols, 100, spans=spans, x=x), want, f"4100 rows spans={spans}")
    cases = [(15, 98592, 256, 0), (3, 248320, 129, 64), (40, 9000, 200, 4)]
    for rep in range(2):
        for rows, c, k, spans in cases:
            mm = family_rows("mixed_nonfinite", rows, c, c, seed=rows + rep)
            log(f"wide state rep={rep} rows={rows} cols={c} k={k} spans={spans}")
            assert_same(gpu_topk(mm, c, k, spans=spans), oracle.topk_bf16(mm, c, k), f"{rows}x{c} k={k}")


def test_shard_with_large_k():
    """A column shard with its global base (tk_topk_bf16_shard) at k > 64."""
    import wide_row_bf16_amd as tk

    cols = 151936
    m = family_rows("normal", 4, cols, cols, seed=21)
    x = upload(m)
    base = 18992 * 3
    part = to_numpy(tk.topk_bf16_shard(x[:, base:base + 18992], 128, base))
    want = oracle.topk_bf16(np.ascontiguousarray(m[:, base:base + 18992]), 18992, 128)
    want = (np.where(want[0] >= 0, want[0] + base, want[0]),) + tuple(want[1:])
    assert_same(part, want, "shard k=128")


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
@pytest.mark.parametrize("k", [128, 256])
def test_configs(name, k):
    cfg = CONFIGS[name]
    m = make_config_input(name)
    log(f"{name} k={k}")
    assert_same(gpu_topk(m, cfg.cols, k), oracle.topk_bf16(m, cfg.cols, k), f"{name} k={k}")


@pytest.mark.parametrize("family", ["ascending", "descending", "normal", "few_levels", "posinf_many", "max_last"])
def test_speculative_floor_and_rescan(family):
    """Wide spans take a speculative floor from the first chunks and verify
    it; on rows where it fails (ascending rows: the sample holds the smallest
    values) the span is scanned again.  Both the default and the exact option
    give the oracle's bytes."""
    cols = 151936
    m = family_rows(family, 3, cols, cols, seed=len(family) * 3)
    x = upload(m)
    for k in (65, 128, 256):
        want = oracle.topk_bf16(m, cols, k)
        for exact in (False, True):
            log(f"wide speculate family={family} k={k} exact={exact}")
            assert_same(gpu_topk(m, cols, k, x=x, exact=exact), want, f"{family} k={k} exact={exact}")
