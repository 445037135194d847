"""Parity of the HIP top-k on IEEE fp16 rows (tk_topk_f16) with the
oracle's fp16 path, byte for byte in all four outputs: every synthetic
family re-encoded as fp16 over widths, strides, k, forced span counts and
misaligned rows; the split path equal to the single-group control; the
speculative floor and the exact mode; the workload shapes at full size."""

import numpy as np
import pytest

import oracle
from gpu_util import assert_same, check_case, gpu_topk, log, need_gpu, upload
from synth import CONFIGS, FAMILIES, bf16_to_f16_bits, family_rows, make_config_input

pytestmark = pytest.mark.gpu

WIDTHS = [1, 9, 65, 1000, 4103, 32768, 98592, 151936]
KS = [1, 8, 20, 33, 64]
SPANS = [0, 1, 3, 16]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_family_widths_f16(family):
    fi = sorted(FAMILIES).index(family)
    for i, w in enumerate(WIDTHS):
        stride = [w, w + 1, w + 3, -(-w // 64) * 64][(i + fi) % 4]
        k = KS[(i + fi) % len(KS)]
        spans = SPANS[(i + 2 * fi) % len(SPANS)]
        if spans > w:
            spans = 0
        offset = (i + fi) % 8
        m = family_rows(family, 3, w, stride, seed=500 + 10 * fi + i, fmt="f16")
        what = f"f16 family={family} cols={w} stride={stride} k={k} spans={spans} offset={offset}"
        log(what)
        check_case(m, w, k, spans=spans, offset=offset, what=what, fmt="f16")


@pytest.mark.parametrize("family", ["normal", "levels64", "mixed_nonfinite", "uniform_bits", "zeros_straddle"])
def test_split_and_exact_f16(family):
    cols = 248320
    m = family_rows(family, 3, cols, cols, seed=21, fmt="f16")
    x = upload(m)
    for k in (1, 20, 64):
        want = oracle.topk_f16(m, cols, k)
        for spans in (1, 2, 7, 12, 64, 65, 130):  # above 64: the merge dispatch
            log(f"f16 split family={family} k={k} spans={spans}")
            assert_same(gpu_topk(m, cols, k, spans=spans, x=x, fmt="f16"), want, f"{family} k={k} spans={spans}")
        assert_same(gpu_topk(m, cols, k, spans=1, x=x, fmt="f16", exact=True), want, f"{family} k={k} exact")


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
def test_configs_full_size_f16(name):
    cfg = CONFIGS[name]
    m = bf16_to_f16_bits(make_config_input(name))
    log(f"f16 config {name}")
    want = oracle.topk_f16(m, cfg.cols, cfg.k)
    x = upload(m)
    for spans in (0, 1):
        assert_same(gpu_topk(m, cfg.cols, cfg.k, spans=spans, x=x, fmt="f16"), want, f"f16 {name} spans={spans}")
