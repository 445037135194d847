"""The automatic plan on 86 to 255 rows, where the 16-bit scan takes twice the
spans the CU count asks for, and on few rows at k <= 32, where it takes 8 to
12 spans by the row's width: parity with the oracle, byte for byte, on the
shapes that pick each branch (and a row width that caps the doubling), and
the same doubling in the k > 64 and fp32 scans."""

import pytest

import oracle
import wide_row_bf16_amd as tk
from gpu_util import assert_same, gpu_topk, log, need_gpu
from synth import family_rows

pytestmark = pytest.mark.gpu

CASES = [
    # rows, cols, k, family
    (96, 98592, 32, "normal"),
    (128, 151936, 64, "normal"),
    (200, 20000, 16, "few_levels"),
    (255, 9000, 8, "nan_sprinkled"),
    (128, 12288, 32, "normal"),        # doubling capped by the 4096-column span floor
    (15, 49152, 32, "normal"),         # 8 spans at k <= 32
    (15, 151936, 20, "neginf_one_finite"),
    (15, 98592, 64, "normal"),         # k = 64 keeps 12
    (3, 98592, 32, "normal"),          # 1 to 5 rows: 16 spans
    (1, 151936, 32, "few_levels"),
    (4, 248320, 20, "nan_sprinkled"),
    (2, 40000, 64, "posinf_many"),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("rows,cols,k,family", CASES)
def test_automatic_plan_parity(rows, cols, k, family):
    m = family_rows(family, rows, cols, cols + 8, seed=rows * 31 + k)
    log(f"plan parity {rows}x{cols} k={k} {family} spans={tk.plan_spans(rows, cols, k)}")
    assert_same(gpu_topk(m, cols, k, spans=0), oracle.topk_bf16(m, cols, k), f"{rows}x{cols} k={k} {family}")


# the k > 64 and fp32 scans double their spans on the same row counts
WIDE_CASES = [(128, 98592, 128, "bf16"), (96, 40000, 256, "bf16"), (128, 98592, 32, "f32"),
              (200, 30000, 200, "f32"), (96, 8192, 64, "f32")]


@pytest.mark.parametrize("rows,cols,k,fmt", WIDE_CASES)
def test_automatic_plan_parity_wide_and_fp32(rows, cols, k, fmt):
    m = family_rows("normal", rows, cols, cols, seed=rows * 17 + k, fmt=fmt)
    want = (oracle.topk_bf16 if fmt == "bf16" else oracle.topk_f32)(m, cols, k)
    log(f"plan parity {fmt} {rows}x{cols} k={k}")
    assert_same(gpu_topk(m, cols, k, spans=0, fmt=fmt), want, f"{fmt} {rows}x{cols} k={k}")
