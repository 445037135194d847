"""The k = 1 fast path (argmax scan) against the CPU oracle, byte for byte,
and against the general top-k scan run as its control (tk_options.general).

k = 1 is the greedy decode step of the drafter on the pages (its draft head
takes the best token of each row).  The order is the same as for every k:
highest score first, the lower column on equal scores, +0 and -0 equal, NaN
never an entry (flagged), infinities ranked (TensorFold PR #713, change 3
and its exactness table).
"""

import numpy as np
import pytest

import oracle
from gpu_util import assert_same, gpu_topk, log, need_gpu, to_numpy, upload
from synth import CONFIGS, FAMILIES, family_rows, make_config_input

pytestmark = pytest.mark.gpu

WIDTHS = [1, 5, 8, 9, 63, 520, 2047, 2048, 4096, 4103, 9000, 65537, 98592, 151936, 248320]
SPANS = [0, 1, 2, 3, 7, 16, 35, 64]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def control(x, cols, spans=0, fmt="bf16"):
    import wide_row_bf16_amd as tk

    fn = {"bf16": tk.topk_bf16, "f16": tk.topk_f16}[fmt]
    return to_numpy(fn(x, 1, cols=cols, spans=spans, general=True))


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_family_widths(family, fmt):
    fi = sorted(FAMILIES).index(family)
    for i, w in enumerate(WIDTHS):
        stride = [w, w + 1, w + 3, w + 128][(i + fi) % 4]
        spans = SPANS[(i + fi) % len(SPANS)]
        if spans > w:
            spans = 0
        offset = (3 * i + fi) % 8
        rows = 4 if w < 100000 else 2
        m = family_rows(family, rows, w, stride, seed=500 + 97 * fi + i, fmt=fmt)
        what = f"{fmt} family={family} rows={rows} cols={w} stride={stride} spans={spans} offset={offset}"
        log(what)
        want = (oracle.topk_bf16 if fmt == "bf16" else oracle.topk_f16)(m, w, 1)
        x = upload(m, offset)
        assert_same(gpu_topk(m, w, 1, spans=spans, x=x, fmt=fmt), want, what)
        assert_same(control(x, w, spans, fmt), want, what + " (general scan)")


@pytest.mark.parametrize("family", ["normal", "levels64", "all_equal", "zeros_straddle", "mixed_nonfinite",
                                    "neginf_one_finite", "posinf_many", "uniform_bits"])
def test_every_span_count(family):
    """The result does not depend on the split (the pages' split == control
    check), for every span count the fast path takes."""
    cols = 98592
    m = family_rows(family, 3, cols, cols + 8, seed=len(family))
    want = oracle.topk_bf16(m, cols, 1)
    x = upload(m, 1)
    for spans in list(range(1, 17)) + [24, 31, 32, 33, 47, 48, 63, 64]:
        log(f"argmax family={family} spans={spans}")
        assert_same(gpu_topk(m, cols, 1, spans=spans, x=x), want, f"{family} spans={spans}")


def _row_with(cols, placements, fill=0x3F80):
    """One bf16 row of `fill` with the given (column, bits) placed."""
    r = np.full(cols, fill, dtype=np.uint16)
    for c, b in placements:
        r[c] = b
    return r


def test_ties_and_classes_at_span_and_wave_edges():
    """The maximum placed at head, tail, span and wave boundaries, tied across
    them (the lower column wins), as -0 before +0, behind NaN, and as +inf."""
    cols = 98592
    S = 16
    nv = cols // 8
    edges = sorted({0, 1, 7, 8, cols - 1, cols - 8, cols - 9}
                   | {8 * (nv * s // S) + d for s in range(1, S) for d in (-1, 0, 1)}
                   | {8 * (nv * s // (4 * S)) for s in range(1, 4 * S)})
    rows = []
    for i, c in enumerate(edges):
        d = edges[(i * 7 + 3) % len(edges)]
        rows.append(_row_with(cols, [(c, 0x4100), (d, 0x4100)]))          # tie: the lower column
        rows.append(_row_with(cols, [(c, 0x7F80), (d, 0x7FC1)], 0xBF80))  # +inf, a NaN elsewhere
    rows.append(_row_with(cols, [(5, 0x8000), (9, 0x0000)], 0xC000))      # -0 before +0: -0 (bits 8000)
    rows.append(_row_with(cols, [(5, 0x0000), (9, 0x8000)], 0xC000))      # +0 before -0: +0
    rows.append(_row_with(cols, [(c, 0xFFC0) for c in range(0, cols, 3)], 0xFF80))  # -inf with NaN
    rows.append(np.full(cols, 0x7FC0, dtype=np.uint16))                  # all NaN: count 0
    m = np.stack(rows)
    want = oracle.topk_bf16(m, cols, 1)
    for offset in (0, 3):
        x = upload(m, offset)
        for spans in (0, 1, 2, S, 64):
            log(f"edges offset={offset} spans={spans}")
            assert_same(gpu_topk(m, cols, 1, spans=spans, x=x), want, f"edges offset={offset} spans={spans}")


def test_rows_beyond_one_batch():
    """More rows than one launch of the split path takes (4096): the second
    batch reuses the arrival counters and slots."""
    cols = 4160
    m = family_rows("logit", 4100, cols, cols, seed=11)
    want = oracle.topk_bf16(m, cols, 1)
    x = upload(m)
    for spans in (2, 0, 1, 2):
        log(f"4100 rows spans={spans}")
        assert_same(gpu_topk(m, cols, 1, spans=spans, x=x), want, f"4100 rows spans={spans}")


def test_state_across_calls_and_streams():
    """Split calls of different shapes back to back, on the default and on a
    second stream: the counters return to zero after every row."""
    import torch

    import wide_row_bf16_amd as tk

    cases = []
    for j, (rows, cols, spans) in enumerate([(15, 98592, 35), (3, 248320, 64), (40, 9000, 4), (1, 4096, 2),
                                             (15, 98592, 0), (64, 151936, 0)]):
        m = family_rows(["normal", "mixed_nonfinite", "levels64"][j % 3], rows, cols, cols, seed=j)
        cases.append((m, cols, spans, upload(m), oracle.topk_bf16(m, cols, 1)))
    side = torch.cuda.Stream()
    for rep in range(3):
        for m, cols, spans, x, want in cases:
            log(f"state rep={rep} rows={m.shape[0]} cols={cols} spans={spans}")
            assert_same(gpu_topk(m, cols, 1, spans=spans, x=x), want, f"default stream {m.shape} spans={spans}")
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                out = tk.topk_bf16(x, 1, cols=cols, spans=spans)
            torch.cuda.current_stream().wait_stream(side)
            assert_same(to_numpy(out), want, f"side stream {m.shape} spans={spans}")


def test_cols_zero_and_row_subset():
    import wide_row_bf16_amd as tk

    m = family_rows("normal", 5, 300, 300, seed=2)
    x = upload(m)
    got = to_numpy(tk.topk_bf16(x, 1, cols=0))
    assert list(got[0][:, 0]) == [-1] * 5 and list(got[1][:, 0]) == [0x7FC0] * 5
    assert list(got[2]) == [0] * 5 and list(got[3]) == [0] * 5
    for cols in (1, 2, 17, 299):
        assert_same(gpu_topk(m, cols, 1, x=x), oracle.topk_bf16(m, cols, 1), f"cols={cols}")


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_configs(name):
    """The five workload shapes at full size with k = 1 (automatic plan and
    the general control)."""
    cfg = CONFIGS[name]
    m = make_config_input(name)
    want = oracle.topk_bf16(m, cfg.cols, 1)
    x = upload(m)
    log(f"{name} k=1")
    assert_same(gpu_topk(m, cfg.cols, 1, x=x), want, f"{name} k=1")
    assert_same(control(x, cfg.cols), want, f"{name} k=1 general")
    # a forced plan always takes the argmax scan (with a row per CU the
    # automatic plan takes the general one)
    assert_same(gpu_topk(m, cfg.cols, 1, spans=1, x=x), want, f"{name} k=1 argmax spans=1")
