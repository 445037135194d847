"""The allocation-free entry point tk_topk_bf16_noalloc, called through the C
ABI, against tk_topk_bf16 on the same inputs: every output byte equal, on two
calls in a row with the second one smaller (the fixed scratch array keeps the
first call's contents), across the scan's split paths -- fused folds of
split rows, the argmax scan's span slots, the multi-register scan's lists
in row batches that shrink to fit the array -- and the one-span path that
needs no scratch.  A row whose span lists cannot fit the array is rejected
before any launch, with nothing written."""

import numpy as np
import pytest

import oracle
from gpu_util import assert_same, log, need_gpu, to_numpy, upload
from synth import family_rows, make_config_input

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _outputs(rows, k):
    import torch

    import wide_row_bf16_amd as tk

    return tk.TopK(torch.full((rows, k), SENTINEL, dtype=torch.int32, device="cuda"),
                   torch.full((rows, k), SENTINEL, dtype=torch.int16, device="cuda"),
                   torch.full((rows,), SENTINEL, dtype=torch.int32, device="cuda"),
                   torch.full((rows,), SENTINEL, dtype=torch.int32, device="cuda"))


def _call(name, x, rows, cols, stride, k, out):
    import torch

    import wide_row_bf16_amd as tk

    stream = torch.cuda.current_stream().cuda_stream
    return int(getattr(tk.load(), name)(rows, cols, stride, k, x.data_ptr(), out.idx.data_ptr(), out.val.data_ptr(),
                                        out.count.data_ptr(), out.nonfinite.data_ptr(), stream))


def _both(m, cols, k, what, oracle_too=False):
    rows, stride = m.shape
    log(f"noalloc {what}: {rows}x{cols} stride {stride} k={k}")
    x = upload(m)
    want, got = _outputs(rows, k), _outputs(rows, k)
    assert _call("tk_topk_bf16", x, rows, cols, stride, k, want) == 0
    assert _call("tk_topk_bf16_noalloc", x, rows, cols, stride, k, got) == 0
    w = to_numpy(want)
    assert_same(to_numpy(got), w, f"noalloc {what}")
    if oracle_too:
        assert_same(w, oracle.topk_bf16(m, cols, k), f"tk_topk_bf16 {what}")


CASES = [
    # (first call, second call: smaller), each (family or config, rows, cols, stride, k)
    (("c2", 15, 98592, 98592, 32), ("mixed_nonfinite", 3, 20000, 20003, 20)),   # fused folds, S = 8 then 4
    (("normal", 15, 98592, 98592, 1), ("logit", 4, 40000, 40000, 1)),            # argmax span slots
    # k > 64 with 62 spans a row (the span width limit): 17 rows need 2.16 MB of lists, so two row batches
    (("normal", 17, 16_000_000, 16_000_000, 256), ("normal", 15, 98592, 98592, 128)),
    (("c4", 64, 151936, 152064, 16), ("c3", 16, 248320, 248448, 20)),            # fills, -inf rows; non-finite mix
    (("uniform_bits", 300, 30000, 30001, 64), ("zeros_straddle", 20, 5000, 5000, 64)),  # one span per row; no scratch
    (("levels64", 3, 261121, 261121, 256), ("ascending", 2, 70000, 70000, 200)),  # span width limit; speculation fails
]


def _input(spec):
    name, rows, cols, stride, k = spec
    if name.startswith("c") and name[1:].isdigit():
        return make_config_input(name)
    return family_rows(name, rows, cols, stride, seed=rows + cols + k)


@pytest.mark.parametrize("case", CASES, ids=[f"{a[0]}{a[1]}x{a[2]}k{a[4]}-then-{b[0]}{b[1]}x{b[2]}k{b[4]}"
                                             for a, b in CASES])
def test_noalloc_equals_topk_twice(case):
    for i, spec in enumerate(case):
        _both(_input(spec), spec[2], spec[4], f"call {i + 1} {spec[0]}", oracle_too=(i == 1))


def test_noalloc_rejects_a_row_beyond_the_array():
    """One row of 1.1e9 columns at k = 64 splits into 4213 spans, whose lists
    alone exceed the 2 MiB array: TK_ERR_SCRATCH, nothing launched, nothing
    written.  The input is a real allocation of that size, so no access can
    leave it whatever happens."""
    import torch

    import wide_row_bf16_amd as tk

    cols, k = 1_100_000_000, 64
    x = torch.empty((cols,), dtype=torch.int16, device="cuda")
    out = _outputs(1, k)
    assert _call("tk_topk_bf16_noalloc", x, 1, cols, cols, k, out) == 8
    assert tk.load().tk_status_string(8)
    for t in out:
        assert np.all(t.cpu().numpy() == SENTINEL)
    del x
