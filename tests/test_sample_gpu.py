"""Seeded top-p sampling on the GPU (tk_sample_topk_bf16) against the
sampling oracle: tokens and kept counts equal, row by row, for top-k results
of synthetic rows of every kind and for hand-built entry lists."""

import numpy as np
import pytest

import oracle
from oracle.sampling import sample_topk
from gpu_util import log, need_gpu, upload
from synth import family_rows

pytestmark = pytest.mark.gpu

PARAMS = [(0.7, 0.95), (1.0, 1.0), (0.0, 0.9), (2.5, 0.5), (0.05, 0.999), (1e-3, 1e-6), (30.0, 0.95)]
SEEDS = [1234, 2**63 + 5]
OFFSETS = [0, 7, 2**40 + 3]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def f32(x):
    return float(np.float32(x))


def gpu_sample(idx, val, count, t, p, seed, off):
    import torch

    import wide_row_bf16_amd as tk

    topk = tk.TopK(torch.from_numpy(np.ascontiguousarray(idx)).cuda(),
                   torch.from_numpy(np.ascontiguousarray(val).view(np.int16)).cuda().view(torch.bfloat16),
                   torch.from_numpy(np.ascontiguousarray(count)).cuda(),
                   torch.zeros(count.shape[0], dtype=torch.int32, device="cuda"))
    tok, kept = tk.sample_topk_bf16(topk, t, p, seed, off)
    return tok.cpu().numpy(), kept.cpu().numpy()


def check(idx, val, count, what):
    for t, p in PARAMS:
        for seed in SEEDS:
            for off in OFFSETS:
                want = sample_topk(idx, val, count, f32(t), f32(p), seed, off)
                got = gpu_sample(idx, val, count, t, p, seed, off)
                for g, w, name in zip(got, want, ("token", "kept")):
                    if not np.array_equal(g, w):
                        r = int(np.argwhere(g != w)[0][0])
                        raise AssertionError(f"{what} T={t} p={p} seed={seed} off={off}: {name} row {r} "
                                             f"gpu {g[r]} oracle {w[r]}")


@pytest.mark.parametrize("family", ["logit", "normal", "levels64", "mixed_nonfinite", "zeros_straddle", "posinf_few",
                                    "neginf_one_finite", "all_nan", "all_equal"])
def test_sampling_of_topk_rows(family):
    cols = 20000
    m = family_rows(family, 6, cols, cols, seed=11)
    for k in (1, 20, 64):
        idx, val, count, _ = oracle.topk_bf16(m, cols, k)
        log(f"sample family={family} k={k}")
        check(idx, val, count, f"{family} k={k}")


def test_sampling_of_built_entry_lists():
    def bits(v):
        b = np.array(v, dtype=np.float32).view(np.uint32) >> 16
        return b.astype(np.uint16)

    k = 8
    rows = [
        ([1.0] * 8, 8),                                                  # equal weights
        ([np.inf, np.inf, 1.0, 0.5, 0.0, -1.0, -np.inf, -np.inf], 8),    # +inf first
        ([2.0, 1.0, -np.inf, -np.inf, -np.inf, 0, 0, 0], 5),             # -inf tail
        ([-np.inf] * 8, 3),                                              # only -inf
        ([3.0, 2.0, 1.0, 0, 0, 0, 0, 0], 0),                             # no entries
        ([100.0, -100.0, -200.0, -300.0, 0, 0, 0, 0], 4),                # far below the top
        ([0.0, -0.0, 0.0, -0.0, -1.0, -2.0, -3.0, -4.0], 8),             # both zeros
    ]
    val = np.stack([bits(v) for v, _ in rows])
    count = np.array([c for _, c in rows], dtype=np.int32)
    idx = np.arange(len(rows) * k, dtype=np.int32).reshape(len(rows), k) * 3 + 1
    idx[count[:, None] <= np.arange(k)[None, :]] = -1
    log("sample built lists")
    check(idx, val, count, "built")


def test_sampling_many_rows():
    import torch

    import wide_row_bf16_amd as tk

    m = family_rows("logit", 1024, 4096, 4096, seed=99)
    x = upload(m)
    res = tk.topk_bf16(x, 64)
    idx, val, count = (t.cpu().numpy() for t in (res.idx, res.val.view(torch.int16), res.count))
    val = val.view(np.uint16)
    for t, p in ((0.7, 0.95), (1.3, 0.8)):
        log(f"sample 1024 rows T={t} p={p}")
        want = sample_topk(idx, val, count, f32(t), f32(p), 1234, 5)
        tok, kept = tk.sample_topk_bf16(res, t, p, 1234, 5)
        assert np.array_equal(tok.cpu().numpy(), want[0]) and np.array_equal(kept.cpu().numpy(), want[1])
