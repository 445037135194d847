"""Vocabulary-sharded top-k on one GPU: every row's columns are cut into
shards, each shard's top k is taken with its global column base
(tk_topk_bf16_shard), the shard results are stacked shard-major and merged
(tk_merge_topk_bf16); the result must be the oracle's top k of the whole row,
byte for byte.  This is the span split and same-order merge of TensorFold PR
#713 (change 3) carried across devices, emulated on one device."""

import numpy as np
import pytest

import oracle
from gpu_util import assert_same, log, need_gpu, to_numpy, upload
from synth import family_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def sharded_topk(x, cols, k, bounds):
    """bounds: increasing column cuts from 0 to cols (len = shards + 1)."""
    import torch

    import wide_row_bf16_amd as tk

    parts = [tk.topk_bf16_shard(x[:, a:b], k, a) for a, b in zip(bounds[:-1], bounds[1:])]
    stacked = [torch.stack([getattr(p, f) for p in parts]).contiguous() for f in ("idx", "val", "count", "nonfinite")]
    return to_numpy(tk.merge_topk_bf16(*stacked))


def even(cols, g):
    return [cols * i // g for i in range(g + 1)]


SPLITS = {
    "one": lambda c: [0, c],
    "even8": lambda c: even(c, 8),
    "ragged": lambda c: sorted([0, 1, 7, 9, 64, 4096, c // 3, c // 3, c // 2 + 5, c - 3, c]),  # one shard is empty
    "tiny64": lambda c: even(c, 64),
}


@pytest.mark.parametrize("split", sorted(SPLITS))
@pytest.mark.parametrize("family", ["normal", "levels64", "zeros_straddle", "mixed_nonfinite", "all_equal",
                                    "neginf_one_finite", "all_nan", "descending"])
def test_sharded_equals_whole_row(family, split):
    cols = 151936 if split != "tiny64" else 3000
    m = family_rows(family, 3, cols, cols, seed=len(family) * 7 + len(split))
    x = upload(m)
    bounds = SPLITS[split](cols)
    for k in (1, 20, 64):
        log(f"sharded family={family} split={split} shards={len(bounds) - 1} k={k}")
        assert_same(sharded_topk(x, cols, k, bounds), oracle.topk_bf16(m, cols, k), f"{family} {split} k={k}")


def test_sharded_full_rows():
    """1024 rows split in 8 shards of 18992 columns (a vocab-parallel head's
    shape on 8 devices)."""
    from synth import make_config_input

    m = make_config_input("c5")
    x = upload(m)
    log("sharded 1024x151936 into 8")
    assert_same(sharded_topk(x, 151936, 64, even(151936, 8)), oracle.topk_bf16(m, 151936, 64), "c5 sharded")


def test_merge_of_shards_with_fewer_entries_than_k():
    """Shards narrower than k, and shards with no entries at all, still merge
    to the whole row's result (count = min(k, total), fill after it)."""
    m = family_rows("nan_sprinkled", 4, 90, 90, seed=3)
    x = upload(m)
    for bounds in ([0, 10, 20, 30, 60, 90], [0, 0, 45, 45, 90], [0, 1, 2, 3, 90]):
        log(f"narrow shards {bounds}")
        assert_same(sharded_topk(x, 90, 64, bounds), oracle.topk_bf16(m, 90, 64), f"narrow {bounds}")
