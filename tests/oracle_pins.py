"""Pins for the CPU oracle: references that do not share its method.

The oracle sorts (value, column) pairs with a comparator.  Each pin below
reaches the same answer another way, so that a plausible mistake in the
oracle (a reversed order, ties to the wrong index, NaN kept, the two zeros
told apart, subnormals flushed, padding read, a wrong fill, a swapped mask
bit, a clipped count) fails at least one of them:

* ``rank_definition``: the O(n^2) rank of every element -- the number of
  non-NaN elements that beat it (larger value, or equal value at a lower
  column) -- computed with numpy broadcasting; entry j is the element of rank j;
* ``lexsort_reference``: numpy's stable lexsort on (column, -value);
* ``python_sorted_reference``: Python's stable ``sorted`` on (-value, column);
* closed forms and hand-derived worked examples;
* invariants that any correct answer satisfies.

Every function takes the oracle library handle, so the same pins also run
against deliberately broken copies of the oracle (``test_oracle_mutants``).
"""

from __future__ import annotations

import itertools
import json
import os

import numpy as np

import oracle
from synth import FAMILIES, family_rows

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")

# Ten symbols that cover every class of bf16 value once.
ALPHABET = np.array(
    [
        0x7FC0,  # +NaN (quiet)
        0xFF81,  # -NaN (signalling payload)
        0xFF80,  # -inf
        0xBF80,  # -1
        0x8001,  # -smallest subnormal
        0x8000,  # -0
        0x0000,  # +0
        0x0001,  # +smallest subnormal
        0x3F80,  # 1
        0x7F80,  # +inf
    ],
    dtype=np.uint16,
)


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly (numpy keeps subnormals)."""
    f32 = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    with np.errstate(invalid="ignore"):  # signalling-NaN payloads raise the invalid flag
        return f32.astype(np.float64)


def expected_mask(bits: np.ndarray, widen_fn=None) -> np.ndarray:
    v = (widen_fn or widen)(bits)
    return (np.isnan(v).any(axis=-1) * 1 | (v == np.inf).any(axis=-1) * 2 | (v == -np.inf).any(axis=-1) * 4).astype(np.uint32)


def rank_definition(bits: np.ndarray, k: int, widen_fn=None, word=np.uint16, fill=0x7FC0):
    """Top-k of each row of an (n, L) matrix of bit patterns (uint16, or
    uint32 with word/fill for fp32) by counting ranks (O(L^2) per row)."""
    bits = np.asarray(bits, dtype=word)
    n, L = bits.shape
    v = (widen_fn or widen)(bits)
    nan = np.isnan(v)
    vi = v[:, :, None]
    vj = v[:, None, :]
    lower = np.arange(L)[None, :] < np.arange(L)[:, None]  # [i, j]: j is left of i
    beats = ((vj > vi) | ((vj == vi) & lower[None])) & ~nan[:, None, :]
    rank = beats.sum(axis=2)
    rank[nan] = L + 1
    idx = np.full((n, k), -1, dtype=np.int32)
    val = np.full((n, k), fill, dtype=word)
    rows = np.arange(n)
    for j in range(min(k, L)):
        hit = rank == j
        has = hit.any(axis=1)
        where = hit.argmax(axis=1)
        idx[has, j] = where[has]
        val[has, j] = bits[rows[has], where[has]]
    count = np.minimum(k, (~nan).sum(axis=1)).astype(np.int32)
    return idx, val, count, expected_mask(bits, widen_fn)


def lexsort_reference(row: np.ndarray, k: int, widen_fn=None):
    v = (widen_fn or widen)(row)
    keep = np.nonzero(~np.isnan(v))[0]
    order = keep[np.lexsort((keep, -v[keep]))]
    return _pack(row, order, k, widen_fn)


def python_sorted_reference(row: np.ndarray, k: int, widen_fn=None):
    v = (widen_fn or widen)(row).tolist()
    order = sorted((c for c in range(len(v)) if v[c] == v[c]), key=lambda c: (-v[c], c))
    return _pack(row, np.array(order, dtype=np.int64), k, widen_fn)


def _pack(row, order, k, widen_fn=None):
    count = min(k, len(order))
    idx = np.full(k, -1, dtype=np.int32)
    val = np.full(k, 0x7FC0, dtype=np.uint16)
    idx[:count] = order[:count]
    val[:count] = row[order[:count]]
    return idx, val, count, int(expected_mask(row[None], widen_fn)[0])


def run(lib, m, cols, k, threads=1):
    return oracle.topk_bf16(m, cols, k, threads=threads, lib=lib)


def check_invariants(m: np.ndarray, cols: int, k: int, idx, val, cnt, mask, widen_fn=None, fill=0x7FC0):
    """Properties that hold for any correct answer, at any size."""
    body = m[:, :cols]
    v = (widen_fn or widen)(body)
    nan = np.isnan(v)
    assert np.array_equal(cnt, np.minimum(k, (~nan).sum(axis=1)))
    assert np.array_equal(mask, expected_mask(body, widen_fn))
    for r in range(m.shape[0]):
        c = int(cnt[r])
        e = idx[r, :c].astype(np.int64)
        assert np.all(idx[r, c:] == -1) and np.all(val[r, c:] == fill)
        assert np.all((e >= 0) & (e < cols))
        assert len(np.unique(e)) == c
        assert np.array_equal(val[r, :c], body[r, e])  # bits copied verbatim
        ev = v[r, e]
        assert not np.isnan(ev).any()
        # strictly ordered: value descending, equal values by ascending column
        assert np.all((ev[:-1] > ev[1:]) | ((ev[:-1] == ev[1:]) & (e[:-1] < e[1:])))
        if c == k and c > 0:
            rest = np.ones(cols, dtype=bool)
            rest[e] = False
            rest &= ~nan[r]
            last_v, last_c = ev[-1], e[-1]
            rv = v[r, rest]
            rc = np.nonzero(rest)[0]
            # every excluded non-NaN element ranks after the k-th entry
            assert np.all((rv < last_v) | ((rv == last_v) & (rc > last_c)))
        elif c < k:
            assert c == (~nan[r]).sum()


# --------------------------------------------------------------------------
# Pins, each usable against any oracle build.
# --------------------------------------------------------------------------


def pin_exhaustive(lib, max_len=5, ks=range(1, 7)):
    """Every row of length <= max_len over ALPHABET, against the rank definition."""
    for L in range(1, max_len + 1):
        rows = np.array(list(itertools.product(range(len(ALPHABET)), repeat=L)), dtype=np.int64)
        m = ALPHABET[rows]
        for k in ks:
            got = run(lib, m, L, k, threads=4)
            want = rank_definition(m, k)
            for g, w, name in zip(got, want, ("idx", "val", "count", "mask")):
                assert np.array_equal(g, w), f"len={L} k={k} {name} differs"


def pin_golden(lib):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        row = np.array([int(h, 16) for h in case["row"]], dtype=np.uint16)[None]
        idx, val, cnt, mask = run(lib, row, row.shape[1], case["k"])
        assert idx[0].tolist() == case["idx"], case["name"]
        assert [f"{x:04X}" for x in val[0]] == case["val"], case["name"]
        assert int(cnt[0]) == case["count"], case["name"]
        assert int(mask[0]) == case["mask"], case["name"]


def pin_library_sorts(lib, widths=(1, 2, 7, 33, 64, 65, 257), ks=(1, 5, 64), seed=1):
    """Random rows of every family against numpy lexsort and Python sorted."""
    for fi, fam in enumerate(sorted(FAMILIES)):
        for w in widths:
            m = family_rows(fam, 3, w, w, seed=seed * 1000 + fi * 17 + w)
            for k in ks:
                got = run(lib, m, w, k)
                for r in range(3):
                    for ref in (lexsort_reference, python_sorted_reference):
                        idx, val, cnt, mask = ref(m[r], k)
                        assert np.array_equal(got[0][r], idx), (fam, w, k, ref.__name__)
                        assert np.array_equal(got[1][r], val), (fam, w, k, ref.__name__)
                        assert int(got[2][r]) == cnt and int(got[3][r]) == mask, (fam, w, k)


def pin_padding(lib):
    """Padding is never read: a strided matrix with poison gives the compact answer."""
    for fam in ("normal", "nan_sprinkled", "neginf_all", "zeros"):
        for cols, stride in ((1, 2), (7, 9), (64, 192), (100, 101)):
            m = family_rows(fam, 4, cols, stride, seed=cols)
            compact = np.ascontiguousarray(m[:, :cols])
            for k in (1, 3, 64):
                a = run(lib, m, cols, k)
                b = rank_definition(compact, k)
                for x, y in zip(a, b):
                    assert np.array_equal(x, y), (fam, cols, stride, k)


def pin_closed_forms(lib):
    k = 6
    # all equal -> the first k columns
    m = np.full((2, 20), 0x4000, dtype=np.uint16)
    idx, val, cnt, mask = run(lib, m, 20, k)
    assert idx.tolist() == [list(range(k))] * 2 and cnt.tolist() == [k, k] and mask.tolist() == [0, 0]
    # strictly ascending -> the last k columns, last first
    asc = np.arange(0x3F80, 0x3F80 + 20, dtype=np.uint16)[None]
    idx, *_ = run(lib, asc, 20, k)
    assert idx[0].tolist() == list(range(19, 19 - k, -1))
    # strictly descending -> the first k columns
    idx, *_ = run(lib, asc[:, ::-1].copy(), 20, k)
    assert idx[0].tolist() == list(range(k))
    # negative ascending bits are descending values: 0xBF80 (-1) > 0xBF81 > ...
    neg = np.arange(0xBF80, 0xBF80 + 20, dtype=np.uint16)[None]
    idx, *_ = run(lib, neg, 20, k)
    assert idx[0].tolist() == list(range(k))
    # all NaN -> count 0, NaN flag, all slots filled
    nan = np.array([[0x7FC0, 0xFFC0, 0x7F81, 0xFFFF]], dtype=np.uint16)
    idx, val, cnt, mask = run(lib, nan, 4, k)
    assert cnt.tolist() == [0] and mask.tolist() == [1]
    assert idx[0].tolist() == [-1] * k and val[0].tolist() == [0x7FC0] * k
    # all -inf but one finite value -> the finite column, then the lowest -inf columns
    row = np.full((1, 30), 0xFF80, dtype=np.uint16)
    row[0, 17] = 0xC2C8  # -100
    idx, val, cnt, mask = run(lib, row, 30, 16)
    assert idx[0].tolist() == [17] + list(range(15)) and mask.tolist() == [4]
    # more +inf than k -> the first k +inf columns
    row = np.full((1, 40), 0x3F80, dtype=np.uint16)
    pinf = [3, 5, 8, 13, 21, 34, 36, 39]
    row[0, pinf] = 0x7F80
    row[0, 0] = 0xFF80
    row[0, 1] = 0x7FC0
    idx, val, cnt, mask = run(lib, row, 40, 5)
    assert idx[0].tolist() == pinf[:5] and val[0].tolist() == [0x7F80] * 5 and mask.tolist() == [7]
    # k larger than cols
    row = np.array([[0x3F80, 0x4000]], dtype=np.uint16)
    idx, val, cnt, mask = run(lib, row, 2, 4)
    assert idx[0].tolist() == [1, 0, -1, -1] and cnt.tolist() == [2]
    # cols == 0: nothing to rank
    idx, val, cnt, mask = run(lib, np.zeros((3, 0), dtype=np.uint16), 0, 2)
    assert cnt.tolist() == [0, 0, 0] and mask.tolist() == [0, 0, 0] and (idx == -1).all()


def pin_invariants(lib, widths=(4096, 4103, 9000), ks=(1, 16, 64), seed=7):
    for fi, fam in enumerate(sorted(FAMILIES)):
        for w in widths:
            m = family_rows(fam, 2, w, w + 3, seed=seed + fi * 31 + w)
            for k in ks:
                check_invariants(m, w, k, *run(lib, m, w, k))


ALL_PINS = (pin_exhaustive, pin_golden, pin_library_sorts, pin_padding, pin_closed_forms, pin_invariants)
