"""Pins of the sampling oracle (oracle/sampling.py) against things other
than itself: the published known-answer vectors of Philox4x32-10, the
mathematical 2^t, exact top-p boundaries, closed forms, and the sampled
frequencies against the softmax probabilities."""

import math

import numpy as np
import pytest

from oracle.sampling import exp2_f32, philox4x32_10, sample_row, sample_topk


def bf16(x):
    """bf16 bits of a float32 that bf16 represents exactly."""
    b = int(np.array([x], dtype=np.float32).view(np.uint32)[0])
    assert b & 0xFFFF == 0, x
    return b >> 16


# Random123 known-answer vectors for philox4x32 with 10 rounds (the
# distribution's kat_vectors file): counter words, key words, output words.
PHILOX_KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", PHILOX_KAT)
def test_philox_known_answers(ctr, key, want):
    assert philox4x32_10(ctr, key) == want


def test_exp2_against_math():
    ts = np.linspace(-125.0, 0.0, 40001).astype(np.float32)
    worst = max(abs(float(exp2_f32(t)) / 2.0 ** float(t) - 1.0) for t in ts)
    assert worst < 2e-7
    for n in range(0, 126):  # integers are exact
        assert float(exp2_f32(-float(n))) == 2.0 ** -n
    assert exp2_f32(np.float32(-125.5)) == 0  # rint -> -126: below the cut
    assert exp2_f32(np.float32(-125.4)) > 0
    assert exp2_f32(np.float32(-np.inf)) == 0


def test_closed_forms():
    one = [bf16(1.0)] * 4
    assert sample_row(one, 0, 0.7, 0.9, 1, 0, 0) == (-1, 0)          # no entries
    assert sample_row(one, 4, 0.0, 0.9, 1, 0, 0) == (0, 1)           # T = 0 is greedy
    # equal weights 1,1,1,1: Z = 4; c_2 = 2 >= 0.5 * 4 exactly, c_2 < 0.51 * 4
    assert sample_row(one, 4, 1.0, 0.5, 1, 0, 0)[1] == 2
    assert sample_row(one, 4, 1.0, 0.51, 1, 0, 0)[1] == 3
    assert sample_row(one, 4, 1.0, 1.0, 1, 0, 0)[1] == 4
    # a tiny nucleus keeps the top entry only, whatever the draw
    vals = [bf16(v) for v in (3.0, 2.0, 1.0, 0.0)]
    assert all(sample_row(vals, 4, 1.0, 1e-6, 9, off, 3) == (0, 1) for off in range(200))
    # +inf first: only the +inf entries can be drawn; -inf entries never are
    inf = [0x7F80, 0x7F80, bf16(1.0), 0xFF80]
    got = {sample_row(inf, 4, 0.7, 1.0, 5, off, 1) for off in range(300)}
    assert got == {(0, 2), (1, 2)}
    fin = [bf16(0.5), bf16(0.25), 0xFF80, 0xFF80]
    assert {sample_row(fin, 4, 2.0, 1.0, 5, off, 2)[0] for off in range(300)} == {0, 1}


def chi2_upper_tail(stat, dof):
    """P(chi-square_dof >= stat) by the series of the regularized gamma."""
    a, x = dof / 2.0, stat / 2.0
    term = total = 1.0 / a
    n = a
    for _ in range(10000):
        n += 1.0
        term *= x / n
        total += term
        if term < total * 1e-15:
            break
    lower = total * math.exp(-x + a * math.log(x) - math.lgamma(a))
    return max(0.0, 1.0 - lower)


@pytest.mark.parametrize("top_p,temperature", [(1.0, 1.0), (0.8, 1.0), (0.95, 0.7), (1.0, 2.5)])
def test_frequencies_follow_the_nucleus_softmax(top_p, temperature):
    logits = [2.0, 1.0, 0.5, 0.0, -1.0, -3.0]
    vals = [bf16(v) for v in logits]
    p = np.exp(np.array(logits) / temperature)
    p /= p.sum()
    cum = np.cumsum(p)
    kept = int(np.argmax(cum >= top_p - 1e-12)) + 1
    want = p[:kept] / p[:kept].sum()
    n = 40000
    counts = np.zeros(len(logits))
    for off in range(n):
        j, kk = sample_row(vals, len(vals), temperature, top_p, 1234, off, 7)
        assert kk == kept
        counts[j] += 1
    assert counts[kept:].sum() == 0
    stat = float(((counts[:kept] - n * want) ** 2 / (n * want)).sum())
    assert chi2_upper_tail(stat, kept - 1) > 1e-4 if kept > 1 else counts[0] == n


def test_rows_and_offsets_draw_independently():
    """Different rows and offsets use different counters: over many rows the
    top entry's share matches its probability."""
    vals = np.array([[bf16(0.0), bf16(0.0)]] * 20000, dtype=np.uint16)
    idx = np.array([[5, 9]] * 20000, dtype=np.int32)
    count = np.full(20000, 2, dtype=np.int32)
    tok, kept = sample_topk(idx, vals, count, 1.0, 1.0, 42, 3)
    assert np.all(kept == 2) and set(np.unique(tok)) == {5, 9}
    share = float(np.mean(tok == 5))
    assert abs(share - 0.5) < 4 * math.sqrt(0.25 / 20000)
