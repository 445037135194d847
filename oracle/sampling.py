"""CPU oracle for seeded top-p sampling over a row's top-k entries.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code,
header, table or constant with the HIP library it checks.

What the pages fix: a drafted decode may sample instead of taking the
argmax, with a temperature, a top-k, a top-p and a seed (the receipt of
TensorFold PR #3069, "qwen27 metal: restore the long-copy driver for a lone
greedy stream on M5", runs T 0.7 with top-k 20, top-p 0.95, seed 1234), and
seeded sampled decodes are reproducible token for token (the seeded sampled
exactness cases in the review of TensorFold PR #713).  The pages give no
algorithm; the steps below are this library's plain reading, each one a
standard definition, all in float32 so that both implementations take every
decision with the same numbers:

  inputs per row: the top-k result (entries sorted by score, count), the
  temperature T >= 0, top_p in (0, 1], a 64-bit seed and a 64-bit offset
  (the decode step).
  1. count == 0: token -1, kept 0.  T == 0: greedy, token = entry 0, kept 1.
  2. x_j = the bf16 value of entry j, exactly, as float32.
     Weights: if x_0 is +inf, w_j = 1 for x_j == +inf, else 0.  Otherwise
     w_j = exp((x_j - x_0) / T), computed as
         s  = float32(log2(e) / T)          (once per call, in float64, with T
                                             the float32 temperature as given)
         t  = float32(float32(x_j - x_0) * s)
         w  = exp2(t) by the routine exp2_f32 below; w = 0 when x_j is -inf.
  3. Cumulative sums in entry order, float32, one addition at a time:
     c_0 = 0, c_{n+1} = c_n + w_n.  Z = c_count.
  4. Nucleus: kept = the smallest n >= 1 with c_n >= float32(top_p * Z)
     (float32 product); top_p == 1 keeps every entry with c_n >= Z.
  5. Uniform: r = word 0 of Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
     "Parallel random numbers: as easy as 1, 2, 3", SC 2011) with key
     (seed low 32 bits, seed high 32 bits) and counter (row, 0, offset low,
     offset high); u = (r >> 8) * 2^-24, exact in float32, in [0, 1).
  6. Threshold h = float32(u * c_kept); token = entry j of the smallest j
     with c_{j+1} > h, or entry kept - 1 if there is none (h rounded up to
     c_kept).

exp2_f32(t), t <= 0: n = rint(t) (round half to even), f = t - n (exact),
p = the degree-7 Taylor polynomial of 2^f = e^(f ln 2) evaluated by Horner's
rule in float32 with coefficients (ln 2)^i / i! rounded to float32, result =
p * 2^n (exact scaling, the result stays a normal number); 0 when n < -125
or t is -inf.  Truncation error below 1e-8 for |f| <= 1/2.
"""

from __future__ import annotations

import math

import numpy as np

F = np.float32

# Philox4x32 round multipliers and Weyl key increments, as published.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds: counter = 4 words, key = 2 words (ints)."""
    c0, c1, c2, c3 = (int(v) & MASK32 for v in counter)
    k0, k1 = (int(v) & MASK32 for v in key)
    for rnd in range(10):
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> 32, p0 & MASK32
        hi1, lo1 = p1 >> 32, p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        if rnd < 9:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
    return c0, c1, c2, c3


# (ln 2)^i / i!, i = 0..7, rounded to float32 from float64.
EXP2_COEF = [F(math.log(2.0) ** i / math.factorial(i)) for i in range(8)]


def exp2_f32(t):
    """2^t for float32 t <= 0 by the routine in the module docstring."""
    t = F(t)
    n = F(np.rint(t))
    if not n >= F(-125.0):  # also t == -inf
        return F(0.0)
    f = F(t - n)
    p = EXP2_COEF[7]
    for c in reversed(EXP2_COEF[:7]):
        p = F(F(p * f) + c)
    return F(p * F(2.0) ** int(n))


def bf16_to_f32(bits):
    return np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0]


def log2e_over(temperature):
    return F(np.float64(math.log2(math.e)) / np.float64(F(temperature)))


def sample_row(vals, count, temperature, top_p, seed, offset, row):
    """(entry position, kept) for one row; vals = bf16 bit patterns of the
    row's entries in order.  The caller maps the position to a column."""
    if count <= 0:
        return -1, 0
    if F(temperature) == 0:
        return 0, 1
    x = [bf16_to_f32(vals[j]) for j in range(count)]
    if math.isinf(x[0]) and x[0] > 0:
        w = [F(1.0) if (math.isinf(v) and v > 0) else F(0.0) for v in x]
    else:
        s = log2e_over(temperature)
        w = []
        for v in x:
            if math.isinf(v):  # only -inf can follow a finite x_0
                w.append(F(0.0))
            else:
                w.append(exp2_f32(F(F(v - x[0]) * s)))
    c = [F(0.0)]
    for wj in w:
        c.append(F(c[-1] + wj))
    z = c[count]
    bound = F(F(top_p) * z)
    kept = next(n for n in range(1, count + 1) if c[n] >= bound)
    r = philox4x32_10((row, 0, offset & MASK32, offset >> 32), (seed & MASK32, seed >> 32))[0]
    u = F((r >> 8) * 2.0 ** -24)
    h = F(u * c[kept])
    for j in range(kept):
        if c[j + 1] > h:
            return j, kept
    return kept - 1, kept


def sample_topk(idx, val, count, temperature, top_p, seed, offset):
    """Rows of a top-k result (idx int32 [rows][k], val uint16 bf16 bits
    [rows][k], count int32 [rows]) -> (token int32 [rows], kept int32 [rows])."""
    idx = np.asarray(idx)
    val = np.asarray(val)
    count = np.asarray(count)
    rows = count.shape[0]
    token = np.full(rows, -1, dtype=np.int32)
    kept = np.zeros(rows, dtype=np.int32)
    for r in range(rows):
        j, n = sample_row(val[r], int(count[r]), temperature, top_p, seed, offset, r)
        kept[r] = n
        token[r] = idx[r, j] if j >= 0 else -1
    return token, kept
