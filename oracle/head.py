"""CPU oracle for the draft head fused with the row top-k.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code,
header, table or constant with the HIP library it checks.

What the pages fix: the drafter of TensorFold PR #713 computes its draft
head and takes the top k of each head row (15 rows of 98592 columns, change
3).  They give no kernel and no precision for the head; the reading checked
here (stated with tk_head_topk_bf16):

  logit[r][n] = bf16_rne(F[r][n]),  F = a float32 accumulation of the
  products h[r][i] * w[n][i] in an order the hardware chooses,

and the top-k is the library's operation on those bf16 logits.  Because the
accumulation order is not fixed, the oracle checks the two halves
separately:

  1. logits: every logit lies within the rounding bound of the exact sum
     S = sum_i h[r][i] w[n][i] (computed here in float64: every bf16 x bf16
     product is exact in float64 and so is their sum for the sizes used),
         |logit - S| <= 2^-8 |S| + (1 + 2^-8) * delta + 2^-125,
         delta = 2 * hidden * 2^-24 * sum_i |h[r][i] w[n][i]|
     (float32 summation error bound, doubled for any order or internal
     precision; bf16 round-to-nearest is within half an ulp, 2^-8 relative;
     2^-125 covers results flushed near zero).  Non-finite sums must match
     in class (NaN, +inf, -inf).
  2. top-k: the library's outputs equal oracle.topk_bf16 over the logits the
     kernel produced, byte for byte.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def head_logits_exact(h_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """S = h . w^T in float64 from bf16 bit patterns: h [rows][hidden],
    w [vocab][hidden] -> [rows][vocab]."""
    h = bf16_to_f64(h_bits)
    w = bf16_to_f64(w_bits)
    with np.errstate(invalid="ignore", over="ignore"):
        return h @ w.T


def head_logit_bound(h_bits: np.ndarray, w_bits: np.ndarray, exact: np.ndarray | None = None) -> np.ndarray:
    """The largest allowed |logit - S| for each logit (finite S)."""
    h = np.abs(bf16_to_f64(h_bits))
    w = np.abs(bf16_to_f64(w_bits))
    if exact is None:
        exact = head_logits_exact(h_bits, w_bits)
    hidden = h.shape[1]
    with np.errstate(invalid="ignore", over="ignore"):
        delta = 2.0 * hidden * 2.0 ** -24 * (h @ w.T)
        return 2.0 ** -8 * np.abs(exact) + (1.0 + 2.0 ** -8) * delta + 2.0 ** -125


def check_head_logits(logit_bits: np.ndarray, h_bits: np.ndarray, w_bits: np.ndarray):
    """(ok, message) for the kernel's bf16 logits against the bound."""
    exact = head_logits_exact(h_bits, w_bits)
    got = bf16_to_f64(logit_bits)
    fin = np.isfinite(exact)
    bad_class = (~fin) & ~((np.isnan(exact) & np.isnan(got)) | (exact == got))
    if bad_class.any():
        r, n = np.argwhere(bad_class)[0]
        return False, f"class differs at ({r}, {n}): got {got[r, n]} want {exact[r, n]}"
    bound = head_logit_bound(h_bits, w_bits, exact)
    with np.errstate(invalid="ignore"):
        err = np.where(fin, np.abs(got - exact), 0.0)
    over = fin & ~(err <= bound)
    if over.any():
        r, n = np.argwhere(over)[0]
        return False, f"logit ({r}, {n}) = {got[r, n]!r}, exact {exact[r, n]!r}, bound {bound[r, n]!r}"
    return True, ""
