"""Seeded generators of bf16 logit rows (inputs only).

Every generator returns a C-contiguous ``uint16`` matrix of shape
``(rows, stride)`` holding bf16 bit patterns.  Columns ``[cols, stride)`` are
row padding; they are filled with a poison mix of +inf and NaN bit patterns so
that a top-k which reads past ``cols`` shows it in its results.

The five named configurations follow the workloads of the wide-row top-k
(TensorFold PR #713, change 3, and the exactness table of the same page):
a 15-row draft head over 98592 columns, rows of up to 248320 columns, ties,
both zeros, NaN and infinities, and padded strides.  Float draws are rounded to
bf16 with round-to-nearest-even on the float32 bit pattern.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

# bf16 bit patterns used by the generators.
BF16_POS_INF = 0x7F80
BF16_NEG_INF = 0xFF80
BF16_POS_ZERO = 0x0000
BF16_NEG_ZERO = 0x8000
NAN_PAYLOADS = (0x7FC0, 0xFFC0, 0x7F81, 0xFFFF, 0x7FA5)
POISON = (0x7F80, 0x7FC0)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round finite float32 values to bf16 bit patterns (round to nearest, ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f16_bits(m: np.ndarray) -> np.ndarray:
    """Re-encodes a matrix of bf16 bit patterns as IEEE fp16 bit patterns:
    numbers by round-to-nearest-even (numpy's float16 conversion; beyond the
    fp16 range they become infinities, below it zeros of the same sign),
    infinities as infinities, NaN as NaN of the same sign with the payload
    moved into the fp16 fraction (the quiet bit stays the quiet bit)."""
    b = np.ascontiguousarray(m, dtype=np.uint16)
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        out = f32.astype(np.float16).view(np.uint16).copy()
    nan = (b & 0x7FFF) > 0x7F80
    payload = ((b & 0x7F).astype(np.uint16) << 3)
    out[nan] = (b[nan] & 0x8000) | 0x7C00 | payload[nan]
    return out


def poison_padding(m: np.ndarray, cols: int) -> np.ndarray:
    """Fill columns [cols, stride) of every row with alternating +inf / NaN bits."""
    pad = m.shape[1] - cols
    if pad > 0:
        pat = np.resize(np.array(POISON, dtype=np.uint16), pad)
        m[:, cols:] = pat[None, :]
    return m


def _strided(rows: int, cols: int, stride: int, body: np.ndarray) -> np.ndarray:
    assert stride >= cols
    m = np.empty((rows, stride), dtype=np.uint16)
    m[:, :cols] = body
    return poison_padding(m, cols)


def sha256_of(m: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(m).tobytes()).hexdigest()


# ---------------------------------------------------------------------------
# The five workload configurations.
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class Config:
    name: str
    rows: int
    cols: int
    stride: int
    k: int
    recipe: str

    @property
    def seed(self) -> int:
        return 0x7B0000 + int(self.name[1:])

    @property
    def input_bytes(self) -> int:
        """bf16 bytes the top-k must read: every valid column once, padding never."""
        return 2 * self.rows * self.cols

    @property
    def output_bytes(self) -> int:
        """idx (4 B) + val (2 B) per entry, count (4 B) + mask (4 B) per row."""
        return self.rows * (6 * self.k + 8)

    @property
    def algorithmic_bytes(self) -> int:
        return self.input_bytes + self.output_bytes


CONFIGS = {
    "c1": Config("c1", 1, 4096, 4096, 8, "N(0,1) rounded to bf16; no non-finite values"),
    "c2": Config("c2", 15, 98592, 98592, 32, "N(0, sd=2) rounded to bf16 (draft-head shape)"),
    "c3": Config(
        "c3", 16, 248320, 248448, 20,
        "64 levels (j-32)/8 uniform; per row at disjoint seeded positions 2483 +-0, "
        "248 NaN (5 payloads), 124 +inf, 124 -inf; poison padding",
    ),
    "c4": Config(
        "c4", 64, 151936, 152064, 16,
        "Gumbel(0,1) + N(0, sd=3); 10 seeded rows all -inf but one finite value; poison padding",
    ),
    "c5": Config("c5", 1024, 151936, 151936, 64, "N(0, sd=4) + per-row offset U(-10,10), rounded to bf16"),
}


def config(name: str) -> Config:
    return CONFIGS[name]


def _c1(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    x = rng.standard_normal((cfg.rows, cfg.cols), dtype=np.float32)
    return _strided(cfg.rows, cfg.cols, cfg.stride, f32_to_bf16_bits(x))


def _c2(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    x = np.float32(2.0) * rng.standard_normal((cfg.rows, cfg.cols), dtype=np.float32)
    return _strided(cfg.rows, cfg.cols, cfg.stride, f32_to_bf16_bits(x))


def _c3(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    rows, cols = cfg.rows, cfg.cols
    levels = (np.arange(64, dtype=np.float32) - np.float32(32.0)) / np.float32(8.0)
    body = f32_to_bf16_bits(levels[rng.integers(0, 64, size=(rows, cols))])
    n_zero = cols // 100           # 1 %, floored
    n_nan = cols // 1000           # 0.1 %
    n_pinf = cols * 5 // 10000     # 0.05 %
    n_ninf = cols * 5 // 10000     # 0.05 %
    for r in range(rows):
        pos = rng.permutation(cols)[: n_zero + n_nan + n_pinf + n_ninf]
        z, rest = pos[:n_zero], pos[n_zero:]
        nan, rest = rest[:n_nan], rest[n_nan:]
        pinf, ninf = rest[:n_pinf], rest[n_pinf:]
        body[r, z] = np.where(rng.integers(0, 2, size=n_zero) == 1, BF16_NEG_ZERO, BF16_POS_ZERO)
        body[r, nan] = np.array(NAN_PAYLOADS, dtype=np.uint16)[rng.integers(0, len(NAN_PAYLOADS), size=n_nan)]
        body[r, pinf] = BF16_POS_INF
        body[r, ninf] = BF16_NEG_INF
    return _strided(rows, cols, cfg.stride, body)


def _c4(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    rows, cols = cfg.rows, cfg.cols
    x = rng.gumbel(0.0, 1.0, size=(rows, cols)).astype(np.float32)
    x += np.float32(3.0) * rng.standard_normal((rows, cols), dtype=np.float32)
    body = f32_to_bf16_bits(x)
    for r in rng.choice(rows, size=10, replace=False):
        keep = int(rng.integers(0, cols))
        finite = body[r, keep]
        body[r, :] = BF16_NEG_INF
        body[r, keep] = finite
    return _strided(rows, cols, cfg.stride, body)


def _c5(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    rows, cols = cfg.rows, cfg.cols
    offset = rng.uniform(-10.0, 10.0, size=(rows, 1)).astype(np.float32)
    body = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, 128):  # bounded float32 temporaries
        r1 = min(rows, r0 + 128)
        x = np.float32(4.0) * rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        x += offset[r0:r1]
        body[r0:r1] = f32_to_bf16_bits(x)
    return _strided(rows, cols, cfg.stride, body)


_MAKERS = {"c1": _c1, "c2": _c2, "c3": _c3, "c4": _c4, "c5": _c5}


def make_config_input(name: str) -> np.ndarray:
    """The full (rows, stride) bf16 matrix of a named configuration, from its fixed seed."""
    cfg = CONFIGS[name]
    return _MAKERS[name](cfg, np.random.default_rng(cfg.seed))


# ---------------------------------------------------------------------------
# Case families for the exactness suite (ties, both zeros, NaN and infinities,
# odd widths and strides).
# ---------------------------------------------------------------------------


def _normal(rng, rows, cols, sd=1.0):
    return f32_to_bf16_bits(np.float32(sd) * rng.standard_normal((rows, cols), dtype=np.float32))


def _fam_normal(rng, rows, cols):
    return _normal(rng, rows, cols)


def _fam_logit(rng, rows, cols):
    x = rng.gumbel(0.0, 1.0, size=(rows, cols)).astype(np.float32)
    x += np.float32(3.0) * rng.standard_normal((rows, cols), dtype=np.float32)
    return f32_to_bf16_bits(x)


def _fam_few_levels(rng, rows, cols):
    levels = np.array([-1.0, 0.5, 1.0, 2.0], dtype=np.float32)
    return f32_to_bf16_bits(levels[rng.integers(0, 4, size=(rows, cols))])


def _fam_levels64(rng, rows, cols):
    levels = (np.arange(64, dtype=np.float32) - np.float32(32.0)) / np.float32(8.0)
    return f32_to_bf16_bits(levels[rng.integers(0, 64, size=(rows, cols))])


def _fam_all_equal(rng, rows, cols):
    v = f32_to_bf16_bits(rng.standard_normal((rows, 1), dtype=np.float32))
    return np.repeat(v, cols, axis=1)


def _fam_zeros(rng, rows, cols):
    return np.where(rng.integers(0, 2, size=(rows, cols)) == 1, BF16_NEG_ZERO, BF16_POS_ZERO).astype(np.uint16)


def _fam_zeros_straddle(rng, rows, cols):
    # a few positive values, then a sea of +-0 and negative values: the k-th place
    # falls among the zeros for any k larger than the positive count
    m = _fam_zeros(rng, rows, cols)
    neg = f32_to_bf16_bits(-np.abs(rng.standard_normal((rows, cols), dtype=np.float32)) - np.float32(0.01))
    m = np.where(rng.random((rows, cols)) < 0.5, neg, m).astype(np.uint16)
    npos = max(1, min(cols, 5))
    for r in range(rows):
        p = rng.choice(cols, size=npos, replace=False)
        m[r, p] = f32_to_bf16_bits(np.abs(rng.standard_normal(npos, dtype=np.float32)) + np.float32(0.01))
    return m


def _fam_nan_sprinkled(rng, rows, cols):
    m = _normal(rng, rows, cols)
    mask = rng.random((rows, cols)) < 0.05
    pay = np.array(NAN_PAYLOADS + (0xFF81, 0x7FFF), dtype=np.uint16)
    m[mask] = pay[rng.integers(0, len(pay), size=int(mask.sum()))]
    return m


def _fam_all_nan(rng, rows, cols):
    pay = np.array(NAN_PAYLOADS + (0xFF81, 0x7FFF), dtype=np.uint16)
    return pay[rng.integers(0, len(pay), size=(rows, cols))]


def _fam_posinf_many(rng, rows, cols):
    m = _normal(rng, rows, cols)
    m[rng.random((rows, cols)) < 0.02] = BF16_POS_INF
    return m


def _fam_posinf_few(rng, rows, cols):
    m = _normal(rng, rows, cols)
    for r in range(rows):
        m[r, rng.choice(cols, size=min(cols, 3), replace=False)] = BF16_POS_INF
    return m


def _fam_neginf_all(rng, rows, cols):
    return np.full((rows, cols), BF16_NEG_INF, dtype=np.uint16)


def _fam_neginf_one_finite(rng, rows, cols):
    m = np.full((rows, cols), BF16_NEG_INF, dtype=np.uint16)
    for r in range(rows):
        m[r, int(rng.integers(0, cols))] = f32_to_bf16_bits(rng.standard_normal(1, dtype=np.float32))[0]
    return m


def _fam_ascending(rng, rows, cols):
    x = np.sort(rng.standard_normal((rows, cols), dtype=np.float32), axis=1)
    return f32_to_bf16_bits(x)


def _fam_descending(rng, rows, cols):
    return np.ascontiguousarray(_fam_ascending(rng, rows, cols)[:, ::-1])


def _fam_max_first(rng, rows, cols):
    m = _normal(rng, rows, cols)
    m[:, 0] = f32_to_bf16_bits(np.full(rows, 100.0, dtype=np.float32))
    return m


def _fam_max_last(rng, rows, cols):
    m = _normal(rng, rows, cols)
    m[:, -1] = f32_to_bf16_bits(np.full(rows, 100.0, dtype=np.float32))
    return m


def _fam_subnormals(rng, rows, cols):
    mag = rng.integers(0, 0x80, size=(rows, cols)).astype(np.uint16)  # exponent field 0
    sign = (rng.integers(0, 2, size=(rows, cols)).astype(np.uint16) << 15).astype(np.uint16)
    return (mag | sign).astype(np.uint16)


def _fam_uniform_bits(rng, rows, cols):
    # every bf16 bit pattern equally likely: all classes, every NaN payload
    return rng.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint16)


def _fam_mixed_nonfinite(rng, rows, cols):
    m = _fam_levels64(rng, rows, cols)
    u = rng.random((rows, cols))
    m[u < 0.01] = np.where(rng.integers(0, 2, size=int((u < 0.01).sum())) == 1, BF16_NEG_ZERO, BF16_POS_ZERO)
    pay = np.array(NAN_PAYLOADS, dtype=np.uint16)
    sel = (u >= 0.01) & (u < 0.011)
    m[sel] = pay[rng.integers(0, len(pay), size=int(sel.sum()))]
    m[(u >= 0.011) & (u < 0.0115)] = BF16_POS_INF
    m[(u >= 0.0115) & (u < 0.012)] = BF16_NEG_INF
    return m


FAMILIES = {
    "normal": _fam_normal,
    "logit": _fam_logit,
    "few_levels": _fam_few_levels,
    "levels64": _fam_levels64,
    "all_equal": _fam_all_equal,
    "zeros": _fam_zeros,
    "zeros_straddle": _fam_zeros_straddle,
    "nan_sprinkled": _fam_nan_sprinkled,
    "all_nan": _fam_all_nan,
    "posinf_many": _fam_posinf_many,
    "posinf_few": _fam_posinf_few,
    "neginf_all": _fam_neginf_all,
    "neginf_one_finite": _fam_neginf_one_finite,
    "ascending": _fam_ascending,
    "descending": _fam_descending,
    "max_first": _fam_max_first,
    "max_last": _fam_max_last,
    "subnormals": _fam_subnormals,
    "uniform_bits": _fam_uniform_bits,
    "mixed_nonfinite": _fam_mixed_nonfinite,
}


# Families whose values are continuous draws: their fp32 form gets random low
# fraction bits (breaking the ties the bf16 grid creates); the others keep
# their exact ties, zeros and special patterns.
F32_JITTER = ("normal", "logit", "nan_sprinkled", "posinf_few", "mixed_nonfinite", "ascending", "descending")


def bf16_to_f32_bits(m: np.ndarray, rng: np.random.Generator | None = None) -> np.ndarray:
    """fp32 bit patterns holding the bf16 patterns' values exactly (bits <<
    16); with rng, finite nonzero values get random low 16 fraction bits (the
    exponent, and so the class, is unchanged)."""
    b = np.ascontiguousarray(m, dtype=np.uint16)
    out = b.astype(np.uint32) << np.uint32(16)
    if rng is not None:
        finite = (b & 0x7FFF) < 0x7F80
        nonzero = (b & 0x7FFF) != 0
        jitter = rng.integers(0, 1 << 16, size=b.shape, dtype=np.uint32)
        out = np.where(finite & nonzero, out | jitter, out).astype(np.uint32)
    return out


def family_rows(name: str, rows: int, cols: int, stride: int | None = None, seed: int = 0,
                fmt: str = "bf16") -> np.ndarray:
    """A (rows, stride) matrix of the named family, poison in the padding.
    fmt "f16" re-encodes the family's values as fp16 bit patterns
    (bf16_to_f16_bits); the uniform_bits family keeps its raw random
    patterns, which cover every fp16 class as they cover every bf16 class.
    fmt "f32" returns a uint32 matrix of fp32 patterns (bf16_to_f32_bits,
    with low fraction bits drawn for the continuous families; uniform_bits
    draws all 32 bits)."""
    stride = cols if stride is None else stride
    rng = np.random.default_rng(seed)
    body = FAMILIES[name](rng, rows, cols) if cols > 0 else np.empty((rows, 0), dtype=np.uint16)
    body = body.astype(np.uint16)
    if fmt == "f32":
        if name == "uniform_bits":
            hi = body.astype(np.uint32) << np.uint32(16)
            body32 = hi | rng.integers(0, 1 << 16, size=body.shape, dtype=np.uint32)
        else:
            body32 = bf16_to_f32_bits(body, rng if name in F32_JITTER else None)
        m = np.empty((rows, stride), dtype=np.uint32)
        m[:, :cols] = body32
        if stride > cols:
            m[:, cols:] = bf16_to_f32_bits(_strided(rows, cols, stride, body)[:, cols:])  # +inf / NaN poison
        return m
    if fmt == "f16" and name != "uniform_bits":
        body = bf16_to_f16_bits(body)
    elif fmt not in ("bf16", "f16"):
        raise ValueError(f"unknown format {fmt}")
    m = _strided(rows, cols, stride, body)
    if fmt == "f16" and stride > cols:
        m[:, cols:] = bf16_to_f16_bits(m[:, cols:])  # poison stays poison: +inf and NaN patterns
    return m


def head_inputs(rows: int, hidden: int, vocab: int, seed: int = 0, h_pad: int = 0, w_pad: int = 0,
                kind: str = "normal"):
    """Draft-head inputs as bf16 bit patterns: hidden states h [rows][hidden
    + h_pad] ~ N(0, 1) and a vocabulary-major weight w [vocab][hidden + w_pad]
    ~ N(0, 1 / sqrt(hidden)), so that logits are of unit scale; padding is
    NaN poison.  kinds: "normal"; "ties" (w rows repeated in blocks of 4, so
    equal logits occur); "integers" (small integers in h and w: exact sums);
    "nonfinite" (a few +-inf and NaN in h)."""
    rng = np.random.default_rng(0x4EAD0000 + seed)
    h = rng.standard_normal((rows, hidden)).astype(np.float32)
    w = (rng.standard_normal((vocab, hidden)) / np.sqrt(hidden)).astype(np.float32)
    if kind == "ties":
        w = np.repeat(w[: (vocab + 3) // 4], 4, axis=0)[:vocab]
    elif kind == "integers":
        h = rng.integers(-4, 5, size=(rows, hidden)).astype(np.float32)
        w = rng.integers(-4, 5, size=(vocab, hidden)).astype(np.float32)
    elif kind == "nonfinite" and rows > 0:
        for r in range(0, rows, 3):
            h[r, rng.integers(0, hidden)] = [np.inf, -np.inf, np.nan][r % 3]
    hb = np.full((rows, hidden + h_pad), 0x7FC0, dtype=np.uint16)
    wb = np.full((vocab, hidden + w_pad), 0x7FC0, dtype=np.uint16)
    hb[:, :hidden] = f32_to_bf16_bits(h)
    wb[:, :hidden] = f32_to_bf16_bits(w)
    return hb, wb

