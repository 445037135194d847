"""Helpers for the GPU tests: upload seeded inputs, call the C ABI through the
binding, and compare with the CPU oracle byte for byte."""

from __future__ import annotations

import sys

import numpy as np

import oracle

POISON_WORD = 0x7FC0


def need_gpu():
    import pytest
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def upload(m: np.ndarray, offset: int = 0):
    """Copies a (rows, stride) uint16 matrix (or uint32, for fp32 rows) to the
    device.  With offset > 0 the rows start `offset` elements past a fresh
    allocation (misaligned rows); the elements before them hold NaN poison."""
    import torch

    rows, stride = m.shape
    wide = m.dtype == np.uint32
    sdt, tdt = (np.int32, torch.int32) if wide else (np.int16, torch.int16)
    poison = np.uint32(POISON_WORD << 16).view(np.int32) if wide else np.uint16(POISON_WORD).view(np.int16)
    base = torch.empty(offset + rows * stride, dtype=tdt, device="cuda")
    if offset:
        base[:offset] = int(poison)
    if rows * stride:
        base[offset:] = torch.from_numpy(np.ascontiguousarray(m).view(sdt).reshape(-1)).to("cuda")
    return base[offset:].view(rows, stride)


def to_numpy(out):
    import torch

    torch.cuda.synchronize()
    wide = out.val.element_size() == 4
    return (
        out.idx.cpu().numpy(),
        out.val.view(torch.int32).cpu().numpy().view(np.uint32) if wide else
        out.val.view(torch.int16).cpu().numpy().view(np.uint16),
        out.count.cpu().numpy(),
        out.nonfinite.cpu().numpy().view(np.uint32),
    )


def gpu_topk(m: np.ndarray, cols: int, k: int, spans: int = 0, offset: int = 0, x=None, fmt: str = "bf16",
             exact: bool = False):
    import wide_row_bf16_amd as tk

    x = upload(m, offset) if x is None else x
    fn = {"bf16": tk.topk_bf16, "f16": tk.topk_f16, "f32": tk.topk_f32}[fmt]
    return to_numpy(fn(x, k, cols=cols, spans=spans, exact=exact))


def assert_same(got, want, what: str):
    names = ("idx", "val", "count", "nonfinite")
    for g, w, n in zip(got, want, names):
        if not np.array_equal(g, w):
            bad = np.argwhere(g != w)
            first = tuple(bad[0])
            raise AssertionError(
                f"{what}: {n} differs at {len(bad)} places, first {first}: got {g[first]} want {w[first]}"
            )


def check_case(m, cols, k, spans=0, offset=0, what="", want=None, fmt="bf16"):
    if want is None:
        want = {"bf16": oracle.topk_bf16, "f16": oracle.topk_f16, "f32": oracle.topk_f32}[fmt](m, cols, k)
    got = gpu_topk(m, cols, k, spans=spans, offset=offset, fmt=fmt)
    assert_same(got, want, what or f"cols={cols} k={k} spans={spans} offset={offset}")
    return got
