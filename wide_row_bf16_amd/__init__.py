"""Exact row-wise bf16 top-k on AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/tk_topk.h``: it checks
tensor metadata, allocates the four outputs with PyTorch and passes raw
device pointers and the current HIP stream to ``libtk_topk.so``.  Every step
of the top-k runs in that library's HIP kernels; there is no other path.

    idx, val, count, nonfinite = topk_bf16(logits, k)

``logits`` is a 2-D bf16 CUDA (HIP) tensor whose last dimension is
contiguous (any row stride >= its width).  Results: ``idx`` int32 [rows, k]
(column of each entry, -1 past ``count``), ``val`` bf16 [rows, k] (the
entry's own bits; 0x7FC0 past ``count``), ``count`` int32 [rows], and
``nonfinite`` int32 [rows] holding the mask bits NAN=1, POSINF=2, NEGINF=4.
"""

from __future__ import annotations

import ctypes
import os
from typing import NamedTuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libtk_topk.so")

TK_OK = 0
STATUS_NAMES = {
    0: "TK_OK", 1: "TK_ERR_NULL", 2: "TK_ERR_SHAPE", 3: "TK_ERR_K", 4: "TK_ERR_ALIGN",
    5: "TK_ERR_ALIAS", 6: "TK_ERR_DEVICE", 7: "TK_ERR_OPTION", 8: "TK_ERR_SCRATCH",
}
NONFINITE_NAN, NONFINITE_POSINF, NONFINITE_NEGINF = 1, 2, 4
FILL_IDX, FILL_VAL = -1, 0x7FC0

# Every symbol the public header declares.
EXPORTS = (
    "tk_topk_bf16", "tk_topk_bf16_ex", "tk_topk_f16", "tk_topk_f16_ex", "tk_topk_f32", "tk_topk_f32_ex",
    "tk_validate_f32", "tk_validate_bf16", "tk_topk_bf16_shard", "tk_merge_topk_bf16",
    "tk_validate_merge_bf16", "tk_sample_topk_bf16", "tk_validate_sample_bf16", "tk_head_topk_bf16",
    "tk_validate_head_bf16", "tk_plan_spans", "tk_max_k", "tk_max_span_cols", "tk_status_string", "tk_build_info",
    "tk_probe_read", "tk_topk_bf16_noalloc", "tk_release_stream",
)


class TkError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({_status_string(status)})")


class TkOptions(ctypes.Structure):
    _fields_ = [("spans", ctypes.c_int32), ("exact", ctypes.c_int32), ("general", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 5)]


class TopK(NamedTuple):
    idx: "object"
    val: "object"
    count: "object"
    nonfinite: "object"


_lib: ctypes.CDLL | None = None


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libtk_topk.so, compiling it with hipcc first only if it is not built."""
    global _lib
    if _lib is not None and path == LIBRARY:
        return _lib
    if not os.path.exists(path):
        if path != LIBRARY:
            raise FileNotFoundError(path)
        from . import build as _build

        _build.build()
    # PyTorch's ROCm wheel carries its own HIP runtime.  Opened first, this
    # library would bind to the system runtime and torch would then map its
    # own beside it: two runtimes in one process, where the device pointers
    # and streams torch hands over are unknown to the runtime that launches
    # these kernels (every call fails with TK_ERR_DEVICE).  Importing torch
    # first makes the library bind to the runtime torch already loaded.
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.tk_topk_bf16.restype = i32
    lib.tk_topk_bf16.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp]
    lib.tk_topk_bf16_noalloc.restype = i32
    lib.tk_topk_bf16_noalloc.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp]
    lib.tk_topk_bf16_ex.restype = i32
    lib.tk_topk_bf16_ex.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, ctypes.POINTER(TkOptions)]
    lib.tk_topk_f16.restype = i32
    lib.tk_topk_f16.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp]
    lib.tk_topk_f16_ex.restype = i32
    lib.tk_topk_f16_ex.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, ctypes.POINTER(TkOptions)]
    lib.tk_topk_f32.restype = i32
    lib.tk_topk_f32.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp]
    lib.tk_topk_f32_ex.restype = i32
    lib.tk_topk_f32_ex.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, ctypes.POINTER(TkOptions)]
    lib.tk_validate_f32.restype = i32
    lib.tk_validate_f32.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp]
    lib.tk_validate_bf16.restype = i32
    lib.tk_validate_bf16.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp]
    lib.tk_topk_bf16_shard.restype = i32
    lib.tk_topk_bf16_shard.argtypes = [i64, i64, i64, i32, i64, vp, vp, vp, vp, vp, vp]
    lib.tk_merge_topk_bf16.restype = i32
    lib.tk_merge_topk_bf16.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.tk_validate_merge_bf16.restype = i32
    lib.tk_validate_merge_bf16.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    f32, u64 = ctypes.c_float, ctypes.c_uint64
    lib.tk_sample_topk_bf16.restype = i32
    lib.tk_sample_topk_bf16.argtypes = [i64, i32, vp, vp, vp, f32, f32, u64, u64, vp, vp, vp]
    lib.tk_validate_sample_bf16.restype = i32
    lib.tk_validate_sample_bf16.argtypes = [i64, i32, vp, vp, vp, f32, f32, vp, vp]
    lib.tk_head_topk_bf16.restype = i32
    lib.tk_head_topk_bf16.argtypes = [i64, i64, i64, i32, vp, i64, vp, i64, vp, vp, vp, vp, vp, i64, vp]
    lib.tk_validate_head_bf16.restype = i32
    lib.tk_validate_head_bf16.argtypes = [i64, i64, i64, i32, vp, i64, vp, i64, vp, vp, vp, vp, vp, i64]
    lib.tk_plan_spans.restype = i32
    lib.tk_plan_spans.argtypes = [i64, i64, i32, i32]
    lib.tk_max_k.restype = i32
    lib.tk_max_k.argtypes = []
    lib.tk_max_span_cols.restype = i64
    lib.tk_max_span_cols.argtypes = []
    lib.tk_status_string.restype = ctypes.c_char_p
    lib.tk_status_string.argtypes = [i32]
    lib.tk_build_info.restype = ctypes.c_char_p
    lib.tk_build_info.argtypes = []
    lib.tk_release_stream.restype = i32
    lib.tk_release_stream.argtypes = [vp]
    lib.tk_probe_read.restype = i32
    lib.tk_probe_read.argtypes = [vp, i64, i32, vp, vp]
    if path == LIBRARY:
        _lib = lib
    return lib


def _status_string(status: int) -> str:
    try:
        return load().tk_status_string(status).decode()
    except OSError:
        return "?"


def max_k() -> int:
    return int(load().tk_max_k())


def max_span_cols() -> int:
    return int(load().tk_max_span_cols())


def plan_spans(rows: int, cols: int, k: int, compute_units: int = 256) -> int:
    return int(load().tk_plan_spans(rows, cols, k, compute_units))


def validate(rows, cols, row_stride, k, in_ptr, idx_ptr, val_ptr, count_ptr, mask_ptr) -> int:
    """The host-side guards on raw pointers (no HIP call); returns a status code."""
    return int(load().tk_validate_bf16(rows, cols, row_stride, k, in_ptr, idx_ptr, val_ptr, count_ptr, mask_ptr))


def topk_bf16_raw(rows, cols, row_stride, k, in_ptr, idx_ptr, val_ptr, count_ptr, mask_ptr, stream=0, spans=0,
                  exact=0, fmt="bf16", general=0) -> int:
    """Calls the C ABI on raw device pointers (fmt "bf16" or "f16"); returns
    the status code."""
    lib = load()
    name = {"bf16": "tk_topk_bf16", "f16": "tk_topk_f16", "f32": "tk_topk_f32"}[fmt]
    if spans or exact or general:
        opt = TkOptions(spans=spans, exact=exact, general=general)
        return int(getattr(lib, name + "_ex")(rows, cols, row_stride, k, in_ptr, idx_ptr, val_ptr, count_ptr, mask_ptr,
                                              stream, ctypes.byref(opt)))
    return int(getattr(lib, name)(rows, cols, row_stride, k, in_ptr, idx_ptr, val_ptr, count_ptr, mask_ptr, stream))


def _current_stream_handle(torch, dev: int) -> int:
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return int(raw(dev))
    return int(torch.cuda.current_stream(dev).cuda_stream)


def _dtypes(torch, fmt: str):
    """Accepted dtypes of an entry-value tensor for an input format."""
    if fmt == "f32":
        return (torch.float32, torch.int32, torch.uint32)
    if fmt == "f16":
        return (torch.float16, torch.int16, torch.uint16)
    return (torch.bfloat16, torch.int16, torch.uint16)


def _check_tensor(t, name: str, dtypes, shape, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: expected dtype in {[str(d) for d in dtypes]}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")


def _check_out(torch, out, rows: int, k: int, fmt: str, device):
    """Caller-supplied outputs must be exactly what the kernels write: int32
    [rows, k] indices, [rows, k] values of the format's width, int32 [rows]
    counts and masks, contiguous, on the input's device.  Anything else would
    let the kernels write past the tensors, so it is rejected before any call."""
    if not isinstance(out, tuple) or len(out) != 4:
        raise ValueError("out: expected a TopK (idx, val, count, nonfinite)")
    i32 = (torch.int32,)
    _check_tensor(out[0], "out.idx", i32, (rows, k), device)
    _check_tensor(out[1], "out.val", _dtypes(torch, fmt), (rows, k), device)
    _check_tensor(out[2], "out.count", i32, (rows,), device)
    _check_tensor(out[3], "out.nonfinite", (torch.int32, torch.uint32), (rows,), device)


def topk_bf16(x, k: int, *, cols: int | None = None, spans: int = 0, exact: bool = False, general: bool = False,
              out: TopK | None = None, stream=None, _fmt: str = "bf16") -> TopK:
    """Row-wise exact top-k of a 2-D bf16 tensor (see the module docstring).

    ``cols`` limits the scan to the first ``cols`` columns (default: all);
    ``spans`` forces the row split (0 = automatic, 1 = one workgroup per row);
    ``exact`` turns off the speculative floor (the result is the same);
    ``general`` makes k = 1 run the general scan instead of the argmax scan
    (the same result; the control of that fast path);
    ``out`` reuses preallocated outputs; ``stream`` is a torch.cuda.Stream
    (default: the current stream).
    """
    import torch

    if x.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    wanted = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[_fmt]
    raw = (torch.int32, torch.uint32) if _fmt == "f32" else (torch.int16, torch.uint16)
    if x.dtype not in (wanted,) + raw:
        raise TypeError(f"expected {_fmt} bit patterns, got {x.dtype}")
    if x.device.type != "cuda":
        raise ValueError("expected a tensor on a HIP device")
    rows, width = x.shape
    if rows > 0 and width > 0 and x.stride(1) != 1:
        raise ValueError("the last dimension must be contiguous")
    cols = width if cols is None else cols
    if cols > width:
        raise ValueError("cols exceeds the tensor width")
    row_stride = x.stride(0) if rows > 1 else max(cols, 1)
    if out is None:
        out = TopK(
            torch.empty((rows, k), dtype=torch.int32, device=x.device),
            torch.empty((rows, k), dtype=wanted, device=x.device),
            torch.empty((rows,), dtype=torch.int32, device=x.device),
            torch.empty((rows,), dtype=torch.int32, device=x.device),
        )
    else:
        _check_out(torch, out, rows, k, _fmt, x.device)
    dev = x.device.index if x.device.index is not None else torch.cuda.current_device()
    handle = stream.cuda_stream if stream is not None else _current_stream_handle(torch, dev)
    args = (rows, cols, row_stride, k, x.data_ptr(), out.idx.data_ptr(), out.val.data_ptr(), out.count.data_ptr(),
            out.nonfinite.data_ptr(), handle, spans, int(exact), _fmt, int(general))
    if dev == torch.cuda.current_device():
        status = topk_bf16_raw(*args)
    else:
        with torch.cuda.device(dev):
            status = topk_bf16_raw(*args)
    if status != TK_OK:
        raise TkError(status, "tk_topk_" + _fmt)
    return out


def topk_f32(x, k: int, **kw) -> TopK:
    """topk_bf16 for IEEE fp32 rows (tk_topk_f32); ``val`` holds fp32 values."""
    return topk_bf16(x, k, _fmt="f32", **kw)


def validate_f32(rows, cols, row_stride, k, in_ptr, idx_ptr, val_ptr, count_ptr, mask_ptr) -> int:
    """The host-side guards of tk_topk_f32 on raw pointers (no HIP call)."""
    return int(load().tk_validate_f32(rows, cols, row_stride, k, in_ptr, idx_ptr, val_ptr, count_ptr, mask_ptr))


def topk_f16(x, k: int, **kw) -> TopK:
    """topk_bf16 for IEEE fp16 rows (tk_topk_f16); ``val`` holds fp16 bits."""
    return topk_bf16(x, k, _fmt="f16", **kw)


def _outputs(torch, rows, k, device):
    return TopK(
        torch.empty((rows, k), dtype=torch.int32, device=device),
        torch.empty((rows, k), dtype=torch.bfloat16, device=device),
        torch.empty((rows,), dtype=torch.int32, device=device),
        torch.empty((rows,), dtype=torch.int32, device=device),
    )


def topk_bf16_shard(x, k: int, col_base: int, *, out: TopK | None = None) -> TopK:
    """Top-k of a column shard whose column 0 is global column ``col_base``:
    like topk_bf16, with global indices in ``idx`` (tk_topk_bf16_shard)."""
    import torch

    if x.dim() != 2 or x.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or x.device.type != "cuda":
        raise ValueError("expected a 2-D bf16 tensor on a HIP device")
    rows, cols = x.shape
    if rows > 0 and cols > 0 and x.stride(1) != 1:
        raise ValueError("the last dimension must be contiguous")
    if out is None:
        out = _outputs(torch, rows, k, x.device)
    else:
        _check_out(torch, out, rows, k, "bf16", x.device)
    status = int(load().tk_topk_bf16_shard(
        rows, cols, x.stride(0) if rows > 1 else max(cols, 1), k, col_base, x.data_ptr(), out.idx.data_ptr(),
        out.val.data_ptr(), out.count.data_ptr(), out.nonfinite.data_ptr(),
        _current_stream_handle(torch, x.device.index if x.device.index is not None else torch.cuda.current_device())))
    if status != TK_OK:
        raise TkError(status, "tk_topk_bf16_shard")
    return out


def merge_topk_bf16(idx, val, count, nonfinite, *, out: TopK | None = None) -> TopK:
    """Merges stacked shard results: idx/val [shards, rows, k], count/nonfinite
    [shards, rows], all contiguous (tk_merge_topk_bf16)."""
    import torch

    if idx.dim() != 3:
        raise ValueError("idx: expected [shards, rows, k]")
    shards, rows, k = idx.shape
    if idx.device.type != "cuda":
        raise ValueError("expected tensors on a HIP device")
    _check_tensor(idx, "idx", (torch.int32,), (shards, rows, k), idx.device)
    _check_tensor(val, "val", _dtypes(torch, "bf16"), (shards, rows, k), idx.device)
    _check_tensor(count, "count", (torch.int32,), (shards, rows), idx.device)
    _check_tensor(nonfinite, "nonfinite", (torch.int32, torch.uint32), (shards, rows), idx.device)
    if out is None:
        out = _outputs(torch, rows, k, idx.device)
    else:
        _check_out(torch, out, rows, k, "bf16", idx.device)
    status = int(load().tk_merge_topk_bf16(
        rows, shards, k, idx.data_ptr(), val.data_ptr(), count.data_ptr(), nonfinite.data_ptr(), out.idx.data_ptr(),
        out.val.data_ptr(), out.count.data_ptr(), out.nonfinite.data_ptr(),
        _current_stream_handle(torch, idx.device.index if idx.device.index is not None else torch.cuda.current_device())))
    if status != TK_OK:
        raise TkError(status, "tk_merge_topk_bf16")
    return out


def validate_merge(rows, shards, k, idx_ptr, val_ptr, count_ptr, mask_ptr, oidx, oval, ocount, omask) -> int:
    """The host-side guards of tk_merge_topk_bf16 on raw pointers (no HIP call)."""
    return int(load().tk_validate_merge_bf16(rows, shards, k, idx_ptr, val_ptr, count_ptr, mask_ptr, oidx, oval, ocount,
                                             omask))


def sample_topk_bf16(topk: TopK, temperature: float, top_p: float, seed: int, offset: int = 0, *, out=None):
    """Seeded top-p sampling over a top-k result (tk_sample_topk_bf16):
    returns (token, kept), int32 [rows] each."""
    import torch

    if topk.idx.dim() != 2 or topk.idx.device.type != "cuda":
        raise ValueError("expected a TopK of [rows, k] tensors on a HIP device")
    rows, k = topk.idx.shape
    _check_out(torch, topk, rows, k, "bf16", topk.idx.device)
    if out is None:
        out = (torch.empty((rows,), dtype=torch.int32, device=topk.idx.device),
               torch.empty((rows,), dtype=torch.int32, device=topk.idx.device))
    else:
        if len(out) != 2:
            raise ValueError("out: expected (token, kept)")
        _check_tensor(out[0], "out token", (torch.int32,), (rows,), topk.idx.device)
        _check_tensor(out[1], "out kept", (torch.int32,), (rows,), topk.idx.device)
    dev = topk.idx.device.index if topk.idx.device.index is not None else torch.cuda.current_device()
    status = int(load().tk_sample_topk_bf16(
        rows, k, topk.idx.data_ptr(), topk.val.data_ptr(), topk.count.data_ptr(), float(temperature), float(top_p),
        int(seed) & (2**64 - 1), int(offset) & (2**64 - 1), out[0].data_ptr(), out[1].data_ptr(),
        _current_stream_handle(torch, dev)))
    if status != TK_OK:
        raise TkError(status, "tk_sample_topk_bf16")
    return out


def head_topk_bf16(h, w, k: int, *, logits: bool = False, out: TopK | None = None):
    """Draft-head logits h . w^T fused with the row top-k (tk_head_topk_bf16).

    ``h``: bf16 [rows][hidden] (rows <= 64), ``w``: bf16 [vocab][hidden], both
    with contiguous last dimensions and row strides that are multiples of 8
    elements, 16-byte aligned.  Returns the TopK of the bf16 logits; with
    ``logits=True`` returns (TopK, logits [rows][vocab] bf16) -- the logits are
    otherwise never materialised.
    """
    import torch

    if h.dim() != 2 or w.dim() != 2 or h.shape[1] != w.shape[1]:
        raise ValueError("expected h [rows][hidden] and w [vocab][hidden]")
    for t in (h, w):
        if t.dtype not in (torch.bfloat16, torch.int16) or t.device.type != "cuda":
            raise TypeError("expected bf16 tensors on a HIP device")
        if t.shape[0] > 0 and t.stride(1) != 1:
            raise ValueError("the last dimension must be contiguous")
    rows, hidden = h.shape
    vocab = w.shape[0]
    if w.device != h.device:
        raise ValueError("h and w must be on the same device")
    if out is None:
        out = TopK(torch.empty((rows, k), dtype=torch.int32, device=h.device),
                   torch.empty((rows, k), dtype=torch.bfloat16, device=h.device),
                   torch.empty((rows,), dtype=torch.int32, device=h.device),
                   torch.empty((rows,), dtype=torch.int32, device=h.device))
    else:
        _check_out(torch, out, rows, k, "bf16", h.device)
    lg = torch.empty((rows, vocab), dtype=torch.bfloat16, device=h.device) if logits else None
    dev = h.device.index if h.device.index is not None else torch.cuda.current_device()
    status = int(load().tk_head_topk_bf16(
        rows, hidden, vocab, k, h.data_ptr(), h.stride(0) if rows > 1 else hidden, w.data_ptr(),
        w.stride(0) if vocab > 1 else hidden, out.idx.data_ptr(), out.val.data_ptr(), out.count.data_ptr(),
        out.nonfinite.data_ptr(), lg.data_ptr() if lg is not None else None, vocab if lg is not None else 0,
        _current_stream_handle(torch, dev)))
    if status != TK_OK:
        raise TkError(status, "tk_head_topk_bf16")
    return (out, lg) if logits else out


def validate_head(rows, hidden, vocab, k, h_ptr, h_stride, w_ptr, w_stride, idx_ptr, val_ptr, count_ptr, mask_ptr,
                  logits_ptr=None, logits_stride=0) -> int:
    """The host-side guards of tk_head_topk_bf16 on raw pointers (no HIP call)."""
    return int(load().tk_validate_head_bf16(rows, hidden, vocab, k, h_ptr, h_stride, w_ptr, w_stride, idx_ptr,
                                            val_ptr, count_ptr, mask_ptr, logits_ptr, logits_stride))


def validate_sample(rows, k, idx_ptr, val_ptr, count_ptr, temperature, top_p, token_ptr, kept_ptr) -> int:
    """The host-side guards of tk_sample_topk_bf16 on raw pointers (no HIP call)."""
    return int(load().tk_validate_sample_bf16(rows, k, idx_ptr, val_ptr, count_ptr, temperature, top_p, token_ptr,
                                              kept_ptr))


def read_probe(x, workgroups: int, sink) -> None:
    """Measurement probe (tk_probe_read): streams the bytes of the contiguous
    device tensor ``x`` with the scan's loads over ``workgroups`` workgroups
    and computes nothing; ``x=None`` launches an empty kernel.  ``sink`` is a
    device int32 tensor of 8192 elements."""
    import torch

    if sink.numel() < 8192 or sink.element_size() != 4 or not sink.is_contiguous():
        raise ValueError("sink: expected 8192 contiguous 4-byte elements")
    if x is not None and not x.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    nbytes = 0 if x is None else x.numel() * x.element_size()
    dev = sink.device.index if sink.device.index is not None else torch.cuda.current_device()
    status = int(load().tk_probe_read(None if x is None else x.data_ptr(), nbytes, workgroups, sink.data_ptr(),
                                      _current_stream_handle(torch, dev)))
    if status != TK_OK:
        raise TkError(status, "tk_probe_read")


def release_stream(stream=None) -> None:
    """Frees the scratch the library caches for ``stream`` (a torch.cuda.Stream;
    default: the current stream) after the work queued on it, before the
    stream is destroyed (tk_release_stream)."""
    import torch

    dev = torch.cuda.current_device()
    handle = stream.cuda_stream if stream is not None else _current_stream_handle(torch, dev)
    status = int(load().tk_release_stream(handle))
    if status != TK_OK:
        raise TkError(status, "tk_release_stream")
