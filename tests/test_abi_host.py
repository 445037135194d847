"""The C-ABI library on the host: it loads, exports what the header declares,
and its guards reject bad arguments before any HIP call (CPU only)."""

import os
import re

import pytest

import wide_row_bf16_amd as tk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tk_topk.h")

OK, NULL, SHAPE, K, ALIGN, ALIAS, DEVICE, OPTION = range(8)

# Fake, well-separated, aligned device addresses: the guards only do arithmetic on them.
IN, IDX, VAL, CNT, MSK = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tk_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(tk.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = tk.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_stamp_build_is_separate():
    # the stage-timestamp build is a second library; the product library has
    # no stamp table and no read-out
    import ctypes
    import os

    from wide_row_bf16_amd.build import STAMP_LIBRARY

    assert not hasattr(tk.load(), "tk_stage_stamps")
    if not os.path.exists(STAMP_LIBRARY):
        pytest.skip("stamp library not built")
    stamps = ctypes.CDLL(STAMP_LIBRARY)
    assert hasattr(stamps, "tk_stage_stamps")
    stamps.tk_build_info.restype = ctypes.c_char_p
    assert b"stage-stamps" in stamps.tk_build_info()
    assert b"stage-stamps" not in tk.load().tk_build_info()


def test_constants():
    text = open(HEADER).read()
    assert tk.max_k() == int(re.search(r"#define TK_MAX_K (\d+)u", text).group(1)) == 256
    assert int(re.search(r"#define TK_MAX_K_LANE (\d+)u", text).group(1)) == 64
    assert tk.max_span_cols() >= 4 * 65000
    assert b"gfx950" in tk.load().tk_build_info()
    for s in range(9):
        assert tk.load().tk_status_string(s)


def v(rows=4, cols=100, stride=100, k=8, i=IN, o=IDX, val=VAL, c=CNT, m=MSK):
    return tk.validate(rows, cols, stride, k, i, o, val, c, m)


def test_guard_accepts_valid_calls():
    assert v() == OK
    assert v(rows=0, i=None, o=None, val=None, c=None, m=None) == OK  # empty: nothing is touched
    assert v(cols=0, stride=0) == OK
    assert v(cols=0, stride=0, i=None) == OK  # nothing of the input is read
    assert v(k=64) == OK and v(k=1) == OK and v(k=65) == OK and v(k=256) == OK
    assert v(k=64, cols=3, stride=3) == OK and v(k=256, cols=3, stride=3) == OK  # k may exceed cols
    assert v(i=IN + 2, val=VAL + 2) == OK    # 2-byte alignment is enough for bf16 buffers


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(rows=-1), SHAPE),
        (dict(cols=-1), SHAPE),
        (dict(cols=2**31, stride=2**31), SHAPE),
        (dict(stride=99), SHAPE),
        (dict(rows=2**40, stride=2**40), SHAPE),
        (dict(k=0), K),
        (dict(k=257), K),
        (dict(k=-3), K),
        (dict(i=None), NULL),
        (dict(o=None), NULL),
        (dict(val=None), NULL),
        (dict(c=None), NULL),
        (dict(m=None), NULL),
        (dict(i=IN + 1), ALIGN),
        (dict(val=VAL + 1), ALIGN),
        (dict(o=IDX + 2), ALIGN),
        (dict(c=CNT + 2), ALIGN),
        (dict(m=MSK + 1), ALIGN),
        (dict(o=IN + 64), ALIAS),                # output inside the input span
        (dict(val=IDX + 4 * 4 * 8 - 2), ALIAS),  # val overlaps the tail of idx
        (dict(c=MSK), ALIAS),                    # count and mask share storage
        (dict(m=IN + 2 * (3 * 100 + 100) - 4), ALIAS),  # mask overlaps the last input row
    ],
)
def test_guard_rejects(kw, status):
    assert v(**kw) == status


def test_guard_ignores_padding_when_cols_zero():
    # with cols == 0 nothing of the input is read, so nothing can alias it
    assert v(cols=0, stride=0, o=IN) == OK


def test_plan():
    assert tk.plan_spans(1024, 151936, 64) == 1      # enough rows for every CU
    assert tk.plan_spans(15, 98592, 32) > 1          # few rows: split
    assert tk.plan_spans(1, 4096, 8) == 1            # too narrow to split
    assert tk.plan_spans(4, 10**7, 8) >= (10**7 // 8 + 32639) // 32640  # span width limit
    assert tk.plan_spans(100000, 10**6, 8) >= 4
    # few rows, k <= 32: spans of about 12288 columns, 8 to 12 of them
    assert tk.plan_spans(15, 98592, 32) == 8
    assert tk.plan_spans(15, 49152, 32) == 8
    assert tk.plan_spans(15, 151936, 32) == 12
    assert tk.plan_spans(16, 248320, 20) == 12
    assert tk.plan_spans(64, 151936, 16) == 4        # the CU count asks for fewer
    assert tk.plan_spans(15, 98592, 64) == 12        # k = 64 keeps 12
    # 86 to 255 rows: twice the spans the CU count asks for (two or more workgroups per CU)
    assert tk.plan_spans(96, 98592, 32) == 6
    assert tk.plan_spans(128, 151936, 64) == 4
    assert tk.plan_spans(255, 98592, 8) == 4
    assert tk.plan_spans(128, 8192, 32) == 2         # no narrower than 4096 columns
    assert tk.plan_spans(128, 12288, 32) == 3
    assert tk.plan_spans(256, 151936, 64) == 1
    assert tk.plan_spans(128, 98592, 128) == 4         # k > 64 doubles too
    # 1 to 5 rows: up to 16 spans
    assert tk.plan_spans(1, 151936, 32) == 16
    assert tk.plan_spans(3, 98592, 32) == 16
    assert tk.plan_spans(5, 248320, 64) == 16
    assert tk.plan_spans(6, 98592, 32) == 8
    assert tk.plan_spans(2, 40000, 16) == 9          # no narrower than 4096 columns
    for rows in (1, 3, 15, 64, 255, 256, 1000):
        for cols in (0, 1, 4095, 4096, 70000, 151936, 248320, 600000):
            s = tk.plan_spans(rows, cols, 16)
            assert 1 <= s and (cols // 8 + s - 1) // s <= tk.max_span_cols() // 8


def test_plan_k1():
    # k = 1 (argmax scan): S = round(sqrt(cols / (150 rows))) on few rows of at
    # least 32768 columns, spans at least 2048 columns wide, at most 64
    assert tk.plan_spans(1024, 151936, 1) == 1
    assert tk.plan_spans(256, 151936, 1) == 1
    assert tk.plan_spans(15, 98592, 1) == 7          # sqrt(43.8) = 6.6
    assert tk.plan_spans(16, 248320, 1) == 10
    assert tk.plan_spans(64, 151936, 1) == 4
    assert tk.plan_spans(1, 151936, 1) == 32
    assert tk.plan_spans(1, 32767, 1) == 1 and tk.plan_spans(1, 4096, 1) == 1
    assert tk.plan_spans(1, 10**6, 1) == 64
    assert tk.plan_spans(4, 10**9, 1) >= 65          # beyond 64 spans: the general scan's plan
    for rows in (1, 3, 15, 64, 255, 256, 511, 512, 1000):
        for cols in (0, 1, 2048, 4095, 32768, 70000, 151936, 248320, 600000):
            s = tk.plan_spans(rows, cols, 1)
            assert 1 <= s <= 64 and (s == 1 or cols // s >= 2048)
            assert rows < 256 or s == max(1, -(-(cols // 8) // 32640))  # only the span width limit


def test_option_general_accepted_for_every_format():
    import ctypes

    lib = tk.load()
    for fmt in ("bf16", "f16", "f32"):
        fn = getattr(lib, f"tk_topk_{fmt}_ex")
        assert fn(0, 100, 100, 1, IN, IDX, VAL, CNT, MSK, 0, ctypes.byref(tk.TkOptions(general=1))) == OK


def test_plan_large_k():
    # k > 64: the k <= 64 plan, at most 12 spans unless the span width needs more
    assert tk.plan_spans(1024, 151936, 128) == 1
    assert tk.plan_spans(15, 98592, 256) == 12
    assert tk.plan_spans(64, 151936, 100) == 4
    assert tk.plan_spans(2, 10**7, 65) == (10**7 // 8 + 32639) // 32640
    for rows in (1, 15, 64, 256, 1000):
        for cols in (1, 4096, 70000, 248320, 600000):
            s = tk.plan_spans(rows, cols, 200)
            assert 1 <= s <= max(12, -(-(cols // 8) // 32640)) and s <= tk.plan_spans(rows, cols, 64)


@pytest.mark.parametrize("fmt", ["bf16", "f16", "f32"])
def test_option_fields(fmt):
    """tk_options: exact and general take 0 or 1, the reserved words must be
    zero; checked before any device work (rows == 0)."""
    import ctypes

    lib = tk.load()
    fn = getattr(lib, f"tk_topk_{fmt}_ex")

    def call(**kw):
        opt = tk.TkOptions(**{k: v for k, v in kw.items() if k != "reserved"})
        for i, v in kw.get("reserved", {}).items():
            opt.reserved[i] = v
        return fn(0, 100, 100, 1, IN, IDX, VAL, CNT, MSK, 0, ctypes.byref(opt))

    assert ctypes.sizeof(tk.TkOptions) == 32
    assert call() == OK and call(general=1) == OK and call(exact=1, general=1, spans=4) == OK
    assert call(general=2) == OPTION and call(general=-1) == OPTION and call(exact=2) == OPTION
    if fmt == "f32":
        def wide32(spans):
            return fn(0, 100000, 100000, 65, IN, IDX, VAL, CNT, MSK, 0, ctypes.byref(tk.TkOptions(spans=spans)))

        assert wide32(64) == OK and wide32(65) == OPTION
    else:
        # k > 64: at most 64 spans, forced or needed by the width
        def wide(spans, cols):
            return fn(0, cols, cols, 65, IN, IDX, VAL, CNT, MSK, 0, ctypes.byref(tk.TkOptions(spans=spans)))

        assert wide(64, 100000) == OK and wide(65, 100000) == OPTION
        assert wide(0, 64 * 261120) == OK and wide(0, 64 * 261120 + 8) == SHAPE
        assert tk.validate(1, 64 * 261120 + 8, 64 * 261120 + 8, 65, IN, IDX, VAL, CNT, MSK) == SHAPE
        assert tk.validate(1, 64 * 261120 + 8, 64 * 261120 + 8, 64, IN, IDX, VAL, CNT, MSK) == OK
    for i in range(5):
        assert call(reserved={i: 1}) == OPTION


def test_oracle_and_library_share_nothing():
    """The oracle and the HIP path are built from disjoint sources."""
    import oracle

    src = open(oracle.SOURCE).read()
    assert "#include \"" not in src  # only system headers
    for name in os.listdir(os.path.join(ROOT, "wide_row_bf16_amd", "csrc")):
        assert name not in src
    for root, _, files in os.walk(os.path.join(ROOT, "wide_row_bf16_amd")):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(root, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "tk_oracle" not in text, f


# Shard merge inputs [shards][rows][k] and outputs, at separated fake addresses.
M_IDX, M_VAL, M_CNT, M_MSK = 0x60000000, 0x70000000, 0x80000000, 0x90000000


def vm(rows=3, shards=4, k=8, idx=M_IDX, val=M_VAL, cnt=M_CNT, msk=M_MSK, oidx=IDX, oval=VAL, ocnt=CNT, omsk=MSK):
    return tk.validate_merge(rows, shards, k, idx, val, cnt, msk, oidx, oval, ocnt, omsk)


def test_merge_guards():
    assert vm() == OK
    assert vm(rows=0, idx=None, val=None, cnt=None, msk=None, oidx=None, oval=None, ocnt=None, omsk=None) == OK
    assert vm(shards=1) == OK and vm(shards=4096) == OK
    assert vm(shards=0) == SHAPE and vm(shards=4097) == SHAPE and vm(rows=-1) == SHAPE
    assert vm(k=0) == K and vm(k=65) == K
    assert vm(val=None) == NULL and vm(omsk=None) == NULL
    assert vm(val=M_VAL + 1) == ALIGN and vm(idx=M_IDX + 2) == ALIGN and vm(ocnt=CNT + 2) == ALIGN
    # an output inside an input, or two outputs overlapping: rejected
    assert vm(oidx=M_IDX + 64) == ALIAS
    assert vm(oval=IDX + 8) == ALIAS
    # inputs may share memory (they are only read)
    assert vm(cnt=M_IDX, msk=M_IDX) == OK


def test_shard_col_base_guard():
    """Global indices must fit int32: rejected on the host before any HIP call."""
    lib = tk.load()
    args = (3, 100, 100, 8)
    bufs = (IN, IDX, VAL, CNT, MSK, 0)
    assert lib.tk_topk_bf16_shard(*args, -1, *bufs) == SHAPE
    assert lib.tk_topk_bf16_shard(*args, 2**31 - 100 + 1, *bufs) == SHAPE
    # rows == 0 returns before any device work; the largest valid base passes the guard
    assert lib.tk_topk_bf16_shard(0, 100, 100, 8, 2**31 - 100, *bufs) == OK


def vs(rows=3, k=8, idx=M_IDX, val=M_VAL, cnt=M_CNT, t=0.7, p=0.95, tok=IDX, kept=CNT):
    return tk.validate_sample(rows, k, idx, val, cnt, t, p, tok, kept)


def test_sample_guards():
    assert vs() == OK
    assert vs(t=0.0) == OK and vs(p=1.0) == OK
    assert vs(rows=0, idx=None, val=None, cnt=None, tok=None, kept=None) == OK
    assert vs(k=0) == K and vs(k=65) == K and vs(rows=-1) == SHAPE
    assert vs(t=-0.1) == OPTION and vs(t=float("nan")) == OPTION and vs(t=float("inf")) == OPTION
    assert vs(p=0.0) == OPTION and vs(p=1.0001) == OPTION and vs(p=float("nan")) == OPTION
    assert vs(val=None) == NULL and vs(kept=None) == NULL
    assert vs(val=M_VAL + 1) == ALIGN and vs(tok=IDX + 2) == ALIGN
    assert vs(tok=M_IDX + 16) == ALIAS and vs(kept=IDX) == ALIAS


def test_f32_guards():
    def v32(rows=3, cols=100, stride=100, k=8, i=IN, idx=IDX, val=VAL, cnt=CNT, msk=MSK):
        return tk.validate_f32(rows, cols, stride, k, i, idx, val, cnt, msk)

    assert v32() == OK
    assert v32(i=IN + 2) == ALIGN and v32(val=VAL + 2) == ALIGN  # 4-byte elements
    assert v32(i=IN + 4) == OK
    assert v32(k=0) == K and v32(stride=99) == SHAPE
    assert v32(k=64) == OK and v32(k=256) == OK and v32(k=257) == K
    # the input spans 4 bytes per element: an output 1000 bytes in overlaps it
    assert v32(idx=IN + 1000) == ALIAS
    assert tk.validate(3, 100, 100, 8, IN, IN + 1000, VAL, CNT, MSK) == OK  # bf16: 600 bytes of input only
    lib = tk.load()
    opt = tk.TkOptions(spans=65, exact=0)
    import ctypes

    assert lib.tk_topk_f32_ex(0, 100, 100, 8, IN, IDX, VAL, CNT, MSK, 0, ctypes.byref(opt)) == OPTION


W_FAKE = 0x100000000  # above every other fake address: the weights span 404 MB


def vh(rows=15, hidden=2048, vocab=98592, k=32, h=0x1000000, hs=2048, w=W_FAKE, ws=2048, idx=IDX, val=VAL,
       cnt=CNT, msk=MSK, lg=None, ls=0):
    return tk.validate_head(rows, hidden, vocab, k, h, hs, w, ws, idx, val, cnt, msk, lg, ls)


def test_head_guards():
    assert vh() == OK and vh(rows=64) == OK and vh(rows=1, vocab=1, hidden=32, hs=32, ws=32) == OK
    assert vh(rows=0, h=None, w=None, idx=None, val=None, cnt=None, msk=None) == OK
    assert vh(rows=65) == SHAPE and vh(rows=-1) == SHAPE
    assert vh(hidden=16, hs=16, ws=16) == SHAPE and vh(hidden=48, hs=48, ws=48) == SHAPE  # multiple of 32
    assert vh(hidden=65536 + 32, hs=65568, ws=65568) == SHAPE and vh(vocab=0) == SHAPE
    assert vh(hs=2047) == SHAPE and vh(ws=2052) == SHAPE and vh(ws=2**21 + 8) == SHAPE    # strides
    assert vh(k=0) == K and vh(k=65) == K and vh(k=64) == OK
    assert vh(h=None) == NULL and vh(msk=None) == NULL
    assert vh(h=0x1000008) == ALIGN and vh(w=W_FAKE + 2) == ALIGN and vh(val=VAL + 1) == ALIGN
    assert vh(lg=0x60000000, ls=98592) == OK and vh(lg=0x60000000, ls=98591) == SHAPE
    assert vh(lg=0x60000001, ls=98592) == ALIGN
    assert vh(idx=W_FAKE + 1024) == ALIAS                  # an output inside the weights
    assert vh(lg=VAL - 64, ls=98592) == ALIAS               # logits over an output
    assert vh(cnt=MSK) == ALIAS
    # logits rows are addressed in 64 bits: a stride that would overflow is rejected
    assert vh(lg=0x60000000, ls=2**62) == SHAPE and vh(lg=0x60000000, ls=2**56) == SHAPE
    assert vh(lg=0x60000000, ls=2**54 - 2**40) != SHAPE  # just inside the bound (then overlaps the outputs)


def _cpu_out(torch, rows, k, val_dtype=None, **over):
    val_dtype = torch.bfloat16 if val_dtype is None else val_dtype
    t = {"idx": torch.empty((rows, k), dtype=torch.int32), "val": torch.empty((rows, k), dtype=val_dtype),
         "count": torch.empty((rows,), dtype=torch.int32), "nonfinite": torch.empty((rows,), dtype=torch.int32)}
    t.update(over)
    return tk.TopK(t["idx"], t["val"], t["count"], t["nonfinite"])


def test_binding_rejects_mismatched_out_tensors():
    """Reused outputs of the wrong shape, dtype or layout would let the kernels
    write past them; the binding's check raises before any call (CPU tensors,
    the check alone)."""
    import torch

    cpu = torch.device("cpu")
    tk._check_out(torch, _cpu_out(torch, 4, 8), 4, 8, "bf16", cpu)
    tk._check_out(torch, _cpu_out(torch, 4, 8, torch.float32), 4, 8, "f32", cpu)
    tk._check_out(torch, _cpu_out(torch, 4, 8, torch.float16), 4, 8, "f16", cpu)
    bad = [
        (_cpu_out(torch, 4, 4), 4, 8, "bf16"),                           # smaller k
        (_cpu_out(torch, 2, 8), 4, 8, "bf16"),                           # fewer rows
        (_cpu_out(torch, 4, 8), 4, 8, "f32"),                            # 2-byte values for 4-byte entries
        (_cpu_out(torch, 4, 8, torch.float32), 4, 8, "bf16"),            # 4-byte values for bf16
        (_cpu_out(torch, 4, 8, idx=torch.empty((4, 8), dtype=torch.int64)), 4, 8, "bf16"),
        (_cpu_out(torch, 4, 8, idx=torch.empty((8, 4), dtype=torch.int32).t()), 4, 8, "bf16"),  # not contiguous
        (_cpu_out(torch, 4, 8, count=torch.empty((5,), dtype=torch.int32)), 4, 8, "bf16"),
        (_cpu_out(torch, 4, 8, nonfinite=torch.empty((4,), dtype=torch.int16)), 4, 8, "bf16"),
        ((1, 2, 3), 4, 8, "bf16"),
    ]
    for out, rows, k, fmt in bad:
        with pytest.raises(ValueError):
            tk._check_out(torch, out, rows, k, fmt, cpu)
    with pytest.raises(ValueError):  # outputs on another device than the input
        tk._check_out(torch, _cpu_out(torch, 4, 8), 4, 8, "bf16", torch.device("cuda", 0))



def test_probe_read_guards():
    """The measurement probe rejects bad arguments before any launch."""
    lib = tk.load()
    S = 0x70000000
    assert lib.tk_probe_read(IN, -16, 4, S, None) == SHAPE
    assert lib.tk_probe_read(IN, 17, 4, S, None) == SHAPE
    assert lib.tk_probe_read(IN, 1024, 0, S, None) == SHAPE
    assert lib.tk_probe_read(IN, 1024, 2**24 + 1, S, None) == SHAPE
    assert lib.tk_probe_read(IN, 16 * 4 * 2**26, 1, S, None) == SHAPE   # a wave's share too large
    assert lib.tk_probe_read(None, 1024, 4, S, None) == NULL
    assert lib.tk_probe_read(IN, 1024, 4, None, None) == NULL
    assert lib.tk_probe_read(IN + 8, 1024, 4, S, None) == ALIGN
    assert lib.tk_probe_read(IN, 1024, 4, S + 2, None) == ALIGN
    assert lib.tk_probe_read(IN, 1 << 20, 4, IN + 4096, None) == ALIAS
