"""Robustness of the HIP path: nothing written outside the outputs, repeat
runs bit-identical, concurrent streams equal to solo runs (the invariant the
TensorFold pages check as "concurrent == solo"), and rejected calls leave the
outputs untouched."""

import numpy as np
import pytest

import oracle
from gpu_util import assert_same, log, need_gpu, to_numpy, upload
from synth import family_rows, make_config_input

pytestmark = pytest.mark.gpu

CANARY = 0x5A5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def canaried_outputs(rows, k, pad=16):
    import torch

    import wide_row_bf16_amd as tk

    bufs = [
        torch.full((rows * k + 2 * pad,), CANARY, dtype=torch.int32, device="cuda"),
        torch.full((rows * k + 2 * pad,), CANARY, dtype=torch.int16, device="cuda"),
        torch.full((rows + 2 * pad,), CANARY, dtype=torch.int32, device="cuda"),
        torch.full((rows + 2 * pad,), CANARY, dtype=torch.int32, device="cuda"),
    ]
    out = tk.TopK(
        bufs[0][pad:pad + rows * k].view(rows, k),
        bufs[1][pad:pad + rows * k].view(rows, k).view(torch.bfloat16),
        bufs[2][pad:pad + rows],
        bufs[3][pad:pad + rows],
    )
    return bufs, out


def canaries_intact(bufs, pad=16):
    for b in bufs:
        h = b.cpu().numpy()
        if not (np.all(h[:pad] == CANARY) and np.all(h[-pad:] == CANARY)):
            return False
    return True


@pytest.mark.parametrize("spans", [0, 1, 7])
def test_nothing_written_outside_outputs(spans):
    import wide_row_bf16_amd as tk

    for fam, rows, cols, k in (("mixed_nonfinite", 5, 70001, 20), ("all_nan", 3, 999, 64), ("normal", 1, 4096, 1)):
        m = family_rows(fam, rows, cols, cols + 5, seed=rows)
        bufs, out = canaried_outputs(rows, k)
        log(f"canary {fam} spans={spans}")
        tk.topk_bf16(upload(m), k, cols=cols, spans=spans if spans <= cols else 0, out=out)
        got = to_numpy(out)
        assert canaries_intact(bufs)
        assert_same(got, oracle.topk_bf16(m, cols, k), f"canary {fam}")


def test_repeat_runs_bit_identical():
    import wide_row_bf16_amd as tk

    m = make_config_input("c4")
    x = upload(m)
    first = to_numpy(tk.topk_bf16(x, 16, cols=151936))
    for _ in range(5):
        again = to_numpy(tk.topk_bf16(x, 16, cols=151936))
        assert_same(again, first, "repeat")


def test_concurrent_streams_equal_solo():
    import torch

    import wide_row_bf16_amd as tk

    ms = [family_rows(f, 16, 151936, 152064, seed=i) for i, f in enumerate(("logit", "normal", "levels64", "mixed_nonfinite"))]
    xs = [upload(m) for m in ms]
    solo = [to_numpy(tk.topk_bf16(x, 16, cols=151936)) for x in xs]
    streams = [torch.cuda.Stream() for _ in xs]
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        for x, s in zip(xs, streams):
            with torch.cuda.stream(s):
                outs.append(tk.topk_bf16(x, 16, cols=151936, spans=4))
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert_same(to_numpy(o), solo[i % 4], f"stream {i % 4}")


def test_rejected_calls_write_nothing():
    import wide_row_bf16_amd as tk

    m = family_rows("normal", 4, 1000, 1000, seed=3)
    x = upload(m)
    bufs, out = canaried_outputs(4, 8)
    for kw in (dict(spans=2000), dict(spans=-1)):
        with pytest.raises(tk.TkError) as e:
            tk.topk_bf16(x, 8, out=out, **kw)
        assert e.value.status == 7
    for b in bufs:
        assert np.all(b.cpu().numpy() == CANARY)
    bufs, out = canaried_outputs(4, 257)  # outputs of the right shape: the library's own k guard rejects
    with pytest.raises(tk.TkError) as e:
        tk.topk_bf16(x, 257, out=out)
    assert e.value.status == 3
    for b in bufs:
        assert np.all(b.cpu().numpy() == CANARY)
    with pytest.raises(ValueError):  # outputs of another k: the binding rejects before any call
        tk.topk_bf16(x, 16, out=out)
    for b in bufs:
        assert np.all(b.cpu().numpy() == CANARY)


def test_many_rows():
    for rows, cols, k in ((70000, 64, 8), (5000, 1500, 64), (300, 30000, 5)):
        m = family_rows("uniform_bits", rows, cols, cols, seed=rows)
        log(f"many rows {rows}x{cols} k={k}")
        from gpu_util import check_case

        check_case(m, cols, k, what=f"{rows}x{cols}")


def test_fused_merge_state_across_calls_and_batches():
    """Split rows are folded by the last scan workgroup of each row, which
    counts arrivals in per-row counters that must return to zero after every
    call.  Alternating shapes on one stream, several row batches in one call
    (more split rows than one launch takes) and span counts on both sides of
    the fused limit (64) must all give the oracle's bytes."""
    cases = [
        ("normal", 15, 98592, 32, 0),
        ("mixed_nonfinite", 40, 20000, 7, 5),
        ("levels64", 15, 98592, 32, 64),
        ("uniform_bits", 3, 98592, 64, 65),
        ("logit", 15, 98592, 32, 0),
        ("zeros_straddle", 9000, 128, 4, 2),
        ("normal", 15, 98592, 32, 18),
    ]
    for family, rows, cols, k, spans in cases:
        m = family_rows(family, rows, cols, cols + 3, seed=rows + spans)
        log(f"fused family={family} rows={rows} cols={cols} k={k} spans={spans}")
        want = oracle.topk_bf16(m, cols, k)
        from gpu_util import gpu_topk

        for _ in range(2):
            assert_same(gpu_topk(m, cols, k, spans=spans), want, f"{family} {rows}x{cols} k={k} spans={spans}")


def test_library_loaded_before_torch():
    """A caller that loads the library before importing torch must get working
    calls: the binding imports torch before opening the library, so both use
    the HIP runtime torch brings (a second, system runtime beside it made
    every call fail with TK_ERR_DEVICE).  Runs in a fresh process, since this
    one has torch loaded already."""
    import json
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import sys, json\n"
        f"sys.path.insert(0, {root!r})\n"
        "import wide_row_bf16_amd as tk\n"
        "tk.load()\n"
        "import numpy as np, torch\n"
        "from synth import family_rows\n"
        "m = family_rows('mixed_nonfinite', 3, 5000, 5003, seed=3)\n"
        "x = torch.from_numpy(m.view(np.int16)).to('cuda')\n"
        "o = tk.topk_bf16(x, 16, cols=5000)\n"
        "print(json.dumps([o.idx.cpu().tolist(), o.count.cpu().tolist()]))\n"
    )
    log("fresh process: library loaded before torch")
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert proc.returncode == 0, proc.stderr[-2000:]
    idx, count = json.loads(proc.stdout.strip().splitlines()[-1])
    m = family_rows("mixed_nonfinite", 3, 5000, 5003, seed=3)
    want = oracle.topk_bf16(m, 5000, 16)
    assert np.array_equal(np.array(idx, dtype=np.int32), want[0])
    assert np.array_equal(np.array(count, dtype=np.int32), want[2])


def test_read_probe_reads_and_writes_nothing():
    """The measurement probe streams a buffer (and, with no buffer, launches an
    empty grid) without writing anything: its sink keeps its contents."""
    import torch

    import wide_row_bf16_amd as tk

    sink = torch.full((8192,), 7, dtype=torch.int32, device="cuda")
    for n, wgs in ((1 << 20, 64), (4096 * 16 + 48, 300), (16, 1)):
        x = torch.zeros((n // 2,), dtype=torch.int16, device="cuda")
        tk.read_probe(x, wgs, sink)
    tk.read_probe(None, 180, sink)
    torch.cuda.synchronize()
    assert np.all(sink.cpu().numpy() == 7)
    with pytest.raises(tk.TkError) as e:
        tk.read_probe(torch.zeros((9,), dtype=torch.int16, device="cuda"), 4, sink)  # 18 bytes
    assert e.value.status == 2


def test_release_stream_then_new_streams():
    """Split-row calls on a stream, tk_release_stream, the stream destroyed,
    then new streams (whose handle values may repeat the old one): every call
    still equals the oracle, and releasing a stream twice, or one the library
    never saw, is harmless."""
    import torch

    import wide_row_bf16_amd as tk

    m = family_rows("normal", 15, 98592, 98592, seed=11)
    want = oracle.topk_bf16(m, 98592, 32)
    x = upload(m)
    for i in range(4):
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            for _ in range(3):
                got = tk.topk_bf16(x, 32)
            tk.release_stream(s)
            tk.release_stream(s)
            again = tk.topk_bf16(x, 32)  # allocates afresh on the same stream
            tk.release_stream(s)
        s.synchronize()
        assert_same(to_numpy(got), want, f"stream {i}")
        assert_same(to_numpy(again), want, f"stream {i} after release")
        del s
    tk.release_stream(torch.cuda.Stream())


def test_stamp_build_same_outputs_and_ordered_stages():
    """The stage-timestamp build (libtk_topk_stamps.so) computes the same
    outputs as the library, and its table holds ordered stages for a split
    and an unsplit launch."""
    import ctypes
    import os

    import torch

    import wide_row_bf16_amd as tk
    from wide_row_bf16_amd.build import STAMP_LIBRARY

    if not os.path.exists(STAMP_LIBRARY):
        pytest.skip("stamp library not built")
    lib = tk.load(STAMP_LIBRARY)
    lib.tk_stage_stamps.restype = ctypes.c_int
    lib.tk_stage_stamps.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    stream = torch.cuda.current_stream().cuda_stream
    for rows, cols, k, spans in ((15, 98592, 32, 12), (6, 40000, 16, 1)):
        log(f"stamp build rows={rows} cols={cols} k={k} spans={spans}")
        m = family_rows("normal", rows, cols, seed=rows + k)
        x = upload(m)
        want = tk.topk_bf16(x, k, spans=spans)
        outs = [torch.empty(sh, dtype=dt, device="cuda") for sh, dt in
                (((rows, k), torch.int32), ((rows, k), torch.int16), ((rows,), torch.int32), ((rows,), torch.int32))]
        opt = tk.TkOptions(spans=spans, exact=0, general=0)
        assert lib.tk_topk_bf16_ex(rows, cols, cols, k, x.data_ptr(), *[o.data_ptr() for o in outs], stream,
                                   ctypes.byref(opt)) == 0
        torch.cuda.synchronize()
        assert_same(to_numpy(tk.TopK(*outs)), to_numpy(want), "stamp build vs library")
        buf = np.zeros(8192 * 16, dtype=np.uint64)
        assert lib.tk_stage_stamps(buf.ctypes.data, buf.nbytes) == 0
        t = buf.reshape(8192, 16)[: rows * spans].astype(np.int64)
        # orders the kernel guarantees (thread 0 stamps 0, 1, 6, 7 in turn; every
        # wave's body ends after the floor barrier and before the publish one)
        assert (t[:, 1] >= t[:, 0]).all() and (t[:, 2:6].min(axis=1) >= t[:, 0]).all()
        assert (t[:, 6] >= t[:, 2:6].max(axis=1)).all() and (t[:, 6] >= t[:, 1]).all()
        assert (t[:, 7] >= t[:, 6]).all()
        if spans > 1:
            last = (t[:, 13] & 1) == 1
            assert last.sum() == rows
            assert (t[last, 12] >= t[last, 11]).all() and (t[last, 11] >= t[last, 10]).all()
            assert (t[last, 10] >= t[last, 9]).all() and (t[:, 9] >= t[:, 8]).all() and (t[:, 8] >= t[:, 7]).all()
        assert ((t[:, 14] >> 32) < 8).all()  # XCC ids
