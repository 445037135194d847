"""The draft head fused with the row top-k (tk_head_topk_bf16) against the
oracle, in two halves (oracle/head.py): the logits the kernel computed are
within the float32-accumulation + bf16-rounding bound of the exact sums, and
the top-k it returned equals the library's operation on those logits byte
for byte -- with and without the logits being written out.  Shapes cover one
to four 16-row matrix-core tiles, ragged vocabulary spans, padded strides,
k beyond the vocabulary, tied logits, exact integer sums, non-finite hidden
states, and the 15 x 98592 draft-head shape at hidden 2048."""

import numpy as np
import pytest

import oracle
from gpu_util import assert_same, log, need_gpu, to_numpy
from oracle.head import check_head_logits
from synth import head_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # rows, hidden, vocab, k, h_pad, w_pad, kind
    (1, 32, 1, 1, 0, 0, "normal"),
    (1, 32, 5, 8, 8, 0, "normal"),
    (3, 64, 255, 16, 0, 8, "normal"),
    (15, 128, 256, 32, 8, 8, "normal"),
    (16, 96, 257, 64, 0, 0, "ties"),
    (17, 160, 1000, 20, 8, 0, "normal"),
    (31, 256, 4097, 64, 0, 8, "ties"),
    (33, 1024, 3000, 10, 0, 0, "normal"),
    (64, 512, 9000, 64, 8, 8, "normal"),
    (5, 64, 700, 16, 0, 0, "integers"),
    (40, 96, 1500, 33, 0, 0, "integers"),
    (9, 64, 500, 16, 0, 0, "nonfinite"),
    (7, 2016, 3000, 24, 8, 8, "normal"),  # one row tile, 32 hidden blocks of which the last is half
    (12, 1056, 2000, 32, 0, 0, "integers"),
    (15, 2048, 98592, 32, 0, 0, "normal"),
    (64, 1024, 151936, 8, 0, 0, "normal"),
    (32, 512, 40000, 16, 0, 8, "normal"),  # a multiple of the CU count as spans: 9-10 tiles each
    (5, 128, 33000, 64, 8, 0, "ties"),  # the same rule at 8-9 tiles a span, ties across spans
    (3, 65536, 300, 8, 0, 0, "normal"),  # the largest hidden: 1024 blocks walked from a rotated start
    (20, 65504, 130, 16, 0, 8, "integers"),  # two row tiles, a half last block, exact sums
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _dev(m):
    import torch

    return torch.from_numpy(np.ascontiguousarray(m).view(np.int16)).to("cuda")


def _check(hb, wb, hidden, vocab, k, what):
    import torch

    import wide_row_bf16_amd as tk

    h = _dev(hb)[:, :hidden]
    w = _dev(wb)[:, :hidden]
    top, lg = tk.head_topk_bf16(h, w, k, logits=True)
    torch.cuda.synchronize()
    lgb = lg.view(torch.int16).cpu().numpy().view(np.uint16)
    ok, msg = check_head_logits(lgb, hb[:, :hidden], wb[:, :hidden])
    assert ok, f"{what}: {msg}"
    want = oracle.topk_bf16(lgb, vocab, k)
    assert_same(to_numpy(top), want, what)
    assert_same(to_numpy(tk.head_topk_bf16(h, w, k)), want, what + " (no logits written)")


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}k{c[3]}{c[6]}" for c in CASES])
def test_head(case):
    rows, hidden, vocab, k, h_pad, w_pad, kind = case
    what = f"head rows={rows} hidden={hidden} vocab={vocab} k={k} pads={h_pad},{w_pad} kind={kind}"
    log(what)
    hb, wb = head_inputs(rows, hidden, vocab, seed=rows * 7 + vocab, h_pad=h_pad, w_pad=w_pad, kind=kind)
    _check(hb, wb, hidden, vocab, k, what)


def test_zero_hidden_states_tie_every_column():
    """h = 0 (both signs): every logit is a zero, all tied, so the first k
    columns win; the sign of each zero logit is carried to the entry."""
    hb, wb = head_inputs(6, 64, 600, seed=5)
    hb[:3, :] = 0x0000
    hb[3:, :] = 0x8000
    _check(hb, wb, 64, 600, 40, "zero hidden states")


def test_every_row_count_and_vocab_edge():
    for rows in (1, 2, 15, 16, 17, 32, 33, 48, 63, 64):
        for vocab in (255, 256, 257, 511, 513):
            what = f"rows={rows} vocab={vocab}"
            log(what)
            hb, wb = head_inputs(rows, 32, vocab, seed=rows + vocab)
            _check(hb, wb, 32, vocab, 8, what)


def test_rejected_and_empty_calls():
    import torch

    import wide_row_bf16_amd as tk

    h = torch.zeros((65, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((10, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tk.TkError) as e:
        tk.head_topk_bf16(h, w, 4)
    assert e.value.status == 2
    with pytest.raises(tk.TkError) as e:
        tk.head_topk_bf16(h[:4, :48], w[:, :48], 4)  # hidden not a multiple of 32
    assert e.value.status == 2
    out = tk.head_topk_bf16(h[:0], w, 4)
    assert out.idx.shape == (0, 4)


def test_wide_pads_on_tight_storage():
    """Row pads wider than one 128-byte block of the kernel's walk, poisoned
    with NaN, and w's storage ending at the last row's hidden-th element (no
    pad after it): the loads past `hidden` must read nothing outside the
    weights and use none of the pad."""
    import torch

    import wide_row_bf16_amd as tk

    for rows, hidden, vocab, k, pad in ((15, 2048, 4000, 32, 136), (3, 96, 700, 16, 200), (33, 512, 1300, 20, 72)):
        what = f"tight w storage rows={rows} hidden={hidden} vocab={vocab} pad={pad}"
        log(what)
        hb, wb = head_inputs(rows, hidden, vocab, seed=vocab + pad, h_pad=pad, w_pad=pad)
        ws = hidden + pad
        flat = np.ascontiguousarray(wb).reshape(-1)[: (vocab - 1) * ws + hidden]
        wdev = torch.from_numpy(flat.view(np.int16).copy()).to("cuda")
        w = wdev.as_strided((vocab, hidden), (ws, 1))
        h = _dev(hb)[:, :hidden]
        top, lg = tk.head_topk_bf16(h, w, k, logits=True)
        torch.cuda.synchronize()
        lgb = lg.view(torch.int16).cpu().numpy().view(np.uint16)
        ok, msg = check_head_logits(lgb, hb[:, :hidden], wb[:, :hidden])
        assert ok, f"{what}: {msg}"
        assert_same(to_numpy(top), oracle.topk_bf16(lgb, vocab, k), what)


def test_mismatched_out_is_rejected_before_launch():
    import torch

    import wide_row_bf16_amd as tk

    hb, wb = head_inputs(4, 64, 300, seed=3)
    h, w = _dev(hb), _dev(wb)
    small = tk.head_topk_bf16(h, w, 8)
    with pytest.raises(ValueError):
        tk.head_topk_bf16(h, w, 16, out=small)
    x = torch.zeros((4, 1000), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        tk.topk_bf16(x, 16, out=small)
    with pytest.raises(ValueError):
        tk.topk_f32(x.float(), 8, out=small)  # bf16 values for 4-byte entries
