"""Pins of the oracle's activation prologue (CPU only).

The layers' set_activation (BinaryConv2dCutlass on the qconv/binary/cutlass/layer page,
BinaryLinearCuda on the BinaryLinearCuda page) shifts the input by bias_a before the sign is
taken, and sets a zero scale_a to 2 * mean|x| (symmetric) or 4 * mean|x|. These tests tie the
oracle to things other than itself: a hand-worked table of IEEE edge cases, torch's own add and
compare under its type promotion (a library routine), and closed forms of the mean.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _from_bits(dt, hexbits):
    v = int(hexbits, 16)
    if dt == "f32":
        return torch.tensor([v - (1 << 32) if v >= 1 << 31 else v], dtype=torch.int32).view(torch.float32)
    return torch.tensor([v - (1 << 16) if v >= 1 << 15 else v], dtype=torch.int16).view(DT[dt])


def _unpack_rows(words, k):
    w = words.numpy().astype(np.uint32).astype(np.int64)
    return ((w[..., None] >> np.arange(32)) & 1).reshape(words.shape[0], k)


def _torch_bits(x, bias):
    """(x + bias >= 0) as computed by torch in the dtype its promotion picks."""
    return ((x + bias) >= 0).numpy().astype(np.int64)


def test_shift_sign_edge_table():
    table = json.load(open(os.path.join(GOLDEN, "shift_sign_edges.json")))
    for xdt, xh, bdt, bh, want, why in table["cases"]:
        x, b = _from_bits(xdt, xh), _from_bits(bdt, bh)
        # one element per word position would not make a word: repeat the pair over 32 columns
        xr, br = x.repeat(32).view(1, 32).contiguous(), b.repeat(32).contiguous()
        bits = _unpack_rows(oracle.pack_rows_shift(xr, br), 32)
        got = 1 if bits[0, 0] else -1
        assert got == want, f"{xdt}:{xh} + {bdt}:{bh}: {why}"
        assert bits.min() == bits.max()
        # the hand-worked expectation agrees with torch's add under type promotion
        assert (1 if bool(((x + b) >= 0)[0]) else -1) == want, why
        # a single bias value (layer-wise form) gives the same bits
        assert torch.equal(oracle.pack_rows_shift(xr, b.contiguous()), oracle.pack_rows_shift(xr, br))


@pytest.mark.parametrize("xdt,bdt", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "f32"),
                                     ("bf16", "f32"), ("f32", "f16")])
def test_rows_shift_matches_torch_per_column(xdt, bdt):
    gen = torch.Generator().manual_seed(11)
    rows, k = 7, 96
    x = torch.randn((rows, k), generator=gen).to(DT[xdt])
    bias = (0.5 * torch.randn(k, generator=gen)).to(DT[bdt])
    # exact cancellations: some bias entries are the negation of an input of their column
    bias[::5] = (-x[3, ::5].float()).to(DT[bdt])
    got = _unpack_rows(oracle.pack_rows_shift(x, bias), k)
    assert np.array_equal(got, _torch_bits(x, bias))
    # per-column indexing: a bias that differs only in column 40 changes only column 40
    b2 = bias.clone()
    b2[40] = 1e4
    diff = got != _unpack_rows(oracle.pack_rows_shift(x, b2), k)
    assert diff[:, [c for c in range(k) if c != 40]].sum() == 0


def test_rows_shift_layerwise_scalar():
    gen = torch.Generator().manual_seed(12)
    x = torch.randn((5, 64), generator=gen)
    for bval in (0.0, 0.3, -0.3, float(-x[2, 7])):
        b = torch.tensor([bval], dtype=torch.float32)
        assert np.array_equal(_unpack_rows(oracle.pack_rows_shift(x, b), 64), _torch_bits(x, b))
    assert torch.equal(oracle.pack_rows_shift(x, torch.zeros(1)), oracle.pack_rows(x))


def test_all_f16_patterns_shift():
    allbits = torch.arange(-(1 << 15), 1 << 15, dtype=torch.int32).to(torch.int16).view(torch.float16)
    x = allbits.view(-1, 64).contiguous()
    for bval in (0.0, -0.0, 1.0, -1.0, 6.1035e-05, -65504.0):
        b = torch.tensor([bval], dtype=torch.float16)
        got = _unpack_rows(oracle.pack_rows_shift(x, b), 64)
        assert np.array_equal(got, _torch_bits(x, b)), bval


@pytest.mark.parametrize("xdt,bdt", [("f32", "f32"), ("f16", "f16"), ("bf16", "f32")])
def test_nchw_shift_matches_torch_per_channel(xdt, bdt):
    gen = torch.Generator().manual_seed(13)
    b, c, h, w = 2, 64, 5, 3
    x = (0.1 + torch.randn((b, c, h, w), generator=gen)).to(DT[xdt])
    bias = (0.5 * torch.randn(c, generator=gen)).to(DT[bdt])
    bias[::7] = (-x[1, ::7, 2, 1].float()).to(DT[bdt])
    want = ((x + bias.view(1, -1, 1, 1)) >= 0)                           # the layer's broadcast
    words = oracle.pack_nchw_shift(x, bias)                                # [b, h, w, c/32]
    bits = _unpack_rows(words.reshape(-1, c // 32), c).reshape(b, h, w, c)
    assert np.array_equal(bits, want.permute(0, 2, 3, 1).numpy().astype(np.int64))
    assert torch.equal(oracle.pack_nchw_shift(x, torch.zeros(c, dtype=DT[bdt])), oracle.pack_nchw(x))


def test_abs_mean_closed_forms():
    n = 1000
    ints = torch.arange(n, dtype=torch.float32)                           # sum = n(n-1)/2
    assert oracle.abs_mean_scale(ints, 2.0) == n - 1
    assert oracle.abs_mean_scale(-ints, 4.0) == 2 * (n - 1)
    alt = torch.tensor([1.0, -1.0] * 64, dtype=torch.float16)
    assert oracle.abs_mean_scale(alt, 2.0) == 2.0 and oracle.abs_mean_scale(alt, 4.0) == 4.0
    assert oracle.abs_mean_scale(torch.tensor([0.5, -2.5]), 2.0) == 3.0
    assert oracle.abs_mean_scale(torch.tensor([-0.0, 0.0]), 2.0) == 0.0
    assert oracle.abs_mean_scale(torch.tensor([1.0, float("-inf")]), 2.0) == float("inf")
    assert np.isnan(oracle.abs_mean_scale(torch.tensor([1.0, float("nan")]), 2.0))


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_abs_mean_matches_numpy(dt):
    gen = torch.Generator().manual_seed(14)
    x = (0.1 + torch.randn(100003, generator=gen)).to(DT[dt])
    want = 4.0 * np.abs(x.float().numpy().astype(np.float64)).mean()      # numpy's pairwise sum
    assert oracle.abs_mean_scale(x, 4.0) == pytest.approx(want, rel=1e-12)
