"""Pins of the oracle's 8-bit containers (CPU only).

The CUTLASS conv layer keeps packed signs in uint8_t containers (bits_binary_word = 8;
BinaryConv2dCutlass.__init__ and _check_forward on the qconv/binary/cutlass/layer page). The
oracle's byte packs are pinned against hand-worked bytes (tests/golden/u8_container.json), against
torch's own x >= 0 compare unpacked bit by bit (all three input dtypes, IEEE edge values), and
against the 32-bit words: the bytes of a row are the leading bytes of its little-endian words.
"""
import json
import os

import numpy as np
import pytest
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "u8_container.json")


def _num(v):
    return {"-0": -0.0, "nan": float("nan"), "-inf": float("-inf"), "inf": float("inf")}[v] \
        if isinstance(v, str) else float(v)


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_u8_golden_rows_and_pixels(oracle_lib, dtype):
    g = json.load(open(GOLDEN))
    for row in g["rows"]:
        x = torch.tensor([[_num(v) for v in row["x"]]], dtype=torch.float32).to(dtype)
        assert torch.equal(oracle_lib.sign(x)[0], torch.tensor(row["signs"], dtype=torch.float32))
        assert oracle_lib.pack_rows_u8(x)[0].tolist() == [int(h, 16) for h in row["bytes"]]
    nc = g["nchw"]
    x = torch.tensor([[_num(a), _num(b)] for a, b in zip(nc["pixel0"], nc["pixel1"])],
                     dtype=torch.float32).view(1, 10, 1, 2).to(dtype)
    got = oracle_lib.pack_nchw_u8(x)
    assert got.shape == (1, 1, 2, 2)
    assert got[0, 0, 0].tolist() == [int(h, 16) for h in nc["bytes0"]]
    assert got[0, 0, 1].tolist() == [int(h, 16) for h in nc["bytes1"]]


def _unpack(t, n):
    return np.unpackbits(t.numpy(), axis=-1, bitorder="little")


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_u8_bits_equal_torch_compare(oracle_lib, dtype):
    gen = torch.Generator().manual_seed(36)
    for rows, k in ((1, 1), (3, 7), (4, 8), (5, 9), (2, 40), (3, 72), (6, 100), (2, 256)):
        x = synth.inject_edges(torch.randn((rows, k), generator=gen).to(dtype), rows + k, max(1, rows * k // 5))
        got = _unpack(oracle_lib.pack_rows_u8(x), k)
        assert got.shape == (rows, (k + 7) // 8 * 8)
        assert np.array_equal(got[:, :k], (x >= 0).numpy())
        assert not got[:, k:].any()                       # bits past k are 0
    for shape in ((2, 40, 3, 5), (1, 72, 4, 4), (2, 5, 2, 3)):
        x = synth.inject_edges(torch.randn(shape, generator=gen).to(dtype), sum(shape), 20)
        c = shape[1]
        got = _unpack(oracle_lib.pack_nchw_u8(x), c)
        assert np.array_equal(got[..., :c], (x >= 0).permute(0, 2, 3, 1).numpy())
        assert not got[..., c:].any()
    w = synth.inject_edges(torch.randn((4, 40, 3, 2), generator=gen).to(dtype), 3, 30)
    got = _unpack(oracle_lib.pack_conv_weight_u8(w), 40)
    assert np.array_equal(got[..., :40], (w >= 0).permute(0, 2, 3, 1).numpy())


def test_u8_bytes_lead_the_little_endian_words(oracle_lib):
    """A row's bytes are the first ceil(k/8) bytes of its 32-bit words read in little-endian
    order (the remaining bytes of the last word are 0)."""
    gen = torch.Generator().manual_seed(37)
    for rows, k in ((3, 32), (2, 40), (4, 72), (1, 100), (5, 8), (2, 1000)):
        x = torch.randn((rows, k), generator=gen)
        words = oracle_lib.pack_rows(x).numpy().astype("<u4")
        as_bytes = words.view(np.uint8).reshape(rows, -1)
        nb = (k + 7) // 8
        assert np.array_equal(oracle_lib.pack_rows_u8(x).numpy(), as_bytes[:, :nb])
        assert not as_bytes[:, nb:].any()
    xn = torch.randn((2, 40, 3, 3), generator=gen)
    wn = oracle_lib.pack_nchw(xn).numpy().astype("<u4").view(np.uint8).reshape(2, 3, 3, -1)
    assert np.array_equal(oracle_lib.pack_nchw_u8(xn).numpy(), wn[..., :5])
