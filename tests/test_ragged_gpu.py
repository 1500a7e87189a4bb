"""GPU parity for reduction lengths that are not whole words (K % 32 != 0 for linear layers,
C % 32 != 0 for convs): packed words bit-exact against the oracle (the last word holds the
remaining signs and zeros above them), int32 accumulators bit-exact on all three paths."""
import math

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
EXPLICIT = ["xor", "mfma", "mfma_fp4"]


@pytest.fixture(scope="module")
def bnn():
    import convolution_bnn_pack_amd as m
    return m


@pytest.fixture(scope="module")
def orc(oracle_lib):
    return oracle_lib


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("xdt", ["f32", "f16", "bf16"])
def test_pack_rows_ragged(bnn, orc, xdt):
    g = torch.Generator().manual_seed(71)
    for rows, k in [(1, 1), (3, 5), (7, 31), (5, 33), (9, 63), (4, 100), (130, 1000), (2, 4097)]:
        x = synth.inject_edges(torch.randn((rows, k), generator=g).to(DT[xdt]), rows + k, max(1, rows * k // 15))
        _say(f"ragged pack {xdt} {rows}x{k}")
        got = bnn.pack_sign(x.to(DEV)).cpu()
        assert got.shape == (rows, (k + 31) // 32)
        assert torch.equal(got, orc.pack_rows(x)), (rows, k)
        for bdt in ("f32", "f16"):
            for nb in (1, k):
                bias = synth.make_shift(nb, bdt, rows * k + nb, axis_values=lambda i: float(x[0, i]))
                got = bnn.pack_sign_shift(x.to(DEV), bias.to(DEV)).cpu()
                assert torch.equal(got, orc.pack_rows_shift(x, bias)), (rows, k, bdt, nb)


def test_pack_rows_unaligned_whole_words(bnn, orc):
    """Whole-word rows whose tensor is not 16-byte aligned take the element-wise kernel."""
    g = torch.Generator().manual_seed(72)
    for dt in (torch.float32, torch.float16):
        big = torch.randn(1 + 6 * 64, generator=g).to(dt).to(DEV)
        x = big[1:].view(6, 64)                                          # offset by one element
        assert x.data_ptr() % 16 != 0
        got = bnn.pack_sign(x).cpu()
        assert torch.equal(got, orc.pack_rows(x.cpu().contiguous()))


@pytest.mark.parametrize("xdt", ["f32", "f16", "bf16"])
def test_pack_nchw_and_weights_ragged(bnn, orc, xdt):
    g = torch.Generator().manual_seed(73)
    for c in [1, 3, 17, 31, 33, 40, 100]:
        for (h, w) in [(5, 3), (4, 4), (7, 8)]:
            x = synth.inject_edges(torch.randn((2, c, h, w), generator=g).to(DT[xdt]), c * h + w, max(1, c * h * w // 10))
            _say(f"ragged nchw {xdt} c={c} {h}x{w}")
            got = bnn.pack_sign_nchw(x.to(DEV)).cpu()
            assert got.shape == (2, h, w, (c + 31) // 32)
            assert torch.equal(got, orc.pack_nchw(x)), (c, h, w)
            bias = synth.make_shift(c, "f32", c + h, axis_values=lambda i: float(x[1, i, 0, 0]))
            got = bnn.pack_sign_nchw_shift(x.to(DEV), bias.to(DEV)).cpu()
            assert torch.equal(got, orc.pack_nchw_shift(x, bias)), (c, h, w)
        wt = torch.randn((9, c, 3, 3), generator=g).to(DT[xdt])
        assert torch.equal(bnn.w_pack(wt.to(DEV)).cpu(), orc.pack_conv_weight(wt)), c
        wl = torch.randn((9, c), generator=g).to(DT[xdt])
        assert torch.equal(bnn.w_pack(wl.to(DEV)).cpu(), orc.pack_rows(wl)), c


def test_linear_ragged_k_all_paths(bnn, orc):
    g = torch.Generator().manual_seed(74)
    for m, n, k in [(1, 1, 1), (5, 3, 7), (33, 17, 31), (64, 64, 33), (70, 130, 95), (200, 100, 100),
                    (129, 257, 257), (300, 70, 1000), (64, 96, 4000)]:
        x = torch.randn((m, k), generator=g).to(torch.float16)
        w = torch.randn((n, k), generator=g)
        want = orc.linear_acc(x, w)
        wp = bnn.w_pack(w.to(DEV))
        xd = x.to(DEV)
        xp = bnn.pack_sign(xd)
        _say(f"ragged linear {m}x{n}x{k}")
        for path in EXPLICIT + ["auto"]:
            got = bnn.gemm(xd, wp, 1.0, 1.0, path=path, out_dtype=torch.int32).cpu()
            assert torch.equal(got, want), (m, n, k, path, "float input")
            got = bnn.gemm(xp, wp, 1.0, 1.0, path=path, k=k, out_dtype=torch.int32).cpu()
            assert torch.equal(got, want), (m, n, k, path, "packed input")
        # scaled f32 output: (float)acc * (float)(sa*sw), within 1e-6 relative of the double product
        sa, sw = 0.37, 0.81
        y = bnn.gemm(xd, wp, sa, sw, out_dtype=torch.float32).cpu().double()
        ref = orc.scale(want, sa, sw)
        assert torch.all((y - ref).abs() <= 1e-6 * ref.abs())


def test_conv_ragged_c_all_paths(bnn, orc):
    g = torch.Generator().manual_seed(75)
    cases = [(2, 1, 9, 7, 5, 3, 1, 1, 1), (1, 3, 8, 8, 40, 3, 2, 1, 1), (2, 17, 11, 6, 33, 5, 1, 2, 1),
             (1, 33, 7, 9, 64, 3, 1, 2, 2), (3, 40, 14, 14, 70, 3, 1, 1, 1), (1, 100, 6, 5, 20, 1, 1, 0, 1),
             (2, 65, 10, 10, 129, 2, 3, 3, 2)]
    for (b, c, h, wd, o, ks, s, p, d) in cases:
        x = torch.randn((b, c, h, wd), generator=g).to(torch.float16)
        w = torch.randn((o, c, ks, ks), generator=g)
        want = orc.conv2d_acc(x, w, s, p, d)
        wp = bnn.w_pack(w.to(DEV))
        xd = x.to(DEV)
        xp = bnn.pack_sign_nchw(xd)
        _say(f"ragged conv b={b} c={c} {h}x{wd} o={o} k={ks} s={s} p={p} d={d}")
        for path in EXPLICIT + ["auto"]:
            got = bnn.conv2d(xd, wp, 1.0, 1.0, ks, s, p, d, path=path, out_dtype=torch.int32).cpu()
            assert torch.equal(got, want), (c, path, "float input")
            got = bnn.conv2d(xp, wp, 1.0, 1.0, ks, s, p, d, path=path, out_dtype=torch.int32,
                             channels=c).cpu()
            assert torch.equal(got, want), (c, path, "packed input")


def test_conv_ragged_many_tiles_and_kvalid(bnn, orc):
    """A ragged-C conv with more fp4 tiles than the device holds at once (whole-word channel
    counts would stream them through persistent workgroups), checked on sampled images, and
    the closed form x = +1, W = +1 -> acc = C * (valid taps) at every pixel."""
    g = torch.Generator().manual_seed(76)
    b, c, h, w, o = 64, 40, 28, 28, 256
    x = torch.randn((b, c, h, w), generator=g).to(torch.float16)
    wt = torch.randn((o, c, 3, 3), generator=g)
    wp = bnn.w_pack(wt.to(DEV))
    _say("ragged conv 64x40x28x28 -> 256")
    got = bnn.conv2d(x.to(DEV), wp, 1.0, 1.0, 3, 1, 1, 1, path="mfma_fp4", out_dtype=torch.int32).cpu()
    imgs = [0, 31, 63]
    assert torch.equal(got[imgs], orc.conv2d_acc(x, wt, 1, 1, 1, images=imgs))
    ones = torch.ones((2, c, 9, 9))
    wp1 = bnn.w_pack(torch.ones((5, c, 3, 3), device=DEV))
    kv = orc.conv2d_kvalid(c, 9, 9, 3, 1, 1, 1)
    for path in EXPLICIT:
        acc = bnn.conv2d(ones.to(DEV), wp1, 1.0, 1.0, 3, 1, 1, 1, path=path, out_dtype=torch.int32).cpu()
        assert torch.equal(acc, kv.expand(2, 5, 9, 9)), path
