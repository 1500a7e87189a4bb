"""GPU parity of the one-pass prologue (bnn_pack_sign_shift_abs_mean and its NCHW form): the
shifted sign+pack and the lazy scale factor * mean|x| of the layers' set_activation from one
read of x.

Bars. The words must equal the oracle's shifted pack bit for bit (and the separate entry point's
words). The scale is a double sum in an order of its own: any order of n non-negative terms is
within (n - 1) * 2^-53 relative of the exact sum, so it agrees with the oracle's sequential sum
within (2n + 4) * 2^-53 relative (the 4 covers the division by n and the factor on both sides);
it is bit-identical from run to run, and the closed forms are met exactly.
"""
import math

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
DTS = ["f32", "f16", "bf16"]


@pytest.fixture(scope="module")
def bnn():
    import convolution_bnn_pack_amd as m
    return m


def _tol(n):
    return (2 * n + 4) * 2.0 ** -53


def _say(msg):
    print(msg, flush=True)


def _scale_ok(got, want, n):
    if math.isnan(want):
        return math.isnan(got)
    if math.isinf(want):
        return got == want
    return abs(got - want) <= _tol(n) * abs(want)


def _finite(x):
    return torch.where(x.float().isfinite(), x, torch.zeros((), dtype=x.dtype))


@pytest.mark.parametrize("xdt", DTS)
@pytest.mark.parametrize("bdt", ["f32", "bf16"])
def test_rows(bnn, oracle_lib, xdt, bdt):
    # whole words (one kernel: 1, 3, 32, 160 words per row, several row groups) and row lengths
    # that are not (the two passes)
    for rows, k in [(1, 32), (3, 96), (17, 1024), (333, 5120), (2, 33), (9, 100), (5, 4097)]:
        for percol in (True, False):
            seed = rows * 7 + k + (3 if percol else 0)
            g = torch.Generator().manual_seed(seed)
            x = synth.inject_edges(torch.randn((rows, k), generator=g).to(DT[xdt]), seed, max(1, rows * k // 25))
            bias = synth.make_shift(k if percol else 1, bdt, seed + 1, axis_values=lambda i: float(x[rows // 2, i]))
            _say(f"one-pass rows x {xdt} bias {bdt} {rows}x{k} percol={percol}")
            bd = bias.to(DEV)
            # IEEE edge values in x (the scale then NaN or inf), and the same x made finite
            for xx in (x, _finite(x)):
                xd = xx.to(DEV)
                words, scale = bnn.pack_sign_shift_abs_mean(xd, bd, 2.0)
                assert torch.equal(words.cpu(), oracle_lib.pack_rows_shift(xx, bias)), (rows, k)
                assert torch.equal(words, bnn.pack_sign_shift(xd, bd))
                want = oracle_lib.abs_mean_scale(xx, 2.0)
                got = float(scale.cpu())
                assert _scale_ok(got, want, xx.numel()), (rows, k, got, want)
                _, again = bnn.pack_sign_shift_abs_mean(xd, bd, 2.0)
                assert torch.equal(scale, again) or (math.isnan(got) and math.isnan(float(again.cpu())))


@pytest.mark.parametrize("xdt", DTS)
def test_nchw(bnn, oracle_lib, xdt):
    # planes that take the one kernel (h*w a multiple of 4 / 8) and planes that do not
    for shape in [(1, 32, 4, 4), (3, 40, 4, 8), (2, 300, 2, 8), (2, 256, 14, 14), (5, 64, 3, 5),
                  (2, 96, 7, 9)]:
        seed = sum(shape) * 5 + len(xdt)
        g = torch.Generator().manual_seed(seed)
        x = synth.inject_edges(torch.randn(shape, generator=g).to(DT[xdt]), seed, max(1, math.prod(shape) // 25))
        bias = synth.make_shift(shape[1], "f16", seed + 1, axis_values=lambda c: float(x[0, c, 0, 0]))
        _say(f"one-pass nchw x {xdt} {shape}")
        bd = bias.to(DEV)
        for xx in (x, _finite(x)):
            words, scale = bnn.pack_sign_nchw_shift_abs_mean(xx.to(DEV), bd, 4.0)
            assert torch.equal(words.cpu(), oracle_lib.pack_nchw_shift(xx, bias)), shape
            want = oracle_lib.abs_mean_scale(xx, 4.0)
            assert _scale_ok(float(scale.cpu()), want, xx.numel()), shape


def test_closed_forms_and_specials(bnn):
    n = 4096
    ints = torch.arange(n, dtype=torch.float32).view(4, 1024).to(DEV)   # sum n(n-1)/2, exact
    zero = torch.zeros(1, device=DEV)
    _, s = bnn.pack_sign_shift_abs_mean(ints, zero, 2.0)
    assert float(s.cpu()) == n - 1
    alt = torch.tensor([1.0, -1.0] * 4096, dtype=torch.bfloat16).view(2, 16, 16, 16).to(DEV)
    _, s = bnn.pack_sign_nchw_shift_abs_mean(alt, torch.zeros(16, device=DEV), 2.0)
    assert float(s.cpu()) == 2.0
    for dt in DTS:
        x = torch.ones((3, 64), dtype=DT[dt])
        x[1, 5] = float("nan")
        _, s = bnn.pack_sign_shift_abs_mean(x.to(DEV), zero, 2.0)
        assert math.isnan(float(s.cpu()))
        x[1, 5] = float("-inf")
        _, s = bnn.pack_sign_shift_abs_mean(x.to(DEV), zero, 2.0)
        assert float(s.cpu()) == float("inf")
        xc = torch.ones((2, 32, 4, 4), dtype=DT[dt])
        xc[1, 7, 2, 3] = float("nan")
        _, s = bnn.pack_sign_nchw_shift_abs_mean(xc.to(DEV), torch.zeros(32, device=DEV), 2.0)
        assert math.isnan(float(s.cpu()))


def test_errors(bnn):
    x = torch.zeros((0, 64), dtype=torch.float16, device=DEV)
    with pytest.raises(AssertionError):
        bnn.pack_sign_shift_abs_mean(x, torch.zeros(1, device=DEV), 2.0)   # mean of no elements


@pytest.mark.parametrize("name,bdt", [("linear_16384x8192x8192_bf16", "f32"), ("conv_down_s2_f16", "f16")])
def test_workloads(bnn, oracle_lib, name, bdt):
    wl = synth.WORKLOADS[name]
    x, _, _, _ = synth.make_inputs(wl, draw_weight=False)
    _say(f"one-pass prologue workload {name}")
    xd = x.to(DEV)
    if wl.kind == "linear":
        bias = synth.make_shift(wl.k, bdt, wl.seed + 50, axis_values=lambda i: float(x[1, i]))
        words, scale = bnn.pack_sign_shift_abs_mean(xd, bias.to(DEV), 2.0)
        assert torch.equal(words.cpu(), oracle_lib.pack_rows_shift(x, bias))
    else:
        bias = synth.make_shift(wl.c, bdt, wl.seed + 50, axis_values=lambda c: float(x[0, c, 3, 3]))
        words, scale = bnn.pack_sign_nchw_shift_abs_mean(xd, bias.to(DEV), 2.0)
        assert torch.equal(words.cpu(), oracle_lib.pack_nchw_shift(x, bias))
    want = oracle_lib.abs_mean_scale(x, 2.0)
    assert abs(float(scale.cpu()) - want) <= _tol(x.numel()) * abs(want)
