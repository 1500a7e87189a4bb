"""GPU parity of the activation prologue (the layers' set_activation) against the oracle.

Shifted sign+pack (x + bias_a >= 0, bias per input feature / one per layer for the linear
layer, per channel for the conv) must match the oracle's words bit for bit, edge values
included. The lazy scale factor * mean|x| is a double sum in a different order from the
oracle's sequential one: for n non-negative terms any order is within (n - 1) * 2^-53
relative of the exact sum, so the two agree within (2n + 4) * 2^-53 relative (the 4 covers
the division by n and the product with the factor on both sides).
"""
import math

import numpy as np
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


@pytest.fixture(scope="module")
def orc(oracle_lib):
    return oracle_lib


def _say(msg):
    print(msg, flush=True)


def _rows_case(rows, k, xdt, bdt, seed, percol=True):
    g = torch.Generator().manual_seed(seed)
    x = synth.inject_edges(torch.randn((rows, k), generator=g).to(DT[xdt]), seed, max(1, rows * k // 25))
    r0 = rows // 2
    n = k if percol else 1
    bias = synth.make_shift(n, bdt, seed + 1, axis_values=lambda i: float(x[r0, i]))
    return x, bias


@pytest.mark.parametrize("xdt", DTS)
@pytest.mark.parametrize("bdt", DTS)
def test_pack_rows_shift_bit_exact(bnn, orc, xdt, bdt):
    # k/32 = 1, 3, 32 (half a 64-word column chunk), 128, 160 (ragged last chunk)
    for rows, k in [(1, 32), (3, 96), (17, 1024), (6, 4096), (333, 5120)]:
        for percol in (True, False):
            x, bias = _rows_case(rows, k, xdt, bdt, rows * 13 + k, percol)
            _say(f"pack_rows_shift x {xdt} bias {bdt} {rows}x{k} percol={percol}")
            got = bnn.pack_sign_shift(x.to(DEV), bias.to(DEV)).cpu()
            assert torch.equal(got, orc.pack_rows_shift(x, bias)), (rows, k, percol)


@pytest.mark.parametrize("xdt", DTS)
@pytest.mark.parametrize("bdt", DTS)
def test_pack_nchw_shift_bit_exact(bnn, orc, xdt, bdt):
    # pixel counts that take the 16-byte vector path and ones that do not
    for shape in [(1, 32, 1, 1), (2, 64, 5, 3), (3, 96, 7, 9), (2, 256, 14, 14), (1, 128, 28, 28),
                  (2, 32, 4, 4), (3, 40, 4, 8), (2, 300, 2, 8), (5, 8, 8, 8)]:
        seed = sum(shape) * 3 + len(xdt) + 7 * len(bdt)
        g = torch.Generator().manual_seed(seed)
        x = synth.inject_edges(torch.randn(shape, generator=g).to(DT[xdt]), seed, max(1, math.prod(shape) // 25))
        bias = synth.make_shift(shape[1], bdt, seed + 1, axis_values=lambda c: float(x[0, c, 0, 0]))
        _say(f"pack_nchw_shift x {xdt} bias {bdt} {shape}")
        got = bnn.pack_sign_nchw_shift(x.to(DEV), bias.to(DEV)).cpu()
        assert torch.equal(got, orc.pack_nchw_shift(x, bias)), shape


def test_zero_shift_equals_plain_pack(bnn):
    g = torch.Generator().manual_seed(31)
    x = synth.inject_edges(torch.randn((64, 512), generator=g).to(torch.float16), 31, 200).to(DEV)
    for z in (torch.zeros(512, dtype=torch.float32), torch.zeros(1, dtype=torch.float16),
              torch.full((1,), -0.0, dtype=torch.bfloat16)):
        assert torch.equal(bnn.pack_sign_shift(x, z.to(DEV)), bnn.pack_sign(x))
    xc = synth.inject_edges(torch.randn((2, 64, 9, 7), generator=g), 32, 100).to(DEV)
    assert torch.equal(bnn.pack_sign_nchw_shift(xc, torch.zeros(64, device=DEV)), bnn.pack_sign_nchw(xc))


@pytest.mark.parametrize("name,bdt", [("linear_2048x4096x4096_f16", "f16"),
                                      ("linear_16384x8192x8192_bf16", "f32"),
                                      ("conv_resnet18_s3_f32", "f32"),
                                      ("conv_down_s2_f16", "f16")])
def test_shift_pack_workloads(bnn, orc, name, bdt):
    wl = synth.WORKLOADS[name]
    x, _, _, _ = synth.make_inputs(wl, draw_weight=False)
    _say(f"shift pack workload {name} bias {bdt}")
    if wl.kind == "linear":
        bias = synth.make_shift(wl.k, bdt, wl.seed + 50, axis_values=lambda i: float(x[1, i]))
        got = bnn.pack_sign_shift(x.to(DEV), bias.to(DEV)).cpu()
        assert torch.equal(got, orc.pack_rows_shift(x, bias))
    else:
        bias = synth.make_shift(wl.c, bdt, wl.seed + 50, axis_values=lambda c: float(x[0, c, 3, 3]))
        got = bnn.pack_sign_nchw_shift(x.to(DEV), bias.to(DEV)).cpu()
        assert torch.equal(got, orc.pack_nchw_shift(x, bias))


def _mean_tol(n):
    return (2 * n + 4) * 2.0 ** -53


@pytest.mark.parametrize("dt", DTS)
def test_abs_mean_small_and_ragged(bnn, orc, dt):
    g = torch.Generator().manual_seed(41)
    # counts around the vector width (4 or 8 elements), the 2048-element workgroup share and
    # the 1024-workgroup cap
    for n in [1, 3, 7, 8, 9, 1001, 2048, 2049, 65537, 3 * 1024 * 2048 + 5]:
        x = (0.1 + torch.randn(n, generator=g)).to(DT[dt])
        for factor in (2.0, 4.0):
            got = float(bnn.abs_mean_scale(x.to(DEV), factor).cpu())
            want = orc.abs_mean_scale(x, factor)
            assert abs(got - want) <= _mean_tol(n) * abs(want), (n, factor, got, want)


def test_abs_mean_closed_forms_and_specials(bnn):
    n = 1000
    ints = torch.arange(n, dtype=torch.float32).to(DEV)                 # sum n(n-1)/2, exact in double
    assert float(bnn.abs_mean_scale(ints, 2.0).cpu()) == n - 1
    assert float(bnn.abs_mean_scale(-ints, 4.0).cpu()) == 2 * (n - 1)
    alt = torch.tensor([1.0, -1.0] * 4096, dtype=torch.bfloat16, device=DEV)
    assert float(bnn.abs_mean_scale(alt, 2.0).cpu()) == 2.0
    z = torch.tensor([-0.0, 0.0] * 9, dtype=torch.float16, device=DEV)
    assert float(bnn.abs_mean_scale(z, 2.0).cpu()) == 0.0
    for dt in DTS:
        ev = synth.edge_values(dt)                                        # holds NaN
        x = torch.cat([torch.ones(37, dtype=DT[dt]), ev]).to(DEV)
        assert math.isnan(float(bnn.abs_mean_scale(x, 2.0).cpu()))
        inf = torch.tensor([1.0, float("-inf"), 2.0], dtype=DT[dt], device=DEV)
        assert float(bnn.abs_mean_scale(inf, 2.0).cpu()) == float("inf")
        # subnormals are summed at their value, not flushed
        sub = ev[5:6].repeat(64).to(DEV)                                 # +smallest subnormal
        want = float(ev[5].double()) * 2.0
        assert float(bnn.abs_mean_scale(sub, 2.0).cpu()) == want


@pytest.mark.parametrize("name", ["linear_16384x8192x8192_bf16", "conv_down_s2_f16"])
def test_abs_mean_workloads_and_determinism(bnn, orc, name):
    wl = synth.WORKLOADS[name]
    x, _, _, _ = synth.make_inputs(wl, draw_weight=False)
    _say(f"abs mean workload {name}")
    xd = x.to(DEV)
    a = bnn.abs_mean_scale(xd, 2.0)
    b = bnn.abs_mean_scale(xd, 2.0)
    got = float(a.cpu())
    want = orc.abs_mean_scale(x, 2.0)
    assert abs(got - want) <= _mean_tol(x.numel()) * abs(want), (got, want)
    assert torch.equal(a, b)


def test_layer_forward_with_prologue(bnn, orc):
    """set_activation then the binary forward: shifted pack, then bnn_gemm / bnn_conv2d on the
    packed words; the oracle side takes the signs from its own shifted pack."""
    g = torch.Generator().manual_seed(51)
    m, n, k = 300, 200, 1024
    x = torch.randn((m, k), generator=g).to(torch.float16)
    w = torch.randn((n, k), generator=g)
    bias = synth.make_shift(k, "f16", 52, axis_values=lambda i: float(x[0, i]))
    words = orc.pack_rows_shift(x, bias)
    signs = ((words.numpy().astype(np.uint32).astype(np.int64)[..., None] >> np.arange(32)) & 1)
    xs = torch.from_numpy(signs.reshape(m, k).astype(np.float32) * 2 - 1)
    want = orc.linear_acc(xs, w)
    xp = bnn.pack_sign_shift(x.to(DEV), bias.to(DEV))
    wp = bnn.w_pack(w.to(DEV))
    for path in ("xor", "mfma", "mfma_fp4"):
        got = bnn.gemm(xp, wp, 1.0, 1.0, path=path, k=k, out_dtype=torch.int32).cpu()
        assert torch.equal(got, want), path
    # conv: per-channel shift, 3x3 s1 p1
    xc = torch.randn((2, 64, 9, 7), generator=g)
    wc = torch.randn((40, 64, 3, 3), generator=g)
    bc = synth.make_shift(64, "f32", 53, axis_values=lambda c: float(xc[1, c, 4, 4]))
    wordsc = orc.pack_nchw_shift(xc, bc)                                  # [b, h, w, c/32]
    sc = ((wordsc.numpy().astype(np.uint32).astype(np.int64)[..., None] >> np.arange(32)) & 1)
    xsc = torch.from_numpy(sc.reshape(2, 9, 7, 64).transpose(0, 3, 1, 2).astype(np.float32) * 2 - 1)
    wantc = orc.conv2d_acc(xsc.contiguous(), wc, 1, 1, 1)
    xpc = bnn.pack_sign_nchw_shift(xc.to(DEV), bc.to(DEV))
    wpc = bnn.w_pack(wc.to(DEV))
    for path in ("xor", "mfma", "mfma_fp4"):
        got = bnn.conv2d(xpc, wpc, 1.0, 1.0, 3, 1, 1, 1, path=path, out_dtype=torch.int32).cpu()
        assert torch.equal(got, wantc), path
