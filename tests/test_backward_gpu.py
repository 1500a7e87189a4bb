"""GPU parity of the straight-through linear backward (grad_input with its clip mask,
grad_scale_a, grad_weight) against the oracle.

Bars. With output gradients that are multiples of 1/8 and dyadic scales every partial sum is
exact in fp32, so grad_input and grad_weight must equal the oracle bit for bit, and
grad_scale_a too (both sides sum exact terms in double and divide once by the same sqrt).
With N(0, 1) gradients each fp32 sum of n exact products is within n * 2^-24 * sum|terms| of
the exact one, plus one rounding for the scale; the tests check that bound per element and
that masked elements are exactly 0. Where the oracle would take too long (the full layer
sizes) whole rows are compared: grad_input rows depend on their own rows of g and x only, and
grad_weight rows on their own columns of g."""
import math

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
HALF = [torch.float16, torch.bfloat16]
U = 2.0 ** -24


@pytest.fixture(scope="module")
def bnn():
    import convolution_bnn_pack_amd as m
    return m


@pytest.fixture(scope="module")
def orc(oracle_lib):
    return oracle_lib


def _inputs(seed, m, n, k, dt, dyadic, zeros=True):
    gen = torch.Generator().manual_seed(seed)
    if dyadic:
        g = torch.randint(-16, 17, (m, n), generator=gen).float() / 8
    else:
        g = torch.randn((m, n), generator=gen)
    w = torch.randn((n, k), generator=gen)
    x = 0.8 * torch.randn((m, k), generator=gen)
    if zeros:
        w.view(-1)[::13] = 0.0
        x.view(-1)[::17] = 0.0
        x.view(-1)[5::19] = -0.0
    return g.to(dt), w.to(dt), x.to(dt)


def _run(bnn, g, w, x, sa, sw):
    gi, gsa = bnn.linear_grad_input(g.to(DEV), w.to(DEV), x.to(DEV), sa, sw)
    gw = bnn.linear_grad_weight(g.to(DEV), x.to(DEV), sa)
    torch.cuda.synchronize()
    return gi.cpu(), float(gsa.cpu()), gw.cpu()


SHAPES = [(1, 8, 8), (5, 24, 40), (128, 128, 128), (300, 200, 392), (129, 520, 264), (64, 0, 128),
          (700, 96, 1000)]


@pytest.mark.parametrize("dt", HALF)
@pytest.mark.parametrize("shape", SHAPES)
def test_exact_sums(bnn, orc, dt, shape):
    m, n, k = shape
    print(f"exact {dt} {shape}", flush=True)
    g, w, x = _inputs(m + n + k, m, n, k, dt, dyadic=True)
    sa, sw = 0.5, 0.25
    gi, gsa, gw = _run(bnn, g, w, x, sa, sw)
    ref_gi, ref_gsa = orc.linear_grad_input(g, w, x, sa, sw)
    assert torch.equal(gi.double(), ref_gi)
    assert gsa == ref_gsa
    assert torch.equal(gw.double(), orc.linear_grad_weight(g, x, sa))


@pytest.mark.parametrize("dt", HALF)
@pytest.mark.parametrize("shape", [(256, 512, 384), (77, 1024, 136), (1024, 256, 512)])
def test_randn_within_bound(bnn, orc, dt, shape):
    m, n, k = shape
    print(f"randn {dt} {shape}", flush=True)
    g, w, x = _inputs(7 * m + n, m, n, k, dt, dyadic=False)
    sa, sw = 0.9, 0.37
    gi, gsa, gw = _run(bnn, g, w, x, sa, sw)
    ref_gi, ref_gsa = orc.linear_grad_input(g, w, x, sa, sw)
    sa32, sw32 = float(torch.tensor(sa)), float(torch.tensor(sw))
    row_abs = g.double().abs().sum(1, keepdim=True)
    bound = (n + 1) * U * sw32 * row_abs + U * ref_gi.abs()
    assert bool(((gi.double() - ref_gi).abs() <= bound).all())
    masked = ref_gi == 0
    assert bool((gi[masked] == 0).all())
    s = torch.sign(x.double())
    gsa_bound = float((bound * s.abs()).sum()) / math.sqrt(m * k) + 1e-12 * float((ref_gi * s).abs().sum())
    assert abs(gsa - ref_gsa) <= gsa_bound, (gsa, ref_gsa, gsa_bound)
    ref_gw = orc.linear_grad_weight(g, x, sa)
    col_abs = g.double().abs().sum(0).unsqueeze(1)
    assert bool(((gw.double() - ref_gw).abs() <= (m + 1) * U * sa32 * col_abs + U * ref_gw.abs()).all())


@pytest.mark.parametrize("dt", HALF)
def test_edges(bnn, orc, dt):
    """The clip boundary (x == +-scale_a kept, the next value above dropped), NaN inputs (mask 1,
    grad_scale_a NaN), NaN and infinite weights, zeros."""
    print(f"edges {dt}", flush=True)
    sa = 0.5
    up = torch.nextafter(torch.tensor(0.5, dtype=dt), torch.tensor(1.0, dtype=dt)).item()
    m, n, k = 4, 16, 16
    g = (torch.arange(m * n, dtype=torch.float32).view(m, n) % 7 - 3).to(dt) / 4
    w = torch.randn((n, k), generator=torch.Generator().manual_seed(3)).to(dt)
    x = torch.full((m, k), 0.25, dtype=dt)
    x[0, :6] = torch.tensor([0.5, -0.5, up, -up, 0.0, -0.0], dtype=dt)
    gi, gsa, gw = _run(bnn, g, w, x, sa, 0.25)
    ref_gi, ref_gsa = orc.linear_grad_input(g, w, x, sa, 0.25)
    assert torch.equal(gi.double(), ref_gi) and gsa == ref_gsa
    assert torch.equal(gw.double(), orc.linear_grad_weight(g, x, sa))
    assert gi[0, 2] == 0 and gi[0, 3] == 0 and gi[0, 0] != 0
    x[1, 3] = float("nan")
    w[2, 5] = float("nan")
    w[3, 6] = float("inf")
    gi, gsa, gw = _run(bnn, g, w, x, sa, 0.25)
    ref_gi, ref_gsa = orc.linear_grad_input(g, w, x, sa, 0.25)
    assert torch.equal(gi.double().nan_to_num(7.0), ref_gi.nan_to_num(7.0))
    assert bool(torch.isnan(gi[:, 5]).all()) and math.isnan(gsa) and math.isnan(ref_gsa)
    assert torch.equal(gw.double().nan_to_num(7.0), orc.linear_grad_weight(g, x, sa).nan_to_num(7.0))


@pytest.mark.parametrize("dt,shape", [(torch.float16, (2048, 4096, 4096)),
                                      (torch.bfloat16, (16384, 8192, 8192))])
def test_full_size_sampled_rows(bnn, orc, dt, shape):
    """The linear layers' full sizes: sampled grad_input rows and grad_weight rows against the
    oracle (dyadic gradients, so bit-exact), grad_scale_a against the double sum of the
    kernel's own grad_input (a property that holds at any size)."""
    m, n, k = shape
    print(f"full {dt} {shape}", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(11)
    g = (torch.randint(-16, 17, (m, n), generator=gen, device=DEV).float() / 8).to(dt)
    w = torch.randn((n, k), generator=gen, device=DEV).to(dt)
    x = (0.8 * torch.randn((m, k), generator=gen, device=DEV)).to(dt)
    sa, sw = 0.5, 0.25
    gi, gsa = bnn.linear_grad_input(g, w, x, sa, sw)
    gw = bnn.linear_grad_weight(g, x, sa)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, m // 3, m // 2 + 5, m - 1])
    ref_rows, _ = orc.linear_grad_input(g[rows.to(DEV)].cpu(), w.cpu(), x[rows.to(DEV)].cpu(), sa, sw)
    assert torch.equal(gi[rows.to(DEV)].cpu().double(), ref_rows)
    cols = torch.tensor([0, n // 2 + 3, n - 1])
    ref_w = orc.linear_grad_weight(g[:, cols.to(DEV)].contiguous().cpu(), x.cpu(), sa)
    assert torch.equal(gw[cols.to(DEV)].cpu().double(), ref_w)
    want = float((gi.double() * torch.sign(x.double())).sum()) / math.sqrt(m * k)
    assert math.isclose(float(gsa), want, rel_tol=1e-9, abs_tol=1e-9)


def test_errors(bnn):
    g = torch.zeros((4, 12), dtype=torch.float16, device=DEV)
    w = torch.zeros((12, 16), dtype=torch.float16, device=DEV)
    x = torch.zeros((4, 16), dtype=torch.float16, device=DEV)
    with pytest.raises(AssertionError):
        bnn.linear_grad_input(g, w, x, 1.0, 1.0)            # n = 12 is not a multiple of 8
    with pytest.raises(TypeError):
        bnn.linear_grad_weight(g.float(), x.float(), 1.0)  # fp32 operands are not taken


@pytest.mark.parametrize("dt", HALF)
@pytest.mark.parametrize("shape", [(1, 8, 8), (300, 200, 392), (129, 520, 264), (0, 64, 128), (700, 96, 1000)])
def test_grad_weight_codes(bnn, orc, dt, shape):
    """int8 codes of grad_weight bit-exact against the oracle (dyadic gradients: the fp32 gradient
    is exact, so amax and every rounding decision are the same on both sides); m = 0 gives a zero
    gradient, amax 0 and zero codes."""
    m, n, k = shape
    print(f"codes {dt} {shape}", flush=True)
    g, _, x = _inputs(3 * m + n + k, m, n, k, dt, dyadic=True)
    gw, codes, amax = bnn.linear_grad_weight_i8(g.to(DEV), x.to(DEV), 0.5)
    torch.cuda.synchronize()
    ref = orc.linear_grad_weight(g, x, 0.5)
    want, want_amax = orc.quant_grad_i8(ref)
    assert torch.equal(gw.cpu().double(), ref)
    assert float(amax.cpu()) == want_amax
    assert torch.equal(codes.cpu(), want)
    if m == 0:
        assert want_amax == 0.0 and not bool(want.any())


def test_grad_weight_codes_nan(bnn, orc):
    g, _, x = _inputs(5, 64, 32, 40, torch.bfloat16, dyadic=True)
    x[3, 9] = float("nan")
    gw, codes, amax = bnn.linear_grad_weight_i8(g.to(DEV), x.to(DEV), 0.5)
    torch.cuda.synchronize()
    want, want_amax = orc.quant_grad_i8(orc.linear_grad_weight(g, x, 0.5))
    assert math.isnan(float(amax.cpu())) and math.isnan(want_amax)
    assert torch.equal(codes.cpu(), want) and not bool(want.any())


def test_grad_weight_codes_full_size(bnn, orc):
    """The 16384 x 8192 x 8192 layer: amax is the max of the kernel's own fp32 gradient, sampled
    gradient rows equal the oracle's (dyadic gradients), and the codes of those rows equal the
    oracle quantizer's with that amax; every code is the quantizer of its fp32 value."""
    m, n, k = 16384, 8192, 8192
    print(f"codes full {(m, n, k)}", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(12)
    g = (torch.randint(-16, 17, (m, n), generator=gen, device=DEV).float() / 8).to(torch.bfloat16)
    x = (0.8 * torch.randn((m, k), generator=gen, device=DEV)).to(torch.bfloat16)
    gw, codes, amax = bnn.linear_grad_weight_i8(g, x, 0.5)
    torch.cuda.synchronize()
    a = float(amax.cpu())
    assert a == float(gw.abs().max().cpu())
    cols = torch.tensor([0, 77, n - 1])
    ref = orc.linear_grad_weight(g[:, cols.to(DEV)].contiguous().cpu(), x.cpu(), 0.5)
    assert torch.equal(gw[cols.to(DEV)].cpu().double(), ref)
    assert torch.equal(codes[cols.to(DEV)].cpu(), orc.quant_i8(ref.float(), a))
    gwc = gw.cpu()
    step = torch.tensor(a, dtype=torch.float32) / 127.0
    assert torch.equal(codes.cpu(), torch.round(gwc / step).clamp(-127, 127).to(torch.int8))


@pytest.mark.parametrize("count", [4, 1000, 4096 * 1024 + 4])
def test_quant_grad_alone(bnn, orc, count):
    """The stand-alone coder on seeded fp32 gradients (with zeros) equals the oracle quantizer,
    codes and amax."""
    print(f"quant alone {count}", flush=True)
    gen = torch.Generator().manual_seed(count)
    v = 3 * torch.randn(count, generator=gen)
    v[::97] = 0.0
    codes, amax = bnn.quant_grad_i8(v.to(DEV))
    torch.cuda.synchronize()
    want, want_amax = orc.quant_grad_i8(v.double())
    assert float(amax.cpu()) == want_amax
    assert torch.equal(codes.cpu(), want)
