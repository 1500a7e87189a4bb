"""GPU parity of the straight-through conv backward (BinaryConv2dForward.backward on the
qconv/binary/cutlass/layer page) against the oracle: grad_input with its clip mask,
grad_scale_a, grad_weight and its int8 codes.

Bars. With output gradients that are multiples of 1/8 and dyadic scales every partial sum is
exact in fp32, so grad_input, grad_weight and grad_scale_a must equal the oracle's bit for bit
(grad_scale_a: both sides sum exact terms in double and divide once by the same square root).
With N(0, 1) gradients each element is a sum of exact products, accumulated in fp32 in two
stages (over output channels, then over at most kh*kw taps for grad_input; over output pixels
for grad_weight), so it is within (terms + 2) * 2^-24 * (scale * sum of |terms|) of the exact
value; masked elements are exactly 0. The sums of |terms| come from the oracle itself, run on
|grad_out| with all-ones signs.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
HALF = [torch.float16, torch.bfloat16]
U = 2.0 ** -24

# (batch, c, h, w, o, (kh, kw), stride, padding, dilation): n*Ho*Wo and c*kh*kw multiples of 8
GEOMS = [
    (2, 8, 6, 6, 16, (3, 3), 1, 1, 1),
    (2, 16, 7, 5, 8, (3, 3), 2, 1, 1),
    (8, 24, 9, 9, 40, (3, 3), 1, 2, 2),
    (2, 40, 8, 9, 24, (1, 1), 1, 0, 1),
    (4, 8, 10, 7, 136, (2, 5), (1, 2), (1, 2), (2, 1)),
    (2, 32, 6, 8, 9, (5, 5), 1, 2, 1),
    (8, 72, 11, 13, 200, (3, 3), (2, 1), (0, 1), (1, 2)),
]


@pytest.fixture(scope="module")
def bnn():
    import convolution_bnn_pack_amd as m
    return m


def _pair(v):
    return (v, v) if isinstance(v, int) else v


def _out_hw(h, w, k, s, p, d):
    (kh, kw), (sh, sw), (ph, pw), (dh, dw) = k, _pair(s), _pair(p), _pair(d)
    return (h + 2 * ph - dh * (kh - 1) - 1) // sh + 1, (w + 2 * pw - dw * (kw - 1) - 1) // sw + 1


def _inputs(seed, geom, dt, dyadic):
    b, c, h, w, o, k, s, p, d = geom
    ho, wo = _out_hw(h, w, k, s, p, d)
    gen = torch.Generator().manual_seed(seed)
    if dyadic:
        g = torch.randint(-16, 17, (b, o, ho, wo), generator=gen).float() / 8
    else:
        g = torch.randn((b, o, ho, wo), generator=gen)
    wt = torch.randn((o, c) + tuple(k), generator=gen)
    x = 0.8 * torch.randn((b, c, h, w), generator=gen)
    wt.view(-1)[::13] = 0.0
    x.view(-1)[::17] = 0.0
    x.view(-1)[5::19] = -0.0
    return g.to(dt), wt.to(dt), x.to(dt)


def _gpu(bnn, g, wt, x, geom, sa, sw, codes=False):
    _, _, _, _, _, k, s, p, d = geom
    gi, gsa = bnn.conv2d_grad_input(g.to(DEV), wt.to(DEV), x.to(DEV), sa, sw, s, p, d)
    res = bnn.conv2d_grad_weight(g.to(DEV), x.to(DEV), k, sa, s, p, d, codes=codes)
    torch.cuda.synchronize()
    if codes:
        gw, q, amax = res
        return gi.cpu(), float(gsa.cpu()), gw.cpu(), q.cpu(), float(amax.cpu())
    return gi.cpu(), float(gsa.cpu()), res.cpu()


@pytest.mark.parametrize("dt", HALF)
@pytest.mark.parametrize("geom", GEOMS)
def test_exact_sums(bnn, oracle_lib, dt, geom):
    g, wt, x = _inputs(hash(geom) % 1000, geom, dt, dyadic=True)
    sa, sw = 0.75, 0.5
    _, _, _, _, _, k, s, p, d = geom
    gi_ref, gsa_ref, gw_ref = oracle_lib.conv2d_grad(g, wt, x, s, p, d, sa, sw)
    gi, gsa, gw = _gpu(bnn, g, wt, x, geom, sa, sw)
    assert torch.equal(gi.double(), gi_ref), geom
    assert torch.equal(gw.double(), gw_ref), geom
    assert gsa == gsa_ref, (geom, gsa, gsa_ref)


@pytest.mark.parametrize("dt", HALF)
@pytest.mark.parametrize("geom", GEOMS[:3] + GEOMS[4:5])
def test_randn_within_bound(bnn, oracle_lib, dt, geom):
    g, wt, x = _inputs(hash(geom) % 1000 + 7, geom, dt, dyadic=False)
    sa, sw = 0.3, 0.7
    b, c, h, w, o, k, s, p, d = geom
    ho, wo = _out_hw(h, w, k, s, p, d)
    gi_ref, gsa_ref, gw_ref = oracle_lib.conv2d_grad(g, wt, x, s, p, d, sa, sw)
    gi, gsa, gw = _gpu(bnn, g, wt, x, geom, sa, sw)
    # sums of |terms|: the oracle on |g| with every sign +1 (weights and inputs of ones, x = 0 so
    # that no element is masked)
    ones_w = torch.ones_like(wt)
    ones_x = torch.ones_like(x)
    abs_in, _, _ = oracle_lib.conv2d_grad(g.abs(), ones_w, torch.zeros_like(x), s, p, d, sa, sw)
    _, _, abs_w = oracle_lib.conv2d_grad(g.abs(), ones_w, ones_x, s, p, d, sa, sw)
    t_in = o * k[0] * k[1] + 2
    t_w = b * ho * wo + 2
    mask = gi_ref == 0
    assert bool((gi.double()[mask & (gi_ref == 0)] == 0).all())
    err_in = (gi.double() - gi_ref).abs()
    assert bool((err_in <= t_in * U * abs_in + U * gi_ref.abs()).all()), geom
    err_w = (gw.double() - gw_ref).abs()
    assert bool((err_w <= t_w * U * abs_w + U * gw_ref.abs()).all()), geom
    bound_sa = float((t_in * U * abs_in).sum()) / (b * c * h * w) ** 0.5 + 1e-12
    assert abs(gsa - gsa_ref) <= bound_sa + 1e-9 * abs(gsa_ref), (gsa, gsa_ref, bound_sa)


@pytest.mark.parametrize("dt", HALF)
def test_grad_weight_codes(bnn, oracle_lib, dt):
    for geom in GEOMS[:4]:
        g, wt, x = _inputs(hash(geom) % 1000 + 3, geom, dt, dyadic=True)
        _, _, _, _, _, k, s, p, d = geom
        _, _, gw_ref = oracle_lib.conv2d_grad(g, wt, x, s, p, d, 0.5, 1.0)
        want_q, want_amax = oracle_lib.quant_grad_i8(gw_ref)
        _, _, gw, q, amax = _gpu(bnn, g, wt, x, geom, 0.5, 1.0, codes=True)
        assert torch.equal(gw.double(), gw_ref)
        assert amax == want_amax
        assert torch.equal(q, want_q.view(q.shape)), geom


def test_clip_boundary_and_nan(bnn, oracle_lib):
    """x exactly at +-scale_a keeps its gradient, the next representable value outward drops
    it; a NaN input keeps it (mask 1) and makes grad_scale_a NaN."""
    geom = (2, 8, 6, 6, 16, (3, 3), 1, 1, 1)
    g, wt, x = _inputs(5, geom, torch.float16, dyadic=True)
    sa = 0.5
    x = x.clone()
    x[0, 0, 0, :4] = torch.tensor([0.5, -0.5, 0.50048828125, -0.50048828125], dtype=torch.float16)
    gi_ref, gsa_ref, gw_ref = oracle_lib.conv2d_grad(g, wt, x, 1, 1, 1, sa, 0.25)
    gi, gsa, gw = _gpu(bnn, g, wt, x, geom, sa, 0.25)
    assert torch.equal(gi.double(), gi_ref) and gsa == gsa_ref
    assert gi[0, 0, 0, 2] == 0 and gi[0, 0, 0, 3] == 0
    x[1, 3, 2, 2] = float("nan")
    gi_ref, gsa_ref, _ = oracle_lib.conv2d_grad(g, wt, x, 1, 1, 1, sa, 0.25)
    gi, gsa, _ = _gpu(bnn, g, wt, x, geom, sa, 0.25)
    assert torch.equal(gi.double(), gi_ref)
    assert gsa != gsa and gsa_ref != gsa_ref


def test_argument_errors(bnn):
    g = torch.zeros((2, 8, 5, 5), dtype=torch.float16, device=DEV)   # n*Ho*Wo = 50: not % 8
    wt = torch.zeros((8, 8, 3, 3), dtype=torch.float16, device=DEV)
    x = torch.zeros((2, 8, 5, 5), dtype=torch.float16, device=DEV)
    with pytest.raises(AssertionError):
        bnn.conv2d_grad_input(g, wt, x, 1.0, 1.0, 1, 1, 1)
    with pytest.raises(AssertionError):
        bnn.conv2d_grad_weight(g, x, 3, 1.0, 1, 1, 1)
    with pytest.raises(ValueError):                                 # grad_out of the wrong size
        bnn.conv2d_grad_input(g[:, :, :4].contiguous(), wt, x, 1.0, 1.0, 1, 1, 1)
    with pytest.raises(TypeError):
        bnn.conv2d_grad_input(g.float(), wt, x, 1.0, 1.0, 1, 1, 1)


@pytest.mark.parametrize("name,images", [("conv_resnet18_s3_f32", None), ("conv_down_s2_f16", 4),
                                         ("conv_dil2_f16", 2)])
def test_workload_shapes(bnn, oracle_lib, name, images):
    """The conv workloads' layer shapes (16-bit copies of their activations and weights, dyadic
    output gradients): the stage-3 layer on the whole batch, the two 128-image layers on their
    first images (every gradient of those images, the weight gradient summed over them)."""
    import synth
    wl = synth.WORKLOADS[name]
    x, w, _, _ = synth.make_inputs(wl)
    if images is not None:
        x = x[:images].contiguous()
    dt = torch.bfloat16
    x, w = x.to(dt), w.to(dt)
    ho, wo = _out_hw(wl.h, wl.w, (wl.ks, wl.ks), wl.stride, wl.padding, wl.dilation)
    gen = torch.Generator().manual_seed(wl.seed + 80)
    g = (torch.randint(-16, 17, (x.shape[0], wl.o, ho, wo), generator=gen).float() / 8).to(dt)
    geom = (x.shape[0], wl.c, wl.h, wl.w, wl.o, (wl.ks, wl.ks), wl.stride, wl.padding, wl.dilation)
    gi_ref, gsa_ref, gw_ref = oracle_lib.conv2d_grad(g, w, x, wl.stride, wl.padding, wl.dilation, 0.5, 0.25)
    gi, gsa, gw = _gpu(bnn, g, w, x, geom, 0.5, 0.25)
    assert torch.equal(gi.double(), gi_ref), name
    assert torch.equal(gw.double(), gw_ref), name
    assert gsa == gsa_ref


def test_grad_out_only_element_aligned(bnn, oracle_lib):
    """A grad_out that is only 2-byte aligned takes the narrow copy into the workspace (the plane
    size alone would allow 16-byte vectors)."""
    geom = (2, 16, 8, 8, 24, (3, 3), 1, 1, 1)
    g, wt, x = _inputs(11, geom, torch.float16, dyadic=True)
    _, _, _, _, _, k, s, p, d = geom
    gi_ref, gsa_ref, gw_ref = oracle_lib.conv2d_grad(g, wt, x, s, p, d, 0.5, 0.25)
    buf = torch.empty(g.numel() + 1, dtype=g.dtype, device=DEV)
    gd = buf[1:].view(g.shape)
    gd.copy_(g.to(DEV))
    assert gd.data_ptr() % 4 == 2
    gi, gsa = bnn.conv2d_grad_input(gd, wt.to(DEV), x.to(DEV), 0.5, 0.25, s, p, d)
    gw = bnn.conv2d_grad_weight(gd, x.to(DEV), k, 0.5, s, p, d)
    torch.cuda.synchronize()
    assert torch.equal(gi.cpu().double(), gi_ref) and torch.equal(gw.cpu().double(), gw_ref)
    assert float(gsa.cpu()) == gsa_ref
