"""Pins of the oracle's straight-through linear backward, shared by its CPU tests and by the
planted-mistake tests (CPU only, no GPU, no HIP library).

Each pin returns True when the oracle agrees with something other than itself: torch's own
gradient routines (torch.nn.grad.conv2d_input / conv2d_weight, the routines the conv page's
backward calls, here with a 1x1 kernel), autograd of a surrogate whose derivative is the
straight-through estimator, closed forms, and the clip boundary taken bit by bit.
"""
import math

import numpy as np
import torch


def sign0(t):
    """torch.sign in float64 (0 for zeros, NaN for NaN)."""
    return torch.sign(t.double())


def mid_fp32(x, scale_a):
    """1 - small - large of the conv page's clip, with the quotient in IEEE fp32 (numpy)."""
    q = x.float().numpy() / np.float32(scale_a)
    return torch.from_numpy(1.0 - (q < -1).astype(np.float64) - (q > 1).astype(np.float64))


def _data(seed, m, n, k, dtype=torch.float32):
    gen = torch.Generator().manual_seed(seed)
    g = torch.randn((m, n), generator=gen).to(dtype)
    w = torch.randn((n, k), generator=gen).to(dtype)
    x = torch.randn((m, k), generator=gen).to(dtype)
    return g, w, x


def pin_vs_torch_grad(orc):
    """The page's steps with torch's gradient routines, 1x1 kernel, float64."""
    for seed, (m, n, k), sa, sw, dt in ((1, (5, 7, 9), 0.8, 0.3, torch.float32),
                                         (2, (16, 3, 40), 1.3, 2.0, torch.bfloat16),
                                         (3, (2, 33, 6), 0.5, 0.125, torch.float16)):
        g, w, x = _data(seed, m, n, k, dt)
        gi, gsa = orc.linear_grad_input(g, w, x, sa, sw)
        wt = (sign0(w) * float(np.float32(sw))).view(n, k, 1, 1)
        ref = torch.nn.grad.conv2d_input((m, k, 1, 1), wt, g.double().view(m, n, 1, 1)).view(m, k)
        ref = ref * mid_fp32(x, sa)
        if not torch.allclose(gi, ref, rtol=1e-12, atol=1e-12):
            return False
        want = float((ref * sign0(x)).sum() / math.sqrt(m * k))
        if not math.isclose(gsa, want, rel_tol=1e-12, abs_tol=1e-12):
            return False
        gw = orc.linear_grad_weight(g, x, sa)
        refw = torch.nn.grad.conv2d_weight((sign0(x) * float(np.float32(sa))).view(m, k, 1, 1), (n, k, 1, 1),
                                           g.double().view(m, n, 1, 1)).view(n, k)
        if not torch.allclose(gw, refw, rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_autograd(orc):
    """grad_in is d/dx of sum(g * y) for y = (sa * hardtanh(x / sa)) @ (sign(W) * sw)^T, and
    grad_w is d/dW of sum(g * y) for y = (sign(x) * sa) @ W^T (values kept off the clip edge)."""
    g, w, x = _data(4, 6, 10, 12)
    sa, sw = 0.75, 0.5
    xd = x.double().requires_grad_(True)
    y = (sa * torch.nn.functional.hardtanh(xd / sa)) @ (sign0(w) * sw).T
    (y * g.double()).sum().backward()
    gi, _ = orc.linear_grad_input(g, w, x, sa, sw)
    if not torch.allclose(gi, xd.grad, rtol=1e-12, atol=1e-12):
        return False
    wd = w.double().requires_grad_(True)
    y = (sign0(x) * sa) @ wd.T
    (y * g.double()).sum().backward()
    return torch.allclose(orc.linear_grad_weight(g, x, sa), wd.grad, rtol=1e-12, atol=1e-12)


def pin_closed_forms(orc):
    g, w, _ = _data(5, 4, 6, 8)
    sa, sw = 0.5, 0.25
    inside = torch.full((4, 8), 0.25)           # positive, unclipped: sign0 = 1, mask = 1
    gi, gsa = orc.linear_grad_input(g, w, inside, sa, sw)
    want = sw * (g.double().sum(0) * sign0(w).sum(1)).sum() / math.sqrt(32)
    if not math.isclose(gsa, float(want), rel_tol=1e-12):
        return False
    gi, gsa = orc.linear_grad_input(g, w, torch.full((4, 8), -1.5), sa, sw)   # all clipped
    if gsa != 0.0 or bool(gi.abs().sum() != 0):
        return False
    # all-ones: every gradient entry is a count
    ones = torch.ones((3, 5))
    gi, _ = orc.linear_grad_input(ones, torch.ones((5, 7)), torch.full((3, 7), 0.1), 1.0, 1.0)
    if not torch.equal(gi, torch.full((3, 7), 5.0, dtype=torch.float64)):
        return False
    gw = orc.linear_grad_weight(torch.ones((9, 2)), -torch.ones((9, 3)), 2.0)
    return torch.equal(gw, torch.full((2, 3), -18.0, dtype=torch.float64))


def pin_edges(orc):
    """Clip boundary (q == +-1 kept, the next fp32 above dropped), zeros (sign0 = 0), NaN."""
    sa = 0.7
    up = float(np.nextafter(np.float32(sa), np.float32(np.inf)))
    x = torch.tensor([[sa, -sa, up, -up, 0.0, -0.0]], dtype=torch.float32)
    g = torch.ones((1, 1))
    w = torch.tensor([[1.0, -2.0, 3.0, 0.0, 5.0, -0.0]])
    gi, gsa = orc.linear_grad_input(g, w, x, sa, 1.0)
    if gi.tolist() != [[1.0, -1.0, 0.0, 0.0, 1.0, 0.0]]:
        return False
    if not math.isclose(gsa, (1.0 * 1 + (-1.0) * -1) / math.sqrt(6), rel_tol=1e-15):
        return False
    gw = orc.linear_grad_weight(torch.tensor([[3.0]]), x, sa)
    if gw[0, 4] != 0.0 or gw[0, 5] != 0.0 or gw[0, 0] != 3.0 * float(np.float32(sa)):
        return False
    xn = torch.tensor([[float("nan"), 0.1]])
    gi, gsa = orc.linear_grad_input(torch.ones((1, 1)), torch.ones((1, 2)), xn, 1.0, 1.0)
    return gi.tolist() == [[1.0, 1.0]] and math.isnan(gsa)


def pin_quant_grad(orc):
    """Codes against torch's half-even round and clamp with the step from torch's amax; the largest
    element codes to +-127; every code times the step is within half a step of the value; all-zero
    and NaN gradients code to 0."""
    gen = torch.Generator().manual_seed(8)
    gw = (torch.randn((12, 40), generator=gen) * 3).double()
    gw[4, 7] = -(gw.abs().max() + 0.5)          # the largest magnitude is negative
    codes, amax = orc.quant_grad_i8(gw)
    v = gw.float()
    want_amax = float(v.abs().max())
    step = torch.tensor(want_amax, dtype=torch.float32) / 127.0
    if amax != want_amax:
        return False
    if not torch.equal(codes, torch.round(v / step).clamp(-127, 127).to(torch.int8)):
        return False
    i = int(v.abs().argmax())
    if abs(int(codes.view(-1)[i])) != 127:
        return False
    if not bool(((codes.double() * float(step) - v.double()).abs() <= float(step) / 2 * (1 + 1e-6)).all()):
        return False
    zc, za = orc.quant_grad_i8(torch.zeros((3, 8), dtype=torch.float64))
    if za != 0.0 or bool(zc.any()):
        return False
    gn = gw.clone()
    gn[1, 2] = float("nan")
    nc, na = orc.quant_grad_i8(gn)
    return math.isnan(na) and not bool(nc.any())


def _conv_cases(seed, count):
    import random
    rnd = random.Random(seed)
    out = []
    while len(out) < count:
        b, c, h, w = rnd.choice([1, 2]), rnd.choice([1, 3, 5]), rnd.randint(2, 7), rnd.randint(2, 7)
        o, kh, kw = rnd.choice([1, 2, 4]), rnd.choice([1, 2, 3]), rnd.choice([1, 2, 3])
        s, p, d = (rnd.choice([1, 2]), rnd.choice([1, 3])), (rnd.randint(0, 2), rnd.randint(0, 1)), \
            (rnd.choice([1, 2]), rnd.choice([1, 2]))
        ho = (h + 2 * p[0] - d[0] * (kh - 1) - 1) // s[0] + 1
        wo = (w + 2 * p[1] - d[1] * (kw - 1) - 1) // s[1] + 1
        if ho > 0 and wo > 0:
            out.append(((b, c, h, w), (o, kh, kw), s, p, d, (ho, wo)))
    return out


def pin_conv_vs_torch_grad(orc):
    """The conv page's backward with torch's gradient routines (float64), over random
    geometries with non-square kernels and per-axis stride / padding / dilation."""
    gen = torch.Generator().manual_seed(21)
    sa, sw = 0.7, 0.3
    sa32, sw32 = float(np.float32(sa)), float(np.float32(sw))
    for (b, c, h, w), (o, kh, kw), s, p, d, (ho, wo) in _conv_cases(21, 12):
        x = torch.randn((b, c, h, w), generator=gen)
        wt = torch.randn((o, c, kh, kw), generator=gen)
        g = torch.randn((b, o, ho, wo), generator=gen)
        gi, gsa, gw = orc.conv2d_grad(g, wt, x, s, p, d, sa, sw)
        ref = torch.nn.grad.conv2d_input((b, c, h, w), sign0(wt) * sw32, g.double(), stride=s,
                                         padding=p, dilation=d)
        ref = ref * mid_fp32(x, sa)
        if not torch.allclose(gi, ref, rtol=1e-12, atol=1e-12):
            return False
        want = float((ref * sign0(x)).sum() / math.sqrt(x.numel()))
        if not math.isclose(gsa, want, rel_tol=1e-12, abs_tol=1e-12):
            return False
        refw = torch.nn.grad.conv2d_weight(sign0(x) * sa32, (o, c, kh, kw), g.double(), stride=s,
                                           padding=p, dilation=d)
        if not torch.allclose(gw, refw, rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_conv_autograd(orc):
    """grad_in is d/dx of sum(g * conv(sa * hardtanh(x / sa), sign(W) * sw)); grad_w is d/dW of
    sum(g * conv(sign(x) * sa, W))."""
    gen = torch.Generator().manual_seed(22)
    sa, sw = 0.75, 0.5
    for (b, c, h, w), (o, kh, kw), s, p, d, (ho, wo) in _conv_cases(22, 6):
        x = torch.randn((b, c, h, w), generator=gen)
        wt = torch.randn((o, c, kh, kw), generator=gen)
        g = torch.randn((b, o, ho, wo), generator=gen)
        gi, _, gw = orc.conv2d_grad(g, wt, x, s, p, d, sa, sw)
        xd = x.double().requires_grad_(True)
        y = torch.nn.functional.conv2d(sa * torch.nn.functional.hardtanh(xd / sa), sign0(wt) * sw,
                                       stride=s, padding=p, dilation=d)
        (y * g.double()).sum().backward()
        if not torch.allclose(gi, xd.grad, rtol=1e-12, atol=1e-12):
            return False
        wd = wt.double().requires_grad_(True)
        y = torch.nn.functional.conv2d(sign0(x) * sa, wd, stride=s, padding=p, dilation=d)
        (y * g.double()).sum().backward()
        if not torch.allclose(gw, wd.grad, rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_conv_as_linear(orc):
    """A 1x1 kernel on 1x1 images is the linear layer: the conv form equals the linear form
    (two separate code paths of the oracle)."""
    g, w, x = _data(23, 7, 5, 9)
    gi, gsa, gw = orc.conv2d_grad(g.view(7, 5, 1, 1), w.view(5, 9, 1, 1), x.view(7, 9, 1, 1), 1, 0, 1,
                                  0.6, 0.4)
    li, lsa = orc.linear_grad_input(g, w, x, 0.6, 0.4)
    lw = orc.linear_grad_weight(g, x, 0.6)
    return torch.equal(gi.view(7, 9), li) and gsa == lsa and torch.equal(gw.view(5, 9), lw)


PINS = {
    "bwd_conv_vs_torch_grad": pin_conv_vs_torch_grad,
    "bwd_conv_autograd": pin_conv_autograd,
    "bwd_conv_as_linear": pin_conv_as_linear,
    "bwd_quant_grad": pin_quant_grad,
    "bwd_vs_torch_grad": pin_vs_torch_grad,
    "bwd_autograd": pin_autograd,
    "bwd_closed_forms": pin_closed_forms,
    "bwd_edges": pin_edges,
}
