"""Pins of the oracle's W8A8 conv (CPU): the im2col + GEMM with INT8 quantizers of the
banghao.live blog post, section 3, read as per-tensor symmetric 8-bit quantizers with a given
amax (step amax/127, codes clamp(rint(v/step), -127, 127), fp32 division, half to even).

The codes are checked against torch's own round-half-even and clamp (library routines), the
accumulators against torch's fp64 conv2d on the codes and against a direct nested loop, the
scaled result against the blog's fake-quantized unfold -> mm -> reshape written with torch
ops in fp64, and closed forms (saturated codes give 127^2 * K_valid)."""
import math
import random

import numpy as np
import pytest
import torch

import oracle

DT = [torch.float32, torch.float16, torch.bfloat16]


def _torch_codes(x, amax):
    step = torch.tensor(amax, dtype=torch.float32) / 127.0
    q = torch.round(x.float() / step).clamp(-127, 127)
    q = torch.where(torch.isnan(q), torch.zeros_like(q), q)
    return q.to(torch.int8)


@pytest.mark.parametrize("dt", DT)
def test_codes_match_torch(dt):
    g = torch.Generator().manual_seed(91)
    x = (3 * torch.randn(20000, generator=g)).to(dt)
    for amax in (0.5, 1.0, 2.75, 6.0):
        assert torch.equal(oracle.quant_i8(x, amax), _torch_codes(x, amax)), amax
    # exact half steps round to even, signed zeros and saturation
    step = torch.tensor(1.0, dtype=torch.float32) / 127.0
    ties = (torch.arange(-20, 20, dtype=torch.float32) + 0.5) * step
    assert torch.equal(oracle.quant_i8(ties, 1.0), _torch_codes(ties, 1.0))
    edge = torch.tensor([0.0, -0.0, 1.0, -1.0, 5.0, -5.0, float("inf"), float("-inf"), float("nan")])
    assert oracle.quant_i8(edge, 1.0).tolist() == [0, 0, 127, -127, 127, -127, 127, -127, 0]


def _cases(count, seed):
    rnd = random.Random(seed)
    out = []
    while len(out) < count:
        b, c = rnd.choice([1, 2]), rnd.choice([1, 3, 16, 33])
        h, w = rnd.randint(1, 8), rnd.randint(1, 8)
        o, kh, kw = rnd.choice([1, 3]), rnd.choice([1, 2, 3]), rnd.choice([1, 2, 3])
        s = (rnd.choice([1, 2]), rnd.choice([1, 2]))
        p = (rnd.randint(0, 2), rnd.randint(0, 2))
        d = (rnd.choice([1, 2]), rnd.choice([1, 2]))
        ho = math.floor((h + 2 * p[0] - d[0] * (kh - 1) - 1) / s[0] + 1)
        wo = math.floor((w + 2 * p[1] - d[1] * (kw - 1) - 1) / s[1] + 1)
        if ho > 0 and wo > 0:
            out.append((b, c, h, w, o, kh, kw, s, p, d))
    return out


def test_acc_matches_torch_conv_on_codes():
    g = torch.Generator().manual_seed(92)
    for (b, c, h, w, o, kh, kw, s, p, d) in _cases(150, 7):
        dt = DT[(b + c + h) % 3]
        x = (2 * torch.randn((b, c, h, w), generator=g)).to(dt)
        wt = torch.randn((o, c, kh, kw), generator=g).to(dt)
        ax, aw = 3.0, 1.5                                           # some codes saturate
        acc = oracle.w8a8_conv2d_acc(x, wt, s, p, d, ax, aw)
        ref = torch.nn.functional.conv2d(_torch_codes(x, ax).double(), _torch_codes(wt, aw).double(),
                                         stride=s, padding=p, dilation=d)
        assert torch.equal(acc.double(), ref), (b, c, h, w, o, kh, kw, s, p, d)


def test_acc_matches_direct_loop():
    g = torch.Generator().manual_seed(93)
    for (b, c, h, w, o, kh, kw, s, p, d) in _cases(25, 8):
        x = torch.randn((b, c, h, w), generator=g)
        wt = torch.randn((o, c, kh, kw), generator=g)
        qx = oracle.quant_i8(x, 2.0).numpy().astype(np.int64)
        qw = oracle.quant_i8(wt, 2.0).numpy().astype(np.int64)
        acc = oracle.w8a8_conv2d_acc(x, wt, s, p, d, 2.0, 2.0).numpy()
        ho, wo = acc.shape[2:]
        want = np.zeros_like(acc)
        for bb in range(b):
            for oo in range(o):
                for oh in range(ho):
                    for ow in range(wo):
                        t = 0
                        for i in range(kh):
                            ih = oh * s[0] - p[0] + i * d[0]
                            for j in range(kw):
                                iw = ow * s[1] - p[1] + j * d[1]
                                if 0 <= ih < h and 0 <= iw < w:
                                    t += int(np.dot(qx[bb, :, ih, iw], qw[oo, :, i, j]))
                        want[bb, oo, oh, ow] = t
        assert np.array_equal(acc, want)


def test_fake_quant_unfold_mm_equivalence():
    """The blog's layer: unfold, fake-quantize both operands (code * step), mm, reshape. In fp64
    this equals step_x * step_w * acc up to the fp64 rounding of the products and sums."""
    g = torch.Generator().manual_seed(94)
    b, c, h, w, o, k, s, p = 2, 8, 9, 7, 5, 3, 1, 1
    x = torch.randn((b, c, h, w), generator=g)
    wt = torch.randn((o, c, k, k), generator=g)
    ax, aw = 2.5, 1.25
    sx = float(torch.tensor(ax, dtype=torch.float32) / 127.0)
    sw = float(torch.tensor(aw, dtype=torch.float32) / 127.0)
    cols = torch.nn.functional.unfold(x.double(), kernel_size=k, padding=p, stride=s)    # [b, ck^2, L]
    ho = math.floor((h + 2 * p - (k - 1) - 1) / s + 1)
    wo = math.floor((w + 2 * p - (k - 1) - 1) / s + 1)
    rows = cols.transpose(1, 2).reshape(-1, c * k * k)
    fq_x = _torch_codes(rows.float(), ax).double() * sx
    fq_w = _torch_codes(wt.view(o, -1), aw).double() * sw
    y = (fq_x @ fq_w.t()).reshape(b, ho * wo, o).transpose(1, 2).reshape(b, o, ho, wo)
    acc = oracle.w8a8_conv2d_acc(x, wt, s, p, 1, ax, aw).double()
    assert torch.allclose(y, acc * (sx * sw), rtol=1e-12, atol=1e-12)


def test_saturated_closed_form():
    c, h, w = 5, 6, 7
    x = torch.full((1, c, h, w), 4.0)                               # amax 2 -> every code 127
    wt = torch.full((3, c, 3, 2), -9.0)                             # -> every code -127
    acc = oracle.w8a8_conv2d_acc(x, wt, (1, 2), (1, 1), (1, 1), 2.0, 1.0)
    kv = oracle.conv2d_kvalid(c, h, w, (3, 2), (1, 2), (1, 1), (1, 1))
    assert torch.equal(acc[0], (-127 * 127 * kv).expand(3, *kv.shape).to(torch.int32))
