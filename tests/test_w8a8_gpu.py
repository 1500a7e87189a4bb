"""GPU parity of the W8A8 conv (int8 codes of per-tensor symmetric quantizers, implicit
im2col on the matrix cores) against the oracle: codes bit-exact, int32 sums bit-exact,
scaled outputs within the parity bar (f32 1e-6 relative, f16 / bf16 one ulp)."""
import pytest
import torch

import synth
from parity_check import check_scaled

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
DT = [torch.float32, torch.float16, torch.bfloat16]


@pytest.fixture(scope="module")
def bnn():
    import convolution_bnn_pack_amd as m
    return m


@pytest.fixture(scope="module")
def orc(oracle_lib):
    return oracle_lib


def _step(amax):
    return float(torch.tensor(amax, dtype=torch.float32) / 127.0)


@pytest.mark.parametrize("dt", DT)
def test_activation_and_weight_codes(bnn, orc, dt):
    g = torch.Generator().manual_seed(101)
    # partial last 64-pixel chunks, channel counts that are not a multiple of 64
    for (n, c, h, w) in [(1, 16, 1, 1), (2, 48, 5, 7), (3, 80, 9, 9), (2, 128, 14, 14), (1, 16, 65, 3),
                         (2, 64, 8, 8), (1, 80, 4, 6), (3, 16, 28, 28), (2, 144, 4, 4)]:
        x = synth.inject_edges((2 * torch.randn((n, c, h, w), generator=g)).to(dt), n + c + h, max(1, n * c * h * w // 30))
        print(f"codes {dt} {(n, c, h, w)}", flush=True)
        got = bnn.quant_i8_nhwc(x.to(DEV), 2.5).cpu()
        assert torch.equal(got, orc.quant_i8(x, 2.5).permute(0, 2, 3, 1).contiguous()), (n, c, h, w)
        wt = torch.randn((7, c, 3, 2), generator=g).to(dt)
        gw = bnn.quant_i8_weight(wt.to(DEV), 1.75).cpu()
        assert torch.equal(gw, orc.quant_i8(wt, 1.75).permute(0, 2, 3, 1).contiguous()), c


CASES = [  # (b, c, h, w, o, (kh, kw), (sh, sw), (ph, pw), (dh, dw))
    (1, 16, 5, 5, 8, (3, 3), (1, 1), (1, 1), (1, 1)),
    (2, 32, 9, 7, 40, (3, 3), (2, 2), (1, 1), (1, 1)),
    (1, 48, 12, 10, 130, (1, 3), (1, 2), (0, 1), (1, 1)),
    (3, 64, 14, 14, 64, (3, 3), (1, 1), (2, 2), (2, 2)),
    (2, 16, 8, 11, 17, (5, 2), (3, 1), (2, 1), (1, 3)),
    (1, 256, 7, 7, 256, (3, 3), (1, 1), (1, 1), (1, 1)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"c{c[1]}_o{c[4]}_k{c[5][0]}x{c[5][1]}")
def test_w8a8_conv_matches_oracle(bnn, orc, case):
    b, c, h, w, o, ks, s, p, d = case
    g = torch.Generator().manual_seed(sum(case[:5]))
    x = (1.5 * torch.randn((b, c, h, w), generator=g)).to(torch.float16)
    wt = torch.randn((o, c) + ks, generator=g)
    ax, aw = 3.0, 2.0                                                 # some codes saturate
    print(f"w8a8 conv {case}", flush=True)
    want = orc.w8a8_conv2d_acc(x, wt, s, p, d, ax, aw)
    xq = bnn.quant_i8_nhwc(x.to(DEV), ax)
    wq = bnn.quant_i8_weight(wt.to(DEV), aw)
    acc = bnn.w8a8_conv2d(xq, wq, ax, aw, ks, s, p, d, out_dtype=torch.int32).cpu()
    assert torch.equal(acc, want)
    y = want.double() * (_step(ax) * _step(aw))
    for odt in (torch.float32, torch.float16, torch.bfloat16):
        out = bnn.w8a8_conv2d(xq, wq, ax, aw, ks, s, p, d, out_dtype=odt)
        check_scaled(out, want, y, f"w8a8 {case} {odt}")


@pytest.mark.parametrize("name", ["conv_down_s2_f16", "conv_dil2_f16"])
def test_w8a8_workload_shapes_sampled(bnn, orc, name):
    """The strided and the dilated 128x128x28x28 -> 256 layers, all images on the GPU, two
    images checked against the oracle."""
    wl = synth.WORKLOADS[name]
    x, w, _, _ = synth.make_inputs(wl)
    ax, aw = 4.0, 3.0
    print(f"w8a8 workload {name}", flush=True)
    xq = bnn.quant_i8_nhwc(x.to(DEV), ax)
    wq = bnn.quant_i8_weight(w.to(DEV), aw)
    acc = bnn.w8a8_conv2d(xq, wq, ax, aw, wl.ks, wl.stride, wl.padding, wl.dilation,
                          out_dtype=torch.int32).cpu()
    imgs = [0, wl.batch - 1]
    want = orc.w8a8_conv2d_acc(x, w, wl.stride, wl.padding, wl.dilation, ax, aw, images=imgs)
    assert torch.equal(acc[imgs], want)
    again = bnn.w8a8_conv2d(xq, wq, ax, aw, wl.ks, wl.stride, wl.padding, wl.dilation,
                            out_dtype=torch.int32).cpu()
    assert torch.equal(acc, again)


def test_w8a8_saturated_closed_form(bnn, orc):
    c = 32
    x = torch.full((1, c, 6, 7), 4.0, device=DEV)
    wt = torch.full((3, c, 3, 2), -9.0, device=DEV)
    xq, wq = bnn.quant_i8_nhwc(x, 2.0), bnn.quant_i8_weight(wt, 1.0)
    acc = bnn.w8a8_conv2d(xq, wq, 2.0, 1.0, (3, 2), (1, 2), (1, 1), (1, 1), out_dtype=torch.int32).cpu()
    kv = orc.conv2d_kvalid(c, 6, 7, (3, 2), (1, 2), (1, 1), (1, 1))
    assert torch.equal(acc[0], (-127 * 127 * kv).expand(3, *kv.shape).to(torch.int32))
