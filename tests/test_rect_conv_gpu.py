"""GPU parity for the general conv geometry (bnn_conv2d_ex): non-square kernels and stride,
padding and dilation given per axis. Packed weights bit-exact against the oracle's layout,
int32 accumulators bit-exact on all three paths, scaled outputs within the parity bar."""
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
EXPLICIT = ["xor", "mfma", "mfma_fp4"]

# (b, c, h, w, o, (kh, kw), (sh, sw), (ph, pw), (dh, dw))
CASES = [
    (2, 32, 9, 11, 40, (1, 3), (1, 1), (0, 1), (1, 1)),
    (1, 64, 12, 7, 33, (3, 1), (2, 1), (1, 0), (1, 1)),
    (2, 96, 10, 10, 70, (2, 5), (1, 2), (0, 2), (2, 1)),
    (1, 40, 8, 13, 17, (5, 2), (3, 1), (2, 1), (1, 3)),
    (3, 128, 14, 14, 64, (3, 3), (2, 1), (1, 2), (1, 2)),
    (1, 33, 6, 20, 9, (1, 7), (1, 3), (0, 3), (1, 1)),
    (2, 256, 7, 7, 256, (7, 1), (1, 1), (3, 0), (1, 1)),
]


@pytest.fixture(scope="module")
def bnn():
    import convolution_bnn_pack_amd as m
    return m


@pytest.fixture(scope="module")
def orc(oracle_lib):
    return oracle_lib


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"c{c[1]}_k{c[5][0]}x{c[5][1]}_s{c[6][0]}{c[6][1]}")
def test_rect_conv_all_paths(bnn, orc, case):
    b, c, h, w, o, ks, s, p, d = case
    g = torch.Generator().manual_seed(sum(case[:5]) + ks[0] * 7 + ks[1])
    x = torch.randn((b, c, h, w), generator=g).to(torch.float16)
    wt = torch.randn((o, c) + ks, generator=g)
    print(f"rect conv {case}", flush=True)
    wp = bnn.w_pack(wt.to(DEV))
    assert torch.equal(wp.cpu(), orc.pack_conv_weight(wt))
    want = orc.conv2d_acc(x, wt, s, p, d)
    xd = x.to(DEV)
    xp = bnn.pack_sign_nchw(xd)
    for path in EXPLICIT + ["auto"]:
        got = bnn.conv2d(xd, wp, 1.0, 1.0, ks, s, p, d, path=path, out_dtype=torch.int32).cpu()
        assert torch.equal(got, want), (path, "float input")
        got = bnn.conv2d(xp, wp, 1.0, 1.0, ks, s, p, d, path=path, out_dtype=torch.int32, channels=c).cpu()
        assert torch.equal(got, want), (path, "packed input")
    sa, sw = 0.3, 0.7
    y = bnn.conv2d(xd, wp, sa, sw, ks, s, p, d, out_dtype=torch.float32).cpu().double()
    ref = orc.scale(want, sa, sw)
    assert torch.all((y - ref).abs() <= 1e-6 * ref.abs())


def test_rect_kvalid_closed_form(bnn, orc):
    """x = +1, W = +1 gives acc = C * (valid taps) for every pixel, per axis."""
    c = 48
    x = torch.ones((1, c, 9, 10), device=DEV)
    for ks, s, p, d in [((1, 5), (1, 2), (0, 2), (1, 1)), ((5, 3), (2, 1), (3, 1), (1, 2))]:
        wp = bnn.w_pack(torch.ones((4, c) + ks, device=DEV))
        kv = orc.conv2d_kvalid(c, 9, 10, ks, s, p, d)
        for path in EXPLICIT:
            acc = bnn.conv2d(x, wp, 1.0, 1.0, ks, s, p, d, path=path, out_dtype=torch.int32).cpu()
            assert torch.equal(acc, kv.expand(1, 4, *kv.shape)), (ks, path)
