"""8-bit sign containers (the CUTLASS conv layer's uint8_t words) through the C ABI, against the
oracle (GPU).

Inputs are made by the oracle's own byte packs (oracle.pack_rows_u8 / pack_nchw_u8 /
pack_conv_weight_u8), so nothing on the device side decides them. Checked bit-exactly:
bnn_u8_to_words against the oracle's 32-bit words of the same data (also with the containers'
unused high bits set, which the conversion must clear), and int32 accumulators of bnn_gemm /
bnn_conv2d / bnn_conv2d_ex / bnn_gemm_noalloc fed BNN_U8_PACKED activations and weights converted
from 8-bit containers, on every path, at C = 40 and 72, K = 40 (repacked in the workspace) and at
whole-word lengths (read in place).
"""
import pytest
import torch

import synth
from parity_check import check_scaled

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PATHS = ["xor", "mfma", "mfma_fp4", "auto"]


@pytest.fixture(scope="module")
def bnn():
    import convolution_bnn_pack_amd as m
    return m


def _dirty_tail(u8: torch.Tensor, bits: int) -> torch.Tensor:
    """Set the unused high bits of each row's last container (they must not matter)."""
    if bits % 8 == 0:
        return u8
    out = u8.clone()
    out[..., -1] |= (0xFF << (bits % 8)) & 0xFF
    return out


def test_u8_to_words_bit_exact(bnn, oracle_lib):
    g = torch.Generator().manual_seed(81)
    for tdt in (torch.float32, torch.float16, torch.bfloat16):
        for rows, k in ((1, 1), (3, 8), (5, 9), (7, 40), (4, 72), (6, 100), (3, 256), (33, 1000)):
            x = synth.inject_edges(torch.randn((rows, k), generator=g).to(tdt), rows * 3 + k, max(1, rows * k // 10))
            want = oracle_lib.pack_rows(x)
            src = oracle_lib.pack_rows_u8(x)
            for dirty in (False, True):
                s = _dirty_tail(src, k) if dirty else src
                got = bnn.u8_to_words(s.to(DEV), k).cpu()
                assert torch.equal(got, want), (tdt, rows, k, dirty)
    # conv weights [o, kh, kw, ceil(c/8)] -> [o, kh, kw, ceil(c/32)]
    for c in (40, 72, 64):
        w = torch.randn((9, c, 3, 2), generator=g)
        got = bnn.u8_to_words(oracle_lib.pack_conv_weight_u8(w).to(DEV), c).cpu()
        assert torch.equal(got, oracle_lib.pack_conv_weight(w)), c


@pytest.mark.parametrize("k", [40, 72, 1000, 4096])
def test_gemm_u8_activations(bnn, oracle_lib, k):
    g = torch.Generator().manual_seed(82 + k)
    m, n = 300, 136
    x = torch.randn((m, k), generator=g).half()
    w = torch.randn((n, k), generator=g).half()
    acc = oracle_lib.linear_acc(x, w)
    y = oracle_lib.scale(acc, 0.6, 0.3)
    xu8 = _dirty_tail(oracle_lib.pack_rows_u8(x), k).to(DEV)
    wp = bnn.u8_to_words(oracle_lib.pack_rows_u8(w).to(DEV), k)
    assert torch.equal(wp.cpu(), oracle_lib.pack_rows(w))
    for path in PATHS:
        got = bnn.gemm(xu8, wp, 0.6, 0.3, path=path, out_dtype=torch.int32, k=k)
        assert torch.equal(got.cpu(), acc), (k, path)
        out = bnn.gemm(xu8, wp, 0.6, 0.3, path=path, out_dtype=torch.float32, k=k)
        check_scaled(out, acc, y, f"u8 gemm k={k} {path}")
    # the no-allocation entry point repacks ragged containers into its own array
    out = torch.empty((m, n), dtype=torch.int32, device=DEV)
    bnn.gemm_noalloc(xu8, wp, 1.0, 1.0, out=out, k=k)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), acc)


@pytest.mark.parametrize("c", [40, 72, 64])
def test_conv_u8_activations(bnn, oracle_lib, c):
    g = torch.Generator().manual_seed(90 + c)
    x = torch.randn((3, c, 11, 9), generator=g)
    for (kh, kw), st, pd, dl in (((3, 3), 1, 1, 1), ((3, 3), 2, 1, 1), ((3, 2), (1, 2), (2, 0), (2, 1))):
        wt = torch.randn((70, c, kh, kw), generator=g)
        acc = oracle_lib.conv2d_acc(x, wt, st, pd, dl)
        xu8 = _dirty_tail(oracle_lib.pack_nchw_u8(x), c).to(DEV)
        wp = bnn.u8_to_words(oracle_lib.pack_conv_weight_u8(wt).to(DEV), c)
        for path in PATHS:
            got = bnn.conv2d(xu8, wp, 1.0, 1.0, (kh, kw), st, pd, dl, path=path, out_dtype=torch.int32,
                             channels=c)
            assert torch.equal(got.cpu(), acc), (c, kh, kw, st, pd, dl, path)
