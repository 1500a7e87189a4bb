"""bnn_gemm_noalloc (static device scratch, no allocation) against bnn_gemm, through the C ABI.

Both entry points run the same kernels, so every output must be identical: int32
accumulators bit for bit, scaled outputs bit for bit (and, against the oracle, within the
parity bar). Two calls in a row, the second smaller, show that what the first call left in
the shared array does not leak into the second; a call whose packed activations exceed the
array is rejected with nothing written.
"""
import ctypes

import pytest
import torch

import synth
from parity_check import check_scaled

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def bnn():
    import convolution_bnn_pack_amd as m
    return m


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _noalloc(bnn, x, xcode, wp, m, n, k, sa, sw, path, out):
    return bnn.lib.bnn_gemm_noalloc(x.data_ptr(), xcode, wp.data_ptr(), m, n, k, sa, sw, path,
                                    out.data_ptr(), bnn._DT[out.dtype], _stream())


def _with_workspace(bnn, x, xcode, wp, m, n, k, sa, sw, path, out):
    need = bnn.lib.bnn_gemm_workspace_bytes(m, k, xcode)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    return bnn.lib.bnn_gemm(x.data_ptr(), xcode, wp.data_ptr(), m, n, k, sa, sw, path,
                            out.data_ptr(), bnn._DT[out.dtype], ws.data_ptr(), ws.numel(), _stream())


def test_noalloc_matches_gemm_twice(bnn, oracle_lib):
    g = torch.Generator().manual_seed(91)
    # first a large call (4 MiB of packed activations), then a smaller ragged one (k % 32 != 0):
    # the second call's packed words overwrite only part of what the first left in the array
    cases = [(8192, 1536, 4096, torch.float16, torch.float16),
             (700, 520, 1000, torch.bfloat16, torch.float32)]
    for m, n, k, xdt, odt in cases:
        x = torch.randn((m, k), generator=g).to(xdt)
        w = torch.randn((n, k), generator=g).to(xdt)
        sa, sw = 0.37, 0.81
        acc_ref = oracle_lib.linear_acc(x, w)
        y_ref = oracle_lib.scale(acc_ref, sa, sw)
        xd, wp = x.to(DEV), bnn.w_pack(w.to(DEV))
        xcode = bnn._DT[xd.dtype]
        for path in (bnn.PATH_AUTO, bnn.PATH_MFMA_FP4, bnn.PATH_MFMA, bnn.PATH_XOR):
            print(f"noalloc {m}x{n}x{k} path={path}", flush=True)
            for out_t in (torch.int32, odt):
                a = torch.full((m, n), -7, dtype=out_t, device=DEV)
                b = torch.full((m, n), -9, dtype=out_t, device=DEV)
                assert _noalloc(bnn, xd, xcode, wp, m, n, k, sa, sw, path, a) == bnn.OK
                assert _with_workspace(bnn, xd, xcode, wp, m, n, k, sa, sw, path, b) == bnn.OK
                torch.cuda.synchronize()
                assert torch.equal(a, b), (m, n, k, path, out_t)
                if out_t == torch.int32:
                    assert torch.equal(a.cpu(), acc_ref), (m, n, k, path)
                else:
                    check_scaled(a, acc_ref, y_ref, f"noalloc {m}x{n}x{k} path {path}")


def test_noalloc_prepacked_and_limit(bnn):
    g = torch.Generator().manual_seed(92)
    m, n, k = 512, 256, 2048
    x = torch.randn((m, k), generator=g).half().to(DEV)
    wp = bnn.w_pack(torch.randn((n, k), generator=g).half().to(DEV))
    # pre-packed activations need no scratch
    xp = bnn.pack_sign(x)
    a = torch.empty((m, n), dtype=torch.int32, device=DEV)
    assert _noalloc(bnn, xp, bnn.U32_PACKED, wp, m, n, k, 1.0, 1.0, bnn.PATH_AUTO, a) == bnn.OK
    ref = bnn.gemm(x, wp, 1.0, 1.0, out_dtype=torch.int32)
    torch.cuda.synchronize()
    assert torch.equal(a, ref)
    # the Python wrapper runs the same entry point
    b = torch.empty((m, n), dtype=torch.int32, device=DEV)
    bnn.gemm_noalloc(x, wp, 1.0, 1.0, out=b)
    torch.cuda.synchronize()
    assert torch.equal(b, ref)
    # packed activations larger than the array: rejected before anything is enqueued. The
    # pointers are never dereferenced (validation fails first), so a small x stands in.
    rows = bnn.NOALLOC_SCRATCH_BYTES // (4 * (k // 32)) + 1
    out = torch.full((4, n), 5, dtype=torch.int32, device=DEV)
    st = _noalloc(bnn, x, bnn._DT[x.dtype], wp, rows, n, k, 1.0, 1.0, bnn.PATH_AUTO, out)
    assert st == bnn.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 5).all())
    # exactly at the limit the packed words fit: the large linear layer's 16384 x 8192
    # activations take 16 MiB
    wl = synth.WORKLOADS["linear_16384x8192x8192_bf16"]
    assert wl.m * (wl.k // 32) * 4 <= bnn.NOALLOC_SCRATCH_BYTES
