"""The C ABI on the host (no GPU): every symbol declared in include/bnn.h is
exported by libbnn.so, and every argument check returns its status before any
HIP call (so these calls run without a device; the fake pointers below are
never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bnn.h")


@pytest.fixture(scope="module")
def bnn():
    lib_path = os.path.join(ROOT, "convolution_bnn_pack_amd", "libbnn.so")
    if not os.path.exists(lib_path):
        # the build script is loaded by its path: the package itself needs the library
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_bnn_build", os.path.join(ROOT, "convolution_bnn_pack_amd", "_build.py"))
        build = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(build)
        build.build()
    import convolution_bnn_pack_amd as m
    return m


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bnn_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported(bnn):
    names = _declared()
    assert len(names) >= 11
    for name in names:
        assert hasattr(bnn.lib, name), name
    assert sorted(bnn.EXPORTS) == names


def test_status_strings(bnn):
    for code in range(8):
        assert bnn.lib.bnn_status_string(code)
    assert bnn.lib.bnn_status_string(99) == b"unknown status"


FAKE = 0x10000          # 64 KiB-aligned, never dereferenced
MISALIGNED = 0x10004


def _gemm(bnn, **kw):
    a = dict(x=FAKE, x_dtype=bnn.F16, w=FAKE, m=64, n=64, k=256, sa=1.0, sw=1.0,
             path=bnn.PATH_AUTO, out=FAKE, out_dtype=bnn.F32, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return bnn.lib.bnn_gemm(a["x"], a["x_dtype"], a["w"], a["m"], a["n"], a["k"], a["sa"], a["sw"],
                            a["path"], a["out"], a["out_dtype"], a["ws"], a["ws_bytes"], a["stream"])


def test_gemm_argument_checks(bnn):
    # any k >= 1 passes the shape checks (ragged k packs a partial last word): a null x then
    # stops the call before anything is enqueued
    assert _gemm(bnn, k=100, x=None) == bnn.ERR_NULL
    assert _gemm(bnn, k=-5) == bnn.ERR_SHAPE
    assert _gemm(bnn, k=0) == bnn.ERR_SHAPE
    assert _gemm(bnn, m=-1) == bnn.ERR_SHAPE
    assert _gemm(bnn, x_dtype=7) == bnn.ERR_DTYPE
    assert _gemm(bnn, out_dtype=bnn.U32_PACKED) == bnn.ERR_DTYPE
    assert _gemm(bnn, path=5) == bnn.ERR_PATH
    # the fp4 path sums in fp32, exact only while K <= 2^24
    assert _gemm(bnn, k=(1 << 24) + 32, path=bnn.PATH_MFMA_FP4) == bnn.ERR_PATH
    assert _gemm(bnn, k=1 << 24, path=bnn.PATH_MFMA_FP4, x=None) == bnn.ERR_NULL
    assert _gemm(bnn, x=None) == bnn.ERR_NULL
    assert _gemm(bnn, w=None) == bnn.ERR_NULL
    assert _gemm(bnn, out=None) == bnn.ERR_NULL
    assert _gemm(bnn, x=FAKE + 1) == bnn.ERR_ALIGN                  # f16 x: 2-byte elements
    assert _gemm(bnn, x=FAKE + 2, x_dtype=bnn.U32_PACKED) == bnn.ERR_ALIGN
    assert _gemm(bnn, out=MISALIGNED) == bnn.ERR_ALIGN
    assert _gemm(bnn, ws=None) == bnn.ERR_WORKSPACE
    assert _gemm(bnn, ws_bytes=64 * 8 * 4 - 1) == bnn.ERR_WORKSPACE
    # empty problems are no-ops and succeed without touching anything
    assert _gemm(bnn, m=0, x=None, out=None) == bnn.OK
    assert _gemm(bnn, n=0, x=None, out=None) == bnn.OK
    # reduction lengths whose 32 * words no longer fit an int are rejected (the kernels count
    # 32 signs per word in int); the largest that fits passes the shape checks
    for k in ((1 << 31) - 1, (1 << 31) - 31):
        assert _gemm(bnn, k=k, path=bnn.PATH_MFMA, x=None) == bnn.ERR_SHAPE
    assert _gemm(bnn, k=(1 << 31) - 32, path=bnn.PATH_MFMA, x=None) == bnn.ERR_NULL


def test_u8_container_argument_checks(bnn):
    # 8-bit containers: any alignment when they are repacked (k % 32 != 0), 4 bytes when the
    # bytes are read in place as words (k % 32 == 0, no workspace needed)
    assert _gemm(bnn, x_dtype=bnn.U8_PACKED, k=40, x=FAKE + 1, w=None) == bnn.ERR_NULL
    assert _gemm(bnn, x_dtype=bnn.U8_PACKED, k=64, x=FAKE + 1) == bnn.ERR_ALIGN
    assert _gemm(bnn, x_dtype=bnn.U8_PACKED, k=64, x=FAKE + 4, ws=None, w=None) == bnn.ERR_NULL
    assert _gemm(bnn, x_dtype=bnn.U8_PACKED, k=40, ws=None) == bnn.ERR_WORKSPACE
    assert bnn.lib.bnn_gemm_workspace_bytes(64, 40, bnn.U8_PACKED) == 64 * 2 * 4
    assert bnn.lib.bnn_gemm_workspace_bytes(64, 64, bnn.U8_PACKED) == 0
    assert bnn.lib.bnn_conv2d_workspace_bytes(2, 40, 5, 5, bnn.U8_PACKED) == 2 * 5 * 5 * 2 * 4
    assert bnn.lib.bnn_conv2d_workspace_bytes(2, 96, 5, 5, bnn.U8_PACKED) == 0
    assert _conv(bnn, x_dtype=bnn.U8_PACKED, c=40, x=FAKE + 3, wp=None) == bnn.ERR_NULL
    assert _conv(bnn, x_dtype=bnn.U8_PACKED, c=64, x=FAKE + 2) == bnn.ERR_ALIGN
    assert _conv(bnn, x_dtype=bnn.U8_PACKED, c=40, ws=None) == bnn.ERR_WORKSPACE
    u8 = bnn.lib.bnn_u8_to_words
    assert u8(FAKE, 4, 0, FAKE, None) == bnn.ERR_SHAPE
    assert u8(FAKE, -1, 8, FAKE, None) == bnn.ERR_SHAPE
    assert u8(FAKE, 0, 8, None, None) == bnn.OK
    assert u8(None, 4, 8, FAKE, None) == bnn.ERR_NULL
    assert u8(FAKE + 1, 4, 8, FAKE + 2, None) == bnn.ERR_ALIGN


def _conv(bnn, **kw):
    a = dict(x=FAKE, x_dtype=bnn.F32, n=2, c=64, h=14, w=14, wp=FAKE, o=32, sa=1.0, sw=1.0, ks=3,
             s=1, p=1, d=1, path=bnn.PATH_AUTO, out=FAKE, out_dtype=bnn.F32, ws=FAKE,
             ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return bnn.lib.bnn_conv2d(a["x"], a["x_dtype"], a["n"], a["c"], a["h"], a["w"], a["wp"], a["o"],
                              a["sa"], a["sw"], a["ks"], a["s"], a["p"], a["d"], a["path"], a["out"],
                              a["out_dtype"], a["ws"], a["ws_bytes"], a["stream"])


def test_conv_argument_checks(bnn):
    assert _conv(bnn, c=48, wp=None) == bnn.ERR_NULL                # ragged C passes the shape checks
    # a channel count whose 32 * words overflows int is rejected before anything else runs
    assert _conv(bnn, c=(1 << 31) - 1, ks=1, p=0, n=1, h=1, w=1, path=bnn.PATH_MFMA) == bnn.ERR_SHAPE
    assert _conv(bnn, c=0) == bnn.ERR_SHAPE
    assert _conv(bnn, ks=0) == bnn.ERR_SHAPE
    assert _conv(bnn, s=0) == bnn.ERR_SHAPE
    assert _conv(bnn, d=0) == bnn.ERR_SHAPE
    assert _conv(bnn, p=-1) == bnn.ERR_SHAPE
    assert _conv(bnn, h=2, ks=5, p=0) == bnn.ERR_SHAPE            # empty output
    assert _conv(bnn, x_dtype=bnn.I32) == bnn.ERR_DTYPE
    assert _conv(bnn, out_dtype=9) == bnn.ERR_DTYPE
    assert _conv(bnn, path=4) == bnn.ERR_PATH
    # fp4 path: K = ks^2 * c must stay <= 2^24 (here 9 * 2^21 = 18.9M)
    assert _conv(bnn, c=1 << 21, path=bnn.PATH_MFMA_FP4) == bnn.ERR_PATH
    assert _conv(bnn, path=bnn.PATH_XOR, ks=9, p=4) == bnn.ERR_PATH  # 81 taps > the XOR table
    assert _conv(bnn, wp=None) == bnn.ERR_NULL
    assert _conv(bnn, out=MISALIGNED) == bnn.ERR_ALIGN
    assert _conv(bnn, ws=None) == bnn.ERR_WORKSPACE
    assert _conv(bnn, ws_bytes=2 * 14 * 14 * 2 * 4 - 1) == bnn.ERR_WORKSPACE
    assert _conv(bnn, n=0, x=None, out=None) == bnn.OK
    assert _conv(bnn, o=0, x=None, out=None) == bnn.OK


def test_conv_ex_argument_checks(bnn):
    L = bnn.lib

    def conv_ex(**kw):
        a = dict(x=FAKE, x_dtype=bnn.F32, n=2, c=64, h=14, w=14, wp=FAKE, o=32, kh=3, kw=1, sh=1, sw=2,
                 ph=1, pw=0, dh=1, dw=1, path=bnn.PATH_AUTO, out=FAKE, out_dtype=bnn.F32, ws=FAKE,
                 ws_bytes=1 << 20)
        a.update(kw)
        return L.bnn_conv2d_ex(a["x"], a["x_dtype"], a["n"], a["c"], a["h"], a["w"], a["wp"], a["o"],
                               1.0, 1.0, a["kh"], a["kw"], a["sh"], a["sw"], a["ph"], a["pw"], a["dh"],
                               a["dw"], a["path"], a["out"], a["out_dtype"], a["ws"], a["ws_bytes"], None)
    for bad in (dict(kw=0), dict(kh=0), dict(sw=0), dict(sh=0), dict(dw=0), dict(dh=0), dict(pw=-1),
                dict(ph=-1), dict(w=2, kw=5, pw=0), dict(h=1, kh=3, ph=0)):
        assert conv_ex(**bad) == bnn.ERR_SHAPE, bad
    assert conv_ex(kh=7, kw=8, ph=3, pw=3, path=bnn.PATH_XOR) == bnn.ERR_PATH    # 56 taps > 49
    assert conv_ex(c=1 << 20, kh=5, kw=4, ph=2, pw=2, path=bnn.PATH_MFMA_FP4) == bnn.ERR_PATH
    assert conv_ex(wp=None) == bnn.ERR_NULL                                      # shapes accepted
    assert conv_ex(n=0, x=None, out=None) == bnn.OK
    assert L.bnn_w_pack_conv(FAKE, bnn.F32, 8, 64, 3, 0, FAKE, None) == bnn.ERR_SHAPE
    assert L.bnn_w_pack_conv(FAKE, bnn.I32, 8, 64, 3, 2, FAKE, None) == bnn.ERR_DTYPE
    assert L.bnn_w_pack_conv(None, bnn.F32, 8, 64, 3, 2, FAKE, None) == bnn.ERR_NULL
    assert L.bnn_w_pack_conv(FAKE + 2, bnn.F32, 8, 64, 3, 2, FAKE, None) == bnn.ERR_ALIGN
    assert L.bnn_w_pack_conv(None, bnn.F32, 0, 64, 3, 2, None, None) == bnn.OK


def test_w8a8_argument_checks(bnn):
    L = bnn.lib

    def conv(**kw):
        a = dict(xq=FAKE, n=2, c=32, h=8, w=8, wq=FAKE, o=16, ax=2.0, aw=1.0, kh=3, kw=3, sh=1, sw=1,
                 ph=1, pw=1, dh=1, dw=1, out=FAKE, odt=bnn.F32)
        a.update(kw)
        return L.bnn_w8a8_conv2d(a["xq"], a["n"], a["c"], a["h"], a["w"], a["wq"], a["o"], a["ax"],
                                 a["aw"], a["kh"], a["kw"], a["sh"], a["sw"], a["ph"], a["pw"], a["dh"],
                                 a["dw"], a["out"], a["odt"], None)
    assert conv(c=24) == bnn.ERR_SHAPE                  # channels must be a multiple of 16
    assert conv(ax=0.0) == bnn.ERR_SHAPE and conv(aw=-1.0) == bnn.ERR_SHAPE
    assert conv(c=16 * 1000, kh=3, kw=3) == bnn.ERR_SHAPE     # 127^2 * K would overflow int32
    assert conv(h=2, kh=5, ph=0) == bnn.ERR_SHAPE
    assert conv(odt=bnn.U32_PACKED) == bnn.ERR_DTYPE
    assert conv(wq=None) == bnn.ERR_NULL
    assert conv(xq=FAKE + 8) == bnn.ERR_ALIGN
    assert conv(n=0, xq=None, out=None) == bnn.OK
    q = L.bnn_quant_i8_nhwc
    assert q(FAKE, bnn.F32, 1, 20, 4, 4, 1.0, FAKE, None) == bnn.ERR_SHAPE
    assert q(FAKE, bnn.F32, 1, 32, 4, 4, 0.0, FAKE, None) == bnn.ERR_SHAPE
    assert q(FAKE, bnn.I32, 1, 32, 4, 4, 1.0, FAKE, None) == bnn.ERR_DTYPE
    assert q(None, bnn.F32, 1, 32, 4, 4, 1.0, FAKE, None) == bnn.ERR_NULL
    assert q(FAKE, bnn.F32, 1, 32, 4, 4, 1.0, FAKE + 4, None) == bnn.ERR_ALIGN
    qw = L.bnn_quant_i8_weight
    assert qw(FAKE, bnn.F32, 4, 32, 0, 3, 1.0, FAKE, None) == bnn.ERR_SHAPE
    assert qw(None, bnn.F32, 4, 32, 3, 3, 1.0, FAKE, None) == bnn.ERR_NULL
    assert qw(None, bnn.F32, 0, 32, 3, 3, 1.0, None, None) == bnn.OK


def test_pack_argument_checks(bnn):
    L = bnn.lib
    assert L.bnn_pack_sign(None, bnn.F32, 4, 33, FAKE, None) == bnn.ERR_NULL     # ragged k accepted
    assert L.bnn_pack_sign(FAKE, bnn.F32, 4, 0, FAKE, None) == bnn.ERR_SHAPE
    assert L.bnn_pack_sign(FAKE, bnn.I32, 4, 32, FAKE, None) == bnn.ERR_DTYPE
    assert L.bnn_pack_sign(None, bnn.F32, 4, 32, FAKE, None) == bnn.ERR_NULL
    assert L.bnn_pack_sign(FAKE + 2, bnn.F32, 4, 32, FAKE, None) == bnn.ERR_ALIGN
    assert L.bnn_pack_sign(None, bnn.F32, 0, 32, None, None) == bnn.OK
    assert L.bnn_pack_sign_nchw(None, bnn.F16, 1, 40, 4, 4, FAKE, None) == bnn.ERR_NULL
    assert L.bnn_pack_sign_nchw(FAKE + 1, bnn.F16, 1, 40, 4, 4, FAKE, None) == bnn.ERR_ALIGN   # odd byte
    assert L.bnn_pack_sign_nchw(FAKE, bnn.F16, 1, 40, 4, 4, FAKE + 2, None) == bnn.ERR_ALIGN
    assert L.bnn_pack_sign_nchw(FAKE, bnn.F16, 1, 32, 0, 4, FAKE, None) == bnn.ERR_SHAPE
    assert L.bnn_w_pack(None, bnn.F32, 8, 48, 0, FAKE, None) == bnn.ERR_NULL
    assert L.bnn_w_pack(FAKE, bnn.F32, 8, 0, 0, FAKE, None) == bnn.ERR_SHAPE
    assert L.bnn_w_pack(FAKE, bnn.F32, 8, 64, -1, FAKE, None) == bnn.ERR_SHAPE
    assert L.bnn_w_pack(FAKE, bnn.U32_PACKED, 8, 64, 3, FAKE, None) == bnn.ERR_DTYPE
    assert L.bnn_w_pack(FAKE + 2, bnn.F32, 8, 64, 0, FAKE, None) == bnn.ERR_ALIGN
    assert L.bnn_w_pack(None, bnn.F32, 0, 64, 3, None, None) == bnn.OK


def test_prologue_argument_checks(bnn):
    L = bnn.lib
    # shifted row pack: bias of one value or one per column
    assert L.bnn_pack_sign_shift(FAKE, bnn.F16, 4, 64, FAKE, bnn.F32, 2, FAKE, None) == bnn.ERR_SHAPE
    assert L.bnn_pack_sign_shift(FAKE, bnn.F16, 4, 48, FAKE, bnn.F32, 47, FAKE, None) == bnn.ERR_SHAPE
    assert L.bnn_pack_sign_shift(None, bnn.F16, 4, 48, FAKE, bnn.F32, 48, FAKE, None) == bnn.ERR_NULL
    assert L.bnn_pack_sign_shift(FAKE, bnn.F16, 4, 64, FAKE, bnn.I32, 64, FAKE, None) == bnn.ERR_DTYPE
    assert L.bnn_pack_sign_shift(FAKE, bnn.U32_PACKED, 4, 64, FAKE, bnn.F32, 1, FAKE, None) == bnn.ERR_DTYPE
    assert L.bnn_pack_sign_shift(FAKE, bnn.F16, 4, 64, None, bnn.F32, 1, FAKE, None) == bnn.ERR_NULL
    assert L.bnn_pack_sign_shift(FAKE, bnn.F16, 4, 64, FAKE + 2, bnn.F32, 64, FAKE, None) == bnn.ERR_ALIGN
    assert L.bnn_pack_sign_shift(FAKE + 1, bnn.F16, 4, 64, FAKE, bnn.F32, 64, FAKE, None) == bnn.ERR_ALIGN
    assert L.bnn_pack_sign_shift(None, bnn.F16, 0, 64, None, bnn.F32, 64, None, None) == bnn.OK
    # shifted NCHW pack: one bias per channel
    assert L.bnn_pack_sign_nchw_shift(FAKE, bnn.F32, 1, 0, 4, 4, FAKE, bnn.F32, FAKE, None) == bnn.ERR_SHAPE
    assert L.bnn_pack_sign_nchw_shift(FAKE, bnn.F32, 1, 32, 4, 4, FAKE, 5, FAKE, None) == bnn.ERR_DTYPE
    assert L.bnn_pack_sign_nchw_shift(FAKE, bnn.F32, 1, 32, 4, 4, None, bnn.F16, FAKE, None) == bnn.ERR_NULL
    assert L.bnn_pack_sign_nchw_shift(FAKE, bnn.F32, 1, 32, 4, 4, FAKE + 1, bnn.F16, FAKE, None) == bnn.ERR_ALIGN
    assert L.bnn_pack_sign_nchw_shift(None, bnn.F32, 0, 32, 4, 4, None, bnn.F16, None, None) == bnn.OK
    # lazy scale: count >= 1, a workspace of the queried size
    need = L.bnn_abs_mean_workspace_bytes(1 << 20)
    assert need == 512 * 8 and L.bnn_abs_mean_workspace_bytes(1 << 30) == 1024 * 8
    assert L.bnn_abs_mean_workspace_bytes(1) == 8 and L.bnn_abs_mean_workspace_bytes(0) == 0
    assert L.bnn_abs_mean_scale(FAKE, bnn.F32, 0, 2.0, FAKE, FAKE, need, None) == bnn.ERR_SHAPE
    assert L.bnn_abs_mean_scale(FAKE, bnn.I32, 1 << 20, 2.0, FAKE, FAKE, need, None) == bnn.ERR_DTYPE
    assert L.bnn_abs_mean_scale(FAKE, bnn.F32, 1 << 20, 2.0, None, FAKE, need, None) == bnn.ERR_NULL
    assert L.bnn_abs_mean_scale(FAKE, bnn.F32, 1 << 20, 2.0, FAKE + 4, FAKE, need, None) == bnn.ERR_ALIGN
    assert L.bnn_abs_mean_scale(FAKE, bnn.F32, 1 << 20, 2.0, FAKE, FAKE, need - 1, None) == bnn.ERR_WORKSPACE
    assert L.bnn_abs_mean_scale(FAKE, bnn.F32, 1 << 20, 2.0, FAKE, None, need, None) == bnn.ERR_WORKSPACE
    # one-pass prologue: rows >= 1 (a mean needs elements), x 16-byte aligned, the bias rules of
    # the shifted pack, a workspace at least the query, which covers both the one-kernel and
    # the two-pass form
    need = L.bnn_pack_sign_shift_abs_mean_workspace_bytes(16384, 8192)
    assert need >= L.bnn_abs_mean_workspace_bytes(16384 * 8192) and need % 8 == 0
    assert L.bnn_pack_sign_shift_abs_mean_workspace_bytes(0, 64) == 0
    assert L.bnn_pack_sign_shift_abs_mean_workspace_bytes(5, 33) == L.bnn_abs_mean_workspace_bytes(5 * 33)
    ps = L.bnn_pack_sign_shift_abs_mean
    assert ps(FAKE, bnn.F16, 0, 64, FAKE, bnn.F32, 1, 2.0, FAKE, FAKE, FAKE, need, None) == bnn.ERR_SHAPE
    assert ps(FAKE, bnn.F16, 4, 64, FAKE, bnn.F32, 2, 2.0, FAKE, FAKE, FAKE, need, None) == bnn.ERR_SHAPE
    assert ps(FAKE, bnn.I32, 4, 64, FAKE, bnn.F32, 1, 2.0, FAKE, FAKE, FAKE, need, None) == bnn.ERR_DTYPE
    assert ps(FAKE, bnn.F16, 4, 64, FAKE, bnn.F32, 1, 2.0, FAKE, None, FAKE, need, None) == bnn.ERR_NULL
    assert ps(FAKE + 2, bnn.F16, 4, 64, FAKE, bnn.F32, 1, 2.0, FAKE, FAKE, FAKE, need, None) == bnn.ERR_ALIGN
    assert ps(FAKE, bnn.F16, 4, 64, FAKE, bnn.F32, 1, 2.0, FAKE, FAKE + 4, FAKE, need, None) == bnn.ERR_ALIGN
    small = L.bnn_pack_sign_shift_abs_mean_workspace_bytes(4, 64)
    assert ps(FAKE, bnn.F16, 4, 64, FAKE, bnn.F32, 1, 2.0, FAKE, FAKE, FAKE, small - 1, None) == bnn.ERR_WORKSPACE
    assert ps(FAKE, bnn.F16, 4, 64, FAKE, bnn.F32, 1, 2.0, FAKE, FAKE, None, small, None) == bnn.ERR_WORKSPACE
    need = L.bnn_pack_sign_nchw_shift_abs_mean_workspace_bytes(bnn.F16, 128, 128, 28, 28)
    assert need >= L.bnn_abs_mean_workspace_bytes(128 * 128 * 28 * 28) and need % 8 == 0
    assert L.bnn_pack_sign_nchw_shift_abs_mean_workspace_bytes(bnn.I32, 1, 32, 4, 4) == 0
    pn = L.bnn_pack_sign_nchw_shift_abs_mean
    assert pn(FAKE, bnn.F16, 0, 32, 4, 4, FAKE, bnn.F16, 2.0, FAKE, FAKE, FAKE, need, None) == bnn.ERR_SHAPE
    assert pn(FAKE, bnn.F16, 1, 32, 4, 4, FAKE, 7, 2.0, FAKE, FAKE, FAKE, need, None) == bnn.ERR_DTYPE
    assert pn(FAKE, bnn.F16, 1, 32, 4, 4, FAKE, bnn.F16, 2.0, None, FAKE, FAKE, need, None) == bnn.ERR_NULL
    assert pn(FAKE + 8, bnn.F16, 1, 32, 4, 4, FAKE, bnn.F16, 2.0, FAKE, FAKE, FAKE, need, None) == bnn.ERR_ALIGN
    assert pn(FAKE, bnn.F16, 1, 32, 4, 4, FAKE, bnn.F16, 2.0, FAKE, FAKE, FAKE, 0, None) == bnn.ERR_WORKSPACE


def test_shift_kernels_keep_subnormals():
    """The shifted sign adds in fp32 and relies on subnormal results being kept: every kernel of
    the packing code object must run with the fp32 denormal mode 'preserve' (3) in its kernel
    descriptor (the descriptor sets the mode at dispatch, whatever the caller's state)."""
    import subprocess
    import sys
    import tempfile
    sys.path.insert(0, os.path.join(ROOT, "convolution_bnn_pack_amd"))
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_bnn_build", os.path.join(ROOT, "convolution_bnn_pack_amd", "_build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    with tempfile.TemporaryDirectory() as td:
        asm = os.path.join(td, "pack.s")
        r = subprocess.run([build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S",
                            os.path.join(build.CSRC, "pack.hip"), "-o", asm],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        text = open(asm).read()
    modes = re.findall(r"\.amdhsa_float_denorm_mode_32\s+(\d+)", text)
    kernels = re.findall(r"\.amdhsa_kernel\s+(\S+)", text)
    assert any("pack_rows_shift_kernel" in k for k in kernels)
    assert len(modes) == len(kernels) and set(modes) == {"3"}


def test_workspace_queries(bnn):
    L = bnn.lib
    assert L.bnn_gemm_workspace_bytes(2048, 4096, bnn.F16) == 2048 * 128 * 4
    assert L.bnn_gemm_workspace_bytes(2048, 4096, bnn.U32_PACKED) == 0
    assert L.bnn_conv2d_workspace_bytes(32, 256, 14, 14, bnn.F32) == 32 * 14 * 14 * 8 * 4
    assert L.bnn_conv2d_workspace_bytes(32, 256, 14, 14, bnn.U32_PACKED) == 0
    # partial last words: ceil(k / 32) words per row, ceil(c / 32) per pixel
    assert L.bnn_gemm_workspace_bytes(3, 33, bnn.F32) == 3 * 2 * 4
    assert L.bnn_conv2d_workspace_bytes(2, 40, 5, 5, bnn.F16) == 2 * 5 * 5 * 2 * 4


def test_last_path_starts_unset(bnn):
    assert bnn.lib.bnn_last_path() in (0, bnn.PATH_XOR, bnn.PATH_MFMA, bnn.PATH_MFMA_FP4)


def test_auto_path_choices(bnn):
    for m, n, k in [(64, 256, 512), (2048, 4096, 4096), (16384, 8192, 8192), (1, 1, 1 << 24)]:
        assert bnn.gemm_auto_path(m, n, k) == bnn.PATH_MFMA_FP4
    assert bnn.gemm_auto_path(64, 64, (1 << 24) + 32) == bnn.PATH_MFMA            # fp4 sums inexact
    assert bnn.conv2d_auto_path(1, 32, 20, 20, 8, 9, 1, 4, 1) == bnn.PATH_MFMA_FP4   # 81 taps
    assert bnn.conv2d_auto_path(1, 1 << 21, 4, 4, 8, 3, 1, 1, 1) == bnn.PATH_MFMA     # K = 9 * 2^21 > 2^24


def test_backward_argument_checks(bnn):
    L = bnn.lib

    def gi(**kw):
        a = dict(g=FAKE, w=FAKE, x=FAKE, dt=bnn.BF16, m=64, n=64, k=128, sa=1.0, sw=1.0, out=FAKE,
                 gsa=FAKE, ws=FAKE, wsb=1 << 20)
        a.update(kw)
        return L.bnn_linear_grad_input(a["g"], a["w"], a["x"], a["dt"], a["m"], a["n"], a["k"], a["sa"],
                                       a["sw"], a["out"], a["gsa"], a["ws"], a["wsb"], None)
    assert L.bnn_linear_grad_input_workspace_bytes(300, 130) == 3 * 2 * 8   # one double per 128x128 tile
    assert L.bnn_linear_grad_input_workspace_bytes(0, 130) == 0
    assert gi(dt=bnn.F32) == bnn.ERR_DTYPE and gi(dt=bnn.I32) == bnn.ERR_DTYPE
    assert gi(m=0) == bnn.ERR_SHAPE and gi(k=0) == bnn.ERR_SHAPE   # the page divides by sqrt(m * k)
    assert gi(n=60) == bnn.ERR_SHAPE and gi(k=100) == bnn.ERR_SHAPE and gi(n=-8) == bnn.ERR_SHAPE
    assert gi(m=1 << 20, k=1 << 12) == bnn.ERR_SHAPE
    assert gi(x=None) == bnn.ERR_NULL and gi(g=None) == bnn.ERR_NULL and gi(gsa=None) == bnn.ERR_NULL
    assert gi(g=FAKE + 8) == bnn.ERR_ALIGN and gi(w=FAKE + 2) == bnn.ERR_ALIGN
    assert gi(out=FAKE + 2) == bnn.ERR_ALIGN and gi(gsa=FAKE + 4) == bnn.ERR_ALIGN
    assert gi(ws=None) == bnn.ERR_WORKSPACE and gi(wsb=7) == bnn.ERR_WORKSPACE
    assert gi(ws=FAKE + 4) == bnn.ERR_ALIGN

    def gw(**kw):
        a = dict(g=FAKE, x=FAKE, dt=bnn.F16, m=64, n=64, k=128, sa=1.0, out=FAKE)
        a.update(kw)
        return L.bnn_linear_grad_weight(a["g"], a["x"], a["dt"], a["m"], a["n"], a["k"], a["sa"], a["out"], None)
    assert gw(dt=bnn.F32) == bnn.ERR_DTYPE
    assert gw(n=12) == bnn.ERR_SHAPE and gw(k=4) == bnn.ERR_SHAPE and gw(m=-1) == bnn.ERR_SHAPE
    assert gw(out=None) == bnn.ERR_NULL and gw(x=None) == bnn.ERR_NULL
    assert gw(g=FAKE + 2) == bnn.ERR_ALIGN and gw(out=FAKE + 1) == bnn.ERR_ALIGN
    assert gw(n=0, g=None, x=None, out=None) == bnn.OK and gw(k=0, out=None) == bnn.OK


def test_backward_i8_argument_checks(bnn):
    L = bnn.lib

    def gq(**kw):
        a = dict(g=FAKE, x=FAKE, dt=bnn.BF16, m=64, n=64, k=128, sa=1.0, out=FAKE, q=FAKE, amax=FAKE,
                 ws=FAKE, wsb=1 << 20)
        a.update(kw)
        return L.bnn_linear_grad_weight_i8(a["g"], a["x"], a["dt"], a["m"], a["n"], a["k"], a["sa"], a["out"],
                                           a["q"], a["amax"], a["ws"], a["wsb"], None)
    assert L.bnn_linear_grad_weight_i8_workspace_bytes(64, 128) == 2 * 4      # 2048 vectors, 1024 a part
    assert L.bnn_linear_grad_weight_i8_workspace_bytes(8192, 8192) == 1024 * 4
    assert L.bnn_linear_grad_weight_i8_workspace_bytes(0, 128) == 0
    assert gq(dt=bnn.F32) == bnn.ERR_DTYPE
    assert gq(n=12) == bnn.ERR_SHAPE and gq(k=4) == bnn.ERR_SHAPE
    assert gq(q=None) == bnn.ERR_NULL and gq(amax=None) == bnn.ERR_NULL and gq(out=None) == bnn.ERR_NULL
    assert gq(out=FAKE + 4) == bnn.ERR_ALIGN and gq(q=FAKE + 2) == bnn.ERR_ALIGN and gq(amax=FAKE + 2) == bnn.ERR_ALIGN
    assert gq(ws=None) == bnn.ERR_WORKSPACE and gq(wsb=3) == bnn.ERR_WORKSPACE
    assert gq(n=0, g=None, x=None, out=None, q=None, amax=None) == bnn.OK


def test_quant_grad_argument_checks(bnn):
    L = bnn.lib
    assert L.bnn_quant_grad_i8_workspace_bytes(0) == 0 and L.bnn_quant_grad_i8_workspace_bytes(4) == 4
    assert L.bnn_quant_grad_i8(FAKE, 6, FAKE, FAKE, FAKE, 1 << 20, None) == bnn.ERR_SHAPE
    assert L.bnn_quant_grad_i8(FAKE, -4, FAKE, FAKE, FAKE, 1 << 20, None) == bnn.ERR_SHAPE
    assert L.bnn_quant_grad_i8(None, 0, None, None, None, 0, None) == bnn.OK
    assert L.bnn_quant_grad_i8(None, 8, FAKE, FAKE, FAKE, 1 << 20, None) == bnn.ERR_NULL
    assert L.bnn_quant_grad_i8(FAKE + 4, 8, FAKE, FAKE, FAKE, 1 << 20, None) == bnn.ERR_ALIGN
    assert L.bnn_quant_grad_i8(FAKE, 8, FAKE, FAKE, None, 0, None) == bnn.ERR_WORKSPACE
