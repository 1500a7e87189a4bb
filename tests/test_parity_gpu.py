"""GPU parity: libbnn (through its C ABI) against the CPU oracle.

Integer results (packed words, int32 accumulators) must be bit-exact. Scaled
outputs: float32 within 1e-6 relative of y = acc * (scale_a * scale_w)
computed in double by the oracle (exactly 0 where acc is 0); float16 and
bfloat16 within one unit in the last place of the output type at y. The
kernel's own error is float32 rounding of acc * alpha (<= 2^-23 relative)
followed by one round-to-nearest-even to the output type.
"""
import math

import numpy as np
import pytest
import torch

import synth
from parity_check import check_scaled

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PATHS = ["xor", "mfma", "mfma_fp4", "auto"]
EXPLICIT = ["xor", "mfma", "mfma_fp4"]


@pytest.fixture(scope="module")
def bnn():
    import convolution_bnn_pack_amd as m
    return m


@pytest.fixture(scope="module")
def orc(oracle_lib):
    return oracle_lib


def _say(msg):
    print(msg, flush=True)


# ----------------------------------------------------------------------------- packing

@pytest.mark.parametrize("tdt", [torch.float32, torch.float16, torch.bfloat16])
def test_pack_rows_bit_exact(bnn, orc, tdt):
    g = torch.Generator().manual_seed(21)
    for rows, k in [(1, 32), (3, 64), (17, 96), (64, 512), (5, 4096), (333, 1024), (1000, 32)]:
        x = synth.inject_edges(torch.randn((rows, k), generator=g).to(tdt), rows * 7 + k, max(1, rows * k // 20))
        _say(f"pack_rows {tdt} {rows}x{k}")
        got = bnn.pack_sign(x.to(DEV)).cpu()
        assert torch.equal(got, orc.pack_rows(x)), (rows, k)


@pytest.mark.parametrize("tdt", [torch.float32, torch.float16, torch.bfloat16])
def test_pack_nchw_bit_exact(bnn, orc, tdt):
    g = torch.Generator().manual_seed(22)
    # 16-byte vector path (pixel planes a multiple of 8) with partly filled last words, more
    # than eight words per pixel (two passes of the slab kernel) and many pixel chunks
    for shape in [(1, 32, 1, 1), (2, 64, 5, 3), (3, 96, 7, 9), (2, 256, 14, 14), (1, 128, 28, 28),
                  (2, 32, 4, 4), (1, 64, 3, 8), (3, 40, 4, 8), (2, 300, 2, 8), (1, 520, 4, 4),
                  (5, 8, 8, 8), (9, 128, 12, 12), (2, 200, 8, 6)]:
        x = synth.inject_edges(torch.randn(shape, generator=g).to(tdt), sum(shape), max(1, math.prod(shape) // 20))
        _say(f"pack_nchw {tdt} {shape}")
        got = bnn.pack_sign_nchw(x.to(DEV)).cpu()
        assert torch.equal(got, orc.pack_nchw(x)), shape


def test_w_pack_bit_exact(bnn, orc):
    g = torch.Generator().manual_seed(23)
    for tdt in (torch.float32, torch.float16, torch.bfloat16):
        w = synth.inject_edges(torch.randn((70, 160), generator=g).to(tdt), 1, 300)
        assert torch.equal(bnn.w_pack(w.to(DEV)).cpu(), orc.pack_rows(w))
        for ks in (1, 3, 5):
            wc = synth.inject_edges(torch.randn((37, 64, ks, ks), generator=g).to(tdt), ks, 300)
            assert torch.equal(bnn.w_pack(wc.to(DEV)).cpu(), orc.pack_conv_weight(wc)), (tdt, ks)


def test_pack_rows_large_stream(bnn, orc):
    # the activation of the large linear workload is 16384 x 8192 bf16; check a slice of rows
    # of the same width plus a ragged word count through the flat stream
    x = torch.randn((2049, 8192), generator=torch.Generator().manual_seed(24)).bfloat16()
    got = bnn.pack_sign(x.to(DEV)).cpu()
    assert torch.equal(got, orc.pack_rows(x))


# ----------------------------------------------------------------------------- workloads

LINEAR = ["linear_64x256x512_f32", "linear_2048x4096x4096_f16"]
CONV = ["conv_resnet18_s3_f32", "conv_down_s2_f16", "conv_dil2_f16"]


@pytest.mark.parametrize("name", LINEAR)
def test_linear_workload(bnn, orc, name):
    wl = synth.WORKLOADS[name]
    x, w, sa, sw = synth.make_inputs(wl)
    acc = orc.linear_acc(x, w)
    y = orc.scale(acc, sa, sw)
    xd, wp = x.to(DEV), bnn.w_pack(w.to(DEV))
    for path in PATHS:
        _say(f"{name} path={path}")
        got = bnn.gemm(xd, wp, sa, sw, path=path, out_dtype=torch.int32)
        assert torch.equal(got.cpu(), acc), f"{name} {path}: accumulators differ"
        out = bnn.gemm(xd, wp, sa, sw, path=path, out_dtype=getattr(torch, {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}[wl.out_dtype]))
        check_scaled(out, acc, y, f"{name} {path}")
        # pre-packed activations give the same result
        xp = bnn.pack_sign(xd)
        got2 = bnn.gemm(xp, wp, sa, sw, path=path, out_dtype=torch.int32, k=wl.k)
        assert torch.equal(got2.cpu(), acc)
    if name == "linear_64x256x512_f32":
        out = bnn.gemm(xd, wp, sa, sw)                      # scale product 0.125 is dyadic: exact
        assert torch.equal(out.cpu().double(), y)


@pytest.mark.parametrize("name", CONV)
def test_conv_workload(bnn, orc, name):
    wl = synth.WORKLOADS[name]
    x, w, sa, sw = synth.make_inputs(wl)
    acc = orc.conv2d_acc(x, w, wl.stride, wl.padding, wl.dilation)
    y = orc.scale(acc, sa, sw)
    kv = orc.conv2d_kvalid(wl.c, wl.h, wl.w, wl.ks, wl.stride, wl.padding, wl.dilation)
    assert bool(((acc - kv) % 2 == 0).all()) and bool((acc.abs() <= kv).all())
    xd, wp = x.to(DEV), bnn.w_pack(w.to(DEV))
    out_t = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[wl.out_dtype]
    for path in PATHS:
        _say(f"{name} path={path}")
        got = bnn.conv2d(xd, wp, sa, sw, wl.ks, wl.stride, wl.padding, wl.dilation, path=path,
                         out_dtype=torch.int32)
        assert torch.equal(got.cpu(), acc), f"{name} {path}: accumulators differ"
        out = bnn.conv2d(xd, wp, sa, sw, wl.ks, wl.stride, wl.padding, wl.dilation, path=path,
                         out_dtype=out_t)
        check_scaled(out, acc, y, f"{name} {path}")
        xp = bnn.pack_sign_nchw(xd)
        got2 = bnn.conv2d(xp, wp, sa, sw, wl.ks, wl.stride, wl.padding, wl.dilation, path=path,
                          out_dtype=torch.int32)
        assert torch.equal(got2.cpu(), acc)


def test_large_linear_full(bnn, orc):
    """16384 x 8192 x 8192, bf16 activations packed on the fly, f32 out, in the launch
    configuration the benchmark uses: every int32 accumulator of every path against the
    oracle (about 2.2e12 binary ops of host work, ~10 s on 16 cores), and every scaled f32
    output against the parity bar."""
    wl = synth.WORKLOADS["linear_16384x8192x8192_bf16"]
    x, w, sa, sw = synth.make_inputs(wl)
    _say("large linear: oracle over all rows")
    acc = orc.linear_acc(x, w)
    y = orc.scale(acc, sa, sw)
    assert bool(((acc - wl.k) % 2 == 0).all()) and bool((acc.abs() <= wl.k).all())
    xd, wp = x.to(DEV), bnn.w_pack(w.to(DEV))
    del w
    for path in ("mfma_fp4", "mfma", "xor", "auto"):
        _say(f"large linear path={path}")
        got = bnn.gemm(xd, wp, sa, sw, path=path, out_dtype=torch.int32)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), acc), f"large linear {path}: accumulators differ"
        del got
        out = bnn.gemm(xd, wp, sa, sw, path=path, out_dtype=torch.float32)
        check_scaled(out, acc, y, f"large linear {path}")
        del out
    assert bnn.gemm_auto_path(wl.m, wl.n, wl.k) == bnn.PATH_MFMA_FP4


def test_tile_variants_full(bnn, orc):
    """Shapes that select the matrix-core kernel's less common tiles, every output against the
    oracle: the 256 x 64 fp4 tile (at most 64 output features and a full round of such
    tiles), and the fp4 fallback from 256 x 256 to 128 x 256 tiles when K/32 is not a multiple
    of 4 (no vector loads); a 64-channel 3x3 conv with 24 images of 56 x 56."""
    g = torch.Generator().manual_seed(61)
    cases = [(65600, 40, 288), (66000, 64, 1024), (4096, 4096, 4128)]
    for m, n, k in cases:
        x = torch.randn((m, k), generator=g).half()
        w = torch.randn((n, k), generator=g).half()
        acc = orc.linear_acc(x, w)
        xd, wp = x.to(DEV), bnn.w_pack(w.to(DEV))
        for path in ("mfma_fp4", "mfma"):
            _say(f"tile variant linear {m}x{n}x{k} path={path}")
            got = bnn.gemm(xd, wp, 1.0, 1.0, path=path, out_dtype=torch.int32)
            torch.cuda.synchronize()
            assert torch.equal(got.cpu(), acc), (m, n, k, path)
            del got
    # 64-channel 3x3 conv on 56x56 with 24 images: 75264 output pixels, 64 output channels
    xc = torch.randn((24, 64, 56, 56), generator=g).half()
    wc = torch.randn((64, 64, 3, 3), generator=g).half()
    acc = orc.conv2d_acc(xc, wc, 1, 1, 1)
    xcd, wpc = xc.to(DEV), bnn.w_pack(wc.to(DEV))
    for path in ("mfma_fp4", "mfma", "xor"):
        _say(f"tile variant conv 24x64x56x56 path={path}")
        got = bnn.conv2d(xcd, wpc, 1.0, 1.0, 3, 1, 1, 1, path=path, out_dtype=torch.int32)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), acc), path


def test_banded_tile_order(bnn, orc):
    """Linear grids of 1024 or more tiles walk bands of four m-tiles: 37 x 28 tiles of 256 x 256
    (a last band of one m-tile; the count is not a multiple of 8, so no per-XCD runs) and, with
    K = 96 (three words, no vector loads: 128 x 256 tiles), 66 x 32 tiles with ragged M and N (a
    last band of two m-tiles, per-XCD runs); every accumulator against the oracle, so a tile
    visited twice or never fails."""
    g = torch.Generator().manual_seed(67)
    for m, n, k in [(37 * 256, 28 * 256, 128), (32 * 256 + 100, 31 * 256 + 40, 96)]:
        x = torch.randn((m, k), generator=g).half()
        w = torch.randn((n, k), generator=g).half()
        acc = orc.linear_acc(x, w)
        xd, wp = x.to(DEV), bnn.w_pack(w.to(DEV))
        _say(f"banded tile order {m}x{n}x{k}")
        got = bnn.gemm(xd, wp, 1.0, 1.0, path="mfma_fp4", out_dtype=torch.int32)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), acc), (m, n, k)
        del got


def test_persistent_conv_tiles(bnn, orc):
    """Conv shapes with more fp4 128 x 256 tiles than the GPU holds at once, which run as
    persistent workgroups streaming several tiles each (tile boundaries at every stage
    count, ragged last tile, planes whose size is not a multiple of 4): full oracle check."""
    g = torch.Generator().manual_seed(71)
    cases = [(48, 32, 27, 27, 256, 3, 1, 1, 1),    # 2 stages per tile, 274 tiles, HW = 729
             (64, 32, 24, 24, 256, 1, 1, 0, 1),    # 1 stage per tile, 288 tiles
             (40, 64, 30, 30, 200, 3, 1, 1, 1)]    # 3 stages, ragged N, 282 tiles
    for (b, c, h, w, o, ks, st, pd, dl) in cases:
        x = torch.randn((b, c, h, w), generator=g).half()
        wt = torch.randn((o, c, ks, ks), generator=g).half()
        acc = orc.conv2d_acc(x, wt, st, pd, dl)
        y = orc.scale(acc, 0.75, 0.5)
        xd, wp = x.to(DEV), bnn.w_pack(wt.to(DEV))
        _say(f"persistent conv {b}x{c}x{h}x{w} -> {o}, k{ks}")
        got = bnn.conv2d(xd, wp, 0.75, 0.5, ks, st, pd, dl, path="mfma_fp4", out_dtype=torch.int32)
        assert torch.equal(got.cpu(), acc), (b, c, h, w, o, ks)
        out = bnn.conv2d(xd, wp, 0.75, 0.5, ks, st, pd, dl, path="mfma_fp4", out_dtype=torch.float16)
        check_scaled(out, acc, y, f"persistent conv {b}x{c}x{h}x{w}")


def test_two_round_conv_tiles(bnn, orc):
    """Conv shapes with two or more rounds of fp4 128 x 256 tiles, which run as 128 x 128 tiles of
    four waves with 4-word stages, three workgroups per compute unit (ragged last tile, ragged N,
    planes whose size is not a multiple of 4 or 8): full oracle check."""
    g = torch.Generator().manual_seed(73)
    cases = [(88, 32, 28, 28, 256, 3, 1, 1, 1),    # 539 row tiles, planes of 784
             (96, 32, 27, 27, 200, 3, 1, 1, 1),    # 547 row tiles, ragged N, planes of 729
             (84, 64, 28, 28, 136, 3, 1, 2, 2)]    # dilated, 515 row tiles
    for (b, c, h, w, o, ks, st, pd, dl) in cases:
        x = torch.randn((b, c, h, w), generator=g).half()
        wt = torch.randn((o, c, ks, ks), generator=g).half()
        acc = orc.conv2d_acc(x, wt, st, pd, dl)
        y = orc.scale(acc, 0.75, 0.5)
        xd, wp = x.to(DEV), bnn.w_pack(wt.to(DEV))
        _say(f"two-round conv {b}x{c}x{h}x{w} -> {o}, k{ks} d{dl}")
        got = bnn.conv2d(xd, wp, 0.75, 0.5, ks, st, pd, dl, path="mfma_fp4", out_dtype=torch.int32)
        assert torch.equal(got.cpu(), acc), (b, c, h, w, o, ks)
        for odt in (torch.float16, torch.float32):
            out = bnn.conv2d(xd, wp, 0.75, 0.5, ks, st, pd, dl, path="mfma_fp4", out_dtype=odt)
            check_scaled(out, acc, y, f"two-round conv {b}x{c}x{h}x{w} {odt}")


# ----------------------------------------------------------------------------- sweeps and edges

def test_random_linear_sweep(bnn, orc):
    for seed in range(40):
        c = synth.random_linear_case(1000 + seed)
        acc = orc.linear_acc(c["x"], c["w"])
        y = orc.scale(acc, c["scale_a"], c["scale_w"])
        xd, wp = c["x"].to(DEV), bnn.w_pack(c["w"].to(DEV))
        out_t = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[c["out_dtype"]]
        for path in PATHS:
            got = bnn.gemm(xd, wp, c["scale_a"], c["scale_w"], path=path, out_dtype=torch.int32)
            assert torch.equal(got.cpu(), acc), (seed, path, c["m"], c["n"], c["k"])
            out = bnn.gemm(xd, wp, c["scale_a"], c["scale_w"], path=path, out_dtype=out_t)
            check_scaled(out, acc, y, f"linear sweep seed {seed} {path}")


def test_random_conv_sweep(bnn, orc):
    for seed in range(40):
        c = synth.random_conv_case(2000 + seed)
        acc = orc.conv2d_acc(c["x"], c["w_"], c["stride"], c["padding"], c["dilation"])
        y = orc.scale(acc, c["scale_a"], c["scale_w"])
        xd, wp = c["x"].to(DEV), bnn.w_pack(c["w_"].to(DEV))
        out_t = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[c["out_dtype"]]
        for path in PATHS:
            args = (c["scale_a"], c["scale_w"], c["ks"], c["stride"], c["padding"], c["dilation"])
            got = bnn.conv2d(xd, wp, *args, path=path, out_dtype=torch.int32)
            key = (seed, path, tuple(c["x"].shape), c["o"], c["ks"], c["stride"], c["padding"], c["dilation"])
            assert torch.equal(got.cpu(), acc), key
            out = bnn.conv2d(xd, wp, *args, path=path, out_dtype=out_t)
            check_scaled(out, acc, y, f"conv sweep {key}")


def test_edge_values_in_both_operands(bnn, orc):
    g = torch.Generator().manual_seed(31)
    for tdt in (torch.float32, torch.float16, torch.bfloat16):
        x = synth.inject_edges(torch.randn((67, 320), generator=g).to(tdt), 1, 2000)
        w = synth.inject_edges(torch.randn((45, 320), generator=g).to(tdt), 2, 2000)
        acc = orc.linear_acc(x, w)
        wp = bnn.w_pack(w.to(DEV))
        for path in EXPLICIT:
            assert torch.equal(bnn.gemm(x.to(DEV), wp, 1.0, 1.0, path=path, out_dtype=torch.int32).cpu(), acc)
        xc = synth.inject_edges(torch.randn((2, 64, 6, 5), generator=g).to(tdt), 3, 300)
        wc = synth.inject_edges(torch.randn((9, 64, 3, 3), generator=g).to(tdt), 4, 300)
        accc = orc.conv2d_acc(xc, wc, 1, 1, 1)
        wpc = bnn.w_pack(wc.to(DEV))
        for path in EXPLICIT:
            got = bnn.conv2d(xc.to(DEV), wpc, 1.0, 1.0, 3, 1, 1, 1, path=path, out_dtype=torch.int32)
            assert torch.equal(got.cpu(), accc)


def test_closed_form_padding_map(bnn, orc):
    # all +1 activations and weights: every output equals its number of real taps
    for (h, s, p, d) in [(14, 1, 1, 1), (28, 2, 1, 1), (28, 1, 2, 2), (5, 3, 3, 2)]:
        x = torch.ones((2, 64, h, h), device=DEV)
        wp = bnn.w_pack(torch.ones((8, 64, 3, 3), device=DEV))
        kv = orc.conv2d_kvalid(64, h, h, 3, s, p, d)
        for path in EXPLICIT:
            got = bnn.conv2d(x, wp, 1.0, 1.0, 3, s, p, d, path=path, out_dtype=torch.int32).cpu()
            assert torch.equal(got, kv.expand_as(got)), (h, s, p, d, path)
            neg = bnn.conv2d(x, bnn.w_pack(-torch.ones((8, 64, 3, 3), device=DEV)), 1.0, 1.0, 3, s, p,
                             d, path=path, out_dtype=torch.int32).cpu()
            assert torch.equal(neg, -kv.expand_as(neg))


def test_determinism_and_paths_agree(bnn):
    g = torch.Generator().manual_seed(41)
    x = torch.randn((1000, 1024), generator=g).half().to(DEV)
    wp = bnn.w_pack(torch.randn((777, 1024), generator=g).half().to(DEV))
    a = bnn.gemm(x, wp, 1.0, 1.0, path="xor", out_dtype=torch.int32)
    b = bnn.gemm(x, wp, 1.0, 1.0, path="mfma", out_dtype=torch.int32)
    c = bnn.gemm(x, wp, 1.0, 1.0, path="mfma_fp4", out_dtype=torch.int32)
    assert torch.equal(a, b) and torch.equal(a, c)
    for _ in range(3):
        assert torch.equal(bnn.gemm(x, wp, 1.0, 1.0, path="mfma", out_dtype=torch.int32), b)
        assert torch.equal(bnn.gemm(x, wp, 1.0, 1.0, path="mfma_fp4", out_dtype=torch.int32), c)
        assert torch.equal(bnn.gemm(x, wp, 1.0, 1.0, path="xor", out_dtype=torch.int32), a)


def test_last_path_and_errors_on_device(bnn):
    x = torch.randn((64, 64), device=DEV)
    wp = bnn.w_pack(torch.randn((32, 64), device=DEV))
    bnn.gemm(x, wp, 1.0, 1.0, path="mfma")
    assert bnn.last_path() == bnn.PATH_MFMA
    bnn.gemm(x, wp, 1.0, 1.0, path="xor")
    assert bnn.last_path() == bnn.PATH_XOR
    bnn.gemm(x, wp, 1.0, 1.0, path="mfma_fp4")
    assert bnn.last_path() == bnn.PATH_MFMA_FP4
    # a too-small workspace is rejected and the output is left untouched
    out = torch.full((64, 32), 7.0, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(bnn.BnnError) as e:
        bnn.gemm(x, wp, 1.0, 1.0, out=out, workspace=ws)
    assert e.value.status == bnn.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    # an empty reduction is a shape error (the layers' AssertionError)
    with pytest.raises(AssertionError):
        bnn.pack_sign(torch.randn((4, 0), device=DEV))
    # a view that is element-aligned but not 16-byte aligned is packed by the element-wise kernel
    buf = torch.randn((65 * 64,), device=DEV)
    view = buf[1:1 + 64 * 64].view(64, 64)
    assert torch.equal(bnn.pack_sign(view), bnn.pack_sign(view.clone()))
    # an output that is not 16-byte aligned is rejected with ERR_ALIGN, nothing written
    obuf = torch.full((64 * 32 + 1,), 7.0, device=DEV)
    with pytest.raises(bnn.BnnError) as e:
        bnn.gemm(x, wp, 1.0, 1.0, out=obuf[1:].view(64, 32))
    assert e.value.status == bnn.ERR_ALIGN
    torch.cuda.synchronize()
    assert bool((obuf == 7.0).all())


def test_graph_replay_matches_eager(bnn):
    """The benchmark times HIP-graph replays of the step; every replay must equal the eager
    result, with other eager work and synchronizations between replays."""
    g = torch.Generator().manual_seed(51)
    x = torch.randn((700, 1024), generator=g).half().to(DEV)
    wp = bnn.w_pack(torch.randn((520, 1024), generator=g).half().to(DEV))
    xc = torch.randn((2, 64, 11, 13), generator=g).to(DEV)
    wpc = bnn.w_pack(torch.randn((48, 64, 3, 3), generator=g).to(DEV))
    for path in EXPLICIT:
        eager = bnn.gemm(x, wp, 0.3, 0.7, path=path)
        eager_c = bnn.conv2d(xc, wpc, 0.3, 0.7, 3, 2, 1, 1, path=path)
        xp = torch.empty((700, 32), dtype=torch.int32, device=DEV)
        xpc = torch.empty((2, 11, 13, 2), dtype=torch.int32, device=DEV)
        out = torch.empty_like(eager)
        out_c = torch.empty_like(eager_c)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            bnn.pack_sign(x, out=xp)
            bnn.gemm(xp, wp, 0.3, 0.7, path=path, out=out, k=1024)
            bnn.pack_sign_nchw(xc, out=xpc)
            bnn.conv2d(xpc, wpc, 0.3, 0.7, 3, 2, 1, 1, path=path, out=out_c)
        for r in range(4):
            out.fill_(-1.0)
            out_c.fill_(-1.0)
            bnn.gemm(x[:64].contiguous(), wp, 1.0, 1.0, path=path)   # unrelated eager work
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), (path, r)
            assert torch.equal(out_c, eager_c), (path, r)


@pytest.mark.parametrize("tdt", [torch.float32, torch.float16, torch.bfloat16])
def test_nchw_input_aligned_to_element_only(bnn, orc, tdt):
    """A float NCHW tensor that is only element-aligned (a view that starts one element into its
    buffer) packs through the element-wise kernel and convolves like an aligned copy."""
    g = torch.Generator().manual_seed(29)
    shape = (2, 40, 8, 8)                                # planes a multiple of the vector width
    x = synth.inject_edges(torch.randn(shape, generator=g).to(tdt), 29, 200)
    buf = torch.empty(x.numel() + 1, dtype=tdt, device=DEV)
    xd = buf[1:].view(shape)
    xd.copy_(x.to(DEV))
    assert xd.data_ptr() % 16 != 0
    assert torch.equal(bnn.pack_sign_nchw(xd).cpu(), orc.pack_nchw(x))
    bias = synth.make_shift(40, "f32", 30)
    assert torch.equal(bnn.pack_sign_nchw_shift(xd, bias.to(DEV)).cpu(), orc.pack_nchw_shift(x, bias))
    w = torch.randn((24, 40, 3, 3), generator=g)
    wp = bnn.w_pack(w.to(DEV))
    want = orc.conv2d_acc(x, w, 1, 1, 1)
    for path in ("xor", "mfma", "mfma_fp4"):
        got = bnn.conv2d(xd, wp, 1.0, 1.0, 3, 1, 1, 1, path=path, out_dtype=torch.int32).cpu()
        assert torch.equal(got, want), path
