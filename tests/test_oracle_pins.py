"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test checks the oracle against something it does not compute itself:
hand-worked values (tests/golden), exhaustive brute force, a direct
definition written differently (nested loops with bounds checks), library
routines that reduce to the same result (torch fp64 conv2d / mm and torch's
own fp16/bf16 widening), closed forms and invariants.
"""
import json
import math
import os
import random

import numpy as np
import pytest
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(v):
    if isinstance(v, str):
        return {"-0": -0.0, "nan": float("nan"), "-inf": float("-inf"), "inf": float("inf")}[v]
    return float(v)


def _tensor(nested):
    arr = np.vectorize(_num, otypes=[np.float64])(np.array(nested, dtype=object))
    return torch.from_numpy(arr.astype(np.float32))


def _lib_sign(t):
    """Sign through torch's own widening to float32 and compare (a library routine)."""
    return torch.where(t.float() >= 0, 1.0, -1.0).double()


# ----------------------------------------------------------------------------- sign rule

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_sign_edge_values_golden(oracle_lib, dtype):
    table = _load("sign_edges.json")[dtype]
    if dtype == "f32":
        ints = [int(h, 16) for h, _ in table]
        t = torch.tensor([b - (1 << 32) if b >= 1 << 31 else b for b in ints], dtype=torch.int32)
        x = t.view(torch.float32)
    else:
        ints = [int(h, 16) for h, _ in table]
        t = torch.tensor([b - (1 << 16) if b >= 1 << 15 else b for b in ints], dtype=torch.int16)
        x = t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
    want = torch.tensor([s for _, s in table], dtype=torch.float32)
    assert torch.equal(oracle_lib.sign(x), want)


@pytest.mark.parametrize("tdt", [torch.float16, torch.bfloat16])
def test_sign_exhaustive_16bit_matches_library_widening(oracle_lib, tdt):
    allbits = torch.arange(-(1 << 15), 1 << 15, dtype=torch.int32).to(torch.int16)
    x = allbits.view(tdt).contiguous()
    assert torch.equal(oracle_lib.sign(x).double(), _lib_sign(x))


def test_sign_f32_random_bits_match_numpy(oracle_lib):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = torch.from_numpy(bits.view(np.float32).copy())
    want = np.where(bits.view(np.float32) >= 0, 1.0, -1.0)
    assert np.array_equal(oracle_lib.sign(x).numpy(), want)


# ----------------------------------------------------------------------------- hand-worked values

def test_linear_hand_worked(oracle_lib):
    g = _load("linear_hand.json")
    x, w = _tensor(g["x"]), _tensor(g["w"])
    acc = oracle_lib.linear_acc(x, w)
    assert acc.tolist() == g["acc"]
    y = oracle_lib.scale(acc, g["scale_a"], g["scale_w"])
    assert y.tolist() == g["y"]


def test_conv_hand_worked_checkerboard(oracle_lib):
    g = _load("conv_checkerboard.json")
    x, w = _tensor(g["x"]), _tensor(g["w"])
    acc = oracle_lib.conv2d_acc(x, w, g["stride"], g["padding"], g["dilation"])
    assert acc.tolist() == g["acc"]


def test_kvalid_hand_worked_maps(oracle_lib):
    for case in _load("kvalid_maps.json")["cases"]:
        kv = oracle_lib.conv2d_kvalid(1, case["h"], case["w"], case["ks"], case["stride"],
                                      case["padding"], case["dilation"])
        assert kv.tolist() == case["kvalid"], case
        # all-(+1) input and weights: every real tap adds exactly 1 (closed form)
        x = torch.ones((1, 1, case["h"], case["w"]))
        w = torch.ones((1, 1, case["ks"], case["ks"]))
        acc = oracle_lib.conv2d_acc(x, w, case["stride"], case["padding"], case["dilation"])
        assert acc[0, 0].tolist() == case["kvalid"]


def test_out_size_formula(oracle_lib):
    # hand values and torch's own conv output shape
    assert oracle_lib.conv_out_size(14, 3, 1, 1, 1) == 14
    assert oracle_lib.conv_out_size(28, 3, 2, 1, 1) == 14
    assert oracle_lib.conv_out_size(28, 3, 1, 2, 2) == 28
    assert oracle_lib.conv_out_size(2, 5, 1, 0, 1) == -2     # floor((2 - 4 - 1)/1 + 1): empty
    assert oracle_lib.conv_out_size(1, 3, 2, 0, 1) == 0      # floor((1 - 2 - 1)/2 + 1): true floor
    for h in range(1, 12):
        for ks in (1, 2, 3, 5):
            for s in (1, 2, 3):
                for p in range(0, 4):
                    for d in (1, 2, 3):
                        n = oracle_lib.conv_out_size(h, ks, s, p, d)
                        if n <= 0:
                            continue
                        shp = torch.nn.functional.conv2d(torch.zeros(1, 1, h, h), torch.zeros(1, 1, ks, ks),
                                                         stride=s, padding=p, dilation=d).shape
                        assert shp[-1] == n


# ----------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("k", list(range(1, 11)))
def test_linear_exhaustive_small_k(oracle_lib, k):
    """Every pair of +-1 vectors of length k: acc = k - 2*popcount(a xor b) (pattern bit 1 = +1)."""
    rng = np.random.default_rng(k)
    pats = np.arange(1 << k)
    bits = (pats[:, None] >> np.arange(k)[None, :]) & 1          # [2^k, k]
    mag = rng.uniform(0.01, 4.0, size=bits.shape)
    mag[rng.random(bits.shape) < 0.1] = 0.0                       # +0 is +1 too
    xs = np.where(bits == 1, mag, -np.maximum(mag, 1e-3))
    x = torch.from_numpy(xs.astype(np.float32))
    acc = oracle_lib.linear_acc(x, x).numpy().astype(np.int64)
    want = np.array([[k - 2 * bin(int(a) ^ int(b)).count("1") for b in pats] for a in pats])
    assert np.array_equal(acc, want)


def _direct_conv(xs, ws, s, p, d):
    """Direct definition with explicit bounds checks: sum over valid taps of sgn(x)*sgn(w)."""
    B, C, H, W = xs.shape
    O, _, K, _ = ws.shape
    Ho = math.floor((H + 2 * p - d * (K - 1) - 1) / s + 1)
    Wo = math.floor((W + 2 * p - d * (K - 1) - 1) / s + 1)
    out = np.zeros((B, O, Ho, Wo), dtype=np.int64)
    for b in range(B):
        for o in range(O):
            for oh in range(Ho):
                for ow in range(Wo):
                    tot = 0
                    for kh in range(K):
                        ih = oh * s - p + kh * d
                        if ih < 0 or ih >= H:
                            continue
                        for kw in range(K):
                            iw = ow * s - p + kw * d
                            if iw < 0 or iw >= W:
                                continue
                            tot += int(np.dot(xs[b, :, ih, iw], ws[o, :, kh, kw]))
                    out[b, o, oh, ow] = tot
    return out


def _tiny_conv_cases(count, seed):
    rnd = random.Random(seed)
    cases = []
    while len(cases) < count:
        b, c = rnd.choice([1, 2]), rnd.choice([1, 3, 32, 33])
        h, w = rnd.randint(1, 7), rnd.randint(1, 7)
        o, k = rnd.choice([1, 3]), rnd.choice([1, 2, 3, 5])
        s, p, d = rnd.choice([1, 2, 3]), rnd.randint(0, 3), rnd.choice([1, 2, 3])
        ho = math.floor((h + 2 * p - d * (k - 1) - 1) / s + 1)
        wo = math.floor((w + 2 * p - d * (k - 1) - 1) / s + 1)
        if ho > 0 and wo > 0:
            cases.append((b, c, h, w, o, k, s, p, d))
    return cases


def test_conv_matches_direct_definition(oracle_lib):
    g = torch.Generator().manual_seed(11)
    for (b, c, h, w, o, k, s, p, d) in _tiny_conv_cases(60, 3):
        x = torch.randn((b, c, h, w), generator=g)
        wt = torch.randn((o, c, k, k), generator=g)
        acc = oracle_lib.conv2d_acc(x, wt, s, p, d).numpy()
        want = _direct_conv(np.where(x.numpy() >= 0, 1, -1), np.where(wt.numpy() >= 0, 1, -1), s, p, d)
        assert np.array_equal(acc, want), (b, c, h, w, o, k, s, p, d)


# ----------------------------------------------------------------------------- library routines

def test_conv_matches_torch_fp64(oracle_lib):
    g = torch.Generator().manual_seed(12)
    for (b, c, h, w, o, k, s, p, d) in _tiny_conv_cases(300, 4):
        dt = [torch.float32, torch.float16, torch.bfloat16][(b + c + h) % 3]
        x = torch.randn((b, c, h, w), generator=g).to(dt)
        wt = torch.randn((o, c, k, k), generator=g).to(dt)
        acc = oracle_lib.conv2d_acc(x, wt, s, p, d)
        ref = torch.nn.functional.conv2d(_lib_sign(x), _lib_sign(wt), stride=s, padding=p, dilation=d)
        assert torch.equal(acc.double(), ref), (b, c, h, w, o, k, s, p, d)


def test_linear_matches_torch_fp64(oracle_lib):
    for seed in range(40):
        case = synth.random_linear_case(seed)
        acc = oracle_lib.linear_acc(case["x"], case["w"])
        ref = _lib_sign(case["x"]) @ _lib_sign(case["w"]).T
        assert torch.equal(acc.double(), ref)


# ----------------------------------------------------------------------------- packing

def _unpack(words, k):
    w = words.numpy().astype(np.uint32).astype(np.int64)
    bits = (w[..., :, None] >> np.arange(32)) & 1
    return bits.reshape(*w.shape[:-1], k)


@pytest.mark.parametrize("tdt", [torch.float32, torch.float16, torch.bfloat16])
def test_pack_rows_bits_are_signs(oracle_lib, tdt):
    x = synth.inject_edges(torch.randn((13, 96), generator=torch.Generator().manual_seed(1)).to(tdt), 5, 200)
    words = oracle_lib.pack_rows(x)
    assert words.shape == (13, 3)
    assert np.array_equal(_unpack(words, 96), (_lib_sign(x) > 0).numpy().astype(np.int64))


def test_pack_popcount_identity(oracle_lib):
    """acc = K - 2*popcount(a xor w) over the packed words (Python integers), vs the float-loop dot."""
    g = torch.Generator().manual_seed(2)
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        x = synth.inject_edges(torch.randn((9, 160), generator=g).to(dt), 3, 50)
        w = synth.inject_edges(torch.randn((7, 160), generator=g).to(dt), 4, 50)
        pa = oracle_lib.pack_rows(x).numpy().astype(np.uint32)
        pw = oracle_lib.pack_rows(w).numpy().astype(np.uint32)
        acc = oracle_lib.linear_acc(x, w).numpy()
        for m in range(9):
            for n in range(7):
                pop = sum(bin(int(a) ^ int(b)).count("1") for a, b in zip(pa[m], pw[n]))
                assert acc[m, n] == 160 - 2 * pop


def test_pack_nchw_layout(oracle_lib):
    x = torch.randn((2, 64, 5, 3), generator=torch.Generator().manual_seed(3)).half()
    got = oracle_lib.pack_nchw(x)
    want = oracle_lib.pack_rows(x.permute(0, 2, 3, 1).contiguous().reshape(-1, 64)).view(2, 5, 3, 2)
    assert torch.equal(got, want)
    bits = _unpack(got, 64)                                       # [b, h, w, c]
    assert np.array_equal(bits, (x.float().permute(0, 2, 3, 1) >= 0).numpy().astype(np.int64))


def test_pack_conv_weight_layout(oracle_lib):
    w = torch.randn((5, 96, 3, 3), generator=torch.Generator().manual_seed(4))
    got = oracle_lib.pack_conv_weight(w)
    assert got.shape == (5, 3, 3, 3)
    bits = _unpack(got, 96)                                       # [o, kh, kw, c]
    assert np.array_equal(bits, (w.permute(0, 2, 3, 1) >= 0).numpy().astype(np.int64))


# ----------------------------------------------------------------------------- invariants and closed forms

def test_linear_additivity_permutation_negation(oracle_lib):
    g = torch.Generator().manual_seed(5)
    x = torch.randn((11, 192), generator=g)
    w = torch.randn((13, 192), generator=g)
    full = oracle_lib.linear_acc(x, w)
    a = oracle_lib.linear_acc(x[:, :64].contiguous(), w[:, :64].contiguous())
    b = oracle_lib.linear_acc(x[:, 64:].contiguous(), w[:, 64:].contiguous())
    assert torch.equal(full, a + b)
    perm = torch.randperm(192, generator=g)
    assert torch.equal(full, oracle_lib.linear_acc(x[:, perm].contiguous(), w[:, perm].contiguous()))
    assert torch.equal(-full, oracle_lib.linear_acc(x, (-w).contiguous()))   # w has no zeros / NaNs


def test_linear_closed_forms(oracle_lib):
    k = 256
    alt = torch.tensor([1.0 if i % 2 == 0 else -1.0 for i in range(k)]).repeat(3, 1)
    assert torch.equal(oracle_lib.linear_acc(alt, torch.ones((4, k))), torch.zeros((3, 4), dtype=torch.int32))
    assert torch.equal(oracle_lib.linear_acc(torch.ones((3, k)), -torch.ones((2, k))),
                       torch.full((3, 2), -k, dtype=torch.int32))


def test_conv_closed_forms_all_ones(oracle_lib):
    # x = +1, W = +1 -> acc = K_valid; W = -1 -> -K_valid (3x3 s1 p1: corners 4C, edges 6C, interior 9C)
    c = 64
    x = torch.ones((1, c, 14, 14))
    acc = oracle_lib.conv2d_acc(x, torch.ones((2, c, 3, 3)), 1, 1, 1)
    kv = oracle_lib.conv2d_kvalid(c, 14, 14, 3, 1, 1, 1)
    assert torch.equal(acc[0, 0], kv) and torch.equal(acc[0, 1], kv)
    assert kv[0, 0] == 4 * c and kv[0, 5] == 6 * c and kv[5, 5] == 9 * c
    neg = oracle_lib.conv2d_acc(x, -torch.ones((1, c, 3, 3)), 1, 1, 1)
    assert torch.equal(neg[0, 0], -kv)


def test_selection_matches_full(oracle_lib):
    g = torch.Generator().manual_seed(6)
    x = torch.randn((20, 64), generator=g)
    w = torch.randn((9, 64), generator=g)
    full = oracle_lib.linear_acc(x, w)
    assert torch.equal(oracle_lib.linear_acc(x, w, rows=[19, 0, 7]), full[[19, 0, 7]])
    xc = torch.randn((4, 32, 6, 6), generator=g)
    wc = torch.randn((3, 32, 3, 3), generator=g)
    fullc = oracle_lib.conv2d_acc(xc, wc, 2, 1, 1)
    assert torch.equal(oracle_lib.conv2d_acc(xc, wc, 2, 1, 1, images=[3, 1]), fullc[[3, 1]])


CONFIG_NAMES = ["linear_64x256x512_f32", "linear_2048x4096x4096_f16", "conv_resnet18_s3_f32",
                "conv_down_s2_f16", "conv_dil2_f16"]


@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_workload_outputs_library_and_invariants(oracle_lib, name):
    wl = synth.WORKLOADS[name]
    x, w, sa, sw = synth.make_inputs(wl)
    if wl.kind == "linear":
        acc = oracle_lib.linear_acc(x, w)
        ref = _lib_sign(x) @ _lib_sign(w).T
        kv = torch.full(acc.shape, wl.k, dtype=torch.int32)
    else:
        acc = oracle_lib.conv2d_acc(x, w, wl.stride, wl.padding, wl.dilation)
        ref = torch.nn.functional.conv2d(_lib_sign(x), _lib_sign(w), stride=wl.stride,
                                         padding=wl.padding, dilation=wl.dilation)
        kv = oracle_lib.conv2d_kvalid(wl.c, wl.h, wl.w, wl.ks, wl.stride, wl.padding, wl.dilation)
        kv = kv.expand(acc.shape)
    assert tuple(acc.shape) == wl.out_shape()
    assert torch.equal(acc.double(), ref)
    assert torch.equal((acc - kv) % 2, torch.zeros_like(acc))         # parity of a sum of K_valid odd terms
    assert bool((acc.abs() <= kv).all())
    y = oracle_lib.scale(acc, sa, sw)
    assert torch.equal(y, acc.double() * (sa * sw))
    if name == "linear_64x256x512_f32":
        # scale_a * scale_w = 0.125 is dyadic: the float32 output is exact
        assert torch.equal(y.float().double(), y)


# ---------------------------------------------------------------- reduction tails (not whole words)

def _bits(words, n):
    w = words.numpy().astype(np.uint32).astype(np.int64)
    return ((w[..., None] >> np.arange(32)) & 1).reshape(*w.shape[:-1], -1)[..., :n], \
        ((w[..., None] >> np.arange(32)) & 1).reshape(*w.shape[:-1], -1)[..., n:]


@pytest.mark.parametrize("dt", [torch.float32, torch.float16, torch.bfloat16])
def test_pack_rows_tail_bits(oracle_lib, dt):
    """A row of k signs fills ceil(k/32) words; bits 0..k-1 follow torch's compare, the rest are 0,
    and the words equal the whole-word pack of the row padded with -1 (a plain value whose bit is 0)."""
    g = torch.Generator().manual_seed(61)
    for k in list(range(1, 70)) + [95, 96, 97, 1000]:
        x = synth.inject_edges(torch.randn((3, k), generator=g).to(dt), k, max(1, k // 7))
        words = oracle_lib.pack_rows(x)
        assert words.shape == (3, (k + 31) // 32)
        real, tail = _bits(words, k)
        assert np.array_equal(real, (x >= 0).numpy().astype(np.int64)), k
        assert not tail.any(), k
        kp = 32 * ((k + 31) // 32)
        padded = torch.cat([x, torch.full((3, kp - k), -1.0, dtype=dt)], dim=1).contiguous()
        assert torch.equal(words, oracle_lib.pack_rows(padded)), k


def test_pack_nchw_and_weight_tail_bits(oracle_lib):
    g = torch.Generator().manual_seed(62)
    for c in [1, 3, 17, 31, 33, 40, 63, 65, 100]:
        x = torch.randn((2, c, 3, 4), generator=g)
        words = oracle_lib.pack_nchw(x)                                   # [2, 3, 4, ceil(c/32)]
        real, tail = _bits(words, c)
        assert np.array_equal(real, (x >= 0).permute(0, 2, 3, 1).numpy().astype(np.int64)), c
        assert not tail.any()
        cp = 32 * ((c + 31) // 32)
        xp = torch.cat([x, torch.full((2, cp - c, 3, 4), -1.0)], dim=1).contiguous()
        assert torch.equal(words, oracle_lib.pack_nchw(xp))
        w = torch.randn((5, c, 3, 3), generator=g)
        ww = oracle_lib.pack_conv_weight(w)                               # [5, 3, 3, ceil(c/32)]
        real, tail = _bits(ww, c)
        assert np.array_equal(real, (w >= 0).permute(0, 2, 3, 1).numpy().astype(np.int64)), c
        assert not tail.any()
        bias = 0.3 * torch.randn(c, generator=g)
        sh = oracle_lib.pack_nchw_shift(x, bias)
        real, tail = _bits(sh, c)
        assert np.array_equal(real, ((x + bias.view(1, -1, 1, 1)) >= 0).permute(0, 2, 3, 1).numpy().astype(np.int64))
        assert not tail.any()


def test_tail_popcount_identity(oracle_lib):
    """With the missing bits 0 in both operands, K - 2*popcount(a XOR w) over the ceil(K/32) words
    is the +-1 dot product over the true K (the oracle's contraction), for K = 1..100."""
    g = torch.Generator().manual_seed(63)
    for k in range(1, 101):
        x = torch.randn((4, k), generator=g)
        w = torch.randn((6, k), generator=g)
        a = oracle_lib.pack_rows(x).numpy().astype(np.uint32)
        b = oracle_lib.pack_rows(w).numpy().astype(np.uint32)
        pop = np.vectorize(lambda v: bin(int(v)).count("1"))(a[:, None, :] ^ b[None, :, :]).sum(-1)
        assert np.array_equal(k - 2 * pop, oracle_lib.linear_acc(x, w).numpy()), k


# ---------------------------------------------------------------- non-square kernels, per-axis parameters

def _direct_conv_rect(xs, ws, s, p, d):
    """Direct definition with explicit bounds checks, (rows, columns) parameters."""
    B, C, H, W = xs.shape
    O, _, KH, KW = ws.shape
    Ho = math.floor((H + 2 * p[0] - d[0] * (KH - 1) - 1) / s[0] + 1)
    Wo = math.floor((W + 2 * p[1] - d[1] * (KW - 1) - 1) / s[1] + 1)
    out = np.zeros((B, O, Ho, Wo), dtype=np.int64)
    for b in range(B):
        for o in range(O):
            for oh in range(Ho):
                for ow in range(Wo):
                    tot = 0
                    for i in range(KH):
                        ih = oh * s[0] - p[0] + i * d[0]
                        if ih < 0 or ih >= H:
                            continue
                        for j in range(KW):
                            iw = ow * s[1] - p[1] + j * d[1]
                            if iw < 0 or iw >= W:
                                continue
                            tot += int(np.dot(xs[b, :, ih, iw], ws[o, :, i, j]))
                    out[b, o, oh, ow] = tot
    return out


def _rect_cases(count, seed):
    rnd = random.Random(seed)
    cases = []
    while len(cases) < count:
        b, c = rnd.choice([1, 2]), rnd.choice([1, 3, 32, 33])
        h, w = rnd.randint(1, 8), rnd.randint(1, 8)
        o, kh, kw = rnd.choice([1, 3]), rnd.choice([1, 2, 3, 5]), rnd.choice([1, 2, 3, 4])
        s = (rnd.choice([1, 2, 3]), rnd.choice([1, 2, 3]))
        p = (rnd.randint(0, 3), rnd.randint(0, 3))
        d = (rnd.choice([1, 2, 3]), rnd.choice([1, 2, 3]))
        ho = math.floor((h + 2 * p[0] - d[0] * (kh - 1) - 1) / s[0] + 1)
        wo = math.floor((w + 2 * p[1] - d[1] * (kw - 1) - 1) / s[1] + 1)
        if ho > 0 and wo > 0 and (kh != kw or s[0] != s[1] or p[0] != p[1] or d[0] != d[1]):
            cases.append((b, c, h, w, o, kh, kw, s, p, d))
    return cases


def test_conv_rect_matches_direct_definition(oracle_lib):
    g = torch.Generator().manual_seed(81)
    for (b, c, h, w, o, kh, kw, s, p, d) in _rect_cases(50, 5):
        x = torch.randn((b, c, h, w), generator=g)
        wt = torch.randn((o, c, kh, kw), generator=g)
        acc = oracle_lib.conv2d_acc(x, wt, s, p, d).numpy()
        want = _direct_conv_rect(np.where(x.numpy() >= 0, 1, -1), np.where(wt.numpy() >= 0, 1, -1), s, p, d)
        assert np.array_equal(acc, want), (b, c, h, w, o, kh, kw, s, p, d)


def test_conv_rect_matches_torch_fp64_and_kvalid(oracle_lib):
    g = torch.Generator().manual_seed(82)
    for (b, c, h, w, o, kh, kw, s, p, d) in _rect_cases(200, 6):
        dt = [torch.float32, torch.float16, torch.bfloat16][(b + c + h) % 3]
        x = torch.randn((b, c, h, w), generator=g).to(dt)
        wt = torch.randn((o, c, kh, kw), generator=g).to(dt)
        acc = oracle_lib.conv2d_acc(x, wt, s, p, d)
        ref = torch.nn.functional.conv2d(_lib_sign(x), _lib_sign(wt), stride=s, padding=p, dilation=d)
        assert torch.equal(acc.double(), ref), (b, c, h, w, o, kh, kw, s, p, d)
        ones = torch.nn.functional.conv2d(torch.ones((1, c, h, w), dtype=torch.float64),
                                          torch.ones((1, c, kh, kw), dtype=torch.float64),
                                          stride=s, padding=p, dilation=d)[0, 0]
        assert torch.equal(oracle_lib.conv2d_kvalid(c, h, w, (kh, kw), s, p, d).double(), ones)
    # equal parameters on both axes give the square entry's results
    x = torch.randn((2, 32, 7, 6), generator=g)
    wt = torch.randn((4, 32, 3, 3), generator=g)
    assert torch.equal(oracle_lib.conv2d_acc(x, wt, (2, 2), (1, 1), (1, 1)), oracle_lib.conv2d_acc(x, wt, 2, 1, 1))


def test_pack_conv_weight_rect_layout(oracle_lib):
    g = torch.Generator().manual_seed(83)
    for (kh, kw, c) in [(1, 3, 32), (3, 1, 64), (2, 5, 40), (5, 2, 7)]:
        w = torch.randn((3, c, kh, kw), generator=g)
        got = oracle_lib.pack_conv_weight(w)
        assert got.shape == (3, kh, kw, (c + 31) // 32)
        assert torch.equal(got, oracle_lib.pack_rows(w.permute(0, 2, 3, 1).contiguous().reshape(-1, c))
                           .view(3, kh, kw, (c + 31) // 32))
