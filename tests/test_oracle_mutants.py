"""Planted mistakes in the oracle are caught by its pins (CPU only).

Each case copies oracle/bnn_oracle.c, plants one plausible mistake (a dropped term, a wrong
sign, a transposed index or operand, a wrong constant), compiles the copy with gcc and runs a
fast subset of the pins against it. At least one pin must fail for every mutant; the
unmodified source must pass them all. Nothing here touches the GPU or the HIP library.
"""
import ctypes
import json
import math
import os
import random

import numpy as np
import pytest
import torch

import oracle
from backward_pins import PINS as BACKWARD_PINS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "bnn_oracle.c")
GOLDEN = os.path.join(ROOT, "tests", "golden")

MUTANTS = {
    "zero_maps_to_minus_one": ("return v >= 0.0f ? 1.0f : -1.0f;", "return v > 0.0f ? 1.0f : -1.0f;"),
    # (a wrong exponent bias only rescales magnitudes, which the sign rule never sees, so such
    # mutants are equivalent; these two change signs)
    "f16_nan_widened_to_inf": ("v = frac ? NAN : INFINITY;", "v = INFINITY;"),
    "f16_subnormals_flushed": ("v = ldexpf((float)frac, -24);", "v = 0.0f;"),
    "bf16_widen_shift": ("(uint32_t)b << 16;", "(uint32_t)b << 15;"),
    "pack_bit_order": ("if (sgn(widen(x, dtype, r * k + 32 * q + j)) > 0.0f) word |= (uint32_t)1 << j;",
                       "if (sgn(widen(x, dtype, r * k + 32 * q + j)) > 0.0f) word |= (uint32_t)1 << (31 - j);"),
    "pack_nchw_hw_swapped": ("int64_t idx = ((b * C + 32 * q + j) * H + ih) * W + iw;",
                             "int64_t idx = ((b * C + 32 * q + j) * W + iw) * H + ih;"),
    "pack_weight_kernel_transposed": ("int64_t idx = ((o * C + 32 * q + jj) * KH + i) * KW + j;",
                                      "int64_t idx = ((o * C + 32 * q + jj) * KW + j) * KH + i;"),
    "linear_drops_last_term": ("for (int64_t k = 0; k < K; k++) s += sx[k] * wr[k];",
                               "for (int64_t k = 0; k < K - 1; k++) s += sx[k] * wr[k];"),
    "linear_x_transposed": ("sx[k] = sgn(widen(x, xdt, m * K + k));",
                            "sx[k] = sgn(widen(x, xdt, (k % M) * K + (m * K + k) / M % K));"),
    "conv_pad_value_plus_one": ("memset(xp, 0, sizeof(float) * (size_t)(C * Hp * Wp));",
                                "for (int64_t z = 0; z < C * Hp * Wp; z++) xp[z] = 1.0f;"),
    "conv_unfold_without_dilation": ("cols[l * R + r] = xp[(c * Hp + oh * sh + i * dh) * Wp + ow * sw + j * dw];",
                                     "cols[l * R + r] = xp[(c * Hp + oh * sh + i) * Wp + ow * sw + j];"),
    "conv_ignores_column_stride": ("cols[l * R + r] = xp[(c * Hp + oh * sh + i * dh) * Wp + ow * sw + j * dw];",
                                   "cols[l * R + r] = xp[(c * Hp + oh * sh + i * dh) * Wp + ow + j * dw];"),
    "conv_row_index_transposed": ("int64_t r = (c * KH + i) * KW + j;", "int64_t r = (c * KW + j) * KH + i;"),
    "conv_swaps_axis_strides": ("cols[l * R + r] = xp[(c * Hp + oh * sh + i * dh) * Wp + ow * sw + j * dw];",
                                "cols[l * R + r] = xp[(c * Hp + oh * sw + i * dh) * Wp + ow * sh + j * dw];"),
    "conv_pad_rows_by_columns": ("xp[(c * Hp + ih + ph) * Wp + iw + pw] = sgn(", "xp[(c * Hp + ih + pw) * Wp + iw + pw] = sgn("),
    "kvalid_off_by_one": ("if (ih >= 0 && ih < H && iw >= 0 && iw < W) taps++;",
                          "if (ih >= 0 && ih <= H && iw >= 0 && iw < W) taps++;"),
    "scale_sum_instead_of_product": ("double alpha = scale_a * scale_w;", "double alpha = scale_a + scale_w;"),
    "shift_subtracts_bias": ("double sum = (double)v + (double)b;", "double sum = (double)v - (double)b;"),
    "shift_zero_sum_negative": ("return sum >= 0.0 ? 1.0f : -1.0f;", "return sum > 0.0 ? 1.0f : -1.0f;"),
    "rows_shift_bias_by_word": ("float b = widen(bias, bdtype, blen == 1 ? 0 : col);",
                                "float b = widen(bias, bdtype, blen == 1 ? 0 : q);"),
    "nchw_shift_bias_by_width": ("widen(bias, bdtype, c)) > 0.0f", "widen(bias, bdtype, iw)) > 0.0f"),
    "abs_mean_drops_abs": ("sum += fabs((double)widen(x, dtype, i));", "sum += (double)widen(x, dtype, i);"),
    "abs_mean_count_minus_one": ("return factor * (sum / (double)count);",
                                 "return factor * (sum / (double)(count - 1));"),
    "quant_truncates": ("float r = rintf(v / step);", "float r = truncf(v / step);"),
    "quant_clamp_128": ("  if (r < -127.0f) r = -127.0f;\n  return (int8_t)r;", "  if (r < -128.0f) r = -128.0f;\n  return (int8_t)r;"),
    "w8a8_step_255": ("static float q_step(float amax) { return amax / 127.0f; }",
                      "static float q_step(float amax) { return amax / 255.0f; }"),
    "abs_mean_fixed_factor": ("return factor * (sum / (double)count);", "return 2.0 * (sum / (double)count);"),
    "bwd_sign0_zero_is_one": ("return v > 0.0f ? 1.0 : (v < 0.0f ? -1.0 : 0.0);", "return v >= 0.0f ? 1.0 : -1.0;"),
    "bwd_clip_inclusive": ("double small = q < -1.0f ? 1.0 : 0.0", "double small = q <= -1.0f ? 1.0 : 0.0"),
    "bwd_clip_on_x_not_quotient": ("float q = v / scale_a;", "float q = v;"),
    "bwd_drops_sqrt": ("*grad_scale_a = total / sqrt((double)M * (double)K);",
                       "*grad_scale_a = total / ((double)M * (double)K);"),
    "bwd_weight_transposed": ("ws[i] = sign0(widen(w, wdt, i)) * (double)scale_w;",
                              "ws[i] = sign0(widen(w, wdt, (i % N) * K + (i / N) % K)) * (double)scale_w;"),
    "bwd_grad_w_drops_scale_a": ("row[k] += gv * (sign0(widen(x, xdt, m * K + k)) * (double)scale_a);",
                                 "row[k] += gv * (sign0(widen(x, xdt, m * K + k)));"),
    "bwd_grad_scale_a_unsigned": ("total += grad_in[i] * sign0(widen(x, xdt, i));", "total += grad_in[i];"),
    "bwd_quant_step_by_255": ("  float step = amax / 127.0f;\n  for (int64_t i = 0; i < count; i++) {\n    float r = rintf((float)grad_w[i] / step);",
                              "  float step = amax / 255.0f;\n  for (int64_t i = 0; i < count; i++) {\n    float r = rintf((float)grad_w[i] / step);"),
    "bwd_quant_amax_signed": ("    float v = fabsf((float)grad_w[i]);", "    float v = (float)grad_w[i];"),
    "bwd_conv_tap_without_dilation": ("int64_t ih = oh * sh - ph + i * dh, iw = ow * sw - pw + j * dw;\n                if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;\n                int64_t xi",
                                      "int64_t ih = oh * sh - ph + i, iw = ow * sw - pw + j * dw;\n                if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;\n                int64_t xi"),
    "bwd_conv_pad_added": ("int64_t ih = oh * sh - ph + i * dh, iw = ow * sw - pw + j * dw;\n                if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;\n                int64_t xi",
                           "int64_t ih = oh * sh + ph + i * dh, iw = ow * sw - pw + j * dw;\n                if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;\n                int64_t xi"),
    "bwd_conv_kernel_transposed": ("wi = ((o * C + c) * KH + i) * KW + j;", "wi = ((o * C + c) * KW + j) * KH + i;"),
    "u8_bit_order_reversed": ("if (sgn(widen(x, dtype, r * k + 8 * q + j)) > 0.0f) byte |= 1u << j;",
                              "if (sgn(widen(x, dtype, r * k + 8 * q + j)) > 0.0f) byte |= 1u << (7 - j);"),
    "u8_nchw_hw_swapped": ("int64_t idx = ((b * C + 8 * q + j) * H + ih) * W + iw;",
                           "int64_t idx = ((b * C + 8 * q + j) * W + iw) * H + ih;"),
    "u8_weight_kernel_transposed": ("int64_t idx = ((o * C + 8 * q + jj) * KH + i) * KW + j;",
                                    "int64_t idx = ((o * C + 8 * q + jj) * KW + j) * KH + i;"),
    "u8_nibble_container": ("      out[r * kb + q] = (uint8_t)byte;", "      out[r * kb + q] = (uint8_t)(byte & 0x0f);"),
    "bwd_conv_weight_grad_unsigned": ("grad_w[wi] += gv * (sign0(widen(x, xdt, xi)) * (double)scale_a);",
                                      "grad_w[wi] += gv * ((double)widen(x, xdt, xi) * (double)scale_a);"),
}


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(v):
    if isinstance(v, str):
        return {"-0": -0.0, "nan": float("nan"), "-inf": float("-inf"), "inf": float("inf")}[v]
    return float(v)


def _tensor(nested):
    return torch.from_numpy(np.vectorize(_num, otypes=[np.float64])(np.array(nested, dtype=object)).astype(np.float32))


def _lib_sign(t):
    return torch.where(t.float() >= 0, 1.0, -1.0).double()


def _pins(orc):
    """Fast pins; returns the names of those that fail."""
    failed = []

    def check(name, fn):
        try:
            if not fn():
                failed.append(name)
        except Exception:  # a crash of the mutant counts as a caught mistake
            failed.append(name)

    g = _golden("linear_hand.json")
    check("linear_hand", lambda: orc.linear_acc(_tensor(g["x"]), _tensor(g["w"])).tolist() == g["acc"]
          and orc.scale(torch.tensor(g["acc"], dtype=torch.int32), g["scale_a"], g["scale_w"]).tolist() == g["y"])
    g2 = _golden("conv_checkerboard.json")
    check("conv_hand", lambda: orc.conv2d_acc(_tensor(g2["x"]), _tensor(g2["w"]), 1, 1, 1).tolist() == g2["acc"])
    km = _golden("kvalid_maps.json")["cases"]
    check("kvalid_maps", lambda: all(orc.conv2d_kvalid(1, c["h"], c["w"], 3, c["stride"], c["padding"],
                                                       c["dilation"]).tolist() == c["kvalid"] for c in km))
    table = _golden("sign_edges.json")

    def signs_ok():
        for dt, tdt, width in (("f32", torch.float32, 32), ("f16", torch.float16, 16), ("bf16", torch.bfloat16, 16)):
            ints = [int(h, 16) for h, _ in table[dt]]
            ints = [b - (1 << width) if b >= 1 << (width - 1) else b for b in ints]
            raw = torch.tensor(ints, dtype=torch.int32 if width == 32 else torch.int16).view(tdt)
            if orc.sign(raw).tolist() != [float(s) for _, s in table[dt]]:
                return False
        allbits = torch.arange(-(1 << 15), 1 << 15, dtype=torch.int32).to(torch.int16)
        for tdt in (torch.float16, torch.bfloat16):
            x = allbits.view(tdt).contiguous()
            if not torch.equal(orc.sign(x).double(), _lib_sign(x)):
                return False
        return True

    check("sign_table_and_widening", signs_ok)

    def brute():
        for k in (1, 3, 6):
            pats = np.arange(1 << k)
            bits = (pats[:, None] >> np.arange(k)[None, :]) & 1
            x = torch.from_numpy(np.where(bits == 1, 1.5, -0.5).astype(np.float32))
            acc = orc.linear_acc(x, x).numpy()
            want = np.array([[k - 2 * bin(int(a) ^ int(b)).count("1") for b in pats] for a in pats])
            if not np.array_equal(acc, want):
                return False
        return True

    check("brute_force", brute)

    def packs():
        gen = torch.Generator().manual_seed(5)
        x = torch.randn((6, 96), generator=gen)
        bits = (orc.pack_rows(x).numpy().astype(np.uint32).astype(np.int64)[..., None] >> np.arange(32)) & 1
        if not np.array_equal(bits.reshape(6, 96), (x >= 0).numpy().astype(np.int64)):
            return False
        xn = torch.randn((2, 64, 5, 3), generator=gen)
        if not torch.equal(orc.pack_nchw(xn),
                           orc.pack_rows(xn.permute(0, 2, 3, 1).contiguous().reshape(-1, 64)).view(2, 5, 3, 2)):
            return False
        wc = torch.randn((3, 32, 3, 3), generator=gen)
        return torch.equal(orc.pack_conv_weight(wc),
                           orc.pack_rows(wc.permute(0, 2, 3, 1).contiguous().reshape(-1, 32)).view(3, 3, 3, 1))

    check("pack_layouts", packs)

    def lib_linear():
        gen = torch.Generator().manual_seed(7)
        for m, n, k in ((5, 7, 64), (9, 3, 96), (1, 4, 32)):
            x, w = torch.randn((m, k), generator=gen), torch.randn((n, k), generator=gen)
            if not torch.equal(orc.linear_acc(x, w).double(), _lib_sign(x) @ _lib_sign(w).T):
                return False
        return True

    check("linear_vs_torch", lib_linear)

    def lib_conv():
        rnd = random.Random(9)
        gen = torch.Generator().manual_seed(9)
        n = 0
        while n < 25:
            b, c, h, w = rnd.choice([1, 2]), rnd.choice([1, 3, 32]), rnd.randint(2, 7), rnd.randint(2, 7)
            o, ks, s, p, d = rnd.choice([1, 3]), rnd.choice([1, 2, 3]), rnd.choice([1, 2]), rnd.randint(0, 2), rnd.choice([1, 2])
            if math.floor((h + 2 * p - d * (ks - 1) - 1) / s + 1) <= 0 or math.floor((w + 2 * p - d * (ks - 1) - 1) / s + 1) <= 0:
                continue
            n += 1
            x, wt = torch.randn((b, c, h, w), generator=gen), torch.randn((o, c, ks, ks), generator=gen)
            ref = torch.nn.functional.conv2d(_lib_sign(x), _lib_sign(wt), stride=s, padding=p, dilation=d)
            if not torch.equal(orc.conv2d_acc(x, wt, s, p, d).double(), ref):
                return False
        return True

    check("conv_vs_torch", lib_conv)

    def lib_conv_rect():
        # non-square kernels, different strides / paddings / dilations per axis
        rnd = random.Random(19)
        gen = torch.Generator().manual_seed(19)
        n = 0
        while n < 25:
            b, c, h, w = rnd.choice([1, 2]), rnd.choice([1, 3, 32]), rnd.randint(2, 8), rnd.randint(2, 8)
            o, kh, kw = rnd.choice([1, 3]), rnd.choice([1, 2, 3]), rnd.choice([1, 2, 3, 4])
            s, p, d = (rnd.choice([1, 2]), rnd.choice([1, 3])), (rnd.randint(0, 2), rnd.randint(0, 2)), (rnd.choice([1, 2]), rnd.choice([1, 3]))
            if math.floor((h + 2 * p[0] - d[0] * (kh - 1) - 1) / s[0] + 1) <= 0 or \
                    math.floor((w + 2 * p[1] - d[1] * (kw - 1) - 1) / s[1] + 1) <= 0:
                continue
            n += 1
            x, wt = torch.randn((b, c, h, w), generator=gen), torch.randn((o, c, kh, kw), generator=gen)
            ref = torch.nn.functional.conv2d(_lib_sign(x), _lib_sign(wt), stride=s, padding=p, dilation=d)
            if not torch.equal(orc.conv2d_acc(x, wt, s, p, d).double(), ref):
                return False
            ones = torch.nn.functional.conv2d(torch.ones((1, c, h, w), dtype=torch.float64),
                                              torch.ones((1, c, kh, kw), dtype=torch.float64),
                                              stride=s, padding=p, dilation=d)[0, 0]
            if not torch.equal(orc.conv2d_kvalid(c, h, w, (kh, kw), s, p, d).double(), ones):
                return False
        wc = torch.randn((3, 32, 2, 3), generator=gen)
        return torch.equal(orc.pack_conv_weight(wc),
                           orc.pack_rows(wc.permute(0, 2, 3, 1).contiguous().reshape(-1, 32)).view(3, 2, 3, 1))

    check("conv_rect_vs_torch", lib_conv_rect)

    def w8a8_vs_torch():
        gen = torch.Generator().manual_seed(29)
        x = 2 * torch.randn((2, 6, 7, 5), generator=gen)
        wt = torch.randn((3, 6, 3, 2), generator=gen)

        def codes(v, amax):
            step = torch.tensor(amax, dtype=torch.float32) / 127.0
            return torch.round(v.float() / step).clamp(-127, 127)
        if not torch.equal(orc.quant_i8(x, 3.0).double(), codes(x, 3.0).double()):
            return False
        ref = torch.nn.functional.conv2d(codes(x, 3.0).double(), codes(wt, 1.0).double(),
                                         stride=(1, 2), padding=(1, 0), dilation=(2, 1))
        return torch.equal(orc.w8a8_conv2d_acc(x, wt, (1, 2), (1, 0), (2, 1), 3.0, 1.0).double(), ref)

    check("w8a8_vs_torch", w8a8_vs_torch)

    edges = _golden("shift_sign_edges.json")["cases"]

    def shift_edges():
        for xdt, xh, bdt, bh, want, _ in edges:
            x, b = _bits_value(xdt, xh), _bits_value(bdt, bh)
            words = orc.pack_rows_shift(x.repeat(32).view(1, 32).contiguous(), b.repeat(32).contiguous())
            if (1 if int(words[0, 0]) & 1 else -1) != want:
                return False
        return True

    check("shift_sign_edges", shift_edges)

    def shift_vs_torch():
        gen = torch.Generator().manual_seed(15)
        x = torch.randn((6, 96), generator=gen)
        bias = 0.5 * torch.randn(96, generator=gen)
        bits = (orc.pack_rows_shift(x, bias).numpy().astype(np.uint32).astype(np.int64)[..., None] >> np.arange(32)) & 1
        if not np.array_equal(bits.reshape(6, 96), ((x + bias) >= 0).numpy().astype(np.int64)):
            return False
        xn = torch.randn((2, 64, 5, 3), generator=gen)
        bn = 0.5 * torch.randn(64, generator=gen)
        want = orc.pack_rows(((xn + bn.view(1, -1, 1, 1)) >= 0).float().sub(0.5)
                             .permute(0, 2, 3, 1).contiguous().reshape(-1, 64)).view(2, 5, 3, 2)
        return torch.equal(orc.pack_nchw_shift(xn, bn), want)

    check("shift_vs_torch", shift_vs_torch)

    def abs_mean():
        ints = torch.arange(1000, dtype=torch.float32)
        return (orc.abs_mean_scale(-ints, 4.0) == 2 * 999 and orc.abs_mean_scale(ints, 2.0) == 999
                and orc.abs_mean_scale(torch.tensor([0.5, -2.5]), 2.0) == 3.0)

    check("abs_mean_closed_forms", abs_mean)

    u8 = _golden("u8_container.json")

    def u8_golden():
        for row in u8["rows"]:
            got = orc.pack_rows_u8(_tensor([row["x"]]))[0].tolist()
            if got != [int(h, 16) for h in row["bytes"]]:
                return False
        nc = u8["nchw"]
        x = torch.stack([_tensor(nc["pixel0"]), _tensor(nc["pixel1"])], dim=1).view(1, 10, 1, 2).contiguous()
        got = orc.pack_nchw_u8(x)
        return (got[0, 0, 0].tolist() == [int(h, 16) for h in nc["bytes0"]]
                and got[0, 0, 1].tolist() == [int(h, 16) for h in nc["bytes1"]])

    check("u8_golden", u8_golden)

    def u8_vs_torch():
        gen = torch.Generator().manual_seed(35)

        def bits(t, n):
            return np.unpackbits(t.numpy(), axis=-1, bitorder="little")[..., :n]

        x = torch.randn((5, 70), generator=gen)
        if not np.array_equal(bits(orc.pack_rows_u8(x), 70), (x >= 0).numpy()):
            return False
        if np.unpackbits(orc.pack_rows_u8(x).numpy(), axis=-1, bitorder="little")[:, 70:].any():
            return False
        xn = torch.randn((2, 20, 3, 4), generator=gen)
        if not np.array_equal(bits(orc.pack_nchw_u8(xn), 20), (xn >= 0).permute(0, 2, 3, 1).numpy()):
            return False
        wc = torch.randn((3, 12, 2, 3), generator=gen)
        return np.array_equal(bits(orc.pack_conv_weight_u8(wc), 12), (wc >= 0).permute(0, 2, 3, 1).numpy())

    check("u8_vs_torch", u8_vs_torch)
    for name, pin in BACKWARD_PINS.items():
        check(name, lambda pin=pin: pin(orc))
    return failed


def _bits_value(dt, hexbits):
    v = int(hexbits, 16)
    if dt == "f32":
        return torch.tensor([v - (1 << 32) if v >= 1 << 31 else v], dtype=torch.int32).view(torch.float32)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    return torch.tensor([v - (1 << 16) if v >= 1 << 15 else v], dtype=torch.int16).view(tdt)


@pytest.fixture()
def swap_oracle():
    saved = oracle._lib
    yield
    oracle._lib = saved


def _compile_variant(tmp_path, name, edit):
    src = open(SRC).read()
    if edit is not None:
        old, new = edit
        assert src.count(old) == 1, f"mutation site for {name} not unique"
        src = src.replace(old, new)
    path = tmp_path / f"{name}.c"
    path.write_text(src)
    lib = oracle.compile_library(str(path), str(tmp_path / f"lib{name}.so"))
    return oracle._bind(ctypes.CDLL(lib))


def test_unmodified_oracle_passes_fast_pins(tmp_path, swap_oracle):
    oracle._lib = _compile_variant(tmp_path, "original", None)
    assert _pins(oracle) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, swap_oracle, name):
    oracle._lib = _compile_variant(tmp_path, name, MUTANTS[name])
    failed = _pins(oracle)
    assert failed, f"mutant {name} passed every pin"
