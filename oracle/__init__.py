"""CPU oracle for the binarized linear / conv2d forward (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this package; the product path never does. The
arithmetic lives in ``bnn_oracle.c`` (plain C loops, OpenMP), built with gcc
into ``liboracle.so`` beside it. It shares no code with the HIP library.

Every function takes contiguous CPU torch tensors and returns CPU tensors.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bnn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# x86-64-v3 (AVX2/FMA) so the library also runs on other x86 hosts; never fast-math:
# the sign rule relies on IEEE compares of NaN, -0 and subnormals.
_CFLAGS = ["-O2", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-Wno-unused-parameter"]

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (also without force when the source is newer than the
    library); returns its path."""
    stale = not os.path.exists(_LIB) or os.path.getmtime(_SRC) > os.path.getmtime(_LIB)
    if force or stale:
        tmp = _LIB + ".tmp"
        compile_library(_SRC, tmp)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    """Declare the C signatures on a loaded oracle library."""
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_num_threads.restype = I
    lib.oracle_sign.argtypes = [P, I, I64, P]
    lib.oracle_pack_rows.argtypes = [P, I, I64, I64, P]
    lib.oracle_pack_nchw.argtypes = [P, I, I64, I64, I64, I64, P]
    lib.oracle_pack_conv_weight.argtypes = [P, I, I64, I64, I64, P]
    lib.oracle_linear_acc.argtypes = [P, I, P, I, I64, I64, I64, P, I64, P]
    lib.oracle_linear_acc.restype = I
    lib.oracle_conv_out_size.argtypes = [I64, I64, I64, I64, I64]
    lib.oracle_conv_out_size.restype = I64
    lib.oracle_conv2d_acc.argtypes = [P, I, P, I, I64, I64, I64, I64, I64, I64, I64, I64,
                                      I64, P, I64, P]
    lib.oracle_conv2d_acc.restype = I
    lib.oracle_conv2d_kvalid.argtypes = [I64, I64, I64, I64, I64, I64, I64, P]
    lib.oracle_conv2d_kvalid.restype = I
    lib.oracle_conv2d_acc2.argtypes = [P, I, P, I] + [I64] * 13 + [P, I64, P]
    lib.oracle_conv2d_acc2.restype = I
    lib.oracle_conv2d_kvalid2.argtypes = [I64] * 11 + [P]
    lib.oracle_conv2d_kvalid2.restype = I
    lib.oracle_pack_conv_weight2.argtypes = [P, I, I64, I64, I64, I64, P]
    lib.oracle_pack_rows_u8.argtypes = [P, I, I64, I64, P]
    lib.oracle_pack_nchw_u8.argtypes = [P, I, I64, I64, I64, I64, P]
    lib.oracle_pack_conv_weight_u8.argtypes = [P, I, I64, I64, I64, I64, P]
    lib.oracle_quant_i8.argtypes = [P, I, I64, ctypes.c_float, P]
    lib.oracle_w8a8_conv2d_acc.argtypes = [P, I, P, I] + [I64] * 13 + [ctypes.c_float, ctypes.c_float,
                                                                       P, I64, P]
    lib.oracle_w8a8_conv2d_acc.restype = I
    lib.oracle_scale.argtypes = [P, I64, ctypes.c_double, ctypes.c_double, P]
    lib.oracle_pack_rows_shift.argtypes = [P, I, I64, I64, P, I, I64, P]
    lib.oracle_pack_nchw_shift.argtypes = [P, I, I64, I64, I64, I64, P, I, P]
    lib.oracle_abs_mean_scale.argtypes = [P, I, I64, ctypes.c_double]
    lib.oracle_linear_grad_input.argtypes = [P, I, P, I, P, I, I64, I64, I64, ctypes.c_float,
                                             ctypes.c_float, P, P]
    lib.oracle_linear_grad_weight.argtypes = [P, I, P, I, I64, I64, I64, ctypes.c_float, P]
    lib.oracle_quant_grad_i8.argtypes = [P, I64, P, P]
    lib.oracle_conv2d_grad.argtypes = [P, I, P, I, P, I] + [I64] * 13 + [ctypes.c_float, ctypes.c_float,
                                                                        P, P, P]
    lib.oracle_abs_mean_scale.restype = ctypes.c_double
    return lib


def compile_library(src: str, out: str) -> str:
    """Compile an oracle source file (this one, or a test's modified copy) into a shared library."""
    subprocess.run(["gcc", *_CFLAGS, src, "-o", out, "-lm"], check=True)
    return out


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


def _code(t: torch.Tensor) -> int:
    if t.dtype not in _CODE:
        raise TypeError(f"oracle: unsupported dtype {t.dtype}")
    return _CODE[t.dtype]


def _cpu(t: torch.Tensor) -> torch.Tensor:
    if t.device.type != "cpu" or not t.is_contiguous():
        raise ValueError("oracle: inputs must be contiguous CPU tensors")
    return t


def num_threads() -> int:
    return _load().oracle_num_threads()


def sign(x: torch.Tensor) -> torch.Tensor:
    """sgn(x) as float32 +-1 (x >= 0 -> +1, else -1), same shape as x."""
    x = _cpu(x)
    out = torch.empty(x.shape, dtype=torch.float32)
    _load().oracle_sign(x.data_ptr(), _code(x), x.numel(), out.data_ptr())
    return out


def _words(n: int) -> torch.Tensor:
    return torch.empty(n, dtype=torch.int32)


def _nw(k: int) -> int:
    """Words that hold k signs (the last one partly, its missing bits 0)."""
    return (k + 31) // 32


def pack_rows(x: torch.Tensor) -> torch.Tensor:
    """x [rows, k] -> int32 words [rows, ceil(k/32)] (bit j of word q = x[r, 32q+j] >= 0;
    bits past k are 0)."""
    x = _cpu(x)
    rows, k = x.shape
    out = _words(rows * _nw(k))
    _load().oracle_pack_rows(x.data_ptr(), _code(x), rows, k, out.data_ptr())
    return out.view(rows, _nw(k))


def pack_nchw(x: torch.Tensor) -> torch.Tensor:
    """x [b, c, h, w] -> int32 words [b, h, w, ceil(c/32)] (channel bits past c are 0)."""
    x = _cpu(x)
    b, c, h, w = x.shape
    out = _words(b * h * w * _nw(c))
    _load().oracle_pack_nchw(x.data_ptr(), _code(x), b, c, h, w, out.data_ptr())
    return out.view(b, h, w, _nw(c))


def pack_conv_weight(w: torch.Tensor) -> torch.Tensor:
    """OIHW w [o, c, kh, kw] -> int32 words [o, kh, kw, ceil(c/32)] (channel bits past c are 0)."""
    w = _cpu(w)
    o, c, kh, kw = w.shape
    out = _words(o * kh * kw * _nw(c))
    if kh == kw:
        _load().oracle_pack_conv_weight(w.data_ptr(), _code(w), o, c, kh, out.data_ptr())
    else:
        _load().oracle_pack_conv_weight2(w.data_ptr(), _code(w), o, c, kh, kw, out.data_ptr())
    return out.view(o, kh, kw, _nw(c))


def _nb(n: int) -> int:
    return (n + 7) // 8


def pack_rows_u8(x: torch.Tensor) -> torch.Tensor:
    """8-bit containers: x [rows, k] -> uint8 [rows, ceil(k/8)] (bit j of byte q = x[r, 8q+j] >= 0;
    bits past k are 0)."""
    x = _cpu(x)
    rows, k = x.shape
    out = torch.empty((rows, _nb(k)), dtype=torch.uint8)
    _load().oracle_pack_rows_u8(x.data_ptr(), _code(x), rows, k, out.data_ptr())
    return out


def pack_nchw_u8(x: torch.Tensor) -> torch.Tensor:
    """8-bit containers: x [b, c, h, w] -> uint8 [b, h, w, ceil(c/8)] (channel bits past c are 0)."""
    x = _cpu(x)
    b, c, h, w = x.shape
    out = torch.empty((b, h, w, _nb(c)), dtype=torch.uint8)
    _load().oracle_pack_nchw_u8(x.data_ptr(), _code(x), b, c, h, w, out.data_ptr())
    return out


def pack_conv_weight_u8(w: torch.Tensor) -> torch.Tensor:
    """8-bit containers: OIHW w [o, c, kh, kw] -> uint8 [o, kh, kw, ceil(c/8)]."""
    w = _cpu(w)
    o, c, kh, kw = w.shape
    out = torch.empty((o, kh, kw, _nb(c)), dtype=torch.uint8)
    _load().oracle_pack_conv_weight_u8(w.data_ptr(), _code(w), o, c, kh, kw, out.data_ptr())
    return out


def _pair(v):
    return (int(v), int(v)) if isinstance(v, int) else (int(v[0]), int(v[1]))


def _index(idx, limit):
    if idx is None:
        return None, limit
    t = torch.as_tensor(list(idx), dtype=torch.int64).contiguous()
    if t.numel() and (int(t.min()) < 0 or int(t.max()) >= limit):
        raise IndexError("oracle: index out of range")
    return t, t.numel()


def linear_acc(x: torch.Tensor, w: torch.Tensor, rows=None) -> torch.Tensor:
    """int32 acc [len(rows) or M, N] = sum_k sgn(x[m,k]) * sgn(W[n,k])."""
    x, w = _cpu(x), _cpu(w)
    m, k = x.shape
    n, k2 = w.shape
    assert k == k2
    idx, nr = _index(rows, m)
    out = torch.empty((nr, n), dtype=torch.int32)
    rc = _load().oracle_linear_acc(x.data_ptr(), _code(x), w.data_ptr(), _code(w), m, n, k,
                                   idx.data_ptr() if idx is not None else None, nr,
                                   out.data_ptr())
    if rc != 0:
        raise RuntimeError("oracle_linear_acc failed")
    return out


def conv_out_size(size, ks, stride, padding, dilation) -> int:
    return int(_load().oracle_conv_out_size(size, ks, stride, padding, dilation))


def conv2d_acc(x: torch.Tensor, w: torch.Tensor, stride, padding, dilation,
               images=None) -> torch.Tensor:
    """int32 acc [len(images) or B, O, Ho, Wo] of the zero-padded binary conv. stride, padding
    and dilation are ints (both axes) or (rows, columns) pairs; the kernel may be non-square."""
    x, w = _cpu(x), _cpu(w)
    b, c, h, wd = x.shape
    o, c2, kh, kw = w.shape
    assert c == c2
    (sh, sw), (ph, pw), (dh, dw) = _pair(stride), _pair(padding), _pair(dilation)
    ho = conv_out_size(h, kh, sh, ph, dh)
    wo = conv_out_size(wd, kw, sw, pw, dw)
    if ho <= 0 or wo <= 0:
        raise ValueError("oracle: empty conv output")
    idx, ni = _index(images, b)
    out = torch.empty((ni, o, ho, wo), dtype=torch.int32)
    ip = idx.data_ptr() if idx is not None else None
    if kh == kw and sh == sw and ph == pw and dh == dw:
        rc = _load().oracle_conv2d_acc(x.data_ptr(), _code(x), w.data_ptr(), _code(w), b, c, h, wd, o,
                                       kh, sh, ph, dh, ip, ni, out.data_ptr())
    else:
        rc = _load().oracle_conv2d_acc2(x.data_ptr(), _code(x), w.data_ptr(), _code(w), b, c, h, wd,
                                        o, kh, kw, sh, sw, ph, pw, dh, dw, ip, ni, out.data_ptr())
    if rc != 0:
        raise RuntimeError("oracle_conv2d_acc failed")
    return out


def conv2d_kvalid(c, h, w, ks, stride, padding, dilation) -> torch.Tensor:
    """int32 [Ho, Wo]: number of real (unpadded) reduction terms per output pixel. ks, stride,
    padding and dilation are ints or (rows, columns) pairs."""
    (kh, kw), (sh, sw), (ph, pw), (dh, dw) = _pair(ks), _pair(stride), _pair(padding), _pair(dilation)
    ho = conv_out_size(h, kh, sh, ph, dh)
    wo = conv_out_size(w, kw, sw, pw, dw)
    out = torch.empty((ho, wo), dtype=torch.int32)
    if kh == kw and sh == sw and ph == pw and dh == dw:
        rc = _load().oracle_conv2d_kvalid(c, h, w, kh, sh, ph, dh, out.data_ptr())
    else:
        rc = _load().oracle_conv2d_kvalid2(c, h, w, kh, kw, sh, sw, ph, pw, dh, dw, out.data_ptr())
    if rc != 0:
        raise RuntimeError("oracle_conv2d_kvalid failed")
    return out


def scale(acc: torch.Tensor, scale_a: float, scale_w: float) -> torch.Tensor:
    """float64 y = acc * (scale_a * scale_w)."""
    acc = _cpu(acc)
    assert acc.dtype == torch.int32
    y = torch.empty(acc.shape, dtype=torch.float64)
    _load().oracle_scale(acc.data_ptr(), acc.numel(), float(scale_a), float(scale_w), y.data_ptr())
    return y


def pack_rows_shift(x: torch.Tensor, bias: torch.Tensor) -> torch.Tensor:
    """x [rows, k] shifted by bias (one value, or [k]) -> int32 words [rows, ceil(k/32)];
    bit j of word q = (x[r, 32q+j] + bias >= 0); bits past k are 0."""
    x, bias = _cpu(x), _cpu(bias)
    rows, k = x.shape
    assert bias.numel() in (1, k)
    out = _words(rows * _nw(k))
    _load().oracle_pack_rows_shift(x.data_ptr(), _code(x), rows, k, bias.data_ptr(), _code(bias),
                                   bias.numel(), out.data_ptr())
    return out.view(rows, _nw(k))


def pack_nchw_shift(x: torch.Tensor, bias: torch.Tensor) -> torch.Tensor:
    """x [b, c, h, w] shifted by bias[c] -> int32 words [b, h, w, ceil(c/32)]."""
    x, bias = _cpu(x), _cpu(bias)
    b, c, h, w = x.shape
    assert bias.numel() == c
    out = _words(b * h * w * _nw(c))
    _load().oracle_pack_nchw_shift(x.data_ptr(), _code(x), b, c, h, w, bias.data_ptr(), _code(bias),
                                   out.data_ptr())
    return out.view(b, h, w, _nw(c))


def abs_mean_scale(x: torch.Tensor, factor: float) -> float:
    """factor * mean(|x|) over every element (the sum in double, in index order)."""
    x = _cpu(x)
    return float(_load().oracle_abs_mean_scale(x.data_ptr(), _code(x), x.numel(), float(factor)))


def quant_i8(x: torch.Tensor, amax: float) -> torch.Tensor:
    """int8 codes of the symmetric per-tensor quantizer: clamp(rint(x / (amax/127)), -127, 127)
    with fp32 arithmetic, NaN -> 0; same shape as x."""
    x = _cpu(x)
    out = torch.empty(x.shape, dtype=torch.int8)
    _load().oracle_quant_i8(x.data_ptr(), _code(x), x.numel(), float(amax), out.data_ptr())
    return out


def w8a8_conv2d_acc(x: torch.Tensor, w: torch.Tensor, stride, padding, dilation, amax_x: float,
                    amax_w: float, images=None) -> torch.Tensor:
    """int32 acc [len(images) or B, O, Ho, Wo] = sum over the zero-padded unfold of
    q(x) * q(w) (W8A8 conv; scale by (amax_x/127) * (amax_w/127) for the output)."""
    x, w = _cpu(x), _cpu(w)
    b, c, h, wd = x.shape
    o, c2, kh, kw = w.shape
    assert c == c2
    (sh, sw), (ph, pw), (dh, dw) = _pair(stride), _pair(padding), _pair(dilation)
    ho = conv_out_size(h, kh, sh, ph, dh)
    wo = conv_out_size(wd, kw, sw, pw, dw)
    if ho <= 0 or wo <= 0:
        raise ValueError("oracle: empty conv output")
    idx, ni = _index(images, b)
    out = torch.empty((ni, o, ho, wo), dtype=torch.int32)
    rc = _load().oracle_w8a8_conv2d_acc(x.data_ptr(), _code(x), w.data_ptr(), _code(w), b, c, h, wd, o,
                                        kh, kw, sh, sw, ph, pw, dh, dw, float(amax_x), float(amax_w),
                                        idx.data_ptr() if idx is not None else None, ni, out.data_ptr())
    if rc != 0:
        raise RuntimeError("oracle_w8a8_conv2d_acc failed")
    return out


def linear_grad_input(g: torch.Tensor, w: torch.Tensor, x: torch.Tensor, scale_a: float,
                      scale_w: float):
    """Straight-through backward of the binarized linear layer, input side: returns
    (grad_in float64 [M, K], grad_scale_a float) for g [M, N], W [N, K], x [M, K]:
    grad_in = (scale_w * g @ sign0(W)) * mid(x), mid = 0 where the fp32 x / scale_a is outside
    [-1, 1]; grad_scale_a = sum(grad_in * sign0(x)) / sqrt(M * K)."""
    g, w, x = _cpu(g), _cpu(w), _cpu(x)
    m, n = g.shape
    n2, k = w.shape
    assert n == n2 and tuple(x.shape) == (m, k)
    out = torch.empty((m, k), dtype=torch.float64)
    gsa = ctypes.c_double(0.0)
    _load().oracle_linear_grad_input(g.data_ptr(), _code(g), w.data_ptr(), _code(w), x.data_ptr(),
                                     _code(x), m, n, k, float(scale_a), float(scale_w),
                                     out.data_ptr(), ctypes.addressof(gsa))
    return out, gsa.value


def linear_grad_weight(g: torch.Tensor, x: torch.Tensor, scale_a: float) -> torch.Tensor:
    """Straight-through backward of the binarized linear layer, weight side: float64 [N, K] =
    g^T @ (sign0(x) * scale_a) for g [M, N], x [M, K]."""
    g, x = _cpu(g), _cpu(x)
    m, n = g.shape
    assert x.shape[0] == m
    k = x.shape[1]
    out = torch.empty((n, k), dtype=torch.float64)
    _load().oracle_linear_grad_weight(g.data_ptr(), _code(g), x.data_ptr(), _code(x), m, n, k,
                                      float(scale_a), out.data_ptr())
    return out


def quant_grad_i8(grad_w: torch.Tensor):
    """int8 codes of a gradient held in fp32 (the conv page's nv_tensor_quant read as the per-tensor
    symmetric quantizer with amax = max|v|): returns (codes int8, same shape; amax float)."""
    gw = _cpu(grad_w).to(torch.float64).contiguous()
    codes = torch.empty(gw.shape, dtype=torch.int8)
    amax = ctypes.c_float(0.0)
    _load().oracle_quant_grad_i8(gw.data_ptr(), gw.numel(), codes.data_ptr(), ctypes.addressof(amax))
    return codes, amax.value


def conv2d_grad(g: torch.Tensor, w: torch.Tensor, x: torch.Tensor, stride, padding, dilation,
                scale_a: float, scale_w: float):
    """Straight-through backward of the binarized conv: returns (grad_in float64 [B, C, H, W],
    grad_scale_a float, grad_w float64 [O, C, KH, KW]) for g [B, O, Ho, Wo], W [O, C, KH, KW],
    x [B, C, H, W]; stride / padding / dilation are ints or (rows, columns) pairs."""
    g, w, x = _cpu(g), _cpu(w), _cpu(x)
    b, c, h, wd = x.shape
    o, c2, kh, kw = w.shape
    assert c == c2 and g.shape[0] == b and g.shape[1] == o
    (sh, sw), (ph, pw), (dh, dw) = _pair(stride), _pair(padding), _pair(dilation)
    assert tuple(g.shape[2:]) == (conv_out_size(h, kh, sh, ph, dh), conv_out_size(wd, kw, sw, pw, dw))
    gi = torch.empty((b, c, h, wd), dtype=torch.float64)
    gw = torch.empty((o, c, kh, kw), dtype=torch.float64)
    gsa = ctypes.c_double(0.0)
    rc = _load().oracle_conv2d_grad(g.data_ptr(), _code(g), w.data_ptr(), _code(w), x.data_ptr(), _code(x),
                                    b, c, h, wd, o, kh, kw, sh, sw, ph, pw, dh, dw, float(scale_a),
                                    float(scale_w), gi.data_ptr(), ctypes.addressof(gsa), gw.data_ptr())
    if rc != 0:
        raise RuntimeError("oracle_conv2d_grad failed")
    return gi, gsa.value, gw
