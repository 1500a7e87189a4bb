"""Binarized linear / conv2d forward for MI355X (gfx950): Python binding of libbnn.

The compute runs in libbnn.so (hand-written HIP kernels behind a C ABI, see
include/bnn.h); this module only marshals arguments with ctypes. PyTorch is
used for device memory (the caller's tensors, output and workspace
allocations) and for the current HIP stream. There is no fallback: if
libbnn.so is missing, importing the module raises.

Entry points mirror the C ABI:
  pack_sign(x)              rows of x -> packed int32 words [rows, ceil(k/32)]
  pack_sign_nchw(x)         NCHW x -> packed words [n, h, w, ceil(c/32)]
  pack_sign_shift(x, bias)  rows of x + bias (one value or one per column) -> packed words
  pack_sign_nchw_shift(x, bias)  NCHW x + bias[c] -> packed words [n, h, w, ceil(c/32)]
  abs_mean_scale(x, factor) factor * mean|x| as a 0-dim float64 device tensor
  w_pack(weight)            linear [out, in] or OIHW conv weight -> packed words
  gemm(x, w_packed, ...)    binary linear forward (bitorch-engine BinaryLinearForward)
  conv2d(x, w_packed, ...)  binary conv2d forward (bitorch-engine BinaryConv2dForward)
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# BNN_LIBRARY may name another build of libbnn.so (e.g. one compiled with different tile
# parameters); the default is the in-tree build.
LIB_PATH = os.environ.get("BNN_LIBRARY") or os.path.join(_PKG, "libbnn.so")

# size of bnn_gemm_noalloc's static device array (BNN_NOALLOC_SCRATCH_BYTES of include/bnn.h)
NOALLOC_SCRATCH_BYTES = 32 << 20

# bnn_dtype / bnn_path / bnn_status codes of include/bnn.h
F32, F16, BF16, I32, U32_PACKED, U8_PACKED = 0, 1, 2, 3, 4, 5
PATH_AUTO, PATH_XOR, PATH_MFMA, PATH_MFMA_FP4 = 0, 1, 2, 3
OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_WORKSPACE, ERR_PATH, ERR_HIP = range(8)

EXPORTS = ("bnn_pack_sign", "bnn_pack_sign_nchw", "bnn_pack_sign_shift", "bnn_pack_sign_nchw_shift",
           "bnn_abs_mean_scale", "bnn_abs_mean_workspace_bytes", "bnn_pack_sign_shift_abs_mean",
           "bnn_pack_sign_shift_abs_mean_workspace_bytes", "bnn_pack_sign_nchw_shift_abs_mean",
           "bnn_pack_sign_nchw_shift_abs_mean_workspace_bytes", "bnn_w_pack", "bnn_w_pack_conv",
           "bnn_conv2d_ex", "bnn_quant_i8_nhwc", "bnn_quant_i8_weight", "bnn_w8a8_conv2d", "bnn_gemm", "bnn_conv2d",
           "bnn_gemm_noalloc", "bnn_u8_to_words", "bnn_conv2d_grad_input",
           "bnn_conv2d_grad_input_workspace_bytes", "bnn_conv2d_grad_weight",
           "bnn_conv2d_grad_weight_workspace_bytes", "bnn_gemm_workspace_bytes", "bnn_conv2d_workspace_bytes", "bnn_gemm_auto_path",
           "bnn_conv2d_auto_path", "bnn_last_path", "bnn_status_string",
           "bnn_linear_grad_input", "bnn_linear_grad_input_workspace_bytes", "bnn_linear_grad_weight",
           "bnn_linear_grad_weight_i8", "bnn_linear_grad_weight_i8_workspace_bytes",
           "bnn_quant_grad_i8", "bnn_quant_grad_i8_workspace_bytes")

_PATHS = {"auto": PATH_AUTO, "xor": PATH_XOR, "mfma": PATH_MFMA, "mfma_fp4": PATH_MFMA_FP4}
_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.int32: I32}
_TORCH = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16, I32: torch.int32}


def _bind(path: str) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    P, I64, I, D, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_size_t
    F = ctypes.c_float
    sig = {
        "bnn_pack_sign": ([P, I, I64, I64, P, P], I),
        "bnn_pack_sign_nchw": ([P, I, I64, I64, I64, I64, P, P], I),
        "bnn_pack_sign_shift": ([P, I, I64, I64, P, I, I64, P, P], I),
        "bnn_pack_sign_nchw_shift": ([P, I, I64, I64, I64, I64, P, I, P, P], I),
        "bnn_abs_mean_scale": ([P, I, I64, D, P, P, SZ, P], I),
        "bnn_abs_mean_workspace_bytes": ([I64], SZ),
        "bnn_pack_sign_shift_abs_mean": ([P, I, I64, I64, P, I, I64, D, P, P, P, SZ, P], I),
        "bnn_pack_sign_shift_abs_mean_workspace_bytes": ([I64, I64], SZ),
        "bnn_pack_sign_nchw_shift_abs_mean": ([P, I, I64, I64, I64, I64, P, I, D, P, P, P, SZ, P], I),
        "bnn_pack_sign_nchw_shift_abs_mean_workspace_bytes": ([I, I64, I64, I64, I64], SZ),
        "bnn_linear_grad_input": ([P, P, P, I, I64, I64, I64, F, F, P, P, P, SZ, P], I),
        "bnn_linear_grad_input_workspace_bytes": ([I64, I64], SZ),
        "bnn_linear_grad_weight": ([P, P, I, I64, I64, I64, F, P, P], I),
        "bnn_linear_grad_weight_i8": ([P, P, I, I64, I64, I64, F, P, P, P, P, SZ, P], I),
        "bnn_linear_grad_weight_i8_workspace_bytes": ([I64, I64], SZ),
        "bnn_quant_grad_i8": ([P, I64, P, P, P, SZ, P], I),
        "bnn_quant_grad_i8_workspace_bytes": ([I64], SZ),
        "bnn_w_pack": ([P, I, I64, I64, I, P, P], I),
        "bnn_w_pack_conv": ([P, I, I64, I64, I, I, P, P], I),
        "bnn_quant_i8_nhwc": ([P, I, I64, I64, I64, I64, D, P, P], I),
        "bnn_quant_i8_weight": ([P, I, I64, I64, I, I, D, P, P], I),
        "bnn_w8a8_conv2d": ([P, I64, I64, I64, I64, P, I64, D, D] + [I] * 8 + [P, I, P], I),
        "bnn_conv2d_ex": ([P, I, I64, I64, I64, I64, P, I64, D, D] + [I] * 9 + [P, I, P, SZ, P], I),
        "bnn_gemm": ([P, I, P, I64, I64, I64, D, D, I, P, I, P, SZ, P], I),
        "bnn_gemm_noalloc": ([P, I, P, I64, I64, I64, D, D, I, P, I, P], I),
        "bnn_u8_to_words": ([P, I64, I64, P, P], I),
        "bnn_conv2d_grad_input": ([P, P, P, I] + [I64] * 5 + [I] * 8 + [F, F, P, P, P, SZ, P], I),
        "bnn_conv2d_grad_input_workspace_bytes": ([I64] * 5 + [I] * 8, SZ),
        "bnn_conv2d_grad_weight": ([P, P, I] + [I64] * 5 + [I] * 8 + [F, P, P, P, P, SZ, P], I),
        "bnn_conv2d_grad_weight_workspace_bytes": ([I64] * 5 + [I] * 8, SZ),
        "bnn_conv2d": ([P, I, I64, I64, I64, I64, P, I64, D, D, I, I, I, I, I, P, I, P, SZ, P], I),
        "bnn_gemm_workspace_bytes": ([I64, I64, I], SZ),
        "bnn_conv2d_workspace_bytes": ([I64, I64, I64, I64, I], SZ),
        "bnn_gemm_auto_path": ([I64, I64, I64], I),
        "bnn_conv2d_auto_path": ([I64, I64, I64, I64, I64, I, I, I, I], I),
        "bnn_last_path": ([], I),
        "bnn_status_string": ([I], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
lib = _bind(LIB_PATH)


class BnnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.bnn_status_string(status).decode()} (status {status})")


def _check(status: int, where: str):
    if status == OK:
        return
    if status == ERR_SHAPE:
        # a size the ABI rejects (e.g. a reduction length that is not a whole number of 32-bit
        # words) is an AssertionError, the exception type the layers use for that check
        raise AssertionError(f"{where}: {lib.bnn_status_string(status).decode()}")
    raise BnnError(status, where)


# Device types accepted for tensor arguments (HIP devices appear as "cuda" in torch).
_DEVICE_TYPES = ("cuda",)


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.device.type not in _DEVICE_TYPES:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _expect(t: torch.Tensor, name: str, dtype, shape) -> torch.Tensor:
    """Raise before any library call unless t (a device tensor) has exactly this dtype (one
    dtype or a tuple of allowed ones) and shape: the C ABI takes raw pointers, so a wrongly
    sized buffer would be read or written out of bounds on the device."""
    _dev(t, name)
    allowed = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in allowed:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in allowed)}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


_OUT_DTYPES = (torch.float32, torch.float16, torch.bfloat16, torch.int32)


def _packed_len(x: torch.Tensor, n: int | None, what: str) -> int:
    """Sign count of a packed tensor whose last axis holds the containers (int32 words of 32
    signs, or uint8 bytes of 8): n when given (it must need exactly that many containers), else
    32 or 8 per container."""
    per = 32 if x.dtype == torch.int32 else 8
    cw = x.shape[-1]
    if n is None:
        return per * cw
    n = int(n)
    if n < 1 or (n + per - 1) // per != cw:
        raise ValueError(f"{what} = {n} needs {(max(n, 1) + per - 1) // per} packed containers of "
                         f"{per} signs, x holds {cw}")
    return n


def _packed_code(x: torch.Tensor):
    """U32_PACKED for int32 words, U8_PACKED for uint8 containers, None for float input."""
    return {torch.int32: U32_PACKED, torch.uint8: U8_PACKED}.get(x.dtype)


def _same_device(name: str, t: torch.Tensor, ref: torch.Tensor):
    if t.device != ref.device:
        raise ValueError(f"{name} must be on {ref.device}, got {t.device}")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _path(path) -> int:
    if isinstance(path, str):
        return _PATHS[path.lower()]
    return int(path)


def _dtype_code(t: torch.Tensor, name: str) -> int:
    if t.dtype not in (torch.float32, torch.float16, torch.bfloat16):
        raise TypeError(f"{name} must be float32, float16 or bfloat16, got {t.dtype}")
    return _DT[t.dtype]


def words(n: int) -> int:
    """Packed words holding n signs (the last one partly when n % 32 != 0)."""
    return (n + 31) // 32


def pack_sign(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Sign+pack along the last axis: [rows, k] -> int32 words [rows, ceil(k/32)]."""
    x = _dev(x, "x")
    k = x.shape[-1]
    rows = x.numel() // k if k else 0
    if out is None:
        out = torch.empty((*x.shape[:-1], words(k)), dtype=torch.int32, device=x.device)
    else:
        _expect(out, "out", torch.int32, (*x.shape[:-1], words(k)))
        _same_device("out", out, x)
    _check(lib.bnn_pack_sign(x.data_ptr(), _dtype_code(x, "x"), rows, k, out.data_ptr(), _stream(x)),
           "bnn_pack_sign")
    return out


def pack_sign_nchw(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Sign+pack of NCHW activations along channels: [n, c, h, w] -> int32 words [n, h, w, ceil(c/32)]."""
    x = _dev(x, "x")
    if x.dim() != 4:
        raise ValueError(f"x must be NCHW (4-D), got {x.dim()}-D")
    n, c, h, w = x.shape
    if out is None:
        out = torch.empty((n, h, w, words(c)), dtype=torch.int32, device=x.device)
    else:
        _expect(out, "out", torch.int32, (n, h, w, words(c)))
        _same_device("out", out, x)
    _check(lib.bnn_pack_sign_nchw(x.data_ptr(), _dtype_code(x, "x"), n, c, h, w, out.data_ptr(),
                                  _stream(x)), "bnn_pack_sign_nchw")
    return out


def _bias(bias: torch.Tensor, x: torch.Tensor) -> torch.Tensor:
    bias = _dev(bias, "bias")
    if bias.device != x.device:
        raise ValueError("bias must be on x's device")
    return bias


def pack_sign_shift(x: torch.Tensor, bias: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Shifted sign+pack along the last axis (the linear layer's activation prologue):
    bit = (x + bias >= 0) with bias one value ([1] or 0-dim) or one per column ([k])."""
    x = _dev(x, "x")
    bias = _bias(bias, x)
    k = x.shape[-1]
    rows = x.numel() // k if k else 0
    if bias.numel() not in (1, k):
        raise ValueError(f"bias must hold one value or one per column ({k}), got {bias.numel()}")
    if out is None:
        out = torch.empty((*x.shape[:-1], words(k)), dtype=torch.int32, device=x.device)
    else:
        _expect(out, "out", torch.int32, (*x.shape[:-1], words(k)))
        _same_device("out", out, x)
    _check(lib.bnn_pack_sign_shift(x.data_ptr(), _dtype_code(x, "x"), rows, k, bias.data_ptr(),
                                   _dtype_code(bias, "bias"), bias.numel(), out.data_ptr(),
                                   _stream(x)), "bnn_pack_sign_shift")
    return out


def pack_sign_nchw_shift(x: torch.Tensor, bias: torch.Tensor,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """Shifted sign+pack of NCHW activations (the conv layer's activation prologue):
    bit = (x[n, c, h, w] + bias[c] >= 0) -> int32 words [n, h, w, ceil(c/32)]."""
    x = _dev(x, "x")
    bias = _bias(bias, x)
    if x.dim() != 4:
        raise ValueError(f"x must be NCHW (4-D), got {x.dim()}-D")
    n, c, h, w = x.shape
    if bias.numel() != c:
        raise ValueError(f"bias must hold one value per channel ({c}), got {bias.numel()}")
    if out is None:
        out = torch.empty((n, h, w, words(c)), dtype=torch.int32, device=x.device)
    else:
        _expect(out, "out", torch.int32, (n, h, w, words(c)))
        _same_device("out", out, x)
    _check(lib.bnn_pack_sign_nchw_shift(x.data_ptr(), _dtype_code(x, "x"), n, c, h, w,
                                        bias.data_ptr(), _dtype_code(bias, "bias"), out.data_ptr(),
                                        _stream(x)), "bnn_pack_sign_nchw_shift")
    return out


def abs_mean_scale(x: torch.Tensor, factor: float, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """factor * mean|x| over every element (the layers' lazy scale_a init, factor 2 or 4),
    as a 0-dim float64 device tensor; no host synchronisation."""
    x = _dev(x, "x")
    if out is None:
        out = torch.empty((), dtype=torch.float64, device=x.device)
    else:
        _expect(out, "out", torch.float64, ())
        _same_device("out", out, x)
    need = lib.bnn_abs_mean_workspace_bytes(x.numel())
    if workspace is None:
        workspace = _workspace(need, x.device)
    else:
        _dev(workspace, "workspace")
        _same_device("workspace", workspace, x)
    _check(lib.bnn_abs_mean_scale(x.data_ptr(), _dtype_code(x, "x"), x.numel(), float(factor),
                                  out.data_ptr(), workspace.data_ptr(),
                                  _nbytes(workspace), _stream(x)),
           "bnn_abs_mean_scale")
    return out


def _scale_out(out, x):
    if out is None:
        return torch.empty((), dtype=torch.float64, device=x.device)
    _expect(out, "scale_out", torch.float64, ())
    _same_device("scale_out", out, x)
    return out


def _prologue_workspace(workspace, need, x):
    if workspace is None:
        return _workspace(need, x.device)
    _dev(workspace, "workspace")
    _same_device("workspace", workspace, x)
    return workspace


def pack_sign_shift_abs_mean(x: torch.Tensor, bias: torch.Tensor, factor: float,
                             out: torch.Tensor | None = None, scale_out: torch.Tensor | None = None,
                             workspace: torch.Tensor | None = None):
    """One-pass prologue of the linear layer: (pack_sign_shift(x, bias), factor * mean|x|) from a
    single read of x; the scale is a 0-dim float64 device tensor."""
    x = _dev(x, "x")
    bias = _bias(bias, x)
    k = x.shape[-1]
    rows = x.numel() // k if k else 0
    if bias.numel() not in (1, k):
        raise ValueError(f"bias must hold one value or one per column ({k}), got {bias.numel()}")
    if out is None:
        out = torch.empty((*x.shape[:-1], words(k)), dtype=torch.int32, device=x.device)
    else:
        _expect(out, "out", torch.int32, (*x.shape[:-1], words(k)))
        _same_device("out", out, x)
    scale_out = _scale_out(scale_out, x)
    workspace = _prologue_workspace(workspace, lib.bnn_pack_sign_shift_abs_mean_workspace_bytes(rows, k), x)
    _check(lib.bnn_pack_sign_shift_abs_mean(x.data_ptr(), _dtype_code(x, "x"), rows, k, bias.data_ptr(),
                                            _dtype_code(bias, "bias"), bias.numel(), float(factor),
                                            out.data_ptr(), scale_out.data_ptr(), workspace.data_ptr(),
                                            _nbytes(workspace), _stream(x)),
           "bnn_pack_sign_shift_abs_mean")
    return out, scale_out


def pack_sign_nchw_shift_abs_mean(x: torch.Tensor, bias: torch.Tensor, factor: float,
                                  out: torch.Tensor | None = None, scale_out: torch.Tensor | None = None,
                                  workspace: torch.Tensor | None = None):
    """One-pass prologue of the conv layer: (pack_sign_nchw_shift(x, bias), factor * mean|x|)
    from a single read of x; the scale is a 0-dim float64 device tensor."""
    x = _dev(x, "x")
    bias = _bias(bias, x)
    if x.dim() != 4:
        raise ValueError(f"x must be NCHW (4-D), got {x.dim()}-D")
    n, c, h, w = x.shape
    if bias.numel() != c:
        raise ValueError(f"bias must hold one value per channel ({c}), got {bias.numel()}")
    if out is None:
        out = torch.empty((n, h, w, words(c)), dtype=torch.int32, device=x.device)
    else:
        _expect(out, "out", torch.int32, (n, h, w, words(c)))
        _same_device("out", out, x)
    scale_out = _scale_out(scale_out, x)
    code = _dtype_code(x, "x")
    need = lib.bnn_pack_sign_nchw_shift_abs_mean_workspace_bytes(code, n, c, h, w)
    workspace = _prologue_workspace(workspace, need, x)
    _check(lib.bnn_pack_sign_nchw_shift_abs_mean(x.data_ptr(), code, n, c, h, w, bias.data_ptr(),
                                                 _dtype_code(bias, "bias"), float(factor), out.data_ptr(),
                                                 scale_out.data_ptr(), workspace.data_ptr(),
                                                 _nbytes(workspace), _stream(x)),
           "bnn_pack_sign_nchw_shift_abs_mean")
    return out, scale_out


def w_pack(weight: torch.Tensor) -> torch.Tensor:
    """Weight pack: linear [out, in] -> [out, ceil(in/32)]; OIHW [out, in, kh, kw] ->
    [out, kh, kw, ceil(in/32)] (square kernels through bnn_w_pack, others bnn_w_pack_conv)."""
    weight = _dev(weight, "weight")
    code = _dtype_code(weight, "weight")
    if weight.dim() == 2:
        o, i = weight.shape
        out = torch.empty((o, words(i)), dtype=torch.int32, device=weight.device)
        _check(lib.bnn_w_pack(weight.data_ptr(), code, o, i, 0, out.data_ptr(), _stream(weight)),
               "bnn_w_pack")
    elif weight.dim() == 4:
        o, i, kh, kw = weight.shape
        out = torch.empty((o, kh, kw, words(i)), dtype=torch.int32, device=weight.device)
        if kh == kw:
            _check(lib.bnn_w_pack(weight.data_ptr(), code, o, i, kh, out.data_ptr(), _stream(weight)),
                   "bnn_w_pack")
        else:
            _check(lib.bnn_w_pack_conv(weight.data_ptr(), code, o, i, kh, kw, out.data_ptr(),
                                       _stream(weight)), "bnn_w_pack_conv")
    else:
        raise ValueError("weight must be 2-D (linear) or 4-D OIHW (conv)")
    return out


def u8_to_words(src: torch.Tensor, bits: int | None = None,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """8-bit sign containers [..., ceil(bits/8)] uint8 (the CUTLASS layer's container type) ->
    int32 words [..., ceil(bits/32)] with the bits past `bits` cleared; bits defaults to 8 per
    byte. Serves weights ([o, kh, kw, ceil(c/8)] -> w_packed) and activations alike."""
    src = _dev(src, "src")
    if src.dtype != torch.uint8 or src.dim() < 1:
        raise TypeError("src must be a uint8 tensor whose last axis holds the containers")
    bits = _packed_len(src, bits, "bits")
    rows = src.numel() // src.shape[-1] if src.shape[-1] else 0
    if out is None:
        out = torch.empty((*src.shape[:-1], words(bits)), dtype=torch.int32, device=src.device)
    else:
        _expect(out, "out", torch.int32, (*src.shape[:-1], words(bits)))
        _same_device("out", out, src)
    _check(lib.bnn_u8_to_words(src.data_ptr(), rows, bits, out.data_ptr(), _stream(src)),
           "bnn_u8_to_words")
    return out


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _nbytes(t: torch.Tensor | None) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def gemm(x: torch.Tensor, w_packed: torch.Tensor, scale_a: float, scale_w: float, path="auto",
         out_dtype=None, k: int | None = None, out: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Binary linear forward: out = scale_a*scale_w * sgn(x) @ sgn(W)^T.

    x is [m, k] float (packed here), int32 [m, ceil(k/32)] already packed (then k defaults to
    32 * x.shape[1]; pass k when it is not a multiple of 32), or uint8 [m, ceil(k/8)] 8-bit
    containers (k defaults to 8 * x.shape[1]). w_packed is int32 [n, ceil(k/32)] from w_pack.
    out_dtype defaults to x's dtype (float32 for packed x); torch.int32 gives
    the raw accumulators.
    """
    x = _dev(x, "x")
    w_packed = _dev(w_packed, "w_packed")
    _same_device("w_packed", w_packed, x)
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D [m, k] (or packed [m, words]), got {x.dim()}-D")
    packed = _packed_code(x) is not None
    m = x.shape[0]
    if packed:
        k = _packed_len(x, k, "k")
        xcode = _packed_code(x)
    else:
        k = x.shape[1]
        xcode = _dtype_code(x, "x")
    if w_packed.dim() != 2:
        raise ValueError(f"w_packed must be 2-D [n, words(k)], got {w_packed.dim()}-D")
    n = w_packed.shape[0]
    _expect(w_packed, "w_packed", torch.int32, (n, words(k)))
    if out_dtype is None:
        out_dtype = torch.float32 if packed else x.dtype
    if out is None:
        if out_dtype not in _OUT_DTYPES:
            raise TypeError(f"out_dtype must be one of {_OUT_DTYPES}, got {out_dtype}")
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    else:
        _expect(out, "out", _OUT_DTYPES, (m, n))
        _same_device("out", out, x)
    ws_bytes = lib.bnn_gemm_workspace_bytes(m, k, xcode)
    if workspace is None and ws_bytes:
        workspace = _workspace(ws_bytes, x.device)
    elif workspace is not None:
        _dev(workspace, "workspace")
        _same_device("workspace", workspace, x)
    _check(lib.bnn_gemm(x.data_ptr(), xcode, w_packed.data_ptr(), m, n, k, float(scale_a),
                        float(scale_w), _path(path), out.data_ptr(), _DT[out.dtype],
                        workspace.data_ptr() if workspace is not None else None,
                        _nbytes(workspace), _stream(x)), "bnn_gemm")
    return out


def gemm_noalloc(x: torch.Tensor, w_packed: torch.Tensor, scale_a: float, scale_w: float,
                 out: torch.Tensor, path="auto", k: int | None = None) -> torch.Tensor:
    """gemm without any device allocation: the caller passes `out`, and float activations are
    packed into the library's static device array (at most NOALLOC_SCRATCH_BYTES; calls that
    overlap on one device race for it)."""
    x = _dev(x, "x")
    w_packed = _dev(w_packed, "w_packed")
    _same_device("w_packed", w_packed, x)
    if x.dim() != 2 or w_packed.dim() != 2:
        raise ValueError("x and w_packed must be 2-D")
    packed = _packed_code(x) is not None
    m = x.shape[0]
    k = _packed_len(x, k, "k") if packed else x.shape[1]
    xcode = _packed_code(x) if packed else _dtype_code(x, "x")
    n = w_packed.shape[0]
    _expect(w_packed, "w_packed", torch.int32, (n, words(k)))
    _expect(out, "out", _OUT_DTYPES, (m, n))
    _same_device("out", out, x)
    _check(lib.bnn_gemm_noalloc(x.data_ptr(), xcode, w_packed.data_ptr(), m, n, k, float(scale_a),
                                float(scale_w), _path(path), out.data_ptr(), _DT[out.dtype],
                                _stream(x)), "bnn_gemm_noalloc")
    return out


def _pair(v, name):
    if isinstance(v, int):
        return v, v
    if len(v) != 2:
        raise ValueError(f"{name} must be an int or a (rows, columns) pair")
    return int(v[0]), int(v[1])


def conv2d(x: torch.Tensor, w_packed: torch.Tensor, scale_a: float, scale_w: float,
           kernel_size, stride=1, padding=0, dilation=1, path="auto",
           out_dtype=None, channels: int | None = None, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Binary conv2d forward, NCHW in and out; padded taps contribute 0.

    x is [n, c, h, w] float, int32 [n, h, w, ceil(c/32)] already packed by pack_sign_nchw, or
    uint8 [n, h, w, ceil(c/8)] 8-bit containers (pass channels when c is not a multiple of the
    container width). w_packed is int32 [o, kh, kw, ceil(c/32)] from w_pack. kernel_size,
    stride, padding and dilation are ints (bnn_conv2d) or (rows, columns) pairs
    (bnn_conv2d_ex).
    """
    x = _dev(x, "x")
    w_packed = _dev(w_packed, "w_packed")
    _same_device("w_packed", w_packed, x)
    if x.dim() != 4:
        raise ValueError(f"x must be 4-D (NCHW float or packed [n, h, w, words]), got {x.dim()}-D")
    packed = _packed_code(x) is not None
    if packed:
        n, h, w, cw = x.shape
        c = _packed_len(x, channels, "channels")
        xcode = _packed_code(x)
    else:
        n, c, h, w = x.shape
        xcode = _dtype_code(x, "x")
    (kh, kw), (sh, sw) = _pair(kernel_size, "kernel_size"), _pair(stride, "stride")
    (ph, pw), (dh, dw) = _pair(padding, "padding"), _pair(dilation, "dilation")
    if w_packed.dim() != 4:
        raise ValueError(f"w_packed must be 4-D [o, kh, kw, words(c)], got {w_packed.dim()}-D")
    o = w_packed.shape[0]
    _expect(w_packed, "w_packed", torch.int32, (o, kh, kw, words(c)))
    ho = (h + 2 * ph - dh * (kh - 1) - 1) // sh + 1 if sh > 0 else 0
    wo = (w + 2 * pw - dw * (kw - 1) - 1) // sw + 1 if sw > 0 else 0
    if out_dtype is None:
        out_dtype = torch.float32 if packed else x.dtype
    if out is None:
        if out_dtype not in _OUT_DTYPES:
            raise TypeError(f"out_dtype must be one of {_OUT_DTYPES}, got {out_dtype}")
        out = torch.empty((n, o, max(ho, 0), max(wo, 0)), dtype=out_dtype, device=x.device)
    else:
        _expect(out, "out", _OUT_DTYPES, (n, o, max(ho, 0), max(wo, 0)))
        _same_device("out", out, x)
    ws_bytes = lib.bnn_conv2d_workspace_bytes(n, c, h, w, xcode)
    if workspace is None and ws_bytes:
        workspace = _workspace(ws_bytes, x.device)
    elif workspace is not None:
        _dev(workspace, "workspace")
        _same_device("workspace", workspace, x)
    wsp = workspace.data_ptr() if workspace is not None else None
    wsn = _nbytes(workspace)
    common = (x.data_ptr(), xcode, n, c, h, w, w_packed.data_ptr(), o, float(scale_a), float(scale_w))
    if kh == kw and sh == sw and ph == pw and dh == dw:
        _check(lib.bnn_conv2d(*common, kh, sh, ph, dh, _path(path), out.data_ptr(), _DT[out.dtype],
                              wsp, wsn, _stream(x)), "bnn_conv2d")
    else:
        _check(lib.bnn_conv2d_ex(*common, kh, kw, sh, sw, ph, pw, dh, dw, _path(path),
                                 out.data_ptr(), _DT[out.dtype], wsp, wsn, _stream(x)),
               "bnn_conv2d_ex")
    return out


def last_path() -> int:
    return lib.bnn_last_path()


def gemm_auto_path(m: int, n: int, k: int) -> int:
    return lib.bnn_gemm_auto_path(m, n, k)


def conv2d_auto_path(n, c, h, w, o, kernel_size, stride=1, padding=0, dilation=1) -> int:
    return lib.bnn_conv2d_auto_path(n, c, h, w, o, kernel_size, stride, padding, dilation)


# ---- W8A8 conv (int8 codes of per-tensor symmetric quantizers; see include/bnn.h)

def quant_i8_nhwc(x: torch.Tensor, amax: float) -> torch.Tensor:
    """NCHW float -> NHWC int8 codes clamp(rint(x / (amax/127)), -127, 127)."""
    x = _dev(x, "x")
    n, c, h, w = x.shape
    out = torch.empty((n, h, w, c), dtype=torch.int8, device=x.device)
    _check(lib.bnn_quant_i8_nhwc(x.data_ptr(), _dtype_code(x, "x"), n, c, h, w, float(amax),
                                 out.data_ptr(), _stream(x)), "bnn_quant_i8_nhwc")
    return out


def quant_i8_weight(weight: torch.Tensor, amax: float) -> torch.Tensor:
    """OIHW float -> int8 codes [o, kh, kw, c]."""
    weight = _dev(weight, "weight")
    o, c, kh, kw = weight.shape
    out = torch.empty((o, kh, kw, c), dtype=torch.int8, device=weight.device)
    _check(lib.bnn_quant_i8_weight(weight.data_ptr(), _dtype_code(weight, "weight"), o, c, kh, kw,
                                   float(amax), out.data_ptr(), _stream(weight)), "bnn_quant_i8_weight")
    return out


def w8a8_conv2d(x_q: torch.Tensor, w_q: torch.Tensor, amax_x: float, amax_w: float, kernel_size,
                stride=1, padding=0, dilation=1, out_dtype=torch.float32,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """W8A8 conv on int8 codes: x_q NHWC [n, h, w, c], w_q [o, kh, kw, c]; NCHW output
    (amax_x/127) * (amax_w/127) * sum q_x q_w, or the raw int32 sums for out_dtype=torch.int32."""
    x_q, w_q = _dev(x_q, "x_q"), _dev(w_q, "w_q")
    _same_device("w_q", w_q, x_q)
    if x_q.dim() != 4 or w_q.dim() != 4 or x_q.dtype != torch.int8 or w_q.dtype != torch.int8:
        raise ValueError("x_q [n, h, w, c] and w_q [o, kh, kw, c] must be 4-D int8 tensors")
    n, h, w, c = x_q.shape
    o, kh, kw, c2 = w_q.shape
    if c != c2:
        raise ValueError("x_q and w_q disagree on the channel count")
    if tuple(_pair(kernel_size, "kernel_size")) != (kh, kw):
        raise ValueError("kernel_size does not match w_q")
    (sh, sw), (ph, pw), (dh, dw) = _pair(stride, "stride"), _pair(padding, "padding"), _pair(dilation, "dilation")
    ho = (h + 2 * ph - dh * (kh - 1) - 1) // sh + 1 if sh > 0 else 0
    wo = (w + 2 * pw - dw * (kw - 1) - 1) // sw + 1 if sw > 0 else 0
    if out is None:
        if out_dtype not in _OUT_DTYPES:
            raise TypeError(f"out_dtype must be one of {_OUT_DTYPES}, got {out_dtype}")
        out = torch.empty((n, o, max(ho, 0), max(wo, 0)), dtype=out_dtype, device=x_q.device)
    else:
        _expect(out, "out", _OUT_DTYPES, (n, o, max(ho, 0), max(wo, 0)))
        _same_device("out", out, x_q)
    _check(lib.bnn_w8a8_conv2d(x_q.data_ptr(), n, c, h, w, w_q.data_ptr(), o, float(amax_x),
                               float(amax_w), kh, kw, sh, sw, ph, pw, dh, dw, out.data_ptr(),
                               _DT[out.dtype], _stream(x_q)), "bnn_w8a8_conv2d")
    return out


def _half_pair(t: torch.Tensor, name: str) -> int:
    if t.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError(f"{name} must be float16 or bfloat16, got {t.dtype}")
    return _DT[t.dtype]


def linear_grad_input(grad_out: torch.Tensor, weight: torch.Tensor, x: torch.Tensor,
                      scale_a: float, scale_w: float, out: torch.Tensor | None = None,
                      grad_scale_a: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None):
    """Straight-through backward of the binarized linear layer, input side. grad_out [M, N],
    weight [N, K] (the float weight) and x [M, K] share one 16-bit dtype. Returns
    (grad_input fp32 [M, K], grad_scale_a 0-dim float64), both on the device:
    grad_input = (scale_w * grad_out @ sign(weight)) * mid(x), mid = 0 where the fp32
    x / scale_a is outside [-1, 1]; grad_scale_a = sum(grad_input * sign(x)) / sqrt(M * K)."""
    g, w, x = _dev(grad_out, "grad_out"), _dev(weight, "weight"), _dev(x, "x")
    dt = _half_pair(g, "grad_out")
    if w.dtype != g.dtype or x.dtype != g.dtype:
        raise TypeError("grad_out, weight and x must share one dtype")
    if g.dim() != 2 or w.dim() != 2 or x.dim() != 2:
        raise ValueError("grad_out, weight and x must be 2-D")
    _same_device("weight", w, g)
    _same_device("x", x, g)
    m, n = g.shape
    n2, k = w.shape
    if n2 != n or tuple(x.shape) != (m, k):
        raise ValueError(f"shape mismatch: grad_out {tuple(g.shape)}, weight {tuple(w.shape)}, x {tuple(x.shape)}")
    if out is None:
        out = torch.empty((m, k), dtype=torch.float32, device=g.device)
    else:
        _expect(out, "out", torch.float32, (m, k))
        _same_device("out", out, g)
    if grad_scale_a is None:
        grad_scale_a = torch.empty((), dtype=torch.float64, device=g.device)
    else:
        _expect(grad_scale_a, "grad_scale_a", torch.float64, ())
        _same_device("grad_scale_a", grad_scale_a, g)
    need = lib.bnn_linear_grad_input_workspace_bytes(m, k)
    if workspace is None:
        workspace = _workspace(need, g.device)
    else:
        _dev(workspace, "workspace")
        _same_device("workspace", workspace, g)
    _check(lib.bnn_linear_grad_input(g.data_ptr(), w.data_ptr(), x.data_ptr(), dt, m, n, k,
                                     float(scale_a), float(scale_w), out.data_ptr(),
                                     grad_scale_a.data_ptr(), workspace.data_ptr(),
                                     _nbytes(workspace), _stream(g)),
           "bnn_linear_grad_input")
    return out, grad_scale_a


def linear_grad_weight(grad_out: torch.Tensor, x: torch.Tensor, scale_a: float,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """Straight-through backward of the binarized linear layer, weight side: fp32 [N, K] =
    scale_a * grad_out^T @ sign(x) for grad_out [M, N] and x [M, K] of one 16-bit dtype."""
    g, x = _dev(grad_out, "grad_out"), _dev(x, "x")
    dt = _half_pair(g, "grad_out")
    if x.dtype != g.dtype:
        raise TypeError("grad_out and x must share one dtype")
    if g.dim() != 2 or x.dim() != 2:
        raise ValueError("grad_out and x must be 2-D")
    _same_device("x", x, g)
    m, n = g.shape
    if x.shape[0] != m:
        raise ValueError(f"shape mismatch: grad_out {tuple(g.shape)}, x {tuple(x.shape)}")
    k = x.shape[1]
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=g.device)
    else:
        _expect(out, "out", torch.float32, (n, k))
        _same_device("out", out, g)
    _check(lib.bnn_linear_grad_weight(g.data_ptr(), x.data_ptr(), dt, m, n, k, float(scale_a),
                                      out.data_ptr(), _stream(g)), "bnn_linear_grad_weight")
    return out


def linear_grad_weight_i8(grad_out: torch.Tensor, x: torch.Tensor, scale_a: float):
    """grad_weight and its int8 codes (per-tensor symmetric, amax = max|grad_weight|): returns
    (grad_w fp32 [N, K], codes int8 [N, K], amax 0-dim float32), all on the device; the
    dequantized gradient is codes * amax / 127."""
    g, x = _dev(grad_out, "grad_out"), _dev(x, "x")
    dt = _half_pair(g, "grad_out")
    if x.dtype != g.dtype:
        raise TypeError("grad_out and x must share one dtype")
    if g.dim() != 2 or x.dim() != 2:
        raise ValueError("grad_out and x must be 2-D")
    _same_device("x", x, g)
    m, n = g.shape
    if x.shape[0] != m:
        raise ValueError(f"shape mismatch: grad_out {tuple(g.shape)}, x {tuple(x.shape)}")
    k = x.shape[1]
    gw = torch.empty((n, k), dtype=torch.float32, device=g.device)
    codes = torch.empty((n, k), dtype=torch.int8, device=g.device)
    amax = torch.empty((), dtype=torch.float32, device=g.device)
    ws = _workspace(lib.bnn_linear_grad_weight_i8_workspace_bytes(n, k), g.device)
    _check(lib.bnn_linear_grad_weight_i8(g.data_ptr(), x.data_ptr(), dt, m, n, k, float(scale_a),
                                         gw.data_ptr(), codes.data_ptr(), amax.data_ptr(),
                                         ws.data_ptr(), _nbytes(ws), _stream(g)),
           "bnn_linear_grad_weight_i8")
    return gw, codes, amax


def quant_grad_i8(grad: torch.Tensor):
    """int8 codes of an fp32 gradient (per-tensor symmetric, amax = max|grad|): returns (codes int8,
    same shape; amax 0-dim float32) on the device; numel must be a multiple of 4."""
    g = _dev(grad, "grad")
    if g.dtype != torch.float32:
        raise TypeError(f"grad must be float32, got {g.dtype}")
    codes = torch.empty(g.shape, dtype=torch.int8, device=g.device)
    amax = torch.empty((), dtype=torch.float32, device=g.device)
    ws = _workspace(lib.bnn_quant_grad_i8_workspace_bytes(g.numel()), g.device)
    _check(lib.bnn_quant_grad_i8(g.data_ptr(), g.numel(), codes.data_ptr(), amax.data_ptr(), ws.data_ptr(),
                                 _nbytes(ws), _stream(g)), "bnn_quant_grad_i8")
    return codes, amax


def _conv_bwd_geom(g, x, kernel_hw, stride, padding, dilation):
    """(n, c, h, w, o, kh, kw, sh, sw, ph, pw, dh, dw) after checking that g has the conv output's
    shape for x."""
    if g.dim() != 4 or x.dim() != 4:
        raise ValueError("grad_out and x must be 4-D (NCHW)")
    n, c, h, w = x.shape
    kh, kw = kernel_hw
    (sh, sw), (ph, pw), (dh, dw) = _pair(stride, "stride"), _pair(padding, "padding"), _pair(dilation, "dilation")
    ho = (h + 2 * ph - dh * (kh - 1) - 1) // sh + 1 if sh > 0 else 0
    wo = (w + 2 * pw - dw * (kw - 1) - 1) // sw + 1 if sw > 0 else 0
    o = g.shape[1]
    if tuple(g.shape) != (n, o, ho, wo):
        raise ValueError(f"grad_out must have shape {(n, o, ho, wo)}, got {tuple(g.shape)}")
    return n, c, h, w, o, kh, kw, sh, sw, ph, pw, dh, dw


def conv2d_grad_input(grad_out: torch.Tensor, weight: torch.Tensor, x: torch.Tensor,
                      scale_a: float, scale_w: float, stride=1, padding=0, dilation=1,
                      out: torch.Tensor | None = None, grad_scale_a: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None):
    """Straight-through backward of the binarized conv, input side: grad_out [n, o, Ho, Wo],
    weight [o, c, kh, kw] (the float weight) and x [n, c, h, w] of one 16-bit dtype. Returns
    (grad_input fp32 [n, c, h, w], grad_scale_a 0-dim float64), both on the device."""
    g, wt, x = _dev(grad_out, "grad_out"), _dev(weight, "weight"), _dev(x, "x")
    dt = _half_pair(g, "grad_out")
    if wt.dtype != g.dtype or x.dtype != g.dtype:
        raise TypeError("grad_out, weight and x must share one dtype")
    _same_device("weight", wt, g)
    _same_device("x", x, g)
    if wt.dim() != 4 or wt.shape[1] != x.shape[1] or wt.shape[0] != g.shape[1]:
        raise ValueError(f"weight must be [o, c, kh, kw] for grad_out {tuple(g.shape)} and x {tuple(x.shape)}")
    geo = _conv_bwd_geom(g, x, tuple(wt.shape[2:]), stride, padding, dilation)
    n, c, h, w = geo[:4]
    if out is None:
        out = torch.empty((n, c, h, w), dtype=torch.float32, device=g.device)
    else:
        _expect(out, "out", torch.float32, (n, c, h, w))
        _same_device("out", out, g)
    if grad_scale_a is None:
        grad_scale_a = torch.empty((), dtype=torch.float64, device=g.device)
    else:
        _expect(grad_scale_a, "grad_scale_a", torch.float64, ())
        _same_device("grad_scale_a", grad_scale_a, g)
    need = lib.bnn_conv2d_grad_input_workspace_bytes(*geo)
    if workspace is None:
        workspace = _workspace(need, g.device)
    else:
        _dev(workspace, "workspace")
        _same_device("workspace", workspace, g)
    _check(lib.bnn_conv2d_grad_input(g.data_ptr(), wt.data_ptr(), x.data_ptr(), dt, *geo,
                                     float(scale_a), float(scale_w), out.data_ptr(),
                                     grad_scale_a.data_ptr(), workspace.data_ptr(),
                                     _nbytes(workspace), _stream(g)), "bnn_conv2d_grad_input")
    return out, grad_scale_a


def conv2d_grad_weight(grad_out: torch.Tensor, x: torch.Tensor, kernel_size, scale_a: float,
                       stride=1, padding=0, dilation=1, codes: bool = False,
                       workspace: torch.Tensor | None = None):
    """Straight-through backward of the binarized conv, weight side: fp32 [o, c, kh, kw] =
    scale_a * conv2d_weight(sign(x), grad_out). With codes=True returns (grad_w, int8 codes,
    amax 0-dim float32): the int8 gradient the page keeps (amax = max|grad_w|)."""
    g, x = _dev(grad_out, "grad_out"), _dev(x, "x")
    dt = _half_pair(g, "grad_out")
    if x.dtype != g.dtype:
        raise TypeError("grad_out and x must share one dtype")
    _same_device("x", x, g)
    geo = _conv_bwd_geom(g, x, _pair(kernel_size, "kernel_size"), stride, padding, dilation)
    n, c, h, w, o, kh, kw = geo[:7]
    gw = torch.empty((o, c, kh, kw), dtype=torch.float32, device=g.device)
    q = torch.empty((o, c, kh, kw), dtype=torch.int8, device=g.device) if codes else None
    amax = torch.empty((), dtype=torch.float32, device=g.device) if codes else None
    need = lib.bnn_conv2d_grad_weight_workspace_bytes(*geo)
    if workspace is None:
        workspace = _workspace(need, g.device)
    else:
        _dev(workspace, "workspace")
        _same_device("workspace", workspace, g)
    _check(lib.bnn_conv2d_grad_weight(g.data_ptr(), x.data_ptr(), dt, *geo, float(scale_a),
                                      gw.data_ptr(), q.data_ptr() if codes else None,
                                      amax.data_ptr() if codes else None, workspace.data_ptr(),
                                      _nbytes(workspace), _stream(g)), "bnn_conv2d_grad_weight")
    return (gw, q, amax) if codes else gw
