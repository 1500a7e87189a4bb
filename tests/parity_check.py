"""The parity bar for scaled outputs, shared by the GPU parity tests and the CPU test that
shows it has teeth (a planted one-bit error must fail it).

Integer results (packed words, int32 accumulators) are compared with torch.equal. Scaled
outputs: float32 within 1e-6 relative of y = acc * (scale_a * scale_w) computed in double by
the oracle; float16 and bfloat16 within one unit in the last place of the output type at y;
a zero accumulator must give exactly +0 (positive scales). The kernel's own error is float32
rounding of acc * alpha (<= 2^-23 relative) followed by one round-to-nearest-even to the output
type.
"""
import numpy as np
import torch


def ulp_at(y: np.ndarray, frac_bits: int, min_spacing: float) -> np.ndarray:
    """Spacing of the output type's grid at |y| (frac_bits fraction bits, subnormal spacing
    min_spacing)."""
    mant, exp = np.frexp(np.abs(y))                      # |y| = mant * 2^exp, mant in [0.5, 1)
    return np.maximum(np.ldexp(1.0, exp - 1 - frac_bits), min_spacing)


def scaled_violations(out: torch.Tensor, acc: torch.Tensor, y: torch.Tensor) -> np.ndarray:
    """Boolean mask of the outputs outside the parity bar."""
    o = out.detach().cpu().double().numpy()
    yy = y.numpy()
    a = acc.numpy()
    assert o.shape == yy.shape
    if out.dtype == torch.float32:
        bad = np.abs(o - yy) > 1e-6 * np.abs(yy)
    elif out.dtype == torch.float16:
        bad = np.abs(o - yy) > ulp_at(yy, 10, 2.0 ** -24)
    else:
        bad = np.abs(o - yy) > ulp_at(yy, 7, 2.0 ** -133)
    zero = a == 0
    bad |= zero & ((o != 0.0) | np.signbit(o))
    return bad


def check_scaled(out: torch.Tensor, acc: torch.Tensor, y: torch.Tensor, what: str):
    bad = scaled_violations(out, acc, y)
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs outside tolerance, first at {np.argwhere(bad)[0]}"
