"""The parity checker has teeth (CPU): outputs computed the way the kernels compute them pass it,
and a single flipped bit in an accumulator, a packed word or a scaled output beyond the stated
tolerance fails it."""
import numpy as np
import pytest
import torch

import synth
from parity_check import scaled_violations


def _flip(t: torch.Tensor, idx: int, bit: int) -> torch.Tensor:
    itype = {torch.float32: torch.int32, torch.int32: torch.int32, torch.float16: torch.int16,
             torch.bfloat16: torch.int16}[t.dtype]
    raw = t.clone().contiguous().view(itype).reshape(-1)
    raw[idx] ^= torch.tensor(1 << bit, dtype=torch.int64).to(itype) if bit < (8 * raw.element_size() - 1) \
        else torch.tensor(-(1 << bit), dtype=torch.int64).to(itype)
    return raw.view(t.dtype).reshape(t.shape)


@pytest.fixture(scope="module")
def case(oracle_lib):
    c = synth.random_linear_case(5, max_m=40, max_n=40, max_kw=8)
    acc = oracle_lib.linear_acc(c["x"], c["w"])
    y = oracle_lib.scale(acc, c["scale_a"], c["scale_w"])
    alpha = torch.tensor(c["scale_a"] * c["scale_w"], dtype=torch.float64).float()
    prod = acc.float() * alpha                                   # (float)acc * (float)alpha, RNE
    return acc, y, prod


def test_kernel_style_outputs_pass(case):
    acc, y, prod = case
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        assert not scaled_violations(prod.to(dt), acc, y).any(), dt


def test_flipped_accumulator_or_word_fails(case, oracle_lib):
    acc, _, _ = case
    for bit in (0, 5, 17, 31):
        assert not torch.equal(_flip(acc, 3, bit), acc)
    g = torch.Generator().manual_seed(3)
    words = oracle_lib.pack_rows(torch.randn((4, 96), generator=g))
    assert not torch.equal(_flip(words, 7, 0), words)


@pytest.mark.parametrize("dt,bits_caught,bits_allowed", [
    (torch.float32, [4, 10, 22, 23, 31], [0]),           # one f32 ulp (2^-23 relative) is inside 1e-6
    (torch.float16, [1, 5, 9, 10, 15], []),              # two f16 ulps and more
    (torch.bfloat16, [1, 4, 6, 7, 15], []),
])
def test_flipped_output_bit_fails(case, dt, bits_caught, bits_allowed):
    acc, y, prod = case
    out = prod.to(dt)
    flat_acc = acc.reshape(-1)
    idx = int(torch.nonzero(flat_acc.abs() > 2).reshape(-1)[0])   # a non-zero, non-tiny output
    for bit in bits_caught:
        assert scaled_violations(_flip(out, idx, bit), acc, y).reshape(-1)[idx], (dt, bit)
    for bit in bits_allowed:
        assert not scaled_violations(_flip(out, idx, bit), acc, y).any(), (dt, bit)


def test_negative_zero_for_zero_accumulator_fails():
    acc = torch.tensor([[0, 4], [-2, 0]], dtype=torch.int32)
    y = acc.double() * 0.25
    out = (acc.float() * 0.25)
    assert not scaled_violations(out, acc, y).any()
    out_neg = out.clone()
    out_neg[0, 0] = -0.0
    assert scaled_violations(out_neg, acc, y)[0, 0]
