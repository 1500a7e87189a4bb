"""The Python binding rejects wrongly sized or typed tensors before any library call (CPU only).

The C ABI takes raw device pointers, so a too-short weight or a too-small output would be read
or written out of bounds on the device. Here the binding's device check is widened to CPU
tensors and its library handle is replaced by a stand-in whose compute entry points fail the
test if reached (the host-only size queries still go to the real library): every mismatched
call must raise ValueError / TypeError / AssertionError first, and a well-formed call must get
as far as the entry point.
"""
import pytest
import torch


class _Launched(Exception):
    pass


class _Guard:
    """Forwards the host-only queries to the real library; any other entry point raises."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name.endswith("_workspace_bytes") or name.endswith("_auto_path") or name in (
                "bnn_status_string", "bnn_last_path"):
            return getattr(self._real, name)

        def launched(*args):
            raise _Launched(name)
        return launched


@pytest.fixture
def bnn(monkeypatch):
    import convolution_bnn_pack_amd as m
    monkeypatch.setattr(m, "_DEVICE_TYPES", ("cuda", "cpu"))
    monkeypatch.setattr(m, "lib", _Guard(m.lib))
    monkeypatch.setattr(m, "_stream", lambda t: 0)
    return m


I32 = torch.int32


def _z(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def test_gemm_rejects_mismatched_tensors(bnn):
    m, n, k = 8, 5, 70                      # 3 words per row, the last one partial
    x, wp = _z(m, k), _z(n, 3, dtype=I32)
    with pytest.raises(_Launched):          # well-formed: reaches the entry point
        bnn.gemm(x, wp, 1.0, 1.0)
    with pytest.raises(_Launched):
        bnn.gemm(_z(m, 3, dtype=I32), wp, 1.0, 1.0, k=k)
    with pytest.raises(_Launched):
        bnn.gemm(x, wp, 1.0, 1.0, out=_z(m, n, dtype=torch.float16))
    with pytest.raises(_Launched):
        bnn.gemm(_z(m, 9, dtype=torch.uint8), wp, 1.0, 1.0, k=k)
    bad = [
        dict(w_packed=_z(n, 2, dtype=I32)),                 # too few words for k
        dict(w_packed=_z(n, 4, dtype=I32)),                 # too many
        dict(w_packed=_z(n, 3)),                            # float weight
        dict(w_packed=_z(n, 3, 1, dtype=I32)),              # wrong rank
        dict(out=_z(m, n + 1)),                             # output too wide
        dict(out=_z(m - 1, n)),                             # too few rows
        dict(out=_z(m, n, dtype=torch.float64)),            # unsupported dtype
        dict(out=_z(m * n)),                                # flat
        dict(x=_z(m, 2, dtype=I32), k=k),                   # packed x too short for k
        dict(x=_z(m, 3, dtype=I32), k=100),                 # k needs 4 words
        dict(x=_z(m, 3, dtype=I32), k=0),
        dict(x=_z(2, m, k)),                                # 3-D activations
        dict(x=_z(m, 8, dtype=torch.uint8), k=k),           # 8-bit containers: 9 bytes needed
        dict(x=_z(m, 9, dtype=torch.uint8), k=64),
        dict(out_dtype=torch.float64),
    ]
    for case in bad:
        args = dict(x=x, w_packed=wp, scale_a=1.0, scale_w=1.0)
        args.update(case)
        with pytest.raises((ValueError, TypeError, AssertionError)):
            bnn.gemm(**args)


def test_conv2d_rejects_mismatched_tensors(bnn):
    n, c, h, w, o = 2, 40, 6, 5, 7          # 2 words per pixel
    x, wp = _z(n, c, h, w), _z(o, 3, 3, 2, dtype=I32)
    with pytest.raises(_Launched):
        bnn.conv2d(x, wp, 1.0, 1.0, 3, 1, 1, 1)
    with pytest.raises(_Launched):
        bnn.conv2d(_z(n, h, w, 2, dtype=I32), wp, 1.0, 1.0, 3, 1, 1, 1, channels=c)
    with pytest.raises(_Launched):
        bnn.conv2d(_z(n, h, w, 5, dtype=torch.uint8), wp, 1.0, 1.0, 3, 1, 1, 1, channels=c)
    with pytest.raises(_Launched):       # rectangular kernel through the general entry point
        bnn.conv2d(x, _z(o, 1, 3, 2, dtype=I32), 1.0, 1.0, (1, 3), 1, (0, 1), 1)
    bad = [
        dict(w_packed=_z(o, 3, 3, 1, dtype=I32)),           # too few channel words
        dict(w_packed=_z(o, 3, 3, 3, dtype=I32)),
        dict(w_packed=_z(o, 5, 5, 2, dtype=I32)),           # kernel size disagrees
        dict(w_packed=_z(o, 9, 2, dtype=I32)),              # rank
        dict(w_packed=_z(o, 3, 3, 2)),                      # float
        dict(out=_z(n, o, h, w + 1)),                       # wrong output size
        dict(out=_z(n, o + 1, h, w)),
        dict(out=_z(n, o, h, w, dtype=torch.int64)),
        dict(x=_z(n, h, w, 1, dtype=I32), channels=c),      # packed x too short
        dict(x=_z(n, h, w, 2, dtype=I32), channels=65),     # needs 3 words
        dict(x=_z(n, c, h)),                                # 3-D
        dict(x=_z(n, h, w, 4, dtype=torch.uint8), channels=c),   # 5 bytes per pixel needed
        dict(out_dtype=torch.uint8),
    ]
    for case in bad:
        args = dict(x=x, w_packed=wp, scale_a=1.0, scale_w=1.0, kernel_size=3, stride=1,
                    padding=1, dilation=1)
        args.update(case)
        with pytest.raises((ValueError, TypeError, AssertionError)):
            bnn.conv2d(**args)


def test_pack_outputs_checked(bnn):
    with pytest.raises(_Launched):
        bnn.pack_sign(_z(4, 40), out=_z(4, 2, dtype=I32))
    for out in (_z(4, 1, dtype=I32), _z(4, 2), _z(5, 2, dtype=I32)):
        with pytest.raises((ValueError, TypeError)):
            bnn.pack_sign(_z(4, 40), out=out)
    with pytest.raises(_Launched):
        bnn.pack_sign_nchw(_z(2, 40, 3, 3), out=_z(2, 3, 3, 2, dtype=I32))
    for out in (_z(2, 3, 3, 1, dtype=I32), _z(2, 2, 3, 3, dtype=I32)):
        with pytest.raises((ValueError, TypeError)):
            bnn.pack_sign_nchw(_z(2, 40, 3, 3), out=out)
    with pytest.raises((ValueError, TypeError)):
        bnn.pack_sign_shift(_z(4, 40), _z(3), out=_z(4, 2, dtype=I32))   # bias length
    with pytest.raises((ValueError, TypeError)):
        bnn.pack_sign_nchw_shift(_z(2, 40, 3, 3), _z(40), out=_z(2, 3, 3, 1, dtype=I32))
    with pytest.raises((ValueError, TypeError)):
        bnn.abs_mean_scale(_z(64), 2.0, out=_z(1))


def test_backward_outputs_checked(bnn):
    m, n, k = 16, 8, 24
    g, w, x = _z(m, n, dtype=torch.bfloat16), _z(n, k, dtype=torch.bfloat16), _z(m, k, dtype=torch.bfloat16)
    with pytest.raises(_Launched):
        bnn.linear_grad_input(g, w, x, 1.0, 1.0)
    for kw in (dict(out=_z(m, k + 1)), dict(out=_z(m, k, dtype=torch.float16)),
               dict(grad_scale_a=_z(1, dtype=torch.float64)), dict(grad_scale_a=_z())):
        with pytest.raises((ValueError, TypeError)):
            bnn.linear_grad_input(g, w, x, 1.0, 1.0, **kw)
    with pytest.raises((ValueError, TypeError)):
        bnn.linear_grad_input(g, w[:, :16].contiguous(), x, 1.0, 1.0)
    with pytest.raises(_Launched):
        bnn.linear_grad_weight(g, x, 1.0)
    for out in (_z(n, k - 8), _z(k, n), _z(n, k, dtype=torch.float64)):
        with pytest.raises((ValueError, TypeError)):
            bnn.linear_grad_weight(g, x, 1.0, out=out)


def test_w8a8_outputs_checked(bnn):
    xq, wq = _z(2, 6, 6, 16, dtype=torch.int8), _z(4, 3, 3, 16, dtype=torch.int8)
    with pytest.raises(_Launched):
        bnn.w8a8_conv2d(xq, wq, 1.0, 1.0, 3, 1, 1, 1)
    for kw in (dict(out=_z(2, 4, 6, 5)), dict(out=_z(2, 4, 6, 6, dtype=torch.float64))):
        with pytest.raises((ValueError, TypeError)):
            bnn.w8a8_conv2d(xq, wq, 1.0, 1.0, 3, 1, 1, 1, **kw)
    with pytest.raises((ValueError, TypeError)):
        bnn.w8a8_conv2d(xq.float(), wq, 1.0, 1.0, 3, 1, 1, 1)
