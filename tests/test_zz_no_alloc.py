"""asf_stack_decode_static, the stack call that allocates nothing (its buffer
between layers is the library's static device array), called through the C
ABI and compared with asf_stack_decode over a caller work buffer: the same
kernels on the same inputs, so the outputs must agree bit for bit.  Two
calls in a row on the same GPU, the second with a smaller input (fewer
tokens, residual on), since every call shares the array and finds the
previous call's contents in it."""
import ctypes

import numpy as np
import pytest
import torch

import workload as wl
from gpu_util import asf, need_gpu

pytestmark = pytest.mark.gpu


def _layers(d, f, shapes_h, max_batch, seed):
    from workload.gpu import make_layer_device
    m = asf()
    out = []
    for l, (H, rho) in enumerate(shapes_h):
        DL = make_layer_device(wl.LayerShape(d, f, H, rho, "f16"), seed + l, torch.device("cuda"))
        out.append(m.Layer(DL.w_up, DL.w_down, DL.p1, DL.p2, b1=DL.b1, b2=DL.b2, c1=DL.c1,
                           c2=DL.c2, neuron_table=DL.perm, max_batch=max_batch))
        del DL
    torch.cuda.synchronize()
    return out


def _pair(lib, arr, n, x, B, residual):
    """(static call's y, work-buffer call's y) through the C ABI."""
    d = x.shape[1]
    y_s = torch.full((B, d), float("nan"), device="cuda")
    y_w = torch.full((B, d), float("nan"), device="cuda")
    work = torch.empty((B, d), device="cuda")
    assert lib.asf_stack_decode_static(arr, n, x.data_ptr(), B, residual, y_s.data_ptr(),
                                       None) == 0
    assert lib.asf_stack_decode(arr, n, x.data_ptr(), B, residual, y_w.data_ptr(),
                                work.data_ptr(), None) == 0
    torch.cuda.synchronize()
    return y_s, y_w


def test_static_stack_matches_work_buffer_call():
    need_gpu()
    m = asf()
    lib = m.library()
    d, f = 1024, 4096
    layers = _layers(d, f, ((128, 0.05), (256, 0.10), (128, 0.08), (64, 0.12)), 8, 880)
    arr = (ctypes.c_void_p * len(layers))(*[l.handle for l in layers])
    rng = np.random.default_rng(881)
    # first call: 8 tokens, plain chain
    x8 = torch.from_numpy(rng.standard_normal((8, d)).astype(np.float32)).cuda()
    y_s, y_w = _pair(lib, arr, len(layers), x8, 8, 0)
    assert torch.isfinite(y_s).all() and torch.equal(y_s, y_w)
    # second call, smaller: 2 tokens with the residual (the array still holds
    # the first call's 8-token intermediates)
    x2 = torch.from_numpy(rng.standard_normal((2, d)).astype(np.float32)).cuda()
    y_s, y_w = _pair(lib, arr, len(layers), x2, 2, 1)
    assert torch.isfinite(y_s).all() and torch.equal(y_s, y_w)
    # an odd layer count puts the first layer's output in the static array
    y_s, y_w = _pair(lib, arr, 3, x2[:1], 1, 0)
    assert torch.equal(y_s, y_w)
    # one layer needs no buffer; y == x in place
    y_s, y_w = _pair(lib, arr, 1, x2, 2, 0)
    assert torch.equal(y_s, y_w)
    xin = x2.clone()
    assert lib.asf_stack_decode_static(arr, len(layers), xin.data_ptr(), 2, 1, xin.data_ptr(),
                                       None) == 0
    ref = m.Stack(layers, residual=True).decode(x2)
    torch.cuda.synchronize()
    assert torch.equal(xin, ref)
    # the binding's form, and the host-side refusals
    out = torch.empty((2, d), device="cuda")
    m.Stack(layers).decode_static(x2, out)
    torch.cuda.synchronize()
    assert torch.equal(out, m.Stack(layers).decode(x2))
    assert lib.asf_stack_decode_static(arr, len(layers), x2.data_ptr(), 0, 0, out.data_ptr(),
                                       None) == 2          # B = 0: ASF_ERR_SHAPE
    assert lib.asf_stack_decode_static(arr, len(layers), x8.data_ptr(), 9, 0, out.data_ptr(),
                                       None) == 2          # B above max_batch
    assert lib.asf_stack_decode_static(None, 1, x2.data_ptr(), 1, 0, out.data_ptr(),
                                       None) == 1          # ASF_ERR_ARG
