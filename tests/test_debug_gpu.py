"""The debug build (libasf_debug.so: the host API compiled with ASF_DEBUG over
the same kernels) checks the caller's device content the release build takes
on trust: asf_create_layer refuses a neuron table that is not a permutation,
asf_sparse_ffn a list with an id out of range or listed twice, or a count
outside 0 .. d_ffn (ASF_ERR_ARG).  Valid calls give the release library's
results bit for bit."""
import ctypes
import os

import numpy as np
import pytest
import torch

import workload as wl
from gpu_util import asf, need_gpu, to_dev

pytestmark = pytest.mark.gpu


def _debug_lib(m):
    lib = ctypes.CDLL(os.path.join(os.path.dirname(m.LIB_PATH), "libasf_debug.so"))
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.asf_layer_storage_bytes.argtypes = [ctypes.POINTER(m.LayerDesc)]
    lib.asf_layer_storage_bytes.restype = ctypes.c_size_t
    lib.asf_create_layer.argtypes = [ctypes.POINTER(m.LayerDesc), ctypes.POINTER(m.LayerWeights),
                                     vp, vp, ctypes.c_size_t, vp, ctypes.POINTER(vp)]
    lib.asf_sparse_ffn.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp]
    lib.asf_destroy_layer.argtypes = [vp]
    lib.asf_version.restype = ctypes.c_char_p
    return lib


def test_debug_build_checks_caller_content():
    need_gpu()
    m = asf()
    lib = _debug_lib(m)
    assert b"debug" in lib.asf_version()
    L = wl.random_layer(256, 1000, 64, "f16", False, 31)
    dev = {k: to_dev(getattr(L, k)) for k in ("w_up", "w_down", "p1", "p2", "b1", "b2", "c1", "c2")}
    w = m.LayerWeights(dev["w_up"].data_ptr(), None, dev["b1"].data_ptr(), dev["w_down"].data_ptr(),
                       dev["b2"].data_ptr(), dev["p1"].data_ptr(), dev["c1"].data_ptr(),
                       dev["p2"].data_ptr(), dev["c2"].data_ptr())
    desc = m.make_desc(256, 1000, 64)
    nbytes = lib.asf_layer_storage_bytes(ctypes.byref(desc))
    storage = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    h = ctypes.c_void_p()

    def create(table):
        t = to_dev(table.astype(np.int32))
        rc = lib.asf_create_layer(ctypes.byref(desc), ctypes.byref(w), t.data_ptr(),
                                  storage.data_ptr(), nbytes, None, ctypes.byref(h))
        torch.cuda.synchronize()
        return rc
    bad = L.perm.copy()
    bad[5] = bad[6]
    assert create(bad) == 1 and h.value is None                  # a repeated entry
    bad = L.perm.copy()
    bad[9] = 1000
    assert create(bad) == 1                                       # an entry out of range
    assert create(L.perm) == 0 and h.value
    rel = m.layer_from_numpy(L)
    x = to_dev(np.random.default_rng(3).standard_normal((1, 256)).astype(np.float32))
    y = torch.empty((1, 256), device="cuda")

    def call(ids, n=None):
        a = to_dev(np.asarray(ids, np.int32))
        c = to_dev(np.array([len(ids) if n is None else n], np.int32))
        rc = lib.asf_sparse_ffn(h.value, x.data_ptr(), 1, a.data_ptr(), c.data_ptr(), None,
                                y.data_ptr(), None)
        torch.cuda.synchronize()
        return rc
    ids = np.random.default_rng(4).choice(1000, 120, replace=False)
    assert call(ids) == 0
    ref = rel.sparse_ffn(x, active=to_dev(ids.astype(np.int32)))
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    assert call(np.concatenate([ids, ids[:1]])) == 1             # an id listed twice
    assert call(np.concatenate([ids, [1000]])) == 1              # an id out of range
    assert call(np.concatenate([ids, [-1]])) == 1
    assert call(ids, n=1001) == 1                                 # a count above d_ffn
    assert call(ids, n=-1) == 1
    assert call(ids[:0]) == 0                                     # an empty list is valid
    lib.asf_destroy_layer(h.value)
