"""Shared helpers of the GPU parity tests (not collected as tests)."""
import numpy as np
import pytest
import torch

MARGIN = 1e-3          # set parity: neurons whose score is within this of theta may go either way
TOL = {"f32": 1e-3, "f16": 5e-3}   # per-token relative L2 of y


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def asf():
    import activation_sparse_ffn_02_amd as m
    return m


def rel_l2(y_gpu, y_ref):
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    nr = np.linalg.norm(y_ref)
    if nr == 0.0:
        return float(np.abs(y_gpu).max())
    return float(np.linalg.norm(y_gpu - y_ref) / nr)


def check_set(gpu_ids, s_orc, theta, perm, who=""):
    """GPU set vs the oracle's scores: every neuron whose margin |s - theta|
    exceeds MARGIN must be decided the same way; the list must hold distinct
    ids in ascending stored-slot order.  Returns the number of ambiguous
    neurons that differ."""
    f = s_orc.shape[0]
    ids = np.asarray(gpu_ids, np.int64)
    assert ids.size == 0 or (ids.min() >= 0 and ids.max() < f), who
    assert np.unique(ids).size == ids.size, who + ": duplicate ids"
    inv = np.empty(f, np.int64)
    inv[np.asarray(perm, np.int64)] = np.arange(f)
    slots = inv[ids]
    assert np.all(np.diff(slots) > 0), who + ": not in ascending slot order"
    g = np.zeros(f, bool)
    g[ids] = True
    o = s_orc > theta
    diff = g != o
    sure = np.abs(s_orc - theta) > MARGIN
    bad = np.nonzero(diff & sure)[0]
    assert bad.size == 0, "%s: %d neurons disagree beyond the margin, e.g. %s (s=%s)" % (
        who, bad.size, bad[:5], s_orc[bad[:5]])
    return int(diff.sum())


def to_dev(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)
