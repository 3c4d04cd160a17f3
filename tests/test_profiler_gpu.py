"""GPU parity of the activation profiler and the hot-first table builder.

* Counts: per original id, the number of calibration tokens whose true
  pre-activation is > 0, against the oracle's fp64 true mask: exact for every
  neuron none of whose tokens lies within the 1e-3 margin, otherwise off by
  at most its number of such tokens.
* Table: integer work, bit-exact against the oracle's hot_first_table.
* A layer created with the profiled table gives the same decode results as
  with the generator's table (the table only reorders storage).
"""
import dataclasses

import numpy as np
import pytest
import torch

import workload as wl
from gpu_util import MARGIN, TOL, asf, need_gpu, rel_l2, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,f,H,gated,use_table", [(1024, 4160, 256, False, False),
                                                   (512, 3000, 128, True, True),
                                                   (256, 40, 64, False, True)])
def test_profile_counts_match_oracle(orc, d, f, H, gated, use_table):
    need_gpu()
    _, sh = wl.CONFIGS["llama7b_gated_relu" if gated else "opt6.7b_ffn"]
    L = wl.make_layer(wl.scaled_shape(sh, d, f, H), 900 + d + f)
    x = wl.make_tokens(d, 48, 950 + f)
    lay = asf().layer_from_numpy(L, use_table=use_table)
    counts = lay.profile_activations(to_dev(x))
    torch.cuda.synchronize()
    got = counts.cpu().numpy().astype(np.int64)
    pre, act = orc.true_mask(L.w_up, x, b1=L.b1, W_gate=L.w_gate)
    want = orc.count_activations(act).astype(np.int64)
    amb = (np.abs(pre) <= MARGIN).sum(axis=0)
    diff = np.abs(got - want)
    assert np.all(diff <= amb), "counts differ beyond the ambiguous tokens: %s" % np.nonzero(diff > amb)[0][:5]
    assert np.array_equal(got[amb == 0], want[amb == 0])
    # accumulation: a second pass over the same tokens doubles the counts
    lay.profile_activations(to_dev(x), counts=counts)
    assert np.array_equal(counts.cpu().numpy().astype(np.int64), 2 * got)


@pytest.mark.parametrize("f,seed", [(40, 1), (3000, 2), (16384, 3), (65536, 4)])
def test_hot_first_table_matches_oracle(orc, f, seed):
    need_gpu()
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, 50, size=f).astype(np.int32)     # many ties
    counts[: min(f, 7)] = 49
    table = asf().hot_first_table(to_dev(counts))
    torch.cuda.synchronize()
    want = orc.hot_first_table(counts.astype(np.int64))
    assert np.array_equal(table.cpu().numpy(), np.asarray(want, np.int64))


def test_profiled_table_roundtrip(orc):
    """Profile on an identity-table layer, build the table on the device,
    create the layer with it: the decode step keeps its sets and outputs."""
    need_gpu()
    m = asf()
    _, sh = wl.CONFIGS["opt6.7b_ffn"]
    L = wl.make_layer(wl.scaled_shape(sh, 1024, 4160, 256), 1234)
    calib = wl.make_tokens(1024, 256, 4321)
    ident = m.layer_from_numpy(L, use_table=False)
    counts = ident.profile_activations(to_dev(calib))
    table = m.hot_first_table(counts)
    torch.cuda.synchronize()
    tab = table.cpu().numpy()
    assert np.array_equal(np.sort(tab), np.arange(L.shape.f))
    # the profiled order follows the firing law: the generator's 100 hottest
    # neurons are almost all among the profiled 200 hottest
    top_law = set(L.perm[:100].tolist())
    assert len(top_law & set(tab[:200].tolist())) >= 90

    prof = m.layer_from_numpy(dataclasses.replace(L, perm=tab.astype(L.perm.dtype)))
    law = m.layer_from_numpy(L)
    x = wl.make_tokens(1024, 4, 99)
    for t in range(4):
        xt = to_dev(x[t:t + 1])
        a1 = torch.empty(L.shape.f, dtype=torch.int32, device="cuda")
        n1 = torch.empty(1, dtype=torch.int32, device="cuda")
        a2 = torch.empty_like(a1)
        n2 = torch.empty_like(n1)
        y1 = law.decode_step(xt, active=a1, n_active=n1)
        y2 = prof.decode_step(xt, active=a2, n_active=n2)
        torch.cuda.synchronize()
        k = int(n1.item())
        assert int(n2.item()) == k
        assert np.array_equal(np.sort(a1[:k].cpu().numpy()), np.sort(a2[:k].cpu().numpy()))
        assert rel_l2(y2.cpu().numpy(), y1.cpu().numpy()) <= 1e-5
        y_orc = orc.ffn(L.w_up, L.w_down, x[t], a2[:k].cpu().numpy(), b1=L.b1, b2=L.b2)
        assert rel_l2(y2.cpu().numpy()[0], y_orc[0]) <= TOL["f16"]
