"""GPU parity of the exact-mask mode (asf_exact_ffn): no predictor, every
pre-activation computed, FC2 over the true set {z > 0}.

* Set: against the oracle's fp64 pre-activations (true_mask) with the margin
  rule (neurons with |z| <= 1e-3 may go either way), ascending slot order.
* Output: against the oracle's FFN over the GPU's own set and against the
  oracle's dense FFN (equal to the FFN over the true set), per-token relative
  L2 <= 1e-3 (fp32 weights) / 5e-3 (fp16); against this library's dense path
  up to fp32 reordering.
"""
import numpy as np
import pytest
import torch

import workload as wl
from gpu_util import TOL, asf, check_set, need_gpu, rel_l2, to_dev

pytestmark = pytest.mark.gpu

REORDER_TOL = 1e-5


def _exact_check(orc, L, x, lay, label):
    tol = TOL[L.shape.wdtype]
    f = L.shape.f
    pre, _ = orc.true_mask(L.w_up, x, b1=L.b1, W_gate=L.w_gate)
    dense = orc.dense_ffn(L.w_up, L.w_down, x, b1=L.b1, b2=L.b2, W_gate=L.w_gate)
    active = torch.zeros(f, dtype=torch.int32, device="cuda")
    n = torch.zeros(1, dtype=torch.int32, device="cuda")
    worst, amb = 0.0, 0
    for t in range(x.shape[0]):
        xt = to_dev(x[t:t + 1])
        y = lay.exact_ffn(xt, active=active, n_active=n)
        yd = lay.dense_ffn_ref(xt)
        torch.cuda.synchronize()
        k = int(n.item())
        ids = active[:k].cpu().numpy()
        amb += check_set(ids, pre[t], 0.0, L.perm, "%s token %d" % (label, t))
        yg = y.cpu().numpy()[0]
        y_own = orc.ffn(L.w_up, L.w_down, x[t], ids, b1=L.b1, b2=L.b2, W_gate=L.w_gate)[0]
        e = max(rel_l2(yg, y_own), rel_l2(yg, dense[t]))
        worst = max(worst, e)
        assert e <= tol, "%s token %d: rel-L2 %.3g" % (label, t, e)
        er = rel_l2(yg, yd.cpu().numpy()[0])
        assert er <= REORDER_TOL, "%s token %d: exact vs dense path %.3g" % (label, t, er)
    print("%s: %d tokens, worst rel-L2 %.3g, ambiguous %d" % (label, x.shape[0], worst, amb))


def test_exact_tiny_fp32(orc):
    need_gpu()
    L = wl.config_layer("tiny_f32")
    x = wl.config_tokens("tiny_f32", 16)
    _exact_check(orc, L, x, asf().layer_from_numpy(L), "exact tiny f32")


@pytest.mark.parametrize("d,f,H,gated", [(512, 2000, 128, False), (256, 40, 64, False),
                                         (2048, 3000, 256, False), (2048, 2500, 512, True),
                                         (5120, 4160, 1024, False), (7168, 2048, 2048, False),
                                         (1024, 4160, 256, True)])
def test_exact_scaled(orc, d, f, H, gated):
    """Tiling variants (d classes), ragged mask words, plain and gated."""
    need_gpu()
    _, sh = wl.CONFIGS["llama7b_gated_relu" if gated else "opt6.7b_ffn"]
    L = wl.make_layer(wl.scaled_shape(sh, d, f, H), 700 + d + f)
    x = wl.make_tokens(d, 4, 800 + f)
    _exact_check(orc, L, x, asf().layer_from_numpy(L),
                 "exact %dx%d%s" % (d, f, " gated" if gated else ""))


def test_exact_full_size(orc):
    """The headline shape, 4096x16384 fp16."""
    need_gpu()
    L = wl.config_layer("opt6.7b_ffn")
    x = wl.config_tokens("opt6.7b_ffn", 2)
    _exact_check(orc, L, x, asf().layer_from_numpy(L), "exact 4096x16384")


def test_exact_residual_repeat_and_batch_rejected():
    need_gpu()
    m = asf()
    L = wl.random_layer(512, 3000, 64, "f16", False, 21)
    lay = m.layer_from_numpy(L, max_batch=4)
    x = to_dev(np.random.default_rng(5).standard_normal((1, 512)).astype(np.float32))
    r = to_dev(np.random.default_rng(6).standard_normal((1, 512)).astype(np.float32))
    y0 = lay.exact_ffn(x).clone()
    y1 = lay.exact_ffn(x).clone()
    yr = lay.exact_ffn(x, residual=r).clone()
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert rel_l2(yr.cpu().numpy(), (y0 + r).cpu().numpy()) <= 1e-6
    # two tokens: refused by the binding, and by the C ABI itself
    x2 = torch.cat([x, x])
    with pytest.raises(ValueError):
        lay.exact_ffn(x2)
    y2 = torch.empty_like(x2)
    rc = m.library().asf_exact_ffn(lay.handle, x2.data_ptr(), 2, None, y2.data_ptr(), None,
                                   None, None)
    assert rc == 5   # ASF_ERR_UNSUPPORTED
