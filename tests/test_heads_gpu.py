"""GPU parity of the attention-head predictor (asf_predict_heads) against the
oracle's predict_heads on the same seeded inputs: every head whose logit is
more than 1e-3 from the threshold is decided the same way (heads inside the
margin may go either way); the per-token lists are ascending, agree with the
mask words and the counts; each token keeps its own set."""
import numpy as np
import pytest
import torch

import workload as wl
from gpu_util import asf, check_set, need_gpu, to_dev

pytestmark = pytest.mark.gpu


def _check(orc, P, x, hp, label, theta=0.0):
    B, nh = x.shape[0], P.q2.shape[0]
    words = (nh + 63) // 64
    masks, heads, counts = hp.predict(to_dev(x))
    torch.cuda.synchronize()
    s, _, _ = orc.predict_heads(P.q1, P.c1, P.q2, P.c2, x, theta=theta)
    mw = masks.cpu().numpy().view(np.uint64)
    bits = ((mw[:, :, None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)).reshape(B, -1)
    hl, cn = heads.cpu().numpy(), counts.cpu().numpy()
    amb = 0
    for b in range(B):
        lst = hl[b, :cn[b]]
        assert np.array_equal(lst, np.flatnonzero(bits[b, :nh])), "%s tok %d" % (label, b)
        assert not bits[b, nh:].any() and np.all(hl[b, cn[b]:] == -1)
        amb += check_set(lst, s[b], theta, np.arange(nh), "%s tok %d" % (label, b))
    print("%s: B=%d heads %d, selected %.3f, ambiguous flips %d"
          % (label, B, nh, cn.mean() / nh, amb))
    return masks, heads, counts


@pytest.mark.parametrize("name", ["opt30b_heads", "heads256"])
def test_head_predictor_configs(orc, name):
    """OPT-30B-shaped attention (7168 wide, 56 heads) and the pages' 256-head
    example, fp16, one token at a time and in batches of 4 and 32."""
    need_gpu()
    P = wl.head_config(name)
    hp = asf().head_predictor_from_numpy(P, max_batch=32)
    x = wl.head_config_tokens(name, 48)
    for t in range(8):
        _check(orc, P, x[t:t + 1], hp, "%s B1" % name)
    _check(orc, P, x[8:12], hp, "%s B4" % name)
    _check(orc, P, x[12:44], hp, "%s B32" % name)
    # a batch gives each token the set it gets alone, bit for bit
    m1 = torch.stack([hp.predict(to_dev(x[t:t + 1]))[0][0] for t in range(12, 16)])
    m4 = hp.predict(to_dev(x[12:16]))[0]
    assert torch.equal(m1, m4)


@pytest.mark.parametrize("d,nh,H,wd", [(256, 40, 64, "f32"), (512, 1, 32, "f16"),
                                       (512, 64, 128, "f16"), (640, 65, 96, "f32"),
                                       (1024, 1000, 256, "f16"), (2048, 4096, 64, "f16")])
def test_head_predictor_shapes(orc, d, nh, H, wd):
    """Ragged head counts (one word, a word and one head, many words up to
    the 4096-head maximum), fp32 and fp16, batches of 1 and 5."""
    need_gpu()
    P = wl.make_head_predictor(wl.HeadShape(d, nh, H, 0.2, wd), 40 + nh)
    rng = np.random.default_rng(nh)
    P.c1 = (rng.standard_normal(H) * 0.1).astype(np.float32)
    hp = asf().head_predictor_from_numpy(P, max_batch=8)
    x = wl.make_tokens(d, 6, 50 + nh)
    _check(orc, P, x[:1], hp, "%dx%d H%d %s" % (d, nh, H, wd))
    _check(orc, P, x[1:6], hp, "%dx%d H%d %s B5" % (d, nh, H, wd))


def test_head_predictor_thresholds_and_errors(orc):
    need_gpu()
    m = asf()
    P = wl.make_head_predictor(wl.HeadShape(512, 100, 64, 0.2, "f16"), 77)
    x = wl.make_tokens(512, 2, 78)
    for theta in (0.4, -1e30, 1e30):
        hp = m.head_predictor_from_numpy(P, max_batch=2, threshold=theta)
        _, _, counts = _check(orc, P, x, hp, "theta %g" % theta, theta=theta)
        if theta == -1e30:
            assert counts.cpu().tolist() == [100, 100]
        if theta == 1e30:
            assert counts.cpu().tolist() == [0, 0]
    lib = m.library()
    xd = to_dev(x)
    c = torch.zeros(2, dtype=torch.int32, device="cuda")
    assert lib.asf_predict_heads(hp.handle, xd.data_ptr(), 2, None, None, None, None) == 1
    assert lib.asf_predict_heads(hp.handle, xd.data_ptr(), 3, None, None, c.data_ptr(),
                                 None) == 2
    # counts only (no list, no masks) through the multi-word path
    assert lib.asf_predict_heads(hp.handle, xd.data_ptr(), 2, None, None, c.data_ptr(),
                                 None) == 0
    torch.cuda.synchronize()
    assert c.cpu().tolist() == [0, 0]
