"""GPU parity of the layer stack (asf_stack_decode).

* The stack call equals the same layers' decode steps chained by hand, bit
  for bit (same kernels, same inputs), with and without the residual.
* Each layer's set and output agree with the oracle on that layer's actual
  input (the previous layer's GPU output): sets bit-exact beyond the 1e-3
  margin, per-token relative L2 <= 5e-3 (fp16 weights).
* The look-ahead form (layer l's set predicted from layer l-1's input, in
  the same launches as layer l-1's FFN) equals asf_predict + asf_sparse_ffn
  chained by hand on those inputs, bit for bit, with oracle parity per layer,
  also over layers of mixed kind (gated / plain, fp16 / fp32).
* The full 48-layer OPT-30B-shaped stack (7168x28672 fp16, predictors of
  512/1024/2048 hidden, ~40 GB resident) runs end to end; the oracle checks
  layers 0, 23 and 47 (their weights are read back from the device).
"""
import numpy as np
import pytest
import torch

import workload as wl
from gpu_util import TOL, asf, check_set, need_gpu, rel_l2, to_dev

pytestmark = pytest.mark.gpu


def _device_layers(shapes, seed0, keep=(), max_batch=1):
    """Create library layers from device-generated weights; keep host copies
    of the layers whose index is in `keep` (for the oracle)."""
    from workload.gpu import make_layer_device
    m = asf()
    layers, host = [], {}
    for l, sh in enumerate(shapes):
        DL = make_layer_device(sh, seed0 + l, torch.device("cuda"))
        layers.append(m.Layer(DL.w_up, DL.w_down, DL.p1, DL.p2, w_gate=DL.w_gate, b1=DL.b1,
                              b2=DL.b2, c1=DL.c1, c2=DL.c2, neuron_table=DL.perm,
                              max_batch=max_batch))
        if l in keep:
            host[l] = DL.to_numpy()
        del DL
    torch.cuda.synchronize()
    return layers, host


def _check_layer(orc, L, xin, y_gpu, ids_gpu, label):
    _, s_orc, _ = orc.predict(L.p1, L.c1, L.p2, L.c2, xin[None, :])
    check_set(ids_gpu, s_orc[0], 0.0, L.perm, label)
    y_orc = orc.ffn(L.w_up, L.w_down, xin, ids_gpu, b1=L.b1, b2=L.b2, W_gate=L.w_gate)
    e = rel_l2(y_gpu, y_orc[0])
    assert e <= TOL["f16"], "%s: rel-L2 %.3g" % (label, e)
    return e


@pytest.mark.parametrize("residual", [False, True])
def test_small_stack_equals_chained_steps(orc, residual):
    need_gpu()
    d, f = 512, 2048
    shapes = [wl.LayerShape(d, f, H, rho, "f16")
              for H, rho in ((64, 0.03), (128, 0.08), (256, 0.15), (128, 0.10), (64, 0.05))]
    layers, host = _device_layers(shapes, 700, keep=range(len(shapes)))
    st = asf().Stack(layers, residual=residual)
    x = wl.make_tokens(d, 3, 701)
    for t in range(x.shape[0]):
        xt = to_dev(x[t:t + 1])
        y = st.decode(xt)
        cur = xt
        for l, lay in enumerate(layers):
            act = torch.empty(f, dtype=torch.int32, device="cuda")
            n = torch.empty(1, dtype=torch.int32, device="cuda")
            nxt = lay.decode_step(cur, residual=cur if residual else None, active=act,
                                  n_active=n)
            torch.cuda.synchronize()
            ids = act[:int(n.item())].cpu().numpy()
            xin = cur.cpu().numpy()[0]
            yl = nxt.cpu().numpy()[0] - (xin if residual else 0.0)
            L = host[l]
            _, s_orc, _ = orc.predict(L.p1, L.c1, L.p2, L.c2, xin[None, :])
            check_set(ids, s_orc[0], 0.0, L.perm, "layer %d token %d" % (l, t))
            y_orc = orc.ffn(L.w_up, L.w_down, xin, ids, b1=L.b1, b2=L.b2)
            assert rel_l2(yl, y_orc[0]) <= TOL["f16"], (l, t)
            cur = nxt
        assert torch.equal(y, cur), "stack output differs from the chained steps"
    # y may equal x (in place)
    xt = to_dev(x[:1])
    ref = st.decode(xt)
    inplace = xt.clone()
    st.decode(inplace, out=inplace)
    assert torch.equal(inplace, ref)


def test_small_stack_batched(orc):
    """B = 4 tokens through the stack: the batched decode step per layer
    (union of the tokens' sets), equal bit for bit to the chained batched
    steps; per layer, the union against the oracle's scores on the layer's
    actual input (a neuron surely in or out of every token's set is decided
    the same way) and every token's output over the GPU's union."""
    need_gpu()
    d, f, B = 512, 2048, 4
    shapes = [wl.LayerShape(d, f, H, rho, "f16")
              for H, rho in ((64, 0.03), (128, 0.08), (256, 0.15), (128, 0.10))]
    layers, host = _device_layers(shapes, 740, keep=range(len(shapes)), max_batch=B)
    for residual in (False, True):
        st = asf().Stack(layers, residual=residual)
        xt = to_dev(wl.make_tokens(d, B, 741 + residual))
        y = st.decode(xt)
        cur = xt
        for l, lay in enumerate(layers):
            act = torch.empty(f, dtype=torch.int32, device="cuda")
            n = torch.empty(1, dtype=torch.int32, device="cuda")
            nxt = lay.decode_step(cur, residual=cur if residual else None, active=act,
                                  n_active=n)
            torch.cuda.synchronize()
            ids = act[:int(n.item())].cpu().numpy()
            xin = cur.cpu().numpy()
            L = host[l]
            _, s_orc, _ = orc.predict(L.p1, L.c1, L.p2, L.c2, xin)
            check_set(ids, s_orc.max(axis=0), 0.0, L.perm, "B%d layer %d union" % (B, l))
            y_orc = orc.ffn(L.w_up, L.w_down, xin, ids, b1=L.b1, b2=L.b2)
            yl = nxt.cpu().numpy() - (xin if residual else 0.0)
            for t in range(B):
                assert rel_l2(yl[t], y_orc[t]) <= TOL["f16"], (residual, l, t)
            cur = nxt
        assert torch.equal(y, cur), "batched stack differs from the chained steps"


def _lookahead_check(orc, shapes, seed, residual):
    """The look-ahead call equals asf_predict on x_{l-1} then asf_sparse_ffn
    on x_l, chained by hand, bit for bit; each layer's set and output agree
    with the oracle on those inputs; in place and repeated calls agree."""
    d, f = shapes[0].d, shapes[0].f
    layers, host = _device_layers(shapes, seed, keep=range(len(shapes)))
    st = asf().Stack(layers, residual=residual)
    x = wl.make_tokens(d, 3, seed + 1)
    for t in range(x.shape[0]):
        xt = to_dev(x[t:t + 1])
        y = st.decode_lookahead(xt)
        prev, cur = xt, xt
        for l, lay in enumerate(layers):
            act = torch.empty(f, dtype=torch.int32, device="cuda")
            n = torch.empty(1, dtype=torch.int32, device="cuda")
            lay.predict(prev, active=act, n_active=n)
            nxt = lay.sparse_ffn(cur, residual=cur if residual else None)
            torch.cuda.synchronize()
            ids = act[:int(n.item())].cpu().numpy()
            xin, xpred = cur.cpu().numpy()[0], prev.cpu().numpy()[0]
            L = host[l]
            _, s_orc, _ = orc.predict(L.p1, L.c1, L.p2, L.c2, xpred[None, :])
            check_set(ids, s_orc[0], 0.0, L.perm, "look-ahead layer %d token %d" % (l, t))
            yl = nxt.cpu().numpy()[0] - (xin if residual else 0.0)
            y_orc = orc.ffn(L.w_up, L.w_down, xin, ids, b1=L.b1, b2=L.b2, W_gate=L.w_gate)
            assert rel_l2(yl, y_orc[0]) <= TOL[shapes[l].wdtype], (l, t)
            prev, cur = cur, nxt
        assert torch.equal(y, cur), "look-ahead stack differs from the chained calls"
    xt = to_dev(x[:1])
    ref = st.decode_lookahead(xt)
    again = st.decode_lookahead(xt)
    inplace = xt.clone()
    st.decode_lookahead(inplace, out=inplace)
    torch.cuda.synchronize()
    assert torch.equal(again, ref) and torch.equal(inplace, ref)


@pytest.mark.parametrize("residual", [False, True])
def test_lookahead_stack_equals_chained_calls(orc, residual):
    """Look-ahead reading: layer l's set is predicted from layer l-1's input
    (layer 0's from its own)."""
    need_gpu()
    d, f = 512, 2048
    shapes = [wl.LayerShape(d, f, H, rho, "f16")
              for H, rho in ((64, 0.03), (128, 0.08), (256, 0.15), (128, 0.10), (64, 0.05))]
    _lookahead_check(orc, shapes, 760, residual)


@pytest.mark.parametrize("residual", [False, True])
def test_lookahead_mixed_stack(orc, residual):
    """Layers of different kinds in one look-ahead stack: gated and plain,
    fp16 and fp32 (a layer whose weight type differs from its predecessor's
    gets its predictor layer 1 as a launch of its own), predictor rows of 1,
    2 and 4 chunks per lane, a d_ffn that is not a multiple of 64."""
    need_gpu()
    d, f = 1024, 1500
    shapes = [wl.LayerShape(d, f, 1024, 0.08, "f16", gated=True),
              wl.LayerShape(d, f, 2048, 0.10, "f16"),
              wl.LayerShape(d, f, 256, 0.06, "f32"),
              wl.LayerShape(d, f, 512, 0.12, "f32", gated=True),
              wl.LayerShape(d, f, 128, 0.05, "f16")]
    _lookahead_check(orc, shapes, 790, residual)


def test_stack_argument_errors():
    """The C ABI refuses a layer listed twice, a d_model mismatch, B above a
    layer's max_batch and a work buffer overlapping x or y (the binding
    refuses the shape errors before the call)."""
    need_gpu()
    m = asf()
    lib = m.library()
    d, f = 256, 512
    layers, _ = _device_layers([wl.LayerShape(d, f, 64, 0.1, "f16")] * 2, 720)
    other, _ = _device_layers([wl.LayerShape(384, f, 64, 0.1, "f16")], 730)
    x = torch.zeros((1, d), device="cuda")
    y = torch.zeros((2, 384), device="cuda")
    w = torch.zeros((2, 384), device="cuda")

    def arr(ls):
        return (m._vp * len(ls))(*[l.handle for l in ls])
    with pytest.raises(m.AsfError):
        m.Stack([layers[0], layers[0]]).decode(x)               # a layer twice
    assert lib.asf_stack_decode(arr([layers[0], other[0]]), 2, x.data_ptr(), 1, 0, y.data_ptr(),
                                w.data_ptr(), None) == 2        # d mismatch: ASF_ERR_SHAPE
    with pytest.raises(ValueError):
        m.Stack([layers[0], other[0]])
    x2 = torch.zeros((2, d), device="cuda")
    assert lib.asf_stack_decode(arr(layers), 2, x2.data_ptr(), 2, 0, y.data_ptr(),
                                w.data_ptr(), None) == 2        # B > max_batch
    with pytest.raises(ValueError):
        m.Stack(layers).decode(x2)
    st = m.Stack(layers)
    buf = torch.zeros((2, d), device="cuda")
    with pytest.raises(m.AsfError):
        st.decode(buf[:1], out=buf[1:], work=buf[:1])           # work overlaps x
    with pytest.raises(m.AsfError):
        m.Stack([layers[0], layers[0]]).decode_lookahead(x)     # a layer twice
    with pytest.raises(m.AsfError):
        st.decode_lookahead(buf[:1], out=buf[1:], work=buf[:1])


def test_opt30b_stack_full_size(orc):
    """48 layers of 7168x28672 fp16, 2 tokens through asf_stack_decode and one
    through the look-ahead form; oracle on layers 0, 23, 47."""
    need_gpu()
    from workload.gpu import stack_layer_device
    m = asf()
    sampled = (0, 23, 47)
    layers, host = [], {}
    for l in range(wl.STACK_LAYERS):
        DL = stack_layer_device(l, torch.device("cuda"))
        layers.append(m.Layer(DL.w_up, DL.w_down, DL.p1, DL.p2, b1=DL.b1, b2=DL.b2,
                              c2=DL.c2, neuron_table=DL.perm))
        if l in sampled:
            host[l] = DL.to_numpy()
        del DL
        torch.cuda.synchronize()
    st = m.Stack(layers)
    x = wl.make_tokens(wl.STACK_D, 2, 2003)
    f = wl.STACK_F
    for t in range(x.shape[0]):
        xt = to_dev(x[t:t + 1])
        y = st.decode(xt)
        cur = xt
        errs = []
        for l, lay in enumerate(layers):
            if l in sampled:
                act = torch.empty(f, dtype=torch.int32, device="cuda")
                n = torch.empty(1, dtype=torch.int32, device="cuda")
                nxt = lay.decode_step(cur, active=act, n_active=n)
                torch.cuda.synchronize()
                ids = act[:int(n.item())].cpu().numpy()
                errs.append(_check_layer(orc, host[l], cur.cpu().numpy()[0],
                                         nxt.cpu().numpy()[0], ids,
                                         "stack layer %d token %d" % (l, t)))
                frac = ids.size / f
                rho = wl.stack_layer_shape(l).rho
                assert 0.5 * rho < frac < 2.0 * rho, (l, frac, rho)
            else:
                nxt = lay.decode_step(cur)
            cur = nxt
        assert torch.equal(y, cur)
        rms = float(y.pow(2).mean().sqrt())
        assert 0.5 < rms < 2.0, rms
        print("token %d: sampled-layer rel-L2 %s, output rms %.3f" % (t, errs, rms))
    # the look-ahead form at this shape (d = 7168: FC1 rows of 14 chunks per
    # lane beside the next layer's predictor layer 1; 448 owners): equal bit
    # for bit to predict(x_{l-1}) + sparse_ffn(x_l) chained by hand; the
    # sampled layers' sets against the oracle on x_{l-1}, outputs on x_l
    xt = to_dev(x[:1])
    y_la = st.decode_lookahead(xt)
    prev, cur = xt, xt
    errs = []
    for l, lay in enumerate(layers):
        if l in sampled:
            act = torch.empty(f, dtype=torch.int32, device="cuda")
            n = torch.empty(1, dtype=torch.int32, device="cuda")
            lay.predict(prev, active=act, n_active=n)
        else:
            lay.predict(prev, want_list=False)
        nxt = lay.sparse_ffn(cur)
        if l in sampled:
            torch.cuda.synchronize()
            ids = act[:int(n.item())].cpu().numpy()
            L = host[l]
            _, s_orc, _ = orc.predict(L.p1, L.c1, L.p2, L.c2, prev.cpu().numpy())
            check_set(ids, s_orc[0], 0.0, L.perm, "look-ahead layer %d" % l)
            y_orc = orc.ffn(L.w_up, L.w_down, cur.cpu().numpy()[0], ids, b1=L.b1, b2=L.b2)
            e = rel_l2(nxt.cpu().numpy()[0], y_orc[0])
            assert e <= TOL["f16"], ("look-ahead", l, e)
            errs.append(e)
        prev, cur = cur, nxt
    torch.cuda.synchronize()
    assert torch.equal(y_la, cur), "look-ahead stack differs from the chained calls"
    print("look-ahead: sampled-layer rel-L2 %s" % errs)
