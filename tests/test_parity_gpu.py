"""GPU parity: the HIP path through the C ABI against the CPU fp64 oracle on
the same seeded inputs.

* Active sets: bit-exact on every neuron whose predictor margin exceeds 1e-3,
  listed in ascending stored-slot order.
* Outputs: per-token relative L2 <= 1e-3 (fp32 weights) / 5e-3 (fp16
  weights, fp32 accumulate), against the oracle evaluated on the GPU's own
  set, so set and output parity are checked separately.
"""
import numpy as np
import pytest
import torch

import workload as wl
from gpu_util import MARGIN, TOL, asf, check_set, need_gpu, rel_l2, to_dev

pytestmark = pytest.mark.gpu


def _run_tokens(orc, L, x, layer, label, check_dense=True, theta=0.0):
    """Per token: predict, decode_step, sparse_ffn on the GPU set, dense."""
    tol = TOL[L.shape.wdtype]
    f = L.shape.f
    _, s_orc, _ = orc.predict(L.p1, L.c1, L.p2, L.c2, x, theta=theta)
    dense_orc = orc.dense_ffn(L.w_up, L.w_down, x, b1=L.b1, b2=L.b2, W_gate=L.w_gate) \
        if check_dense else None
    amb = 0
    worst = 0.0
    for t in range(x.shape[0]):
        xt = to_dev(x[t:t + 1])
        active, n = layer.predict(xt)
        y1 = layer.sparse_ffn(xt)
        a2 = torch.empty_like(active)
        n2 = torch.empty_like(n)
        y2 = layer.decode_step(xt, active=a2, n_active=n2)
        torch.cuda.synchronize()
        k = int(n.item())
        ids = active[:k].cpu().numpy()
        assert int(n2.item()) == k and np.array_equal(a2[:k].cpu().numpy(), ids)
        assert torch.equal(y1, y2), "decode_step differs from predict + sparse_ffn"
        amb += check_set(ids, s_orc[t], theta, L.perm, "%s token %d" % (label, t))
        y_orc = orc.ffn(L.w_up, L.w_down, x[t], ids, b1=L.b1, b2=L.b2, W_gate=L.w_gate)
        e = max(rel_l2(y1.cpu().numpy()[0], y_orc[0]), rel_l2(y2.cpu().numpy()[0], y_orc[0]))
        worst = max(worst, e)
        assert e <= tol, "%s token %d: rel-L2 %.3g > %.3g" % (label, t, e, tol)
        if check_dense:
            yd = layer.dense_ffn_ref(xt)
            ed = rel_l2(yd.cpu().numpy()[0], dense_orc[t])
            assert ed <= tol, "%s token %d dense: rel-L2 %.3g" % (label, t, ed)
    print("%s: %d tokens, worst rel-L2 %.3g, ambiguous flips %d" % (label, x.shape[0], worst, amb))
    return worst


def test_tiny_fp32_full_config(orc):
    """256x1024 fp32, predictor 256->64->1024, 64 decode tokens (full size)."""
    need_gpu()
    L = wl.config_layer("tiny_f32")
    x = wl.config_tokens("tiny_f32", 64)
    lay = asf().layer_from_numpy(L)
    _run_tokens(orc, L, x, lay, "tiny_f32")


@pytest.mark.parametrize("d,f,H", [(512, 2000, 128), (1024, 4160, 256), (256, 40, 64)])
def test_scaled_fp16_ragged(orc, d, f, H):
    """fp16 layers with the OPT-6.7B firing law at sizes that span several
    workgroups and end in a ragged mask word."""
    need_gpu()
    _, sh = wl.CONFIGS["opt6.7b_ffn"]
    L = wl.make_layer(wl.scaled_shape(sh, d, f, H), 31 + f)
    x = wl.make_tokens(d, 6, 41 + f)
    lay = asf().layer_from_numpy(L)
    _run_tokens(orc, L, x, lay, "fp16 %dx%d H%d" % (d, f, H))


def test_opt67_full_size(orc):
    """The headline shape: 4096x16384 fp16, predictor 4096->1024->16384."""
    need_gpu()
    L = wl.config_layer("opt6.7b_ffn")
    x = wl.config_tokens("opt6.7b_ffn", 4)
    lay = asf().layer_from_numpy(L)
    _run_tokens(orc, L, x, lay, "opt6.7b_ffn")


def test_gated_scaled_and_full(orc):
    need_gpu()
    _, sh = wl.CONFIGS["llama7b_gated_relu"]
    Ls = wl.make_layer(wl.scaled_shape(sh, 512, 1376, 128), 77)
    xs = wl.make_tokens(512, 6, 78)
    _run_tokens(orc, Ls, xs, asf().layer_from_numpy(Ls), "gated 512x1376")
    L = wl.config_layer("llama7b_gated_relu")
    x = wl.config_tokens("llama7b_gated_relu", 3)
    _run_tokens(orc, L, x, asf().layer_from_numpy(L), "llama7b_gated_relu")


def test_user_list_any_order_and_bad_ids(orc):
    """A caller's id list in any order; out-of-range ids are skipped."""
    need_gpu()
    L = wl.random_layer(384, 1000, 64, "f16", False, 5)
    lay = asf().layer_from_numpy(L)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 384)).astype(np.float32)
    ids = rng.choice(1000, 300, replace=False).astype(np.int32)
    dev = to_dev(np.concatenate([ids, np.array([-5, 1000, 99999], np.int32)]))
    n = to_dev(np.array([dev.numel()], np.int32))
    y = lay.sparse_ffn(to_dev(x), active=dev, n_active=n)
    y_orc = orc.ffn(L.w_up, L.w_down, x, ids, b1=L.b1, b2=L.b2)
    assert rel_l2(y.cpu().numpy(), y_orc) <= TOL["f16"]
    # every neuron through the list equals the dense comparator
    allids = to_dev(rng.permutation(1000).astype(np.int32))
    yall = lay.sparse_ffn(to_dev(x), active=allids, n_active=to_dev(np.array([1000], np.int32)))
    yd = lay.dense_ffn_ref(to_dev(x))
    assert rel_l2(yall.cpu().numpy(), yd.cpu().numpy()) <= 1e-5


def test_empty_set_and_residual_alias(orc):
    need_gpu()
    L = wl.random_layer(256, 512, 64, "f32", False, 6)
    lay = asf().layer_from_numpy(L)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 256)).astype(np.float32)
    r = rng.standard_normal((1, 256)).astype(np.float32)
    empty = to_dev(np.zeros(4, np.int32))
    zero = to_dev(np.array([0], np.int32))
    y = lay.sparse_ffn(to_dev(x), active=empty, n_active=zero, residual=to_dev(r))
    expect = (np.float32(0.0) + L.b2) + r
    assert np.array_equal(y.cpu().numpy(), expect)
    # y aliasing the residual (in-place residual stream)
    rd = to_dev(r)
    ids = to_dev(np.arange(0, 512, 3).astype(np.int32))
    cnt = to_dev(np.array([ids.numel()], np.int32))
    lay.sparse_ffn(to_dev(x), active=ids, n_active=cnt, residual=rd, out=rd)
    y_orc = orc.ffn(L.w_up, L.w_down, x, np.arange(0, 512, 3), b1=L.b1, b2=L.b2, resid=r)
    assert rel_l2(rd.cpu().numpy(), y_orc) <= TOL["f32"]


@pytest.mark.parametrize("B,gated", [(3, False), (6, False), (32, False), (5, True)])
def test_batched_caller_lists(orc, B, gated):
    """Batches over a caller's list on the matrix-core kernels (k-sliced FC1,
    hi + lo FC2), at a d whose last k slice is partly past the row: out-of-
    range ids skipped, a repeated id computed once per listing, an empty list
    giving b2 + residual exactly, and every id in a shuffled order matching
    the dense comparator's slot order to summation rounding."""
    need_gpu()
    d, f = 1408, 1000
    L = wl.random_layer(d, f, 64, "f16", gated, 40 + B)
    lay = asf().layer_from_numpy(L, max_batch=32)
    rng = np.random.default_rng(B)
    x = rng.standard_normal((B, d)).astype(np.float32)
    r = rng.standard_normal((B, d)).astype(np.float32)
    ids = rng.choice(f, 230, replace=False).astype(np.int32)
    lst = np.concatenate([ids[:100], np.array([-3, f, 1 << 30], np.int32), ids[100:],
                          ids[:5]]).astype(np.int32)
    y = lay.sparse_ffn(to_dev(x), active=to_dev(lst),
                       n_active=to_dev(np.array([lst.size], np.int32)), residual=to_dev(r))
    # the five repeated ids count twice: the oracle over the list as given
    # (valid entries, repeats kept)
    valid = lst[(lst >= 0) & (lst < f)]
    y_orc = np.zeros((B, d))
    for once in (valid[:230], valid[230:]):
        y_orc += orc.ffn(L.w_up, L.w_down, x, once, b1=L.b1, b2=None, W_gate=L.w_gate)
    y_orc += L.b2.astype(np.float64) + r
    yg = y.cpu().numpy()
    for t in range(B):
        assert rel_l2(yg[t], y_orc[t]) <= TOL["f16"], t
    # an empty list: b2 + residual, exactly
    y0 = lay.sparse_ffn(to_dev(x), active=to_dev(np.zeros(4, np.int32)),
                        n_active=to_dev(np.array([0], np.int32)), residual=to_dev(r))
    assert np.array_equal(y0.cpu().numpy(), (np.float32(0.0) + L.b2) + r)
    # every neuron, shuffled, against the dense comparator
    allids = to_dev(rng.permutation(f).astype(np.int32))
    ya = lay.sparse_ffn(to_dev(x), active=allids, n_active=to_dev(np.array([f], np.int32)))
    yd = lay.dense_ffn_ref(to_dev(x))
    torch.cuda.synchronize()
    for t in range(B):
        assert rel_l2(ya.cpu().numpy()[t], yd.cpu().numpy()[t]) <= 1e-5, t


def test_true_mask_sparse_equals_dense_on_gpu(orc):
    """With the true mask as the set, the sparse FFN equals the dense one."""
    need_gpu()
    L = wl.config_layer("opt6.7b_ffn", shape=wl.scaled_shape(wl.CONFIGS["opt6.7b_ffn"][1],
                                                             1024, 4096, 256))
    lay = asf().layer_from_numpy(L)
    x = wl.make_tokens(1024, 3, 9)
    _, tm = orc.true_mask(L.w_up, x, b1=L.b1)
    for t in range(3):
        ids = np.nonzero(tm[t])[0].astype(np.int32)
        y = lay.sparse_ffn(to_dev(x[t:t + 1]), active=to_dev(ids),
                           n_active=to_dev(np.array([ids.size], np.int32)))
        yd = lay.dense_ffn_ref(to_dev(x[t:t + 1]))
        assert rel_l2(y.cpu().numpy(), yd.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("B", [2, 4, 7, 32])
def test_batched_union(orc, B):
    """B tokens: the union of their predicted sets, every token computing
    every neuron of the union."""
    need_gpu()
    _, sh = wl.CONFIGS["opt13b_batched"]
    L = wl.make_layer(wl.scaled_shape(sh, 640, 2560, 128), 100 + B)
    lay = asf().layer_from_numpy(L, max_batch=32)
    x = wl.make_tokens(640, B, 200 + B)
    masks = torch.zeros((B, (L.shape.f + 63) // 64), dtype=torch.int64, device="cuda")
    active, n = lay.predict(to_dev(x), token_masks=masks)
    y = lay.sparse_ffn(to_dev(x))
    torch.cuda.synchronize()
    k = int(n.item())
    ids = active[:k].cpu().numpy()
    _, s_orc, act = orc.predict(L.p1, L.c1, L.p2, L.c2, x)
    # per-token masks (stored order) against the oracle, margin rule
    mw = masks.cpu().numpy().view(np.uint64)
    bits = ((mw[:, :, None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)).reshape(B, -1)
    bits = bits[:, :L.shape.f].astype(bool)
    for t in range(B):
        tok_ids = L.perm[np.nonzero(bits[t])[0]]          # ascending slot order
        check_set(tok_ids, s_orc[t], 0.0, L.perm, "B%d tok %d" % (B, t))
    # union list: its members are exactly the OR of the token masks
    u = bits.any(axis=0)
    assert np.array_equal(ids, L.perm[np.nonzero(u)[0]])
    # union margin rule: a neuron surely in / out of every token's set
    s_max = s_orc.max(axis=0)
    check_set(ids, s_max, 0.0, L.perm, "B%d union" % B)
    y_orc = orc.ffn(L.w_up, L.w_down, x, ids, b1=L.b1, b2=L.b2)
    yg = y.cpu().numpy()
    for t in range(B):
        assert rel_l2(yg[t], y_orc[t]) <= TOL["f16"]
    yd = lay.dense_ffn_ref(to_dev(x)).cpu().numpy()
    yd_orc = orc.dense_ffn(L.w_up, L.w_down, x, b1=L.b1, b2=L.b2)
    for t in range(B):
        assert rel_l2(yd[t], yd_orc[t]) <= TOL["f16"]


def test_identity_table_and_threshold(orc):
    """No neuron table (stored order = original order) and a nonzero logit
    threshold; all-active and none-active thresholds."""
    need_gpu()
    L = wl.random_layer(256, 700, 32, "f32", False, 12)
    x = np.random.default_rng(3).standard_normal((2, 256)).astype(np.float32)
    for theta in (0.3, -1e30, 1e30):
        lay = asf().layer_from_numpy(L, use_table=False, threshold=theta)
        _, s_orc, _ = orc.predict(L.p1, L.c1, L.p2, L.c2, x, theta=theta)
        for t in range(2):
            active, n = lay.predict(to_dev(x[t:t + 1]))
            y = lay.sparse_ffn(to_dev(x[t:t + 1]))
            k = int(n.item())
            if theta == -1e30:
                assert k == 700
            if theta == 1e30:
                assert k == 0
            ids = active[:k].cpu().numpy()
            check_set(ids, s_orc[t], theta, np.arange(700), "theta %g" % theta)
            y_orc = orc.ffn(L.w_up, L.w_down, x[t], ids, b1=L.b1, b2=L.b2)
            assert rel_l2(y.cpu().numpy()[0], y_orc[0]) <= TOL["f32"]


def test_deterministic_repeat():
    need_gpu()
    L = wl.random_layer(512, 3000, 64, "f16", True, 13)
    lay = asf().layer_from_numpy(L)
    x = to_dev(np.random.default_rng(4).standard_normal((1, 512)).astype(np.float32))
    y1 = lay.decode_step(x).clone()
    y2 = lay.decode_step(x).clone()
    d1 = lay.dense_ffn_ref(x).clone()
    d2 = lay.dense_ffn_ref(x).clone()
    assert torch.equal(y1, y2) and torch.equal(d1, d2)


@pytest.mark.parametrize("d,f,H,gated", [(2048, 3000, 256, False), (2048, 2500, 512, True),
                                         (5120, 4160, 1024, False), (7168, 2048, 2048, False)])
def test_decode_step_tiling_variants(orc, d, f, H, gated):
    """The decode-step kernels (fp16, B = 1) across their register-tiling
    variants (d and H classes): same bits as predict + sparse_ffn, oracle
    parity."""
    need_gpu()
    _, sh = wl.CONFIGS["llama7b_gated_relu" if gated else "opt6.7b_ffn"]
    L = wl.make_layer(wl.scaled_shape(sh, d, f, H), 500 + d + f)
    lay = asf().layer_from_numpy(L)
    x = wl.make_tokens(d, 5, 600 + f)
    worst = _run_tokens(orc, L, x, lay, "fused %dx%d H%d%s" % (d, f, H, " gated" if gated else ""),
                        check_dense=False)
    assert worst <= TOL["f16"]


def _batched_check(orc, L, x, lay, label, check_dense=True, user_list=True):
    """B tokens through the batched (matrix-core) path: per-token masks and
    the union against the oracle's scores (margin rule); decode_step equal bit
    for bit to predict + sparse_ffn; outputs against the oracle over the GPU's
    union; a caller id list in any order; the dense comparator."""
    B, f = x.shape[0], L.shape.f
    tol = TOL[L.shape.wdtype]
    xd = to_dev(x)
    masks = torch.zeros((B, (f + 63) // 64), dtype=torch.int64, device="cuda")
    active, n = lay.predict(xd, token_masks=masks)
    y1 = lay.sparse_ffn(xd)
    a2 = torch.empty_like(active)
    n2 = torch.empty_like(n)
    y2 = lay.decode_step(xd, active=a2, n_active=n2)
    torch.cuda.synchronize()
    k = int(n.item())
    ids = active[:k].cpu().numpy()
    assert int(n2.item()) == k and np.array_equal(a2[:k].cpu().numpy(), ids)
    assert torch.equal(y1, y2), label + ": decode_step differs from predict + sparse_ffn"
    _, s_orc, _ = orc.predict(L.p1, L.c1, L.p2, L.c2, x)
    mw = masks.cpu().numpy().view(np.uint64)
    bits = ((mw[:, :, None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)).reshape(B, -1)
    bits = bits[:, :f].astype(bool)
    amb = 0
    for t in range(B):
        amb += check_set(L.perm[np.nonzero(bits[t])[0]], s_orc[t], 0.0, L.perm,
                         "%s tok %d" % (label, t))
    assert np.array_equal(ids, L.perm[np.nonzero(bits.any(axis=0))[0]])
    y_orc = orc.ffn(L.w_up, L.w_down, x, ids, b1=L.b1, b2=L.b2, W_gate=L.w_gate)
    yg = y1.cpu().numpy()
    worst = max(rel_l2(yg[t], y_orc[t]) for t in range(B))
    assert worst <= tol, "%s: rel-L2 %.3g" % (label, worst)
    if user_list:
        rng = np.random.default_rng(B)
        sub = rng.permutation(ids)[: max(1, k // 2)].astype(np.int32)
        yl = lay.sparse_ffn(xd, active=to_dev(sub), n_active=to_dev(np.array([sub.size], np.int32)))
        yl_orc = orc.ffn(L.w_up, L.w_down, x, sub, b1=L.b1, b2=L.b2, W_gate=L.w_gate)
        ylg = yl.cpu().numpy()
        for t in range(B):
            assert rel_l2(ylg[t], yl_orc[t]) <= tol
    if check_dense:
        yd = lay.dense_ffn_ref(xd).cpu().numpy()
        yd_orc = orc.dense_ffn(L.w_up, L.w_down, x, b1=L.b1, b2=L.b2, W_gate=L.w_gate)
        for t in range(B):
            assert rel_l2(yd[t], yd_orc[t]) <= tol
    print("%s: B=%d union %d (%.3f), worst rel-L2 %.3g, ambiguous flips %d"
          % (label, B, k, k / f, worst, amb))


@pytest.mark.parametrize("B,gated", [(3, False), (16, False), (5, True), (32, True), (4, True),
                                     (8, False)])
def test_batched_matrix_core_path(orc, B, gated):
    """Scaled layers with ragged tiles (d not a multiple of 256, H not of 64,
    f not of 64) through the batched kernels; B = 4 is the largest batch whose
    predictor layer 1 runs as a vector kernel, B = 5 the smallest on the
    matrix cores."""
    need_gpu()
    _, sh = wl.CONFIGS["llama7b_gated_relu" if gated else "opt13b_batched"]
    L = wl.make_layer(wl.scaled_shape(sh, 1152, 3000 + 7 * B, 200), 900 + B)
    lay = asf().layer_from_numpy(L, max_batch=32)
    x = wl.make_tokens(1152, B, 950 + B)
    _batched_check(orc, L, x, lay, "mm %s" % ("gated" if gated else "plain"))


@pytest.mark.parametrize("gated", [False, True])
def test_largest_d_model(orc, gated):
    """d_model 8192, the largest an fp16 layer takes (16 KiB rows): the
    one-token kernels at 16 chunks per lane, and the batched path at its
    limits (8 FC1 k slices, 16 predictor k slices at B = 5, the vector
    predictor at B = 3), with a ragged f."""
    need_gpu()
    _, sh = wl.CONFIGS["llama7b_gated_relu" if gated else "opt6.7b_ffn"]
    d, f, H = 8192, 1500 + (37 if gated else 0), 512
    L = wl.make_layer(wl.scaled_shape(sh, d, f, H), 1700 + f)
    lay = asf().layer_from_numpy(L, max_batch=8)
    x = wl.make_tokens(d, 3, 1800 + f)
    worst = _run_tokens(orc, L, x, lay, "d8192 B=1%s" % (" gated" if gated else ""),
                        check_dense=False)
    assert worst <= TOL["f16"]
    for B in (3, 5):
        xb = wl.make_tokens(d, B, 1900 + B + f)
        _batched_check(orc, L, xb, lay, "d8192 B=%d%s" % (B, " gated" if gated else ""),
                       check_dense=(B == 5))


@pytest.mark.parametrize("gated", [False, True])
def test_largest_d_model_fp32(orc, gated):
    """d_model 4096 with fp32 weights (16 KiB rows, the largest fp32 layer):
    one token at 16 chunks per lane and batches of 4 on the vector kernels,
    plain and gated, ragged f."""
    need_gpu()
    import dataclasses
    _, sh = wl.CONFIGS["tiny_f32"]
    shp = dataclasses.replace(wl.scaled_shape(sh, 4096, 1200 + (29 if gated else 0), 256),
                              gated=gated)
    L = wl.make_layer(shp, 2100 + shp.f)
    lay = asf().layer_from_numpy(L, max_batch=8)
    x = wl.make_tokens(4096, 2, 2200 + shp.f)
    worst = _run_tokens(orc, L, x, lay, "fp32 d4096 B=1%s" % (" gated" if gated else ""),
                        check_dense=False)
    assert worst <= TOL["f32"]
    xb = wl.make_tokens(4096, 4, 2300 + shp.f)
    _batched_check(orc, L, xb, lay, "fp32 d4096 B=4%s" % (" gated" if gated else ""))


@pytest.mark.parametrize("B", [2, 4, 5, 32])
def test_batched_fp32_weights(orc, B):
    """fp32 weights with B >= 2 run the vector kernels (predictor layer 1
    over token chunks of 4, scores per token chunk, FC1 over the union, the
    grouped FC2): per-token sets, the union, outputs over it, a caller list
    and the dense comparator against the oracle, at a ragged d_ffn."""
    need_gpu()
    _, sh = wl.CONFIGS["tiny_f32"]
    L = wl.make_layer(wl.scaled_shape(sh, 640, 2500 + 3 * B, 128), 1300 + B)
    lay = asf().layer_from_numpy(L, max_batch=32)
    x = wl.make_tokens(640, B, 1350 + B)
    _batched_check(orc, L, x, lay, "fp32 B%d" % B)


def test_batched_full_size(orc):
    """The OPT-13B-shaped layer (5120x20480 fp16, predictor 5120->1024->20480)
    at batch 4 and 32."""
    need_gpu()
    L = wl.config_layer("opt13b_batched")
    lay = asf().layer_from_numpy(L, max_batch=32)
    X = wl.config_tokens("opt13b_batched", 36)
    for B, off in ((4, 0), (32, 4)):
        _batched_check(orc, L, X[off:off + B], lay, "opt13b B%d" % B, check_dense=(B == 4),
                       user_list=(B == 32))


def test_max_ffn_size(orc):
    """d_ffn at its maximum (65536: 1024 owners, 1024 mask words): the
    single-token step, the batched step at max_batch = 32 and the exact-mask
    mode against the oracle."""
    need_gpu()
    _, sh = wl.CONFIGS["opt6.7b_ffn"]
    L = wl.make_layer(wl.scaled_shape(sh, 512, 65536, 128), 65536)
    lay = asf().layer_from_numpy(L, max_batch=32)
    x = wl.make_tokens(512, 32, 655)
    worst = _run_tokens(orc, L, x[:2], lay, "f=65536", check_dense=False)
    assert worst <= TOL["f16"]
    _batched_check(orc, L, x, lay, "f=65536 B=32", check_dense=False, user_list=False)
    pre, _ = orc.true_mask(L.w_up, x[:1], b1=L.b1)
    act = torch.empty(L.shape.f, dtype=torch.int32, device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")
    y = lay.exact_ffn(to_dev(x[:1]), active=act, n_active=n)
    torch.cuda.synchronize()
    ids = act[:int(n.item())].cpu().numpy()
    check_set(ids, pre[0], 0.0, L.perm, "f=65536 exact")
    y_orc = orc.dense_ffn(L.w_up, L.w_down, x[:1], b1=L.b1, b2=L.b2)
    assert rel_l2(y.cpu().numpy()[0], y_orc[0]) <= TOL["f16"]


@pytest.mark.parametrize("cfg,d,f,H", [("opt6.7b_ffn", 4096, 16384, 1024), ("opt6.7b_ffn", 512, 1000, 64),
                                       ("llama7b_gated_relu", 1024, 3000, 256),
                                       ("tiny_f32", 256, 1024, 64)])
def test_one_token_list_is_the_decode_step(orc, cfg, d, f, H):
    """One token over a caller's list runs the decode step's owner kernels:
    the predicted list (in any order, with repeats and out-of-range ids
    mixed in) gives decode_step's y bit for bit; a sampled set at 10%
    matches the oracle."""
    need_gpu()
    _, sh = wl.CONFIGS[cfg]
    L = wl.make_layer(wl.scaled_shape(sh, d, f, H), 300 + f)
    lay = asf().layer_from_numpy(L)
    x = wl.make_tokens(d, 3, 400 + f)
    rng = np.random.default_rng(f)
    for t in range(3):
        xt = to_dev(x[t:t + 1])
        active = torch.empty(f, dtype=torch.int32, device="cuda")
        n = torch.empty(1, dtype=torch.int32, device="cuda")
        y_step = lay.decode_step(xt, active=active, n_active=n)
        torch.cuda.synchronize()
        ids = active[:int(n.item())].cpu().numpy()
        mixed = np.concatenate([rng.permutation(ids), ids[:5], np.array([-1, f, 1 << 30], np.int32)])
        y_list = lay.sparse_ffn(xt, active=to_dev(mixed.astype(np.int32)),
                                n_active=to_dev(np.array([mixed.size], np.int32)))
        torch.cuda.synchronize()
        assert torch.equal(y_list, y_step), "token %d: list path differs from decode_step" % t
    sets = wl.sampled_sets(L.perm, 0.10, 2, seed=9)
    for t, st in enumerate(sets):
        y = lay.sparse_ffn(to_dev(x[t:t + 1]), active=to_dev(st),
                           n_active=to_dev(np.array([st.size], np.int32)))
        y_orc = orc.ffn(L.w_up, L.w_down, x[t], st, b1=L.b1, b2=L.b2, W_gate=L.w_gate)
        assert rel_l2(y.cpu().numpy()[0], y_orc[0]) <= TOL[sh.wdtype]


def test_one_token_long_lists(orc):
    """Caller lists longer than one pass of the list kernel (2048 ids per
    pass): 40% of the neurons against the oracle, every neuron against the
    dense comparator, both in shuffled order."""
    need_gpu()
    _, sh = wl.CONFIGS["opt6.7b_ffn"]
    L = wl.make_layer(wl.scaled_shape(sh, 1024, 16384, 256), 555)
    lay = asf().layer_from_numpy(L)
    x = wl.make_tokens(1024, 2, 556)
    rng = np.random.default_rng(557)
    ids = rng.choice(16384, 6554, replace=False).astype(np.int32)
    y = lay.sparse_ffn(to_dev(x[:1]), active=to_dev(ids), n_active=to_dev(np.array([ids.size], np.int32)))
    y_orc = orc.ffn(L.w_up, L.w_down, x[0], ids, b1=L.b1, b2=L.b2)
    assert rel_l2(y.cpu().numpy()[0], y_orc[0]) <= TOL["f16"]
    allids = rng.permutation(16384).astype(np.int32)
    yall = lay.sparse_ffn(to_dev(x[1:]), active=to_dev(allids),
                          n_active=to_dev(np.array([allids.size], np.int32)))
    yd = lay.dense_ffn_ref(to_dev(x[1:]))
    assert rel_l2(yall.cpu().numpy(), yd.cpu().numpy()) <= 1e-5
