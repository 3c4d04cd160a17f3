"""Pins of the CPU fp64 oracle against facts fixed outside the oracle itself:
closed forms, brute force on tiny layers, library routines (numpy float64,
numpy's binary16 decode) and the pages' single-layer worked example.

Each test is chosen so that a plausible slip in the oracle (a dropped bias, a
wrong sign, a transposed operand, an off-by-one in a table) fails it.
"""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------- binary16
def test_half_decode_exhaustive(orc):
    """All 65,536 binary16 patterns decode exactly as numpy's float16 -> float64."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])
    # through the weight path: an fp16 weight matrix behaves like its exact widening
    w = bits[0x0001:0x7C00:97].view(np.float16).reshape(1, -1)     # finite, subnormals included
    x = np.ones((1, w.shape[1]), np.float32)
    h, _, _ = orc.predict(np.ascontiguousarray(w), None, np.ones((1, 1), np.float16), None, x)
    assert h[0, 0] == max(0.0, float(np.sum(w.astype(np.float64))))


# --------------------------------------------------------------- predictor
def test_predictor_identity_closed_form(orc):
    """P1 = [I; -I], c1 = 0, P2 = [I, -I] gives h = [x+, x-] and s = x exactly,
    so the active set is {i : x_i > theta} with ties inactive."""
    n = 32
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, n)).astype(np.float32)
    x[0, 4] = 0.0
    x[1, 7] = 0.25
    I = np.eye(n, dtype=np.float32)
    P1 = np.concatenate([I, -I], axis=0)
    P2 = np.concatenate([I, -I], axis=1)
    for theta in (0.0, 0.25, -0.5):
        h, s, act = orc.predict(P1, None, P2, None, x, theta=theta)
        xd = x.astype(np.float64)
        assert np.array_equal(h, np.concatenate([np.maximum(xd, 0), np.maximum(-xd, 0)], axis=1))
        assert np.array_equal(s, xd)
        assert np.array_equal(act, (xd > theta).astype(np.uint8))
    # strict comparison at the tie points
    _, _, act = orc.predict(P1, None, P2, None, x, theta=0.25)
    assert act[1, 7] == 0
    _, _, act = orc.predict(P1, None, P2, None, x, theta=0.0)
    assert act[0, 4] == 0


@pytest.mark.parametrize("dt", [np.float32, np.float16])
def test_predictor_vs_numpy_float64(orc, dt):
    rng = np.random.default_rng(11)
    d, H, f, B = 96, 40, 130, 3
    P1 = (rng.standard_normal((H, d)) * 0.1).astype(dt)
    P2 = (rng.standard_normal((f, H)) * 0.2).astype(dt)
    c1 = (rng.standard_normal(H) * 0.1).astype(np.float32)
    c2 = (rng.standard_normal(f) * 0.1).astype(np.float32)
    x = rng.standard_normal((B, d)).astype(np.float32)
    h, s, act = orc.predict(P1, c1, P2, c2, x, theta=0.05)
    hr = np.maximum(0.0, x.astype(np.float64) @ P1.astype(np.float64).T + c1.astype(np.float64))
    sr = hr @ P2.astype(np.float64).T + c2.astype(np.float64)
    np.testing.assert_allclose(h, hr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, sr, rtol=1e-12, atol=1e-12)
    # away from the threshold the decision agrees with the library scores
    far = np.abs(sr - 0.05) > 1e-9
    assert np.array_equal(act[far], (sr[far] > 0.05).astype(np.uint8)[...])
    # c1 and c2 matter (dropped-bias slips fail here)
    h0, s0, _ = orc.predict(P1, None, P2, None, x)
    assert not np.allclose(h0, h)


def test_predictor_bruteforce_sign_patterns(orc):
    """Dyadic weights (exact in fp64): every x in {-1,0,1}^8 against a hand loop."""
    rng = np.random.default_rng(3)
    d, H, f = 8, 8, 16
    P1 = (rng.integers(-4, 5, (H, d)) / 4.0).astype(np.float32)
    P2 = (rng.integers(-4, 5, (f, H)) / 4.0).astype(np.float32)
    c1 = (rng.integers(-4, 5, H) / 4.0).astype(np.float32)
    c2 = (rng.integers(-4, 5, f) / 4.0).astype(np.float32)
    grid = np.array(np.meshgrid(*[[-1.0, 0.0, 1.0]] * d, indexing="ij")).reshape(d, -1).T
    xs = grid.astype(np.float32)
    h, s, act = orc.predict(P1, c1, P2, c2, xs, theta=0.0)
    for t in range(0, xs.shape[0], 37):
        x = [float(v) for v in xs[t]]
        hh = []
        for k in range(H):
            acc = float(c1[k])
            for j in range(d):
                acc += float(P1[k, j]) * x[j]
            hh.append(acc if acc > 0 else 0.0)
        for i in range(f):
            acc = float(c2[i])
            for k in range(H):
                acc += float(P2[i, k]) * hh[k]
            assert s[t, i] == acc
            assert act[t, i] == (1 if acc > 0 else 0)


# --------------------------------------------------------------- FFN
def test_ffn_identity_closed_form(orc):
    """d = f, W_up = W_down = I: y = max(0, x + b1) + b2 (plain)."""
    n = 24
    rng = np.random.default_rng(7)
    I = np.eye(n, dtype=np.float32)
    x = rng.standard_normal((2, n)).astype(np.float32)
    b1 = rng.standard_normal(n).astype(np.float32)
    b2 = rng.standard_normal(n).astype(np.float32)
    y = orc.ffn(I, I, x, np.arange(n), b1=b1, b2=b2)
    ref = np.maximum(0.0, x.astype(np.float64) + b1) + b2.astype(np.float64)
    assert np.array_equal(y, ref)


def test_ffn_gated_closed_form(orc):
    """W_up = W_gate = I, bias 0, W_down = I: a_i = max(0, x_i) * x_i = max(0, x_i)^2."""
    n = 24
    rng = np.random.default_rng(8)
    I = np.eye(n, dtype=np.float32)
    x = rng.standard_normal((2, n)).astype(np.float32)
    y = orc.ffn(I, I, x, np.arange(n), W_gate=I)
    xd = x.astype(np.float64)
    assert np.array_equal(y, np.maximum(0.0, xd) ** 2)
    # a gate that differs from up: a = relu(g) * u with g = 2x, u = -x
    y2 = orc.ffn(-I, I, x, np.arange(n), W_gate=2 * I)
    assert np.array_equal(y2, np.maximum(0.0, 2 * xd) * (-xd))


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dt", [np.float32, np.float16])
def test_dense_ffn_vs_numpy_float64(orc, gated, dt):
    rng = np.random.default_rng(21 + gated)
    d, f, B = 72, 200, 3
    Wu = (rng.standard_normal((f, d)) * 0.1).astype(dt)
    Wg = (rng.standard_normal((f, d)) * 0.1).astype(dt) if gated else None
    Wd = (rng.standard_normal((d, f)) * 0.1).astype(dt)       # [d][f] like nn.Linear
    b1 = (rng.standard_normal(f) * 0.1).astype(np.float32)
    b2 = (rng.standard_normal(d) * 0.1).astype(np.float32)
    r = rng.standard_normal((B, d)).astype(np.float32)
    x = rng.standard_normal((B, d)).astype(np.float32)
    y = orc.dense_ffn(Wu, Wd, x, b1=b1, b2=b2, W_gate=Wg, resid=r)
    X = x.astype(np.float64)
    if gated:
        a = np.maximum(0.0, X @ Wg.astype(np.float64).T + b1) * (X @ Wu.astype(np.float64).T)
    else:
        a = np.maximum(0.0, X @ Wu.astype(np.float64).T + b1)
    ref = a @ Wd.astype(np.float64).T + b2 + r.astype(np.float64)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


def _dyadic_layer(rng, d, f, gated=False):
    Wu = (rng.integers(-4, 5, (f, d)) / 4.0).astype(np.float32)
    Wg = (rng.integers(-4, 5, (f, d)) / 4.0).astype(np.float32) if gated else None
    Wd = (rng.integers(-4, 5, (d, f)) / 4.0).astype(np.float32)
    b1 = (rng.integers(-4, 5, f) / 4.0).astype(np.float32)
    b2 = (rng.integers(-4, 5, d) / 4.0).astype(np.float32)
    return Wu, Wg, Wd, b1, b2


@pytest.mark.parametrize("gated", [False, True])
def test_ffn_bruteforce_all_subsets(orc, gated):
    """d = 8, f = 16, dyadic weights (fp64-exact): all 2^16 neuron sets S
    against an integer-arithmetic evaluation with numpy."""
    rng = np.random.default_rng(99 + gated)
    d, f = 8, 16
    Wu, Wg, Wd, b1, b2 = _dyadic_layer(rng, d, f, gated)
    x = (rng.integers(-4, 5, d) / 2.0).astype(np.float32)
    # integer model: scale weights by 4, x by 2
    Xi = (x * 2).astype(np.int64)
    Ui = (Wu * 4).astype(np.int64)
    Di = (Wd * 4).astype(np.int64)
    B1 = (b1 * 4).astype(np.int64)
    B2 = (b2 * 4).astype(np.int64)
    if gated:
        Gi = (Wg * 4).astype(np.int64)
        g = Gi @ Xi + 2 * B1                      # 8 * gate pre-activation
        u = Ui @ Xi                               # 8 * up
        a8x8 = np.maximum(g, 0) * u               # 64 * a
        scale = 64 * 4                            # a*Wd scale
        base = B2 * 64
    else:
        z = Ui @ Xi + 2 * B1                      # 8 * pre-activation
        a8x8 = np.maximum(z, 0)                   # 8 * a
        scale = 8 * 4
        base = B2 * 8
    masks = ((np.arange(1 << f)[:, None] >> np.arange(f)[None, :]) & 1).astype(np.int64)
    Yint = base[None, :] + (masks * a8x8[None, :]) @ Di.T     # scale * y
    ref = Yint.astype(np.float64) / scale
    for m in range(1 << f):
        S = np.nonzero(masks[m])[0]
        y = orc.ffn(Wu, Wd, x, S, b1=b1, b2=b2, W_gate=Wg)
        if not np.array_equal(y[0], ref[m]):
            raise AssertionError("subset %d: %r != %r" % (m, y[0], ref[m]))


def test_ffn_invariants_true_mask_superset_additivity(orc):
    """Neurons outside the true mask add exact zeros: sparse(true) == dense,
    sparse(superset) == dense bit for bit (both sum in ascending id); adding
    one neuron adds a_i * W_down[:, i] (exact with dyadic weights)."""
    rng = np.random.default_rng(1234)
    d, f = 64, 300
    Wu = (rng.standard_normal((f, d)) * 0.1).astype(np.float32)
    Wd = (rng.standard_normal((d, f)) * 0.1).astype(np.float32)
    b1 = (rng.standard_normal(f) * 0.3 - 0.3).astype(np.float32)
    b2 = (rng.standard_normal(d) * 0.1).astype(np.float32)
    x = rng.standard_normal((4, d)).astype(np.float32)
    dense = orc.dense_ffn(Wu, Wd, x, b1=b1, b2=b2)
    _, tm = orc.true_mask(Wu, x, b1=b1)
    for b in range(4):
        T = np.nonzero(tm[b])[0]
        assert 0 < T.size < f
        y = orc.ffn(Wu, Wd, x[b], T, b1=b1, b2=b2)
        assert np.array_equal(y[0], dense[b])
        extra = rng.choice(np.setdiff1d(np.arange(f), T), 40, replace=False)
        ys = orc.ffn(Wu, Wd, x[b], rng.permutation(np.concatenate([T, extra])), b1=b1, b2=b2)
        assert np.array_equal(ys[0], dense[b])
        # dropping a truly active neuron changes the result
        yd = orc.ffn(Wu, Wd, x[b], T[1:], b1=b1, b2=b2)
        assert not np.array_equal(yd[0], dense[b])
    # additivity with dyadic weights
    Wu2, _, Wd2, b12, b22 = _dyadic_layer(rng, 8, 20)
    x2 = (rng.integers(-4, 5, 8) / 2.0).astype(np.float32)
    S = np.array([1, 4, 9, 13])
    y0, a0 = orc.ffn(Wu2, Wd2, x2, S, b1=b12, b2=b22, return_a=True)
    for i in (0, 7, 19):
        y1, a1 = orc.ffn(Wu2, Wd2, x2, np.append(S, i), b1=b12, b2=b22, return_a=True)
        ai = max(0.0, float(Wu2[i].astype(np.float64) @ x2.astype(np.float64)) + float(b12[i]))
        assert np.array_equal(y1[0] - y0[0], ai * Wd2[:, i].astype(np.float64))


def test_ffn_empty_set_and_residual(orc):
    rng = np.random.default_rng(2)
    d, f = 16, 40
    Wu = rng.standard_normal((f, d)).astype(np.float32)
    Wd = rng.standard_normal((d, f)).astype(np.float32)
    b2 = rng.standard_normal(d).astype(np.float32)
    r = rng.standard_normal((2, d)).astype(np.float32)
    x = rng.standard_normal((2, d)).astype(np.float32)
    y = orc.ffn(Wu, Wd, x, [], b2=b2, resid=r)
    assert np.array_equal(y, r.astype(np.float64) + b2.astype(np.float64))
    y = orc.ffn(Wu, Wd, x, [])
    assert np.array_equal(y, np.zeros((2, d)))
    with pytest.raises(ValueError):
        orc.ffn(Wu, Wd, x, [3, 3])        # duplicates are rejected
    with pytest.raises(ValueError):
        orc.ffn(Wu, Wd, x, [f])           # out of range


def test_batched_union_readings(orc):
    """Union reading vs per-token masking: both equal dense per token when the
    sets are the true masks; the union grows with B; B = 1 equals the single
    token path."""
    rng = np.random.default_rng(77)
    d, f, B = 48, 256, 6
    Wu = (rng.standard_normal((f, d)) * 0.1).astype(np.float32)
    Wd = (rng.standard_normal((d, f)) * 0.1).astype(np.float32)
    b1 = (rng.standard_normal(f) * 0.3 - 0.4).astype(np.float32)
    x = rng.standard_normal((B, d)).astype(np.float32)
    dense = orc.dense_ffn(Wu, Wd, x, b1=b1)
    _, tm = orc.true_mask(Wu, x, b1=b1)
    U = orc.union(tm)
    assert np.array_equal(U, (tm.max(axis=0) > 0).astype(np.uint8))
    S = np.nonzero(U)[0]
    yu = orc.ffn(Wu, Wd, x, S, b1=b1)
    yt = orc.ffn(Wu, Wd, x, S, b1=b1, token_act=tm)
    assert np.array_equal(yu, dense) and np.array_equal(yt, dense)
    sizes = [int(orc.union(tm[:b]).sum()) for b in range(1, B + 1)]
    assert sizes == sorted(sizes) and sizes[-1] > sizes[0]
    y1 = orc.ffn(Wu, Wd, x[:1], np.nonzero(orc.union(tm[:1]))[0], b1=b1)
    assert np.array_equal(y1[0], dense[0])
    # per-token masking drops every neuron a token does not activate
    S2 = S[::2]
    ta = np.zeros_like(tm)
    ta[:, S2] = 1
    ta[0, :] = 0
    yt2 = orc.ffn(Wu, Wd, x, S2, b1=b1, token_act=ta)
    assert np.array_equal(yt2[0], np.zeros(d))


# --------------------------------------------------------------- neuron table
def test_worked_example_single_layer(orc):
    """The single-layer example: hot {3,5,7} stored first, predicted {3,4,5};
    3 and 5 come from the hot part, 4 from the cold part, 7 is skipped."""
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    perm = orc.hot_first_table(np.array(g["counts"]))
    assert perm.tolist() == g["expected_table"]
    active = np.zeros(g["f"], np.uint8)
    active[g["predicted_active"]] = 1
    lst = orc.active_list(active, perm)
    assert lst.tolist() == g["expected_active_list"]
    slot_of = np.argsort(perm)
    assert sorted(slot_of[lst].tolist()) == g["expected_active_slots"]
    hot = set(perm[: g["hot_count"]].tolist())
    assert sorted(set(lst.tolist()) & hot) == g["expected_hot_computed"]
    assert sorted(set(lst.tolist()) - hot) == g["expected_cold_computed"]
    assert sorted(hot - set(lst.tolist())) == g["expected_hot_skipped"]


def test_hot_first_table_bruteforce(orc):
    rng = np.random.default_rng(4)
    for f in (1, 2, 7, 50, 333):
        counts = rng.integers(0, 5, f)
        perm = orc.hot_first_table(counts)
        ref = sorted(range(f), key=lambda i: (-int(counts[i]), i))
        assert perm.tolist() == ref
    # identity table when every count ties
    assert orc.hot_first_table(np.zeros(9)).tolist() == list(range(9))


def test_count_and_active_list(orc):
    rng = np.random.default_rng(6)
    act = (rng.random((5, 70)) < 0.3).astype(np.uint8)
    c = orc.count_activations(act)
    assert np.array_equal(c, act.sum(axis=0).astype(np.int64))
    perm = rng.permutation(70).astype(np.int32)
    lst = orc.active_list(act[2], perm)
    assert lst.tolist() == [int(i) for i in perm if act[2, i]]
    assert orc.active_list(act[2]).tolist() == np.nonzero(act[2])[0].tolist()


# --------------------------------------------------------------- true mask
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dt", [np.float32, np.float16])
def test_true_mask_pre_activations_vs_numpy_float64(orc, gated, dt):
    """The true set rests on the FFN's own ReLU zero pattern ("Técnicas
    dispersas…", section "Viabilidad de la sparsidad de activación"):
    pre = W x + b1 with W the gate matrix when gated (the gated layer's set is
    decided by ReLU(gate)), else the up matrix; act = pre > 0, strict."""
    rng = np.random.default_rng(77 + 2 * gated + (dt == np.float16))
    d, f, B = 48, 130, 4
    Wu = (rng.standard_normal((f, d)) * 0.2).astype(dt)
    Wg = (rng.standard_normal((f, d)) * 0.2).astype(dt) if gated else None
    b1 = (rng.standard_normal(f) * 0.3).astype(np.float32)
    x = rng.standard_normal((B, d)).astype(np.float32)
    pre, act = orc.true_mask(Wu, x, b1=b1, W_gate=Wg)
    W = (Wg if gated else Wu).astype(np.float64)
    ref = x.astype(np.float64) @ W.T + b1.astype(np.float64)
    np.testing.assert_allclose(pre, ref, rtol=1e-12, atol=1e-13)
    assert np.array_equal(act, (pre > 0).astype(np.uint8))
    # the set differs from the other matrix's (a swapped W would fail here)
    if gated:
        other = x.astype(np.float64) @ Wu.astype(np.float64).T + b1
        assert not np.array_equal(act, (other > 0).astype(np.uint8))
    # the gated FFN over the true set is the dense gated FFN bit for bit (the
    # terms off the set are exact zeros and both sums run in ascending id)
    Wd = (rng.standard_normal((d, f)) * 0.2).astype(dt)
    b2 = (rng.standard_normal(d) * 0.1).astype(np.float32)
    dense = orc.dense_ffn(Wu, Wd, x, b1=b1, b2=b2, W_gate=Wg)
    for b in range(B):
        T = np.nonzero(act[b])[0]
        y = orc.ffn(Wu, Wd, x[b], T, b1=b1, b2=b2, W_gate=Wg)
        assert np.array_equal(y[0], dense[b])


def test_true_mask_bias_and_tie(orc):
    """b1 is added before the comparison (not after the store), no bias means
    zero, and a pre-activation of exactly 0 is inactive."""
    d, f = 4, 6
    W = np.zeros((f, d), np.float32)
    W[0, 0] = 1.0          # z0 = x0
    W[1, 1] = -1.0         # z1 = -x1
    W[2, 2] = 0.5          # z2 = x2 / 2
    x = np.array([[2.0, 3.0, -4.0, 1.0]], np.float32)
    b1 = np.array([-2.0, 3.0, 2.5, 0.0, -1.0, 0.75], np.float32)
    pre, act = orc.true_mask(W, x, b1=b1)
    assert pre[0].tolist() == [0.0, 0.0, 0.5, 0.0, -1.0, 0.75]
    assert act[0].tolist() == [0, 0, 1, 0, 0, 1]
    pre0, act0 = orc.true_mask(W, x)
    assert pre0[0].tolist() == [2.0, -3.0, -2.0, 0.0, 0.0, 0.0]
    assert act0[0].tolist() == [1, 0, 0, 0, 0, 0]
    # gated: the gate decides, up never does
    Wg = np.zeros((f, d), np.float32)
    Wg[3, 3] = 1.0
    pre_g, act_g = orc.true_mask(W, x, W_gate=Wg)
    assert pre_g[0].tolist() == [0.0, 0.0, 0.0, 1.0, 0.0, 0.0]
    assert act_g[0].tolist() == [0, 0, 0, 1, 0, 0]


# --------------------------------------------------------------- attention-head predictor
def test_head_predictor_identity_closed_form(orc):
    """The head predictor is the two-layer MLP with one output per head
    ("LLM模型之PowerInfer1.0", appendix "DejaVu", SP_A): with Q1 = [I; -I],
    Q2 = [I, -I] the head logits are x itself, so token b selects the heads
    {j : x_bj > theta}, listed in ascending order, each token on its own."""
    n = 40
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, n)).astype(np.float32)
    x[2, 5] = 0.0
    I = np.eye(n, dtype=np.float32)
    for theta in (0.0, 0.5):
        s, act, lists = orc.predict_heads(np.concatenate([I, -I]), None,
                                          np.concatenate([I, -I], axis=1), None, x, theta=theta)
        assert np.array_equal(s, x.astype(np.float64))
        for b in range(3):
            assert lists[b].tolist() == [j for j in range(n) if x[b, j] > theta]
            assert np.array_equal(act[b], (x[b] > theta).astype(np.uint8))
        assert 5 not in lists[2].tolist()      # a logit equal to theta = 0 is not selected


def test_head_predictor_bruteforce(orc):
    """d = 3, H = 4, 5 heads, dyadic weights (fp64-exact): every x in
    {-1, 0, 1}^3 against a hand loop of relu(Q1 x + c1), Q2 h + c2, s > 0."""
    rng = np.random.default_rng(9)
    Q1 = (rng.integers(-4, 5, (4, 3)) / 4.0).astype(np.float32)
    c1 = (rng.integers(-4, 5, 4) / 4.0).astype(np.float32)
    Q2 = (rng.integers(-4, 5, (5, 4)) / 4.0).astype(np.float32)
    c2 = (rng.integers(-4, 5, 5) / 8.0).astype(np.float32)
    xs = np.array([[a, b, c] for a in (-1, 0, 1) for b in (-1, 0, 1) for c in (-1, 0, 1)],
                  np.float32)
    s, act, lists = orc.predict_heads(Q1, c1, Q2, c2, xs)
    for t, xv in enumerate(xs):
        h = [max(0.0, sum(float(Q1[k, j]) * float(xv[j]) for j in range(3)) + float(c1[k]))
             for k in range(4)]
        ref = [sum(float(Q2[i, k]) * h[k] for k in range(4)) + float(c2[i]) for i in range(5)]
        assert s[t].tolist() == ref
        assert lists[t].tolist() == [i for i in range(5) if ref[i] > 0.0]
