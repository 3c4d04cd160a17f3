"""The synthetic workload has the shape the pages describe: a power-law firing
law at the configured activation fraction, a predictor with recall near 0.95,
and batch unions that densify as the closed form says."""
import numpy as np
import pytest

import workload as wl


@pytest.mark.parametrize("name,cap_count", [("tiny_f32", 25), ("opt6.7b_ffn", 264),
                                            ("llama7b_gated_relu", 271), ("opt13b_batched", 223)])
def test_firing_law(name, cap_count):
    idx, sh = wl.CONFIGS[name]
    rng = np.random.Generator(np.random.PCG64(wl.layer_seed(idx)))
    p, rank = wl.firing_probabilities(sh.f, sh.rho, rng)
    assert abs(p.mean() - sh.rho) < 1e-9
    assert np.all(np.diff(p[np.argsort(rank)]) <= 0)        # decreasing in rank
    assert int((p >= wl.P_CAP - 1e-12).sum()) == cap_count
    assert sorted(rank.tolist()) == list(range(1, sh.f + 1))


def test_stack_schedule():
    Hs = [wl.stack_layer_shape(l).H for l in range(wl.STACK_LAYERS)]
    assert Hs.count(512) == 16 and Hs.count(1024) == 16 and Hs.count(2048) == 16
    rhos = [wl.stack_layer_shape(l).rho for l in range(wl.STACK_LAYERS)]
    assert abs(rhos[0] - 0.03) < 1e-12 and abs(rhos[-1] - 0.15) < 1e-12


def test_tiny_layer_statistics(orc):
    """Empirical firing frequencies follow p_i; the predictor sees ~95% of the
    true activations; the neuron table is the hotness order."""
    L = wl.config_layer("tiny_f32")
    x = wl.make_tokens(L.shape.d, 3000, 424242)
    _, tm = orc.true_mask(L.w_up, x, b1=L.b1)
    freq = tm.mean(axis=0)
    assert abs(freq.mean() - L.shape.rho) < 0.01
    # per-neuron binomial check (6 sigma, plus a small slack for fp rounding of b)
    sd = np.sqrt(L.p * (1 - L.p) / x.shape[0])
    assert np.all(np.abs(freq - L.p) < 6 * sd + 0.01)
    _, _, act = orc.predict(L.p1, L.c1, L.p2, L.c2, x)
    tp = (act & tm).sum()
    recall = tp / tm.sum()
    precision = tp / act.sum()
    assert 0.93 < recall < 0.97, recall
    assert precision > 0.9, precision
    # hot-first table: stored slots in order of decreasing firing probability
    assert np.all(np.diff(L.p[L.perm]) <= 0)


def test_union_closed_form(orc):
    """E|U|/f = mean_i[1 - (1 - p_i)^B] for independent tokens (checked on a
    scaled-down layer with the batched workload's firing law)."""
    _, sh = wl.CONFIGS["opt13b_batched"]
    L = wl.make_layer(wl.scaled_shape(sh, 128, 2048, 64), 5)
    B, nb = 16, 40
    x = wl.make_tokens(128, B * nb, 77)
    _, tm = orc.true_mask(L.w_up, x, b1=L.b1)
    fr = np.mean([orc.union(tm[i * B:(i + 1) * B]).mean() for i in range(nb)])
    expect = np.mean(1 - (1 - L.p) ** B)
    assert abs(fr - expect) < 0.02, (fr, expect)
    fr1 = tm.mean()
    assert abs(fr1 - sh.rho) < 0.01


def test_generator_is_deterministic():
    a = wl.make_layer(wl.LayerShape(64, 256, 32, 0.1, "f16"), 9)
    b = wl.make_layer(wl.LayerShape(64, 256, 32, 0.1, "f16"), 9)
    for k in ("w_up", "w_down", "b1", "b2", "p1", "p2", "c2", "perm"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    assert a.w_up.dtype == np.float16 and a.b1.dtype == np.float32


def test_relu_second_moment_closed_form():
    """E[ReLU(z)^2], z ~ N(mu, s^2), against Monte Carlo and two exact cases
    (mu = 0 gives s^2/2; mu >> s gives mu^2 + s^2)."""
    from workload.gpu import relu_second_moment
    rng = np.random.Generator(np.random.PCG64(3))
    mu = np.array([-2.0, -0.5, 0.0, 0.7, 1.5])
    s = np.array([1.0, 0.3, 2.0, 1.2, 0.5])
    z = rng.standard_normal((400000, 1)) * s + mu
    mc = (np.maximum(z, 0.0) ** 2).mean(axis=0)
    cf = relu_second_moment(mu, s)
    assert np.all(np.abs(mc - cf) < 0.01 * (cf + 0.01)), (mc, cf)
    assert abs(relu_second_moment(np.array([0.0]), np.array([3.0]))[0] - 4.5) < 1e-12
    assert abs(relu_second_moment(np.array([40.0]), np.array([1.0]))[0] - 1601.0) < 1e-9


def test_stack_generator_keeps_layer_inputs_calibrated(orc):
    """Stack layers drawn by the device generator (here on the CPU device):
    each layer fires at its rho on N(0,1) inputs, and chaining
    x_{l+1} = FFN_l(x_l) over the predicted sets keeps the next layer's input
    near unit RMS, so deeper layers still fire at their own rho."""
    import torch
    from workload.gpu import make_layer_device
    d, f = 256, 2048
    rhos, Hs = [0.03, 0.09, 0.15], [64, 128, 256]
    x = wl.make_tokens(d, 64, 99).astype(np.float64)
    for l, (rho, H) in enumerate(zip(rhos, Hs)):
        sh = wl.LayerShape(d, f, H, rho, "f16")
        DL = make_layer_device(sh, 500 + l, torch.device("cpu"))
        L = DL.to_numpy()
        assert L.w_up.dtype == np.float16 and L.w_down.shape == (d, f)
        assert np.all(np.diff(L.p[L.perm]) <= 0)
        xin = x.astype(np.float32)
        rms_in = np.sqrt((xin.astype(np.float64) ** 2).mean())
        assert 0.8 < rms_in < 1.2, (l, rms_in)
        _, tm = orc.true_mask(L.w_up, xin, b1=L.b1)
        assert abs(tm.mean() - rho) < 0.35 * rho + 0.005, (l, tm.mean(), rho)
        _, _, act = orc.predict(L.p1, L.c1, L.p2, L.c2, xin)
        ys = []
        for t in range(xin.shape[0]):
            ids = orc.active_list(act[t], L.perm)
            ys.append(orc.ffn(L.w_up, L.w_down, xin[t:t + 1], ids, b1=L.b1, b2=L.b2)[0])
        x = np.asarray(ys)
    assert 0.75 < np.sqrt((x ** 2).mean()) < 1.2


def test_sampled_sets_follow_the_law():
    """Sets drawn at mean activation rho have mean size rho*f, and the hottest
    slots of the table fire most often."""
    f = 4096
    perm = np.random.Generator(np.random.PCG64(5)).permutation(f).astype(np.int32)
    sets = wl.sampled_sets(perm, 0.10, 400, seed=11)
    sizes = np.array([len(s) for s in sets])
    assert abs(sizes.mean() / f - 0.10) < 0.004
    cnt = np.zeros(f)
    for s in sets:
        assert np.all(np.diff(s) > 0)
        cnt[s] += 1
    assert cnt[perm[:32]].mean() > 300 and cnt[perm[-1024:]].mean() < 20


def test_head_predictor_workload():
    """The head predictor generator selects about its configured fraction of
    heads per token, head by head near its selection probability (the
    recipe's moment matching of the logits)."""
    import oracle
    oracle.build()
    for name in ("opt30b_heads", "heads256"):
        P = wl.head_config(name)
        x = wl.head_config_tokens(name, 96)
        _, act, _ = oracle.predict_heads(P.q1, P.c1, P.q2, P.c2, x)
        assert abs(act.mean() - P.shape.frac) < 0.03, (name, act.mean())
        assert np.corrcoef(act.mean(axis=0), P.p)[0, 1] > 0.9
