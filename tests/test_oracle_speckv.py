"""Pins of the oracle's draft statistics and adaptive-gamma controller (SpecKV notes: architecture
and mechanism, and the implementation guide's controller listing): confidence = largest softmax
probability, entropy = -sum p log(p + 1e-9), and the Linear(3 -> 64), ReLU,
Linear(64 -> max_gamma + 1), argmax controller.  Checked against closed forms and against torch's
own float64 softmax / linear layers, which the page's listing is written in."""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si


def _mlp_weights(seed, G1):
    r = si.rng(seed)
    return (r.standard_normal((64, 3)).astype(np.float32), r.standard_normal(64).astype(np.float32) * 0.1,
            r.standard_normal((G1, 64)).astype(np.float32) * 0.3, r.standard_normal(G1).astype(np.float32) * 0.1)


def _zero_mlp(G1):
    return (np.zeros((64, 3), np.float32), np.zeros(64, np.float32), np.zeros((G1, 64), np.float32),
            np.zeros(G1, np.float32))


@pytest.mark.parametrize("V", [1, 7, 1000, 128256])
def test_uniform_logits_closed_form(V):
    g, f, _ = oracle.speckv_gamma(np.full((2, V), 0.75, np.float32), 0.0, *_zero_mlp(9))
    assert f[0, 0] == pytest.approx(1.0 / V, rel=1e-14)
    # a sequential fp64 sum of V terms is within about V unit roundoffs of the exact value
    assert f[0, 1] == pytest.approx(-math.log(1.0 / V + 1e-9), rel=max(1e-14, 2.3e-16 * V), abs=1e-15)
    assert np.all(g == 0)                        # all-zero outputs: ties take the lowest index


def test_one_hot_distribution():
    V = 5000
    logits = np.full((3, V), -1e30, np.float32)
    logits[np.arange(3), [0, 17, V - 1]] = 2.0   # one finite logit: p is exactly one-hot
    _, f, _ = oracle.speckv_gamma(logits, 0.0, *_zero_mlp(3))
    assert np.all(f[:, 0] == 1.0)
    assert np.allclose(f[:, 1], -math.log(1.0 + 1e-9), rtol=1e-12, atol=0)


def test_two_level_distribution_closed_form():
    # k logits at +1 and V - k at 0: two probability levels, entropy in closed form
    V = 1000
    for k in (1, 10, 100, 999):
        logits = np.zeros((1, V), np.float32)
        logits[0, V - k:] = 1.0
        _, f, _ = oracle.speckv_gamma(logits, 0.0, *_zero_mlp(2))
        z = k * math.e + (V - k)
        p_hi, p_lo = math.e / z, 1.0 / z
        ent = -(k * p_hi * math.log(p_hi + 1e-9) + (V - k) * p_lo * math.log(p_lo + 1e-9))
        assert f[0, 0] == pytest.approx(p_hi, rel=1e-13)
        assert f[0, 1] == pytest.approx(ent, rel=2.3e-16 * V)
        assert 0.0 < f[0, 1] < math.log(V)


@pytest.mark.parametrize("R,V,G1", [(4, 1024, 9), (3, 30011, 9), (2, 128256, 17)])
def test_matches_torch_float64_softmax_and_linear_layers(R, V, G1):
    t, _ = si.logits(R, 0, V, seed=V)
    logits = t.reshape(R, V)
    qf = 1.0
    w1, b1, w2, b2 = _mlp_weights(V + G1, G1)
    g, f, mlp = oracle.speckv_gamma(logits, qf, w1, b1, w2, b2)
    L = torch.from_numpy(logits).double()
    p = torch.softmax(L, dim=-1)
    conf = p.max(dim=-1).values
    ent = -(p * torch.log(p + 1e-9)).sum(dim=-1)
    tol = max(1e-13, 2.3e-16 * V)                # both sums carry up to ~V roundoffs
    assert np.allclose(f[:, 0], conf.numpy(), rtol=tol, atol=0)
    assert np.allclose(f[:, 1], ent.numpy(), rtol=tol, atol=0)
    x = torch.stack([conf, ent, torch.full_like(conf, qf)], dim=-1)
    h = torch.relu(torch.nn.functional.linear(x, torch.from_numpy(w1).double(), torch.from_numpy(b1).double()))
    o = torch.nn.functional.linear(h, torch.from_numpy(w2).double(), torch.from_numpy(b2).double())
    assert np.allclose(mlp, o.numpy(), rtol=1e-10, atol=1e-10)
    top2 = np.sort(o.numpy(), axis=1)[:, -2:]
    clear = (top2[:, 1] - top2[:, 0]) > 1e-9
    assert np.array_equal(g[clear], o.argmax(dim=-1).numpy()[clear])


def test_controller_closed_form_threshold_on_entropy():
    """Hidden unit 0 carries the entropy, output j = j * (h0 - 1): gamma = max_gamma when the
    entropy exceeds 1, else 0 (at entropy <= 1 every output <= 0 and output 0 is exactly 0)."""
    G1 = 9
    w1, b1, w2, b2 = _zero_mlp(G1)
    w1[0, 1] = 1.0
    w2[:, 0] = np.arange(G1, dtype=np.float32)
    b2[:] = -np.arange(G1, dtype=np.float32)
    V = 64
    low = np.zeros((1, V), np.float32)
    low[0, 0] = 30.0                              # nearly one-hot: entropy ~ 0
    high = np.zeros((1, V), np.float32)           # uniform: entropy ~ log 64 = 4.16
    g, f, _ = oracle.speckv_gamma(np.concatenate([low, high]), 0.0, w1, b1, w2, b2)
    assert f[0, 1] < 1.0 < f[1, 1]
    assert g.tolist() == [0, G1 - 1]


def test_third_input_enters_the_first_layer():
    G1 = 3
    w1, b1, w2, b2 = _zero_mlp(G1)
    w1[5, 2] = 1.0                                # hidden unit 5 = relu(quant feature)
    w2[2, 5] = 1.0
    logits = np.zeros((1, 16), np.float32)
    assert oracle.speckv_gamma(logits, 1.0, w1, b1, w2, b2)[0][0] == 2
    assert oracle.speckv_gamma(logits, -1.0, w1, b1, w2, b2)[0][0] == 0   # relu cuts it: all outputs 0
