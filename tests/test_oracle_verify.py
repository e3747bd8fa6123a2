"""Pins for the oracle's verification step (greedy and speculative sampling).

QSPEC notes, speculative-decoding background: acceptance probability
min(1, p/q); greedy acceptance when the target's top-1 equals the draft; the
first rejection ends the round; L = A + 1; E[A] and E[L] closed forms.  The
sampling pins are statistical (closed forms, chi-square against the target
distribution) plus exact special cases; the greedy pins use numpy's argmax.
"""
import json
import os

import numpy as np
import pytest
from scipy import stats

import oracle
import synthetic_inputs as si

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


# ---------------------------------------------------------------- greedy

@pytest.mark.parametrize("B,gamma,V", [(6, 4, 50), (3, 1, 7), (4, 0, 9), (5, 8, 1024)])
def test_greedy_invariants(B, gamma, V):
    t, d = si.logits(B, gamma, V, seed=B + gamma)
    toks = si.draft_tokens_greedy(d)
    acc, out = oracle.verify_greedy(t, toks)
    tops = np.argmax(t, axis=-1)
    for b in range(B):
        A = acc[b]
        assert 0 <= A <= gamma
        assert np.array_equal(out[b, :A], toks[b, :A])
        assert np.array_equal(out[b, :A + 1], tops[b, :A + 1])   # committed == target's greedy choices
        if A < gamma:
            assert toks[b, A] != tops[b, A]
        assert np.all(out[b, A + 1:] == -1)


def test_greedy_all_match_and_first_mismatch():
    B, gamma, V = 2, 5, 40
    t, _ = si.logits(B, gamma, V, seed=1)
    tops = np.argmax(t, axis=-1).astype(np.int32)
    acc, out = oracle.verify_greedy(t, tops[:, :gamma])
    assert np.all(acc == gamma) and np.array_equal(out, tops)
    bad = tops[:, :gamma].copy()
    bad[:, 0] = (bad[:, 0] + 1) % V
    acc, out = oracle.verify_greedy(t, bad)
    assert np.all(acc == 0) and np.array_equal(out[:, 0], tops[:, 0])
    oob = tops[:, :gamma].copy()
    oob[0, 2] = V
    oob[1, 1] = -3
    acc, _ = oracle.verify_greedy(t, oob)
    assert acc.tolist() == [2, 1]


def test_greedy_ties_take_lowest_index():
    V = 12
    t = np.zeros((1, 2, V), np.float32)
    t[0, 0, [3, 7, 9]] = 5.0
    t[0, 1, [1, 11]] = 2.0
    acc, out = oracle.verify_greedy(t, np.array([[3]], np.int32))
    assert acc[0] == 1 and out[0].tolist() == [3, 1]
    acc, out = oracle.verify_greedy(t, np.array([[7]], np.int32))
    assert acc[0] == 0 and out[0].tolist() == [3, -1]
    assert np.argmax(t[0, 0]) == 3


# ---------------------------------------------------------------- sampling

def _known_alpha_pair(V, alpha, seed):
    """p = alpha r + (1-alpha) a, q = alpha r + (1-alpha) b, a and b on disjoint supports,
    so sum_x min(p, q) = alpha exactly."""
    r = si.rng(seed)
    base = r.dirichlet(np.ones(V))
    half = V // 2
    a = np.zeros(V)
    a[:half] = r.dirichlet(np.ones(half))
    b = np.zeros(V)
    b[half:] = r.dirichlet(np.ones(V - half))
    p = alpha * base + (1 - alpha) * a
    q = alpha * base + (1 - alpha) * b
    return p, q


def _run_iid(p, q, B, gamma, seed):
    V = len(p)
    t = np.broadcast_to(np.log(p).astype(np.float32), (B, gamma + 1, V)).copy()
    d = np.broadcast_to(np.log(q).astype(np.float32), (B, gamma, V)).copy()
    toks = si.draft_tokens_sampled(d, seed)
    u = si.uniforms((B, gamma), seed)
    v = si.uniforms((B,), seed + 1000)
    return oracle.verify_sample(t, d, toks, u, v)


@pytest.mark.parametrize("case", GOLDEN["expected_committed_tokens"]["cases"],
                         ids=lambda c: "a%.1f_K%d" % (c["alpha"], c["K"]))
def test_sampling_mean_committed_tokens_closed_form(case):
    alpha, gamma = case["alpha"], case["K"]
    closed = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert abs(closed - case["E_L"]) < 1e-4            # the printed closed form vs the hand sum
    p, q = _known_alpha_pair(16, alpha, seed=int(alpha * 10))
    B = 40000
    acc, out, _ = _run_iid(p, q, B, gamma, seed=int(alpha * 100) + gamma)
    L = acc.astype(np.float64) + 1
    se = L.std() / np.sqrt(B)
    assert abs(L.mean() - closed) < 4.5 * se, (L.mean(), closed, se)
    # E[A] closed form from the same page
    ea = alpha * (1 - alpha ** gamma) / (1 - alpha)
    assert abs(acc.mean() - ea) < 4.5 * se


def test_sampling_accept_count_distribution_is_truncated_geometric():
    alpha, gamma, B = 0.7, 4, 40000
    p, q = _known_alpha_pair(12, alpha, seed=4)
    acc, _, _ = _run_iid(p, q, B, gamma, seed=77)
    expect = np.array([alpha ** a * (1 - alpha) for a in range(gamma)] + [alpha ** gamma])
    counts = np.bincount(acc, minlength=gamma + 1)
    chi = stats.chisquare(counts, expect * B)
    assert chi.pvalue > 1e-4, (counts, expect * B)


def test_sampling_committed_tokens_follow_target_distribution():
    alpha, gamma, B, V = 0.6, 3, 60000, 10
    p, q = _known_alpha_pair(V, alpha, seed=5)
    acc, out, _ = _run_iid(p, q, B, gamma, seed=91)
    # first committed token: always present
    c0 = np.bincount(out[:, 0], minlength=V)
    assert stats.chisquare(c0, p * B).pvalue > 1e-4
    # second committed token: present when A >= 1; its conditional law is p again
    sel = out[acc >= 1, 1]
    c1 = np.bincount(sel, minlength=V)
    assert stats.chisquare(c1, p * len(sel)).pvalue > 1e-4
    # the correction token alone is *not* distributed as p (it follows the residual)
    rej = out[acc == 0, 0]
    resid = np.maximum(p - q, 0)
    resid /= resid.sum()
    cr = np.bincount(rej, minlength=V)
    sup = resid > 0
    assert np.all(cr[~sup] == 0)
    assert stats.chisquare(cr[sup], resid[sup] * len(rej)).pvalue > 1e-4


def test_sampling_identical_distributions_accept_everything():
    B, gamma, V = 64, 4, 33
    t, _ = si.logits(B, gamma, V, seed=8)
    d = t[:, :gamma, :].copy()
    toks = si.draft_tokens_sampled(d, 8)
    u = si.uniforms((B, gamma), 8)
    v = si.uniforms((B,), 9)
    acc, out, _ = oracle.verify_sample(t, d, toks, u, v)
    assert np.all(acc == gamma)
    assert np.array_equal(out[:, :gamma], toks)


def test_sampling_disjoint_supports_reject_first_and_draw_from_target():
    B, gamma, V = 4000, 3, 8
    p0 = np.array([0.1, 0.2, 0.3, 0.4, 0, 0, 0, 0])
    t = np.full((B, gamma + 1, V), -1e30, np.float32)
    t[:, :, :4] = np.log(p0[:4]).astype(np.float32)
    d = np.full((B, gamma, V), -1e30, np.float32)
    d[:, :, 4:] = 0.0
    toks = si.draft_tokens_sampled(d, 3)
    assert np.all(toks >= 4)
    acc, out, _ = oracle.verify_sample(t, d, toks, si.uniforms((B, gamma), 3), si.uniforms((B,), 4))
    assert np.all(acc == 0)
    c = np.bincount(out[:, 0], minlength=V)
    assert np.all(c[4:] == 0)
    assert stats.chisquare(c[:4], p0[:4] * B).pvalue > 1e-4


def test_sampling_zero_mass_residual_falls_back_to_target_row():
    """After a rejection the correction token is drawn from the target's distribution (the
    residual max(0, p - q) normalised; p itself when that residual has no mass).  With q == p at
    every position the residual is exactly zero wherever a rejection happens, and a rejection is
    forced at position j by an out-of-range draft token, so the token at j must follow p_j.
    The target rows differ from one another, so a draw from another row, a uniform draw, or no
    draw at all fails; drawing from q_j instead of p_j is the same distribution here, since a zero
    residual means q_j = p_j up to rounding."""
    B, gamma, V, j = 30000, 4, 8, 2
    rows = np.array([[0.30, 0.05, 0.05, 0.20, 0.10, 0.10, 0.15, 0.05],
                     [0.02, 0.40, 0.08, 0.10, 0.10, 0.05, 0.05, 0.20],
                     [0.05, 0.05, 0.50, 0.02, 0.03, 0.15, 0.10, 0.10],
                     [0.25, 0.25, 0.02, 0.03, 0.15, 0.10, 0.10, 0.10],
                     [0.10, 0.10, 0.10, 0.40, 0.05, 0.05, 0.10, 0.10]])
    t = np.broadcast_to(np.log(rows).astype(np.float32), (B, gamma + 1, V)).copy()
    d = t[:, :gamma, :].copy()                       # q_i == p_i bit for bit
    toks = si.draft_tokens_sampled(d, 21)
    toks[:, j] = V                                   # out of range: rejected
    acc, out, diag = oracle.verify_sample(t, d, toks, si.uniforms((B, gamma), 21), si.uniforms((B,), 22))
    assert np.all(acc == j)                          # p/q == 1 > u before j
    assert np.array_equal(out[:, :j], toks[:, :j]) and np.all(out[:, j + 1:] == -1)
    counts = np.bincount(out[:, j], minlength=V)
    assert counts.sum() == B
    assert stats.chisquare(counts, rows[j] * B).pvalue > 1e-4
    for other in [rows[j - 1], rows[j + 1], np.full(V, 1.0 / V)]:
        assert stats.chisquare(counts, other * B).pvalue < 1e-12


def test_sampling_with_one_hot_distributions_equals_greedy():
    B, gamma, V = 50, 4, 64
    r = si.rng(12)
    t = np.stack([np.stack([r.permutation(V) for _ in range(gamma + 1)]) for _ in range(B)])
    t = (t * 1000.0).astype(np.float32)            # gaps >= 1000: softmax is exactly one-hot in fp64
    d = t[:, :gamma, :].copy()
    # make some drafts disagree with the target
    for b in range(0, B, 3):
        j = b % gamma
        d[b, j] = np.roll(d[b, j], 1)
    toks = si.draft_tokens_greedy(d)
    acc_s, out_s, _ = oracle.verify_sample(t, d, toks, si.uniforms((B, gamma), 12), si.uniforms((B,), 13))
    acc_g, out_g = oracle.verify_greedy(t, toks)
    assert np.array_equal(acc_s, acc_g) and np.array_equal(out_s, out_g)
    assert acc_g.min() < gamma and acc_g.max() == gamma


def test_sampling_gamma_zero_is_a_plain_draw_from_target():
    B, V = 20000, 6
    p = np.array([0.05, 0.15, 0.3, 0.2, 0.1, 0.2])
    t = np.broadcast_to(np.log(p).astype(np.float32), (B, 1, V)).copy()
    d = np.zeros((B, 0, V), np.float32)
    acc, out, _ = oracle.verify_sample(t, d, np.zeros((B, 0), np.int32), np.zeros((B, 0), np.float32),
                                       si.uniforms((B,), 5))
    assert np.all(acc == 0)
    assert stats.chisquare(np.bincount(out[:, 0], minlength=V), p * B).pvalue > 1e-4


def test_sampling_inverse_cdf_boundaries():
    # p = (0.25, 0.25, 0.5): thresholds v*1 land in [0,.25) -> 0, [.25,.5) -> 1, [.5,1) -> 2
    V = 3
    t = np.log(np.array([[[0.25, 0.25, 0.5]]])).astype(np.float32)
    for v, tok in [(0.0, 0), (0.2, 0), (0.3, 1), (0.49, 1), (0.51, 2), (0.999, 2)]:
        _, out, _ = oracle.verify_sample(t, np.zeros((1, 0, V), np.float32), np.zeros((1, 0), np.int32),
                                         np.zeros((1, 0), np.float32), np.array([v], np.float32))
        assert out[0, 0] == tok, (v, out)
