"""GPU parity of the draft-side head (qspec_draft_sample) against the oracle's verification with
gamma = 0, reading each step's rows in place from a [B][gamma][V] draft-logit buffer and writing
each step's tokens into column j of the [B][gamma] draft-token buffer; then the verification of
the tokens the head produced.  Greedy tokens are exact; sampled tokens are exact except draws the
oracle flags as near ties of the inverse CDF (below 1e-9 relative), which must stay rare."""
import numpy as np
import pytest
import torch

import oracle
import quantized_speculative_decoding_amd as q
import synthetic_inputs as si
from gpu_helpers import DEV, cu, note

pytestmark = pytest.mark.gpu

NEAR_TIE = 1e-9


def heads(mode, d, us):
    """Run the head for every step j over the draft logits d [B][gamma][V] (in place, strided)."""
    B, gamma, V = d.shape
    dd = cu(d)
    toks = torch.full((B, gamma), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty((q.qspec_draft_sample_workspace_bytes(mode, B, V),), dtype=torch.uint8, device=DEV)
    for j in range(gamma):
        q.qspec_draft_sample(mode, dd[:, j, :], toks[:, j], cu(us[:, j].copy()) if us is not None else None, ws)
        # columns after j are untouched so far
        assert torch.all(toks[:, j + 1:] == -7)
    return toks.cpu().numpy()


@pytest.mark.parametrize("B,gamma,V", [(16, 4, 128256), (3, 2, 1000), (5, 1, 77), (4, 3, 8193)])
def test_greedy_head_matches_oracle(B, gamma, V):
    note(f"draft_sample greedy B={B} gamma={gamma} V={V}")
    _, d = si.logits(B, gamma, V, seed=B + V)
    toks = heads(q.QSPEC_GREEDY, d, None)
    for j in range(gamma):
        _, oo = oracle.verify_greedy(d[:, j:j + 1, :], np.zeros((B, 0), np.int32))
        assert np.array_equal(toks[:, j], oo[:, 0])
    assert np.array_equal(toks, si.draft_tokens_greedy(d))          # numpy's argmax, lowest index


@pytest.mark.parametrize("B,gamma,V", [(16, 4, 128256), (3, 2, 1000), (5, 1, 77), (4, 3, 8193)])
def test_sampling_head_then_verification(B, gamma, V):
    note(f"draft_sample sample B={B} gamma={gamma} V={V}")
    t, d = si.logits(B, gamma, V, seed=3 * B + V)
    us = si.uniforms((B, gamma), seed=B + 7)
    toks = heads(q.QSPEC_SAMPLE, d, us)
    excused = 0
    for j in range(gamma):
        _, oo, diag = oracle.verify_sample(d[:, j:j + 1, :], np.zeros((B, 0, V), np.float32),
                                           np.zeros((B, 0), np.int32), np.zeros((B, 0), np.float32),
                                           us[:, j].copy())
        for b in range(B):
            if toks[b, j] != oo[b, 0]:
                assert diag[b, 0] < NEAR_TIE, (b, j, toks[b, j], oo[b, 0], diag[b, 0])
                excused += 1
    assert excused <= max(1, B * gamma // 100)
    assert np.all((toks >= 0) & (toks < V))
    # the verification then reads the head's tokens from the same buffer
    acc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    out = torch.full((B, gamma + 1), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty((q.qspec_verify_workspace_bytes(q.QSPEC_SAMPLE, B, gamma, V),), dtype=torch.uint8, device=DEV)
    u = si.uniforms((B, gamma), seed=B + 8)
    v = si.uniforms((B,), seed=B + 9)
    q.qspec_verify_accept(q.QSPEC_SAMPLE, cu(t), cu(d), cu(toks), cu(u), cu(v), acc, out, ws)
    oa, oo, diag = oracle.verify_sample(t, d, toks, u, v)
    a, o = acc.cpu().numpy(), out.cpu().numpy()
    for b in range(B):
        if a[b] != oa[b]:
            assert any(diag[b, j] < NEAR_TIE for j in range(min(a[b], oa[b]) + 1) if j < gamma)
            continue
        assert np.array_equal(o[b, :a[b]], toks[b, :a[b]])
        if o[b, a[b]] != oo[b, oa[b]]:
            assert diag[b, gamma] < NEAR_TIE


def test_head_distribution_matches_softmax():
    """Draws from one fixed row follow softmax(row) (chi-square over 4000 uniforms)."""
    from scipy import stats
    note("draft_sample distribution")
    V, B = 12, 4000
    row = np.linspace(-1.0, 1.5, V).astype(np.float32)
    d = np.broadcast_to(row, (B, 1, V)).copy()
    us = si.uniforms((B, 1), seed=77)
    toks = heads(q.QSPEC_SAMPLE, d, us)[:, 0]
    p = np.exp(row.astype(np.float64) - row.max())
    p /= p.sum()
    counts = np.bincount(toks, minlength=V)
    assert stats.chisquare(counts, p * B).pvalue > 1e-4
