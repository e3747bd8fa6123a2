"""GPU parity of the verification step against the CPU oracle, through the C ABI.

Greedy: accept counts and committed tokens bit-exact (argmax over fp32 logits is exact).
Sampling: accept counts and tokens exact, except decisions the oracle flags as near ties
(|u - p/q| or the CDF distance of the draw below 1e-9 relative, where fp64 rounding order may
decide); such excused cases are counted and must stay rare.  Statistical checks of the closed
forms run through the GPU kernels as well."""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import quantized_speculative_decoding_amd as q
import synthetic_inputs as si
from gpu_helpers import DEV, Guarded, cu, note

pytestmark = pytest.mark.gpu

NEAR_TIE = 1e-9


def run_verify(mode, t, d, toks, u, v):
    B, g1, V = t.shape
    gamma = g1 - 1
    acc = Guarded((B,), torch.int32, fill=-7)
    out = Guarded((B, g1), torch.int32, fill=-7)
    ws = Guarded((q.qspec_verify_workspace_bytes(mode, B, gamma, V),), torch.uint8)
    q.qspec_verify_accept(mode, cu(t), cu(d) if mode == q.QSPEC_SAMPLE else None,
                          cu(toks) if gamma > 0 else None,
                          cu(u) if mode == q.QSPEC_SAMPLE else None,
                          cu(v) if mode == q.QSPEC_SAMPLE else None, acc.t, out.t, ws.t)
    acc.check("verify_accept accept_count")
    out.check("verify_accept out_tokens")
    ws.check("verify_accept workspace")
    return acc.t.cpu().numpy(), out.t.cpu().numpy()


# gamma = 0 is the draft-side sampling head: one token per row from softmax(row) (or its argmax).
# (2, 2, 600000): more residual chunks than a workgroup has threads (one thread walks them);
# (2, 0, 2200000): the same for the gamma = 0 draw's chunk statistics
SHAPES = [(1, 4, 1024), (3, 2, 100), (5, 0, 77), (4, 8, 50001), (2, 16, 8191), (7, 3, 8193),
          (32, 4, 128256), (16, 0, 128256), (2, 2, 600000), (2, 0, 2200000)]


@pytest.mark.parametrize("B,gamma,V", SHAPES)
def test_greedy_exact(B, gamma, V):
    note(f"verify_accept greedy B={B} gamma={gamma} V={V}")
    t, d = si.logits(B, gamma, V, seed=B * 31 + V)
    toks = si.draft_tokens_greedy(d)
    acc, out = run_verify(q.QSPEC_GREEDY, t, d, toks, None, None)
    oa, oo = oracle.verify_greedy(t, toks)
    assert np.array_equal(acc, oa) and np.array_equal(out, oo)


def test_greedy_ties_across_chunks_and_invalid_tokens():
    note("verify_accept greedy ties")
    B, gamma, V = 4, 3, 30000
    t, d = si.logits(B, gamma, V, seed=5)
    t[:, :, [9000, 17000, 25000]] = 50.0           # equal maxima in different chunks
    t[0, 1, 5] = 50.0                              # ...and in the first chunk for one row
    toks = np.array([[9000, 5, 9000], [9000, 9000, 9000], [V + 3, 9000, 9000], [-1, 0, 0]], np.int32)
    acc, out = run_verify(q.QSPEC_GREEDY, t, d, toks, None, None)
    oa, oo = oracle.verify_greedy(t, toks)
    assert np.array_equal(acc, oa) and np.array_equal(out, oo)
    assert acc.tolist() == [3, 3, 0, 0]          # row 0 matches at 9000, 5 (lowest tie), 9000


def test_greedy_wide_chunks_ties():
    """1024 target rows of 16400 logits take the 16384-logit argmax chunks: ties across that
    boundary resolve to the lowest index, and the 16-logit ragged chunk is searched too."""
    B, gamma, V = 256, 3, 16400
    note(f"verify_accept greedy wide chunks B={B} gamma={gamma} V={V}")
    t, d = si.logits(B, gamma, V, seed=77)
    top = np.float32(100.0)
    t[0, :, 100] = top
    t[0, :, 16390] = top                          # tie across the chunk boundary: 100 wins
    t[1, :, 16399] = top                          # maximum in the ragged chunk
    t[2, :, 16383] = top
    t[2, :, 16384] = top                          # adjacent tie on the boundary: 16383 wins
    toks = si.draft_tokens_greedy(d)
    toks[0, :] = 100
    toks[1, :] = 16399
    toks[2, :] = 16383
    acc, out = run_verify(q.QSPEC_GREEDY, t, d, toks, None, None)
    oa, oo = oracle.verify_greedy(t, toks)
    assert np.array_equal(acc, oa) and np.array_equal(out, oo)
    assert acc[:3].tolist() == [gamma, gamma, gamma]
    assert out[0, gamma] == 100 and out[1, gamma] == 16399 and out[2, gamma] == 16383


def _compare_sampling(t, d, toks, u, v):
    acc, out = run_verify(q.QSPEC_SAMPLE, t, d, toks, u, v)
    oa, oo, diag = oracle.verify_sample(t, d, toks, u, v)
    B, g1 = oo.shape
    gamma = g1 - 1
    excused = 0
    for b in range(B):
        near = [j for j in range(min(acc[b], oa[b]) + 1) if j < gamma and diag[b, j] < NEAR_TIE]
        if acc[b] != oa[b]:
            assert near, (b, acc[b], oa[b], diag[b])
            excused += 1
            continue
        assert np.array_equal(out[b, :acc[b]], oo[b, :oa[b]])
        assert np.all(out[b, acc[b] + 1:] == -1)
        if out[b, acc[b]] != oo[b, oa[b]]:
            assert diag[b, gamma] < NEAR_TIE, (b, out[b], oo[b], diag[b])
            excused += 1
    return excused, acc, out


@pytest.mark.parametrize("B,gamma,V", SHAPES)
def test_sampling_matches_oracle(B, gamma, V):
    note(f"verify_accept sample B={B} gamma={gamma} V={V}")
    t, d = si.logits(B, gamma, V, seed=B * 17 + V)
    toks = si.draft_tokens_sampled(d, seed=B)
    u = si.uniforms((B, gamma), seed=B)
    v = si.uniforms((B,), seed=B + 1)
    excused, _, _ = _compare_sampling(t, d, toks, u, v)
    assert excused <= max(1, B // 100)


def test_sampling_special_cases():
    note("verify_accept sample special cases")
    B, gamma, V = 64, 4, 4099
    t, _ = si.logits(B, gamma, V, seed=9)
    d = t[:, :gamma, :].copy()                             # q == p: everything accepted
    toks = si.draft_tokens_sampled(d, seed=9)
    acc, out = run_verify(q.QSPEC_SAMPLE, t, d, toks, si.uniforms((B, gamma), 9), si.uniforms((B,), 10))
    assert np.all(acc == gamma) and np.array_equal(out[:, :gamma], toks)
    # disjoint supports: first candidate rejected, token from the target's support
    t2 = np.full((B, gamma + 1, V), -1e30, np.float32)
    t2[:, :, :100] = si.rng(1).standard_normal((B, gamma + 1, 100)).astype(np.float32)
    d2 = np.full((B, gamma, V), -1e30, np.float32)
    d2[:, :, 100:] = 0.0
    toks2 = si.draft_tokens_sampled(d2, seed=2)
    u2, v2 = si.uniforms((B, gamma), 3), si.uniforms((B,), 4)
    excused, acc, out = _compare_sampling(t2, d2, toks2, u2, v2)
    assert excused == 0 and np.all(acc == 0) and np.all(out[:, 0] < 100)
    # invalid draft tokens are rejections
    toks3 = toks.copy()
    toks3[:, 1] = V
    toks3[0, 0] = -5
    excused, acc, _ = _compare_sampling(t, d, toks3, si.uniforms((B, gamma), 9), si.uniforms((B,), 10))
    assert acc[0] == 0 and np.all(acc <= 1)


def test_sampling_closed_form_through_gpu():
    """E[L] = (1 - alpha^(K+1)) / (1 - alpha) and the committed-token law, on the GPU path."""
    note("verify_accept sample statistics")
    alpha, gamma, B, V = 0.75, 4, 40000, 16
    r = si.rng(77)
    base = r.dirichlet(np.ones(V))
    a = np.zeros(V); a[:8] = r.dirichlet(np.ones(8))
    bb = np.zeros(V); bb[8:] = r.dirichlet(np.ones(8))
    p = alpha * base + (1 - alpha) * a
    qd = alpha * base + (1 - alpha) * bb
    t = np.broadcast_to(np.log(p).astype(np.float32), (B, gamma + 1, V)).copy()
    d = np.broadcast_to(np.log(qd).astype(np.float32), (B, gamma, V)).copy()
    toks = si.draft_tokens_sampled(d, seed=78)
    acc, out = run_verify(q.QSPEC_SAMPLE, t, d, toks, si.uniforms((B, gamma), 79), si.uniforms((B,), 80))
    L = acc + 1.0
    closed = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert abs(L.mean() - closed) < 4.5 * L.std() / np.sqrt(B)
    assert stats.chisquare(np.bincount(out[:, 0], minlength=V), p * B).pvalue > 1e-4
    expect = np.array([alpha ** k * (1 - alpha) for k in range(gamma)] + [alpha ** gamma])
    assert stats.chisquare(np.bincount(acc, minlength=gamma + 1), expect * B).pvalue > 1e-4
