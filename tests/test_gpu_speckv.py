"""GPU parity of the draft statistics and adaptive-gamma controller (qspec_speckv_gamma) against
the oracle: confidence and entropy within the fp64 summation-order bound, gamma exact wherever the
controller's two largest outputs are not within rounding of each other."""
import numpy as np
import pytest
import torch

import oracle
import quantized_speculative_decoding_amd as q
import synthetic_inputs as si
from gpu_helpers import DEV, cu, note

pytestmark = pytest.mark.gpu


def _weights(seed, G1):
    r = si.rng(seed)
    return (r.standard_normal((64, 3)).astype(np.float32), (r.standard_normal(64) * 0.1).astype(np.float32),
            (r.standard_normal((G1, 64)) * 0.3).astype(np.float32), (r.standard_normal(G1) * 0.1).astype(np.float32))


def run_speckv(logits, qf, w1, b1, w2, b2):
    R, V = logits.shape
    gamma = torch.full((R,), -7, dtype=torch.int32, device=DEV)
    feats = torch.full((R, 2), np.nan, dtype=torch.float64, device=DEV)
    ws = torch.empty((q.qspec_speckv_workspace_bytes(R, V),), dtype=torch.uint8, device=DEV)
    q.qspec_speckv_gamma(cu(logits), qf, cu(w1), cu(b1), cu(w2), cu(b2), gamma, feats, ws)
    return gamma.cpu().numpy(), feats.cpu().numpy()


def compare(logits, qf, w):
    R, V = logits.shape
    g, f = run_speckv(logits, qf, *w)
    og, of, mlp = oracle.speckv_gamma(logits, qf, *w)
    tol = max(1e-12, 5e-16 * V)                  # two fp64 sums over V terms in different orders
    assert np.allclose(f[:, 0], of[:, 0], rtol=tol, atol=0)
    assert np.allclose(f[:, 1], of[:, 1], rtol=tol, atol=1e-15)
    top2 = np.sort(mlp, axis=1)[:, -2:] if mlp.shape[1] > 1 else np.concatenate([mlp - 1, mlp], axis=1)
    clear = (top2[:, 1] - top2[:, 0]) > 1e-9 * np.maximum(1.0, np.abs(top2[:, 1]))
    assert np.array_equal(g[clear], og[clear]), (g, og)
    assert np.all((g >= 0) & (g < w[2].shape[0]))
    return g, f


@pytest.mark.parametrize("R,V,max_gamma", [(16, 128256, 8), (3, 1000, 8), (5, 8193, 16), (1, 1, 0), (2, 77, 63)])
def test_speckv_matches_oracle(R, V, max_gamma):
    note(f"speckv_gamma R={R} V={V} max_gamma={max_gamma}")
    t, _ = si.logits(R, 0, V, seed=V + R)
    logits = t.reshape(R, V)
    compare(logits, 1.0, _weights(V, max_gamma + 1))


def test_speckv_special_rows():
    note("speckv_gamma special rows")
    V = 20000
    logits = np.zeros((4, V), np.float32)            # row 0 uniform
    logits[1, :] = -1e30                             # row 1 one-hot
    logits[1, 12345] = 1.0
    logits[2, [3, 19999]] = 5.0                      # row 2: two equal maxima in different chunks
    logits[3] = si.logits(1, 0, V, seed=3)[0].reshape(V) * 10.0   # row 3: very peaked
    g, f = compare(logits, 0.0, _weights(7, 9))
    assert f[0, 0] == pytest.approx(1.0 / V, rel=1e-12)
    assert f[1, 0] == 1.0 and abs(f[1, 1]) < 1e-8


def test_speckv_gamma_follows_the_controller_weights():
    """A hand-built controller (output j = j * (entropy - 1)) picks max_gamma for flat rows and 0
    for peaked ones on the GPU too."""
    note("speckv_gamma hand-built controller")
    G1, V = 9, 4096
    w1 = np.zeros((64, 3), np.float32)
    w1[0, 1] = 1.0
    b1 = np.zeros(64, np.float32)
    w2 = np.zeros((G1, 64), np.float32)
    w2[:, 0] = np.arange(G1, dtype=np.float32)
    b2 = -np.arange(G1, dtype=np.float32)
    logits = np.zeros((2, V), np.float32)
    logits[0, 5] = 40.0
    g, _ = run_speckv(logits, 0.0, w1, b1, w2, b2)
    assert g.tolist() == [0, G1 - 1]


@pytest.mark.parametrize("mode", [q.QSPEC_GREEDY, q.QSPEC_SAMPLE], ids=["greedy", "sample"])
@pytest.mark.parametrize("B,V,gamma_buf", [(16, 128256, 4), (3, 1000, 1), (5, 8193, 2)])
def test_draft_sample_speckv_equals_the_two_calls(mode, B, V, gamma_buf):
    """One draft step of a [B][gamma][V] draft-logit buffer read in place (strided rows) and its
    tokens written into column j of the [B][gamma] token buffer: the shared-statistics call gives
    exactly qspec_draft_sample's tokens and qspec_speckv_gamma's gamma and features, and those
    match the oracle (tokens through the verification oracle with gamma = 0)."""
    note(f"draft_sample_speckv mode={mode} B={B} V={V}")
    t, _ = si.logits(B, gamma_buf - 1, V, seed=V + 7 * B)
    buf = cu(np.ascontiguousarray(t))                     # [B][gamma_buf][V]
    j = gamma_buf - 1
    rows = buf[:, j, :]
    u = cu(si.uniforms((B,), seed=B + 3))
    w = _weights(V + 1, 9)
    wd = [cu(a) for a in w]
    tok_buf = torch.full((B, gamma_buf), -5, dtype=torch.int32, device=DEV)
    gam = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    feats = torch.full((B, 2), np.nan, dtype=torch.float64, device=DEV)
    ws = torch.full((q.qspec_draft_sample_speckv_workspace_bytes(mode, B, V),), 0xFF, dtype=torch.uint8, device=DEV)
    uu = u if mode == q.QSPEC_SAMPLE else None
    q.qspec_draft_sample_speckv(mode, rows, tok_buf[:, j], uu, 0.5, *wd, gam, feats, ws)
    # the two separate calls
    tok2 = torch.full((B, gamma_buf), -5, dtype=torch.int32, device=DEV)
    ws1 = torch.empty((q.qspec_draft_sample_workspace_bytes(mode, B, V),), dtype=torch.uint8, device=DEV)
    q.qspec_draft_sample(mode, rows, tok2[:, j], uu, ws1)
    gam2 = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    feats2 = torch.full((B, 2), np.nan, dtype=torch.float64, device=DEV)
    ws2 = torch.empty((q.qspec_speckv_workspace_bytes(B, V),), dtype=torch.uint8, device=DEV)
    q.qspec_speckv_gamma(rows.contiguous(), 0.5, *wd, gam2, feats2, ws2)
    assert torch.equal(tok_buf, tok2)
    assert torch.equal(gam, gam2)
    assert torch.equal(feats, feats2)
    assert bool((tok_buf[:, :j] == -5).all())               # other columns untouched
    # the oracle: the controller on the rows, the head as the verification with gamma = 0
    logits = np.ascontiguousarray(t[:, j, :])
    compare(logits, 0.5, w)
    if mode == q.QSPEC_GREEDY:
        ref = np.argmax(logits, axis=1)
        assert np.array_equal(tok_buf[:, j].cpu().numpy(), ref)
    else:
        A, out, diag = oracle.verify_sample(logits.reshape(B, 1, V), np.zeros((B, 0, V), np.float32),
                                            np.zeros((B, 0), np.int32), np.zeros((B, 0), np.float32),
                                            si.uniforms((B,), seed=B + 3))
        got = tok_buf[:, j].cpu().numpy()
        for b in range(B):          # a draw may differ only where the oracle flags a CDF near tie
            assert got[b] == out[b, 0] or diag[b, 0] < 1e-9, (b, got[b], out[b, 0], diag[b, 0])
