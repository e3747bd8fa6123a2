"""GPU parity of the KV replacement against the oracle (bit-exact), including the full
32-layer x 32-sequence x 8-head x 4096 x 128 cache driven by device-resident accept counts."""
import numpy as np
import pytest
import torch

import oracle
import quantized_speculative_decoding_amd as q
import synthetic_inputs as si
from gpu_helpers import DEV, Guarded, bf16_dev, cu, host_bits16, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("L,B,H,T,D,gamma", [(2, 3, 2, 32, 128, 4), (1, 5, 1, 16, 8, 2), (3, 2, 3, 10, 12, 0),
                                             (2, 4, 2, 40, 64, 16), (1, 2, 1, 9, 5, 3)])
def test_kv_overwrite_exact(L, B, H, T, D, gamma):
    note(f"kv_overwrite L={L} B={B} H={H} T={T} D={D} gamma={gamma}")
    cache = si.kv_canary(L, B, H, T, D).reshape(L, B, 2, H, T, D)
    stage = si.kv_staging(L, B, H, gamma, D, seed=L * B)
    start = si.start_positions(B, T, gamma, seed=B)
    start[0] = T - 2                                  # rows falling off the end are skipped
    acc = si.rng(B).integers(-1, gamma + 3, size=B).astype(np.int32)   # includes clamped values
    gc = Guarded(cache.shape, torch.bfloat16)
    gc.t.copy_(bf16_dev(cache))
    q.qspec_kv_overwrite(gc.t, bf16_dev(stage), cu(start), cu(acc))
    gc.check("kv_overwrite cache")
    ref = oracle.kv_overwrite(cache.copy(), stage, start, acc)
    assert np.array_equal(host_bits16(gc.t), ref)


def test_kv_overwrite_full_cache_from_verify_accept():
    L, B, H, T, D, gamma, V = 32, 32, 8, 4096, 128, 4, 128256
    note("kv_overwrite full cache after verify_accept sample")
    t, d = si.logits(B, gamma, V, seed=3)
    toks = si.draft_tokens_sampled(d, seed=3)
    acc = torch.empty((B,), dtype=torch.int32, device=DEV)
    out = torch.empty((B, gamma + 1), dtype=torch.int32, device=DEV)
    ws = torch.empty((q.qspec_verify_workspace_bytes(q.QSPEC_SAMPLE, B, gamma, V),), dtype=torch.uint8,
                     device=DEV)
    q.qspec_verify_accept(q.QSPEC_SAMPLE, cu(t), cu(d), cu(toks), cu(si.uniforms((B, gamma), 3)),
                          cu(si.uniforms((B,), 4)), acc, out, ws)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1234)
    cache = torch.empty((L, B, 2, H, T, D), dtype=torch.int16, device=DEV)
    cache.random_(generator=gen)                       # canary: 16 GiB of seeded bit patterns
    cache = cache.view(torch.bfloat16)
    expect = cache.clone()
    stage = bf16_dev(si.kv_staging(L, B, H, gamma, D, seed=5))
    start = si.start_positions(B, T, gamma, seed=6)
    q.qspec_kv_overwrite(cache, stage, cu(start), acc)
    torch.cuda.synchronize()
    a = acc.cpu().numpy()
    assert a.min() >= 0 and a.max() <= gamma
    # the oracle on sampled (layer, sequence) slices: each slice is a [1][1][2][H][T][D] cache
    stage_h = si.kv_staging(L, B, H, gamma, D, seed=5)
    r = si.rng(17)
    picks = [(0, 0), (L - 1, B - 1)] + [(int(r.integers(L)), int(r.integers(B))) for _ in range(6)]
    for (l, b) in picks:
        before = host_bits16(expect[l, b])[None, None]
        ref = oracle.kv_overwrite(before, stage_h[l, b][None, None], start[b:b + 1], a[b:b + 1])
        assert np.array_equal(host_bits16(cache[l, b])[None, None], ref), (l, b)
    # everything else: the whole cache against the expected copy
    for b in range(B):
        rows = slice(int(start[b]), int(start[b]) + int(a[b]) + 1)
        expect[:, b, :, :, rows, :] = stage[:, b, :, :, : int(a[b]) + 1, :]
    assert torch.equal(cache.view(torch.int16), expect.view(torch.int16))
