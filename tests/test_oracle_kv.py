"""Pins for the oracle's KV replacement (QSPEC notes, QSPEC structure: accepted
positions get the verifier's KV in place of the draft's).  Checked against numpy
slicing and a canary pattern: exactly the committed rows change."""
import numpy as np
import pytest

import oracle
import synthetic_inputs as si


@pytest.mark.parametrize("L,B,H,T,D,gamma", [(2, 3, 2, 32, 8, 4), (1, 5, 1, 16, 4, 2), (3, 2, 3, 10, 16, 0)])
def test_kv_overwrite_matches_slicing(L, B, H, T, D, gamma):
    cache = si.kv_canary(L, B, H, T, D).reshape(L, B, 2, H, T, D)
    staging = si.kv_staging(L, B, H, gamma, D, seed=L + B)
    start = si.start_positions(B, T, gamma, seed=B)
    acc = si.rng(3).integers(0, gamma + 1, size=B).astype(np.int32)
    expect = cache.copy()
    for b in range(B):
        n = acc[b] + 1
        expect[:, b, :, :, start[b]:start[b] + n, :] = staging[:, b, :, :, :n, :]
    got = oracle.kv_overwrite(cache.copy(), staging, start, acc)
    assert np.array_equal(got, expect)
    changed = np.any(got != si.kv_canary(L, B, H, T, D).reshape(cache.shape), axis=-1)
    # only positions start..start+A can differ from the canary
    for b in range(B):
        rows = np.nonzero(changed[:, b].any(axis=(0, 1, 2)))[0]
        assert set(rows.tolist()) <= set(range(start[b], start[b] + acc[b] + 1))


def test_kv_overwrite_zero_accept_copies_one_row_and_clips_at_end():
    L, B, H, T, D, gamma = 1, 2, 1, 8, 4, 3
    cache = si.kv_canary(L, B, H, T, D).reshape(L, B, 2, H, T, D)
    staging = si.kv_staging(L, B, H, gamma, D, seed=1)
    start = np.array([2, 6], np.int32)
    acc = np.array([0, 3], np.int32)                   # b=1 would write rows 6..9: 8, 9 fall off
    got = oracle.kv_overwrite(cache.copy(), staging, start, acc)
    assert np.array_equal(got[:, 0, :, :, 2], staging[:, 0, :, :, 0])
    assert np.array_equal(got[:, 0, :, :, 3:], cache[:, 0, :, :, 3:])
    assert np.array_equal(got[:, 1, :, :, 6:8], staging[:, 1, :, :, 0:2])
    assert np.array_equal(got[:, 1, :, :, :6], cache[:, 1, :, :, :6])
    # accept counts outside [0, gamma] are clamped
    got2 = oracle.kv_overwrite(cache.copy(), staging, np.array([0, 0], np.int32), np.array([-5, 99], np.int32))
    assert np.array_equal(got2[:, 0, :, :, 0], staging[:, 0, :, :, 0])
    assert np.array_equal(got2[:, 0, :, :, 1:], cache[:, 0, :, :, 1:])
    assert np.array_equal(got2[:, 1, :, :, :gamma + 1], staging[:, 1])
