"""Pins of the oracle's attention over the shared KV cache (the plainest reading: causal scaled
dot-product attention with grouped KV heads; the pages fix no attention arithmetic): closed forms
for one position, equal keys and a dominant key, the causal extent per query token, and torch's
float64 scaled_dot_product_attention on the same bf16 inputs."""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si


def bf16(a):
    return si.f32_to_bf16_bits(np.asarray(a, np.float32))


def as_f64(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_case(B, Q, Hq, Hkv, T, D, seed):
    r = si.rng(seed)
    q = bf16(r.standard_normal((B, Q, Hq, D)))
    cache = bf16(r.standard_normal((B, 2, Hkv, T, D)))
    return q, cache


def test_single_position_returns_that_value():
    q, cache = rand_case(2, 1, 4, 2, 8, 16, seed=1)
    out = oracle.attention(q, cache, np.zeros(2, np.int32), 0.25)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, 0, h], cache[b, 1, h // 2, 0])    # weight 1 on position 0


def test_equal_keys_average_the_values():
    B, Q, Hq, Hkv, T, D = 1, 3, 2, 1, 10, 8
    q, cache = rand_case(B, Q, Hq, Hkv, T, D, seed=2)
    cache[:, 0] = cache[:, 0, :, :1]                 # every key equal: uniform weights
    pos = np.array([4], np.int32)
    out = oracle.attention(q, cache, pos, 0.5)
    v = as_f64(cache[0, 1, 0])
    for j in range(Q):
        mean = v[: pos[0] + j + 1].mean(axis=0)
        assert np.array_equal(out[0, j, 0], bf16(mean))


def test_dominant_key_selects_its_value():
    B, Q, Hq, Hkv, T, D = 1, 1, 1, 1, 32, 16
    q = bf16(np.ones((B, Q, Hq, D)))
    cache = bf16(np.zeros((B, 2, Hkv, T, D)))
    cache[0, 0, 0, 7] = bf16(np.full(D, 8.0))        # score 8 * 16 * scale on position 7, 0 elsewhere
    cache[0, 1, 0] = bf16(np.arange(T)[:, None] * np.ones(D))
    out = oracle.attention(q, cache, np.array([T - 1], np.int32), 1.0)
    w_other = 1.0 / (1.0 + (T - 1) * math.exp(-128.0))
    assert as_f64(out[0, 0, 0]) == pytest.approx(np.full(D, 7.0 * w_other), rel=1e-2)


def test_causal_extent_and_clipping():
    # query j of sequence b sees exactly positions 0 .. pos + j: changing a later position's
    # value changes no earlier query; positions past T - 1 are clipped
    B, Q, Hq, Hkv, T, D = 2, 4, 2, 2, 12, 8
    q, cache = rand_case(B, Q, Hq, Hkv, T, D, seed=3)
    pos = np.array([3, T - 2], np.int32)
    base = oracle.attention(q, cache, pos, 0.3)
    c2 = cache.copy()
    c2[0, 1, :, 5] = bf16(np.full((Hkv, D), 100.0))  # position 5: seen by queries 2, 3 of sequence 0
    out = oracle.attention(q, c2, pos, 0.3)
    assert np.array_equal(out[0, :2], base[0, :2]) and not np.array_equal(out[0, 2:], base[0, 2:])
    assert np.array_equal(out[1], base[1])
    # sequence 1: queries 1..3 sit at or past T - 1, so all see the whole cache
    assert np.array_equal(base[1, 1, :], oracle.attention(q[:, 1:2], cache, pos + 1, 0.3)[1, 0])


@pytest.mark.parametrize("B,Q,Hq,Hkv,T,D", [(2, 1, 8, 2, 70, 128), (1, 5, 4, 1, 300, 64), (3, 2, 2, 2, 17, 32)])
def test_matches_torch_float64_sdpa(B, Q, Hq, Hkv, T, D):
    q, cache = rand_case(B, Q, Hq, Hkv, T, D, seed=T)
    pos = si.rng(T).integers(0, T - Q + 3, size=B).astype(np.int32)
    scale = 1.0 / math.sqrt(D)
    out = oracle.attention(q, cache, pos, scale)
    G = Hq // Hkv
    for b in range(B):
        qq = torch.from_numpy(as_f64(q[b])).permute(1, 0, 2)                        # [Hq][Q][D]
        k = torch.from_numpy(as_f64(cache[b, 0])).repeat_interleave(G, dim=0)      # [Hq][T][D]
        v = torch.from_numpy(as_f64(cache[b, 1])).repeat_interleave(G, dim=0)
        t = torch.arange(T)[None, :]
        mask = t <= torch.clamp(pos[b] + torch.arange(Q)[:, None], max=T - 1)     # [Q][T]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, k, v, attn_mask=mask, scale=float(np.float32(scale)))
        got = torch.from_numpy(as_f64(out[b])).permute(1, 0, 2)
        # the oracle rounds once to bfloat16: within half an ulp of bf16 (2^-9 relative)
        assert torch.allclose(got, ref, rtol=2 ** -8, atol=1e-6)
