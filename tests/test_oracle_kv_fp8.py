"""Pins of the oracle's quantized KV cache (the reading of the QSPEC notes' "quantized KV": FP8
E4M3 codes with one binary32 scale per (position, KV head) row, written when the verifier's rows
replace the draft's, and read back by attention as scale * decoded code).

The overwrite is pinned against its definition written with torch's float8_e4m3fn conversion
(an independent implementation of E4M3 rounding), against a canary cache (exactly the committed
rows change), and against the read-back error bound of E4M3; the attention over the quantized
cache against the pinned bf16 oracle attention (codes whose decoded values are bf16 values, unit
scales) and against torch's float64 scaled_dot_product_attention on the decoded cache."""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si


def f64(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def torch_row_quant(rows_bits):
    """Per-row E4M3 quantization written with torch: s = max|v| / 448 (binary32), codes = the
    float8_e4m3fn conversion of v / s (binary32 quotient)."""
    v = torch.from_numpy(f64(rows_bits).astype(np.float32))
    a = v.abs().amax(dim=-1, keepdim=True)
    s = a / 448.0
    q = torch.where(a > 0, v / torch.where(a > 0, s, torch.ones_like(s)), torch.zeros_like(v))
    return q.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), s.squeeze(-1).numpy()


def fresh_cache(L, B, H, T, D, seed):
    r = si.rng(seed)
    codes = r.integers(0, 256, size=(L, B, 2, H, T, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] ^= 1                      # no NaN codes
    scales = (r.random((L, B, 2, H, T)) + 0.5).astype(np.float32)
    return codes, scales


@pytest.mark.parametrize("L,B,H,T,D,gamma", [(2, 3, 2, 16, 128, 4), (1, 4, 1, 9, 32, 0), (1, 2, 3, 6, 64, 5)])
def test_overwrite_matches_its_torch_definition_and_touches_only_committed_rows(L, B, H, T, D, gamma):
    codes, scales = fresh_cache(L, B, H, T, D, seed=T + D)
    c0, s0 = codes.copy(), scales.copy()
    r = si.rng(gamma + 11)
    stage = si.f32_to_bf16_bits(r.standard_normal((L, B, 2, H, gamma + 1, D)).astype(np.float32) * 3.0)
    stage[0, 0, 0, 0, 0] = 0                                 # an all-zero row
    start = r.integers(-2, T, size=B).astype(np.int32)
    start[0] = 0
    acc = r.integers(-1, gamma + 3, size=B).astype(np.int32)  # clamped to [0, gamma]
    oracle.kv_overwrite_fp8(codes, scales, stage, start, acc)
    written = np.zeros((L, B, 2, H, T), bool)
    for l in range(L):
        for b in range(B):
            A = min(max(int(acc[b]), 0), gamma)
            for rr in range(A + 1):
                t = int(start[b]) + rr
                if 0 <= t < T:
                    written[l, b, :, :, t] = True
                    ec, es = torch_row_quant(stage[l, b, :, :, rr])
                    assert np.array_equal(codes[l, b, :, :, t], ec)
                    assert np.array_equal(scales[l, b, :, :, t].view(np.uint32), es.astype(np.float32).view(np.uint32))
    assert np.array_equal(codes[~written], c0[~written])
    assert np.array_equal(scales[~written], s0[~written])
    assert scales[0, 0, 0, 0, 0] == 0 and not codes[0, 0, 0, 0, 0].any()   # the zero row (start 0, r 0)


def test_read_back_bound_and_row_maximum():
    """Every value reads back within half an E4M3 step of itself (relative 2^-4 in the normal
    range, 2^-9 * s absolute below it), and each row's largest magnitude maps to +-448 exactly."""
    L, B, H, T, D, gamma = 1, 2, 2, 8, 128, 3
    codes, scales = fresh_cache(L, B, H, T, D, seed=5)
    stage_f = si.rng(6).standard_normal((L, B, 2, H, gamma + 1, D)).astype(np.float32) * 10.0
    stage = si.f32_to_bf16_bits(stage_f)
    start = np.array([0, 4], np.int32)
    acc = np.array([gamma, gamma], np.int32)
    oracle.kv_overwrite_fp8(codes, scales, stage, start, acc)
    for b in range(B):
        for rr in range(gamma + 1):
            t = start[b] + rr
            v = f64(stage[0, b, :, :, rr])                       # [2][H][D]
            s = scales[0, b, :, :, t].astype(np.float64)[..., None]
            back = s * decode(codes[0, b, :, :, t])
            step = np.where(np.abs(v) >= s * 2.0 ** -6, np.abs(v) * 2.0 ** -4, s * 2.0 ** -9)
            assert np.all(np.abs(back - v) <= step * (1 + 1e-6))
            top = np.argmax(np.abs(v), axis=-1)
            tc = np.take_along_axis(codes[0, b, :, :, t], top[..., None], axis=-1)[..., 0]
            assert np.all((tc & 0x7F) == 0x7E)


def test_attention_on_bf16_representable_codes_equals_the_bf16_oracle():
    """Unit scales and codes whose decoded values are bf16 values (every E4M3 value is one): the
    quantized-cache attention is the bf16-cache attention on the decoded cache."""
    B, Q, Hq, Hkv, T, D = 2, 3, 4, 2, 40, 128
    r = si.rng(9)
    codes = r.integers(0, 256, size=(B, 2, Hkv, T, D)).astype(np.uint8)
    codes[(codes & 0x7F) >= 0x70] &= 0x8F                   # keep |value| modest, no NaN
    scales = np.ones((B, 2, Hkv, T), np.float32)
    q = si.f32_to_bf16_bits(r.standard_normal((B, Q, Hq, D)).astype(np.float32) * 0.05)
    cache_bf16 = si.f32_to_bf16_bits(decode(codes).astype(np.float32))
    assert np.array_equal(f64(cache_bf16), decode(codes))    # the decoded values are bf16-exact
    pos = np.array([5, T - 2], np.int32)
    got = oracle.attention_fp8(q, codes, scales, pos, 0.0883883)
    ref = oracle.attention(q, cache_bf16, pos, 0.0883883)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("B,Q,Hq,Hkv,T", [(2, 1, 8, 2, 70), (1, 5, 4, 1, 200), (3, 2, 2, 2, 17)])
def test_attention_matches_torch_float64_sdpa_on_the_decoded_cache(B, Q, Hq, Hkv, T):
    D = 128
    r = si.rng(T + Q)
    codes, _ = fresh_cache(1, B, Hkv, T, D, seed=T)
    codes = codes[0]
    codes[(codes & 0x7F) >= 0x70] &= 0x8F
    scales = (r.random((B, 2, Hkv, T)) * 0.02 + 0.005).astype(np.float32)
    q = si.f32_to_bf16_bits(r.standard_normal((B, Q, Hq, D)).astype(np.float32))
    pos = r.integers(0, T - Q + 3, size=B).astype(np.int32)
    got = f64(oracle.attention_fp8(q, codes, scales, pos, 1.0 / np.sqrt(D)))
    kv = decode(codes) * scales.astype(np.float64)[..., None]          # [B][2][Hkv][T][D]
    qt = torch.from_numpy(f64(q))
    for b in range(B):
        for j in range(Q):
            last = min(max(int(pos[b]), 0) + j, T - 1)
            for h in range(Hq):
                k = torch.from_numpy(kv[b, 0, h // (Hq // Hkv), : last + 1])
                v = torch.from_numpy(kv[b, 1, h // (Hq // Hkv), : last + 1])
                o = torch.nn.functional.scaled_dot_product_attention(qt[b, j, h][None, None], k[None], v[None],
                                                                      scale=1.0 / np.sqrt(D))[0, 0].numpy()
                ref = f64(si.f32_to_bf16_bits(o.astype(np.float32)))
                assert np.allclose(got[b, j, h], ref, rtol=2 ** -7, atol=1e-6), (b, j, h)
