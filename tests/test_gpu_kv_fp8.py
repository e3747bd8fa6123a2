"""GPU parity of the quantized (FP8 E4M3, one scale per row of 128) KV cache: the quantizing
overwrite (qspec_kv_overwrite_fp8) bit-exact against the oracle (codes and scales, with guard
regions and a canary cache: nothing but the committed rows changes), and attention over the
quantized cache (qspec_attention_fp8) against the oracle's fp64 attention over the decoded cache
(bfloat16 tolerance, rel 1e-2 / abs 1e-3), over ragged contexts, both query-row tilings, clipped
and negative positions, a NaN tail past the visible range, and sampled sequences of the
Llama-3-8B-shaped decode and verify workloads at a 4096-token context."""
import math

import numpy as np
import pytest
import torch

import oracle
import quantized_speculative_decoding_amd as q
import synthetic_inputs as si
from gpu_helpers import DEV, Guarded, assert_close, bf16_dev, cu, host_bits16, note

pytestmark = pytest.mark.gpu


def as_f64(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def quantized_cache(cache_bits):
    """FP8 codes [B][2][Hkv][T][D] and scales [B][2][Hkv][T] of a bf16 cache, row by row (oracle)."""
    B, two, Hkv, T, D = cache_bits.shape
    codes, scales = oracle.quantize_act_fp8(cache_bits.reshape(-1, D))
    return codes.reshape(B, two, Hkv, T, D), scales.reshape(B, two, Hkv, T)


def run_attention_fp8(qb, codes, scales, pos, scale):
    B, Q, Hq, D = qb.shape
    Hkv, T = codes.shape[2], codes.shape[3]
    out = Guarded((B, Q, Hq, D), torch.bfloat16)
    ws = torch.empty((q.qspec_attention_workspace_bytes(B, Q, Hq, Hkv, T),), dtype=torch.uint8, device=DEV)
    q.qspec_attention_fp8(bf16_dev(qb), cu(codes), cu(scales), cu(pos), scale, out.t, ws)
    out.check(f"attention_fp8 B={B} Q={Q} T={T}")
    return host_bits16(out.t)


def check(qb, codes, scales, pos, scale, what, seqs=None):
    out = run_attention_fp8(qb, codes, scales, pos, scale)
    for b in (range(qb.shape[0]) if seqs is None else seqs):
        ref = oracle.attention_fp8(qb[b:b + 1], codes[b:b + 1], scales[b:b + 1], np.maximum(pos[b:b + 1], 0), scale)[0]
        assert_close(as_f64(out[b]), as_f64(ref), bf16=True, what=f"{what} b={b}")
    return out


# (B, Q, Hq, Hkv, T): as the bfloat16 attention's cases -- contexts shorter than one 32-position
# step, ragged chunk tails, one and two 16-row tiles and several passes, G = 1 and 8, more than 8
# chunks of 512 -- and a context whose length is not a multiple of 4 (per-position scale loads)
CASES = [(2, 1, 4, 1, 7), (3, 1, 32, 8, 70), (2, 5, 32, 8, 600), (2, 4, 8, 1, 1100), (1, 8, 32, 8, 513),
         (2, 5, 64, 8, 301), (2, 17, 8, 2, 259), (2, 3, 8, 2, 5001)]


@pytest.mark.parametrize("B,Q,Hq,Hkv,T", CASES)
def test_attention_fp8_matches_oracle(B, Q, Hq, Hkv, T):
    note(f"attention_fp8 B={B} Q={Q} Hq={Hq} Hkv={Hkv} T={T}")
    qb, cache = si.attention_inputs(B, Q, Hq, Hkv, T, 128, seed=T + Q + 1)
    codes, scales = quantized_cache(cache)
    pos = si.rng(T + 5 * Q).integers(0, T, size=B).astype(np.int32)
    pos[0] = T - Q
    check(qb, codes, scales, pos, 1.0 / math.sqrt(128), "attention_fp8")


def test_attention_fp8_clipped_negative_positions_and_nan_tail():
    """pos + j past T - 1 sees the whole cache; pos < 0 reads as 0 (one visible position gives its
    value, decoded and rounded to bfloat16); codes and scales after the last visible position (NaN
    codes 0x7F, NaN scales) are never read."""
    note("attention_fp8 clipped / negative / NaN tail")
    B, Q, Hq, Hkv, T = 4, 5, 8, 2, 300
    qb, cache = si.attention_inputs(B, Q, Hq, Hkv, T, 128, seed=15)
    codes, scales = quantized_cache(cache)
    pos = np.array([T - 1, T + 1000, -7, 0], np.int32)
    for b in (2, 3):                                   # visible: position 0 .. Q - 1 only
        codes[b, :, :, Q:] = 0x7F
        scales[b, :, :, Q:] = np.nan
    out = check(qb, codes, scales, pos, 0.1, "clipped")
    assert not np.isnan(as_f64(out)).any()
    dec = torch.from_numpy(codes[2, 1, :, 0]).view(torch.float8_e4m3fn).double().numpy() * scales[2, 1, :, 0, None]
    for h in range(Hq):                                # query 0 of sequence 2 sees position 0 only
        assert np.array_equal(out[2, 0, h], si.f32_to_bf16_bits(dec[h // 4].astype(np.float32)))


@pytest.mark.parametrize("L,B,H,T,gamma", [(2, 3, 2, 16, 4), (1, 4, 8, 9, 0), (3, 5, 1, 40, 7)])
def test_kv_overwrite_fp8_bit_exact(L, B, H, T, gamma):
    note(f"kv_overwrite_fp8 L={L} B={B} H={H} T={T} gamma={gamma}")
    D = 128
    r = si.rng(T + gamma)
    codes = r.integers(0, 256, size=(L, B, 2, H, T, D)).astype(np.uint8)
    scales = r.random((L, B, 2, H, T)).astype(np.float32)
    stage = si.kv_staging(L, B, H, gamma, D, seed=T)
    stage[0, 0, 1, 0, 0] = 0                           # an all-zero row
    start = r.integers(-2, T, size=B).astype(np.int32)
    start[0] = 0
    start[-1] = T - 1                                  # only row 0 of the last sequence fits
    acc = r.integers(-1, gamma + 3, size=B).astype(np.int32)
    gc, gs = Guarded(codes.shape, torch.uint8), Guarded(scales.shape, torch.float32)
    gc.t.copy_(cu(codes))
    gs.t.copy_(cu(scales))
    q.qspec_kv_overwrite_fp8(gc.t, gs.t, bf16_dev(stage), cu(start), cu(acc))
    gc.check("kv_overwrite_fp8 codes")
    gs.check("kv_overwrite_fp8 scales")
    rc, rs = oracle.kv_overwrite_fp8(codes.copy(), scales.copy(), stage, start, acc)
    assert np.array_equal(gc.t.cpu().numpy(), rc)
    assert np.array_equal(gs.t.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_kv_overwrite_fp8_then_attention_reads_the_committed_rows():
    """Rows committed by the quantizing overwrite (one call writing every position of the cache)
    are what the quantized attention reads: its result equals the oracle's on the oracle's own
    overwrite of the same rows."""
    note("kv_overwrite_fp8 -> attention_fp8")
    B, Hkv, Hq, T, Q, D = 2, 2, 8, 64, 3, 128
    stage = si.kv_staging(1, B, Hkv, T - 1, D, seed=77)          # gamma = T - 1: rows for every position
    start = np.zeros(B, np.int32)
    acc = np.full(B, T - 1, np.int32)
    codes = torch.zeros((1, B, 2, Hkv, T, D), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((1, B, 2, Hkv, T), dtype=torch.float32, device=DEV)
    q.qspec_kv_overwrite_fp8(codes, scales, bf16_dev(stage), cu(start), cu(acc))
    rc, rs = oracle.kv_overwrite_fp8(np.zeros((1, B, 2, Hkv, T, D), np.uint8), np.zeros((1, B, 2, Hkv, T), np.float32),
                                     stage, start, acc)
    assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs)
    qb = si.attention_inputs(B, Q, Hq, Hkv, T, D, seed=78)[0]
    pos = np.array([T - Q, 20], np.int32)
    outd = torch.empty((B, Q, Hq, D), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty((q.qspec_attention_workspace_bytes(B, Q, Hq, Hkv, T),), dtype=torch.uint8, device=DEV)
    q.qspec_attention_fp8(bf16_dev(qb), codes[0], scales[0], cu(pos), 1.0 / math.sqrt(D), outd, ws)
    out = host_bits16(outd)
    for b in range(B):
        ref = oracle.attention_fp8(qb[b:b + 1], rc[0, b:b + 1], rs[0, b:b + 1], pos[b:b + 1], 1.0 / math.sqrt(D))[0]
        assert_close(as_f64(out[b]), as_f64(ref), bf16=True, what=f"committed b={b}")


@pytest.mark.parametrize("Q", [1, 5])
def test_attention_fp8_full_workload_sampled(Q):
    """Llama-3-8B heads at B = 16 and a 4096-token context (the draft step Q = 1, the verify pass
    Q = gamma + 1 = 5), codes drawn on the device; four sequences checked in full."""
    note(f"attention_fp8 full B=16 Q={Q} T=4096")
    B, Hq, Hkv, T, D = 16, 32, 8, 4096, 128
    qd, cache = si.attention_inputs_device(B, Q, Hq, Hkv, T, D, seed=Q + 40, device=DEV)
    codes = torch.empty((B, 2, Hkv, T, D), dtype=torch.uint8, device=DEV)
    scales = torch.empty((B, 2, Hkv, T), dtype=torch.float32, device=DEV)
    # every row quantized on the device by the FP8 activation quantizer (validated elsewhere)
    q.qspec_quantize_act_fp8(cache.view(-1, D), codes.view(-1, D), scales.view(-1))
    pos = torch.from_numpy(si.start_positions(B, T, Q - 1, seed=Q)).to(DEV)
    out = torch.empty((B, Q, Hq, D), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty((q.qspec_attention_workspace_bytes(B, Q, Hq, Hkv, T),), dtype=torch.uint8, device=DEV)
    q.qspec_attention_fp8(qd, codes, scales, pos, 1.0 / math.sqrt(D), out, ws)
    qb, cb, sb, pb, ob = (host_bits16(qd), codes.cpu().numpy(), scales.cpu().numpy(), pos.cpu().numpy(),
                          host_bits16(out))
    oc, osc = oracle.quantize_act_fp8(host_bits16(cache).reshape(-1, D))
    assert np.array_equal(cb.reshape(-1, D), oc) and np.array_equal(sb.reshape(-1), osc)
    for b in (0, 5, 10, 15):
        ref = oracle.attention_fp8(qb[b:b + 1], cb[b:b + 1], sb[b:b + 1], pb[b:b + 1], 1.0 / math.sqrt(D))[0]
        assert_close(as_f64(ob[b]), as_f64(ref), bf16=True, what=f"full Q={Q} b={b}")
