"""GPU parity of attention over the shared KV cache (qspec_attention) against the oracle's fp64
causal attention: every output element within the bfloat16 tolerance (rel 1e-2, abs 1e-3), over
ragged contexts, every query-row tiling the kernel uses, clipped and degenerate positions, and
sampled sequences of the Llama-3-8B-shaped decode and verify workloads at a 4096-token context."""
import math

import numpy as np
import pytest
import torch

import oracle
import quantized_speculative_decoding_amd as q
import synthetic_inputs as si
from gpu_helpers import DEV, assert_close, bf16_dev, cu, host_bits16, note

pytestmark = pytest.mark.gpu


def as_f64(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_attention(qd, cached, posd, scale):
    B, Q, Hq, D = qd.shape
    Hkv, T = cached.shape[2], cached.shape[3]
    out = torch.full((B, Q, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty((q.qspec_attention_workspace_bytes(B, Q, Hq, Hkv, T),), dtype=torch.uint8, device=DEV)
    q.qspec_attention(qd, cached, posd, scale, out, ws)
    return out


def check(qb, cache, pos, scale, what, seqs=None):
    out = host_bits16(run_attention(bf16_dev(qb), bf16_dev(cache), cu(pos), scale))
    seqs = range(qb.shape[0]) if seqs is None else seqs
    for b in seqs:
        ref = oracle.attention(qb[b:b + 1], cache[b:b + 1], np.maximum(pos[b:b + 1], 0), scale)[0]
        assert_close(as_f64(out[b]), as_f64(ref), bf16=True, what=f"{what} b={b}")
    return out


# (B, Q, Hq, Hkv, T): contexts shorter than one 32-position step, ragged chunk tails, one and two
# 16-row tiles per pass and several passes (Q * Hq / Hkv = 4, 20, 32, 40, 64, 68), G = 1 and 8,
# and contexts of more than 8 chunks of 512 (the merge takes chunks 8 at a time)
CASES = [(2, 1, 4, 1, 7, ), (3, 1, 32, 8, 70), (2, 5, 32, 8, 600), (2, 4, 8, 1, 1100), (1, 8, 32, 8, 513),
         (2, 5, 64, 8, 300), (1, 16, 32, 8, 200), (2, 17, 8, 2, 260), (2, 2, 8, 8, 1500), (2, 3, 8, 2, 5000),
         (1, 1, 32, 8, 32768)]


@pytest.mark.parametrize("B,Q,Hq,Hkv,T", CASES)
def test_attention_matches_oracle(B, Q, Hq, Hkv, T):
    note(f"attention B={B} Q={Q} Hq={Hq} Hkv={Hkv} T={T}")
    qb, cache = si.attention_inputs(B, Q, Hq, Hkv, T, 128, seed=T + Q)
    pos = si.rng(T + 7 * Q).integers(0, T, size=B).astype(np.int32)
    pos[0] = T - Q                                    # the last query sits at the last position
    check(qb, cache, pos, 1.0 / math.sqrt(128), "attention")


def test_attention_positions_past_the_context_and_negative():
    """pos + j beyond T - 1 sees the whole cache; pos < 0 reads as 0 (query 0 sees one position)."""
    note("attention clipped and negative positions")
    B, Q, Hq, Hkv, T = 4, 5, 8, 2, 300
    qb, cache = si.attention_inputs(B, Q, Hq, Hkv, T, 128, seed=5)
    pos = np.array([T - 1, T + 1000, -7, 0], np.int32)
    out = check(qb, cache, pos, 0.1, "clipped")
    for h in range(Hq):                               # one visible position: exactly its value
        assert np.array_equal(out[2, 0, h], cache[2, 1, h // 4, 0])
        assert np.array_equal(out[3, 0, h], cache[3, 1, h // 4, 0])


def test_attention_ignores_cache_past_the_visible_range():
    """Cache rows after the last visible position (here NaN bit patterns) are never read."""
    note("attention NaN past the visible range")
    B, Q, Hq, Hkv, T = 2, 3, 32, 8, 1200
    qb, cache = si.attention_inputs(B, Q, Hq, Hkv, T, 128, seed=9)
    pos = np.array([100, 700], np.int32)
    for b in range(B):
        cache[b, :, :, pos[b] + Q:] = 0x7FC0          # quiet NaN
    out = check(qb, cache, pos, 1.0 / math.sqrt(128), "nan tail")
    assert not np.isnan(as_f64(out)).any()


def test_attention_extreme_scores():
    """Large score ranges (one dominant key, exp underflow elsewhere) and equal keys."""
    note("attention extreme scores")
    B, Q, Hq, Hkv, T = 2, 2, 4, 1, 900
    qb, cache = si.attention_inputs(B, Q, Hq, Hkv, T, 128, seed=11)
    cache[0, 0, 0, 650] = si.f32_to_bf16_bits(as_f64(qb[0, 0, 0]).astype(np.float32) * 4)
    cache[1, 0] = cache[1, 0, :, :1]                  # every key equal: the mean of the values
    check(qb, cache, np.array([T - Q, 777], np.int32), 1.0, "extreme")


@pytest.mark.parametrize("B,Q", [(16, 1), (16, 5), (32, 5)])
def test_attention_llama3_8b_context_4096(B, Q):
    """Llama-3-8B attention shape (32 query heads, 8 KV heads, d 128) at a 4096-token context, the
    configuration timed by the benchmark; sampled sequences against the oracle."""
    note(f"attention Llama-3-8B B={B} Q={Q} T=4096")
    Hq, Hkv, T = 32, 8, 4096
    qb, cache = si.attention_inputs(B, Q, Hq, Hkv, T, 128, seed=B * 10 + Q)
    pos = np.full(B, T - Q, np.int32)
    pos[1::3] = si.rng(Q).integers(0, T - Q, size=len(pos[1::3]))
    check(qb, cache, pos, 1.0 / math.sqrt(128), "llama3-8b", seqs=[0, 1, B // 2, B - 1])


def test_attention_is_row_independent_of_batch():
    """A sequence's output does not depend on the other sequences in the batch."""
    note("attention batch independence")
    B, Q, Hq, Hkv, T = 6, 5, 32, 8, 800
    qb, cache = si.attention_inputs(B, Q, Hq, Hkv, T, 128, seed=13)
    pos = si.rng(13).integers(0, T, size=B).astype(np.int32)
    full = host_bits16(run_attention(bf16_dev(qb), bf16_dev(cache), cu(pos), 0.09))
    one = host_bits16(run_attention(bf16_dev(qb[3:4]), bf16_dev(cache[3:4]), cu(pos[3:4]), 0.09))
    assert np.array_equal(full[3], one[0])
