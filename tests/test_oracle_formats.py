"""Pins for the oracle's number-format helpers and the dequantization rule.

Pinned against library conversions (numpy binary16, torch bfloat16), hand-derived
rounding cases stored in tests/golden/closed_forms.json, and exact identities of
W_hat = s (W_INT4 - z) from the QSPEC notes (background terms: dequantization
example).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def _torch_bf16_bits(values_f64):
    t = torch.tensor(np.asarray(values_f64, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_fp16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_to_double(b) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_double(b) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])


def test_bf16_rounding_matches_torch_on_float32_values():
    r = np.random.default_rng(1)
    vals = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(5000) * 1e-30).astype(np.float32),
        (r.standard_normal(5000) * 1e30).astype(np.float32),
        # float32 values that sit exactly on bfloat16 halfway points
        (np.float32(1.0) + np.float32(2.0 ** -8) * (2 * r.integers(0, 128, 2000) + 1)).astype(np.float32),
    ])
    ref = _torch_bf16_bits(vals)
    got = np.array([oracle.double_to_bf16(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


def _parse_value(s):
    env = {"__builtins__": {}}
    return eval(s.replace("^", "**"), env)  # only the fixture's own arithmetic strings


@pytest.mark.parametrize("case", [c for c in GOLDEN["bf16_rounding"]["cases"] if "scale_bits" not in c],
                         ids=lambda c: c["value"])
def test_bf16_rounding_golden(case):
    v = _parse_value(case["value"])
    assert oracle.double_to_bf16(v) == int(case["bits"], 16)


def test_dequant_golden_worked_example():
    case = [c for c in GOLDEN["bf16_rounding"]["cases"] if "scale_bits" in c][0]
    s = int(case["scale_bits"], 16)
    d = case["w_minus_z"]
    assert oracle.dequant_one(s, d, 0) == int(case["bits"], 16)
    assert oracle.dequant_one(s, 15, 15 - d) == int(case["bits"], 16)


def test_dequant_unit_scale_is_exact_difference():
    one = int(np.float16(1.0).view(np.uint16))
    for w in range(16):
        for z in range(16):
            assert oracle.bf16_to_double(oracle.dequant_one(one, w, z)) == float(w - z)


def test_dequant_power_of_two_scales_exact():
    for e in range(-14, 5):
        s = int(np.float16(2.0 ** e).view(np.uint16))
        for w in range(16):
            for z in range(16):
                assert oracle.bf16_to_double(oracle.dequant_one(s, w, z)) == (w - z) * 2.0 ** e


def test_dequant_all_codes_random_scales_match_library_rounding():
    r = np.random.default_rng(2)
    scales = r.uniform(1e-3, 1e-2, 200).astype(np.float16)
    scales = np.concatenate([scales, (-scales[:20]).astype(np.float16),
                             np.array([6.1e-5, 65504.0, 3.0e-5], np.float16)])
    for s in scales:
        sb = int(s.view(np.uint16))
        w = np.repeat(np.arange(16), 16)
        z = np.tile(np.arange(16), 16)
        prod = float(s) * (w - z).astype(np.float64)
        # the product has at most 15 significant bits: exact in float32, so torch's
        # float32 -> bfloat16 conversion rounds the exact value once
        assert np.all(prod.astype(np.float32).astype(np.float64) == prod)
        ref = _torch_bf16_bits(prod)
        got = np.array([oracle.dequant_one(sb, int(a), int(b)) for a, b in zip(w, z)], np.uint16)
        assert np.array_equal(got, ref), float(s)


def test_dequant_w_equal_z_is_zero():
    r = np.random.default_rng(3)
    for s in r.uniform(1e-3, 1e-2, 50).astype(np.float16):
        for w in range(16):
            assert oracle.bf16_to_double(oracle.dequant_one(int(s.view(np.uint16)), w, w)) == 0.0


def test_dequant_layout_nibble_and_group_placement():
    """Single planted codes land where the tile-major layout definition puts them."""
    import synthetic_inputs as si
    K, N = 384, 48
    codes = np.zeros((N, K // 2), np.uint8)
    one = np.float16(1.0).view(np.uint16)
    scales = np.full((N, K // 128), one, np.uint16)
    zeros = np.zeros((N, K // 128), np.uint8)
    codes[17, 70] = 0x5A          # column 17, k = 140 -> low nibble 0xA, k = 141 -> high nibble 0x5
    codes[33, 191] = 0x0C         # column 33, k = 382 (last group, last quarter)
    scales[17, 1] = np.float16(0.5).view(np.uint16)   # group 1 covers k = 128..255
    zeros[2, 2] = 3
    tc, meta = si.pack_weights(codes, scales, zeros)
    assert tc.shape == (3, 3, 1024) and meta.shape == (3, 3, 16)
    # byte of (n=17, k=140): tile 1, group 1, quarter 0, column 1, byte 6
    assert tc[1, 1, 0 * 256 + 1 * 16 + 6] == 0x5A
    assert tc[2, 2, 3 * 256 + 1 * 16 + 15] == 0x0C
    assert meta[1, 1, 1] == (np.uint32(np.float16(0.5).view(np.uint16)))
    assert meta[0, 2, 2] == (np.uint32(one) | np.uint32(3 << 16))
    w = np.vectorize(oracle.bf16_to_double)(oracle.dequant(tc, meta))
    expect = np.zeros((N, K))
    expect[17, 140] = 10 * 0.5
    expect[17, 141] = 5 * 0.5
    expect[33, 382] = 12.0
    expect[2, 256:384] = -3.0
    assert np.array_equal(w, expect)


def test_fp16_scale_subnormal_decode():
    assert oracle.fp16_to_double(0x0001) == 2.0 ** -24
    assert oracle.fp16_to_double(0x0400) == 2.0 ** -14
    assert oracle.fp16_to_double(0x7BFF) == 65504.0
    assert math.isinf(oracle.fp16_to_double(0x7C00))
