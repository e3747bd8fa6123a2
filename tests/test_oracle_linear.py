"""Pins for the oracle's quantizer, W4A16 and W4A4 linear layers.

QSPEC notes, background terms: W4A16 keeps 4-bit weights and 16-bit activations
and multiplies by the dequantized W_hat = s (W_INT4 - z); W4A4 quantizes the
activations to 4 bits too, accumulates the integer products in INT32 and applies
the scales afterwards.  The pins below use library routines (numpy matmul and
einsum in float64 / int64), closed forms and invariants -- never the oracle's
own loops.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synthetic_inputs as si

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def bf16_to_f64(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()


def unpack_unsigned(codes):
    """[R][K/2] bytes -> [R][K] nibbles, even k from the low nibble (the storage format)."""
    lo = codes & 0x0F
    hi = codes >> 4
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def unpack_signed(codes):
    u = unpack_unsigned(codes)
    return np.where(u >= 8, u - 16, u)


# ---------------------------------------------------------------- quantizer

def test_quantizer_golden_ties():
    g = GOLDEN["quantizer_ties"]
    head = np.array(g["group_head"], np.float32)
    x = np.zeros((1, 256), np.float32)
    x[0, :len(head)] = head
    xb = si.f32_to_bf16_bits(x)
    assert np.array_equal(bf16_to_f64(xb)[0, :len(head)], head)   # all exactly representable
    codes, scales = oracle.quantize_act(xb)
    q = unpack_signed(codes)[0]
    assert scales[0, 0] == g["scale"]
    assert list(q[:len(head)]) == g["codes_head"]
    assert np.all(q[len(head):128] == 0)
    assert scales[0, 1] == 0.0 and np.all(q[128:] == 0)


def _round_binary32(q):
    """Nearest binary32 value to a positive rational q (normal range), ties to even:
    the IEEE 754 definition of a correctly rounded binary32 result, in exact arithmetic."""
    from fractions import Fraction
    e = 0
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    m = q / ulp
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return lo * ulp


def _nearest_even_int(q):
    from fractions import Fraction
    lo = q.numerator // q.denominator
    rem = q - lo
    return lo + 1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1) else lo


@pytest.mark.parametrize("case", GOLDEN["quantizer_division"]["cases"], ids=lambda c: "a" + c["absmax"])
def test_quantizer_golden_division(case):
    """The quotient x / s_a is one correctly rounded binary32 division (not x * (1 / s_a), not an
    exact or binary64 quotient), rounded to the nearest integer with ties to even."""
    from fractions import Fraction
    a, xv = Fraction(case["absmax"]), Fraction(case["x"])
    # the stated codes follow from the IEEE definitions, in exact rational arithmetic
    s_a = _round_binary32(a / 7)
    assert _nearest_even_int(_round_binary32(xv / s_a)) == case["code"]
    assert _nearest_even_int(_round_binary32(xv * _round_binary32(1 / s_a))) == case["reciprocal_multiply_code"]
    assert case["code"] != case["reciprocal_multiply_code"]
    if "exact_quotient_code" in case:
        assert _nearest_even_int(xv / s_a) == case["exact_quotient_code"] != case["code"]
    # the oracle on a group holding a, x, -x and zeros
    vals = np.zeros((1, 128), np.float32)
    vals[0, :3] = [float(a), float(xv), -float(xv)]
    xb = si.f32_to_bf16_bits(vals)
    assert np.array_equal(bf16_to_f64(xb)[0, :3], vals[0, :3])   # exactly representable
    codes, scales = oracle.quantize_act(xb)
    q = unpack_signed(codes)[0]
    assert Fraction(float(scales[0, 0])) == s_a
    assert q[:3].tolist() == [7, case["code"], case["code_of_neg_x"]]
    assert np.all(q[3:] == 0)


@pytest.fixture(scope="module")
def act():
    return si.activations(7, 1024, seed=11)


def test_quantizer_range_and_absmax_code(act):
    codes, scales = oracle.quantize_act(act)
    q = unpack_signed(codes).reshape(7, 8, 128)
    x = bf16_to_f64(act).reshape(7, 8, 128)
    assert q.min() >= -7 and q.max() <= 7          # divisor 7: nothing reaches -8
    amax = np.abs(x).max(axis=2)
    # s_a * 7 reproduces the group's absmax to within one float32 rounding
    assert np.allclose(scales.astype(np.float64) * 7.0, amax, rtol=2 ** -23, atol=0)
    # the absmax element(s) quantize to +-7 exactly
    at_max = np.abs(x) == amax[..., None]
    assert np.all(np.abs(q[at_max]) == 7)


def test_quantizer_error_bound(act):
    codes, scales = oracle.quantize_act(act)
    q = unpack_signed(codes).reshape(7, 8, 128).astype(np.float64)
    x = bf16_to_f64(act).reshape(7, 8, 128)
    s = scales.astype(np.float64)[..., None]
    assert np.all(np.abs(x - q * s) <= s / 2 * (1 + 2 ** -20))


def test_quantizer_sign_symmetry_and_scaling(act):
    codes, scales = oracle.quantize_act(act)
    neg = act ^ np.uint16(0x8000)
    codes_n, scales_n = oracle.quantize_act(neg)
    assert np.array_equal(unpack_signed(codes_n), -unpack_signed(codes))
    assert np.array_equal(scales_n, scales)
    # doubling x (exact in bfloat16) doubles the scale and keeps the codes
    dbl = si.f32_to_bf16_bits(bf16_to_f64(act).astype(np.float32) * 2)
    codes_d, scales_d = oracle.quantize_act(dbl)
    assert np.array_equal(codes_d, codes)
    assert np.array_equal(scales_d, scales * 2)


def test_quantizer_groups_are_independent(act):
    codes, scales = oracle.quantize_act(act)
    mod = act.copy()
    mod[3, 300] = si.f32_to_bf16_bits(np.array([50.0], np.float32))[0]   # group 2 of row 3
    codes_m, scales_m = oracle.quantize_act(mod)
    qa, qb = unpack_signed(codes), unpack_signed(codes_m)
    changed = np.argwhere(qa != qb)
    assert len(changed) > 0
    assert np.all(changed[:, 0] == 3) and np.all((changed[:, 1] >= 256) & (changed[:, 1] < 384))
    diff_s = np.argwhere(scales != scales_m)
    assert diff_s.tolist() == [[3, 2]]


def test_quantizer_zero_group_and_packing():
    x = np.zeros((2, 256), np.float32)
    x[1, 129] = -3.0    # odd k in group 1 -> high nibble of byte 64
    codes, scales = oracle.quantize_act(si.f32_to_bf16_bits(x))
    assert np.all(codes[0] == 0) and np.all(scales[0] == 0)
    assert scales[1, 0] == 0 and scales[1, 1] == np.float32(3.0) / np.float32(7.0)
    assert codes[1, 64] == ((-7) & 15) << 4
    assert np.count_nonzero(codes[1]) == 1


# ---------------------------------------------------------------- W4A16

def rowmajor(w):
    """(codes [N][K], scales f64 [N][G], zeros i64 [N][G]) of a tile-major store, via numpy layout ops."""
    rm, sb, z = si.unpack_weights(w["codes"], w["meta"])
    return unpack_unsigned(rm), sb.view(np.float16).astype(np.float64), z.astype(np.int64)


def with_params(w, scales_bits=None, zeros=None):
    rm, sb, z = si.unpack_weights(w["codes"], w["meta"])
    sb = sb if scales_bits is None else np.broadcast_to(np.asarray(scales_bits, np.uint16), sb.shape)
    z = z if zeros is None else np.broadcast_to(np.asarray(zeros, np.uint8), z.shape)
    c, m = si.pack_weights(rm, sb, z)
    return {"codes": c, "meta": m, "K": w["K"], "N": w["N"]}


@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (5, 384, 48), (3, 512, 16)])
def test_w4a16_unit_scale_reduces_to_plain_matmul(M, K, N):
    w = with_params(si.weights(K, N, seed=M), scales_bits=np.float16(1.0).view(np.uint16), zeros=0)
    x = si.activations(M, K, seed=N)
    y = oracle.gemm_w4a16(x, w["codes"], w["meta"])
    W, _, _ = rowmajor(w)
    ref = bf16_to_f64(x) @ W.astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("M,K,N", [(2, 256, 32), (5, 640, 48)])
def test_w4a16_matches_matmul_with_dequantized_weights(M, K, N):
    w = si.weights(K, N, seed=7 + M)
    x = si.activations(M, K, seed=3)
    y = oracle.gemm_w4a16(x, w["codes"], w["meta"])
    what = bf16_to_f64(oracle.dequant(w["codes"], w["meta"]))   # [N][K]
    ref = bf16_to_f64(x) @ what.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    # power-of-two scale and zero point 0: W_hat = w * 2^-6 exactly, recomputed by hand
    w2 = with_params(w, scales_bits=np.float16(2.0 ** -6).view(np.uint16), zeros=0)
    y2 = oracle.gemm_w4a16(x, w2["codes"], w2["meta"])
    W, _, _ = rowmajor(w2)
    ref2 = bf16_to_f64(x) @ (W.astype(np.float64).T * 2.0 ** -6)
    assert np.allclose(y2, ref2, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- W4A4

@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (4, 512, 32), (3, 384, 16)])
def test_w4a4_group_dots_exact(M, K, N):
    w = si.weights(K, N, seed=20 + M)
    x = si.activations(M, K, seed=21)
    ac, asc = oracle.quantize_act(x)
    y, D = oracle.gemm_w4a4(ac, asc, w["codes"], w["meta"])
    W, s, z = rowmajor(w)
    qa = unpack_signed(ac).reshape(M, K // 128, 128)
    wu = W.reshape(N, K // 128, 128) - z[..., None]
    ref = np.einsum("mgk,ngk->gmn", qa, wu)
    assert np.array_equal(D, ref)
    assert np.abs(D).max() <= 7 * 15 * 128
    # y is the scale-weighted sum of the exact group dots
    yref = np.einsum("mg,ng,gmn->mn", asc.astype(np.float64), s, D.astype(np.float64))
    assert np.allclose(y, yref, rtol=1e-12, atol=1e-15)


def test_w4a4_zero_point_equal_to_code_gives_zero():
    K, N, M = 256, 16, 2
    rm, sb, _ = si.unpack_weights(*[si.weights(K, N, seed=5)[k] for k in ("codes", "meta")])
    rm[:] = 0x77       # every code 7
    c, m = si.pack_weights(rm, sb, np.full(sb.shape, 7, np.uint8))
    ac, asc = oracle.quantize_act(si.activations(M, K, seed=5))
    y, D = oracle.gemm_w4a4(ac, asc, c, m)
    assert np.all(D == 0) and np.all(y == 0)


def test_w4a4_on_grid_activations_match_exact_dequant_product():
    """When x already lies on its own quantization grid, W4A4 equals X (s (W - z))
    computed with the exact (unrounded) dequantized weights."""
    M, K, N = 3, 384, 16
    r = np.random.default_rng(9)
    q = r.integers(-7, 8, size=(M, K)).astype(np.float32)
    q[:, ::128] = 7                                           # absmax 7 in every group
    step = (2.0 ** r.integers(-4, 3, size=(M, K // 128))).astype(np.float32)
    x = q * np.repeat(step, 128, axis=1)                      # exact in bfloat16
    xb = si.f32_to_bf16_bits(x)
    ac, asc = oracle.quantize_act(xb)
    assert np.array_equal(asc, step)                          # s_a = 7*step/7 exactly
    w = si.weights(K, N, seed=9)
    y, _ = oracle.gemm_w4a4(ac, asc, w["codes"], w["meta"])
    W, s, z = rowmajor(w)
    wexact = (W - np.repeat(z, 128, axis=1)) * np.repeat(s, 128, axis=1)
    ref = x.astype(np.float64) @ wexact.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_w4a4_dots_are_linear_in_activation_codes():
    K, N = 256, 16
    w = si.weights(K, N, seed=31)
    e = np.zeros((1, K), np.float32)
    e[0, 130] = 7.0                      # one-hot activation: code 7 at k = 130, scale 1
    ac, asc = oracle.quantize_act(si.f32_to_bf16_bits(e))
    _, D = oracle.gemm_w4a4(ac, asc, w["codes"], w["meta"])
    W, _, z = rowmajor(w)
    col = W[:, 130] - z[:, 1]
    assert np.array_equal(D[1, 0], 7 * col)
    assert np.all(D[0] == 0)
