"""Pins of the oracle's FP8 parent variant (SpecQuant notes: INT4 / FP8 / FP16 variants of one
model by post-training quantization; the reading: OCP E4M3, per-column weight and per-token
activation scales of absmax / 448).  Decoding and rounding are checked against torch's own
float8_e4m3fn conversions, the quantizers against their definitions written with torch
primitives, the product against numpy's float64 matmul of the decoded operands."""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si


def torch_e4m3_bits(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_e4m3_value(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def as_f32(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def test_decode_table_matches_torch():
    ours = np.array([oracle.e4m3_to_double(c) for c in range(256)])
    ref = torch_e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(ours), np.isnan(ref)) and np.isnan(ours).sum() == 2
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6 and ours[0x38] == 1.0


def test_rounding_matches_torch_inside_the_range():
    r = si.rng(1)
    every_bf16 = as_f32(np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16))
    every_bf16 = every_bf16[np.isfinite(every_bf16) & (np.abs(every_bf16) <= 448)]
    vals = np.concatenate([r.uniform(-448, 448, 20000), r.uniform(-1, 1, 20000), r.uniform(-2 ** -5, 2 ** -5, 20000)])
    vals = np.concatenate([vals.astype(np.float32), every_bf16])
    # every midpoint between neighbouring codes: ties go to the even code
    pos = torch_e4m3_value(np.arange(0x7F))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals = np.concatenate([vals, mids, -mids])
    ours = np.array([oracle.double_to_e4m3(float(v)) for v in vals], np.uint8)
    assert np.array_equal(ours, torch_e4m3_bits(vals))
    assert np.all(np.array([oracle.double_to_e4m3(float(m)) for m in mids]) % 2 == 0)


def test_rounding_closed_forms_and_saturation():
    assert oracle.double_to_e4m3(448.0) == 0x7E and oracle.double_to_e4m3(-448.0) == 0xFE
    assert oracle.double_to_e4m3(463.99) == 0x7E and oracle.double_to_e4m3(1e9) == 0x7E   # saturates
    assert oracle.double_to_e4m3(2.0 ** -10) == 0x00          # halfway between 0 and 2^-9: even
    assert oracle.double_to_e4m3(3 * 2.0 ** -10) == 0x02      # halfway between codes 1 and 2
    assert oracle.double_to_e4m3(-0.0) == 0x80 and oracle.double_to_e4m3(0.0) == 0x00
    assert oracle.double_to_e4m3(1.0625) == 0x38              # halfway 1 and 1.125: even code 0x38


@pytest.mark.parametrize("M,K", [(1, 128), (5, 3584), (3, 1000)])
def test_activation_quantizer_definition(M, K):
    x = si.activations(M, K, seed=K)
    codes, scales = oracle.quantize_act_fp8(x)
    xf = torch.from_numpy(as_f32(x))
    a = xf.abs().amax(dim=1)
    s = a / torch.tensor(448.0, dtype=torch.float32)
    assert np.array_equal(scales, s.numpy())
    ref = (xf / s[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    # the row maximum lands on +-448
    i = np.argmax(np.abs(as_f32(x)), axis=1)
    assert np.all(codes[np.arange(M), i] & 0x7F == 0x7E)


def test_activation_quantizer_zero_row_and_range():
    x = si.f32_to_bf16_bits(np.array([[0.0] * 128, [-0.0] * 128, [1e-38] + [0.0] * 127], np.float32))
    codes, scales = oracle.quantize_act_fp8(x)
    assert scales[0] == 0 and scales[1] == 0 and np.all(codes[:2] == 0)
    assert codes[2, 0] == 0x7E and scales[2] > 0


def test_weight_ptq_definition_and_error_bound():
    K, N = 384, 48
    w = si.f32_to_bf16_bits((si.rng(3).standard_normal((K, N)) * 0.02).astype(np.float32))
    codes, scales = oracle.quantize_weights_fp8(w)
    wf = torch.from_numpy(as_f32(w))
    s = wf.abs().amax(dim=0) / torch.tensor(448.0, dtype=torch.float32)
    assert np.array_equal(scales, s.numpy())
    assert np.array_equal(codes, (wf / s).T.contiguous().to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    # dequantized within half an E4M3 step: 2^-4 relative for normal codes, 2^-10 s absolute below
    deq = torch_e4m3_value(codes).T * scales.astype(np.float64)
    err = np.abs(deq - as_f32(w).astype(np.float64))
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(as_f32(w)), 2.0 ** -10 * scales))


def test_store_layout_round_trip_and_reader():
    N, K = 32, 256
    codes = si.fp8_codes((N, K), seed=4)
    store = si.pack_fp8_weights(codes)
    assert np.array_equal(si.unpack_fp8_weights(store), codes)
    # one nonzero code at (n, k): the oracle's reader must find it there
    for (n, k) in [(0, 0), (17, 200), (31, 255), (5, 47)]:
        c = np.zeros((N, K), np.uint8)
        c[n, k] = 0x38
        a = np.zeros((1, K), np.uint8)
        a[0, k] = 0x38
        y = oracle.gemm_w8a8(a, np.ones(1, np.float32), si.pack_fp8_weights(c), np.ones(N, np.float32))
        assert y[0, n] == 1.0 and np.count_nonzero(y) == 1


@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (5, 512, 64), (17, 1024, 48)])
def test_gemm_matches_numpy_matmul_of_decoded_operands(M, K, N):
    a = si.fp8_codes((M, K), seed=M)
    w = si.fp8_codes((N, K), seed=N)
    sa = si.rng(5).uniform(0.5, 2, M).astype(np.float32)
    sw = si.rng(6).uniform(1e-4, 1e-3, N).astype(np.float32)
    y = oracle.gemm_w8a8(a, sa, si.pack_fp8_weights(w), sw)
    ref = (torch_e4m3_value(a) @ torch_e4m3_value(w).T) * sa[:, None].astype(np.float64) * sw[None, :].astype(np.float64)
    assert np.allclose(y, ref, rtol=1e-12, atol=0)


def test_gemm_closed_form():
    M, K, N = 2, 256, 32
    a = np.full((M, K), 0x38, np.uint8)          # 1.0
    w = np.full((N, K), 0x40, np.uint8)          # 2.0
    y = oracle.gemm_w8a8(a, np.array([0.5, 3.0], np.float32), si.pack_fp8_weights(w), np.full(N, 0.25, np.float32))
    assert np.array_equal(y, np.outer([0.5 * 0.25 * 2 * K, 3.0 * 0.25 * 2 * K], np.ones(N)))
