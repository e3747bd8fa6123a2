"""GPU parity of the FP8 parent variant (SpecQuant notes: an FP8 variant of the model verifies;
reading: OCP E4M3 with per-token activation and per-column weight scales) against the oracle:
activation codes and scales bit-exact; layer outputs within the bound the FP8 MFMA's own
accumulation allows, over split and unsplit K, partial column blocks, several row tiles and row
blocks, and sampled column tiles of the Qwen2.5-7B-shaped layer the pages evaluate on.

The bound: gfx950's FP8 MFMAs combine products in groups of 8 consecutive k and drop what lies
more than about 2^15 below a group's largest product (measured: 1 x 1 plus seven products of
2^-18 in one group gives exactly 1, with both the 16x16x32 and the 16x16x128 instructions), so
an output may differ from the exact sum by up to MFMA_REL = 2^-12 of the sum of the magnitudes
of its scaled products (the worst measured was 2^-13.4 on full-range random codes), plus the
output's own rounding (half a bfloat16 ulp, 2^-9 relative; fp32 rounding is far below the
1e-6 allowed)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_speculative_decoding_amd as q
import synthetic_inputs as si
from gpu_helpers import DEV, Guarded, assert_close, bf16_dev, cu, note, sample_tiles

pytestmark = pytest.mark.gpu


MFMA_REL = 2.0 ** -12


def dec_abs(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().abs().numpy()


def check_w8a8(got, ref, a, sa, w_nk, sw, bf16, what):
    """|got - ref| <= MFMA_REL * sum_k |s_a a_k s_w w_k| + (2^-8 for bfloat16, 1e-6 for fp32) |ref|."""
    mag = (dec_abs(a) @ dec_abs(w_nk).T) * np.asarray(sa, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    bound = MFMA_REL * mag + (2.0 ** -8 if bf16 else 1e-6) * np.abs(ref) + 1e-30
    bad = np.abs(got - ref) > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside the bound; first at {i}: gpu {got[i]!r} "
                             f"oracle {ref[i]!r} magnitude sum {mag[i]!r}")


def ptq_store(K, N, seed):
    """An FP8 store quantized (by the oracle) from N(0, 0.02^2) bfloat16 weights."""
    w = si.f32_to_bf16_bits((si.rng(seed).standard_normal((K, N)) * 0.02).astype(np.float32))
    codes, scales = oracle.quantize_weights_fp8(w)
    return si.pack_fp8_weights(codes), scales


def gpu_quantize(x):
    M, K = x.shape
    codes = Guarded((M, K), torch.uint8)
    scales = Guarded((M,), torch.float32)
    q.qspec_quantize_act_fp8(bf16_dev(x), codes.t, scales.t)
    codes.check("quantize_act_fp8 codes")
    scales.check("quantize_act_fp8 scales")
    return codes.t, scales.t


def gpu_gemm(a, sa, store, sw, M, out=torch.bfloat16):
    T, G, _ = store.shape
    K, N = G * 128, 16 * T
    y = Guarded((M, N), out, fill=float("nan"))
    nbytes = q.qspec_gemm_w8a8_workspace_bytes(M, K, N)
    ws = Guarded((max(nbytes, 1),), torch.uint8) if nbytes else None
    q.qspec_gemm_w8a8(a, sa, cu(store) if isinstance(store, np.ndarray) else store,
                      cu(sw) if isinstance(sw, np.ndarray) else sw, y.t, ws.t if ws is not None else None)
    y.check("gemm_w8a8 y")
    if ws is not None:
        ws.check("gemm_w8a8 workspace")
    return y.t


@pytest.mark.parametrize("M,K", [(1, 128), (5, 3584), (17, 18944), (80, 4096), (3, 1024)])
def test_quantize_act_fp8_bit_exact(M, K):
    note(f"quantize_act_fp8 M={M} K={K}")
    x = si.activations(M, K, seed=M + K)
    codes, scales = gpu_quantize(x)
    oc, os_ = oracle.quantize_act_fp8(x)
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)


def test_quantize_act_fp8_special_rows():
    """A zero row, a row of negative zeros, tiny (subnormal-range) values, exact midpoints."""
    note("quantize_act_fp8 special rows")
    K = 256
    rows = np.zeros((5, K), np.float32)
    rows[1] = -0.0
    rows[2] = np.linspace(-1e-3, 1e-3, K)
    rows[2, 0] = 1.0                                       # most codes in the subnormal range
    e4 = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = (e4[:-1] + e4[1:]) / 2                           # 126 midpoints, each x / s exact
    rows[3, :126], rows[3, 126] = mids, 448.0
    rows[4, :126], rows[4, 126] = -mids, -448.0
    x = si.f32_to_bf16_bits(rows)
    codes, scales = gpu_quantize(x)
    oc, os_ = oracle.quantize_act_fp8(x)
    assert np.array_equal(scales.cpu().numpy(), os_) and np.array_equal(codes.cpu().numpy(), oc)
    assert np.all(oc[:2] == 0)


# (M, K, N): one/several row tiles and row blocks, odd column-tile counts, split and unsplit K
SHAPES = [(1, 128, 16), (5, 512, 64), (17, 1024, 48), (33, 384, 80), (80, 1280, 160), (100, 256, 32),
          (5, 18944, 112), (64, 4096, 272)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_gemm_w8a8_matches_oracle(M, K, N):
    note(f"gemm_w8a8 M={M} K={K} N={N}")
    store, sw = ptq_store(K, N, seed=K + N)
    x = si.activations(M, K, seed=M)
    a, sa = gpu_quantize(x)
    an, san = oracle.quantize_act_fp8(x)                 # the oracle's own codes feed the oracle
    assert np.array_equal(a.cpu().numpy(), an) and np.array_equal(sa.cpu().numpy(), san)
    ref = oracle.gemm_w8a8(an, san, store, sw)
    w_nk = si.unpack_fp8_weights(store)
    y16 = gpu_gemm(a, sa, store, sw, M).float().cpu().numpy().astype(np.float64)
    check_w8a8(y16, ref, an, san, w_nk, sw, True, "w8a8 bf16")
    y32 = gpu_gemm(a, sa, store, sw, M, torch.float32).cpu().numpy().astype(np.float64)
    check_w8a8(y32, ref, an, san, w_nk, sw, False, "w8a8 f32")
    # on these weights (post-training quantized from N(0, 0.02^2)) the bf16 outputs also meet the
    # rel 1e-2 / abs 1e-3 bar of the shared-INT4 layers
    assert_close(y16, ref, bf16=True, what="w8a8 bf16 vs the INT4 layers' bar")


def test_gemm_w8a8_random_codes_full_range():
    """Codes drawn over the whole finite E4M3 range (products up to 448^2)."""
    note("gemm_w8a8 random codes")
    M, K, N = 9, 2048, 96
    a = si.fp8_codes((M, K), seed=1)
    w = si.fp8_codes((N, K), seed=2)
    sa = si.rng(3).uniform(0.5, 2, M).astype(np.float32)
    sw = si.rng(4).uniform(1e-4, 1e-3, N).astype(np.float32)
    store = si.pack_fp8_weights(w)
    y = gpu_gemm(cu(a), cu(sa), store, sw, M, torch.float32).cpu().numpy().astype(np.float64)
    check_w8a8(y, oracle.gemm_w8a8(a, sa, store, sw), a, sa, w, sw, False, "w8a8 random codes")


def test_gemm_w8a8_rows_do_not_depend_on_m():
    """The reduction order depends on (K, N) only: every row is bit-identical at M = 1, 5, 80."""
    note("gemm_w8a8 batch invariance")
    K, N = 3584, 4608
    ws, wsw = si.fp8_weights_device(K, N, seed=7, device=DEV)
    x = si.activations(80, K, seed=9)
    a, sa = gpu_quantize(x)
    y80 = gpu_gemm(a, sa, ws, wsw, 80, torch.float32).cpu().numpy()
    for M in (1, 5, 17):
        yM = gpu_gemm(a[:M].contiguous(), sa[:M].contiguous(), ws, wsw, M, torch.float32).cpu().numpy()
        assert np.array_equal(yM, y80[:M]), M


@pytest.mark.parametrize("name", ["qkv", "o", "gate_up", "down", "lm_head"])
def test_gemm_w8a8_qwen25_7b_sampled_tiles(name):
    """The Qwen2.5-7B-shaped layer at a verify shape (gamma = 4: M = 5): the whole layer on the GPU,
    eight sampled 16-column tiles against the oracle on the sliced store."""
    K, N = si.QWEN25_7B_PROJ[name]
    note(f"gemm_w8a8 Qwen2.5-7B {name} K={K} N={N} M=5")
    M = 5
    wst, wsc = si.fp8_weights_device(K, N, seed=1, device=DEV)
    x = si.activations(M, K, seed=11)
    a, sa = gpu_quantize(x)
    an, san = oracle.quantize_act_fp8(x)
    assert np.array_equal(a.cpu().numpy(), an) and np.array_equal(sa.cpu().numpy(), san)
    y = gpu_gemm(a, sa, wst, wsc, M, torch.float32).cpu().numpy().astype(np.float64)
    tiles = sample_tiles(N // 16, 32, seed=N)
    sub = wst[torch.from_numpy(tiles).to(DEV)].cpu().numpy()
    cols = (tiles[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)
    ref = oracle.gemm_w8a8(an, san, sub, wsc.cpu().numpy()[cols])
    check_w8a8(y[:, cols], ref, an, san, si.unpack_fp8_weights(sub), wsc.cpu().numpy()[cols], False,
               f"w8a8 {name}")
