"""Host-side checks of the C ABI that need no GPU: the library loads, exports exactly the
entry points include/qspec.h declares, and rejects invalid arguments with the documented
status before launching anything.  The binding rejects host tensors."""
import ctypes
import os
import re

import pytest
import torch

import quantized_speculative_decoding_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qspec.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_HIP, ERR_WS, ERR_ALIGN, ERR_TOO_LARGE = 0, -1, -2, -3, -4, -5, -6, -7
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int|size_t)\s*(qspec_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "qspec_status_string", "qspec_quantize_act", "qspec_gemm_w4a4", "qspec_gemm_w4a16",
        "qspec_gemm_w4a16_workspace_bytes", "qspec_verify_workspace_bytes", "qspec_verify_accept",
        "qspec_kv_overwrite", "qspec_speckv_workspace_bytes", "qspec_speckv_gamma",
        "qspec_attention_workspace_bytes", "qspec_attention", "qspec_quantize_act_fp8",
        "qspec_gemm_w8a8_workspace_bytes", "qspec_gemm_w8a8", "qspec_draft_sample_workspace_bytes",
        "qspec_draft_sample", "qspec_gemm_w4a16_tier", "qspec_gemm_w4a4_tier", "qspec_verify_accept_noalloc",
        "qspec_draft_sample_speckv", "qspec_draft_sample_speckv_workspace_bytes", "qspec_kv_overwrite_fp8",
        "qspec_attention_fp8"])


def test_library_exports_every_declared_symbol_and_nothing_else():
    L = q.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r"\bT (qspec_\w+)", out)))
    assert exported == declared_functions()


def test_status_strings():
    L = q.lib()
    for s in (OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_HIP, ERR_WS, ERR_ALIGN, ERR_TOO_LARGE):
        assert L.qspec_status_string(s)
    assert L.qspec_status_string(-99) == b"unknown status"


def test_quantize_act_validation():
    L = q.lib()
    assert L.qspec_quantize_act(None, 1, 128, FAKE, FAKE, None) == ERR_NULL
    assert L.qspec_quantize_act(FAKE, 0, 128, FAKE, FAKE, None) == ERR_SHAPE
    assert L.qspec_quantize_act(FAKE, 1, 100, FAKE, FAKE, None) == ERR_SHAPE
    assert L.qspec_quantize_act(FAKE, 1, 0, FAKE, FAKE, None) == ERR_SHAPE


def test_gemm_validation():
    L = q.lib()
    args = [FAKE, FAKE, 4, FAKE, FAKE, 256, 64, FAKE, 0, None, None]
    for i in (0, 1, 3, 4, 7):
        bad = list(args)
        bad[i] = None
        assert L.qspec_gemm_w4a4(*bad) == ERR_NULL, i
    for (M, K, N) in [(0, 256, 64), (4, 200, 64), (4, 256, 0), (-1, 256, 64), (4, 64, 64), (4, 256, 40)]:
        assert L.qspec_gemm_w4a4(FAKE, FAKE, M, FAKE, FAKE, K, N, FAKE, 0, None, None) == ERR_SHAPE
    assert L.qspec_gemm_w4a4(FAKE, FAKE, 4, FAKE, FAKE, 256, 64, FAKE, 7, None, None) == ERR_UNSUPPORTED
    assert L.qspec_gemm_w4a16(None, 4, FAKE, FAKE, 256, 64, FAKE, 0, None, 0, None) == ERR_NULL
    assert L.qspec_gemm_w4a16(FAKE, 4, FAKE, None, 256, 64, FAKE, 0, None, 0, None) == ERR_NULL
    assert L.qspec_gemm_w4a16(FAKE, 4, FAKE, FAKE, 129, 64, FAKE, 0, None, 0, None) == ERR_SHAPE
    assert L.qspec_gemm_w4a16(FAKE, 4, FAKE, FAKE, 256, 72, FAKE, 0, None, 0, None) == ERR_SHAPE
    assert L.qspec_gemm_w4a16(FAKE, 4, FAKE, FAKE, 256, 64, FAKE, 2, None, 0, None) == ERR_UNSUPPORTED
    # split-K verify shapes need a workspace; decode shapes need none
    assert L.qspec_gemm_w4a16_workspace_bytes(4, 4096, 4096) == 0
    # decode tier up to M = 32 for a 4096 x 4096 projection, verify tier (split K) above it
    assert L.qspec_gemm_w4a16_workspace_bytes(32, 4096, 4096) == 0
    assert L.qspec_gemm_w4a16_workspace_bytes(33, 4096, 4096) == 6 * 33 * 4096 * 4
    assert L.qspec_gemm_w4a16_workspace_bytes(20, 14336, 4096) == 8 * 20 * 4096 * 4
    need = L.qspec_gemm_w4a16_workspace_bytes(80, 4096, 4096)
    assert need >= 80 * 4096 * 4 * 2
    assert L.qspec_gemm_w4a16(FAKE, 80, FAKE, FAKE, 4096, 4096, FAKE, 0, None, 0, None) == ERR_WS
    assert L.qspec_gemm_w4a16(FAKE, 80, FAKE, FAKE, 4096, 4096, FAKE, 0, FAKE, need - 1, None) == ERR_WS
    assert L.qspec_gemm_w4a16_workspace_bytes(80, 4096, 70) == 0
    # verify tier past 80 rows (row blocks): its own split count
    assert L.qspec_gemm_w4a16_workspace_bytes(96, 32768, 512) == 16 * 96 * 512 * 4
    assert L.qspec_gemm_w4a16_workspace_bytes(128, 14336, 4096) == 8 * 128 * 4096 * 4
    # large tier: K is split only for few 256-column blocks and long K
    assert L.qspec_gemm_w4a16_workspace_bytes(1280, 8192, 57344) == 0
    assert L.qspec_gemm_w4a16_workspace_bytes(1280, 28672, 8192) == 4 * 1280 * 8192 * 4
    assert L.qspec_gemm_w4a16_workspace_bytes(600, 32768, 512) == 8 * 600 * 512 * 4
    assert L.qspec_gemm_w4a16(FAKE, 1280, FAKE, FAKE, 28672, 8192, FAKE, 0, None, 0, None) == ERR_WS


def test_verify_validation_and_workspace_sizes():
    L = q.lib()
    ws = L.qspec_verify_workspace_bytes(0, 32, 4, 128256)
    assert ws > 0 and L.qspec_verify_workspace_bytes(1, 32, 4, 128256) > ws
    assert L.qspec_verify_workspace_bytes(2, 1, 1, 10) == 0
    assert L.qspec_verify_workspace_bytes(0, 0, 1, 10) == 0
    assert L.qspec_verify_workspace_bytes(0, 1, -1, 10) == 0
    # greedy needs target, tokens (gamma > 0), outputs
    assert L.qspec_verify_accept(0, None, None, FAKE, None, None, 1, 4, 100, FAKE, FAKE, FAKE, 1 << 20, None) == ERR_NULL
    assert L.qspec_verify_accept(0, FAKE, None, None, None, None, 1, 4, 100, FAKE, FAKE, FAKE, 1 << 20, None) == ERR_NULL
    # sampling additionally needs draft logits, u_accept and u_resample
    assert L.qspec_verify_accept(1, FAKE, None, FAKE, FAKE, FAKE, 1, 4, 100, FAKE, FAKE, FAKE, 1 << 20, None) == ERR_NULL
    assert L.qspec_verify_accept(1, FAKE, FAKE, FAKE, FAKE, None, 1, 4, 100, FAKE, FAKE, FAKE, 1 << 20, None) == ERR_NULL
    assert L.qspec_verify_accept(3, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 100, FAKE, FAKE, FAKE, 1 << 20, None) == ERR_UNSUPPORTED
    assert L.qspec_verify_accept(0, FAKE, None, FAKE, None, None, 0, 4, 100, FAKE, FAKE, FAKE, 1 << 20, None) == ERR_SHAPE
    assert L.qspec_verify_accept(0, FAKE, None, FAKE, None, None, 1, 4, 0, FAKE, FAKE, FAKE, 1 << 20, None) == ERR_SHAPE
    need = L.qspec_verify_workspace_bytes(0, 2, 3, 5000)
    assert L.qspec_verify_accept(0, FAKE, None, FAKE, None, None, 2, 3, 5000, FAKE, FAKE, FAKE, need - 1, None) == ERR_WS
    assert L.qspec_verify_accept(0, FAKE, None, FAKE, None, None, 2, 3, 5000, FAKE, FAKE, None, need, None) == ERR_WS


def test_kv_overwrite_validation():
    L = q.lib()
    assert L.qspec_kv_overwrite(None, FAKE, FAKE, FAKE, 1, 1, 1, 8, 8, 2, None) == ERR_NULL
    assert L.qspec_kv_overwrite(FAKE, FAKE, FAKE, None, 1, 1, 1, 8, 8, 2, None) == ERR_NULL
    # the last case: 64 x 1024 x 2 x 64 x 5 x 128 = 5.4e9 staging elements, past the 32-bit indices
    for (Lx, B, H, T, D, g) in [(0, 1, 1, 8, 8, 2), (1, 1, 1, 8, 0, 2), (1, 1, 1, 2, 8, 2), (1, 1, 1, 8, 8, -1),
                                (64, 1024, 64, 4096, 128, 4)]:
        assert L.qspec_kv_overwrite(FAKE, FAKE, FAKE, FAKE, Lx, B, H, T, D, g, None) == ERR_SHAPE


def test_binding_rejects_host_tensors():
    x = torch.zeros((2, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device"):
        q.qspec_quantize_act(x, torch.zeros((2, 128), dtype=torch.uint8), torch.zeros((2, 2)))


def test_alignment_validation():
    L = q.lib()
    odd = ctypes.c_void_p(0x1001)
    assert L.qspec_quantize_act(odd, 1, 128, FAKE, FAKE, None) == ERR_ALIGN
    assert L.qspec_gemm_w4a16(FAKE, 4, ctypes.c_void_p(0x1008), FAKE, 256, 64, FAKE, 0, None, 0, None) == ERR_ALIGN
    assert L.qspec_gemm_w4a4(FAKE, odd, 4, FAKE, FAKE, 256, 64, FAKE, 1, None, None) == ERR_ALIGN
    # GEMM outputs are written with 16-byte stores
    assert L.qspec_gemm_w4a16(FAKE, 4, FAKE, FAKE, 256, 64, ctypes.c_void_p(0x1008), 0, None, 0, None) == ERR_ALIGN
    assert L.qspec_gemm_w4a4(FAKE, FAKE, 4, FAKE, FAKE, 256, 64, ctypes.c_void_p(0x1004), 1, None, None) == ERR_ALIGN
    need = L.qspec_verify_workspace_bytes(0, 2, 3, 5000)
    assert L.qspec_verify_accept(0, FAKE, None, FAKE, None, None, 2, 3, 5000, FAKE, FAKE,
                                 ctypes.c_void_p(0x1004), need, None) == ERR_ALIGN
    assert L.qspec_kv_overwrite(odd, FAKE, FAKE, FAKE, 1, 1, 1, 8, 8, 2, None) == ERR_ALIGN


def test_speckv_validation():
    L = q.lib()
    L.qspec_speckv_gamma.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_float] + \
        [ctypes.c_void_p] * 4 + [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p]
    L.qspec_speckv_workspace_bytes.restype = ctypes.c_size_t
    need = L.qspec_speckv_workspace_bytes(16, 128256)
    assert need > 0 and L.qspec_speckv_workspace_bytes(0, 10) == 0 and L.qspec_speckv_workspace_bytes(1, 0) == 0

    def call(**kw):
        a = dict(logits=FAKE, R=16, V=128256, qf=0.0, w1=FAKE, b1=FAKE, w2=FAKE, b2=FAKE, g=8, feat=None,
                 out=FAKE, ws=FAKE, nbytes=need)
        a.update(kw)
        return L.qspec_speckv_gamma(a["logits"], a["R"], a["V"], a["qf"], a["w1"], a["b1"], a["w2"], a["b2"],
                                    a["g"], a["feat"], a["out"], a["ws"], a["nbytes"], None)
    for k in ("logits", "w1", "b1", "w2", "b2", "out"):
        assert call(**{k: None}) == ERR_NULL, k
    assert call(R=0) == ERR_SHAPE and call(V=0) == ERR_SHAPE
    assert call(g=-1) == ERR_SHAPE and call(g=64) == ERR_SHAPE
    assert call(ws=None) == ERR_WS and call(nbytes=need - 1) == ERR_WS
    assert call(feat=ctypes.c_void_p(0x1004)) == ERR_ALIGN


def test_attention_validation():
    L = q.lib()
    need = q.qspec_attention_workspace_bytes(16, 5, 32, 8, 4096)
    # chunk partials of 1024 positions: (max, sum, 128 outputs) fp32 per (query row, chunk)
    assert need >= 16 * 5 * 32 * 4 * (2 + 128) * 4
    assert q.qspec_attention_workspace_bytes(0, 1, 1, 1, 8) == 0
    assert q.qspec_attention_workspace_bytes(1, 65, 1, 1, 8) == 0          # Q above the limit
    assert q.qspec_attention_workspace_bytes(1, 1, 6, 4, 8) == 0           # Hq not a multiple of Hkv
    assert q.qspec_attention_workspace_bytes(65536, 1, 1, 1, 8) == 0       # B * Hkv above 65535

    def call(**kw):
        a = dict(q=FAKE, cache=FAKE, pos=FAKE, B=16, Q=5, Hq=32, Hkv=8, T=4096, D=128, scale=0.088, out=FAKE,
                 ws=FAKE, nbytes=need)
        a.update(kw)
        return L.qspec_attention(a["q"], a["cache"], a["pos"], a["B"], a["Q"], a["Hq"], a["Hkv"], a["T"], a["D"],
                                 a["scale"], a["out"], a["ws"], a["nbytes"], None)
    for k in ("q", "cache", "pos", "out"):
        assert call(**{k: None}) == ERR_NULL, k
    for kw in (dict(B=0), dict(Q=0), dict(Hq=0), dict(Hkv=0), dict(T=0), dict(D=64), dict(Q=65), dict(Hkv=6)):
        assert call(**kw) == ERR_SHAPE, kw
    assert call(ws=None) == ERR_WS and call(nbytes=need - 1) == ERR_WS
    assert call(q=ctypes.c_void_p(0x1008)) == ERR_ALIGN and call(cache=ctypes.c_void_p(0x1002)) == ERR_ALIGN
    assert call(ws=ctypes.c_void_p(0x1004)) == ERR_ALIGN


def test_fp8_validation():
    L = q.lib()
    assert L.qspec_quantize_act_fp8(None, 4, 256, FAKE, FAKE, None) == ERR_NULL
    assert L.qspec_quantize_act_fp8(FAKE, 0, 256, FAKE, FAKE, None) == ERR_SHAPE
    assert L.qspec_quantize_act_fp8(FAKE, 4, 200, FAKE, FAKE, None) == ERR_SHAPE
    assert L.qspec_quantize_act_fp8(FAKE, 4, 256, ctypes.c_void_p(0x1008), FAKE, None) == ERR_ALIGN
    # splits depend on (K, N) only: none for a wide N, some for narrow N with long K
    assert q.qspec_gemm_w8a8_workspace_bytes(5, 3584, 152064) == 0
    need = q.qspec_gemm_w8a8_workspace_bytes(5, 18944, 3584)
    assert need > 0 and need % (5 * 3584 * 4) == 0 and need // (5 * 3584 * 4) <= 16
    assert q.qspec_gemm_w8a8_workspace_bytes(80, 18944, 3584) == need // 5 * 80
    assert q.qspec_gemm_w8a8_workspace_bytes(0, 256, 64) == 0
    assert q.qspec_gemm_w8a8_workspace_bytes(1, 65536, 65536) == 0          # K * N = 2^32

    def call(**kw):
        a = dict(a=FAKE, sa=FAKE, M=5, w=FAKE, sw=FAKE, K=18944, N=3584, y=FAKE, dt=0, ws=FAKE, nbytes=need)
        a.update(kw)
        return L.qspec_gemm_w8a8(a["a"], a["sa"], a["M"], a["w"], a["sw"], a["K"], a["N"], a["y"], a["dt"], a["ws"],
                                 a["nbytes"], None)
    for k in ("a", "sa", "w", "sw", "y"):
        assert call(**{k: None}) == ERR_NULL, k
    for kw in (dict(M=0), dict(K=200), dict(N=40), dict(K=65536, N=65536)):
        assert call(**kw) == ERR_SHAPE, kw
    assert call(dt=5) == ERR_UNSUPPORTED
    assert call(ws=None) == ERR_WS and call(nbytes=need - 1) == ERR_WS
    assert call(w=ctypes.c_void_p(0x1008)) == ERR_ALIGN and call(ws=ctypes.c_void_p(0x1010)) == ERR_ALIGN


def test_draft_sample_validation():
    L = q.lib()
    need = q.qspec_draft_sample_workspace_bytes(1, 16, 128256)
    assert need >= q.qspec_verify_workspace_bytes(1, 16, 0, 128256) + 16 * 4
    assert q.qspec_draft_sample_workspace_bytes(2, 16, 100) == 0 and q.qspec_draft_sample_workspace_bytes(0, 0, 9) == 0

    def call(**kw):
        a = dict(mode=1, logits=FAKE, B=16, V=128256, ld=4 * 128256, u=FAKE, tok=FAKE, lt=4, ws=FAKE, nbytes=need)
        a.update(kw)
        return L.qspec_draft_sample(a["mode"], a["logits"], a["B"], a["V"], a["ld"], a["u"], a["tok"], a["lt"],
                                    a["ws"], a["nbytes"], None)
    assert call(mode=3) == ERR_UNSUPPORTED
    for k in ("logits", "u", "tok"):
        assert call(**{k: None}) == ERR_NULL, k
    for kw in (dict(B=0), dict(V=0), dict(ld=128255), dict(lt=0)):
        assert call(**kw) == ERR_SHAPE, kw
    assert call(ws=None) == ERR_WS and call(nbytes=need - 1) == ERR_WS
    assert call(tok=ctypes.c_void_p(0x1002)) == ERR_ALIGN


# Batch tiers: (K, N) -> the last M of the W4A16 decode tier and of the verify tier, from the
# rules the header states.
W4A16_DECODE_LAST = [
    (4096, 4096, 32, 384),      # 256 workgroups, K * N = 4096 * 4096: small projection
    (4096, 6144, 32, 384),      # 192 workgroups (two tiles each), K * N = 4096 * 6144
    (3584, 4608, 12, 384),      # Qwen qkv: 288 one-tile workgroups, more than 256
    (14336, 4096, 8, 384),      # Llama down: long K over one-tile workgroups
    (18944, 3584, 8, 256),      # Qwen down
    (12160, 4096, 8, 384),     # K just below 12288
    (28672, 8192, 8, 160),     # 70B down: two-tile workgroups; 32 blocks x 4 splits per row block
    (4096, 28672, 12, 160),     # 896 workgroups; 112 large-tier blocks per row block
    (3584, 152064, 24, 80),     # vocabulary head: four tiles per workgroup
    (4096, 128256, 24, 80),
    (512, 512, 32, 384),
    (8192, 57344, 12, 80),     # 70B gate+up: 224 blocks per row block
    (3584, 37888, 20, 80),     # Qwen gate+up: 296 verify workgroups, the second generation nearly idle
]


def _large_splits(K, N):
    blocks, G, S = -(-N // 256), K // 128, 1
    while S < 8 and 2 * S * blocks <= 128 and G // (2 * S) >= 32:
        S *= 2
    return S


def _verify_last(K, N):
    P = -(-N // 256) * _large_splits(K, N)
    return 384 if P <= 32 else 256 if P <= 64 else 160 if P <= 128 else 80


def _verify_splits(K, N):
    blocks, G = -(-N // 128), K // 128
    return 1 if blocks >= 192 else max(1, min(256 // blocks, 16, G // 5))


def _decode_last(K, N):
    T = N // 16
    nt = 4 if T >= 4096 else 2 if T >= 384 else 1
    wgs = -(-T // nt)
    if nt == 4:
        return 24
    if wgs <= 256 and K * N <= 4096 * 6144:
        return 32
    if nt == 1:
        return 8 if K >= 8192 else 12
    if K >= 12288:
        return 8
    w1 = -(-N // 128) * _verify_splits(K, N)
    return 20 if 4 * w1 < 3 * 256 * -(-w1 // 256) else 12


@pytest.mark.parametrize("K,N,last,vlast", W4A16_DECODE_LAST)
def test_w4a16_tier_boundaries(K, N, last, vlast):
    D, V = _decode_last(K, N), _verify_last(K, N)
    assert D == last and V == vlast
    for M, tier, lo, hi in [(1, 0, 1, D), (D, 0, 1, D), (D + 1, 1, D + 1, V), (80, 1, D + 1, V), (V, 1, D + 1, V),
                            (V + 1, 2, V + 1, 2 ** 31 - 1), (1280, 2, V + 1, 2 ** 31 - 1)]:
        assert q.qspec_gemm_w4a16_tier(M, K, N) == (tier, lo, hi), (M, K, N)
    # the workspace follows the tiers: none in the decode tier
    assert q.qspec_gemm_w4a16_workspace_bytes(D, K, N) == 0


def test_w4a16_tier_rule_on_the_workload_shapes():
    """The header's rule, on the Llama-3-8B and Qwen2.5-7B projections and heads."""
    assert _decode_last(4096, 4096) == 32 and _decode_last(4096, 6144) == 32
    assert _decode_last(3584, 4608) == 12 and _decode_last(3584, 3584) == 32
    assert _decode_last(14336, 4096) == 8 and _decode_last(18944, 3584) == 8
    assert _decode_last(4096, 28672) == 12 and _decode_last(3584, 37888) == 20
    assert _decode_last(3584, 152064) == 24


def test_w4a4_tier_boundaries():
    for K, N in [(4096, 4096), (4096, 28672), (3584, 152064), (128, 16)]:
        for M, tier, lo, hi in [(1, 0, 1, 16), (16, 0, 1, 16), (17, 1, 17, 64), (64, 1, 17, 64),
                                (65, 2, 65, 2 ** 31 - 1), (256, 2, 65, 2 ** 31 - 1)]:
            assert q.qspec_gemm_w4a4_tier(M, K, N) == (tier, lo, hi)


def test_tier_validation():
    L = q.lib()
    lo, hi = ctypes.c_int32(), ctypes.c_int32()
    assert L.qspec_gemm_w4a16_tier(4, 256, 64, None, ctypes.byref(hi)) == ERR_NULL
    assert L.qspec_gemm_w4a4_tier(4, 256, 64, ctypes.byref(lo), None) == ERR_NULL
    for (M, K, N) in [(0, 256, 64), (4, 200, 64), (4, 256, 40)]:
        assert L.qspec_gemm_w4a16_tier(M, K, N, ctypes.byref(lo), ctypes.byref(hi)) == ERR_SHAPE
        assert L.qspec_gemm_w4a4_tier(M, K, N, ctypes.byref(lo), ctypes.byref(hi)) == ERR_SHAPE


def test_gemm_32bit_range_limits():
    """Shapes whose activation rows or weight-tile range would overflow a 32-bit buffer range
    are rejected before any launch (QSPEC_ERR_SHAPE), not silently computed from zeros."""
    L = q.lib()
    # W4A16: min(M, 128) * K * 2 < 2^32 and K * 8 < 2^32
    K_big = 2 ** 24                  # 128 rows * 2^24 * 2 = 2^32
    assert L.qspec_gemm_w4a16(FAKE, 128, FAKE, FAKE, K_big, 16, FAKE, 0, FAKE, 1 << 40, None) == ERR_SHAPE
    assert L.qspec_gemm_w4a16(FAKE, 1280, FAKE, FAKE, K_big, 16, FAKE, 0, FAKE, 1 << 40, None) == ERR_SHAPE
    assert L.qspec_gemm_w4a16_workspace_bytes(128, K_big, 16) == 0
    assert L.qspec_gemm_w4a16(FAKE, 32, FAKE, FAKE, 2 ** 26, 16, FAKE, 0, FAKE, 1 << 40, None) == ERR_SHAPE
    # just inside the range: validation passes up to the alignment check (FAKE is aligned, so
    # the call would launch; use a misaligned output to stop it before that)
    odd = ctypes.c_void_p(0x1002)
    assert L.qspec_gemm_w4a16(FAKE, 127, FAKE, FAKE, K_big, 16, odd, 0, FAKE, 1 << 40, None) == ERR_ALIGN
    # W4A4: min(M, 64) * K / 2 < 2^32 and K * 8 < 2^32
    assert L.qspec_gemm_w4a4(FAKE, FAKE, 64, FAKE, FAKE, 2 ** 27, 16, FAKE, 0, None, None) == ERR_SHAPE
    assert L.qspec_gemm_w4a4(FAKE, FAKE, 256, FAKE, FAKE, 2 ** 27, 16, FAKE, 0, None, None) == ERR_SHAPE
    assert L.qspec_gemm_w4a4(FAKE, FAKE, 1, FAKE, FAKE, 2 ** 29, 16, FAKE, 0, None, None) == ERR_SHAPE
    assert L.qspec_gemm_w4a4(FAKE, FAKE, 63, FAKE, FAKE, 2 ** 27, 16, odd, 0, None, None) == ERR_ALIGN


def test_verify_accept_noalloc_validation():
    """The scratch-buffer verification rejects what qspec_verify_accept rejects, and problems whose
    workspace would exceed its fixed 1 MiB scratch, before touching the GPU."""
    L = q.lib()
    g = [0, FAKE, None, FAKE, None, None, 4, 4, 1000, FAKE, FAKE, None]
    assert L.qspec_verify_accept_noalloc(5, *g[1:]) == ERR_UNSUPPORTED
    bad = list(g); bad[1] = None
    assert L.qspec_verify_accept_noalloc(*bad) == ERR_NULL
    bad = list(g); bad[3] = None
    assert L.qspec_verify_accept_noalloc(*bad) == ERR_NULL
    s = [1, FAKE, FAKE, FAKE, FAKE, None, 4, 4, 1000, FAKE, FAKE, None]
    assert L.qspec_verify_accept_noalloc(*s) == ERR_NULL            # sampling needs u_resample
    bad = list(g); bad[6] = 0
    assert L.qspec_verify_accept_noalloc(*bad) == ERR_SHAPE
    cap = 1 << 20
    # largest B that fits the scratch at gamma = 4, V = 128256, sampling; one more does not
    fits = [B for B in (32, 64, 128, 256, 512, 1024)
            if L.qspec_verify_workspace_bytes(1, B, 4, 128256) <= cap]
    assert 32 in fits
    too_big = next(B for B in (64, 128, 256, 512, 1024, 4096) if L.qspec_verify_workspace_bytes(1, B, 4, 128256) > cap)
    s = [1, FAKE, FAKE, FAKE, FAKE, FAKE, too_big, 4, 128256, FAKE, FAKE, None]
    assert L.qspec_verify_accept_noalloc(*s) == ERR_TOO_LARGE
    odd = ctypes.c_void_p(0x1002)
    s = [1, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 4, 128256, odd, FAKE, None]
    assert L.qspec_verify_accept_noalloc(*s) == ERR_ALIGN


def test_draft_sample_speckv_validation():
    """The shared-statistics head + controller checks the arguments of both calls it combines and
    needs the head's workspace plus the controller's entropies (sampling) or its whole layout."""
    L = q.lib()
    f = ctypes.c_float(0.0)
    for mode in (0, 1):
        ws = L.qspec_draft_sample_speckv_workspace_bytes(mode, 16, 128256)
        assert ws >= L.qspec_draft_sample_workspace_bytes(mode, 16, 128256)
    assert (L.qspec_draft_sample_speckv_workspace_bytes(0, 16, 128256) - L.qspec_draft_sample_workspace_bytes(0, 16, 128256)
            >= L.qspec_speckv_workspace_bytes(16, 128256))
    assert L.qspec_draft_sample_speckv_workspace_bytes(2, 16, 1000) == 0
    assert L.qspec_draft_sample_speckv_workspace_bytes(1, 0, 1000) == 0
    need = L.qspec_draft_sample_speckv_workspace_bytes(1, 4, 1000)
    args = [1, FAKE, 4, 1000, 1000, FAKE, FAKE, 1, f, FAKE, FAKE, FAKE, FAKE, 4, None, FAKE, FAKE, need, None]
    bad = list(args); bad[0] = 3
    assert L.qspec_draft_sample_speckv(*bad) == ERR_UNSUPPORTED
    for i in (1, 5, 6, 9, 10, 11, 12, 15):
        bad = list(args); bad[i] = None
        assert L.qspec_draft_sample_speckv(*bad) == ERR_NULL, i
    g = list(args); g[0] = 0; g[5] = None; g[17] = L.qspec_draft_sample_speckv_workspace_bytes(0, 4, 1000) - 1
    assert L.qspec_draft_sample_speckv(*g) == ERR_WS                  # greedy: u may be NULL
    for i, v in ((2, 0), (3, 0), (4, 999), (7, 0), (13, -1), (13, 64)):
        bad = list(args); bad[i] = v
        assert L.qspec_draft_sample_speckv(*bad) == ERR_SHAPE, (i, v)
    bad = list(args); bad[17] = need - 1
    assert L.qspec_draft_sample_speckv(*bad) == ERR_WS
    bad = list(args); bad[14] = ctypes.c_void_p(0x1004)              # features are f64
    assert L.qspec_draft_sample_speckv(*bad) == ERR_ALIGN


def test_quantized_kv_validation():
    """The FP8 cache calls check what their bfloat16 counterparts check, plus the head dimension
    (128) of the overwrite and the alignment of codes and scales."""
    L = q.lib()
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 3, 2, 16, 128, 4, None]
    for i in range(5):
        bad = list(ok); bad[i] = None
        assert L.qspec_kv_overwrite_fp8(*bad) == ERR_NULL, i
    for i, v in ((5, 0), (6, 0), (7, 0), (8, 0), (9, 64), (10, -1), (10, 16)):
        bad = list(ok); bad[i] = v
        assert L.qspec_kv_overwrite_fp8(*bad) == ERR_SHAPE, (i, v)
    bad = list(ok); bad[1] = ctypes.c_void_p(0x1002)
    assert L.qspec_kv_overwrite_fp8(*bad) == ERR_ALIGN
    bad = list(ok); bad[0] = ctypes.c_void_p(0x1001)
    assert L.qspec_kv_overwrite_fp8(*bad) == ERR_ALIGN
    need = L.qspec_attention_workspace_bytes(2, 1, 8, 2, 100)
    f = ctypes.c_float(0.088)
    ok = [FAKE, FAKE, FAKE, FAKE, 2, 1, 8, 2, 100, 128, f, FAKE, FAKE, need, None]
    for i in (0, 1, 2, 3, 11):
        bad = list(ok); bad[i] = None
        assert L.qspec_attention_fp8(*bad) == ERR_NULL, i
    for i, v in ((4, 0), (9, 64), (6, 7), (5, 65)):
        bad = list(ok); bad[i] = v
        assert L.qspec_attention_fp8(*bad) == ERR_SHAPE, (i, v)
    bad = list(ok); bad[13] = need - 1
    assert L.qspec_attention_fp8(*bad) == ERR_WS
    bad = list(ok); bad[1] = ctypes.c_void_p(0x1008)
    assert L.qspec_attention_fp8(*bad) == ERR_ALIGN
    bad = list(ok); bad[2] = ctypes.c_void_p(0x1002)
    assert L.qspec_attention_fp8(*bad) == ERR_ALIGN
