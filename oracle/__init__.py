"""Plain CPU oracle for the shared-INT4 speculative-decoding hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never touches it, and it shares no code
with them.

The arithmetic lives in ``qspec_oracle.c`` (scalar loops, fp64/int64); this
module only marshals numpy arrays into it.  ``build()`` compiles the C file with
gcc; ``_lib()`` builds it on first use when no built copy exists.

Every function follows a definition on the QSPEC study-notes page ("QSPEC 논문
요점 정리", notes on "QSPEC: Speculative Decoding with Complementary Quantization
Schemes"); the C source cites the section for each.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

GROUP = 128
_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qspec_oracle.c")
_SO = os.path.join(_HERE, "libqspec_oracle.so")
_LIB = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-fexcess-precision=standard", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.orc_fp16_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_fp16_to_double.restype = ctypes.c_double
        lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_double.restype = ctypes.c_double
        lib.orc_double_to_bf16.argtypes = [ctypes.c_double]
        lib.orc_double_to_bf16.restype = ctypes.c_uint16
        lib.orc_dequant_one.argtypes = [ctypes.c_uint16, ctypes.c_int, ctypes.c_int]
        lib.orc_dequant_one.restype = ctypes.c_uint16
        lib.orc_dequant.argtypes = [P, P, I, I, P]
        lib.orc_gemm_w4a16.argtypes = [P, I, P, P, I, I, P]
        lib.orc_quantize_act.argtypes = [P, I, I, P, P]
        lib.orc_gemm_w4a4.argtypes = [P, P, I, P, P, I, I, P, P]
        lib.orc_verify_greedy.argtypes = [P, P, I, I, I, P, P]
        lib.orc_verify_sample.argtypes = [P, P, P, P, P, I, I, I, P, P, P]
        lib.orc_kv_overwrite.argtypes = [P, P, P, P, I, I, I, I, I, I]
        lib.orc_speckv_gamma.argtypes = [P, I, I, ctypes.c_float, P, P, P, P, I, P, P, P]
        lib.orc_attention.argtypes = [P, P, P, I, I, I, I, I, I, ctypes.c_float, P]
        lib.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_to_double.restype = ctypes.c_double
        lib.orc_double_to_e4m3.argtypes = [ctypes.c_double]
        lib.orc_double_to_e4m3.restype = ctypes.c_uint8
        lib.orc_quantize_act_fp8.argtypes = [P, I, I, P, P]
        lib.orc_kv_overwrite_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, I]
        lib.orc_attention_fp8.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_float, P]
        lib.orc_quantize_weights_fp8.argtypes = [P, I, I, P, P]
        lib.orc_gemm_w8a8.argtypes = [P, P, I, P, P, I, I, P]
        for name in ("orc_dequant", "orc_gemm_w4a16", "orc_quantize_act", "orc_gemm_w4a4",
                     "orc_verify_greedy", "orc_verify_sample", "orc_kv_overwrite", "orc_speckv_gamma",
                     "orc_attention"):
            getattr(lib, name).restype = None
        _LIB = lib
    return _LIB


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


# ---- scalar format helpers (exposed so the tests can pin them) -------------

def fp16_to_double(bits: int) -> float:
    return _lib().orc_fp16_to_double(int(bits))


def bf16_to_double(bits: int) -> float:
    return _lib().orc_bf16_to_double(int(bits))


def double_to_bf16(v: float) -> int:
    return int(_lib().orc_double_to_bf16(float(v)))


def dequant_one(scale_bits: int, w: int, z: int) -> int:
    return int(_lib().orc_dequant_one(int(scale_bits), int(w), int(z)))


# ---- the hot-path operations --------------------------------------------------

def _weights(codes, meta):
    """Shared weight store: codes u8 [N/16][K/128][1024], meta u32 [N/16][K/128][16]."""
    codes = _c(codes, np.uint8)
    meta = _c(meta, np.uint32)
    T, G, blk = codes.shape
    assert blk == 1024 and meta.shape == (T, G, 16)
    return codes, meta, G * GROUP, 16 * T


def dequant(codes, meta):
    """W_hat = bf16(s * (w - z)) for every (n, k); returns u16 [N][K]."""
    codes, meta, K, N = _weights(codes, meta)
    out = np.empty((N, K), np.uint16)
    _lib().orc_dequant(_p(codes), _p(meta), K, N, _p(out))
    return out


def gemm_w4a16(x, codes, meta):
    """y = X W_hat in fp64; x u16 bf16 [M][K]; returns f64 [M][N]."""
    codes, meta, K, N = _weights(codes, meta)
    x = _c(x, np.uint16)
    M = x.shape[0]
    assert x.shape == (M, K)
    y = np.empty((M, N), np.float64)
    _lib().orc_gemm_w4a16(_p(x), M, _p(codes), _p(meta), K, N, _p(y))
    return y


def quantize_act(x):
    """Per-(token, group) symmetric INT4; returns (codes u8 [M][K/2], scales f32 [M][K/128])."""
    x = _c(x, np.uint16)
    M, K = x.shape
    assert K % GROUP == 0
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.empty((M, K // GROUP), np.float32)
    _lib().orc_quantize_act(_p(x), M, K, _p(codes), _p(scales))
    return codes, scales


def gemm_w4a4(a_codes, a_scales, codes, meta, want_dots: bool = True):
    """Returns (y f64 [M][N], D i64 [K/128][M][N] or None)."""
    codes, meta, K, N = _weights(codes, meta)
    a_codes = _c(a_codes, np.uint8)
    a_scales = _c(a_scales, np.float32)
    M = a_codes.shape[0]
    assert a_codes.shape == (M, K // 2) and a_scales.shape == (M, K // GROUP)
    y = np.empty((M, N), np.float64)
    D = np.empty((K // GROUP, M, N), np.int64) if want_dots else None
    _lib().orc_gemm_w4a4(_p(a_codes), _p(a_scales), M, _p(codes), _p(meta), K, N, _p(D), _p(y))
    return y, D


def verify_greedy(target, draft_tokens):
    """target f32 [B][g+1][V], draft_tokens i32 [B][g] -> (accept i32 [B], out i32 [B][g+1])."""
    target = _c(target, np.float32)
    B, g1, V = target.shape
    gamma = g1 - 1
    d = _c(draft_tokens, np.int32).reshape(B, gamma)
    acc = np.empty(B, np.int32)
    out = np.empty((B, g1), np.int32)
    _lib().orc_verify_greedy(_p(target), _p(d), B, gamma, V, _p(acc), _p(out))
    return acc, out


def verify_sample(target, draft, draft_tokens, u, v, with_diag: bool = True):
    """Speculative-sampling verification.  Returns (accept, out, diag)."""
    target = _c(target, np.float32)
    B, g1, V = target.shape
    gamma = g1 - 1
    draft = _c(draft, np.float32).reshape(B, gamma, V)
    d = _c(draft_tokens, np.int32).reshape(B, gamma)
    u = _c(u, np.float32).reshape(B, gamma)
    v = _c(v, np.float32).reshape(B)
    acc = np.empty(B, np.int32)
    out = np.empty((B, g1), np.int32)
    diag = np.empty((B, g1), np.float64) if with_diag else None
    _lib().orc_verify_sample(_p(target), _p(draft), _p(d), _p(u), _p(v), B, gamma, V,
                             _p(acc), _p(out), _p(diag))
    return acc, out, diag


def speckv_gamma(logits, quant_feature, w1, b1, w2, b2):
    """Draft statistics and the adaptive-gamma controller (SpecKV notes).
    logits f32 [R][V]; w1 [64][3], b1 [64], w2 [G1][64], b2 [G1] (f32).
    Returns (gamma i32 [R], features f64 [R][2] = (confidence, entropy), mlp f64 [R][G1])."""
    logits = _c(logits, np.float32)
    R, V = logits.shape
    w1, b1 = _c(w1, np.float32).reshape(64, 3), _c(b1, np.float32).reshape(64)
    w2 = _c(w2, np.float32)
    G1 = w2.shape[0]
    w2, b2 = w2.reshape(G1, 64), _c(b2, np.float32).reshape(G1)
    gamma = np.empty(R, np.int32)
    feats = np.empty((R, 2), np.float64)
    mlp = np.empty((R, G1), np.float64)
    _lib().orc_speckv_gamma(_p(logits), R, V, float(quant_feature), _p(w1), _p(b1), _p(w2), _p(b2), G1 - 1,
                            _p(feats), _p(gamma), _p(mlp))
    return gamma, feats, mlp


def attention(q, cache, pos, scale):
    """Causal attention of Q query tokens per sequence over one layer of the KV cache.
    q u16 [B][Q][Hq][D] (bf16 bits); cache u16 [B][2][Hkv][T][D]; pos i32 [B]; returns u16
    [B][Q][Hq][D].  Query j of sequence b attends to positions 0 .. min(pos[b] + j, T - 1)."""
    q = _c(q, np.uint16)
    B, Q, Hq, D = q.shape
    cache = _c(cache, np.uint16)
    assert cache.shape[:2] == (B, 2) and cache.shape[4] == D
    Hkv, T = cache.shape[2], cache.shape[3]
    assert Hq % Hkv == 0
    pos = _c(pos, np.int32).reshape(B)
    out = np.empty_like(q)
    _lib().orc_attention(_p(q), _p(cache), _p(pos), B, Q, Hq, Hkv, T, D, float(scale), _p(out))
    return out


def e4m3_to_double(code: int) -> float:
    return _lib().orc_e4m3_to_double(int(code))


def double_to_e4m3(v: float) -> int:
    return int(_lib().orc_double_to_e4m3(float(v)))


def quantize_act_fp8(x):
    """Per-token FP8 (E4M3) activation codes: x u16 bf16 [M][K] -> (codes u8 [M][K], scales f32 [M])."""
    x = _c(x, np.uint16)
    M, K = x.shape
    codes = np.empty((M, K), np.uint8)
    scales = np.empty(M, np.float32)
    _lib().orc_quantize_act_fp8(_p(x), M, K, _p(codes), _p(scales))
    return codes, scales


def quantize_weights_fp8(w):
    """Per-column FP8 post-training quantization: w u16 bf16 [K][N] -> (codes u8 [N][K], scales f32 [N])."""
    w = _c(w, np.uint16)
    K, N = w.shape
    codes = np.empty((N, K), np.uint8)
    scales = np.empty(N, np.float32)
    _lib().orc_quantize_weights_fp8(_p(w), K, N, _p(codes), _p(scales))
    return codes, scales


def gemm_w8a8(a_codes, a_scales, w_store, w_scales):
    """y f64 [M][N] = s_a s_w sum_k dec(a) dec(w); a_codes u8 [M][K], a_scales f32 [M], w_store u8
    [N/16][K/128][2048], w_scales f32 [N]."""
    a_codes = _c(a_codes, np.uint8)
    M, K = a_codes.shape
    a_scales = _c(a_scales, np.float32).reshape(M)
    w_store = _c(w_store, np.uint8)
    T, G, blk = w_store.shape
    assert blk == 2048 and G * 128 == K
    N = 16 * T
    w_scales = _c(w_scales, np.float32).reshape(N)
    y = np.empty((M, N), np.float64)
    _lib().orc_gemm_w8a8(_p(a_codes), _p(a_scales), M, _p(w_store), _p(w_scales), K, N, _p(y))
    return y


def kv_overwrite(cache, verify_kv, start_pos, accept):
    """In place on ``cache`` (u16 [L][B][2][H][T][D]); verify_kv u16 [L][B][2][H][g+1][D]."""
    assert cache.dtype == np.uint16 and cache.flags["C_CONTIGUOUS"]
    L, B, two, H, T, D = cache.shape
    assert two == 2
    verify_kv = _c(verify_kv, np.uint16)
    gamma = verify_kv.shape[4] - 1
    assert verify_kv.shape == (L, B, 2, H, gamma + 1, D)
    start_pos = _c(start_pos, np.int32).reshape(B)
    accept = _c(accept, np.int32).reshape(B)
    _lib().orc_kv_overwrite(_p(cache), _p(verify_kv), _p(start_pos), _p(accept), L, B, H, T, D,
                            gamma)
    return cache


def kv_overwrite_fp8(codes, scales, verify_kv, start_pos, accept):
    """In place on the FP8 cache (codes u8 [L][B][2][H][T][D], scales f32 [L][B][2][H][T]): rows
    0..A_b of verify_kv (u16 bf16 [L][B][2][H][g+1][D]) quantized per row at start_pos[b] + r."""
    assert codes.dtype == np.uint8 and codes.flags["C_CONTIGUOUS"]
    assert scales.dtype == np.float32 and scales.flags["C_CONTIGUOUS"]
    L, B, two, H, T, D = codes.shape
    assert two == 2 and scales.shape == (L, B, 2, H, T)
    verify_kv = _c(verify_kv, np.uint16)
    gamma = verify_kv.shape[4] - 1
    assert verify_kv.shape == (L, B, 2, H, gamma + 1, D)
    start_pos = _c(start_pos, np.int32).reshape(B)
    accept = _c(accept, np.int32).reshape(B)
    _lib().orc_kv_overwrite_fp8(_p(codes), _p(scales), _p(verify_kv), _p(start_pos), _p(accept), L, B, H, T, D,
                                gamma)
    return codes, scales


def attention_fp8(q, codes, scales, pos, scale):
    """Causal attention over one layer of the FP8 cache: q u16 [B][Q][Hq][D]; codes u8
    [B][2][Hkv][T][D]; scales f32 [B][2][Hkv][T]; returns u16 bf16 [B][Q][Hq][D]."""
    q = _c(q, np.uint16)
    B, Q, Hq, D = q.shape
    codes = _c(codes, np.uint8)
    assert codes.shape[:2] == (B, 2) and codes.shape[4] == D
    Hkv, T = codes.shape[2], codes.shape[3]
    scales = _c(scales, np.float32)
    assert scales.shape == (B, 2, Hkv, T) and Hq % Hkv == 0
    pos = _c(pos, np.int32).reshape(B)
    out = np.empty_like(q)
    _lib().orc_attention_fp8(_p(q), _p(codes), _p(scales), _p(pos), B, Q, Hq, Hkv, T, D, float(scale), _p(out))
    return out

