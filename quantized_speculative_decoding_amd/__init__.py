"""Python binding of libqspec (include/qspec.h): argument marshalling only.

Each function takes torch CUDA tensors, checks dtype / shape / device /
contiguity, and passes raw device pointers, sizes and the current HIP stream to
the C entry point of the same name.  Every step of the computation runs in the
library's HIP kernels; there is no fallback.  A missing or unloadable library
raises at first use.

Tensor conventions (contiguous):
  activations / KV   torch.bfloat16, row-major
  weight codes       torch.uint8 [N/16][K/128][1024]   the tile-major shared store
  weight meta        torch.int32 (or uint32) [N/16][K/128][16]: fp16 scale bits 0..15, zero 16..23
  activation codes   torch.uint8 [M][K/2]    (4-bit two's complement, even k in the low nibble)
  activation scales  torch.float32 [M][K/128]
"""
from __future__ import annotations

import ctypes
import os

import torch

GROUP = 128
QSPEC_GREEDY = 0
QSPEC_SAMPLE = 1
QSPEC_OUT_BF16 = 0
QSPEC_OUT_F32 = 1

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqspec.so")

_lib = None


class QspecError(RuntimeError):
    """A negative status returned by the C ABI."""

    def __init__(self, fn: str, status: int):
        msg = _lib.qspec_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libqspec.so (building it once if no built copy exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.qspec_status_string.argtypes = [ctypes.c_int]
        L.qspec_status_string.restype = ctypes.c_char_p
        L.qspec_quantize_act.argtypes = [P, I, I, P, P, P]
        L.qspec_gemm_w4a4.argtypes = [P, P, I, P, P, I, I, P, I, P, P]
        L.qspec_gemm_w4a16.argtypes = [P, I, P, P, I, I, P, I, P, S, P]
        L.qspec_gemm_w4a16_workspace_bytes.argtypes = [I, I, I]
        L.qspec_gemm_w4a16_workspace_bytes.restype = S
        L.qspec_gemm_w4a16_tier.argtypes = [I, I, I, P, P]
        L.qspec_gemm_w4a4_tier.argtypes = [I, I, I, P, P]
        L.qspec_verify_workspace_bytes.argtypes = [I, I, I, I]
        L.qspec_verify_workspace_bytes.restype = S
        L.qspec_verify_accept.argtypes = [I, P, P, P, P, P, I, I, I, P, P, P, S, P]
        L.qspec_verify_accept_noalloc.argtypes = [I, P, P, P, P, P, I, I, I, P, P, P]
        L.qspec_kv_overwrite.argtypes = [P, P, P, P, I, I, I, I, I, I, P]
        L.qspec_speckv_workspace_bytes.argtypes = [I, I]
        L.qspec_speckv_workspace_bytes.restype = S
        L.qspec_speckv_gamma.argtypes = [P, I, I, ctypes.c_float, P, P, P, P, I, P, P, P, S, P]
        L.qspec_attention_workspace_bytes.argtypes = [I, I, I, I, I]
        L.qspec_attention_workspace_bytes.restype = S
        L.qspec_attention.argtypes = [P, P, P, I, I, I, I, I, I, ctypes.c_float, P, P, S, P]
        L.qspec_attention_fp8.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_float, P, P, S, P]
        L.qspec_kv_overwrite_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P]
        L.qspec_quantize_act_fp8.argtypes = [P, I, I, P, P, P]
        L.qspec_gemm_w8a8_workspace_bytes.argtypes = [I, I, I]
        L.qspec_gemm_w8a8_workspace_bytes.restype = S
        L.qspec_gemm_w8a8.argtypes = [P, P, I, P, P, I, I, P, I, P, S, P]
        L.qspec_draft_sample_workspace_bytes.argtypes = [I, I, I]
        L.qspec_draft_sample_workspace_bytes.restype = S
        L.qspec_draft_sample.argtypes = [I, P, I, I, ctypes.c_int64, P, P, I, P, S, P]
        L.qspec_draft_sample_speckv_workspace_bytes.argtypes = [I, I, I]
        L.qspec_draft_sample_speckv_workspace_bytes.restype = S
        L.qspec_draft_sample_speckv.argtypes = [I, P, I, I, ctypes.c_int64, P, P, I, ctypes.c_float, P, P, P, P, I, P,
                                                P, P, S, P]
        for fn in ("qspec_quantize_act", "qspec_gemm_w4a4", "qspec_gemm_w4a16", "qspec_verify_accept",
                   "qspec_kv_overwrite", "qspec_speckv_gamma", "qspec_attention", "qspec_quantize_act_fp8",
                   "qspec_gemm_w8a8", "qspec_draft_sample", "qspec_gemm_w4a16_tier", "qspec_gemm_w4a4_tier", "qspec_verify_accept_noalloc",
                   "qspec_draft_sample_speckv", "qspec_attention_fp8", "qspec_kv_overwrite_fp8"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise QspecError(fn, status)


def _stream(stream, ref: torch.Tensor):
    if stream is None:
        stream = torch.cuda.current_stream(ref.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _req(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _weights(w_codes, w_meta):
    if w_codes.dim() != 3 or w_codes.shape[2] != 1024:
        raise ValueError("w_codes must be [N/16][K/128][1024]")
    T, G, _ = w_codes.shape
    _req(w_codes, "w_codes", torch.uint8)
    if w_meta.dtype not in (torch.int32, torch.uint32):
        raise TypeError("w_meta must be int32 or uint32")
    _req(w_meta, "w_meta", w_meta.dtype, (T, G, 16))
    return G * GROUP, 16 * T


def _out_dtype(y: torch.Tensor) -> int:
    if y.dtype == torch.bfloat16:
        return QSPEC_OUT_BF16
    if y.dtype == torch.float32:
        return QSPEC_OUT_F32
    raise TypeError("y must be bfloat16 or float32")


def qspec_quantize_act(x, codes, scales, stream=None) -> None:
    """x bf16 [M][K] -> codes u8 [M][K/2], scales f32 [M][K/128]."""
    _req(x, "x", torch.bfloat16)
    M, K = x.shape
    _req(codes, "codes", torch.uint8, (M, K // 2))
    _req(scales, "scales", torch.float32, (M, K // GROUP))
    _check("qspec_quantize_act",
           lib().qspec_quantize_act(_ptr(x), M, K, _ptr(codes), _ptr(scales), _stream(stream, x)))


def qspec_gemm_w4a4(a_codes, a_scales, w_codes, w_meta, y, group_dots=None, stream=None) -> None:
    """W4A4 draft layer: y [M][N] (bf16 or f32); optional exact group dots i32 [K/128][M][N]."""
    K, N = _weights(w_codes, w_meta)
    _req(a_codes, "a_codes", torch.uint8)
    M = a_codes.shape[0]
    _req(a_codes, "a_codes", torch.uint8, (M, K // 2))
    _req(a_scales, "a_scales", torch.float32, (M, K // GROUP))
    dt = _out_dtype(y)
    _req(y, "y", y.dtype, (M, N))
    if group_dots is not None:
        _req(group_dots, "group_dots", torch.int32, (K // GROUP, M, N))
    _check("qspec_gemm_w4a4",
           lib().qspec_gemm_w4a4(_ptr(a_codes), _ptr(a_scales), M, _ptr(w_codes), _ptr(w_meta), K, N,
                                 _ptr(y), dt, _ptr(group_dots), _stream(stream, y)))


def qspec_gemm_w4a16_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(lib().qspec_gemm_w4a16_workspace_bytes(M, K, N))


def _tier(fn: str, M: int, K: int, N: int):
    lo, hi = ctypes.c_int32(0), ctypes.c_int32(0)
    t = getattr(lib(), fn)(M, K, N, ctypes.byref(lo), ctypes.byref(hi))
    _check(fn, t if t < 0 else 0)
    return t, lo.value, hi.value


def qspec_gemm_w4a16_tier(M: int, K: int, N: int):
    """(tier index, first M, last M) of the batch tier of M for a K x N layer: rows of
    qspec_gemm_w4a16 are bit-identical for every M in [first, last]."""
    return _tier("qspec_gemm_w4a16_tier", M, K, N)


def qspec_gemm_w4a4_tier(M: int, K: int, N: int):
    """(tier index, first M, last M) of the batch tier of M in qspec_gemm_w4a4."""
    return _tier("qspec_gemm_w4a4_tier", M, K, N)


def gemm_w4a16_workspace(M: int, K: int, N: int, device) -> torch.Tensor:
    """A workspace of the size qspec_gemm_w4a16 needs (at least one byte; no initialization needed)."""
    return torch.empty(max(1, qspec_gemm_w4a16_workspace_bytes(M, K, N)), dtype=torch.uint8, device=device)


def qspec_gemm_w4a16(x, w_codes, w_meta, y, workspace=None, stream=None) -> None:
    """W4A16 verify layer: y [M][N] = x W_hat (bf16 or f32 out).  ``workspace``: a uint8
    device tensor of qspec_gemm_w4a16_workspace_bytes(M, K, N) bytes (None if that is 0)."""
    K, N = _weights(w_codes, w_meta)
    _req(x, "x", torch.bfloat16)
    M = x.shape[0]
    _req(x, "x", torch.bfloat16, (M, K))
    dt = _out_dtype(y)
    _req(y, "y", y.dtype, (M, N))
    if workspace is not None:
        _req(workspace, "workspace", torch.uint8)
    _check("qspec_gemm_w4a16",
           lib().qspec_gemm_w4a16(_ptr(x), M, _ptr(w_codes), _ptr(w_meta), K, N, _ptr(y), dt,
                                  _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                  _stream(stream, y)))


def qspec_verify_workspace_bytes(mode: int, B: int, gamma: int, V: int) -> int:
    return int(lib().qspec_verify_workspace_bytes(mode, B, gamma, V))


def qspec_verify_accept(mode, target_logits, draft_logits, draft_tokens, u_accept, u_resample,
                        accept_count, out_tokens, workspace, stream=None) -> None:
    """Greedy (mode 0) or sampling (mode 1) verification; see include/qspec.h."""
    _req(target_logits, "target_logits", torch.float32)
    B, g1, V = target_logits.shape
    gamma = g1 - 1
    if gamma > 0 or draft_tokens is not None:
        _req(draft_tokens, "draft_tokens", torch.int32, (B, gamma))
    if mode == QSPEC_SAMPLE:
        if gamma > 0 or draft_logits is not None:
            _req(draft_logits, "draft_logits", torch.float32, (B, gamma, V))
        if gamma > 0 or u_accept is not None:
            _req(u_accept, "u_accept", torch.float32, (B, gamma))
        _req(u_resample, "u_resample", torch.float32, (B,))
    _req(accept_count, "accept_count", torch.int32, (B,))
    _req(out_tokens, "out_tokens", torch.int32, (B, g1))
    _req(workspace, "workspace", torch.uint8)
    _check("qspec_verify_accept",
           lib().qspec_verify_accept(mode, _ptr(target_logits),
                                     _ptr(draft_logits) if mode == QSPEC_SAMPLE else None,
                                     _ptr(draft_tokens), _ptr(u_accept) if mode == QSPEC_SAMPLE else None,
                                     _ptr(u_resample) if mode == QSPEC_SAMPLE else None, B, gamma, V,
                                     _ptr(accept_count), _ptr(out_tokens), _ptr(workspace),
                                     workspace.numel(), _stream(stream, target_logits)))


def qspec_verify_accept_noalloc(mode, target_logits, draft_logits, draft_tokens, u_accept, u_resample,
                                accept_count, out_tokens, stream=None) -> None:
    """qspec_verify_accept with the library's fixed device scratch instead of a workspace (for
    callers that cannot allocate); calls that overlap on one GPU race."""
    _req(target_logits, "target_logits", torch.float32)
    B, g1, V = target_logits.shape
    gamma = g1 - 1
    if gamma > 0 or draft_tokens is not None:
        _req(draft_tokens, "draft_tokens", torch.int32, (B, gamma))
    if mode == QSPEC_SAMPLE:
        if gamma > 0 or draft_logits is not None:
            _req(draft_logits, "draft_logits", torch.float32, (B, gamma, V))
        if gamma > 0 or u_accept is not None:
            _req(u_accept, "u_accept", torch.float32, (B, gamma))
        _req(u_resample, "u_resample", torch.float32, (B,))
    _req(accept_count, "accept_count", torch.int32, (B,))
    _req(out_tokens, "out_tokens", torch.int32, (B, g1))
    _check("qspec_verify_accept_noalloc",
           lib().qspec_verify_accept_noalloc(mode, _ptr(target_logits),
                                             _ptr(draft_logits) if mode == QSPEC_SAMPLE else None,
                                             _ptr(draft_tokens), _ptr(u_accept) if mode == QSPEC_SAMPLE else None,
                                             _ptr(u_resample) if mode == QSPEC_SAMPLE else None, B, gamma, V,
                                             _ptr(accept_count), _ptr(out_tokens), _stream(stream, target_logits)))


def qspec_draft_sample_workspace_bytes(mode: int, B: int, V: int) -> int:
    return int(lib().qspec_draft_sample_workspace_bytes(mode, B, V))


def qspec_draft_sample(mode, logits, tokens, u, workspace, stream=None) -> None:
    """The draft-side head of one step: logits f32 [B][V] with unit stride along V (rows may be
    strided, e.g. draft_logits[:, j, :]); tokens i32 [B] (may be strided, e.g. draft_tokens[:, j]);
    u f32 [B] (SAMPLE) or None (GREEDY); workspace u8 of qspec_draft_sample_workspace_bytes bytes."""
    for t, name, dt in ((logits, "logits", torch.float32), (tokens, "tokens", torch.int32)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA (HIP) device tensor")
        if t.dtype != dt:
            raise TypeError(f"{name} must have dtype {dt}")
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [B][V] with unit stride along V")
    B, V = logits.shape
    if tokens.dim() != 1 or tokens.shape[0] != B:
        raise ValueError("tokens must be [B]")
    if u is not None:
        _req(u, "u", torch.float32, (B,))
    _req(workspace, "workspace", torch.uint8)
    _check("qspec_draft_sample",
           lib().qspec_draft_sample(mode, _ptr(logits), B, V, logits.stride(0), _ptr(u), _ptr(tokens),
                                    tokens.stride(0), _ptr(workspace), workspace.numel(), _stream(stream, logits)))


def qspec_draft_sample_speckv_workspace_bytes(mode: int, B: int, V: int) -> int:
    return int(lib().qspec_draft_sample_speckv_workspace_bytes(mode, B, V))


def qspec_draft_sample_speckv(mode, logits, tokens, u, quant_feature, w1, b1, w2, b2, gamma_out, features,
                              workspace, stream=None) -> None:
    """The draft-side head and the adaptive-gamma controller of one step (see include/qspec.h):
    logits / tokens / u as qspec_draft_sample; w1..b2, gamma_out i32 [B] and features f64 [B][2]
    (or None) as qspec_speckv_gamma; workspace u8 (qspec_draft_sample_speckv_workspace_bytes)."""
    for t, name, dt in ((logits, "logits", torch.float32), (tokens, "tokens", torch.int32)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA (HIP) device tensor")
        if t.dtype != dt:
            raise TypeError(f"{name} must have dtype {dt}")
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [B][V] with unit stride along V")
    B, V = logits.shape
    if tokens.dim() != 1 or tokens.shape[0] != B:
        raise ValueError("tokens must be [B]")
    if u is not None:
        _req(u, "u", torch.float32, (B,))
    _req(w1, "w1", torch.float32, (64, 3))
    _req(b1, "b1", torch.float32, (64,))
    _req(w2, "w2", torch.float32)
    G1 = w2.shape[0]
    _req(w2, "w2", torch.float32, (G1, 64))
    _req(b2, "b2", torch.float32, (G1,))
    _req(gamma_out, "gamma_out", torch.int32, (B,))
    if features is not None:
        _req(features, "features", torch.float64, (B, 2))
    _req(workspace, "workspace", torch.uint8)
    _check("qspec_draft_sample_speckv",
           lib().qspec_draft_sample_speckv(mode, _ptr(logits), B, V, logits.stride(0), _ptr(u), _ptr(tokens),
                                           tokens.stride(0), float(quant_feature), _ptr(w1), _ptr(b1), _ptr(w2),
                                           _ptr(b2), G1 - 1, _ptr(features), _ptr(gamma_out), _ptr(workspace),
                                           workspace.numel(), _stream(stream, logits)))


def qspec_kv_overwrite(cache, verify_kv, start_pos, accept_count, stream=None) -> None:
    """cache bf16 [L][B][2][H][T][D] <- verify_kv bf16 [L][B][2][H][gamma+1][D] for rows 0..A_b."""
    _req(cache, "cache", torch.bfloat16)
    if cache.dim() != 6 or cache.shape[2] != 2:
        raise ValueError("cache must be [L][B][2][H][T][D]")
    L, B, _, H, T, D = cache.shape
    _req(verify_kv, "verify_kv", torch.bfloat16)
    if verify_kv.dim() != 6:
        raise ValueError("verify_kv must be [L][B][2][H][gamma+1][D]")
    gamma = verify_kv.shape[4] - 1
    _req(verify_kv, "verify_kv", torch.bfloat16, (L, B, 2, H, gamma + 1, D))
    _req(start_pos, "start_pos", torch.int32, (B,))
    _req(accept_count, "accept_count", torch.int32, (B,))
    _check("qspec_kv_overwrite",
           lib().qspec_kv_overwrite(_ptr(cache), _ptr(verify_kv), _ptr(start_pos), _ptr(accept_count),
                                    L, B, H, T, D, gamma, _stream(stream, cache)))


def qspec_speckv_workspace_bytes(R: int, V: int) -> int:
    return int(lib().qspec_speckv_workspace_bytes(R, V))


def qspec_speckv_gamma(draft_logits, quant_feature, w1, b1, w2, b2, gamma_out, features=None, workspace=None,
                       stream=None) -> None:
    """Draft statistics and the adaptive-gamma controller; see include/qspec.h.
    draft_logits f32 [R][V]; w1 f32 [64][3], b1 [64], w2 [G1][64], b2 [G1]; gamma_out i32 [R];
    features f64 [R][2] or None; workspace u8 (qspec_speckv_workspace_bytes(R, V) bytes)."""
    _req(draft_logits, "draft_logits", torch.float32)
    R, V = draft_logits.shape
    _req(w1, "w1", torch.float32, (64, 3))
    _req(b1, "b1", torch.float32, (64,))
    _req(w2, "w2", torch.float32)
    G1 = w2.shape[0]
    _req(w2, "w2", torch.float32, (G1, 64))
    _req(b2, "b2", torch.float32, (G1,))
    _req(gamma_out, "gamma_out", torch.int32, (R,))
    if features is not None:
        _req(features, "features", torch.float64, (R, 2))
    _req(workspace, "workspace", torch.uint8)
    _check("qspec_speckv_gamma",
           lib().qspec_speckv_gamma(_ptr(draft_logits), R, V, float(quant_feature), _ptr(w1), _ptr(b1), _ptr(w2),
                                    _ptr(b2), G1 - 1, _ptr(features), _ptr(gamma_out), _ptr(workspace),
                                    workspace.numel(), _stream(stream, draft_logits)))


def qspec_kv_overwrite_fp8(cache_codes, cache_scales, verify_kv, start_pos, accept_count, stream=None) -> None:
    """Quantized cache: codes u8 [L][B][2][H][T][D], scales f32 [L][B][2][H][T] <- rows 0..A_b of
    verify_kv bf16 [L][B][2][H][gamma+1][D], quantized per row (FP8 E4M3, absmax / 448)."""
    _req(cache_codes, "cache_codes", torch.uint8)
    if cache_codes.dim() != 6 or cache_codes.shape[2] != 2:
        raise ValueError("cache_codes must be [L][B][2][H][T][D]")
    L, B, _, H, T, D = cache_codes.shape
    _req(cache_scales, "cache_scales", torch.float32, (L, B, 2, H, T))
    _req(verify_kv, "verify_kv", torch.bfloat16)
    if verify_kv.dim() != 6:
        raise ValueError("verify_kv must be [L][B][2][H][gamma+1][D]")
    gamma = verify_kv.shape[4] - 1
    _req(verify_kv, "verify_kv", torch.bfloat16, (L, B, 2, H, gamma + 1, D))
    _req(start_pos, "start_pos", torch.int32, (B,))
    _req(accept_count, "accept_count", torch.int32, (B,))
    _check("qspec_kv_overwrite_fp8",
           lib().qspec_kv_overwrite_fp8(_ptr(cache_codes), _ptr(cache_scales), _ptr(verify_kv), _ptr(start_pos),
                                        _ptr(accept_count), L, B, H, T, D, gamma, _stream(stream, cache_codes)))


def qspec_attention_fp8(q, cache_codes, cache_scales, pos, scale, out, workspace, stream=None) -> None:
    """Causal attention over one layer of the quantized cache; see include/qspec.h.
    q bf16 [B][Q][Hq][D]; cache_codes u8 [B][2][Hkv][T][D]; cache_scales f32 [B][2][Hkv][T];
    pos i32 [B]; out bf16 [B][Q][Hq][D]; workspace u8 (qspec_attention_workspace_bytes)."""
    _req(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B][Q][Hq][D]")
    B, Q, Hq, D = q.shape
    _req(cache_codes, "cache_codes", torch.uint8)
    if cache_codes.dim() != 5 or cache_codes.shape[0] != B or cache_codes.shape[1] != 2 or cache_codes.shape[4] != D:
        raise ValueError("cache_codes must be [B][2][Hkv][T][D]")
    Hkv, T = cache_codes.shape[2], cache_codes.shape[3]
    _req(cache_scales, "cache_scales", torch.float32, (B, 2, Hkv, T))
    _req(pos, "pos", torch.int32, (B,))
    _req(out, "out", torch.bfloat16, (B, Q, Hq, D))
    _req(workspace, "workspace", torch.uint8)
    _check("qspec_attention_fp8",
           lib().qspec_attention_fp8(_ptr(q), _ptr(cache_codes), _ptr(cache_scales), _ptr(pos), B, Q, Hq, Hkv, T, D,
                                     float(scale), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream, q)))


def qspec_attention_workspace_bytes(B: int, Q: int, Hq: int, Hkv: int, T: int) -> int:
    return int(lib().qspec_attention_workspace_bytes(B, Q, Hq, Hkv, T))


def qspec_attention(q, cache, pos, scale, out, workspace, stream=None) -> None:
    """Causal attention over one layer of the shared KV cache; see include/qspec.h.
    q bf16 [B][Q][Hq][D]; cache bf16 [B][2][Hkv][T][D]; pos i32 [B]; out bf16 [B][Q][Hq][D];
    workspace u8 (qspec_attention_workspace_bytes(B, Q, Hq, Hkv, T) bytes)."""
    _req(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B][Q][Hq][D]")
    B, Q, Hq, D = q.shape
    _req(cache, "cache", torch.bfloat16)
    if cache.dim() != 5 or cache.shape[0] != B or cache.shape[1] != 2 or cache.shape[4] != D:
        raise ValueError("cache must be [B][2][Hkv][T][D]")
    Hkv, T = cache.shape[2], cache.shape[3]
    _req(pos, "pos", torch.int32, (B,))
    _req(out, "out", torch.bfloat16, (B, Q, Hq, D))
    _req(workspace, "workspace", torch.uint8)
    _check("qspec_attention",
           lib().qspec_attention(_ptr(q), _ptr(cache), _ptr(pos), B, Q, Hq, Hkv, T, D, float(scale), _ptr(out),
                                 _ptr(workspace), workspace.numel(), _stream(stream, q)))


def qspec_quantize_act_fp8(x, codes, scales, stream=None) -> None:
    """x bf16 [M][K] -> per-token FP8 (E4M3) codes u8 [M][K] and scales f32 [M]."""
    _req(x, "x", torch.bfloat16)
    M, K = x.shape
    _req(codes, "codes", torch.uint8, (M, K))
    _req(scales, "scales", torch.float32, (M,))
    _check("qspec_quantize_act_fp8",
           lib().qspec_quantize_act_fp8(_ptr(x), M, K, _ptr(codes), _ptr(scales), _stream(stream, x)))


def qspec_gemm_w8a8_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(lib().qspec_gemm_w8a8_workspace_bytes(M, K, N))


def qspec_gemm_w8a8(a_codes, a_scales, w_store, w_scales, y, workspace=None, stream=None) -> None:
    """FP8 parent layer: y [M][N] (bf16 or f32) = s_a s_w sum E4M3(a) E4M3(w).  w_store u8
    [N/16][K/128][2048], w_scales f32 [N]; workspace u8 of qspec_gemm_w8a8_workspace_bytes bytes."""
    _req(w_store, "w_store", torch.uint8)
    if w_store.dim() != 3 or w_store.shape[2] != 2048:
        raise ValueError("w_store must be [N/16][K/128][2048]")
    K, N = w_store.shape[1] * GROUP, w_store.shape[0] * 16
    _req(w_scales, "w_scales", torch.float32, (N,))
    _req(a_codes, "a_codes", torch.uint8)
    M = a_codes.shape[0]
    _req(a_codes, "a_codes", torch.uint8, (M, K))
    _req(a_scales, "a_scales", torch.float32, (M,))
    dt = _out_dtype(y)
    _req(y, "y", y.dtype, (M, N))
    if workspace is not None:
        _req(workspace, "workspace", torch.uint8)
    _check("qspec_gemm_w8a8",
           lib().qspec_gemm_w8a8(_ptr(a_codes), _ptr(a_scales), M, _ptr(w_store), _ptr(w_scales), K, N, _ptr(y), dt,
                                 _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                 _stream(stream, y)))


__all__ = [
    "GROUP", "QSPEC_GREEDY", "QSPEC_SAMPLE", "QSPEC_OUT_BF16", "QSPEC_OUT_F32", "QspecError", "lib",
    "qspec_quantize_act", "qspec_gemm_w4a4", "qspec_gemm_w4a16", "qspec_gemm_w4a16_workspace_bytes",
    "gemm_w4a16_workspace", "qspec_verify_workspace_bytes",
    "qspec_verify_accept", "qspec_kv_overwrite", "qspec_speckv_workspace_bytes", "qspec_speckv_gamma",
    "qspec_attention_workspace_bytes", "qspec_attention", "qspec_quantize_act_fp8",
    "qspec_gemm_w8a8_workspace_bytes", "qspec_gemm_w8a8", "qspec_draft_sample_workspace_bytes",
    "qspec_draft_sample",
]
