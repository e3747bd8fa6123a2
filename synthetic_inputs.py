"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out in the storage formats;
it holds none of the method's arithmetic (no quantizer, no dequantization, no
product, no softmax).  Both the oracle side and the HIP side read what it makes.

Storage formats (fixed by this project):
  weight codes  u8  [N/16][K/128][1024]  tile-major: block (t, g) holds columns 16t..16t+15 and
                k = 128g..128g+127 as [quarter q = (k%128)/32][column c][16 bytes of k%32],
                two unsigned 4-bit codes per byte, even k in the low nibble
  weight meta   u32 [N/16][K/128][16]    binary16 scale in bits 0..15, zero point in bits 16..23
  activations   u16 [M][K]     bfloat16 bit patterns
  logits        f32

Distributions (one PCG64 stream per tensor, seeded by a fixed table):
  * weight codes uniform 0..15 (so each packed byte is uniform 0..255);
  * weight scales uniform [1e-3, 1e-2], rounded to binary16; zero points uniform 0..15;
  * activations N(0, 1) with round(1% of K) channels (same for every token) scaled
    by 20, then rounded to bfloat16 (nearest-even, by torch's conversion);
  * target logits N(0, sigma=3); draft logits = target + N(0, 0.5);
  * uniforms in [0, 1) as float32;
  * KV: a position-dependent canary pattern in the cache, N(0, 1) bfloat16 staging rows;
  * FP8 stores: E4M3 codes drawn uniformly from the 254 finite codes, column scales uniform
    [1e-4, 1e-3] (benchmark); the tests also quantize N(0, 0.02^2) bfloat16 weights with the oracle;
  * attention: queries N(0, 2^2) (scores of standard deviation 2 at scale 1/sqrt(D)), cached
    keys and values N(0, 1), all bfloat16.
"""
from __future__ import annotations

import numpy as np

GROUP = 128

# seed table: one base per tensor kind; a config index or layer index is added.
SEED_WEIGHTS = 100
SEED_ACT = 200
SEED_OUTLIER = 300
SEED_LOGITS = 400
SEED_NOISE = 500
SEED_UNIFORM = 600
SEED_START = 700
SEED_KV = 800
SEED_GUMBEL = 900
SEED_ATTN = 1000
SEED_FP8 = 1100


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (torch's nearest-even conversion); u16 patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def pack_weights(codes_rm, scales_bits, zeros):
    """Row-major weights -> the tile-major store.  codes_rm u8 [N][K/2] (even k low nibble),
    scales_bits u16 [N][K/128] (binary16), zeros u8 [N][K/128] -> (codes u8 [N/16][G][1024],
    meta u32 [N/16][G][16]).  Pure layout: no arithmetic on the values."""
    codes_rm = np.ascontiguousarray(codes_rm, np.uint8)
    N, K2 = codes_rm.shape
    assert N % 16 == 0 and (2 * K2) % GROUP == 0
    G = 2 * K2 // GROUP
    # [N][K/2] -> [t][c][g][q][16] -> [t][g][q][c][16]
    blocks = codes_rm.reshape(N // 16, 16, G, 4, 16).transpose(0, 2, 3, 1, 4)
    codes = np.ascontiguousarray(blocks).reshape(N // 16, G, 1024)
    meta = (np.asarray(scales_bits, np.uint32) | (np.asarray(zeros, np.uint32) << np.uint32(16)))
    meta = np.ascontiguousarray(meta.reshape(N // 16, 16, G).transpose(0, 2, 1))
    return codes, meta


def unpack_weights(codes, meta):
    """Inverse of pack_weights: (codes_rm u8 [N][K/2], scales_bits u16 [N][G], zeros u8 [N][G])."""
    T, G, _ = codes.shape
    rm = np.ascontiguousarray(codes.reshape(T, G, 4, 16, 16).transpose(0, 3, 1, 2, 4)).reshape(16 * T, G * 64)
    m = np.ascontiguousarray(meta.transpose(0, 2, 1)).reshape(16 * T, G)
    return rm, (m & np.uint32(0xFFFF)).astype(np.uint16), ((m >> np.uint32(16)) & np.uint32(0xFF)).astype(np.uint8)


def pack_fp8_weights(codes_nk):
    """FP8 codes u8 [N][K] (column n's codes contiguous) -> the tile-major FP8 store u8
    [N/16][K/128][2048]: byte (h, l, b), l = c + 16 q, is column 16t + c at k = 128g + 32q + 16h + b.
    Pure layout."""
    codes_nk = np.ascontiguousarray(codes_nk, np.uint8)
    N, K = codes_nk.shape
    assert N % 16 == 0 and K % GROUP == 0
    G = K // GROUP
    # [t][c][g][q][h][b] -> [t][g][h][q][c][b]
    blocks = codes_nk.reshape(N // 16, 16, G, 4, 2, 16).transpose(0, 2, 4, 3, 1, 5)
    return np.ascontiguousarray(blocks).reshape(N // 16, G, 2048)


def unpack_fp8_weights(store):
    """Inverse of pack_fp8_weights: codes u8 [N][K]."""
    T, G, _ = store.shape
    return np.ascontiguousarray(store.reshape(T, G, 2, 4, 16, 16).transpose(0, 4, 1, 3, 2, 5)).reshape(16 * T, G * GROUP)


def fp8_codes(shape, seed: int) -> np.ndarray:
    """Uniformly drawn finite E4M3 codes (every byte except 0x7F and 0xFF)."""
    c = rng(SEED_FP8 + seed).integers(0, 254, size=shape).astype(np.uint8)
    return c + (c >= 0x7F).astype(np.uint8)


def slice_tiles(w: dict, tiles) -> dict:
    """The sub-store of the given 16-column tiles (columns 16t..16t+15 of each tile t)."""
    tiles = np.asarray(tiles)
    return {"codes": np.ascontiguousarray(w["codes"][tiles]), "meta": np.ascontiguousarray(w["meta"][tiles]),
            "K": w["K"], "N": 16 * len(tiles)}


def weights(K: int, N: int, seed: int) -> dict:
    """Shared INT4 weights in the tile-major store (see pack_weights)."""
    assert K % GROUP == 0 and N % 16 == 0
    G = K // GROUP
    r = rng(SEED_WEIGHTS + seed)
    codes_rm = r.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = r.uniform(1e-3, 1e-2, size=(N, G)).astype(np.float16).view(np.uint16)
    zeros = r.integers(0, 16, size=(N, G), dtype=np.uint8)
    codes, meta = pack_weights(codes_rm, scales, zeros)
    return {"codes": codes, "meta": meta, "K": K, "N": N}


def outlier_channels(K: int, seed: int) -> np.ndarray:
    n_out = int(round(0.01 * K))
    return rng(SEED_OUTLIER + seed).choice(K, size=n_out, replace=False)


def activations(M: int, K: int, seed: int, outlier_seed: int | None = None) -> np.ndarray:
    """bfloat16 [M][K] with 1% outlier channels x20."""
    x = rng(SEED_ACT + seed).standard_normal((M, K)).astype(np.float32)
    cols = outlier_channels(K, seed if outlier_seed is None else outlier_seed)
    x[:, cols] *= 20.0
    return f32_to_bf16_bits(x)


def logits(B: int, gamma: int, V: int, seed: int, sigma: float = 3.0, noise: float = 0.5):
    """target f32 [B][gamma+1][V] ~ N(0, sigma); draft f32 [B][gamma][V] = target rows + N(0, noise)."""
    t = (rng(SEED_LOGITS + seed).standard_normal((B, gamma + 1, V)) * sigma).astype(np.float32)
    e = (rng(SEED_NOISE + seed).standard_normal((B, gamma, V)) * noise).astype(np.float32)
    d = (t[:, :gamma, :] + e).astype(np.float32)
    return t, d


def draft_tokens_greedy(draft: np.ndarray) -> np.ndarray:
    """The draft's own greedy choices (argmax of each draft row), i32 [B][gamma]."""
    return np.argmax(draft, axis=-1).astype(np.int32)


def draft_tokens_sampled(draft: np.ndarray, seed: int) -> np.ndarray:
    """Draft tokens drawn from softmax(draft row) with the Gumbel-max rule."""
    g = rng(SEED_GUMBEL + seed).gumbel(size=draft.shape)
    return np.argmax(draft.astype(np.float64) + g, axis=-1).astype(np.int32)


def uniforms(shape, seed: int) -> np.ndarray:
    return rng(SEED_UNIFORM + seed).random(size=shape, dtype=np.float32)


def kv_canary(L: int, B: int, H: int, T: int, D: int) -> np.ndarray:
    """A cache filled with a pattern that encodes (l, b, kv, h, t, e); u16 [L][B][2][H][T][D]."""
    idx = np.arange(L * B * 2 * H * T * D, dtype=np.uint64)
    return ((idx * np.uint64(2654435761)) >> np.uint64(7)).astype(np.uint16)


def kv_staging(L: int, B: int, H: int, gamma: int, D: int, seed: int) -> np.ndarray:
    x = rng(SEED_KV + seed).standard_normal((L, B, 2, H, gamma + 1, D)).astype(np.float32)
    return f32_to_bf16_bits(x)


def start_positions(B: int, T: int, gamma: int, seed: int) -> np.ndarray:
    return rng(SEED_START + seed).integers(0, T - gamma - 1 + 1, size=B).astype(np.int32)


def attention_inputs(B: int, Q: int, Hq: int, Hkv: int, T: int, D: int, seed: int, q_sigma: float = 2.0):
    """(q u16 [B][Q][Hq][D], cache u16 [B][2][Hkv][T][D]) as bfloat16 bits."""
    r = rng(SEED_ATTN + seed)
    q = f32_to_bf16_bits((r.standard_normal((B, Q, Hq, D)) * q_sigma).astype(np.float32))
    cache = f32_to_bf16_bits(r.standard_normal((B, 2, Hkv, T, D), dtype=np.float32))
    return q, cache


# ---- named workloads (shapes only; see the design doc for the recipe) -------------

LLAMA3_8B_PROJ = {"qkv": (4096, 6144), "o": (4096, 4096), "gate_up": (4096, 2 * 14336),
                  "down": (14336, 4096)}
LLAMA3_8B_HEAD = (4096, 128256)          # the vocabulary projection (hidden -> vocabulary)
QWEN25_7B_PROJ = {"qkv": (3584, 4608), "o": (3584, 3584), "gate_up": (3584, 2 * 18944),
                  "down": (18944, 3584), "lm_head": (3584, 152064)}
LLAMA3_70B_FFN = {"gate_up": (8192, 2 * 28672), "down": (28672, 8192)}
SMALL_LAYER = {"proj": (512, 512)}


# ---- device-side generators for large benchmark inputs (same distributions) -----------------
# torch.Generator streams seeded from the same table; used where host generation and copies of
# gigabytes of weights would dominate start-up.

def _gen(device, base: int, seed: int):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(base * 1_000_003 + seed)
    return g


def weights_device(K: int, N: int, seed: int, device):
    """(codes u8 [N/16][G][1024], meta i32 [N/16][G][16]) drawn directly in the tile-major store."""
    import torch

    G = K // GROUP
    g = _gen(device, SEED_WEIGHTS, seed)
    codes = torch.randint(0, 256, (N // 16, G, 1024), dtype=torch.uint8, device=device, generator=g)
    scales = (torch.rand((N // 16, G, 16), device=device, generator=g) * 9e-3 + 1e-3).to(torch.float16)
    zeros = torch.randint(0, 16, (N // 16, G, 16), dtype=torch.int32, device=device, generator=g)
    meta = (scales.view(torch.int16).to(torch.int32) & 0xFFFF) | (zeros << 16)
    return codes, meta


def activations_device(M: int, K: int, seed: int, device):
    import torch

    x = torch.randn((M, K), device=device, generator=_gen(device, SEED_ACT, seed))
    cols = torch.from_numpy(outlier_channels(K, seed)).to(device)
    x[:, cols] *= 20.0
    return x.to(torch.bfloat16)


def logits_device(B: int, gamma: int, V: int, seed: int, device, sigma: float = 3.0, noise: float = 0.5):
    import torch

    t = torch.randn((B, gamma + 1, V), device=device, generator=_gen(device, SEED_LOGITS, seed)) * sigma
    e = torch.randn((B, gamma, V), device=device, generator=_gen(device, SEED_NOISE, seed)) * noise
    return t, (t[:, :gamma, :] + e).contiguous()


def draft_tokens_sampled_device(draft, seed: int):
    """Gumbel-max draws from softmax(draft row), on the device."""
    import torch

    u = torch.rand(draft.shape, device=draft.device, generator=_gen(draft.device, SEED_GUMBEL, seed))
    gumbel = -torch.log(-torch.log(u.clamp_min(1e-20)))
    return torch.argmax(draft + gumbel, dim=-1).to(torch.int32)


def attention_inputs_device(B: int, Q: int, Hq: int, Hkv: int, T: int, D: int, seed: int, device,
                            q_sigma: float = 2.0):
    """(q bf16 [B][Q][Hq][D], cache bf16 [B][2][Hkv][T][D]) drawn on the device."""
    import torch

    g = _gen(device, SEED_ATTN, seed)
    q = (torch.randn((B, Q, Hq, D), device=device, generator=g) * q_sigma).to(torch.bfloat16)
    cache = torch.randn((B, 2, Hkv, T, D), device=device, generator=g).to(torch.bfloat16)
    return q, cache


def fp8_weights_device(K: int, N: int, seed: int, device):
    """(FP8 store u8 [N/16][K/128][2048] of uniformly drawn finite E4M3 codes, column scales f32 [N]
    uniform [1e-4, 1e-3]) drawn on the device."""
    import torch

    g = _gen(device, SEED_FP8, seed)
    c = torch.randint(0, 254, (N // 16, K // GROUP, 2048), dtype=torch.uint8, device=device, generator=g)
    c = c + (c >= 0x7F).to(torch.uint8)
    s = torch.rand((N,), device=device, generator=g) * 9e-4 + 1e-4
    return c, s


def uniforms_device(shape, seed: int, device):
    import torch

    return torch.rand(shape, device=device, generator=_gen(device, SEED_UNIFORM, seed))
