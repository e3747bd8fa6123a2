// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qspec {

constexpr int kGroup = 128;   // quantization group along K (weights and activations)
constexpr int kWave = 64;     // CDNA wavefront width

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

// 16-byte load marked non-temporal (streamed once: weights, logits).
__device__ __forceinline__ uint4 load_stream16(const void *p) {
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)p);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Buffer loads: a wave-uniform resource (base address and size in SGPRs), a 32-bit per-lane
// offset and a wave-uniform offset.  Reads past `bytes` return zero instead of faulting.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufCachePolicyNT = 2;   // non-temporal: streamed once

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint4 buf_load16_stream(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kBufCachePolicyNT));
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
// 16 bytes per lane from a buffer straight into LDS (no registers): lane l's bytes land at
// dst + 16 l, dst being wave-uniform.  Kept out of kernel bodies: a kernel whose own body casts to
// the LDS address space gets no host-side launch stub.
__device__ __forceinline__ void buf_load16_to_lds(rsrc_t r, unsigned char *dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, soff, 0, 0);
}

// Nearest E4M3 code to a finite binary32 value, ties to even, saturating at +-448; the sign bit
// is the value's.  Normal range: a * 2^(3 - e) lies in [8, 16) and rounds (exactly, nearest
// even) to the 4-bit significand, a carry to 16 moving into the exponent field; below 2^-6 the
// subnormal step is 2^-9.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    uint32_t code;
    if (!(a < 448.0f)) {
        code = 0x7Eu;
    } else if (a < 0x1p-6f) {
        code = (uint32_t)__builtin_rintf(a * 0x1p9f);
    } else {
        const int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;        // -6 .. 8
        const float sig = a * __uint_as_float((uint32_t)(127 + 3 - e) << 23);  // [8, 16), exact
        code = (uint32_t)((e + 7) << 3) + (uint32_t)__builtin_rintf(sig) - 8u;
    }
    return sign | code;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
    return __uint_as_float(b << 16);
}

__device__ __forceinline__ float fp16_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// Nearest-even conversion of two floats into a packed bfloat16 pair (lo = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float a) {
    return __builtin_bit_cast(uint16_t, (__bf16)a);
}

// Wave-wide reductions (64 lanes) through cross-lane shuffles.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

}  // namespace qspec

namespace qspec {

// (a & m) | o in one VALU op; m and o are loop-invariant constants the compiler keeps in VGPRs
// (gfx9 VOP3 encodings take no literals, so the fused form is not selected on its own).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
    return r;
}

// Number of waves per workgroup that split the K groups of one column tile between them.  It
// depends on (K, N) only, so every batch size reduces each output in the same order.  Small-N
// layers get more waves per tile so the chip still holds thousands of waves in flight.
constexpr int kMaxSplitWaves = 16;

__host__ __device__ inline int skinny_waves_for_shape(int K, int N) {
    const int G = K / kGroup;
    const int tiles = (N + 15) / 16;
    int kw = 1;
    while (kw < kMaxSplitWaves && tiles * kw * 2 <= 8192) kw *= 2;
    while (kw > G) kw >>= 1;
    return kw < 1 ? 1 : kw;
}

// The dispatcher deals workgroup i to XCD i % 8.  xcd_remap(i, n) is a bijection of [0, n) that
// gives each XCD one contiguous range of logical tiles, walked in order, so neighbouring logical
// tiles (which share operands) meet in the same L2.
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_remap(int i, int n) {
    const int per = (n + kXcds - 1) / kXcds;          // tiles of the larger XCD ranges
    int tall = n % kXcds;                             // XCDs holding `per` tiles
    if (tall == 0) tall = kXcds;
    const int xcd = i % kXcds, local = i / kXcds;
    return xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

// Decode kernels (M <= 16), W4A4 and W4A16 alike: column tiles per workgroup (nt) and K-splitting
// waves (kw), a function of (K, N) only, so the reduction order is too.  Chosen from measured
// sweeps of every (nt, kw) over the Llama-3-8B / Qwen2.5-7B projection shapes at M = 1, 5, 16:
// about 500 - 2000 waves in flight, wider workgroups rather than more K splits, two groups per
// wave at least.
constexpr int kMaxDecodeWaves = 8;

struct DecodeShape {
    int nt, kw;
};

__host__ __device__ inline DecodeShape decode_shape(int K, int N) {
    const int T = N / 16, G = K / kGroup;
    DecodeShape d;
    if (T >= 4096) {
        d = {4, 1};
    } else if (T >= 1024) {
        // one wave per workgroup while the workgroups fit the 1024 SIMDs in one pass (Llama-3-8B
        // gate+up, 896); past that (Qwen2.5-7B gate+up, 1184) a second pass of single waves
        // measured 5 - 15% slower than splitting K over two waves
        d = {2, T / 2 > 1024 ? 2 : 1};
    } else if (T >= 384) {
        d = {2, 4};
    } else {
        d = {1, 4};
    }
    while (d.kw > 1 && 2 * d.kw > G) d.kw >>= 1;
    return d;
}

}  // namespace qspec
