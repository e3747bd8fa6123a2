// W4A16 verify linear layer on gfx950.
//
// y[m][n] = sum_k x[m][k] * W_hat[k][n],  W_hat = bf16_nearest_even(s[n][g] * (w[k][n] - z[n][g]))
// (QSPEC notes, background terms: dequantization example Y = X W_hat, W_hat = s (W_INT4 - z);
//  QSPEC structure: the verifier scores gamma+1 positions in one pass.)
//
// The shared weight store is tile-major (include/qspec.h): one 1 KB block per (16-column tile,
// 128-k group), laid out so that lane l = col + 16 q of a wave reads bytes 16 l .. 16 l + 15 --
// exactly the 32 codes its v_mfma_f32_16x16x32_bf16 B fragments need.  Every wave-wide weight
// load is one contiguous kilobyte.
//
// Two kernels share the dequantization routine:
//  * k_w4a16_skinny (M <= 80): HBM-bound decode/verify shapes.  A workgroup owns NT column tiles
//    and KW waves split the K groups between them; every wave keeps U groups of loads in flight,
//    dequantizes in registers and feeds the MFMA with the activations as the A operand (rows =
//    tokens, padded to 16) and W_hat as the B operand.  Wave partials are summed through LDS in
//    a fixed order, so the reduction order depends on (K, N) and the batch tier only.
//  * k_w4a16_tiled (M > 80): MFMA-bound shapes.  128x128 output tiles, one K group per step; the
//    activation tile and the dequantized weight tile are staged in LDS and each of the 4 waves
//    computes a 64x64 sub-tile with 16 MFMAs per 32-wide k step.
#include "common.hpp"
#include "kernels.hpp"

namespace qspec {

// Per-group constants of the exact dequantization below.
struct DqConst {
    float s;     // scale
    float s16;   // scale / 16 (exact)
    float c_lo;  // -(1024 + z) * s   (exact: 11-bit integer times an 11-bit significand)
    float c_hi;  // -(64 + z) * s     (exact)
};

// meta word: binary16 scale in bits 0..15, zero point in bits 16..23.
__device__ __forceinline__ DqConst make_dq(uint32_t meta) {
    const int z = (int)((meta >> 16) & 0xFFu);
    DqConst c;
    c.s = fp16_bits_to_float((uint16_t)(meta & 0xFFFFu));
    c.s16 = c.s * 0.0625f;
    c.c_lo = -(float)(1024 + z) * c.s;
    c.c_hi = -(float)(64 + z) * c.s;
    return c;
}

// Dequantize the 8 codes of one dword (code i = bits 4i..4i+3 = k offset i) into 8 bfloat16
// values in k order, packed two per dword.  Each code is planted into the mantissa of a binary16
// 1024.0 (codes 0,2,4,6 -> 1024 + w; codes 1,3,5,7 -> 1024 + 16 w, read with s/16), so
// v_fma_mix_f32 forms (1024 + w) s - (1024 + z) s = (w - z) s exactly (every term has at most
// 22 significant bits), and the only rounding is the nearest-even conversion to bfloat16.
__device__ __forceinline__ void dequant8(uint32_t p, const DqConst &c, uint32_t out[4]) {
    const uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, one = 0x64006400u;
    const uint32_t p8 = p >> 8;
    const f16x2_t v0 = __builtin_bit_cast(f16x2_t, and_or(p, mlo, one));    // w0, w4
    const f16x2_t v1 = __builtin_bit_cast(f16x2_t, and_or(p, mhi, one));    // 16 w1, 16 w5
    const f16x2_t v2 = __builtin_bit_cast(f16x2_t, and_or(p8, mlo, one));   // w2, w6
    const f16x2_t v3 = __builtin_bit_cast(f16x2_t, and_or(p8, mhi, one));   // 16 w3, 16 w7
    const float f0 = __builtin_fmaf((float)v0[0], c.s, c.c_lo);
    const float f4 = __builtin_fmaf((float)v0[1], c.s, c.c_lo);
    const float f1 = __builtin_fmaf((float)v1[0], c.s16, c.c_hi);
    const float f5 = __builtin_fmaf((float)v1[1], c.s16, c.c_hi);
    const float f2 = __builtin_fmaf((float)v2[0], c.s, c.c_lo);
    const float f6 = __builtin_fmaf((float)v2[1], c.s, c.c_lo);
    const float f3 = __builtin_fmaf((float)v3[0], c.s16, c.c_hi);
    const float f7 = __builtin_fmaf((float)v3[1], c.s16, c.c_hi);
    out[0] = pack_bf16x2(f0, f1);
    out[1] = pack_bf16x2(f2, f3);
    out[2] = pack_bf16x2(f4, f5);
    out[3] = pack_bf16x2(f6, f7);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    uint4 u = make_uint4(a, b, c, d);
    return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ void store_out(void *y, int y_f32, size_t idx, float v) {
    if (y_f32)
        ((float *)y)[idx] = v;
    else
        ((uint16_t *)y)[idx] = to_bf16_bits(v);
}

// ---------------------------------------------------------------------------------------------
// Skinny kernel.  Lane l: col = l % 16 (B column / A row), kq = l / 16 (k quarter of a group).
// In MFMA j (0..3) of a group, k slot (kq, i) holds k = 128 g + 32 kq + 8 j + i for both operands.
// Output of v_mfma_f32_16x16x32_bf16: lane l, element r holds D[4 (l / 16) + r][l % 16].
//
// Memory pipeline: one stage holds everything a group needs (codes and meta of NT column tiles,
// and the lane's 64 bytes of activations for MT row tiles).  U stages are in flight; each stage
// is consumed in place and refilled with group i + U, and a scheduling barrier keeps the stages'
// loads in group order, so the in-order vmcnt wait for a stage never covers a younger one.  Rows
// past M read row M - 1 (their MFMA rows are discarded), so no load is predicated.
template <int MT, int NT>
struct W16Stage {
    uint4 w[NT];
    uint32_t meta[NT];
    uint4 a[MT][4];
};

template <int MT, int NT, int U, int MAXW>
__global__ void __launch_bounds__(64 * MAXW)
k_w4a16_skinny(const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
               const uint32_t *__restrict__ meta, int K, int N, void *__restrict__ y, int y_f32, int kw) {
    __shared__ float red[kMaxSplitWaves * 4 * 64];   // [kw][4][64]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int G = K / kGroup;
    const int g0 = (wave * G) / kw;
    const int ng = ((wave + 1) * G) / kw - g0;
    const int T = N / 16;
    const int tbase = blockIdx.x * NT;

    const uint8_t *wblk[NT];
    const uint32_t *mblk[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int t = min(tbase + nt, T - 1);                 // ragged tile tail: clamp the loads
        wblk[nt] = codes + ((size_t)t * G + g0) * 1024 + lane * 16;
        mblk[nt] = meta + ((size_t)t * G + g0) * 16 + col;
    }
    const uint16_t *xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        xrow[mt] = x + (size_t)min(16 * mt + col, M - 1) * K + (size_t)g0 * kGroup + kq * 32;

    auto load = [&](W16Stage<MT, NT> &st, int i) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            st.w[nt] = load_stream16(wblk[nt] + (size_t)i * 1024);
            st.meta[nt] = mblk[nt][(size_t)i * 16];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint4 *xp = (const uint4 *)(xrow[mt] + (size_t)i * kGroup);
#pragma unroll
            for (int j = 0; j < 4; ++j) st.a[mt][j] = xp[j];
        }
    };

    f32x4_t acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const W16Stage<MT, NT> &cur) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const DqConst dq = make_dq(cur.meta[nt]);
            const uint32_t words[4] = {cur.w[nt].x, cur.w[nt].y, cur.w[nt].z, cur.w[nt].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t b[4];
                dequant8(words[j], dq, b);
                const bf16x8_t bv = as_bf16x8(b[0], b[1], b[2], b[3]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, cur.a[mt][j]), bv, acc[mt][nt], 0, 0, 0);
            }
        }
    };

    // Steady state: full blocks of U groups, every stage refilled unconditionally (indices past
    // the end re-read the last group); the remaining ng % U groups are in registers afterwards.
    W16Stage<MT, NT> st[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        load(st[u], min(u, ng - 1));
        __builtin_amdgcn_sched_barrier(0);
    }
    const int nfull = ng - ng % U;
    for (int base = 0; base < nfull; base += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            compute(st[u]);
            load(st[u], min(base + u + U, ng - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int u = 0; u < U - 1; ++u)
        if (nfull + u < ng) compute(st[u]);

    // Fixed-order reduction of the kw wave partials, one 16x16 output tile at a time.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc[mt][nt][r];
            __syncthreads();
            for (int e = threadIdx.x; e < 256; e += blockDim.x) {
                const int r = e >> 6, l = e & 63;
                float sum = 0.f;
                for (int w = 0; w < kw; ++w) sum += red[(w * 4 + r) * 64 + l];
                const int m = 16 * mt + 4 * (l >> 4) + r;
                const int n = 16 * (tbase + nt) + (l & 15);
                if (m < M && n < N) store_out(y, y_f32, (size_t)m * N + n, sum);
            }
            __syncthreads();
        }
}

// ---------------------------------------------------------------------------------------------
// Tiled kernel for large M.  256 threads = 4 waves in a 2x2 arrangement over a 128x128 tile.
constexpr int TBM = 128, TBN = 128, TBK = kGroup;
constexpr int TLDS = TBK + 8;   // padded row pitch (bf16 elements) against bank conflicts

__global__ void __launch_bounds__(256)
k_w4a16_tiled(const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
              const uint32_t *__restrict__ meta, int K, int N, void *__restrict__ y, int y_f32) {
    __shared__ __attribute__((aligned(16))) uint16_t As[TBM * TLDS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[TBN * TLDS];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int col = lane & 15, kq = lane >> 4;
    const int G = K / kGroup;
    const int T = N / 16;
    const int m0 = blockIdx.y * TBM, n0 = blockIdx.x * TBN;

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int g = 0; g < G; ++g) {
        // activations: 128 rows x 128 k bf16 = 2048 uint4, 8 per thread
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int idx = tid + it * 256;
            const int r = idx >> 4, c = idx & 15;
            const int m = min(m0 + r, M - 1);
            *(uint4 *)(As + r * TLDS + c * 8) = *(const uint4 *)(x + (size_t)m * K + (size_t)g * kGroup + c * 8);
        }
        // weights: 8 column tiles x 1 KB = 512 uint4, 2 per thread; dequantized into LDS.  Chunk b
        // of a tile block holds column b % 16, k = 32 (b / 16) .. + 31 of the group.
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int idx = tid + it * 256;
            const int tj = idx >> 6, b = idx & 63;
            const int t = min(n0 / 16 + tj, T - 1);
            const uint4 w = load_stream16(codes + ((size_t)t * G + g) * 1024 + b * 16);
            const DqConst dq = make_dq(meta[((size_t)t * G + g) * 16 + (b & 15)]);
            const int r = tj * 16 + (b & 15), kc = (b >> 4) * 32;
            const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t bb[4];
                dequant8(words[j], dq, bb);
                *(uint4 *)(Bs + r * TLDS + kc + j * 8) = make_uint4(bb[0], bb[1], bb[2], bb[3]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < TBK / 32; ++ks) {
            bf16x8_t af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 64 + i * 16 + col;
                af[i] = __builtin_bit_cast(bf16x8_t, *(const uint4 *)(As + r * TLDS + ks * 32 + kq * 8));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = wn * 64 + j * 16 + col;
                bfr[j] = __builtin_bit_cast(bf16x8_t, *(const uint4 *)(Bs + r * TLDS + ks * 32 + kq * 8));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + i * 16 + 4 * kq + r;
                const int n = n0 + wn * 64 + j * 16 + col;
                if (m < M && n < N) store_out(y, y_f32, (size_t)m * N + n, acc[i][j][r]);
            }
}

// ---------------------------------------------------------------------------------------------
// Host launchers.

template <int MT, int NT, int U, int MAXW>
static hipError_t launch_skinny(const uint16_t *x, int M, const uint8_t *codes, const uint32_t *meta,
                                int K, int N, void *y, int y_f32, hipStream_t st) {
    const int kw = min(skinny_waves_for_shape(K, N), MAXW);
    const int T = N / 16;
    dim3 grid((T + NT - 1) / NT);
    dim3 block(64 * kw);
    hipLaunchKernelGGL((k_w4a16_skinny<MT, NT, U, MAXW>), grid, block, 0, st, x, M, codes, meta, K, N, y,
                       y_f32, kw);
    return hipGetLastError();
}

hipError_t launch_gemm_w4a16(const uint16_t *x, int M, const uint8_t *codes, const uint32_t *meta, int K,
                             int N, void *y, int y_f32, hipStream_t st) {
    // Two batch tiers, each with one reduction order for all its M: M <= 16 and 16 < M <= 80
    // (the latter at most 4 waves per tile, so its larger activation stages fit in registers).
    if (M <= 16) return launch_skinny<1, 1, 4, kMaxSplitWaves>(x, M, codes, meta, K, N, y, y_f32, st);
    if (M <= 32) return launch_skinny<2, 2, 2, 4>(x, M, codes, meta, K, N, y, y_f32, st);
    if (M <= 48) return launch_skinny<3, 2, 2, 4>(x, M, codes, meta, K, N, y, y_f32, st);
    if (M <= 64) return launch_skinny<4, 2, 2, 4>(x, M, codes, meta, K, N, y, y_f32, st);
    if (M <= 80) return launch_skinny<5, 2, 2, 4>(x, M, codes, meta, K, N, y, y_f32, st);
    dim3 grid((N + TBN - 1) / TBN, (M + TBM - 1) / TBM);
    hipLaunchKernelGGL(k_w4a16_tiled, grid, dim3(256), 0, st, x, M, codes, meta, K, N, y, y_f32);
    return hipGetLastError();
}

}  // namespace qspec
