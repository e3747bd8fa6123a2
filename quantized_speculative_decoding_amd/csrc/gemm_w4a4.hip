// W4A4 draft linear layer on gfx950.
//
//   D[g][m][n] = sum_{k in g} q_a[m][k] * (w[k][n] - z[n][g])   exact in int32
//   y[m][n]    = sum_g s_a[m][g] * s[n][g] * D[g][m][n]          fp32 accumulation
// (QSPEC notes, background terms: the 4-bit MACs accumulate in INT32 and the scale is applied
//  afterwards; QSPEC structure: the draft runs W4A4 on the verifier's 4-bit weights.)
//
// CDNA4 has no 4-bit integer MFMA, so both operands are widened to int8 in registers (two SWAR
// ops per 4 codes) and fed to v_mfma_i32_16x16x64_i8, whose int32 sums are exact.
//  * k_w4a4_skinny (M <= 64): HBM-bound draft shapes.  Same work split as the W4A16 skinny
//    kernel: 16*NT columns per workgroup, KW waves splitting the K groups, U groups of weight
//    loads in flight, fixed-order LDS reduction of the wave partials.  Weights stay unsigned
//    (0..15) and the zero point is applied after the MFMA as D = sum(q_a w) - z sum(q_a); the
//    per-(token, group) code sums come from one extra MFMA against a matrix of ones, which lands
//    them in the accumulator layout.
//  * k_w4a4_tiled (M > 64): 128x128 tiles per workgroup; the codes of one K group are widened
//    into LDS once (weights as signed w - z), 4 waves each own a 64x64 sub-tile.
#include "common.hpp"
#include "kernels.hpp"

namespace qspec {

// Unsigned codes: bytes hold the even-k (lo) or odd-k (hi) nibbles of a dword of 8 codes.
__device__ __forceinline__ uint32_t nib_lo(uint32_t d) { return d & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t nib_hi(uint32_t d) { return (d >> 4) & 0x0F0F0F0Fu; }

// Signed (two's complement) nibbles widened to signed bytes without cross-byte borrows:
// t = n ^ 8 is the code plus 8; (t | 0x80) - 8 = v + 128 stays in [120, 135]; ^0x80 gives v.
__device__ __forceinline__ uint32_t snib_lo(uint32_t e) {
    return (((e & 0x0F0F0F0Fu) ^ 0x88888888u) - 0x08080808u) ^ 0x80808080u;
}
__device__ __forceinline__ uint32_t snib_hi(uint32_t e) { return snib_lo(e >> 4); }

// Unsigned weight nibbles minus a zero point, as signed bytes: (w | 0x80) - z in [113, 143].
__device__ __forceinline__ uint32_t wz_bytes(uint32_t lo_nibbles, uint32_t zz) {
    return ((lo_nibbles | 0x80808080u) - zz) ^ 0x80808080u;
}

__device__ __forceinline__ i32x4_t as_i32x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return i32x4_t{(int)a, (int)b, (int)c, (int)d};
}

__device__ __forceinline__ void store_out4(void *y, int y_f32, size_t idx, float v) {
    if (y_f32)
        ((float *)y)[idx] = v;
    else
        ((uint16_t *)y)[idx] = to_bf16_bits(v);
}

// ---------------------------------------------------------------------------------------------
// Skinny kernel.  Lane l: col = l % 16, kq = l / 16.  A group's 128 codes split into 4 lane
// quarters of 32; MFMA j (0, 1) takes the lane's codes 16 j .. 16 j + 15 of its quarter, in the
// order [even k of dword 2j, odd k of dword 2j, even k of dword 2j+1, odd k of dword 2j+1] for
// both operands.  Output of v_mfma_i32_16x16x64_i8: lane l, element r holds D[4 (l/16) + r][l%16].
template <int MT, int NT, int U>
__global__ void __launch_bounds__(512)
k_w4a4_skinny(const uint8_t *__restrict__ a_codes, const float *__restrict__ a_scales, int M,
              const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
              const uint8_t *__restrict__ zeros, int K, int N, void *__restrict__ y, int y_f32,
              int32_t *__restrict__ dots, int kw) {
    __shared__ float red[8 * 4 * 64];   // [kw <= 8][4][64]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int G = K / kGroup;
    const int g0 = (wave * G) / kw;
    const int ng = ((wave + 1) * G) / kw - g0;
    const int nbase = blockIdx.x * 16 * NT;
    const size_t row_bytes = (size_t)K / 2;
    const i32x4_t ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    const i32x4_t izero = {0, 0, 0, 0};

    f32x4_t acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const uint8_t *wrow[NT];
    const uint16_t *srow[NT];
    const uint8_t *zrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        int n = nbase + 16 * nt + col;
        n = n < N ? n : N - 1;
        wrow[nt] = codes + (size_t)n * row_bytes + (size_t)g0 * 64 + kq * 16;
        srow[nt] = scales + (size_t)n * G + g0;
        zrow[nt] = zeros + (size_t)n * G + g0;
    }
    // A operand rows (one per lane) and the output rows whose activation scales this lane needs.
    const uint8_t *arow[MT];
    bool avalid[MT];
    const float *asrow[MT][4];
    bool ovalid[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + col;
        avalid[mt] = m < M;
        arow[mt] = a_codes + (size_t)(avalid[mt] ? m : 0) * row_bytes + (size_t)g0 * 64 + kq * 16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int mo = 16 * mt + 4 * kq + r;
            ovalid[mt][r] = mo < M;
            asrow[mt][r] = a_scales + (size_t)(ovalid[mt][r] ? mo : 0) * G + g0;
        }
    }

    uint4 wbuf[U][NT];
    uint16_t sbuf[U][NT];
    uint8_t zbuf[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (u < ng)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                wbuf[u][nt] = load_stream16(wrow[nt] + u * 64);
                sbuf[u][nt] = srow[nt][u];
                zbuf[u][nt] = zrow[nt][u];
            }

    for (int base = 0; base < ng; base += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u;
            if (i < ng) {
                i32x4_t A0[MT], A1[MT], sa[MT];
                float as[MT][4];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    // rows past M read as code 0, so they add nothing to any sum
                    const uint4 e = avalid[mt] ? *(const uint4 *)(arow[mt] + (size_t)i * 64)
                                               : make_uint4(0, 0, 0, 0);
                    A0[mt] = as_i32x4(snib_lo(e.x), snib_hi(e.x), snib_lo(e.y), snib_hi(e.y));
                    A1[mt] = as_i32x4(snib_lo(e.z), snib_hi(e.z), snib_lo(e.w), snib_hi(e.w));
                    sa[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0[mt], ones, izero, 0, 0, 0);
                    sa[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1[mt], ones, sa[mt], 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) as[mt][r] = ovalid[mt][r] ? asrow[mt][r][i] : 0.f;
                }
                uint4 cur[NT];
                float sw[NT];
                int zw[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    cur[nt] = wbuf[u][nt];
                    sw[nt] = fp16_bits_to_float(sbuf[u][nt]);
                    zw[nt] = zbuf[u][nt];
                }
                if (i + U < ng) {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        wbuf[u][nt] = load_stream16(wrow[nt] + (size_t)(i + U) * 64);
                        sbuf[u][nt] = srow[nt][i + U];
                        zbuf[u][nt] = zrow[nt][i + U];
                    }
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const uint4 d = cur[nt];
                    const i32x4_t B0 = as_i32x4(nib_lo(d.x), nib_hi(d.x), nib_lo(d.y), nib_hi(d.y));
                    const i32x4_t B1 = as_i32x4(nib_lo(d.z), nib_hi(d.z), nib_lo(d.w), nib_hi(d.w));
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        i32x4_t ia = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0[mt], B0, izero, 0, 0, 0);
                        ia = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1[mt], B1, ia, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int Dv = ia[r] - zw[nt] * sa[mt][r];
                            acc[mt][nt][r] = __builtin_fmaf(as[mt][r] * sw[nt], (float)Dv, acc[mt][nt][r]);
                            if (dots) {
                                const int mo = 16 * mt + 4 * kq + r;
                                const int n = nbase + 16 * nt + col;
                                if (mo < M && n < N)
                                    dots[((size_t)(g0 + i) * M + mo) * N + n] = Dv;
                            }
                        }
                    }
                }
            }
        }
    }

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
                float s = 0.f;
                for (int w = 0; w < kw; ++w) s += red[(w * 4 + r) * 64 + l];
                const int m = 16 * mt + 4 * (l >> 4) + r;
                const int n = nbase + 16 * nt + (l & 15);
                if (m < M && n < N) store_out4(y, y_f32, (size_t)m * N + n, s);
            }
            __syncthreads();
        }
}

// ---------------------------------------------------------------------------------------------
// Tiled kernel for large M.  256 threads = 4 waves (2x2) over a 128x128 output tile.
constexpr int QBM = 128, QBN = 128;
constexpr int QLDS = kGroup + 16;   // padded row pitch in bytes

__global__ void __launch_bounds__(256)
k_w4a4_tiled(const uint8_t *__restrict__ a_codes, const float *__restrict__ a_scales, int M,
             const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
             const uint8_t *__restrict__ zeros, int K, int N, void *__restrict__ y, int y_f32,
             int32_t *__restrict__ dots) {
    __shared__ __attribute__((aligned(16))) uint8_t As[QBM * QLDS];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[QBN * QLDS];
    __shared__ float sA[QBM], sB[QBN];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int col = lane & 15, kq = lane >> 4;
    const int G = K / kGroup;
    const size_t row_bytes = (size_t)K / 2;
    const int m0 = blockIdx.y * QBM, n0 = blockIdx.x * QBN;
    const i32x4_t izero = {0, 0, 0, 0};

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int g = 0; g < G; ++g) {
        // 128 rows x 64 bytes of codes per operand = 512 uint4 each, 2 + 2 per thread.
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int idx = tid + it * 256;
            const int r = idx >> 2, c = idx & 3;
            const int m = m0 + r;
            uint4 e = make_uint4(0, 0, 0, 0);
            if (m < M) e = *(const uint4 *)(a_codes + (size_t)m * row_bytes + (size_t)g * 64 + c * 16);
            uint4 *dst = (uint4 *)(As + r * QLDS + c * 32);   // rows past M stay code 0
            dst[0] = make_uint4(snib_lo(e.x), snib_hi(e.x), snib_lo(e.y), snib_hi(e.y));
            dst[1] = make_uint4(snib_lo(e.z), snib_hi(e.z), snib_lo(e.w), snib_hi(e.w));

            int n = n0 + r;
            n = n < N ? n : N - 1;
            const uint4 d = load_stream16(codes + (size_t)n * row_bytes + (size_t)g * 64 + c * 16);
            const uint32_t zz = (uint32_t)zeros[(size_t)n * G + g] * 0x01010101u;
            uint4 *bd = (uint4 *)(Bs + r * QLDS + c * 32);
            bd[0] = make_uint4(wz_bytes(nib_lo(d.x), zz), wz_bytes(nib_hi(d.x), zz),
                               wz_bytes(nib_lo(d.y), zz), wz_bytes(nib_hi(d.y), zz));
            bd[1] = make_uint4(wz_bytes(nib_lo(d.z), zz), wz_bytes(nib_hi(d.z), zz),
                               wz_bytes(nib_lo(d.w), zz), wz_bytes(nib_hi(d.w), zz));
        }
        if (tid < QBM) {
            const int m = m0 + tid;
            sA[tid] = m < M ? a_scales[(size_t)m * G + g] : 0.f;
        } else {
            int n = n0 + tid - QBM;
            n = n < N ? n : N - 1;
            sB[tid - QBM] = fp16_bits_to_float(scales[(size_t)n * G + g]);
        }
        __syncthreads();
        i32x4_t ia[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) ia[i][j] = izero;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            i32x4_t af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 v = *(const uint4 *)(As + (wm * 64 + i * 16 + col) * QLDS + ks * 64 + kq * 16);
                af[i] = as_i32x4(v.x, v.y, v.z, v.w);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 v = *(const uint4 *)(Bs + (wn * 64 + j * 16 + col) * QLDS + ks * 64 + kq * 16);
                bfr[j] = as_i32x4(v.x, v.y, v.z, v.w);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    ia[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bfr[j], ia[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float sbj = sB[wn * 64 + j * 16 + col];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ml = wm * 64 + i * 16 + 4 * kq + r;
                    acc[i][j][r] = __builtin_fmaf(sA[ml] * sbj, (float)ia[i][j][r], acc[i][j][r]);
                    if (dots) {
                        const int m = m0 + ml, n = n0 + wn * 64 + j * 16 + col;
                        if (m < M && n < N) dots[((size_t)g * M + m) * N + n] = ia[i][j][r];
                    }
                }
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
                if (m < M && n < N) store_out4(y, y_f32, (size_t)m * N + n, acc[i][j][r]);
            }
}

// ---------------------------------------------------------------------------------------------

template <int MT, int NT>
static hipError_t launch_skinny4(const uint8_t *a_codes, const float *a_scales, int M,
                                 const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                                 int K, int N, void *y, int y_f32, int32_t *dots, hipStream_t st) {
    constexpr int U = 4;
    const int kw = skinny_waves_for_shape(K, N);
    const int cols = 16 * NT;
    dim3 grid((N + cols - 1) / cols);
    dim3 block(64 * kw);
    hipLaunchKernelGGL((k_w4a4_skinny<MT, NT, U>), grid, block, 0, st, a_codes, a_scales, M, codes,
                       scales, zeros, K, N, y, y_f32, dots, kw);
    return hipGetLastError();
}

hipError_t launch_gemm_w4a4(const uint8_t *a_codes, const float *a_scales, int M,
                            const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                            int K, int N, void *y, int y_f32, int32_t *group_dots, hipStream_t st) {
    if (M <= 16)
        return launch_skinny4<1, 1>(a_codes, a_scales, M, codes, scales, zeros, K, N, y, y_f32, group_dots, st);
    if (M <= 32)
        return launch_skinny4<2, 1>(a_codes, a_scales, M, codes, scales, zeros, K, N, y, y_f32, group_dots, st);
    if (M <= 64)
        return launch_skinny4<4, 1>(a_codes, a_scales, M, codes, scales, zeros, K, N, y, y_f32, group_dots, st);
    dim3 grid((N + QBN - 1) / QBN, (M + QBM - 1) / QBM);
    hipLaunchKernelGGL(k_w4a4_tiled, grid, dim3(256), 0, st, a_codes, a_scales, M, codes, scales, zeros,
                       K, N, y, y_f32, group_dots);
    return hipGetLastError();
}

}  // namespace qspec
