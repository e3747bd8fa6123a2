// The FP8 parent variant on gfx950 (SpecQuant notes, one-line summary, key contributions and
// approach: INT4, FP8 and FP16 variants of one model by post-training quantization with shared
// base weights; a draft proposes and a parent variant verifies).  FP8 is OCP E4M3 (bias 7, no
// infinities, largest finite 448); weights carry one scale per output column, activations one
// per token, both absmax / 448; y = s_a[m] s_w[n] sum_k dec(a[m][k]) dec(w[k][n]).
//
//   k_quantize_act_fp8  one workgroup per token: the row's absmax, s = absmax / 448 (one binary32
//                       division), codes = E4M3(x / s) rounded to nearest even, saturating; the row
//                       stays in registers between the two passes.
//   k_w8a8              v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E4M3 and unit
//                       scales: products of E4M3 values are exact, sums fp32.  Lane l = c + 16 q
//                       holds 32 consecutive k (128 g + 32 q + 0..31) of its A row and of its B
//                       column, so the activation row and the weight store feed the MFMA without
//                       any reordering; a wave owns two column tiles over one K split.
#include "common.hpp"
#include "kernels.hpp"

namespace qspec {

constexpr int kW8Waves = 4;              // waves per workgroup
constexpr int kW8NT = 2;                 // 16-column tiles per wave
constexpr int kW8MaxMT = 5;              // 16-row tiles per workgroup (M <= 80 in one pass)
constexpr int kW8MaxSplits = 16;         // the split-K reduce adds at most 16 partials
constexpr int kW8Ring = 4;               // register ring depth (groups in flight per wave), MT <= 2
constexpr int kW8TargetWaves = 2048;     // K splits aim at this many waves

typedef __attribute__((ext_vector_type(8))) int w8_i32x8_t;

// One workgroup of kQThreads per token.  Rows of up to kQThreads * 8 * kQCache elements are read
// once and kept in registers for the second pass; longer rows are read again.
constexpr int kQThreads = 1024;
constexpr int kQCache = 4;

__global__ void __launch_bounds__(kQThreads)
k_quantize_act_fp8(const uint16_t *__restrict__ x, int K, uint8_t *__restrict__ codes, float *__restrict__ scales) {
    __shared__ float red[kQThreads / kWave];
    const int m = blockIdx.x;
    const uint16_t *xr = x + (size_t)m * K;
    constexpr int STEP = kQThreads * 8;
    uint4 keep[kQCache];
    float a = 0.f;
    auto absmax8 = [](uint4 u, float acc) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = fmaxf(acc, fmaxf(fabsf(bf16_bits_to_float(w[i] & 0xFFFFu)), fabsf(bf16_bits_to_float(w[i] >> 16))));
        return acc;
    };
#pragma unroll
    for (int it = 0; it < kQCache; ++it) {
        const int k = it * STEP + threadIdx.x * 8;
        keep[it] = k < K ? *(const uint4 *)(xr + k) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int it = 0; it < kQCache; ++it) a = absmax8(keep[it], a);
    for (int k = kQCache * STEP + threadIdx.x * 8; k < K; k += STEP) a = absmax8(*(const uint4 *)(xr + k), a);
    a = wave_max(a);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = red[0];
#pragma unroll
    for (int i = 1; i < kQThreads / kWave; ++i) a = fmaxf(a, red[i]);
    const float s = a / 448.0f;
    if (threadIdx.x == 0) scales[m] = s;
    auto encode8 = [&](uint4 u, int k) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
        uint32_t out[2] = {0u, 0u};
        if (a != 0.f) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = f32_to_e4m3(bf16_bits_to_float(w[i] & 0xFFFFu) / s);
                const uint32_t hi = f32_to_e4m3(bf16_bits_to_float(w[i] >> 16) / s);
                out[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
            }
        }
        *(uint2 *)(codes + (size_t)m * K + k) = make_uint2(out[0], out[1]);
    };
#pragma unroll
    for (int it = 0; it < kQCache; ++it) {
        const int k = it * STEP + threadIdx.x * 8;
        if (k < K) encode8(keep[it], k);
    }
    for (int k = kQCache * STEP + threadIdx.x * 8; k < K; k += STEP) encode8(*(const uint4 *)(xr + k), k);
}

// K splits: a function of (K, N) only (so a row's sum order does not depend on M).  Enough
// splits for about kW8TargetWaves waves, at least 4 groups per split, at most 16.
static int w8a8_splits(int K, int N) {
    const int G = K / kGroup;
    const int wave_cols = (N / 16 + kW8NT - 1) / kW8NT;
    int S = min(min((kW8TargetWaves + wave_cols - 1) / wave_cols, kW8MaxSplits), max(1, G / 4));
    S = max(S, 1);
    const int gps = (G + S - 1) / S;
    return (G + gps - 1) / gps;                                  // no empty split
}

size_t gemm_w8a8_workspace_bytes(int M, int K, int N) {
    const int S = w8a8_splits(K, N);
    return S == 1 ? 0 : (size_t)S * M * N * sizeof(float);
}

// One workgroup: kW8Waves waves x kW8NT column tiles, MT row tiles from row 16 MT rb, one K split.
// out = y (S == 1) or the split's partials [S][M][N] (scaled; the reduce adds them in split order).
template <int MT>
__global__ void __launch_bounds__(kW8Waves * kWave)
k_w8a8(const uint8_t *__restrict__ a_codes, const float *__restrict__ a_scales, int M,
       const uint8_t *__restrict__ w_store, const float *__restrict__ w_scales, int K, int N, int S, int RB,
       void *__restrict__ out, int out_f32) {
    const int G = K / kGroup;
    const int t = blockIdx.x;
    const int rb = t % RB, split = (t / RB) % S, cb = t / RB / S;
    const int lane = threadIdx.x & 63, c = lane & 15, kq = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tile0 = (cb * kW8Waves + w) * kW8NT;                 // first column tile of the wave
    if (tile0 >= N / 16) return;
    const int gps = (G + S - 1) / S;
    const int g0 = split * gps, g1 = min(G, g0 + gps);
    const int row0 = rb * 16 * MT;

    const rsrc_t ar = make_rsrc(a_codes, (uint32_t)((size_t)M * K));
    const rsrc_t wr = make_rsrc(w_store, (uint32_t)((size_t)K * N));
    uint32_t aoff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) aoff[mt] = (uint32_t)min(row0 + 16 * mt + c, M - 1) * (uint32_t)K + 32u * kq;
    uint32_t woff[kW8NT];
#pragma unroll
    for (int nt = 0; nt < kW8NT; ++nt)
        woff[nt] = (uint32_t)min(tile0 + nt, N / 16 - 1) * (uint32_t)G * 2048u + 16u * lane;

    struct Stage {
        uint4 a[MT][2], b[kW8NT][2];
    };
    auto load = [&](int g, Stage &st) {
#pragma unroll
        for (int nt = 0; nt < kW8NT; ++nt)
#pragma unroll
            for (int h = 0; h < 2; ++h) st.b[nt][h] = buf_load16(wr, woff[nt] + 1024u * h, (uint32_t)g * 2048u);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int h = 0; h < 2; ++h) st.a[mt][h] = buf_load16(ar, aoff[mt] + 16u * h, (uint32_t)g * 128u);
    };
    f32x4_t acc[MT][kW8NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kW8NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // U-deep register ring: group g's loads are issued U - 1 groups ahead of its MFMAs (two deep
    // for three or more row tiles, whose stages are larger)
    constexpr int U = MT <= 2 ? kW8Ring : 2;
    Stage st[U];
#pragma unroll
    for (int u = 0; u + 1 < U; ++u)
        if (g0 + u < g1) load(g0 + u, st[u]);
    for (int gb = g0; gb < g1; gb += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = gb + u;
            if (g < g1) {
                if (g + U - 1 < g1) load(g + U - 1, st[(u + U - 1) % U]);
                const Stage &cur = st[u];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const w8_i32x8_t av = {(int)cur.a[mt][0].x, (int)cur.a[mt][0].y, (int)cur.a[mt][0].z,
                                           (int)cur.a[mt][0].w, (int)cur.a[mt][1].x, (int)cur.a[mt][1].y,
                                           (int)cur.a[mt][1].z, (int)cur.a[mt][1].w};
#pragma unroll
                    for (int nt = 0; nt < kW8NT; ++nt) {
                        const w8_i32x8_t bv = {(int)cur.b[nt][0].x, (int)cur.b[nt][0].y, (int)cur.b[nt][0].z,
                                               (int)cur.b[nt][0].w, (int)cur.b[nt][1].x, (int)cur.b[nt][1].y,
                                               (int)cur.b[nt][1].z, (int)cur.b[nt][1].w};
                        // formats 0, 0: both operands E4M3; E8M0 scales 127 = 2^0
                        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[mt][nt], 0, 0, 0,
                                                                                        127, 0, 127);
                    }
                }
            }
        }
    }

    // lane l, element e holds D[4 kq + e][c]: row row0 + 16 mt + 4 kq + e, column 16 tile + c
    float *part = S > 1 ? (float *)out + (size_t)split * M * N : nullptr;
#pragma unroll
    for (int nt = 0; nt < kW8NT; ++nt) {
        const int tile = tile0 + nt;
        if (tile >= N / 16) break;
        const int n = 16 * tile + c;
        const float sw = w_scales[n];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = row0 + 16 * mt + 4 * kq + e;
                if (m >= M) continue;
                const float v = acc[mt][nt][e] * (a_scales[m] * sw);
                const size_t idx = (size_t)m * N + n;
                if (part)
                    part[idx] = v;
                else if (out_f32)
                    ((float *)out)[idx] = v;
                else
                    ((uint16_t *)out)[idx] = to_bf16_bits(v);
            }
    }
}

hipError_t launch_quantize_act_fp8(const uint16_t *x, int M, int K, uint8_t *codes, float *scales, hipStream_t st) {
    hipLaunchKernelGGL(k_quantize_act_fp8, dim3(M), dim3(kQThreads), 0, st, x, K, codes, scales);
    return hipGetLastError();
}

template <int MT>
static void launch_w8a8_mt(const uint8_t *a, const float *as, int M, const uint8_t *w, const float *ws_, int K, int N,
                           int S, void *out, int out_f32, hipStream_t st) {
    const int RB = (M + 16 * MT - 1) / (16 * MT);
    const int wave_cols = (N / 16 + kW8NT - 1) / kW8NT;
    const int cbs = (wave_cols + kW8Waves - 1) / kW8Waves;
    hipLaunchKernelGGL(k_w8a8<MT>, dim3(cbs * S * RB), dim3(kW8Waves * kWave), 0, st, a, as, M, w, ws_, K, N, S, RB,
                       out, out_f32);
}

hipError_t launch_gemm_w8a8(const uint8_t *a_codes, const float *a_scales, int M, const uint8_t *w_store,
                            const float *w_scales, int K, int N, void *y, int y_f32, void *workspace,
                            hipStream_t st) {
    const int S = w8a8_splits(K, N);
    void *out = S > 1 ? workspace : y;
    const int MT = M <= 16 ? 1 : M <= 32 ? 2 : M <= 48 ? 3 : M <= 64 ? 4 : 5;
    switch (MT) {
    case 1: launch_w8a8_mt<1>(a_codes, a_scales, M, w_store, w_scales, K, N, S, out, y_f32, st); break;
    case 2: launch_w8a8_mt<2>(a_codes, a_scales, M, w_store, w_scales, K, N, S, out, y_f32, st); break;
    case 3: launch_w8a8_mt<3>(a_codes, a_scales, M, w_store, w_scales, K, N, S, out, y_f32, st); break;
    case 4: launch_w8a8_mt<4>(a_codes, a_scales, M, w_store, w_scales, K, N, S, out, y_f32, st); break;
    default: launch_w8a8_mt<5>(a_codes, a_scales, M, w_store, w_scales, K, N, S, out, y_f32, st); break;
    }
    if (S > 1) launch_splitk_reduce((const float *)workspace, S, M, N, y, y_f32, st);
    return hipGetLastError();
}

}  // namespace qspec
