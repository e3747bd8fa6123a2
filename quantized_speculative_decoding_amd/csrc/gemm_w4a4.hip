// W4A4 draft linear layer on gfx950.
//
//   D[g][m][n] = sum_{k in g} q_a[m][k] * (w[k][n] - z[n][g])   exact in int32
//   y[m][n]    = sum_g s_a[m][g] * s[n][g] * D[g][m][n]          fp32 accumulation
// (QSPEC notes, background terms: the 4-bit MACs accumulate in INT32 and the scale is applied
//  afterwards; QSPEC structure: the draft runs W4A4 on the verifier's 4-bit weights.)
//
// CDNA4 has no 4-bit integer MFMA, so both operands are widened to int8 in registers (two SWAR
// ops per 4 codes) and fed to v_mfma_i32_16x16x64_i8, whose int32 sums are exact.
//  * k_w4a4_decode (M <= 16) and k_w4a4_skinny (16 < M <= 64): HBM-bound draft shapes.  A
//    workgroup owns 16 NT columns, KW waves split the K groups, U groups of weight loads stay in
//    flight, and the wave partials are reduced through LDS in a fixed order.  Weights stay
//    unsigned (0..15) and the zero point is applied after the MFMA as
//    D = sum(q_a w) - z sum(q_a); the per-(token, group) code sums come from one extra MFMA
//    against a matrix of ones, which lands them in the accumulator layout.
//  * k_w4a4_lds (M > 64): 64-row blocks; the block's activation codes are widened once per group
//    into LDS and shared by the workgroup's waves, weights are widened as signed w - z in the
//    registers of the wave that feeds them to the MFMA.
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
// quarters of 32 (the tile-major block gives lane l exactly bytes 16 l .. 16 l + 15); MFMA j
// (0, 1) takes the lane's codes 16 j .. 16 j + 15 of its quarter, in the order [even k of dword
// 2j, odd k of dword 2j, even k of dword 2j+1, odd k of dword 2j+1] for both operands.  Output of
// v_mfma_i32_16x16x64_i8: lane l, element r holds D[4 (l/16) + r][l%16].
// The memory pipeline is the one of the W4A16 skinny kernel: a stage holds one group's codes and
// meta of NT column tiles plus the activation codes and scales of MT row tiles; U stages stay in
// flight; rows past M read row M - 1 and are discarded.
template <int MT, int NT>
struct W4Stage {
    uint4 w[NT];
    uint32_t meta[NT];
    uint4 a[MT];
    float as[MT][4];
};

template <int MT, int NT, int U, int MAXW, bool DOTS>
__global__ void __launch_bounds__(64 * MAXW)
k_w4a4_skinny(const uint8_t *__restrict__ a_codes, const float *__restrict__ a_scales, int M,
              const uint8_t *__restrict__ codes, const uint32_t *__restrict__ meta, int K, int N,
              void *__restrict__ y, int y_f32, int32_t *__restrict__ dots, int kw) {
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
    const size_t row_bytes = (size_t)K / 2;
    const i32x4_t ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    const i32x4_t izero = {0, 0, 0, 0};

    const uint8_t *wblk[NT];
    const uint32_t *mblk[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int t = min(tbase + nt, T - 1);
        wblk[nt] = codes + ((size_t)t * G + g0) * 1024 + lane * 16;
        mblk[nt] = meta + ((size_t)t * G + g0) * 16 + col;
    }
    // A operand row of this lane, and the output rows whose activation scales it needs.
    const uint8_t *arow[MT];
    const float *asrow[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        arow[mt] = a_codes + (size_t)min(16 * mt + col, M - 1) * row_bytes + (size_t)g0 * 64 + kq * 16;
#pragma unroll
        for (int r = 0; r < 4; ++r) asrow[mt][r] = a_scales + (size_t)min(16 * mt + 4 * kq + r, M - 1) * G + g0;
    }

    auto load = [&](W4Stage<MT, NT> &st, int i) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            st.w[nt] = load_stream16(wblk[nt] + (size_t)i * 1024);
            st.meta[nt] = mblk[nt][(size_t)i * 16];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            st.a[mt] = *(const uint4 *)(arow[mt] + (size_t)i * 64);
#pragma unroll
            for (int r = 0; r < 4; ++r) st.as[mt][r] = asrow[mt][r][i];
        }
    };

    f32x4_t acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const W4Stage<MT, NT> &cur, int i) {
        i32x4_t A0[MT], A1[MT], sa[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint4 e = cur.a[mt];
            A0[mt] = as_i32x4(snib_lo(e.x), snib_hi(e.x), snib_lo(e.y), snib_hi(e.y));
            A1[mt] = as_i32x4(snib_lo(e.z), snib_hi(e.z), snib_lo(e.w), snib_hi(e.w));
            sa[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0[mt], ones, izero, 0, 0, 0);
            sa[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1[mt], ones, sa[mt], 0, 0, 0);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const uint4 d = cur.w[nt];
            const float sw = fp16_bits_to_float((uint16_t)(cur.meta[nt] & 0xFFFFu));
            const int zw = (int)((cur.meta[nt] >> 16) & 0xFFu);
            const i32x4_t B0 = as_i32x4(nib_lo(d.x), nib_hi(d.x), nib_lo(d.y), nib_hi(d.y));
            const i32x4_t B1 = as_i32x4(nib_lo(d.z), nib_hi(d.z), nib_lo(d.w), nib_hi(d.w));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                i32x4_t ia = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0[mt], B0, izero, 0, 0, 0);
                ia = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1[mt], B1, ia, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int Dv = ia[r] - __mul24(zw, sa[mt][r]);   // |z sa| <= 15 * 896: 24-bit product
                    acc[mt][nt][r] = __builtin_fmaf(cur.as[mt][r] * sw, (float)Dv, acc[mt][nt][r]);
                    if (DOTS) {
                        const int mo = 16 * mt + 4 * kq + r;
                        const int n = 16 * (tbase + nt) + col;
                        if (mo < M && n < N) dots[((size_t)(g0 + i) * M + mo) * N + n] = Dv;
                    }
                }
            }
        }
    };

    W4Stage<MT, NT> st[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        load(st[u], min(u, ng - 1));
        __builtin_amdgcn_sched_barrier(0);
    }
    // Steady passes refill every slot with a real group; the last pass refills only the slots
    // whose group exists, and the drain consumes them.
    int base = 0;
    for (; base + 2 * U <= ng; base += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            compute(st[u], base + u);
            load(st[u], base + u + U);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (base + u < ng) compute(st[u], base + u);
        if (base + u + U < ng) load(st[u], base + u + U);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < U - 1; ++u)
        if (base + U + u < ng) compute(st[u], base + U + u);

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
                if (m < M && n < N) store_out4(y, y_f32, (size_t)m * N + n, sum);
            }
            __syncthreads();
        }
}

// ---------------------------------------------------------------------------------------------
// Decode kernel (M <= 16): one row tile, NT column tiles per wave.  A workgroup owns NT tiles and
// KW waves split the K groups; each wave widens the group's activation codes once and feeds them
// to the 2 NT MFMAs of its tiles (plus the two against ones for the code sums).  Loads are buffer
// loads from wave-uniform bases; U groups stay in flight in a register ring; wave partials are
// summed through LDS in wave order (the reduction order depends on (K, N) only).
// Activation scales: a wave reads those of up to kScaleChunk of its groups at once, 16 groups of
// one row per lane and 16-byte load, and parks them in its own LDS region as [group][row]; a
// group then costs one ds_read_b128 (the four rows a lane's outputs hold) instead of four 4-byte
// loads that touch 16 lines.  The region is private to the wave, so no barrier guards it: a
// wave's LDS accesses execute in program order.
constexpr int kScaleChunk = 64;

template <int NT>
struct W4DStage {
    uint4 w[NT];
    uint32_t meta[NT];
    uint4 a;
};

// Groups per wave-private scale chunk, and the decode kernel's dynamic LDS bytes.
__host__ __device__ inline int decode_scale_chunk(int G, int kw) {
    const int per_wave = (G + kw - 1) / kw;
    return per_wave < kScaleChunk ? per_wave : kScaleChunk;
}

__host__ inline size_t decode4_lds_bytes(int G, int kw, int NT) {
    return ((size_t)kw * NT * 256 + (size_t)kw * decode_scale_chunk(G, kw) * 16) * sizeof(float);
}

template <int NT, int U, bool DOTS>
__global__ void __launch_bounds__(64 * kMaxDecodeWaves)
k_w4a4_decode(const uint8_t *__restrict__ a_codes, const float *__restrict__ a_scales, int M,
              const uint8_t *__restrict__ codes, const uint32_t *__restrict__ meta, int K, int N,
              void *__restrict__ y, int y_f32, int32_t *__restrict__ dots, int kw) {
    // dynamic LDS: red [kw][NT][4][64] floats, then per wave a scale chunk [sch][16] floats
    extern __shared__ __attribute__((aligned(16))) float red[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int G = K / kGroup;
    const int sch = decode_scale_chunk(G, kw);
    float *const sl = red + kw * NT * 256 + wave * sch * 16;
    const int g0 = (wave * G) / kw;
    const int ng = ((wave + 1) * G) / kw - g0;
    const int T = N / 16;
    const int tbase = blockIdx.x * NT;
    const i32x4_t ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    const i32x4_t izero = {0, 0, 0, 0};

    rsrc_t wr[NT], mr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int t = min(tbase + nt, T - 1);                 // ragged tile tail: clamp the loads
        wr[nt] = make_rsrc(codes + ((size_t)t * G + g0) * 1024, (uint32_t)ng * 1024);
        mr[nt] = make_rsrc(meta + ((size_t)t * G + g0) * 16, (uint32_t)ng * 64);
    }
    const rsrc_t ar = make_rsrc(a_codes + (size_t)g0 * 64, (uint32_t)((size_t)M * K / 2 - (size_t)g0 * 64));
    const rsrc_t sr = make_rsrc(a_scales + g0, (uint32_t)(((size_t)M * G - g0) * 4));
    // lane offsets: A row = the lane's MFMA row; the scale row this lane parks.  Rows past M read
    // row M - 1 (their outputs are discarded).
    const uint32_t aoff = (uint32_t)(min(col, M - 1) * (K / 2) + kq * 16);
    const uint32_t srow = (uint32_t)min(col, M - 1) * G;

    f32x4_t acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < ng; c0 += sch) {
        const int cn = min(sch, ng - c0);
        // Group c0 + i of this wave; prologue loads past a chunk shorter than the ring re-read its
        // first group.
        auto load = [&](W4DStage<NT> &st, int i) {
            const uint32_t g = (uint32_t)(c0 + (i < cn ? i : 0));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                st.w[nt] = buf_load16_stream(wr[nt], lane * 16, g * 1024);
                st.meta[nt] = buf_load4(mr[nt], col * 4, g * 64);
            }
            st.a = buf_load16(ar, aoff, g * 64);
        };

        auto compute = [&](const W4DStage<NT> &cur, int i) {
            const uint4 e = cur.a;
            const float4 s4 = *(const float4 *)&sl[i * 16 + 4 * kq];   // rows 4 kq .. 4 kq + 3
            const float as[4] = {s4.x, s4.y, s4.z, s4.w};
            const i32x4_t A0 = as_i32x4(snib_lo(e.x), snib_hi(e.x), snib_lo(e.y), snib_hi(e.y));
            const i32x4_t A1 = as_i32x4(snib_lo(e.z), snib_hi(e.z), snib_lo(e.w), snib_hi(e.w));
            i32x4_t sa = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, ones, izero, 0, 0, 0);
            sa = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, ones, sa, 0, 0, 0);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const uint4 d = cur.w[nt];
                const float sw = fp16_bits_to_float((uint16_t)(cur.meta[nt] & 0xFFFFu));
                const int zw = (int)((cur.meta[nt] >> 16) & 0xFFu);
                const i32x4_t B0 = as_i32x4(nib_lo(d.x), nib_hi(d.x), nib_lo(d.y), nib_hi(d.y));
                const i32x4_t B1 = as_i32x4(nib_lo(d.z), nib_hi(d.z), nib_lo(d.w), nib_hi(d.w));
                i32x4_t ia = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, B0, izero, 0, 0, 0);
                ia = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, B1, ia, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int Dv = ia[r] - __mul24(zw, sa[r]);   // |z sa| <= 15 * 896: 24-bit product
                    acc[nt][r] = __builtin_fmaf(as[r] * sw, (float)Dv, acc[nt][r]);
                    if (DOTS) {
                        const int mo = 4 * kq + r;
                        const int n = 16 * (tbase + nt) + col;
                        if (mo < M && n < N) dots[((size_t)(g0 + c0 + i) * M + mo) * N + n] = Dv;
                    }
                }
            }
        };

        W4DStage<NT> st[U];
        // The chunk's scales (from L2) are loaded first, the ring's first U groups (from HBM) right
        // behind them, and only then are the scales parked in LDS, so the two latencies overlap
        // (the in-order vmcnt wait for the scales leaves the ring's loads in flight).  Lane l reads
        // row l % 16, groups c0 + c + 4 (l / 16) .. + 3 for c = 0, 16, 32, 48, and parks those
        // inside the chunk at [group][row].  Reads past the array return 0.
        static_assert(kScaleChunk == 64, "four 16-group scale loads per chunk");
        uint4 sv[4];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // previous chunk's reads first
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            if (16 * q4 < cn) sv[q4] = buf_load16(sr, (srow + (uint32_t)(c0 + 16 * q4 + 4 * kq)) * 4, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            load(st[u], u);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            if (16 * q4 < cn) {
                const int gl = 16 * q4 + 4 * kq;
                const float vv[4] = {__uint_as_float(sv[q4].x), __uint_as_float(sv[q4].y),
                                     __uint_as_float(sv[q4].z), __uint_as_float(sv[q4].w)};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (gl + e < cn) sl[(gl + e) * 16 + col] = vv[e];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // Steady passes refill every slot with a group of the chunk (no branch around a load); the
        // last pass refills only the slots whose group exists, and the drain consumes them, so no
        // wave waits at its end on loads of groups it never uses.
        int base = 0;
        for (; base + 2 * U <= cn; base += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                compute(st[u], base + u);
                load(st[u], base + u + U);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (base + u < cn) compute(st[u], base + u);
            if (base + u + U < cn) load(st[u], base + u + U);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int u = 0; u < U - 1; ++u)
            if (base + U + u < cn) compute(st[u], base + U + u);
    }

    // Fixed-order reduction of the kw wave partials: every wave parks its NT tiles in LDS (lane
    // layout of the MFMA output), one barrier, then each thread sums 8 consecutive columns of one
    // row over the waves in wave order and writes them with one 16-byte (bf16) or two 16-byte
    // (f32) stores.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave * NT + nt) * 4 + r) * 64 + lane] = acc[nt][r];
    __syncthreads();
    for (int e = threadIdx.x; e < NT * 32; e += blockDim.x) {
        const int nt = e >> 5, m = (e >> 1) & 15, c0 = (e & 1) * 8;
        const int t = tbase + nt;
        if (m >= M || t >= T) continue;
        const int base = (nt * 4 + (m & 3)) * 64 + 16 * (m >> 2) + c0;
        float4 lo = *(const float4 *)&red[base], hi = *(const float4 *)&red[base + 4];
        for (int w = 1; w < kw; ++w) {
            const float4 a = *(const float4 *)&red[w * NT * 256 + base];
            const float4 b = *(const float4 *)&red[w * NT * 256 + base + 4];
            lo.x += a.x; lo.y += a.y; lo.z += a.z; lo.w += a.w;
            hi.x += b.x; hi.y += b.y; hi.z += b.z; hi.w += b.w;
        }
        const size_t idx = (size_t)m * N + 16 * t + c0;
        if (y_f32) {
            *(float4 *)((float *)y + idx) = lo;
            *(float4 *)((float *)y + idx + 4) = hi;
        } else {
            uint4 o;
            o.x = pack_bf16x2(lo.x, lo.y);
            o.y = pack_bf16x2(lo.z, lo.w);
            o.z = pack_bf16x2(hi.x, hi.y);
            o.w = pack_bf16x2(hi.z, hi.w);
            *(uint4 *)((uint16_t *)y + idx) = o;
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Shared-activation kernel (M > 64): 64-row blocks x 128 columns per workgroup, 4 waves, each
// wave 2 column tiles x all rows of the block (128-row blocks spill registers: the per-group
// int32 products and their rescale need more than 256 VGPRs next to 64 accumulators).  Per group, the waves widen the block's activation
// codes once into LDS as int8 MFMA fragments (fragment (row tile, MFMA j), lane l's 16 bytes at
// slot l: conflict-free) next to the rows' activation scales; every wave widens its own weight
// blocks in registers as signed bytes w - z, so D = sum q_a (w - z) comes straight out of
// v_mfma_i32_16x16x64_i8 and is rescaled in registers: y += s_a s D.  Codes, meta and scales
// travel through a U-deep register ring in group order; one barrier per step.  A 1-D grid walks
// row blocks fastest inside each XCD's range of tiles.
constexpr int Q_NT = 2, Q_CW = 4, Q_MT = 4;
constexpr int Q_TILES = Q_NT * Q_CW;

// Two waves per SIMD (two workgroups per CU) with a 3-deep ring fit 256 registers per lane; the
// 4-deep ring took 337 (VGPRs and AGPRs) and one wave per SIMD, which measured 28-34% slower on
// the shapes with enough workgroups to fill the chip twice.  The variant that also stores the
// exact group dots keeps one wave per SIMD and the 4-deep ring (its extra stores do not fit).
template <int U, bool DOTS, int NT>
__global__ void __launch_bounds__(Q_CW * 64) __attribute__((amdgpu_waves_per_eu(DOTS ? 1 : 2)))
k_w4a4_lds(const uint8_t *__restrict__ a_codes, const float *__restrict__ a_scales, int M,
           const uint8_t *__restrict__ codes, const uint32_t *__restrict__ meta, int K, int N,
           void *__restrict__ y, int y_f32, int32_t *__restrict__ dots, int row_blocks) {
    constexpr int MT = Q_MT, CW = Q_CW;
    constexpr int TILES = NT * CW;          // column tiles per workgroup
    constexpr int THREADS = CW * 64;
    constexpr int NFW = MT / CW;            // activation row tiles staged per wave
    static_assert(MT % CW == 0, "row tiles per wave");
    constexpr int AB = MT * 2 * 64;         // uint4 per staging buffer: [row tile][MFMA j][lane]
    constexpr int CHUNK = 64, CHUNK_WAVES = CHUNK / (NT * 16), OPITCH = CHUNK + 4;   // epilogue
    constexpr int LDS_U4 = (2 * AB > (MT * 16 * OPITCH + 3) / 4) ? 2 * AB : (MT * 16 * OPITCH + 3) / 4;
    __shared__ uint4 lds[LDS_U4];           // staging buffers, reused by the epilogue
    __shared__ float sbuf[2][MT * 16];      // [buffer][row] activation scales
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int cw = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, kq = lane >> 4;
    const int G = K / kGroup;
    const int T = N / 16;
    const int t_log = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int rblk = t_log % row_blocks, cblk = t_log / row_blocks;
    const int m0 = rblk * MT * 16;
    const int Mb = min(MT * 16, M - m0);
    const int tile0 = cblk * TILES + cw * NT;
    const i32x4_t izero = {0, 0, 0, 0};

    rsrc_t wr[NT], mr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int t = min(tile0 + nt, T - 1);              // ragged tile tail: clamp the loads
        wr[nt] = make_rsrc(codes + (size_t)t * G * 1024, (uint32_t)G * 1024);
        mr[nt] = make_rsrc(meta + (size_t)t * G * 16, (uint32_t)G * 64);
    }
    const rsrc_t ar = make_rsrc(a_codes + (size_t)m0 * (K / 2), (uint32_t)Mb * (K / 2));
    const rsrc_t sr = make_rsrc(a_scales + (size_t)m0 * G, (uint32_t)Mb * G * 4);
    // staged row tile q = cw * NFW + u: lane l loads the 16 code bytes of row 16 q + l % 16,
    // k-quarter l / 16 (its own MFMA A fragment), and that row's scale; rows past the block read
    // its last row (their MFMA rows are discarded)
    uint32_t aoff[NFW], soff[NFW];
#pragma unroll
    for (int u = 0; u < NFW; ++u) {
        const int row = min(16 * (cw * NFW + u) + col, Mb - 1);
        aoff[u] = (uint32_t)(row * (K / 2) + kq * 16);
        soff[u] = (uint32_t)(row * G) * 4;
    }

    struct Stage {
        uint4 w[NT];
        uint32_t m[NT];
        uint4 a[NFW];
        uint32_t s[NFW];
    };
    auto load = [&](Stage &st, int i) {
        const uint32_t g = (uint32_t)(i < G ? i : 0);  // past the end: re-read the first group
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            st.w[nt] = buf_load16_stream(wr[nt], lane * 16, g * 1024);
            st.m[nt] = buf_load4(mr[nt], col * 4, g * 64);
        }
#pragma unroll
        for (int u = 0; u < NFW; ++u) {
            st.a[u] = buf_load16(ar, aoff[u], g * 64);
            st.s[u] = buf_load4(sr, soff[u], g * 4);
        }
    };
    auto stage_act = [&](const Stage &st, int buf) {
#pragma unroll
        for (int u = 0; u < NFW; ++u) {
            const int q = cw * NFW + u;
            const uint4 e = st.a[u];
            lds[buf * AB + (q * 2 + 0) * 64 + lane] = make_uint4(snib_lo(e.x), snib_hi(e.x), snib_lo(e.y), snib_hi(e.y));
            lds[buf * AB + (q * 2 + 1) * 64 + lane] = make_uint4(snib_lo(e.z), snib_hi(e.z), snib_lo(e.w), snib_hi(e.w));
            if (kq == 0) sbuf[buf][q * 16 + col] = __uint_as_float(st.s[u]);
        }
    };

    f32x4_t acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Stage &st, int buf, int g) {
        i32x4_t B0[NT], B1[NT];
        float sw[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const uint4 d = st.w[nt];
            const uint32_t zz = ((st.m[nt] >> 16) & 0xFFu) * 0x01010101u;
            sw[nt] = fp16_bits_to_float((uint16_t)(st.m[nt] & 0xFFFFu));
            B0[nt] = as_i32x4(wz_bytes(nib_lo(d.x), zz), wz_bytes(nib_hi(d.x), zz), wz_bytes(nib_lo(d.y), zz),
                              wz_bytes(nib_hi(d.y), zz));
            B1[nt] = as_i32x4(wz_bytes(nib_lo(d.z), zz), wz_bytes(nib_hi(d.z), zz), wz_bytes(nib_lo(d.w), zz),
                              wz_bytes(nib_hi(d.w), zz));
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint4 a0 = lds[buf * AB + (mt * 2 + 0) * 64 + lane];
            const uint4 a1 = lds[buf * AB + (mt * 2 + 1) * 64 + lane];
            const float4 sa = *(const float4 *)&sbuf[buf][mt * 16 + 4 * kq];
            const float sar[4] = {sa.x, sa.y, sa.z, sa.w};
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                i32x4_t ia = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_i32x4(a0.x, a0.y, a0.z, a0.w), B0[nt], izero, 0, 0, 0);
                ia = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_i32x4(a1.x, a1.y, a1.z, a1.w), B1[nt], ia, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[mt][nt][r] = __builtin_fmaf(sar[r] * sw[nt], (float)ia[r], acc[mt][nt][r]);
                    if (DOTS) {
                        const int m = 16 * mt + 4 * kq + r;
                        const int n = 16 * (tile0 + nt) + col;
                        if (m < Mb && n < N) dots[((size_t)g * M + m0 + m) * N + n] = ia[r];
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);   // one row tile at a time: bounded register use
        }
    };

    // Ring: step i refills slot (i + U - 1) % U with group i + U - 1, consumes slot i % U and
    // stages slot (i + 1) % U into the other LDS buffer; as in the W4A16 shared-activation kernel.
    Stage st[U];
#pragma unroll
    for (int u = 0; u < U - 1; ++u) {
        load(st[u], u);
        __builtin_amdgcn_sched_barrier(0);
    }
    stage_act(st[0], 0);
    __syncthreads();
    const int nfull = ((G - 1) / U) * U;
    for (int base = 0; base < nfull; base += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u;
            load(st[(u + U - 1) % U], i + U - 1);
            compute(st[u], i & 1, i);
            __builtin_amdgcn_sched_barrier(0);
            stage_act(st[(u + 1) % U], (i + 1) & 1);
            __syncthreads();
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = nfull + u;
        if (i < G) {
            if (i + U - 1 < G) load(st[(u + U - 1) % U], i + U - 1);
            compute(st[u], i & 1, i);
            if (i + 1 < G) {
                stage_act(st[(u + 1) % U], (i + 1) & 1);
                __syncthreads();
            }
        }
    }
    __syncthreads();

    // Epilogue: in rounds of 64 columns (two waves), the sums go row-major through LDS and out
    // in 16-byte pieces (bfloat16 or f32).
    float *red = (float *)&lds[0];
    for (int rnd = 0; rnd < CW / CHUNK_WAVES; ++rnd) {
        if (cw / CHUNK_WAVES == rnd) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        red[(16 * mt + 4 * kq + r) * OPITCH + (cw % CHUNK_WAVES) * (NT * 16) + 16 * nt + col] =
                            acc[mt][nt][r];
        }
        __syncthreads();
        const int n0 = cblk * TILES * 16 + rnd * CHUNK;
        const int ncols = min(CHUNK, N - n0);
        if (y_f32) {
            float *dst = (float *)y + (size_t)m0 * N;
            for (int e = tid; e < Mb * (CHUNK / 4); e += THREADS) {
                const int m = e / (CHUNK / 4), c = (e % (CHUNK / 4)) * 4;
                if (c < ncols) *(float4 *)(dst + (size_t)m * N + n0 + c) = *(const float4 *)(red + m * OPITCH + c);
            }
        } else {
            uint16_t *dst = (uint16_t *)y + (size_t)m0 * N;
            for (int e = tid; e < Mb * (CHUNK / 8); e += THREADS) {
                const int m = e / (CHUNK / 8), c = (e % (CHUNK / 8)) * 8;
                if (c < ncols) {
                    const float4 lo = *(const float4 *)(red + m * OPITCH + c);
                    const float4 hi = *(const float4 *)(red + m * OPITCH + c + 4);
                    uint4 o;
                    o.x = pack_bf16x2(lo.x, lo.y);
                    o.y = pack_bf16x2(lo.z, lo.w);
                    o.z = pack_bf16x2(hi.x, hi.y);
                    o.w = pack_bf16x2(hi.z, hi.w);
                    *(uint4 *)(dst + (size_t)m * N + n0 + c) = o;
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------------

template <int MT, int NT, int U, int MAXW>
static hipError_t launch_skinny4(const uint8_t *a_codes, const float *a_scales, int M,
                                 const uint8_t *codes, const uint32_t *meta, int K, int N, void *y,
                                 int y_f32, int32_t *dots, hipStream_t st) {
    const int kw = min(skinny_waves_for_shape(K, N), MAXW);
    const int T = N / 16;
    dim3 grid((T + NT - 1) / NT);
    dim3 block(64 * kw);
    if (dots)
        hipLaunchKernelGGL((k_w4a4_skinny<MT, NT, U, MAXW, true>), grid, block, 0, st, a_codes, a_scales, M,
                           codes, meta, K, N, y, y_f32, dots, kw);
    else
        hipLaunchKernelGGL((k_w4a4_skinny<MT, NT, U, MAXW, false>), grid, block, 0, st, a_codes, a_scales, M,
                           codes, meta, K, N, y, y_f32, dots, kw);
    return hipGetLastError();
}

template <int NT, int U>
static hipError_t launch_decode4(const uint8_t *a_codes, const float *a_scales, int M, const uint8_t *codes,
                                 const uint32_t *meta, int K, int N, void *y, int y_f32, int32_t *dots, int kw,
                                 hipStream_t st) {
    dim3 grid((N / 16 + NT - 1) / NT), block(64 * kw);
    const size_t lds = decode4_lds_bytes(K / kGroup, kw, NT);
    if (dots)
        hipLaunchKernelGGL((k_w4a4_decode<NT, U, true>), grid, block, lds, st, a_codes, a_scales, M, codes, meta, K,
                           N, y, y_f32, dots, kw);
    else
        hipLaunchKernelGGL((k_w4a4_decode<NT, U, false>), grid, block, lds, st, a_codes, a_scales, M, codes, meta, K,
                           N, y, y_f32, dots, kw);
    return hipGetLastError();
}

// Batch tiers: [1, 16] (decode kernel), [17, 64] (skinny kernel, 2 or 4 row tiles per wave),
// above 64 (shared-activation kernel, 64-row blocks of 64 or 128 columns).  Inside a tier the
// per-output reduction order depends on (K, N) only.
int gemm_w4a4_tier(int M, int K, int N, int *m_first, int *m_last) {
    (void)K;
    (void)N;
    if (M <= 16) {
        *m_first = 1;
        *m_last = 16;
        return 0;
    }
    if (M <= 64) {
        *m_first = 17;
        *m_last = 64;
        return 1;
    }
    *m_first = 65;
    *m_last = 0x7FFFFFFF;
    return 2;
}

hipError_t launch_gemm_w4a4(const uint8_t *a_codes, const float *a_scales, int M, const uint8_t *codes,
                            const uint32_t *meta, int K, int N, void *y, int y_f32, int32_t *group_dots,
                            hipStream_t st) {
    // Batch tiers with one reduction order each: M <= 16 and 16 < M <= 64.
    if (M <= 16) {
        const DecodeShape d = decode_shape(K, N);
        if (d.nt == 4)
            return launch_decode4<4, 4>(a_codes, a_scales, M, codes, meta, K, N, y, y_f32, group_dots, d.kw, st);
        if (d.nt == 2)
            return launch_decode4<2, 4>(a_codes, a_scales, M, codes, meta, K, N, y, y_f32, group_dots, d.kw, st);
        return launch_decode4<1, 4>(a_codes, a_scales, M, codes, meta, K, N, y, y_f32, group_dots, d.kw, st);
    }
    if (M <= 32)
        return launch_skinny4<2, 1, 3, 4>(a_codes, a_scales, M, codes, meta, K, N, y, y_f32, group_dots, st);
    if (M <= 64)
        return launch_skinny4<4, 1, 2, 4>(a_codes, a_scales, M, codes, meta, K, N, y, y_f32, group_dots, st);
    // M > 64: 64-row blocks x 128 columns, one XCD-remapped 1-D grid; 64-column blocks (one tile
    // per wave) when 128-column blocks would give at most one workgroup per CU, so that more than
    // one wave per SIMD is resident (measured: 70B down at M = 256 183 -> 168 us, Llama-3-8B down
    // at M = 128 88 -> 64 us; with 448 wide blocks, gate+up at M = 80, narrow ones were slower).
    // Every output's reduction order is the same in both widths.
    const int rbs = (M + Q_MT * 16 - 1) / (Q_MT * 16);
    const int wide_cbs = (N / 16 + Q_TILES - 1) / Q_TILES;
    const bool narrow = (long long)wide_cbs * rbs <= 256;
    const int cbs = narrow ? (N / 16 + Q_CW - 1) / Q_CW : wide_cbs;
    const dim3 grid(cbs * rbs), block(Q_CW * 64);
    if (group_dots) {
        if (narrow)
            hipLaunchKernelGGL((k_w4a4_lds<4, true, 1>), grid, block, 0, st, a_codes, a_scales, M, codes, meta, K, N,
                               y, y_f32, group_dots, rbs);
        else
            hipLaunchKernelGGL((k_w4a4_lds<4, true, Q_NT>), grid, block, 0, st, a_codes, a_scales, M, codes, meta, K,
                               N, y, y_f32, group_dots, rbs);
    } else {
        if (narrow)
            hipLaunchKernelGGL((k_w4a4_lds<3, false, 1>), grid, block, 0, st, a_codes, a_scales, M, codes, meta, K, N,
                               y, y_f32, group_dots, rbs);
        else
            hipLaunchKernelGGL((k_w4a4_lds<3, false, Q_NT>), grid, block, 0, st, a_codes, a_scales, M, codes, meta, K,
                               N, y, y_f32, group_dots, rbs);
    }
    return hipGetLastError();
}

}  // namespace qspec
