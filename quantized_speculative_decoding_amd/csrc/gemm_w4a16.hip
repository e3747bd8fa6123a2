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
// Three kernels share the dequantization routine:
//  * k_w4a16_decode (M <= 16, and M <= 24 or 32 for the (K, N) where that measured faster):
//    HBM-bound decode / short-verify shapes; NT column tiles and one or two row tiles per
//    workgroup, K groups split between its waves, activations in registers.
//  * k_w4a16_mid (the verify tier, from there up to 80 rows and, where the large tier would not
//    fill the chip, up to 384 in row blocks of at most 80): each group's activation tile goes
//    straight from memory into LDS and is shared by the workgroup's waves; K is split between two
//    wave groups (and across workgroups with an ordered reduction).
//  * k_w4a16_lds (the large tier): 128-row blocks, activations staged through registers into LDS,
//    2 or 3 column tiles per wave.
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
// Decode kernel (MT 16-row tiles, MT = 1 or 2): HBM-bound decode / short-verify shapes.  Lane l:
// col = l % 16 (B column / A row within a row tile), kq = l / 16 (k quarter of a group).  In MFMA j (0..3) of a group, k slot
// (kq, i) holds k = 128 g + 32 kq + 8 j + i for both operands.  Output of
// v_mfma_f32_16x16x32_bf16: lane l, element r holds D[4 (l / 16) + r][l % 16].
//
// A workgroup owns NT column tiles and KW waves split the K groups; every wave loads the group's
// activations once (64 bytes per lane and row tile) and dequantizes each weight block once, for
// the 4 MT MFMAs of that tile.  A row's MFMAs see the same operands in the same order whatever MT
// is, so rows do not depend on the batch inside the tier.  Loads are
// buffer loads from wave-uniform bases through a U-deep register ring: each stage is consumed in
// place and refilled with group i + U, and a scheduling barrier keeps the stages' loads in group
// order, so the in-order vmcnt wait for a stage never covers a younger one.  Rows past M read row
// M - 1 (their MFMA rows are discarded).  Wave partials are summed through LDS in wave order, so
// the reduction order depends on (K, N) only.
template <int NT, int MT>
struct W16DStage {
    uint4 w[NT];
    uint32_t meta[NT];
    uint4 a[4 * MT];
};

template <int NT, int U, int MT>
__global__ void __launch_bounds__(64 * kMaxDecodeWaves)
k_w4a16_decode(const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
               const uint32_t *__restrict__ meta, int K, int N, void *__restrict__ y, int y_f32, int kw) {
    extern __shared__ __attribute__((aligned(16))) float red[];   // [kw][MT][NT][4][64], sized at launch
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int G = K / kGroup;
    const int g0 = (wave * G) / kw;
    const int ng = ((wave + 1) * G) / kw - g0;
    const int T = N / 16;
    const int tbase = blockIdx.x * NT;

    rsrc_t wr[NT], mr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int t = min(tbase + nt, T - 1);                 // ragged tile tail: clamp the loads
        wr[nt] = make_rsrc(codes + ((size_t)t * G + g0) * 1024, (uint32_t)ng * 1024);
        mr[nt] = make_rsrc(meta + ((size_t)t * G + g0) * 16, (uint32_t)ng * 64);
    }
    const rsrc_t xr = make_rsrc(x + (size_t)g0 * kGroup, (uint32_t)(((size_t)M * K - (size_t)g0 * kGroup) * 2));
    uint32_t xoff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xoff[mt] = (uint32_t)(min(col + 16 * mt, M - 1) * K + kq * 32) * 2;

    // Group i of this wave; prologue loads past a range shorter than the ring re-read its first group.
    auto load = [&](W16DStage<NT, MT> &st, int i) {
        const uint32_t g = (uint32_t)(i < ng ? i : 0);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            st.w[nt] = buf_load16_stream(wr[nt], lane * 16, g * 1024);
            st.meta[nt] = buf_load4(mr[nt], col * 4, g * 64);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) st.a[4 * mt + j] = buf_load16(xr, xoff[mt] + 16 * j, g * 256);
    };

    f32x4_t acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const W16DStage<NT, MT> &cur) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const DqConst dq = make_dq(cur.meta[nt]);
            const uint32_t words[4] = {cur.w[nt].x, cur.w[nt].y, cur.w[nt].z, cur.w[nt].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t b[4];
                dequant8(words[j], dq, b);
                const bf16x8_t bw = as_bf16x8(b[0], b[1], b[2], b[3]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, cur.a[4 * mt + j]), bw, acc[mt][nt], 0, 0, 0);
            }
        }
    };

    W16DStage<NT, MT> st[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        load(st[u], u);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Steady passes refill every slot with a group of this wave (no branch around a load); the
    // last pass refills only the slots whose group exists, and the drain consumes them.
    int base = 0;
    for (; base + 2 * U <= ng; base += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            compute(st[u]);
            load(st[u], base + u + U);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (base + u < ng) compute(st[u]);
        if (base + u + U < ng) load(st[u], base + u + U);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < U - 1; ++u)
        if (base + U + u < ng) compute(st[u]);

    // Fixed-order reduction of the kw wave partials: every wave parks its NT tiles in LDS (lane
    // layout of the MFMA output), one barrier, then each thread sums 8 consecutive columns of one
    // row over the waves in wave order and writes them with one 16-byte (bf16) or two 16-byte
    // (f32) stores.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[(((wave * MT + mt) * NT + nt) * 4 + r) * 64 + lane] = acc[mt][nt][r];
    __syncthreads();
    for (int e = threadIdx.x; e < MT * NT * 32; e += blockDim.x) {
        const int mnt = e >> 5, nt = mnt % NT, mt = mnt / NT, m = (e >> 1) & 15, c0 = (e & 1) * 8;
        const int t = tbase + nt, row = 16 * mt + m;
        if (row >= M || t >= T) continue;
        const int base = (mnt * 4 + (m & 3)) * 64 + 16 * (m >> 2) + c0;
        float4 lo = *(const float4 *)&red[base], hi = *(const float4 *)&red[base + 4];
        for (int w = 1; w < kw; ++w) {
            const float4 a = *(const float4 *)&red[w * MT * NT * 256 + base];
            const float4 b = *(const float4 *)&red[w * MT * NT * 256 + base + 4];
            lo.x += a.x; lo.y += a.y; lo.z += a.z; lo.w += a.w;
            hi.x += b.x; hi.y += b.y; hi.z += b.z; hi.w += b.w;
        }
        const size_t idx = (size_t)row * N + 16 * t + c0;
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
// Shared-activation kernels: the verify tier (k_w4a16_mid, further below) and the large tier
// (k_w4a16_lds).  At these M a group's activation tile (M x 128 bf16: 20 KB for 80 rows, 32 KB
// for a 128-row block) is as large as 20 - 32 weight blocks, so it is staged once in LDS and
// shared by the workgroup's waves, while every weight block is dequantized exactly once, in
// registers, by the wave whose MFMA B operand it is.  In the verify tier each wave owns LDS_NT = 2
// column tiles; in the large tier NT = 2 or 3.
//  * verify tier: 2 K parts x 4 column waves (8 waves, 128 columns, up to 80 rows), two waves per
//    SIMD (a single wave per SIMD issues MFMA and VALU work at about half the rate two reach);
//  * large tier: 8 column waves (256 or 384 columns, 128-row blocks).
// k_w4a16_lds: per group, the waves stage the activation tile into LDS in fragment-major order
// (fragment f = (row tile, 32-k step), lane l's 16 bytes in f's 1 KB block, XOR-swizzled:
// conflict-free 128-bit writes and reads) and every wave reads all fragments from there, each
// feeding NT MFMAs.  Activations and weights travel through one U-deep register ring in group
// order (the in-order vmcnt wait for a stage never covers a younger one); a stage's activations
// are written to LDS one step before they are consumed, its weights are dequantized in registers
// when consumed.  One barrier per step.  With S > 1 K splits (a function of (K, N) only), each
// workgroup writes an fp32 partial tile and k_w4a16_splitk_reduce adds the S partials in split
// order, so every output has one fixed reduction order per (K, N) in each tier.
constexpr int LDS_NT = 2;                    // column tiles per wave
constexpr int MID_KP = 2, MID_CW = 4;        // verify tier
constexpr int MID_TILES = MID_CW * LDS_NT;   // column tiles per verify-tier workgroup
constexpr int BIG_MT = 8, BIG_CW = 8;        // large tier: 128-row blocks, 8 column waves
constexpr int BIG_TILES = BIG_CW * LDS_NT;   // with 2 tiles per wave (the tier and split rules)

template <int MT, int U, int CW, int NT>
__global__ void __launch_bounds__(CW * 64)
k_w4a16_lds(const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
            const uint32_t *__restrict__ meta, int K, int N, void *__restrict__ y, int y_f32, int S,
            float *__restrict__ partials, int row_blocks) {
    constexpr int THREADS = CW * 64;
    constexpr int TILES = CW * NT;          // column tiles per workgroup
    constexpr int NF = MT * 4;              // activation fragments per group
    constexpr int NFW = NF / CW;            // staged by each wave
    static_assert(NF % CW == 0, "activation fragments per wave");
    // LDS: two staging buffers [buffer][fragment][lane]; the epilogue reuses them
    constexpr int STAGE_U4 = 2 * NF * 64;
    __shared__ uint4 lds[STAGE_U4];
    auto abuf = [&](int buf) -> uint4 * { return lds + buf * NF * 64; };
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int cw = __builtin_amdgcn_readfirstlane(tid >> 6);     // wave-uniform (SGPR)
    const int col = lane & 15, kq = lane >> 4;
    const int G = K / kGroup;
    const int T = N / 16;
    // Workgroup -> (column block, split, row block).  Several row blocks: a 1-D grid remapped so
    // that each XCD owns a contiguous range of logical tiles, row blocks fastest, then splits, so
    // the workgroups that share a column block's weights run together on one XCD and its L2.  One
    // row block: a 2-D (column block, split) grid.
    int cblk = blockIdx.x, split = blockIdx.y, rblk = 0;
    if (gridDim.y == 1 && row_blocks > 1) {
        const int t = xcd_remap((int)blockIdx.x, (int)gridDim.x);
        rblk = t % row_blocks;
        split = (t / row_blocks) % S;
        cblk = t / row_blocks / S;
    }
    const int m0 = rblk * MT * 16;           // this workgroup's row block
    const int Mb = min(MT * 16, M - m0);
    const int hstart = (split * G) / S;
    const int nsteps = ((split + 1) * G) / S - hstart;    // groups of this split
    const int hlast = nsteps - 1;
    const int tile0 = cblk * TILES + cw * NT;

    // Buffer resources per column tile (SGPRs) plus one 32-bit lane offset per stream; the
    // group index enters as the wave-uniform offset.
    rsrc_t wr[NT], mr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int t = min(tile0 + nt, T - 1);              // ragged tile tail: clamp the loads
        wr[nt] = make_rsrc(codes + (size_t)t * G * 1024, (uint32_t)G * 1024);
        mr[nt] = make_rsrc(meta + (size_t)t * G * 16, (uint32_t)G * 64);
    }
    const rsrc_t xr = make_rsrc(x + (size_t)m0 * K, (uint32_t)Mb * K * 2);
    // Activation staging: load q = cw * NFW + u reads rows 4 q .. 4 q + 3 of the
    // group, 16 lanes per row (row-contiguous: 8 cache lines per load).  The 16 bytes of (row, 8-k
    // chunk c) are element (row % 16, k = 8 c) of fragment f = 4 (row / 16) + c % 4, i.e. lane
    // l = row % 16 + 16 (c / 4) of it; they are stored at slot l ^ (c / 4) ^ 4 (c % 4) of the
    // fragment's 1 KB block, so a reader lane l of fragment (row tile, 32-k step j) finds its data
    // at slot l ^ (l / 16) ^ 4 j.  Lane p of a row loads chunk c = 4 (p % 4) + p / 4, which makes
    // the low four slot bits of a staging write p ^ row.  Measured on gfx950 with 16-byte LDS
    // accesses: reads whose lane-dependent XOR reaches slot bit 3 (such as l ^ 4 (l / 16)) and
    // writes whose low slot bits are not the lane XOR a uniform value run 15 - 18% slower; this
    // layout has neither.  Rows past the block read its last row (their MFMA rows are discarded).
    uint32_t xoff[NFW], xslot[NFW];
#pragma unroll
    for (int u = 0; u < NFW; ++u) {
        const int row = 4 * (cw * NFW + u) + (lane >> 4);
        const int p = lane & 15;
        const int c = ((p & 3) << 2) | (p >> 2);
        xoff[u] = (uint32_t)(min(row, Mb - 1) * K + c * 8) * 2;
        xslot[u] = (uint32_t)((4 * (row >> 4) + (c & 3)) * 64 +
                              (((row & 15) + 16 * (c >> 2)) ^ (c >> 2) ^ (4 * (c & 3))));
    }
    const int rslot = lane ^ kq;   // reader slot, before the 32-k step j

    struct Stage {
        uint4 w[NT];
        uint32_t m[NT];
        uint4 a[NFW];
    };
    // Group i of the split; a refill past the end re-reads the first group (long since arrived)
    // rather than a group whose load may still be in flight.
    auto load = [&](Stage &st, int i) {
        const uint32_t g = (uint32_t)(hstart + (i <= hlast ? i : 0));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            st.w[nt] = buf_load16_stream(wr[nt], lane * 16, g * 1024);
            st.m[nt] = buf_load4(mr[nt], col * 4, g * 64);
        }
#pragma unroll
        for (int u = 0; u < NFW; ++u) st.a[u] = buf_load16(xr, xoff[u], g * 256);
    };
    auto stage_act = [&](const Stage &st, int buf) {
#pragma unroll
        for (int u = 0; u < NFW; ++u) abuf(buf)[xslot[u]] = st.a[u];
    };

    f32x4_t acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Each 32-k step is dequantized right before its MFMAs (8 row tiles of accumulators leave no
    // registers for carrying the next step's operand).
    auto compute = [&](const Stage &st, int buf) {
        DqConst dq[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) dq[nt] = make_dq(st.m[nt]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x8_t av[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                av[mt] = __builtin_bit_cast(bf16x8_t, abuf(buf)[(mt * 4 + j) * 64 + (rslot ^ (4 * j))]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const uint32_t word = j == 0 ? st.w[nt].x : j == 1 ? st.w[nt].y : j == 2 ? st.w[nt].z : st.w[nt].w;
                uint32_t b[4];
                dequant8(word, dq[nt], b);
                const bf16x8_t bv = as_bf16x8(b[0], b[1], b[2], b[3]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], bv, acc[mt][nt], 0, 0, 0);
            }
        }
    };

    // Ring slot s % U holds group s.  Step i first refills slot (i + U - 1) % U (it held group
    // i - 1: weights consumed at step i - 1, activations staged at step i - 2) with group
    // i + U - 1, then consumes the weights of slot i % U and writes the activations of slot
    // (i + 1) % U to LDS for step i + 1; the compiler spreads the refill loads through the MFMA /
    // VALU stream.  The steady loop never runs the last step and loads unconditionally (indices past
    // the end re-read the first group), so no load is predicated there.
    Stage st[U];
#pragma unroll
    for (int u = 0; u < U - 1; ++u) {
        load(st[u], u);
        __builtin_amdgcn_sched_barrier(0);
    }
    stage_act(st[0], 0);
    __syncthreads();
    const int nfull = ((nsteps - 1) / U) * U;
    for (int base = 0; base < nfull; base += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u;
            load(st[(u + U - 1) % U], i + U - 1);
            compute(st[u], i & 1);
            __builtin_amdgcn_sched_barrier(0);
            stage_act(st[(u + 1) % U], (i + 1) & 1);
            __syncthreads();
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = nfull + u;
        if (i < nsteps) {                        // uniform over the workgroup
            if (i + U - 1 < nsteps) load(st[(u + U - 1) % U], i + U - 1);
            compute(st[u], i & 1);
            if (i + 1 < nsteps) {
                stage_act(st[(u + 1) % U], (i + 1) & 1);
                __syncthreads();
            }
        }
    }
    __syncthreads();   // every wave is done reading the staging buffers

    // Epilogue: the 128 x 256 block of sums exceeds the staging buffers, so the waves write rounds
    // of 64 columns (two column waves) to LDS and all waves store them: bfloat16 / f32 output, or
    // the fp32 partial of this split.
    float *dstf = S > 1 ? partials + (size_t)split * M * N + (size_t)m0 * N : (float *)y + (size_t)m0 * N;
    uint16_t *dsth = (uint16_t *)y + (size_t)m0 * N;
    float *red = (float *)lds;
    constexpr int CHUNK_WAVES = NT * 16 >= 64 ? 1 : 64 / (NT * 16);   // column waves per round
    constexpr int CHUNK = CHUNK_WAVES * NT * 16;    // output columns per round
    constexpr int OPITCH = CHUNK + 4;               // floats per output row in LDS
    static_assert(MT * 16 * OPITCH <= STAGE_U4 * 4, "output buffer");
    static_assert(CW % CHUNK_WAVES == 0, "column rounds");
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
        const int n0 = (cblk * TILES) * 16 + rnd * CHUNK;
        const int ncols = min(CHUNK, N - n0);   // a multiple of 16 (possibly <= 0)
        if (S > 1 || y_f32) {
            for (int e = tid; e < Mb * (CHUNK / 4); e += THREADS) {     // 4 floats per thread
                const int m = e / (CHUNK / 4), c = (e % (CHUNK / 4)) * 4;
                if (c < ncols) *(float4 *)(dstf + (size_t)m * N + n0 + c) = *(const float4 *)(red + m * OPITCH + c);
            }
        } else {
            for (int e = tid; e < Mb * (CHUNK / 8); e += THREADS) {     // 8 outputs per thread
                const int m = e / (CHUNK / 8), c = (e % (CHUNK / 8)) * 8;
                if (c < ncols) {
                    const float4 lo = *(const float4 *)(red + m * OPITCH + c);
                    const float4 hi = *(const float4 *)(red + m * OPITCH + c + 4);
                    uint4 o;
                    o.x = pack_bf16x2(lo.x, lo.y);
                    o.y = pack_bf16x2(lo.z, lo.w);
                    o.z = pack_bf16x2(hi.x, hi.y);
                    o.w = pack_bf16x2(hi.z, hi.w);
                    *(uint4 *)(dsth + (size_t)m * N + n0 + c) = o;
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------------
// Verify-tier kernel k_w4a16_mid<MT, U>: a workgroup of 2 K parts x 4 column waves covers 128
// columns of one K split and one block of up to 16 MT rows (row blocks of equal height in whole
// row tiles, at most 80 rows each).  The parts are added in part order and the K splits by
// k_w4a16_splitk_reduce, so a row's reduction order depends on (K, N) only, whatever the block.
// Each part's activation tile travels from memory straight into a U-deep LDS ring
// (buffer_load ... lds: no registers, no LDS write instructions), and only the weights and their
// meta words go through a U-deep register ring.  Step i waits for its own group (vmcnt counts the
// loads of the U - 2 younger groups still in flight), crosses one barrier, refills the ring slot
// freed by step i - 1 with group i + U - 1, then computes group i.
// LDS activation layout, per (part, buffer): row-major, 256 bytes per row (128 k), the row's 16
// chunks of 8 k stored at chunk position c ^ (row % 16).  A direct load writes 4 consecutive rows
// (lane l: row 4 q + l / 16, position l % 16, so it loads chunk (l % 16) ^ (row % 16)).  The
// weight packing gives lane group kq the 32 consecutive k of chunks 4 kq .. 4 kq + 3, one chunk
// per 32-k step j, so the MFMA A fragment (row tile t, step j) of lane l = r + 16 kq reads row
// 16 t + r, chunk 4 kq + j at position (4 kq + j) ^ r: each 16-lane phase of a ds_read_b128
// covers the 64 banks once.
// Each ring slot is an LDS variable of its own, holding both parts' tiles: the compiler tracks
// direct loads per LDS variable, so a read of slot b waits only for the loads into slot b, where
// a single array would make every LDS read wait for all direct loads in flight.  For the same
// reason the step barrier carries no memory fence (a workgroup release fence waits for every
// direct load in flight): each wave waits for its own loads into the slot, then the barrier.
// The epilogue keeps part p's sums in slot p: 128 floats per row, column c of row r at
// c ^ 16 ((r / 4) % 4), so the four row quads of an accumulator store hit distinct banks.
template <int MT, int U, int B>
__device__ __forceinline__ unsigned char *mid_slot_var() {
    static_assert(MID_TILES * 16 * 4 <= 256 * MID_KP, "a part's sums fit one slot");
    __shared__ __attribute__((aligned(16))) unsigned char slot[MID_KP * MT * 16 * 256];
    return slot;
}
template <int MT, int U, int B = 0>
__device__ __forceinline__ unsigned char *mid_slot(int b) {   // b: a compile-time value after unrolling
    if constexpr (B + 1 >= U) return mid_slot_var<MT, U, B>();
    else return b == B ? mid_slot_var<MT, U, B>() : mid_slot<MT, U, B + 1>(b);
}
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

template <int MT, int U>
__global__ void __launch_bounds__(MID_KP * MID_CW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_w4a16_mid(const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
            const uint32_t *__restrict__ meta, int K, int N, void *__restrict__ y, int y_f32, int S,
            float *__restrict__ partials, int row_blocks) {
    constexpr int NT = LDS_NT, CW = MID_CW, KP = MID_KP;
    constexpr int THREADS = KP * CW * 64;
    constexpr int TILES = CW * NT;
    constexpr int ROWS = MT * 16;
    constexpr int NLD = ROWS / 4 / CW;                     // direct loads per wave per group (4 rows each)
    static_assert(ROWS % (4 * CW) == 0, "rows per staging wave");
    constexpr int PBYTES = ROWS * 256;                     // one part's tile in a slot
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = wave / CW, cw = wave % CW;
    const int col = lane & 15, kq = lane >> 4;
    const int G = K / kGroup;
    const int T = N / 16;
    // Workgroup -> (row block, column block, split), row blocks fastest, then column blocks: the
    // workgroups that read one column block's weights share an XCD (and its L2), and those of one
    // split, which read the same activation slice, share one or two.
    int cblk = blockIdx.x, split = 0, rblk = 0;
    if (S > 1 || row_blocks > 1) {
        int t = xcd_remap((int)blockIdx.x, (int)gridDim.x);
        const int cbs = (int)gridDim.x / (S * row_blocks);
        rblk = t % row_blocks;
        t /= row_blocks;
        cblk = t % cbs;
        split = t / cbs;
    }
    const int m0 = rblk * ROWS;                            // this workgroup's row block
    const int Mb = min(ROWS, M - m0);
    const int gs0 = (split * G) / S;
    const int n = ((split + 1) * G) / S - gs0;
    const int hstart = gs0 + (kh * n) / KP;
    const int nh = ((kh + 1) * n) / KP - (kh * n) / KP;    // groups of this part
    const int nsteps = (n + KP - 1) / KP;                  // all parts step together
    const int hlast = max(nh, 1) - 1;
    const int tile0 = cblk * TILES + cw * NT;

    rsrc_t wr[NT], mr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int t = min(tile0 + nt, T - 1);
        wr[nt] = make_rsrc(codes + (size_t)t * G * 1024, (uint32_t)G * 1024);
        mr[nt] = make_rsrc(meta + (size_t)t * G * 16, (uint32_t)G * 64);
    }
    const rsrc_t xr = make_rsrc(x + (size_t)m0 * K, (uint32_t)((size_t)Mb * K * 2));
    // direct-load lane offsets: load u of this wave covers rows 4 (cw NLD + u) .. + 3 of the part's
    // tile; rows past the block read its last row (their MFMA rows are discarded)
    uint32_t xoff[NLD];
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
        const int row = 4 * (cw * NLD + u) + (lane >> 4);
        const int chunk = (lane & 15) ^ (row & 15);
        xoff[u] = (uint32_t)(min(row, Mb - 1) * K + chunk * 8) * 2;
    }

    struct Stage {
        uint4 w[NT];
        uint32_t m[NT];
    };
    // Group i of the part into ring slot b = i % U: the weights into registers, the activation
    // tile into LDS slot b.  Past the end the first group is re-read (long since arrived).
    auto load = [&](Stage &st, int i, int b) {
        const uint32_t g = (uint32_t)(hstart + (i <= hlast ? i : 0));
        unsigned char *dst = mid_slot<MT, U>(b) + kh * PBYTES;
#pragma unroll
        for (int u = 0; u < NLD; ++u)
            buf_load16_to_lds(xr, dst + (cw * NLD + u) * 1024, xoff[u], g * 256);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            st.w[nt] = buf_load16_stream(wr[nt], lane * 16, g * 1024);
            st.m[nt] = buf_load4(mr[nt], col * 4, g * 64);
        }
    };

    f32x4_t acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // dequantization one 32-k step ahead of the MFMAs (as the verify tier of k_w4a16_lds)
    auto dq_step = [&](const Stage &st, const DqConst (&dq)[NT], int j, bf16x8_t (&bq)[NT]) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const uint32_t word = j == 0 ? st.w[nt].x : j == 1 ? st.w[nt].y : j == 2 ? st.w[nt].z : st.w[nt].w;
            uint32_t b[4];
            dequant8(word, dq[nt], b);
            bq[nt] = as_bf16x8(b[0], b[1], b[2], b[3]);
        }
    };
    auto make_dqs = [&](const Stage &st, DqConst (&dq)[NT]) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) dq[nt] = make_dq(st.m[nt]);
    };
    bf16x8_t bq[NT];
    DqConst dc[NT];
    auto compute = [&](const Stage &st, const Stage &next, int b) {
        const unsigned char *a = mid_slot<MT, U>(b) + kh * PBYTES;
        DqConst dq[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) dq[nt] = dc[nt];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x8_t av[MT], bv[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bv[nt] = bq[nt];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                av[mt] = *(const bf16x8_t *)(a + (16 * mt + col) * 256 + (((4 * kq + j) ^ col) * 16));
            if (j < 3) {
                dq_step(st, dq, j + 1, bq);
            } else {
                make_dqs(next, dc);
                dq_step(next, dc, 0, bq);
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], bv[nt], acc[mt][nt], 0, 0, 0);
        }
    };

    // One load per group and wave: NLD direct loads + NT weight and NT meta loads, all counted by
    // vmcnt in issue order.  At step i the U - 2 younger groups' loads may stay in flight.
    constexpr int PER = NLD + 2 * NT;
    Stage st[U];
#pragma unroll
    for (int u = 0; u < U - 1; ++u) {
        load(st[u], u, u);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Wait until group i's loads (its activation tile in particular, whose arrival the barrier
    // must cover for every wave) have landed, leaving `younger` groups' loads in flight.  The
    // prologue issues groups 0 .. U - 2 and every step of the steady loop one more group, past the
    // end too (re-reading the first group: a fixed count of loads in flight, and no predicated
    // load for the compiler's own wait counting to merge); the tail issues only groups that exist.
    static_assert(PER * (U - 2) < 64, "vmcnt range");
    auto wait_younger = [&](int younger) {
        switch (younger) {
#define QSPEC_WAIT_CASE(k) \
    case k: if constexpr (k <= U - 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER * k) : "memory"); break;
            QSPEC_WAIT_CASE(0) QSPEC_WAIT_CASE(1) QSPEC_WAIT_CASE(2) QSPEC_WAIT_CASE(3)
            QSPEC_WAIT_CASE(4) QSPEC_WAIT_CASE(5) QSPEC_WAIT_CASE(6)
#undef QSPEC_WAIT_CASE
            default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        }
    };
    static_assert(U - 2 <= 6, "wait cases");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER * (U - 2)) : "memory");
    make_dqs(st[0], dc);
    dq_step(st[0], dc, 0, bq);
    barrier_no_fence();
    // Step i uses ring slot i % U, a compile-time index once the loops below are unrolled by U.
    // Slot (i + U - 1) % U held group i - 1; its LDS buffer was last read at step i - 1, which
    // every wave finished before this step's barrier.  The steady loop never runs the last step,
    // so every part computes in it.
    const int nfull = ((nsteps - 1) / U) * U;
    for (int base = 0; base < nfull; base += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u;
            if (u > 0 || base > 0) {
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER * (U - 2)) : "memory");
                barrier_no_fence();
            }
            load(st[(u + U - 1) % U], i + U - 1, (u + U - 1) % U);
            __builtin_amdgcn_sched_barrier(0);
            compute(st[u], st[(u + 1) % U], u);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = nfull + u;
        if (i < nsteps) {                                  // uniform over the workgroup
            if (i > 0) {
                wait_younger(max(nfull + U - 2, min(i + U - 2, nsteps - 1)) - i);
                barrier_no_fence();
            }
            if (i + U - 1 < nsteps) load(st[(u + U - 1) % U], i + U - 1, (u + U - 1) % U);
            __builtin_amdgcn_sched_barrier(0);
            if (i < nh) compute(st[u], st[(u + 1) % U], u);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");         // no direct load may land on the epilogue
    __syncthreads();

    // Epilogue (the sums of K part p in slot p): every wave writes its sums, one barrier, and all
    // waves add the parts in part order and store 16-byte pieces.
    constexpr int WCOLS = TILES * 16;
    static_assert(WCOLS == 128, "epilogue row pitch");
    auto red_at = [](int m, int c) { return m * WCOLS + (c ^ (16 * ((m >> 2) & 3))); };
    {
        float *red = (float *)mid_slot<MT, U>(kh);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    red[red_at(16 * mt + 4 * kq + r, cw * NT * 16 + 16 * nt + col)] = acc[mt][nt][r];
    }
    __syncthreads();
    const int n0 = cblk * TILES * 16;
    const int ncols = min(WCOLS, N - n0);
    auto part_sum4 = [&](int m, int c) {             // c: a multiple of 4 (the swizzle keeps the 4)
        float4 v = *(const float4 *)((const float *)mid_slot<MT, U>(0) + red_at(m, c));
#pragma unroll
        for (int p = 1; p < KP; ++p) {
            const float4 w = *(const float4 *)((const float *)mid_slot<MT, U>(p) + red_at(m, c));
            v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
        }
        return v;
    };
    float *dstf = S > 1 ? partials + (size_t)split * M * N + (size_t)m0 * N : (float *)y + (size_t)m0 * N;
    uint16_t *dsth = (uint16_t *)y + (size_t)m0 * N;
    if (S > 1 || y_f32) {
        for (int e = tid; e < Mb * (WCOLS / 4); e += THREADS) {
            const int m = e / (WCOLS / 4), c = (e % (WCOLS / 4)) * 4;
            if (c < ncols) *(float4 *)(dstf + (size_t)m * N + n0 + c) = part_sum4(m, c);
        }
    } else {
        for (int e = tid; e < Mb * (WCOLS / 8); e += THREADS) {
            const int m = e / (WCOLS / 8), c = (e % (WCOLS / 8)) * 8;
            if (c < ncols) {
                const float4 lo = part_sum4(m, c), hi = part_sum4(m, c + 4);
                uint4 o;
                o.x = pack_bf16x2(lo.x, lo.y);
                o.y = pack_bf16x2(lo.z, lo.w);
                o.z = pack_bf16x2(hi.x, hi.y);
                o.w = pack_bf16x2(hi.z, hi.w);
                *(uint4 *)(dsth + (size_t)m * N + n0 + c) = o;
            }
        }
    }
}

// y = sum of the S <= kMaxSplits fp32 partials in split order (4 outputs per thread; M * N is a
// multiple of 16).  All S loads are issued before the first add.  A second kernel rather than a
// last-arriving workgroup: the device-scope fence that hand-off needs writes back the XCD's L2,
// which measured 35 - 50 us slower per call than this launch on the verify shapes.
constexpr int kMaxSplits = 16;

__global__ void __launch_bounds__(256)
k_w4a16_splitk_reduce(const float *__restrict__ partials, int S, size_t MN, void *__restrict__ y, int y_f32) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= MN) return;
    float4 v[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
        if (s < S) v[s] = *(const float4 *)(partials + (size_t)s * MN + i);
    float4 a = v[0];
#pragma unroll
    for (int s = 1; s < kMaxSplits; ++s)
        if (s < S) {
            a.x += v[s].x;
            a.y += v[s].y;
            a.z += v[s].z;
            a.w += v[s].w;
        }
    if (y_f32) {
        *(float4 *)((float *)y + i) = a;
    } else {
        uint2 o;
        o.x = pack_bf16x2(a.x, a.y);
        o.y = pack_bf16x2(a.z, a.w);
        *(uint2 *)((uint16_t *)y + i) = o;
    }
}

// ---------------------------------------------------------------------------------------------
// Host launchers.

template <int NT, int U, int MT>
static hipError_t launch_decode(const uint16_t *x, int M, const uint8_t *codes, const uint32_t *meta, int K, int N,
                                void *y, int y_f32, hipStream_t st) {
    const int kw = decode_shape(K, N).kw;
    const size_t lds = (size_t)kw * MT * NT * 256 * sizeof(float);
    hipLaunchKernelGGL((k_w4a16_decode<NT, U, MT>), dim3((N / 16 + NT - 1) / NT), dim3(64 * kw), lds, st, x, M,
                       codes, meta, K, N, y, y_f32, kw);
    return hipGetLastError();
}

// Largest batch of the decode tier for (K, N); above 16 rows a wave carries two row tiles
// (MT = 2).  Every workgroup of the decode kernel reads all M rows of the activations for its
// column tiles, about 4 M / NT times the bytes of its weights, where the verify tier stages them
// once per 128 columns; the second row tile pays only where the weights are small (latency-bound
// launches in one generation of workgroups) or the workgroups are wide (NT = 4).  From an A/B run
// at M = 17, 24, 32 on the Llama-3-8B and Qwen2.5-7B projections and vocabulary head (µs, verify
// tier -> decode tier): Llama qkv 11.3 -> 9.0 (M = 17) and 12.5 -> 11.2 (M = 32), Qwen o 10.0 ->
// 7.5 and 11.0 -> 9.8, Qwen head 99 -> 88 (M = 17) and 100 -> 94 (M = 24), 103 both at M = 32;
// losses where the activation re-reads dominate: Llama down 16.2 -> 20.4 (M = 17), 18.0 -> 34.7
// (M = 32), gate+up 23 -> 25 .. 34, and Qwen qkv (288 workgroups, some CUs run two) 10.2 -> 11.4.
static int mid_splits(int K, int N);

static int decode_max_m(int K, int N) {
    const DecodeShape d = decode_shape(K, N);
    const int wgs = (N / 16 + d.nt - 1) / d.nt;
    const int G = K / kGroup;
    if (d.nt == 4) return 24;
    if (wgs <= 256 && (long long)K * N <= 4096LL * 6144) return 32;
    // Every decode wave re-reads all M activation rows of its groups, so past a few rows the verify
    // tier, which stages them once per 128 columns, wins: from 9 rows on long K (graph-timed,
    // decode / verify at M = 9 - 16: Llama-3-8B and Qwen2.5-7B down, K = 12160 x 4096 12 - 15 /
    // 12 us, Llama-70B down 33 - 38 / 30 - 32 us), from 13 rows otherwise (Llama-3-8B gate+up at 16
    // rows 20.6 / 17.3 us, Llama-70B gate+up 71.5 / 64, Qwen2.5-7B qkv 9.9 / 8.8) -- unless the
    // verify tier's workgroups leave its last generation mostly idle (Qwen2.5-7B gate+up, 296
    // workgroups on 256 CUs: decode 22 - 27 / verify 27 - 30 us up to 17 rows, 29.6 / 30.2 at 20).
    if (d.nt == 1) return G >= 64 ? 8 : 12;
    if (G >= 96) return 8;
    const int vw = ((N / 16 + MID_TILES - 1) / MID_TILES) * mid_splits(K, N);   // verify workgroups
    const int gens = (vw + 255) / 256;
    return 4 * vw < 3 * 256 * gens ? 20 : 12;
}

// K splits of the verify-tier kernel: a function of (K, N) only.  Column blocks alone fill the
// chip when there are at least 192 of them; otherwise split K as far as the grid still fits one
// workgroup per CU (256), keeping at least 5 groups per split, and at most kMaxSplits splits.
// From sweeps of S = 1 .. 9 over the Llama-3-8B and Qwen2.5-7B projections at M = 20 and 80: a
// grid past 256 workgroups runs a second generation (Llama qkv: 4 splits 11.9 us, 6 splits
// 16.5 us at M = 20); with fewer than about 5 groups per split the fp32 partials cost more than
// the extra workgroups gain; in between, Qwen2.5-7B qkv and o (28 groups) ran 10 - 16% faster
// with 5 splits than with the 3 a floor of 8 groups allowed.
static int mid_splits(int K, int N) {
    const int G = K / kGroup;
    const int cbs = (N / 16 + MID_TILES - 1) / MID_TILES;
    if (cbs >= 192) return 1;
    const int fit = 256 / cbs;
    return max(1, min(min(fit, kMaxSplits), G / 5));
}

// K splits of the large tier: a function of (K, N) only.  Its 128-row x 256-column blocks run one
// workgroup per CU, so a shape with few column blocks leaves a last, mostly empty generation of
// workgroups (Llama-70B down, 32 column blocks x 10 row blocks at M = 1280: 320 workgroups, 1.25
// generations); splitting K multiplies the workgroups by S (a power of two up to 128 / column
// blocks) while every split keeps at least 32 groups.
static int big_splits(int K, int N) {
    const int G = K / kGroup;
    const int cbs = (N / 16 + BIG_TILES - 1) / BIG_TILES;
    int S = 1;
    while (S < 8 && 2 * S * cbs <= 128 && G / (2 * S) >= 32) S *= 2;
    return S;
}

// Largest batch of the verify tier for (K, N), a step function of P, the large tier's workgroups
// per 128-row block: 384 rows for P <= 32, 256 for P <= 64, 160 for P <= 128, 80 above.  Past 80
// rows the verify tier runs row blocks of at most 80 rows, each re-reading the weights, but fills
// the chip where the large tier's few workgroups leave CUs idle.  From graph-timed sweeps of both
// tiers at M = 96 - 512 (us, verify / large): Llama-3-8B down (P = 32) 40 / 100 at 128 and 87 / 107
// at 384, o (16) 47 / 62 at 384, qkv (24) 62 / 62 at 384 and 79 / 64 at 512; Qwen2.5-7B down (56)
// 71 / 77 at 256 and 95 / 82 at 384; Llama-3-8B gate+up (112) 58 / 68 at 160 and 75 / 69 at 192;
// Llama-70B down (128) 102 / 117 at 160 and 132 / 120 at 192; Llama-70B gate+up (224) 154 / 126
// at 96.
static int mid_max_m(int K, int N) {
    const int P = ((N / 16 + BIG_TILES - 1) / BIG_TILES) * big_splits(K, N);
    return P <= 32 ? 384 : P <= 64 ? 256 : P <= 128 ? 160 : 80;
}

// Batch tiers: [1, decode_max_m] (decode kernel, one or two row tiles), (decode_max_m,
// mid_max_m] (verify tier: direct-to-LDS kernel with K parts, row blocks of at most 80 rows),
// above (large tier: shared-activation kernel, 128-row blocks).  Inside a tier the per-output
// reduction order depends on (K, N) only.
int gemm_w4a16_tier(int M, int K, int N, int *m_first, int *m_last) {
    const int dm = decode_max_m(K, N);
    if (M <= dm) {
        *m_first = 1;
        *m_last = dm;
        return 0;
    }
    const int mm = mid_max_m(K, N);
    if (M <= mm) {
        *m_first = dm + 1;
        *m_last = mm;
        return 1;
    }
    *m_first = mm + 1;
    *m_last = 0x7FFFFFFF;
    return 2;
}

size_t gemm_w4a16_workspace_bytes(int M, int K, int N) {
    if (M <= decode_max_m(K, N)) return 0;
    const int S = M <= mid_max_m(K, N) ? mid_splits(K, N) : big_splits(K, N);
    return S == 1 ? 0 : (size_t)S * M * N * sizeof(float);
}

void launch_splitk_reduce(const float *partials, int S, int M, int N, void *y, int y_f32, hipStream_t st) {
    const size_t MN = (size_t)M * N;
    const unsigned blocks = (unsigned)((MN / 4 + 255) / 256);
    hipLaunchKernelGGL(k_w4a16_splitk_reduce, dim3(blocks), dim3(256), 0, st, partials, S, MN, y, y_f32);
}

// Verify tier: row_blocks blocks of up to 16 MT rows, cbs column blocks, S K splits, one 1-D grid
// remapped inside the kernel.
template <int MT, int U>
static hipError_t launch_mid(const uint16_t *x, int M, const uint8_t *codes, const uint32_t *meta, int K, int N,
                             void *y, int y_f32, void *ws, int row_blocks, hipStream_t st) {
    const int S = mid_splits(K, N);
    const int cbs = (N / 16 + MID_TILES - 1) / MID_TILES;
    float *partials = S > 1 ? (float *)ws : nullptr;
    hipLaunchKernelGGL((k_w4a16_mid<MT, U>), dim3(cbs * S * row_blocks), dim3(MID_KP * MID_CW * 64), 0, st, x, M,
                       codes, meta, K, N, y, y_f32, S, partials, row_blocks);
    if (S > 1) launch_splitk_reduce(partials, S, M, N, y, y_f32, st);
    return hipGetLastError();
}

hipError_t launch_gemm_w4a16(const uint16_t *x, int M, const uint8_t *codes, const uint32_t *meta, int K,
                             int N, void *y, int y_f32, void *ws, hipStream_t st) {
    // Batch tiers, each with one reduction order for all its M: M <= decode_max_m(K, N) (decode,
    // one or two row tiles), up to mid_max_m(K, N) (verify tier: direct-to-LDS activations, K
    // parts, optional split-K, row blocks of at most 80), above (large tier, 128-row blocks).
    const int dm = decode_max_m(K, N);
    // Decode tier.  The ring depth does not change the reduction order, so it follows M: a 2-deep
    // ring for the wide workgroups where their registers are full (graph-timed, 4 -> 2 deep: Qwen
    // head at M = 3 - 9 68 -> 63 us, at 17 - 24 81 - 89 -> 77 - 85 us; Llama qkv at M = 16 7.8 -> 7.4
    // us, at 17 - 32 8.8 - 11.2 -> 8.2 - 10.7 us; Llama gate+up at M = 9 - 12 16.5 - 17.5 -> 17.7 -
    // 18.0 us, so only above 12 rows there).
    if (M <= 16 && M <= dm) {
        const int nt = decode_shape(K, N).nt;
        if (nt == 4)
            return M >= 2 ? launch_decode<4, 2, 1>(x, M, codes, meta, K, N, y, y_f32, st)
                          : launch_decode<4, 4, 1>(x, M, codes, meta, K, N, y, y_f32, st);
        if (nt == 2)
            return M > 12 ? launch_decode<2, 2, 1>(x, M, codes, meta, K, N, y, y_f32, st)
                          : launch_decode<2, 4, 1>(x, M, codes, meta, K, N, y, y_f32, st);
        return launch_decode<1, 4, 1>(x, M, codes, meta, K, N, y, y_f32, st);
    }
    if (M <= dm) {
        const int nt = decode_shape(K, N).nt;
        if (nt == 4) return launch_decode<4, 2, 2>(x, M, codes, meta, K, N, y, y_f32, st);
        if (nt == 2) return launch_decode<2, 2, 2>(x, M, codes, meta, K, N, y, y_f32, st);
        return launch_decode<1, 3, 2>(x, M, codes, meta, K, N, y, y_f32, st);
    }
    if (M <= mid_max_m(K, N)) {
        // ceil(M / 80) row blocks of equal height in whole row tiles; ring depth 3 up to 3 row
        // tiles, 2 above (a sweep over depths 2 - 8 at M = 20 - 80 on the Llama-3-8B projections:
        // the shallow rings were 1 - 14% faster than 4 - 8 deep ones)
        const int rbs = (M + 79) / 80;
        const int mt = ((M + rbs - 1) / rbs + 15) / 16;
        switch (mt) {
        case 1: return launch_mid<1, 3>(x, M, codes, meta, K, N, y, y_f32, ws, rbs, st);
        case 2: return launch_mid<2, 3>(x, M, codes, meta, K, N, y, y_f32, ws, rbs, st);
        case 3: return launch_mid<3, 3>(x, M, codes, meta, K, N, y, y_f32, ws, rbs, st);
        case 4: return launch_mid<4, 2>(x, M, codes, meta, K, N, y, y_f32, ws, rbs, st);
        default: return launch_mid<5, 2>(x, M, codes, meta, K, N, y, y_f32, ws, rbs, st);
        }
    }
    // Large tier: 128-row blocks x 256 columns, K splits for shapes with few column blocks, one
    // XCD-remapped 1-D grid (a 2-D (column block, split) grid for a single row block).  Where even
    // 384-column blocks give at least four workgroups per CU, the waves take 3 column tiles each
    // (fewer activation fragment reads from LDS per MFMA) with a 3-deep ring.  A row's reduction
    // order does not depend on the tiles per wave, so this choice may follow M.
    const int rbs = (M + BIG_MT * 16 - 1) / (BIG_MT * 16);
    const int S = big_splits(K, N);
    float *partials = S > 1 ? (float *)ws : nullptr;
    const int cbs3 = (N / 16 + BIG_CW * 3 - 1) / (BIG_CW * 3);
    if ((long long)cbs3 * S * rbs >= 4 * 256) {
        const dim3 grid = rbs > 1 ? dim3(cbs3 * S * rbs) : dim3(cbs3, S);
        hipLaunchKernelGGL((k_w4a16_lds<BIG_MT, 3, BIG_CW, 3>), grid, dim3(BIG_CW * 64), 0, st, x, M, codes, meta,
                           K, N, y, y_f32, S, partials, rbs);
    } else {
        const int cbs = (N / 16 + BIG_TILES - 1) / BIG_TILES;
        const dim3 grid = rbs > 1 ? dim3(cbs * S * rbs) : dim3(cbs, S);
        hipLaunchKernelGGL((k_w4a16_lds<BIG_MT, 4, BIG_CW, LDS_NT>), grid, dim3(BIG_CW * 64), 0, st, x, M, codes,
                           meta, K, N, y, y_f32, S, partials, rbs);
    }
    if (S > 1) launch_splitk_reduce(partials, S, M, N, y, y_f32, st);
    return hipGetLastError();
}

}  // namespace qspec
