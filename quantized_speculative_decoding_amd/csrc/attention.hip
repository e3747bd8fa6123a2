// Attention over the shared KV cache on gfx950 (QSPEC notes, QSPEC structure: the draft and the
// verifier attend over one KV cache in which the verifier's KV replaces the draft's for accepted
// tokens).  The pages fix no attention arithmetic; this is causal scaled dot-product attention:
// query token j of sequence b sits at position pos[b] + j and sees the cached positions
// 0 .. min(pos[b] + j, T - 1); query head h reads KV head h / (Hq / Hkv).
//
// All Q * G query rows that read one KV head (G = Hq / Hkv) are handled by one workgroup, so
// every cached key and value is read from HBM once per pass of up to 16 * RT rows.  Both
// contractions are bf16 MFMAs (v_mfma_f32_16x16x32_bf16; lane l = c + 16 kq):
//   scores  S^T = K Q^T: A = keys (row = position 16 tt + c), B = queries (col = row r = c), the
//           contraction over d in slots d = 32 j + 8 kq + i; lane l receives S[16 tt + 4 kq + e][c].
//   outputs O^T = V^T P^T: A = values transposed in registers (row c <-> d = 8 c + m for MFMA m),
//           B = probabilities (col = row r = c) in the 8 position slots {4 kq + e, 16 + 4 kq + e}
//           where the scores left them; lane l receives O[c][8 (4 kq + e) + m].
// So a row's scores, running max, running sum and outputs all sit on the 4 lanes c + 16 kq, and
// the online softmax needs only two cross-lane steps per reduction.  Probabilities enter the MFMA
// as a bf16 pair hi + lo (p - hi is exact in fp32), which keeps them to about 2^-17 relative.
//
// A wave streams 256 positions (8 steps of 32) through a 2-deep register ring; the 4 waves of a
// workgroup cover a chunk of 1024 positions and merge their (max, sum, outputs) through LDS in
// wave order; k_attn_combine merges the chunks of each query row in chunk order.  Keys and values
// are buffer loads whose range ends after the group's last visible position, so later rows of
// the cache are never read.
#include "common.hpp"
#include "kernels.hpp"

namespace qspec {

constexpr int kAttnD = 128;                      // head dimension
constexpr int kAttnWaves = 4;
constexpr int kAttnStep = 32;                    // positions per MFMA step
constexpr int kAttnSteps = 8;                    // steps per wave
constexpr int kAttnChunk = kAttnWaves * kAttnSteps * kAttnStep;   // 1024 positions per workgroup
constexpr int kAttnOPitch = kAttnD + 4;          // floats per LDS output row
constexpr int kAttnQPitch = kAttnD + 8;          // bf16 per LDS query row

typedef __attribute__((ext_vector_type(8))) __bf16 attn_bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float attn_f32x4_t;

struct AttnLayout {
    int NC;                                      // chunks per sequence
    size_t m, l, o, total;
};

static AttnLayout attn_layout(int B, int Q, int Hq, int T) {
    AttnLayout L = {};
    L.NC = (T + kAttnChunk - 1) / kAttnChunk;
    const size_t rows = (size_t)B * Q * Hq * L.NC;
    size_t off = 0;
    L.m = off; off = (off + rows * sizeof(float) + 255) & ~(size_t)255;
    L.l = off; off = (off + rows * sizeof(float) + 255) & ~(size_t)255;
    L.o = off; off = (off + rows * kAttnD * sizeof(float) + 255) & ~(size_t)255;
    L.total = off;
    return L;
}

size_t attention_workspace_bytes(int B, int Q, int Hq, int T) { return attn_layout(B, Q, Hq, T).total; }

// Last position visible to query token j of a sequence whose first query sits at p (p < 0 reads as 0).
__device__ __forceinline__ int attn_last(int p, int j, int T) {
    const long long v = (long long)max(p, 0) + j;
    return v < T ? (int)v : T - 1;
}

__device__ __forceinline__ attn_bf16x8_t attn_as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint4 u = {a, b, c, d};
    return __builtin_bit_cast(attn_bf16x8_t, u);
}

// Eight E4M3 codes (two dwords, code i in byte i) as eight bfloat16 values in the same order (every
// E4M3 value is a bfloat16 value: the conversion is exact).
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 c) {
    typedef __attribute__((ext_vector_type(2))) float f32x2_t;
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, true);
    const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, false), e = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, true);
    return make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(b[0], b[1]), pack_bf16x2(d[0], d[1]), pack_bf16x2(e[0], e[1]));
}

// FP8: the cache is E4M3 codes [B][2][Hkv][T][D] (kv) with one scale per (position, head) row,
// [B][2][Hkv][T] (kvs).  Keys and values are read as codes (half the bytes), widened exactly to
// bfloat16 in registers for the same MFMAs, and the scales enter where they factor out: a score
// is multiplied by its key's scale, and a probability by its value's scale before the PV product
// (the row sum keeps the unscaled probability).
template <int RT, bool FP8>
__global__ void __launch_bounds__(kAttnWaves * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_attn_partial(const uint16_t *__restrict__ q, const void *__restrict__ kv, const float *__restrict__ kvs,
               const int32_t *__restrict__ pos, int Q, int Hq, int Hkv, int T, float scale, int NC,
               float *__restrict__ wm, float *__restrict__ wl, float *__restrict__ wo) {
    constexpr int ROWS = 16 * RT;
    __shared__ float sm[kAttnWaves][ROWS], sl[kAttnWaves][ROWS];
    __shared__ __attribute__((aligned(16))) float so[kAttnWaves][ROWS][kAttnOPitch];
    __shared__ __attribute__((aligned(16))) uint16_t qs[ROWS][kAttnQPitch];

    const int chunk = blockIdx.x;
    const int b = blockIdx.y / Hkv, hk = blockIdx.y % Hkv;
    const int G = Hq / Hkv, R = Q * G;
    const int p0 = pos[b];
    const int lastmax = attn_last(p0, Q - 1, T);
    const int cbase = chunk * kAttnChunk;
    if (cbase > lastmax) return;                                  // uniform: nothing visible

    const int lane = threadIdx.x & 63, c = lane & 15, kq = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wbase = cbase + w * kAttnSteps * kAttnStep;
    const int ns = wbase > lastmax ? 0 : min(kAttnSteps, (lastmax - wbase) / kAttnStep + 1);
    // Wave-uniform buffer resources over the group's key and value planes, ending after the last
    // visible position: rows past it read as zero (their probabilities are zero).
    const size_t plane = (size_t)T * kAttnD;
    constexpr uint32_t ROWB = FP8 ? kAttnD : 2 * kAttnD;         // bytes per cached row
    const uint8_t *kvb = (const uint8_t *)kv;
    const rsrc_t kr = make_rsrc(kvb + ((size_t)(b * 2 + 0) * Hkv + hk) * plane * (ROWB / kAttnD),
                                (uint32_t)(lastmax + 1) * ROWB);
    const rsrc_t vr = make_rsrc(kvb + ((size_t)(b * 2 + 1) * Hkv + hk) * plane * (ROWB / kAttnD),
                                (uint32_t)(lastmax + 1) * ROWB);
    // per-row scales (FP8): the same positions' key and value scales; rows past the last visible
    // position read as zero (their probabilities are zero)
    const rsrc_t ksr = make_rsrc(FP8 ? kvs + ((size_t)(b * 2 + 0) * Hkv + hk) * T : kvs, FP8 ? (uint32_t)(lastmax + 1) * 4u : 0u);
    const rsrc_t vsr = make_rsrc(FP8 ? kvs + ((size_t)(b * 2 + 1) * Hkv + hk) * T : kvs, FP8 ? (uint32_t)(lastmax + 1) * 4u : 0u);
    constexpr uint32_t EB = FP8 ? 1u : 2u;                        // bytes per element
    const uint32_t kvo = (uint32_t)c * ROWB + 8u * EB * kq;      // key row c of a tile, d = 8 kq ..
    const uint32_t vvo = (uint32_t)kq * 4u * ROWB + 8u * EB * c; // value rows 4 kq + i, d = 8 c ..

    // K of step s: [position tile tt][d step j]; V of step s: [position slot i]
    // FP8 keys: lane (c, kq) holds the 32 contiguous codes d = 32 kq .. 32 kq + 31 of its row (two
    // 16-byte loads per tile) and MFMA j takes d = 32 kq + 8 j + i, the queries in the same slots;
    // the contraction over d is the same sum, and a quarter of the bfloat16 layout's loads.
    auto load_k = [&](int s, uint4 (&kb)[2][4]) {
        const uint32_t so = (uint32_t)(wbase + s * kAttnStep) * ROWB;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            if constexpr (FP8) {
                const uint32_t off = (uint32_t)c * ROWB + 32u * kq + tt * 16u * ROWB;
                kb[tt][0] = buf_load16(kr, off, so);
                kb[tt][1] = buf_load16(kr, off + 16u, so);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) kb[tt][j] = buf_load16(kr, kvo + tt * 16u * ROWB + 32u * EB * j, so);
            }
        }
    };
    auto load_v = [&](int s, uint4 (&vb)[8]) {
        const uint32_t so = (uint32_t)(wbase + s * kAttnStep) * ROWB;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t off = vvo + (i < 4 ? i : 12 + i) * ROWB;
            if constexpr (FP8) {
                typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
                const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(vr, off, so, 0));
                vb[i].x = v[0];
                vb[i].y = v[1];
            } else {
                vb[i] = buf_load16(vr, off, so);
            }
        }
    };
    // scales of the lane's 8 position slots of step s: tile tt, positions 16 tt + 4 kq + e; one
    // dword load each, so that every position up to the last visible one reads its own scale and
    // every later one reads zero (a 16-byte load straddling the range end is not split)
    auto load_scales = [&](const rsrc_t &r, int s, float (&sc8)[8]) {
        const uint32_t so = (uint32_t)(wbase + s * kAttnStep) * 4u;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) sc8[4 * tt + e] = __uint_as_float(buf_load4(r, (16u * tt + 4u * kq + e) * 4u, so));
    };

    for (int rp = 0; rp < R; rp += ROWS) {
        // the pass's query rows into LDS (rows past R repeat row R - 1; their results are dropped)
        for (int e = threadIdx.x; e < ROWS * (kAttnD / 8); e += kAttnWaves * kWave) {
            const int rr = e / (kAttnD / 8), d8 = (e % (kAttnD / 8)) * 8;
            const int r = min(rp + rr, R - 1);
            const int jq = r / G, g = r % G;
            *(uint4 *)&qs[rr][d8] = *(const uint4 *)(q + (((size_t)b * Q + jq) * Hq + hk * G + g) * kAttnD + d8);
        }
        int last[RT];
        float m[RT], l[RT];
        attn_f32x4_t o[RT][8];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            last[rt] = attn_last(p0, min(rp + rt * 16 + c, R - 1) / G, T);
            m[rt] = -INFINITY;
            l[rt] = 0.f;
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) o[rt][mm] = attn_f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();

        // K: two-deep ring, step s + 1 issued before step s's scores.  V: with one row tile, a
        // two-deep ring (step s + 1 issued after step s's scores); with two, step s is issued
        // before its own scores (registers for two row tiles of outputs leave no room for more).
        constexpr bool VRING = RT == 1;
        uint4 kb[2][2][4], vb[VRING ? 2 : 1][8];
        if (ns > 0) {
            load_k(0, kb[0]);
            if (VRING) load_v(0, vb[0]);
        }
#pragma unroll
        for (int s = 0; s < kAttnSteps; ++s) {
            if (s < ns) {
                const int cb = s & 1;
                float ks[8], vs[8];
                if constexpr (FP8) {
                    load_scales(ksr, s, ks);
                    load_scales(vsr, s, vs);
                }
                if (s + 1 < ns) load_k(s + 1, kb[cb ^ 1]);
                if (!VRING) load_v(s, vb[0]);
                const int tb = wbase + s * kAttnStep;
                uint4 kw[2][4];                                   // this step's keys as bfloat16
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if constexpr (FP8) {
                            const uint4 raw = kb[cb][tt][j >> 1];
                            kw[tt][j] = e4m3x8_to_bf16x8(j & 1 ? make_uint2(raw.z, raw.w) : make_uint2(raw.x, raw.y));
                        } else {
                            kw[tt][j] = kb[cb][tt][j];
                        }
                    }
                attn_bf16x8_t phi[RT], plo[RT];
                float alpha[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    float sc[8];
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        attn_f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(attn_bf16x8_t, kw[tt][j]),
                                __builtin_bit_cast(attn_bf16x8_t, *(const uint4 *)&qs[rt * 16 + c][FP8 ? 32 * kq + 8 * j : 32 * j + 8 * kq]),
                                acc, 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int t = tb + 16 * tt + 4 * kq + e;
                            const float a = FP8 ? acc[e] * ks[tt * 4 + e] : acc[e];
                            sc[tt * 4 + e] = t <= last[rt] ? a * scale : -INFINITY;
                        }
                    }
                    float mk = sc[0];
#pragma unroll
                    for (int i = 1; i < 8; ++i) mk = fmaxf(mk, sc[i]);
                    mk = fmaxf(mk, __shfl_xor(mk, 16, kWave));
                    mk = fmaxf(mk, __shfl_xor(mk, 32, kWave));
                    const float mn = fmaxf(m[rt], mk);
                    float p[8];
                    alpha[rt] = 1.f;
                    if (mn == -INFINITY) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) p[i] = 0.f;
                    } else {
                        alpha[rt] = __expf(m[rt] - mn);
#pragma unroll
                        for (int i = 0; i < 8; ++i) p[i] = __expf(sc[i] - mn);
                    }
                    m[rt] = mn;
                    float ps = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) ps += p[i];
                    l[rt] = __builtin_fmaf(l[rt], alpha[rt], ps);
                    if constexpr (FP8) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) p[i] *= vs[i];
                    }
                    uint32_t ph[4], pl[4];
#pragma unroll
                    for (int k2 = 0; k2 < 4; ++k2) {
                        ph[k2] = pack_bf16x2(p[2 * k2], p[2 * k2 + 1]);
                        const float h0 = __uint_as_float(ph[k2] << 16), h1 = __uint_as_float(ph[k2] & 0xFFFF0000u);
                        pl[k2] = pack_bf16x2(p[2 * k2] - h0, p[2 * k2 + 1] - h1);
                    }
                    phi[rt] = attn_as_bf16x8(ph[0], ph[1], ph[2], ph[3]);
                    plo[rt] = attn_as_bf16x8(pl[0], pl[1], pl[2], pl[3]);
                }
                if (VRING && s + 1 < ns) load_v(s + 1, vb[(cb ^ 1) % (VRING ? 2 : 1)]);
                const int vc = VRING ? cb : 0;
                uint4 vw[8];                                      // this step's values as bfloat16
#pragma unroll
                for (int i = 0; i < 8; ++i) vw[i] = FP8 ? e4m3x8_to_bf16x8(make_uint2(vb[vc][i].x, vb[vc][i].y)) : vb[vc][i];
#pragma unroll
                for (int mm = 0; mm < 8; ++mm) {
                    // V[slot i][8 c + mm] for the 8 position slots, transposed in registers
                    uint32_t d4[4];
#pragma unroll
                    for (int k2 = 0; k2 < 4; ++k2) {
                        const uint32_t x = ((const uint32_t *)&vw[2 * k2])[mm >> 1];
                        const uint32_t y = ((const uint32_t *)&vw[2 * k2 + 1])[mm >> 1];
                        d4[k2] = (mm & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
                    }
                    const attn_bf16x8_t vt = attn_as_bf16x8(d4[0], d4[1], d4[2], d4[3]);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        attn_f32x4_t acc = o[rt][mm] * alpha[rt];
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, phi[rt], acc, 0, 0, 0);
                        o[rt][mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, plo[rt], acc, 0, 0, 0);
                    }
                }
            }
        }

        // wave results into LDS: row r = rt * 16 + c on lanes c + 16 kq
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float lt = l[rt];
            lt += __shfl_xor(lt, 16, kWave);
            lt += __shfl_xor(lt, 32, kWave);
            const int r = rt * 16 + c;
            if (kq == 0) {
                sm[w][r] = m[rt];
                sl[w][r] = lt;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float *dst = &so[w][r][32 * kq + 8 * e];
                *(float4 *)dst = float4{o[rt][0][e], o[rt][1][e], o[rt][2][e], o[rt][3][e]};
                *(float4 *)(dst + 4) = float4{o[rt][4][e], o[rt][5][e], o[rt][6][e], o[rt][7][e]};
            }
        }
        __syncthreads();
        // merge the waves in wave order; one (row, 4 dimensions) item per thread and round
        for (int it = threadIdx.x; it < ROWS * (kAttnD / 4); it += kAttnWaves * kWave) {
            const int r = it / (kAttnD / 4), d = (it % (kAttnD / 4)) * 4;
            const int rg = rp + r;
            if (rg >= R) continue;
            float M = sm[0][r];
            for (int v = 1; v < kAttnWaves; ++v) M = fmaxf(M, sm[v][r]);
            float L = 0.f;
            float4 acc = {0.f, 0.f, 0.f, 0.f};
            if (M != -INFINITY) {
                for (int v = 0; v < kAttnWaves; ++v) {
                    const float wt = __expf(sm[v][r] - M);
                    const float4 x = *(const float4 *)&so[v][r][d];
                    L = __builtin_fmaf(sl[v][r], wt, L);
                    acc.x = __builtin_fmaf(x.x, wt, acc.x);
                    acc.y = __builtin_fmaf(x.y, wt, acc.y);
                    acc.z = __builtin_fmaf(x.z, wt, acc.z);
                    acc.w = __builtin_fmaf(x.w, wt, acc.w);
                }
            }
            const int jq = rg / G, g = rg % G;
            const size_t prow = (((size_t)b * Q + jq) * Hq + hk * G + g) * NC + chunk;
            *(float4 *)(wo + prow * kAttnD + d) = acc;
            if (d == 0) {
                wm[prow] = M;
                wl[prow] = L;
            }
        }
        __syncthreads();                                          // LDS reused by the next pass
    }
}

// One workgroup per query row (b, j, h), one thread per dimension: the chunks up to the row's
// causal limit, merged in chunk order with weights exp(m_c - M).  Chunks are taken 8 at a time
// with all their loads issued together; a later block with a larger maximum rescales the sums.
constexpr int kAttnMergeBlock = 8;

__global__ void __launch_bounds__(kAttnD)
k_attn_combine(const int32_t *__restrict__ pos, int Q, int Hq, int T, int NC, const float *__restrict__ wm,
               const float *__restrict__ wl, const float *__restrict__ wo, uint16_t *__restrict__ out) {
    const int row = blockIdx.x;
    const int j = (row / Hq) % Q, b = row / (Hq * Q);
    const int d = threadIdx.x;
    const int nc = attn_last(pos[b], j, T) / kAttnChunk + 1;
    const size_t base = (size_t)row * NC;
    float M = -INFINITY, L = 0.f, acc = 0.f;
    for (int c0 = 0; c0 < nc; c0 += kAttnMergeBlock) {
        float mv[kAttnMergeBlock], lv[kAttnMergeBlock], ov[kAttnMergeBlock];
#pragma unroll
        for (int i = 0; i < kAttnMergeBlock; ++i) {
            const int c = min(c0 + i, nc - 1);
            mv[i] = wm[base + c];
            lv[i] = wl[base + c];
            ov[i] = wo[(base + c) * kAttnD + d];
        }
        float Mb = M;
#pragma unroll
        for (int i = 0; i < kAttnMergeBlock; ++i)
            if (c0 + i < nc) Mb = fmaxf(Mb, mv[i]);
        const float r = __expf(M - Mb);                           // 0 on the first block
        L *= r;
        acc *= r;
#pragma unroll
        for (int i = 0; i < kAttnMergeBlock; ++i)
            if (c0 + i < nc) {
                const float wt = __expf(mv[i] - Mb);
                L = __builtin_fmaf(lv[i], wt, L);
                acc = __builtin_fmaf(ov[i], wt, acc);
            }
        M = Mb;
    }
    out[(size_t)row * kAttnD + d] = to_bf16_bits(acc / L);
}

template <bool FP8>
static hipError_t launch_attn(const uint16_t *q, const void *kv, const float *kvs, const int32_t *pos, int B, int Q,
                              int Hq, int Hkv, int T, float scale, uint16_t *out, void *ws, hipStream_t st) {
    const AttnLayout L = attn_layout(B, Q, Hq, T);
    char *w = (char *)ws;
    float *wm = (float *)(w + L.m), *wl = (float *)(w + L.l), *wo = (float *)(w + L.o);
    const dim3 grid(L.NC, B * Hkv);
    if (Q * (Hq / Hkv) <= 16)
        hipLaunchKernelGGL((k_attn_partial<1, FP8>), grid, dim3(kAttnWaves * kWave), 0, st, q, kv, kvs, pos, Q, Hq,
                           Hkv, T, scale, L.NC, wm, wl, wo);
    else
        hipLaunchKernelGGL((k_attn_partial<2, FP8>), grid, dim3(kAttnWaves * kWave), 0, st, q, kv, kvs, pos, Q, Hq,
                           Hkv, T, scale, L.NC, wm, wl, wo);
    hipLaunchKernelGGL(k_attn_combine, dim3(B * Q * Hq), dim3(kAttnD), 0, st, pos, Q, Hq, T, L.NC, wm, wl, wo, out);
    return hipGetLastError();
}

hipError_t launch_attention(const uint16_t *q, const uint16_t *cache, const int32_t *pos, int B, int Q, int Hq,
                            int Hkv, int T, float scale, uint16_t *out, void *ws, hipStream_t st) {
    return launch_attn<false>(q, cache, nullptr, pos, B, Q, Hq, Hkv, T, scale, out, ws, st);
}

hipError_t launch_attention_fp8(const uint16_t *q, const uint8_t *codes, const float *scales, const int32_t *pos,
                                int B, int Q, int Hq, int Hkv, int T, float scale, uint16_t *out, void *ws,
                                hipStream_t st) {
    return launch_attn<true>(q, codes, scales, pos, B, Q, Hq, Hkv, T, scale, out, ws, st);
}

}  // namespace qspec
