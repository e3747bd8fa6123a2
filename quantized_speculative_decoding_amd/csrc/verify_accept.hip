// Verification of gamma draft tokens per sequence on gfx950.
// (QSPEC notes, speculative-decoding background: greedy acceptance when the target's top-1 equals
//  the draft; otherwise acceptance with probability min(1, p/q); the first rejection discards the
//  rest; a correction token follows a rejection and an extra target token follows full
//  acceptance.  QSPEC structure: the verifier produces gamma+1 distributions.)
//
// Logit rows are far larger than one workgroup's LDS (a 128256-wide fp32 row is 501 KB), so every
// row is cut into chunks of VCHUNK logits (2 VCHUNK for a plentiful greedy argmax) and reduced in
// two deterministic stages:
//   greedy:   k_argmax_partial (one workgroup per row chunk: max and its lowest index)
//             -> k_greedy_accept (one thread per sequence: combine chunks in order, prefix match)
//   sampling: k_softmax_partial (per row chunk: chunk max and sum of exp(l - max) in fp64)
//             -> k_sample_accept (one wave per sequence: lanes combine the rows' chunk statistics
//                and test the candidates u < p(d)/q(d) in fp64; a ballot finds the first rejection)
//             -> k_residual_partial (per RCHUNK-logit chunk of the last row: mass of max(0, p - q),
//                or of p)
//             -> k_residual_pick (per sequence: locate the chunk and its 8-logit segment with
//                block-wide prefix sums in one fixed order, then walk that segment in logit order)
//   sampling with gamma = 0 (the draft-side head): k_softmax_partial -> k_head_pick (per row: the
//             chunk statistics are the chunk masses, so the chunk, a 32-logit segment inside it
//             and the token follow without a residual pass)
// Softmax normalizers, ratios and running sums are fp64; the exponentials are fp64 as well.  The
// residual stages use shorter chunks than the softmax statistics: they touch two rows per
// sequence instead of 2 gamma + 1, so 8192-logit chunks left most of the chip idle.
#include <float.h>
#include <limits.h>

#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace qspec {

constexpr int VCHUNK = 8192;     // logits per workgroup chunk (argmax and softmax statistics)
constexpr int RCHUNK = 2048;     // logits per workgroup chunk of the residual stages
constexpr int VT = 256;          // threads per workgroup
constexpr int RSEG = RCHUNK / VT;

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct VerifyLayout {
    int C;            // chunks per row
    int GCH;          // logits per greedy argmax chunk
    int CR;           // residual chunks per row
    size_t gval, gidx;                                   // greedy partials
    size_t pmax, psum, rowM, rowS, accA, resid, pmass;   // sampling partials
    size_t total;
};

static VerifyLayout verify_layout(int mode, int B, int gamma, int V) {
    VerifyLayout L = {};
    L.C = (V + VCHUNK - 1) / VCHUNK;
    L.CR = (V + RCHUNK - 1) / RCHUNK;
    const size_t Rt = (size_t)B * (gamma + 1);
    size_t off = 0;
    if (mode == 0) {
        const size_t wide = ((size_t)V + 2 * VCHUNK - 1) / (2 * VCHUNK);
        L.GCH = Rt * wide >= 1024 ? 2 * VCHUNK : VCHUNK;
        L.C = (V + L.GCH - 1) / L.GCH;
        L.gval = off; off = align256(off + Rt * L.C * sizeof(float));
        L.gidx = off; off = align256(off + Rt * L.C * sizeof(int));
    } else {
        const size_t R = Rt + (size_t)B * gamma;
        L.pmax = off; off = align256(off + R * L.C * sizeof(float));
        L.psum = off; off = align256(off + R * L.C * sizeof(double));
        L.rowM = off; off = align256(off + R * sizeof(float));
        L.rowS = off; off = align256(off + R * sizeof(double));
        L.accA = off; off = align256(off + (size_t)B * sizeof(int));
        L.resid = off; off = align256(off + (size_t)B * L.CR * sizeof(double));
        L.pmass = off; off = align256(off + (size_t)B * L.CR * sizeof(double));
    }
    L.total = off;
    return L;
}

size_t verify_workspace_bytes(int mode, int B, int gamma, int V) {
    return verify_layout(mode, B, gamma, V).total;
}

// ---------------------------------------------------------------------------------------------
// Block reductions (4 waves).  Shuffle trees at a fixed lane give a run-to-run fixed order.

struct ArgMax {
    float v;
    int i;
};

__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
    return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

__device__ ArgMax block_argmax(ArgMax a) {
    __shared__ float sv[VT / kWave];
    __shared__ int si[VT / kWave];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        ArgMax o = {__shfl_xor(a.v, off, kWave), __shfl_xor(a.i, off, kWave)};
        a = better(a, o);
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { sv[w] = a.v; si[w] = a.i; }
    __syncthreads();
    ArgMax r = {sv[0], si[0]};
    for (int k = 1; k < VT / kWave; ++k) r = better(r, ArgMax{sv[k], si[k]});
    return r;
}

__device__ float block_max(float v) {
    __shared__ float s[VT / kWave];
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = s[0];
    for (int k = 1; k < VT / kWave; ++k) r = fmaxf(r, s[k]);
    __syncthreads();
    return r;
}

__device__ double block_sum(double v) {
    __shared__ double s[VT / kWave];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_down(v, off, kWave);
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = s[0];
    for (int k = 1; k < VT / kWave; ++k) r += s[k];
    __syncthreads();
    return r;
}

// Visit the logits of [lo, hi) of one row, 16-byte vectors when the row allows it.
template <typename F>
__device__ __forceinline__ void for_chunk(const float *row, int lo, int hi, bool vec, F &&f) {
    if (vec) {
        for (int x = lo + 4 * (int)threadIdx.x; x < hi; x += 4 * VT) {
            const uint4 q = load_stream16(row + x);
            f(x, __uint_as_float(q.x));
            f(x + 1, __uint_as_float(q.y));
            f(x + 2, __uint_as_float(q.z));
            f(x + 3, __uint_as_float(q.w));
        }
    } else {
        for (int x = lo + (int)threadIdx.x; x < hi; x += VT) f(x, row[x]);
    }
}

// The N logits of a full, 16-byte-aligned chunk of N VT logits held by this thread: slot 4 k + e
// is logit lo + 4 VT k + 4 threadIdx.x + e, the order for_chunk visits them in.  All N / 4 loads
// are issued before the first is used, so a wave waits on one memory latency instead of N / 4.
constexpr int VPT = VCHUNK / VT;
template <int N>
__device__ __forceinline__ void load_full_chunk(const float *row, int lo, float (&v)[N]) {
    uint4 q[N / 4];
#pragma unroll
    for (int k = 0; k < N / 4; ++k) q[k] = load_stream16(row + lo + 4 * VT * k + 4 * (int)threadIdx.x);
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
        v[4 * k] = __uint_as_float(q[k].x);
        v[4 * k + 1] = __uint_as_float(q[k].y);
        v[4 * k + 2] = __uint_as_float(q[k].z);
        v[4 * k + 3] = __uint_as_float(q[k].w);
    }
}

// ---------------------------------------------------------------------------------------------
// Greedy.

// CH logits per workgroup: 2 VCHUNK when the rows give at least 1024 such workgroups (one
// generation on the chip, twice the bytes in flight per wave), else VCHUNK.
template <int CH>
__global__ void __launch_bounds__(VT)
k_argmax_partial(const float *__restrict__ target, size_t ldt, int V, int C, bool vec, float *__restrict__ gval,
                 int *__restrict__ gidx) {
    constexpr int PT = CH / VT;
    const int row = blockIdx.x / C, c = blockIdx.x % C;
    const float *p = target + (size_t)row * ldt;
    const int lo = c * CH, hi = min(V, lo + CH);
    ArgMax a = {-INFINITY, INT_MAX};
    // each thread visits increasing x, so keeping strict improvements keeps the lowest index
    auto visit = [&](int x, float v) {
        if (a.i == INT_MAX || v > a.v) { a.v = v; a.i = x; }
    };
    if (vec && hi - lo == CH) {
        float v[PT];
        load_full_chunk(p, lo, v);
#pragma unroll
        for (int k = 0; k < PT; ++k) visit(lo + 4 * VT * (k / 4) + 4 * (int)threadIdx.x + k % 4, v[k]);
    } else {
        for_chunk(p, lo, hi, vec, visit);
    }
    a = block_argmax(a);
    if (threadIdx.x == 0) {
        gval[blockIdx.x] = a.v;
        gidx[blockIdx.x] = a.i;
    }
}

__global__ void k_greedy_accept(const float *__restrict__ gval, const int *__restrict__ gidx, int C,
                                const int32_t *__restrict__ tokens, int B, int gamma, int V,
                                int32_t *__restrict__ accept, int32_t *__restrict__ out, int ldo) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    int A = 0;
    int top = 0;
    for (int j = 0; j <= gamma; ++j) {
        const size_t base = ((size_t)b * (gamma + 1) + j) * C;
        ArgMax r = {gval[base], gidx[base]};
        for (int c = 1; c < C; ++c) r = better(r, ArgMax{gval[base + c], gidx[base + c]});
        top = r.i;
        if (j == gamma) break;
        const int d = tokens[(size_t)b * gamma + j];
        if (d < 0 || d >= V || d != top) break;
        ++A;
    }
    accept[b] = A;
    for (int j = 0; j <= gamma; ++j) {
        int t = -1;
        if (j < A) t = tokens[(size_t)b * gamma + j];
        else if (j == A) t = top;
        out[(size_t)b * ldo + j] = t;
    }
}

// ---------------------------------------------------------------------------------------------
// Speculative sampling.

__device__ __forceinline__ const float *logit_row(const float *target, size_t ldt, const float *draft, int B,
                                                  int gamma, int V, long long row) {
    const long long Rt = (long long)B * (gamma + 1);
    return row < Rt ? target + (size_t)row * ldt : draft + (size_t)(row - Rt) * V;
}

__global__ void __launch_bounds__(VT)
k_softmax_partial(const float *__restrict__ target, size_t ldt, const float *__restrict__ draft, int B, int gamma,
                  int V, int C, bool vec, float *__restrict__ pmax, double *__restrict__ psum) {
    const long long row = blockIdx.x / C;
    const int c = blockIdx.x % C;
    const float *p = logit_row(target, ldt, draft, B, gamma, V, row);
    const int lo = c * VCHUNK, hi = min(V, lo + VCHUNK);
    float m = -INFINITY;
    double s = 0.0;
    if (vec && hi - lo == VCHUNK) {   // one read of the chunk, kept in registers for both passes
        float v[VPT];
        load_full_chunk(p, lo, v);
#pragma unroll
        for (int k = 0; k < VPT; ++k) m = fmaxf(m, v[k]);
        m = block_max(m);
        const double md = (double)m;
#pragma unroll
        for (int k = 0; k < VPT; ++k) s += exp((double)v[k] - md);
    } else {
        for_chunk(p, lo, hi, vec, [&](int, float v) { m = fmaxf(m, v); });
        m = block_max(m);
        const double md = (double)m;
        for_chunk(p, lo, hi, vec, [&](int, float v) { s += exp((double)v - md); });
    }
    s = block_sum(s);
    if (threadIdx.x == 0) {
        pmax[blockIdx.x] = m;
        psum[blockIdx.x] = s;
    }
}

// One wave per sequence.  Lane j combines the chunk statistics of row j of the sequence (target
// rows 0..gamma, then draft rows) in chunk order; then lane j tests candidate j, and the first
// rejection (an invalid token, or not u < p/q) among the candidates in order ends acceptance.
__global__ void __launch_bounds__(kWave)
k_sample_accept(const float *__restrict__ target, size_t ldt, const float *__restrict__ draft,
                const int32_t *__restrict__ tokens, const float *__restrict__ u,
                int B, int gamma, int V, int C, const float *__restrict__ pmax,
                const double *__restrict__ psum, float *__restrict__ rowM,
                double *__restrict__ rowS, int *__restrict__ accA,
                int32_t *__restrict__ accept, int32_t *__restrict__ out, int ldo) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const long long Rt = (long long)B * (gamma + 1);
    for (int j = lane; j < 2 * gamma + 1; j += kWave) {
        const long long row = j <= gamma ? (long long)b * (gamma + 1) + j : Rt + (long long)b * gamma + (j - gamma - 1);
        const size_t base = (size_t)row * C;
        float M = pmax[base];
        for (int c = 1; c < C; ++c) M = fmaxf(M, pmax[base + c]);
        double S = 0.0;
        for (int c = 0; c < C; ++c) S += psum[base + c] * exp((double)pmax[base + c] - (double)M);
        rowM[row] = M;
        rowS[row] = S;
    }
    __syncthreads();   // the rows' statistics, written above by other lanes
    int A = gamma;
    for (int j0 = 0; j0 < gamma; j0 += kWave) {
        const int j = j0 + lane;
        bool ok = false;
        if (j < gamma) {
            const int d = tokens[(size_t)b * gamma + j];
            if (d >= 0 && d < V) {
                const long long rt = (long long)b * (gamma + 1) + j;
                const long long rd = Rt + (long long)b * gamma + j;
                const double p = exp((double)target[(size_t)rt * ldt + d] - (double)rowM[rt]) / rowS[rt];
                const double q = exp((double)draft[(size_t)(rd - Rt) * V + d] - (double)rowM[rd]) / rowS[rd];
                ok = (double)u[(size_t)b * gamma + j] < p / q;
            }
        }
        const unsigned long long rej = __ballot(j < gamma && !ok);
        if (rej != 0ull) {
            A = j0 + __ffsll((long long)rej) - 1;
            break;
        }
    }
    if (lane == 0) {
        accA[b] = A;
        accept[b] = A;
    }
    for (int j = lane; j <= gamma; j += kWave)
        if (j != A) out[(size_t)b * ldo + j] = j < A ? tokens[(size_t)b * gamma + j] : -1;
}

// Residual (or target) mass at one logit of the last committed row.  The probabilities multiply
// by the reciprocals of the row normalizers (one rounding more than a division, about 1e-16
// relative, far inside the draw's near-tie band).  Contraction is off: fusing the draft product
// into the subtraction would leave the rounding error of p where p == q must give exactly 0
// (equal rows have zero residual mass and fall back to p).
struct ResidRow {
    const float *t;  // target row A
    const float *d;  // draft row A, or nullptr for the extra token (A == gamma)
    double Mt, iSt, Md, iSd;
    __device__ __forceinline__ double p(int x) const {
#pragma clang fp contract(off)
        return exp((double)t[x] - Mt) * iSt;
    }
    __device__ __forceinline__ double r_of(int x, double pv) const {
#pragma clang fp contract(off)
        if (!d) return pv;
        const double qv = exp((double)d[x] - Md) * iSd;
        const double dv = pv - qv;
        return dv > 0.0 ? dv : 0.0;
    }
    __device__ __forceinline__ double r(int x) const { return r_of(x, p(x)); }
    // the same residual from already loaded logits (tv = t[x], dv = d[x] when d is set)
    __device__ __forceinline__ double r_val(float tv, float dv) const {
#pragma clang fp contract(off)
        const double pv = exp((double)tv - Mt) * iSt;
        if (!d) return pv;
        const double rv = pv - exp((double)dv - Md) * iSd;
        return rv > 0.0 ? rv : 0.0;
    }
};

__device__ __forceinline__ ResidRow resid_row(const float *target, size_t ldt, const float *draft, int B,
                                              int gamma, int V, int b, int A, const float *rowM,
                                              const double *rowS) {
    const long long Rt = (long long)B * (gamma + 1);
    const long long rt = (long long)b * (gamma + 1) + A;
    ResidRow R;
    R.t = target + (size_t)rt * ldt;
    R.Mt = rowM[rt];
    R.iSt = 1.0 / rowS[rt];
    if (A < gamma) {
        const long long rd = Rt + (long long)b * gamma + A;
        R.d = draft + (size_t)(rd - Rt) * V;
        R.Md = rowM[rd];
        R.iSd = 1.0 / rowS[rd];
    } else {
        R.d = nullptr;
        R.Md = 0.0;
        R.iSd = 1.0;
    }
    return R;
}

__global__ void __launch_bounds__(VT)
k_residual_partial(const float *__restrict__ target, size_t ldt, const float *__restrict__ draft, int B,
                   int gamma, int V, int C, const float *__restrict__ rowM, const double *__restrict__ rowS,
                   const int *__restrict__ accA, double *__restrict__ resid, double *__restrict__ pmass) {
    const int b = blockIdx.x / C, c = blockIdx.x % C;   // C: residual chunks per row
    const ResidRow R = resid_row(target, ldt, draft, B, gamma, V, b, accA[b], rowM, rowS);
    const int lo = c * RCHUNK, hi = min(V, lo + RCHUNK);
    double sr = 0.0, sp = 0.0;
    for (int x = lo + (int)threadIdx.x; x < hi; x += VT) {
        const double pv = R.p(x);
        sr += R.r_of(x, pv);
        sp += pv;
    }
    sr = block_sum(sr);
    sp = block_sum(sp);
    if (threadIdx.x == 0) {
        resid[blockIdx.x] = sr;
        pmass[blockIdx.x] = sp;
    }
}

// Block-wide helpers for k_residual_pick (VT threads = 4 waves); every result is the same in all
// threads and comes from one fixed order of operations.
// Inclusive prefix sum in thread order: a shuffle scan per wave, then the wave totals in order.
__device__ double block_scan(double v) {
    __shared__ double wsum[VT / kWave];
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
    }
    if (lane == kWave - 1) wsum[w] = v;
    __syncthreads();
    double base = 0.0;
    for (int k = 0; k < w; ++k) base += wsum[k];
    __syncthreads();
    return base + v;
}

// The smallest (first = true) or largest thread index whose flag is set, or -1.
__device__ int block_find(bool f, bool first) {
    __shared__ int wpick[VT / kWave];
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const unsigned long long m = __ballot(f);
    if (lane == 0)
        wpick[w] = m == 0ull ? -1 : w * kWave + (first ? __ffsll((long long)m) - 1 : 63 - __clzll((long long)m));
    __syncthreads();
    int r = -1;
    for (int k = 0; k < VT / kWave; ++k) {
        const int c = first ? wpick[k] : wpick[VT / kWave - 1 - k];
        if (r < 0) r = c;
    }
    __syncthreads();
    return r;
}

// The value of v held by thread t (t uniform).
__device__ double block_bcast(double v, int t) {
    __shared__ double s;
    if ((int)threadIdx.x == t) s = v;
    __syncthreads();
    const double r = s;
    __syncthreads();
    return r;
}

// One workgroup per sequence: the chunk holding the threshold v * (total residual mass), the
// segment inside it and the token.  The chunk and segment searches are block-wide prefix sums
// (fixed order) and ballots; the token's own segment is walked in logit order.
__global__ void __launch_bounds__(VT)
k_residual_pick(const float *__restrict__ target, size_t ldt, const float *__restrict__ draft,
                const float *__restrict__ v, int B, int gamma, int V, int C,
                const float *__restrict__ rowM, const double *__restrict__ rowS,
                const int *__restrict__ accA, const double *__restrict__ resid,
                const double *__restrict__ pmass, int32_t *__restrict__ out, int ldo) {
    __shared__ double seg[VT];
    __shared__ int s_chunk, s_fallback, s_usep;
    __shared__ double s_thr;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int A = accA[b];
    ResidRow R = resid_row(target, ldt, draft, B, gamma, V, b, A, rowM, rowS);
    if (C <= VT) {   // one chunk mass per thread
        double part = tid < C ? resid[(size_t)b * C + tid] : 0.0;
        double pre = block_scan(part);
        double tot = block_bcast(pre, C - 1);
        const bool usep = !(tot > 0.0);
        if (usep) {
            part = tid < C ? pmass[(size_t)b * C + tid] : 0.0;
            pre = block_scan(part);
            tot = block_bcast(pre, C - 1);
        }
        const double thr = (double)v[b] * tot;
        int chunk = block_find(tid < C && pre > thr, true);
        const bool fallback = chunk < 0;
        double before = 0.0;
        if (fallback) {
            chunk = block_find(tid < C && part > 0.0, false);
            if (chunk < 0) chunk = C - 1;
        } else {
            before = block_bcast(pre - part, chunk);
        }
        if (tid == 0) {
            s_chunk = chunk;
            s_fallback = fallback;
            s_usep = usep;
            s_thr = thr - before;
        }
    } else if (tid == 0) {   // more chunks than threads: one thread walks them in order
        const double *part = resid + (size_t)b * C;
        double tot = 0.0;
        for (int c = 0; c < C; ++c) tot += part[c];
        int usep = 0;
        if (!(tot > 0.0)) {
            usep = 1;
            part = pmass + (size_t)b * C;
            tot = 0.0;
            for (int c = 0; c < C; ++c) tot += part[c];
        }
        const double thr = (double)v[b] * tot;
        double run = 0.0, before = 0.0;
        int chunk = -1;
        for (int c = 0; c < C; ++c) {
            before = run;
            run += part[c];
            if (run > thr) { chunk = c; break; }
        }
        int fallback = 0;
        if (chunk < 0) {
            fallback = 1;
            for (int c = C - 1; c >= 0; --c)
                if (part[c] > 0.0) { chunk = c; break; }
            if (chunk < 0) chunk = C - 1;
        }
        s_chunk = chunk;
        s_fallback = fallback;
        s_usep = usep;
        s_thr = thr - before;
    }
    __syncthreads();
    if (s_usep) R.d = nullptr;
    const int lo = s_chunk * RCHUNK, hi = min(V, lo + RCHUNK);
    const int x0 = lo + tid * RSEG, x1 = min(hi, x0 + RSEG);
    // the segment's logits first (all loads in flight), then its residual mass in logit order
    float tv[RSEG], dv[RSEG];
#pragma unroll
    for (int k = 0; k < RSEG; ++k) {
        const int x = x0 + k;
        tv[k] = x < x1 ? R.t[x] : 0.f;
        dv[k] = (R.d && x < x1) ? R.d[x] : 0.f;
    }
    double mine = 0.0;
#pragma unroll
    for (int k = 0; k < RSEG; ++k)
        if (x0 + k < x1) mine += R.r_val(tv[k], dv[k]);
    // The segment holding the threshold: the first whose inclusive prefix exceeds it.
    const double thr = s_thr;
    const double pre = block_scan(mine);
    const int tsel = s_fallback ? -1 : block_find(pre > thr, true);
    if (tsel >= 0) {
        const double run = block_bcast(pre - mine, tsel);   // mass before the segment
        // the segment's residuals in parallel, then the running sum through them in order
        const int a = lo + tsel * RSEG, e = min(hi, a + RSEG);
        if (tid < e - a) seg[tid] = R.r(a + tid);
        __syncthreads();
        if (tid == 0) {
            int tok = -1;
            double rr = run;
            for (int x = a; x < e; ++x) {
                rr += seg[x - a];
                if (rr > thr) { tok = x; break; }
            }
            if (tok < 0)   // rounding left the threshold at the segment's end
                for (int x = e - 1; x >= a; --x)
                    if (seg[x - a] > 0.0) { tok = x; break; }
            if (tok < 0) tok = min(a, hi - 1);
            out[(size_t)b * ldo + A] = tok;
        }
        return;
    }
    // No crossing: the last logit of positive mass in the chunk (each thread finds the last one in
    // its segment; the highest wins), else the chunk's last logit.
    int last = -1;
    for (int x = x1 - 1; x >= x0; --x)
        if (R.r(x) > 0.0) { last = x; break; }
    const int owner = block_find(last >= 0, false);
    if (tid == 0 && owner < 0) out[(size_t)b * ldo + A] = hi - 1;
    if (owner >= 0 && tid == owner) out[(size_t)b * ldo + A] = last;
}

// Sampling with gamma = 0 (the draft-side head; a verification with no draft tokens): the draw
// from softmax(row) needs no residual pass, because the row's own chunk statistics are its chunk
// masses.  One workgroup per row: the row's maximum M and total S from the chunk statistics in
// chunk order, chunk c's mass W_c = psum_c exp(pmax_c - M), the chunk holding u S by a block-wide
// prefix sum over the chunks, then inside that chunk a prefix sum over 32-logit segments of
// exp(x - M) and a walk through the crossing segment in logit order (by the thread that holds
// it).  Rounding can put u S past a chunk's recomputed mass; then, as in k_residual_pick, the
// last logit of positive mass in the chunk is drawn (a near tie of the inverse CDF).
constexpr int HSEG = VCHUNK / VT;   // logits per thread in the chunk walk
static_assert(VCHUNK % VT == 0, "whole segments per chunk");

__global__ void __launch_bounds__(VT)
k_head_pick(const float *__restrict__ logits, size_t ldt, const float *__restrict__ u, int V, int C, bool vec,
            const float *__restrict__ pmax, const double *__restrict__ psum, int32_t *__restrict__ accept,
            int32_t *__restrict__ out, int ldo) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const float *row = logits + (size_t)b * ldt;
    const float *pm = pmax + (size_t)b * C;
    const double *ps = psum + (size_t)b * C;
    // the row's statistics in chunk order (every thread the same loop, the same result)
    float Mf = pm[0];
    for (int c = 1; c < C; ++c) Mf = fmaxf(Mf, pm[c]);
    const double M = (double)Mf;
    __shared__ int s_chunk, s_fallback;
    __shared__ double s_thr;
    if (C <= VT) {
        const double part = tid < C ? ps[tid] * exp((double)pm[tid] - M) : 0.0;
        const double pre = block_scan(part);
        const double tot = block_bcast(pre, C - 1);
        const double thr = (double)u[b] * tot;
        int chunk = block_find(tid < C && pre > thr, true);
        const bool fallback = chunk < 0;
        double before = 0.0;
        if (fallback) {
            chunk = block_find(tid < C && part > 0.0, false);
            if (chunk < 0) chunk = C - 1;
        } else {
            before = block_bcast(pre - part, chunk);
        }
        if (tid == 0) {
            s_chunk = chunk;
            s_fallback = fallback;
            s_thr = thr - before;
        }
    } else if (tid == 0) {   // more chunks than threads: one thread walks them in order
        double tot = 0.0;
        for (int c = 0; c < C; ++c) tot += ps[c] * exp((double)pm[c] - M);
        const double thr = (double)u[b] * tot;
        double run = 0.0, before = 0.0;
        int chunk = -1;
        for (int c = 0; c < C; ++c) {
            before = run;
            run += ps[c] * exp((double)pm[c] - M);
            if (run > thr) { chunk = c; break; }
        }
        int fallback = 0;
        if (chunk < 0) {
            fallback = 1;
            for (int c = C - 1; c >= 0; --c)
                if (ps[c] > 0.0) { chunk = c; break; }
            if (chunk < 0) chunk = C - 1;
        }
        s_chunk = chunk;
        s_fallback = fallback;
        s_thr = thr - before;
    }
    __syncthreads();
    const int lo = s_chunk * VCHUNK, hi = min(V, lo + VCHUNK);
    const int x0 = lo + tid * HSEG, x1 = min(hi, x0 + HSEG);
    // The chunk is read with coalesced loads into LDS (4-logit piece q at slot (q / 8) * 8 +
    // (q % 8) ^ (q / 8 % 8), so that the segment reads below hit distinct bank groups), then each
    // thread takes its HSEG contiguous logits from there.  Logits past the row read as 0 and are
    // never used.
    __shared__ float4 stage[VCHUNK / 4];
    static_assert(HSEG == 32, "eight 4-logit pieces per thread");
#pragma unroll
    for (int k = 0; k < VCHUNK / 4 / VT; ++k) {
        const int q = tid + VT * k;
        const int x = lo + 4 * q;
        float4 v;
        if (vec && x + 3 < hi) {
            v = *(const float4 *)(row + x);
        } else {
            v.x = x < hi ? row[x] : 0.f;
            v.y = x + 1 < hi ? row[x + 1] : 0.f;
            v.z = x + 2 < hi ? row[x + 2] : 0.f;
            v.w = x + 3 < hi ? row[x + 3] : 0.f;
        }
        const int t = q >> 3, i = q & 7;
        stage[t * 8 + (i ^ (t & 7))] = v;
    }
    __syncthreads();
    float lv[HSEG];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 v = stage[tid * 8 + (i ^ (tid & 7))];
        lv[4 * i] = v.x;
        lv[4 * i + 1] = v.y;
        lv[4 * i + 2] = v.z;
        lv[4 * i + 3] = v.w;
    }
    double wv[HSEG];   // exp(x - M) of the segment's logits (0 past the chunk), kept for the walk
#pragma unroll
    for (int k = 0; k < HSEG; ++k) wv[k] = x0 + k < x1 ? exp((double)lv[k] - M) : 0.0;
    double mine = 0.0;
#pragma unroll
    for (int k = 0; k < HSEG; ++k) mine += wv[k];
    const double thr = s_thr;
    const double pre = block_scan(mine);
    const int tsel = s_fallback ? -1 : block_find(pre > thr, true);
    if (tid == 0) accept[b] = 0;
    if (tsel >= 0) {
        if (tid == tsel) {
            double run = pre - mine;
            int tok = -1, lastpos = -1;
#pragma unroll
            for (int k = 0; k < HSEG; ++k) {
                if (tok < 0 && x0 + k < x1) {
                    if (wv[k] > 0.0) lastpos = x0 + k;
                    run += wv[k];
                    if (run > thr) tok = x0 + k;
                }
            }
            if (tok < 0) tok = lastpos >= 0 ? lastpos : min(x0, hi - 1);   // rounding at the segment's end
            out[(size_t)b * ldo] = tok;
        }
        return;
    }
    // No crossing: the last logit of positive mass in the chunk, else the chunk's last logit.
    int last = -1;
    for (int k = HSEG - 1; k >= 0; --k)
        if (x0 + k < x1 && wv[k] > 0.0) { last = x0 + k; break; }
    const int owner = block_find(last >= 0, false);
    if (tid == 0 && owner < 0) out[(size_t)b * ldo] = hi - 1;
    if (owner >= 0 && tid == owner) out[(size_t)b * ldo] = last;
}

// ---------------------------------------------------------------------------------------------
// Draft statistics and the adaptive-gamma controller (SpecKV notes, architecture and mechanism;
// the implementation guide's controller): per draft row, confidence = max p and entropy =
// -sum p log(p + 1e-9) of softmax(row) in fp64, then Linear(3 -> 64), ReLU, Linear(64 -> G1) and
// the index of the largest output (lowest on ties).  Stages: k_softmax_partial (chunk max and
// sum of exp), k_entropy_partial (per chunk: sum of p log(p + 1e-9) with the row's max and
// normalizer), k_speckv_head (one wave per row: combine in chunk order, run the MLP).
constexpr int kSpeckvHidden = 64;
// The entropy pass spends two fp64 transcendentals per logit; its chunks are a quarter of the
// statistics chunks, so a few draft rows still give about four workgroups per CU.
constexpr int ECHUNK = VCHUNK / 4;

struct SpeckvLayout {
    int C, CE;   // statistics chunks and entropy chunks per row
    size_t pmax, psum, pent, total;
};

static SpeckvLayout speckv_layout(int R, int V) {
    SpeckvLayout L = {};
    L.C = (V + VCHUNK - 1) / VCHUNK;
    L.CE = (V + ECHUNK - 1) / ECHUNK;
    size_t off = 0;
    L.pmax = off; off = align256(off + (size_t)R * L.C * sizeof(float));
    L.psum = off; off = align256(off + (size_t)R * L.C * sizeof(double));
    L.pent = off; off = align256(off + (size_t)R * L.CE * sizeof(double));
    L.total = off;
    return L;
}

size_t speckv_workspace_bytes(int R, int V) { return speckv_layout(R, V).total; }

// The row's max and softmax normalizer from its chunk statistics, in chunk order.
__device__ __forceinline__ void row_stats(const float *pmax, const double *psum, int C, float &M, double &S) {
    M = pmax[0];
    for (int c = 1; c < C; ++c) M = fmaxf(M, pmax[c]);
    S = 0.0;
    for (int c = 0; c < C; ++c) S += psum[c] * exp((double)pmax[c] - (double)M);
}

__global__ void __launch_bounds__(VT)
k_entropy_partial(const float *__restrict__ logits, size_t ldt, int V, int C, int CE, const float *__restrict__ pmax,
                  const double *__restrict__ psum, double *__restrict__ pent) {
    __shared__ float sM;
    __shared__ double sS;
    const int row = blockIdx.x / CE, c = blockIdx.x % CE;
    if (threadIdx.x == 0) {
        float M;
        double S;
        row_stats(pmax + (size_t)row * C, psum + (size_t)row * C, C, M, S);
        sM = M;
        sS = S;
    }
    __syncthreads();
    const double M = (double)sM, S = sS;
    const float *p = logits + (size_t)row * ldt;
    const int lo = c * ECHUNK, hi = min(V, lo + ECHUNK);
    double t = 0.0;
    for (int x = lo + (int)threadIdx.x; x < hi; x += VT) {
        const double pv = exp((double)p[x] - M) / S;
        t += pv * log(pv + 1e-9);
    }
    t = block_sum(t);
    if (threadIdx.x == 0) pent[blockIdx.x] = t;
}

__global__ void __launch_bounds__(kWave)
k_speckv_head(int C, int CE, const float *__restrict__ pmax, const double *__restrict__ psum,
              const double *__restrict__ pent, float quant_feature, const float *__restrict__ w1,
              const float *__restrict__ b1, const float *__restrict__ w2, const float *__restrict__ b2, int G1,
              double *__restrict__ features, int32_t *__restrict__ gamma_out) {
#pragma clang fp contract(off)
    __shared__ double h[kSpeckvHidden];
    const int row = blockIdx.x;
    const int lane = threadIdx.x;
    float M;
    double S;
    row_stats(pmax + (size_t)row * C, psum + (size_t)row * C, C, M, S);
    double ent = 0.0;
    for (int c = 0; c < CE; ++c) ent += pent[(size_t)row * CE + c];
    ent = -ent;
    const double conf = 1.0 / S;       // the largest probability: exp(M - M) / S
    const double in[3] = {conf, ent, (double)quant_feature};
    {
        double t = (double)b1[lane];
        for (int k = 0; k < 3; ++k) t += (double)w1[lane * 3 + k] * in[k];
        h[lane] = t > 0.0 ? t : 0.0;
    }
    __syncthreads();
    double o = -INFINITY;
    if (lane < G1) {
        o = (double)b2[lane];
        for (int i = 0; i < kSpeckvHidden; ++i) o += (double)w2[lane * kSpeckvHidden + i] * h[i];
    }
    // argmax over the lanes, lowest index on ties (lanes past G1 hold -inf and lose)
    int best = lane < G1 ? lane : INT_MAX;
    double bv = o;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double ov = __shfl_xor(bv, off, kWave);
        const int oi = __shfl_xor(best, off, kWave);
        if (ov > bv || (ov == bv && oi < best)) {
            bv = ov;
            best = oi;
        }
    }
    if (lane == 0) {
        gamma_out[row] = best;
        if (features) {
            features[2 * (size_t)row] = conf;
            features[2 * (size_t)row + 1] = ent;
        }
    }
}

hipError_t launch_speckv_gamma(const float *logits, int R, int V, float quant_feature, const float *w1,
                               const float *b1, const float *w2, const float *b2, int max_gamma,
                               double *features, int32_t *gamma_out, void *ws, hipStream_t st) {
    const SpeckvLayout L = speckv_layout(R, V);
    char *w = (char *)ws;
    const int C = L.C;
    float *pmax = (float *)(w + L.pmax);
    double *psum = (double *)(w + L.psum);
    double *pent = (double *)(w + L.pent);
    const bool vec = (V % 4 == 0) && ((uintptr_t)logits % 16 == 0);
    // R rows of "target" logits and no draft rows: the verification's chunk pass with gamma = 0
    hipLaunchKernelGGL(k_softmax_partial, dim3((unsigned)((long long)R * C)), dim3(VT), 0, st, logits, (size_t)V,
                       (const float *)nullptr, R, 0, V, C, vec, pmax, psum);
    hipLaunchKernelGGL(k_entropy_partial, dim3((unsigned)((long long)R * L.CE)), dim3(VT), 0, st, logits, (size_t)V, V,
                       C, L.CE, pmax, psum, pent);
    hipLaunchKernelGGL(k_speckv_head, dim3(R), dim3(kWave), 0, st, C, L.CE, pmax, psum, pent, quant_feature, w1, b1, w2, b2,
                       max_gamma + 1, features, gamma_out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------

// Target row r starts at target + r * ldt; out row b at out + b * ldo (verification: ldt = V,
// ldo = gamma + 1; the draft-side head reads one step's rows of a [B][gamma][V] buffer).
static hipError_t launch_verify(int mode, const float *target, size_t ldt, const float *draft,
                                const int32_t *tokens, const float *u_accept, const float *u_resample,
                                int B, int gamma, int V, int32_t *accept, int32_t *out, int ldo, void *ws,
                                hipStream_t st) {
    const VerifyLayout L = verify_layout(mode, B, gamma, V);
    char *w = (char *)ws;
    const int C = L.C;
    const bool vec_t = (V % 4 == 0) && (ldt % 4 == 0) && ((uintptr_t)target % 16 == 0);
    const long long Rt = (long long)B * (gamma + 1);
    if (mode == 0) {
        float *gval = (float *)(w + L.gval);
        int *gidx = (int *)(w + L.gidx);
        if (L.GCH == 2 * VCHUNK)
            hipLaunchKernelGGL(k_argmax_partial<2 * VCHUNK>, dim3((unsigned)(Rt * C)), dim3(VT), 0, st, target, ldt, V,
                               C, vec_t, gval, gidx);
        else
            hipLaunchKernelGGL(k_argmax_partial<VCHUNK>, dim3((unsigned)(Rt * C)), dim3(VT), 0, st, target, ldt, V, C,
                               vec_t, gval, gidx);
        hipLaunchKernelGGL(k_greedy_accept, dim3((B + 63) / 64), dim3(64), 0, st, gval, gidx, C, tokens,
                           B, gamma, V, accept, out, ldo);
        return hipGetLastError();
    }
    const bool vec = vec_t && (gamma == 0 || (uintptr_t)draft % 16 == 0);
    const long long R = Rt + (long long)B * gamma;
    float *pmax = (float *)(w + L.pmax);
    double *psum = (double *)(w + L.psum);
    float *rowM = (float *)(w + L.rowM);
    double *rowS = (double *)(w + L.rowS);
    int *accA = (int *)(w + L.accA);
    double *resid = (double *)(w + L.resid);
    double *pmass = (double *)(w + L.pmass);
    hipLaunchKernelGGL(k_softmax_partial, dim3((unsigned)(R * C)), dim3(VT), 0, st, target, ldt, draft, B,
                       gamma, V, C, vec, pmax, psum);
    if (gamma == 0) {   // no candidates: the draw from each row's softmax, straight from its statistics
        hipLaunchKernelGGL(k_head_pick, dim3(B), dim3(VT), 0, st, target, ldt, u_resample, V, C, vec_t, pmax, psum,
                           accept, out, ldo);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_sample_accept, dim3(B), dim3(kWave), 0, st, target, ldt, draft, tokens,
                       u_accept, B, gamma, V, C, pmax, psum, rowM, rowS, accA, accept, out, ldo);
    hipLaunchKernelGGL(k_residual_partial, dim3((unsigned)((long long)B * L.CR)), dim3(VT), 0, st, target, ldt,
                       draft, B, gamma, V, L.CR, rowM, rowS, accA, resid, pmass);
    hipLaunchKernelGGL(k_residual_pick, dim3(B), dim3(VT), 0, st, target, ldt, draft, u_resample, B, gamma, V,
                       L.CR, rowM, rowS, accA, resid, pmass, out, ldo);
    return hipGetLastError();
}

hipError_t launch_verify_accept(int mode, const float *target, const float *draft,
                                const int32_t *tokens, const float *u_accept, const float *u_resample,
                                int B, int gamma, int V, int32_t *accept, int32_t *out, void *ws,
                                hipStream_t st) {
    return launch_verify(mode, target, (size_t)V, draft, tokens, u_accept, u_resample, B, gamma, V, accept, out,
                         gamma + 1, ws, st);
}

// The verification's scratch for callers that cannot allocate: a fixed device array, one copy per
// GPU, alive until the process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a registration handle); the device address comes from hipGetSymbolAddress, once
// per device, on that device's first call.
static __device__ __align__(256) unsigned char scratch[kVerifyScratchBytes];

constexpr int kMaxScratchDevices = 64;
static void *scratch_ptr[kMaxScratchDevices];
static std::mutex scratch_mutex;

hipError_t verify_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return hipSuccess;
}

// The draft-side head: one token per row of a draft step's logits (row b at logits + b * ldt),
// written to tokens[b * ldo]; the verification with gamma = 0 (greedy: the argmax; sampling: the
// inverse-CDF draw from softmax(row) at u[b]).  Its accept counts (always 0) go to the workspace
// after the verification's own layout.
size_t draft_sample_workspace_bytes(int mode, int B, int V) {
    return align256(verify_layout(mode, B, 0, V).total) + align256((size_t)B * sizeof(int32_t));
}

hipError_t launch_draft_sample(int mode, const float *logits, size_t ldt, const float *u, int B, int V,
                               int32_t *tokens, int ldo, void *ws, hipStream_t st) {
    int32_t *acc = (int32_t *)((char *)ws + align256(verify_layout(mode, B, 0, V).total));
    return launch_verify(mode, logits, ldt, nullptr, nullptr, nullptr, u, B, 0, V, acc, tokens, ldo, ws, st);
}

// The draft-side head and the adaptive-gamma controller on the same draft rows.  SAMPLE: the
// head's chunk statistics (max and sum of exp per chunk, k_softmax_partial) are the ones the
// controller needs, so one statistics pass over the rows feeds both and the controller adds only
// its entropy pass and its MLP.  GREEDY: the head takes argmaxes, so the controller's statistics
// pass runs after it.  Workspace: the head's, then the controller's per-chunk entropies (SAMPLE)
// or its whole layout (GREEDY).
size_t draft_speckv_workspace_bytes(int mode, int B, int V) {
    const size_t head = align256(draft_sample_workspace_bytes(mode, B, V));
    if (mode == 0) return head + speckv_layout(B, V).total;
    const int CE = (V + ECHUNK - 1) / ECHUNK;
    return head + align256((size_t)B * CE * sizeof(double));
}

hipError_t launch_draft_speckv(int mode, const float *logits, size_t ldt, const float *u, int B, int V,
                               int32_t *tokens, int ldo, float quant_feature, const float *w1, const float *b1,
                               const float *w2, const float *b2, int max_gamma, double *features,
                               int32_t *gamma_out, void *ws, hipStream_t st) {
    hipError_t e = launch_draft_sample(mode, logits, ldt, u, B, V, tokens, ldo, ws, st);
    if (e != hipSuccess) return e;
    char *w = (char *)ws;
    const size_t head = align256(draft_sample_workspace_bytes(mode, B, V));
    const int C = (V + VCHUNK - 1) / VCHUNK;
    const float *pmax;
    const double *psum;
    double *pent;
    if (mode == 0) {
        const SpeckvLayout S = speckv_layout(B, V);
        float *m = (float *)(w + head + S.pmax);
        double *sum = (double *)(w + head + S.psum);
        pent = (double *)(w + head + S.pent);
        const bool vec = (V % 4 == 0) && (ldt % 4 == 0) && ((uintptr_t)logits % 16 == 0);
        hipLaunchKernelGGL(k_softmax_partial, dim3((unsigned)((long long)B * C)), dim3(VT), 0, st, logits, ldt,
                           (const float *)nullptr, B, 0, V, C, vec, m, sum);
        pmax = m;
        psum = sum;
    } else {
        const VerifyLayout L = verify_layout(mode, B, 0, V);
        pmax = (const float *)(w + L.pmax);
        psum = (const double *)(w + L.psum);
        pent = (double *)(w + head);
    }
    const int CE = (V + ECHUNK - 1) / ECHUNK;
    hipLaunchKernelGGL(k_entropy_partial, dim3((unsigned)((long long)B * CE)), dim3(VT), 0, st, logits, ldt, V, C, CE,
                       pmax, psum, pent);
    hipLaunchKernelGGL(k_speckv_head, dim3(B), dim3(kWave), 0, st, C, CE, pmax, psum, pent, quant_feature, w1, b1, w2,
                       b2, max_gamma + 1, features, gamma_out);
    return hipGetLastError();
}

}  // namespace qspec
