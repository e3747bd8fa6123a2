/*
 * Plain CPU oracle for the shared-INT4 speculative-decoding hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file: only the tests, the package smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no source, header, table or helper with the HIP
 * library; the two meet only through the seeded synthetic inputs.
 *
 * Style: scalar loops, one output at a time, fp64 / int64 accumulation, no
 * SIMD, no blocking, no reordering beyond what each definition states.  Built
 * with -ffp-contract=off so that the few fp32 operations the definitions fix
 * (the activation quantizer) are single IEEE operations.
 *
 * Sources (page titles as published):
 *   [QSPEC notes]  "QSPEC 논문 요점 정리" -- study notes on "QSPEC: Speculative
 *                  Decoding with Complementary Quantization Schemes" (Zhao et al.)
 *   [SpecQuant notes] "SpecQuant: Speculative Decoding with Multi-Parent Quantization
 *                  for Adaptive LLM Inference" -- a summary page (sections: one-line
 *                  summary, key contributions, approach, limitations)
 *   Sections of that page are named by content: background terms (weight-only
 *   vs weight-activation quantization, the dequantization example),
 *   speculative-decoding background (acceptance rule, first-reject cutoff,
 *   E[A], L = A + 1, E[L]), QSPEC structure (draft, verify, shared weights,
 *   KV replacement).
 *
 * Data formats (the pages fix none of them; these are this project's choices):
 *   weight codes  u8  [N/16][K/128][4][16][16]   tile-major: for column tile t = n/16 and group
 *                 g = k/128 one 1024-byte block; inside it quarter q = (k%128)/32, column
 *                 c = n%16, then 16 bytes holding k%32 = 0..31, even k in the low nibble.
 *                 Codes are unsigned 0..15.  N is a multiple of 16.
 *   weight meta   u32 [N/16][K/128][16]   bits 0..15 binary16 scale s, bits 16..23 zero
 *                 point z (0..15), bits 24..31 zero; entry (t, g, c) is column 16t + c.
 *   activations   u16 [M][K]     bfloat16 bit patterns
 *   act. codes    u8  [M][K/2]   4-bit two's complement, low nibble = even k
 *   act. scales   f32 [M][K/128]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_GROUP 128

/* ---- number formats, written from the IEEE 754 / bfloat16 definitions ---- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_fp16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of a binary32 pattern. */
double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Nearest bfloat16 to a finite double, ties to even.  bfloat16 keeps binary32's
 * exponent range with an 8-bit significand, so the spacing of representable
 * values around |v| = m * 2^e (m in [0.5, 1)) is 2^(e-8), never finer than the
 * subnormal spacing 2^-133.  nearbyint() rounds half to even in the default
 * rounding mode.
 */
uint16_t orc_double_to_bf16(double v)
{
    if (v != v) return 0x7FC0;
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    uint32_t bits;
    if (a == 0.0) {
        bits = 0;
    } else {
        int e;
        (void)frexp(a, &e);
        int qexp = e - 8;
        if (qexp < -133) qexp = -133;
        double r = ldexp(nearbyint(ldexp(a, -qexp)), qexp);
        if (r >= ldexp(1.0, 128)) {
            bits = 0x7F800000u;                     /* overflow to infinity */
        } else {
            float f = (float)r;                     /* exact: r has <= 8 significant bits */
            memcpy(&bits, &f, sizeof bits);
        }
    }
    return (uint16_t)((bits >> 16) | (neg ? 0x8000u : 0u));
}

/* ---- O1: shared-weight dequantization --------------------------------------
 * [QSPEC notes, background terms: dequantization example]  W_hat = s (W_INT4 - z),
 * then the 16-bit W_hat enters the matrix product.  The 16-bit type is bfloat16
 * (the activations are bfloat16); the product s*(w-z) is exact in double, so the
 * only rounding is the one to bfloat16.
 */
/* The weight store, read one element at a time through the layout definition above. */
static int weight_code(const uint8_t *codes, int64_t K, int64_t n, int64_t k)
{
    int64_t G = K / ORC_GROUP;
    int64_t block = (n / 16) * G + k / ORC_GROUP;
    int64_t q = (k % ORC_GROUP) / 32;
    int64_t byte_index = block * 1024 + q * 256 + (n % 16) * 16 + (k % 32) / 2;
    uint8_t byte = codes[byte_index];
    return (k & 1) ? (byte >> 4) & 15 : byte & 15;
}

static uint32_t meta_word(const uint32_t *meta, int64_t K, int64_t n, int64_t g)
{
    int64_t G = K / ORC_GROUP;
    return meta[((n / 16) * G + g) * 16 + n % 16];
}

static uint16_t meta_scale(uint32_t word) { return (uint16_t)(word & 0xFFFFu); }
static int meta_zero(uint32_t word) { return (int)((word >> 16) & 0xFFu); }

uint16_t orc_dequant_one(uint16_t scale_fp16, int w, int z)
{
    double s = orc_fp16_to_double(scale_fp16);
    return orc_double_to_bf16(s * (double)(w - z));
}

/* w_hat: u16 [N][K] bfloat16 patterns. */
void orc_dequant(const uint8_t *codes, const uint32_t *meta, int64_t K, int64_t N, uint16_t *w_hat)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint32_t word = meta_word(meta, K, n, k / ORC_GROUP);
            w_hat[n * K + k] = orc_dequant_one(meta_scale(word), weight_code(codes, K, n, k), meta_zero(word));
        }
}

/* ---- O2: W4A16 verify linear layer -----------------------------------------
 * [QSPEC notes, background terms: W4A16 and the dequantization example]
 * Y = X W_hat with bfloat16 X and the dequantized W_hat; the sum is taken in
 * double (every product of two bfloat16 values is exact in double).
 * y: f64 [M][N].
 */
void orc_gemm_w4a16(const uint16_t *x, int64_t M, const uint8_t *codes, const uint32_t *meta,
                    int64_t K, int64_t N, double *y)
{
    double *col = (double *)malloc(sizeof(double) * (size_t)K);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            uint32_t word = meta_word(meta, K, n, k / ORC_GROUP);
            col[k] = orc_bf16_to_double(
                orc_dequant_one(meta_scale(word), weight_code(codes, K, n, k), meta_zero(word)));
        }
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += orc_bf16_to_double(x[m * K + k]) * col[k];
            y[m * N + n] = acc;
        }
    }
    free(col);
}

/* ---- O3: per-token, per-group activation quantization ----------------------
 * [QSPEC notes, background terms: weight-activation quantization; W4A4 quantizes
 * both operands to 4 bits].  The page fixes no quantizer; the reading used here
 * is symmetric INT4 per (token, 128-wide group):
 *     a   = max |x|                        (exact)
 *     s_a = a / 7                          (one binary32 division, nearest-even)
 *     q   = clamp(nearest_even(x / s_a), -8, 7), or 0 when a == 0
 * x / s_a is one binary32 division.  Codes are stored as 4-bit two's complement,
 * even k in the low nibble.  codes: u8 [M][K/2], scales: f32 [M][K/128].
 */
void orc_quantize_act(const uint16_t *x, int64_t M, int64_t K, uint8_t *codes, float *scales)
{
    int64_t G = K / ORC_GROUP;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < G; ++g) {
            const uint16_t *xg = x + m * K + g * ORC_GROUP;
            float a = 0.0f;
            for (int k = 0; k < ORC_GROUP; ++k) {
                float v = fabsf(bf16_to_float(xg[k]));
                if (v > a) a = v;
            }
            float s = a / 7.0f;
            scales[m * G + g] = s;
            for (int k = 0; k < ORC_GROUP; ++k) {
                int q = 0;
                if (a != 0.0f) {
                    float r = bf16_to_float(xg[k]) / s;
                    float t = nearbyintf(r);
                    if (t < -8.0f) t = -8.0f;
                    if (t > 7.0f) t = 7.0f;
                    q = (int)t;
                }
                int64_t kk = g * ORC_GROUP + k;
                uint8_t *byte = &codes[m * (K / 2) + kk / 2];
                uint8_t nib = (uint8_t)(q & 15);
                if (kk & 1)
                    *byte = (uint8_t)((*byte & 0x0F) | (nib << 4));
                else
                    *byte = (uint8_t)((*byte & 0xF0) | nib);
            }
        }
}

static int act_code(const uint8_t *codes, int64_t K, int64_t m, int64_t k)
{
    uint8_t byte = codes[m * (K / 2) + k / 2];
    int nib = (k & 1) ? (byte >> 4) & 15 : byte & 15;
    return nib >= 8 ? nib - 16 : nib;
}

/* ---- O4: W4A4 draft linear layer --------------------------------------------
 * [QSPEC notes, background terms: W4A4 runs a low-precision kernel without
 * dequantization; the 4-bit MACs accumulate in INT32 and the scale is applied
 * afterwards.  QSPEC structure: the draft uses the same 4-bit weights.]
 * Because both scales are per group, the integer accumulation runs per group:
 *     D[g][m][n] = sum_{k in g} q_a[m][k] * (w[k][n] - z[n][g])     (integer)
 *     y[m][n]    = sum_g s_a[m][g] * s[n][g] * D[g][m][n]            (double)
 * D: i64 [K/128][M][N] (may be NULL), y: f64 [M][N].
 */
void orc_gemm_w4a4(const uint8_t *a_codes, const float *a_scales, int64_t M,
                   const uint8_t *codes, const uint32_t *meta, int64_t K, int64_t N, int64_t *D,
                   double *y)
{
    int64_t G = K / ORC_GROUP;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                uint32_t word = meta_word(meta, K, n, g);
                int z = meta_zero(word);
                int64_t dot = 0;
                for (int64_t k = g * ORC_GROUP; k < (g + 1) * ORC_GROUP; ++k)
                    dot += (int64_t)act_code(a_codes, K, m, k) * (int64_t)(weight_code(codes, K, n, k) - z);
                if (D) D[(g * M + m) * N + n] = dot;
                acc += (double)a_scales[m * G + g] * orc_fp16_to_double(meta_scale(word)) * (double)dot;
            }
            y[m * N + n] = acc;
        }
}

/* ---- O5: greedy verification ------------------------------------------------
 * [QSPEC notes, speculative-decoding background: under greedy decoding a draft
 * candidate is accepted when it equals the target's most probable token;
 * candidates after the first rejection are discarded; one more target token
 * follows, so L = A + 1.  QSPEC structure: the verifier scores gamma+1 positions.]
 * target: f32 [B][gamma+1][V]; draft_tokens: i32 [B][gamma].
 * accept: i32 [B]; out: i32 [B][gamma+1] (entries after position A are set to -1).
 * argmax ties go to the lowest index.  A draft token outside [0, V) never matches.
 */
static int64_t row_argmax(const float *row, int64_t V)
{
    int64_t best = 0;
    for (int64_t x = 1; x < V; ++x)
        if (row[x] > row[best]) best = x;
    return best;
}

void orc_verify_greedy(const float *target, const int32_t *draft_tokens, int64_t B, int64_t gamma,
                       int64_t V, int32_t *accept, int32_t *out)
{
    for (int64_t b = 0; b < B; ++b) {
        const float *tb = target + b * (gamma + 1) * V;
        int64_t A = 0;
        while (A < gamma) {
            int32_t d = draft_tokens[b * gamma + A];
            if (d < 0 || d >= V || (int64_t)d != row_argmax(tb + A * V, V)) break;
            ++A;
        }
        accept[b] = (int32_t)A;
        for (int64_t j = 0; j <= gamma; ++j) out[b * (gamma + 1) + j] = -1;
        for (int64_t j = 0; j < A; ++j) out[b * (gamma + 1) + j] = draft_tokens[b * gamma + j];
        out[b * (gamma + 1) + A] = (int32_t)row_argmax(tb + A * V, V);
    }
}

/* ---- O6: speculative-sampling verification ----------------------------------
 * [QSPEC notes, speculative-decoding background: candidate x is accepted with
 * probability min(1, p(x|h)/q(x|h)); the first rejection ends the round; a
 * correction token is drawn on rejection, and one extra target token is used
 * when every candidate is accepted, so L = A + 1.]
 * Readings where the page is silent: temperature 1; acceptance is the strict
 * test u < p/q with caller-supplied u in [0,1); the correction token is drawn
 * from the residual max(0, p - q) normalised (the distribution that makes the
 * committed token follow p), falling back to p when the residual has zero
 * mass; the extra token after full acceptance is drawn from p at position
 * gamma; drawing uses the inverse CDF at v * total mass with an inclusive
 * running sum (first x whose running sum exceeds the threshold; if rounding
 * leaves no such x, the last x of positive mass).
 * target: f32 [B][gamma+1][V]; draft: f32 [B][gamma][V]; draft_tokens i32 [B][gamma];
 * u: f32 [B][gamma]; v: f32 [B].
 * diag (may be NULL): f64 [B][gamma+1]; diag[b][j] for j < gamma is the accept
 * margin |u - p/q| / max(1, p/q) of each decision that was taken (NaN if not
 * taken); diag[b][gamma] is the distance from the threshold to the nearest
 * boundary of the drawn token's CDF interval, divided by the total mass.
 */
static void softmax_row(const float *logits, int64_t V, double *p)
{
    double mx = -INFINITY;
    for (int64_t x = 0; x < V; ++x)
        if ((double)logits[x] > mx) mx = (double)logits[x];
    double sum = 0.0;
    for (int64_t x = 0; x < V; ++x) {
        p[x] = exp((double)logits[x] - mx);
        sum += p[x];
    }
    for (int64_t x = 0; x < V; ++x) p[x] /= sum;
}

void orc_verify_sample(const float *target, const float *draft, const int32_t *draft_tokens,
                       const float *u, const float *v, int64_t B, int64_t gamma, int64_t V,
                       int32_t *accept, int32_t *out, double *diag)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    for (int64_t b = 0; b < B; ++b) {
        const float *tb = target + b * (gamma + 1) * V;
        const float *db = draft + b * gamma * V;
        if (diag)
            for (int64_t j = 0; j <= gamma; ++j) diag[b * (gamma + 1) + j] = NAN;
        int64_t A = 0;
        while (A < gamma) {
            int32_t d = draft_tokens[b * gamma + A];
            if (d < 0 || d >= V) break;
            softmax_row(tb + A * V, V, p);
            softmax_row(db + A * V, V, q);
            double ratio = p[d] / q[d];
            double ua = (double)u[b * gamma + A];
            if (diag) diag[b * (gamma + 1) + A] = fabs(ua - ratio) / (ratio > 1.0 ? ratio : 1.0);
            if (!(ua < ratio)) break;
            ++A;
        }
        /* distribution of the last committed token */
        softmax_row(tb + A * V, V, p);
        double total = 0.0;
        if (A < gamma) {
            softmax_row(db + A * V, V, q);
            for (int64_t x = 0; x < V; ++x) {
                double t = p[x] - q[x];
                r[x] = t > 0.0 ? t : 0.0;
                total += r[x];
            }
            if (!(total > 0.0)) {
                total = 0.0;
                for (int64_t x = 0; x < V; ++x) { r[x] = p[x]; total += r[x]; }
            }
        } else {
            for (int64_t x = 0; x < V; ++x) { r[x] = p[x]; total += r[x]; }
        }
        double thr = (double)v[b] * total;
        int64_t tok = -1;
        double run = 0.0, lo = 0.0, hi = 0.0;
        for (int64_t x = 0; x < V; ++x) {
            double before = run;
            run += r[x];
            if (run > thr) { tok = x; lo = before; hi = run; break; }
        }
        if (tok < 0) {
            for (int64_t x = V - 1; x >= 0; --x)
                if (r[x] > 0.0) { tok = x; break; }
            lo = hi = thr;
        }
        if (diag) {
            double dl = fabs(thr - lo), dh = fabs(hi - thr);
            diag[b * (gamma + 1) + gamma] = (dl < dh ? dl : dh) / total;
        }
        accept[b] = (int32_t)A;
        for (int64_t j = 0; j <= gamma; ++j) out[b * (gamma + 1) + j] = -1;
        for (int64_t j = 0; j < A; ++j) out[b * (gamma + 1) + j] = draft_tokens[b * gamma + j];
        out[b * (gamma + 1) + A] = (int32_t)tok;
    }
    free(p);
    free(q);
    free(r);
}

/* ---- O8: draft statistics and the adaptive-gamma controller ----------------
 * [SpecKV notes, architecture and mechanism: the draft's confidence is its
 * largest softmax probability and its uncertainty is the entropy of the
 * softmax; together with the compression level they feed a small MLP that
 * picks gamma.  Implementation guide (the controller listing): the entropy
 * adds 1e-9 inside the logarithm, the MLP is Linear(3 -> 64), ReLU,
 * Linear(64 -> max_gamma + 1), and gamma is the index of the largest output.]
 * Readings: softmax at temperature 1 in fp64 as in O6; confidence = max_x p(x);
 * entropy = -sum_x p(x) log(p(x) + 1e-9), summed in x order; the third input is
 * one caller-supplied number for all rows (the page feeds one column of the
 * compression-level one-hot); the MLP runs in fp64 on fp32 weights, every dot
 * product summed in input order after the bias; ties in the argmax take the
 * lowest index.
 * logits: f32 [R][V]; w1: f32 [64][3]; b1: f32 [64]; w2: f32 [G1][64]; b2: f32 [G1]
 * with G1 = max_gamma + 1.  features (may be NULL): f64 [R][2] = (confidence,
 * entropy); gamma: i32 [R]; logits_out (may be NULL): f64 [R][G1].
 */
void orc_speckv_gamma(const float *logits, int64_t R, int64_t V, float quant_feature,
                      const float *w1, const float *b1, const float *w2, const float *b2,
                      int64_t max_gamma, double *features, int32_t *gamma, double *logits_out)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    const int64_t G1 = max_gamma + 1;
    for (int64_t r = 0; r < R; ++r) {
        softmax_row(logits + r * V, V, p);
        double conf = 0.0, ent = 0.0;
        for (int64_t x = 0; x < V; ++x) {
            if (p[x] > conf) conf = p[x];
            ent += p[x] * log(p[x] + 1e-9);
        }
        ent = -ent;
        if (features) {
            features[2 * r] = conf;
            features[2 * r + 1] = ent;
        }
        const double in[3] = {conf, ent, (double)quant_feature};
        double h[64];
        for (int i = 0; i < 64; ++i) {
            double t = (double)b1[i];
            for (int k = 0; k < 3; ++k) t += (double)w1[i * 3 + k] * in[k];
            h[i] = t > 0.0 ? t : 0.0;
        }
        int32_t best = 0;
        double best_v = 0.0;
        for (int64_t j = 0; j < G1; ++j) {
            double t = (double)b2[j];
            for (int i = 0; i < 64; ++i) t += (double)w2[j * 64 + i] * h[i];
            if (logits_out) logits_out[r * G1 + j] = t;
            if (j == 0 || t > best_v) {
                best_v = t;
                best = (int32_t)j;
            }
        }
        gamma[r] = best;
    }
    free(p);
}

/* ---- O9: attention over the shared KV cache ---------------------------------
 * [QSPEC notes, QSPEC structure: the draft and the verifier attend over one KV
 * cache, in which the verifier's KV replaces the draft's for accepted tokens.]
 * The pages fix no attention arithmetic; the plainest reading is scaled
 * dot-product attention: query token j of sequence b sits at position
 * pos[b] + j and attends to the cached positions 0 .. min(pos[b] + j, T - 1)
 * (causal); query head h reads KV head h / (Hq / Hkv); scores s_t = scale *
 * q . k_t, weights softmax(s) (fp64, max subtracted), output sum_t p_t v_t
 * rounded to bfloat16 (nearest-even).
 * q: u16 [B][Q][Hq][D] bf16; cache: u16 [B][2][Hkv][T][D] bf16 (one layer; 0 = key,
 * 1 = value); pos: i32 [B]; out: u16 [B][Q][Hq][D] bf16.
 */
void orc_attention(const uint16_t *q, const uint16_t *cache, const int32_t *pos, int64_t B, int64_t Q,
                   int64_t Hq, int64_t Hkv, int64_t T, int64_t D, float scale, uint16_t *out)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)T);
    double *o = (double *)malloc(sizeof(double) * (size_t)D);
    const int64_t G = Hq / Hkv;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t j = 0; j < Q; ++j)
            for (int64_t h = 0; h < Hq; ++h) {
                const int64_t hk = h / G;
                const uint16_t *qv = q + ((b * Q + j) * Hq + h) * D;
                const uint16_t *kb = cache + ((b * 2 + 0) * Hkv + hk) * T * D;
                const uint16_t *vb = cache + ((b * 2 + 1) * Hkv + hk) * T * D;
                int64_t last = (int64_t)pos[b] + j;
                if (last > T - 1) last = T - 1;
                double mx = -INFINITY;
                for (int64_t t = 0; t <= last; ++t) {
                    double d = 0.0;
                    for (int64_t e = 0; e < D; ++e)
                        d += (double)bf16_to_float(qv[e]) * (double)bf16_to_float(kb[t * D + e]);
                    s[t] = (double)scale * d;
                    if (s[t] > mx) mx = s[t];
                }
                double sum = 0.0;
                for (int64_t t = 0; t <= last; ++t) {
                    s[t] = exp(s[t] - mx);
                    sum += s[t];
                }
                for (int64_t e = 0; e < D; ++e) o[e] = 0.0;
                for (int64_t t = 0; t <= last; ++t)
                    for (int64_t e = 0; e < D; ++e) o[e] += s[t] / sum * (double)bf16_to_float(vb[t * D + e]);
                uint16_t *ov = out + ((b * Q + j) * Hq + h) * D;
                for (int64_t e = 0; e < D; ++e) ov[e] = orc_double_to_bf16(o[e]);
            }
    free(s);
    free(o);
}

/* ---- O7: KV replacement for accepted positions ------------------------------
 * [QSPEC notes, QSPEC structure: for accepted tokens the low-precision KV the
 * W4A4 draft wrote is replaced by the KV the W4A16 verifier computed.]
 * The verifier scores gamma+1 positions starting at start_pos (the previous
 * round's last token followed by the gamma drafts), so the committed positions
 * start_pos .. start_pos + A all receive verify KV: rows r = 0..A are copied.
 * cache: u16 [L][B][2][H][T][D]; verify_kv: u16 [L][B][2][H][gamma+1][D].
 * Rows whose position falls outside [0, T) are skipped; accept counts outside
 * [0, gamma] are clamped.
 */
void orc_kv_overwrite(uint16_t *cache, const uint16_t *verify_kv, const int32_t *start_pos,
                      const int32_t *accept, int64_t L, int64_t B, int64_t H, int64_t T, int64_t D,
                      int64_t gamma)
{
    for (int64_t l = 0; l < L; ++l)
        for (int64_t b = 0; b < B; ++b) {
            int64_t A = accept[b];
            if (A < 0) A = 0;
            if (A > gamma) A = gamma;
            for (int64_t kv = 0; kv < 2; ++kv)
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t r = 0; r <= A; ++r) {
                        int64_t t = (int64_t)start_pos[b] + r;
                        if (t < 0 || t >= T) continue;
                        int64_t head = ((l * B + b) * 2 + kv) * H + h;
                        uint16_t *dst = cache + (head * T + t) * D;
                        const uint16_t *src = verify_kv + (head * (gamma + 1) + r) * D;
                        for (int64_t e = 0; e < D; ++e) dst[e] = src[e];
                    }
        }
}

/* ---- O11: the quantized KV cache -------------------------------------------
 * [QSPEC notes: the opening summary speaks of quantized KV; QSPEC structure: the
 * draft's low-precision KV is replaced by the verifier's for accepted tokens.]
 * Reading used here (the page fixes no format): the cache holds FP8 (OCP E4M3)
 * codes with one binary32 scale per (position, KV head) row of D values, made by
 * the per-row quantizer of the FP8 variant (O10): s = max |v| / 448, code =
 * nearest E4M3 value to v / s (ties to even, binary32 quotient), 0 and s = 0 for an
 * all-zero row; a value reads back as s * dec(code).
 * Layout: codes u8 [L][B][2][H][T][D], scales f32 [L][B][2][H][T] (2 = key, value).
 * orc_kv_overwrite_fp8 writes rows r = 0..A_b of the verifier's bfloat16 rows
 * there, quantized, at positions start_pos[b] + r (as O7, positions outside [0, T)
 * skipped, A clamped to [0, gamma]); orc_attention_fp8 is O9 (causal attention)
 * with each key and value read back from the codes and scales. */
void orc_quantize_act_fp8(const uint16_t *x, int64_t M, int64_t K, uint8_t *codes, float *scales);
double orc_e4m3_to_double(uint8_t c);

void orc_kv_overwrite_fp8(uint8_t *codes, float *scales, const uint16_t *verify_kv, const int32_t *start_pos,
                          const int32_t *accept, int64_t L, int64_t B, int64_t H, int64_t T, int64_t D,
                          int64_t gamma)
{
    for (int64_t l = 0; l < L; ++l)
        for (int64_t b = 0; b < B; ++b) {
            int64_t A = accept[b];
            if (A < 0) A = 0;
            if (A > gamma) A = gamma;
            for (int64_t kv = 0; kv < 2; ++kv)
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t r = 0; r <= A; ++r) {
                        int64_t t = (int64_t)start_pos[b] + r;
                        if (t < 0 || t >= T) continue;
                        int64_t head = ((l * B + b) * 2 + kv) * H + h;
                        const uint16_t *src = verify_kv + (head * (gamma + 1) + r) * D;
                        orc_quantize_act_fp8(src, 1, D, codes + (head * T + t) * D, scales + head * T + t);
                    }
        }
}

void orc_attention_fp8(const uint16_t *q, const uint8_t *codes, const float *scales, const int32_t *pos, int64_t B,
                       int64_t Q, int64_t Hq, int64_t Hkv, int64_t T, int64_t D, float scale, uint16_t *out)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)T);
    double *o = (double *)malloc(sizeof(double) * (size_t)D);
    const int64_t G = Hq / Hkv;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t j = 0; j < Q; ++j)
            for (int64_t h = 0; h < Hq; ++h) {
                const int64_t hk = h / G;
                const uint16_t *qv = q + ((b * Q + j) * Hq + h) * D;
                const int64_t kh = (b * 2 + 0) * Hkv + hk, vh = (b * 2 + 1) * Hkv + hk;
                int64_t last = (int64_t)pos[b] + j;
                if (last > T - 1) last = T - 1;
                double mx = -INFINITY;
                for (int64_t t = 0; t <= last; ++t) {
                    const double sk = (double)scales[kh * T + t];
                    double d = 0.0;
                    for (int64_t e = 0; e < D; ++e)
                        d += (double)bf16_to_float(qv[e]) * (sk * orc_e4m3_to_double(codes[(kh * T + t) * D + e]));
                    s[t] = (double)scale * d;
                    if (s[t] > mx) mx = s[t];
                }
                double sum = 0.0;
                for (int64_t t = 0; t <= last; ++t) {
                    s[t] = exp(s[t] - mx);
                    sum += s[t];
                }
                for (int64_t e = 0; e < D; ++e) o[e] = 0.0;
                for (int64_t t = 0; t <= last; ++t) {
                    const double sv = (double)scales[vh * T + t];
                    for (int64_t e = 0; e < D; ++e)
                        o[e] += s[t] / sum * (sv * orc_e4m3_to_double(codes[(vh * T + t) * D + e]));
                }
                uint16_t *ov = out + ((b * Q + j) * Hq + h) * D;
                for (int64_t e = 0; e < D; ++e) ov[e] = orc_double_to_bf16(o[e]);
            }
    free(s);
    free(o);
}

/* ---- O10: the FP8 parent variant ---------------------------------------------
 * [SpecQuant notes, one-line summary, key contributions and approach: INT4, FP8
 * and FP16 variants of one FP16 model are made by post-training quantization
 * with shared base weights; a low-precision draft proposes and a parent variant
 * verifies.  Limitations: the quantization recipe itself is not given.]
 * Reading used here (the page fixes none of it):
 *   - FP8 is OCP E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits, no
 *     infinities, 0x7F / 0xFF are NaN, largest finite value 448;
 *   - weights: one scale per output column, s_w = max_k |W[k][n]| / 448;
 *   - activations: one scale per token (row), s_a = max_k |x[m][k]| / 448, taken
 *     at run time (no calibration data is described);
 *   - codes: the nearest finite E4M3 value to (value / scale), ties to the even
 *     code, saturating at +-448; the quotient is one binary32 division;
 *   - y[m][n] = s_a[m] s_w[n] sum_k dec(a[m][k]) dec(w[k][n]).
 * Weight store u8 [N/16][K/128][2][64][16]: block (t, g) holds columns 16t..16t+15
 * and k = 128g..128g+127; byte (h, l, b) with l = c + 16 q is column 16t + c at
 * k = 128g + 32q + 16h + b.  Activation codes u8 [M][K] row-major.
 */
double orc_e4m3_to_double(uint8_t c)
{
    int e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    /* subnormal: m/8 * 2^-6; normal: (1 + m/8) * 2^(e-7) */
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (c & 0x80) ? -v : v;
}

uint8_t orc_double_to_e4m3(double v)
{
    double a = fabs(v);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {        /* finite non-negative codes, increasing values */
        double d = fabs(orc_e4m3_to_double((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best_d = d;
            best = c;
        }
    }
    return (uint8_t)((signbit(v) ? 0x80 : 0x00) | best);
}

void orc_quantize_act_fp8(const uint16_t *x, int64_t M, int64_t K, uint8_t *codes, float *scales)
{
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * K;
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(bf16_to_float(xr[k]));
            if (v > a) a = v;
        }
        float s = a / 448.0f;
        scales[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            float r = (a != 0.0f) ? bf16_to_float(xr[k]) / s : 0.0f;
            codes[m * K + k] = (a != 0.0f) ? orc_double_to_e4m3((double)r) : 0;
        }
    }
}

/* Post-training quantization of a bfloat16 weight matrix w [K][N] into codes [N][K]
 * (column n's codes contiguous) and per-column scales [N]. */
void orc_quantize_weights_fp8(const uint16_t *w, int64_t K, int64_t N, uint8_t *codes_nk, float *scales)
{
    for (int64_t n = 0; n < N; ++n) {
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(bf16_to_float(w[k * N + n]));
            if (v > a) a = v;
        }
        float s = a / 448.0f;
        scales[n] = s;
        for (int64_t k = 0; k < K; ++k) {
            float r = (a != 0.0f) ? bf16_to_float(w[k * N + n]) / s : 0.0f;
            codes_nk[n * K + k] = (a != 0.0f) ? orc_double_to_e4m3((double)r) : 0;
        }
    }
}

static uint8_t fp8_weight_code(const uint8_t *store, int64_t K, int64_t n, int64_t k)
{
    int64_t G = K / ORC_GROUP;
    int64_t kk = k % ORC_GROUP;
    int64_t block = (n / 16) * G + k / ORC_GROUP;
    int64_t lane = (n % 16) + 16 * (kk / 32);
    return store[block * 2048 + ((kk % 32) / 16) * 1024 + lane * 16 + kk % 16];
}

/* y f64 [M][N]: the exact products summed in double, then both scales. */
void orc_gemm_w8a8(const uint8_t *a_codes, const float *a_scales, int64_t M, const uint8_t *w_store,
                   const float *w_scales, int64_t K, int64_t N, double *y)
{
    double *col = (double *)malloc(sizeof(double) * (size_t)K);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) col[k] = orc_e4m3_to_double(fp8_weight_code(w_store, K, n, k));
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += orc_e4m3_to_double(a_codes[m * K + k]) * col[k];
            y[m * N + n] = (double)a_scales[m] * (double)w_scales[n] * acc;
        }
    }
    free(col);
}
