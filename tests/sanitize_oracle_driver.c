/*
 * Test driver for the oracle under AddressSanitizer and UndefinedBehaviorSanitizer: calls every
 * entry point of oracle/qspec_oracle.c on small shapes, with every buffer allocated at exactly
 * the size its documented layout states, including the edge cases the definitions name (draft
 * tokens outside [0, V), accept counts outside [0, gamma], positions past the cache end, gamma
 * = 0, a single row, zero groups).  It checks memory safety and defined behaviour only; the
 * values are pinned by the Python tests.  Built and run by tests/test_oracle_sanitizers.py.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_fp16_to_double(uint16_t h);
double orc_bf16_to_double(uint16_t b);
uint16_t orc_double_to_bf16(double v);
uint16_t orc_dequant_one(uint16_t scale_fp16, int w, int z);
void orc_dequant(const uint8_t *codes, const uint32_t *meta, int64_t K, int64_t N, uint16_t *w_hat);
void orc_gemm_w4a16(const uint16_t *x, int64_t M, const uint8_t *codes, const uint32_t *meta, int64_t K,
                    int64_t N, double *y);
void orc_quantize_act(const uint16_t *x, int64_t M, int64_t K, uint8_t *codes, float *scales);
void orc_gemm_w4a4(const uint8_t *a_codes, const float *a_scales, int64_t M, const uint8_t *codes,
                   const uint32_t *meta, int64_t K, int64_t N, int64_t *D, double *y);
void orc_verify_greedy(const float *target, const int32_t *draft_tokens, int64_t B, int64_t gamma, int64_t V,
                       int32_t *accept, int32_t *out);
void orc_verify_sample(const float *target, const float *draft, const int32_t *draft_tokens, const float *u,
                       const float *v, int64_t B, int64_t gamma, int64_t V, int32_t *accept, int32_t *out,
                       double *diag);
void orc_speckv_gamma(const float *logits, int64_t R, int64_t V, float quant_feature, const float *w1,
                      const float *b1, const float *w2, const float *b2, int64_t max_gamma, double *features,
                      int32_t *gamma, double *logits_out);
void orc_attention(const uint16_t *q, const uint16_t *cache, const int32_t *pos, int64_t B, int64_t Q,
                   int64_t Hq, int64_t Hkv, int64_t T, int64_t D, float scale, uint16_t *out);
void orc_kv_overwrite(uint16_t *cache, const uint16_t *verify_kv, const int32_t *start_pos,
                      const int32_t *accept, int64_t L, int64_t B, int64_t H, int64_t T, int64_t D, int64_t gamma);
double orc_e4m3_to_double(uint8_t c);
uint8_t orc_double_to_e4m3(double v);
void orc_quantize_act_fp8(const uint16_t *x, int64_t M, int64_t K, uint8_t *codes, float *scales);
void orc_quantize_weights_fp8(const uint16_t *w, int64_t K, int64_t N, uint8_t *codes_nk, float *scales);
void orc_gemm_w8a8(const uint8_t *a_codes, const float *a_scales, int64_t M, const uint8_t *w_store,
                   const float *w_scales, int64_t K, int64_t N, double *y);
void orc_kv_overwrite_fp8(uint8_t *codes, float *scales, const uint16_t *verify_kv, const int32_t *start_pos,
                          const int32_t *accept, int64_t L, int64_t B, int64_t H, int64_t T, int64_t D,
                          int64_t gamma);
void orc_attention_fp8(const uint16_t *q, const uint8_t *codes, const float *scales, const int32_t *pos, int64_t B,
                       int64_t Q, int64_t Hq, int64_t Hkv, int64_t T, int64_t D, float scale, uint16_t *out);

static uint64_t state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void)
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(state >> 32);
}

static float uniform01(void) { return (float)(next_u32() >> 8) * (1.0f / 16777216.0f); }

static void *alloc(size_t bytes)
{
    void *p = malloc(bytes ? bytes : 1);
    if (!p) abort();
    return p;
}

/* bfloat16 patterns of moderate finite values (exponent field 120..131), random signs. */
static void fill_bf16(uint16_t *a, size_t n)
{
    for (size_t i = 0; i < n; ++i) a[i] = (uint16_t)(((next_u32() & 1u) << 15) | ((120u + next_u32() % 12u) << 7) |
                                                      (next_u32() & 127u));
}

static void fill_bytes(uint8_t *a, size_t n)
{
    for (size_t i = 0; i < n; ++i) a[i] = (uint8_t)next_u32();
}

static void fill_logits(float *a, size_t n)
{
    for (size_t i = 0; i < n; ++i) a[i] = 6.0f * uniform01() - 3.0f;
}

/* Weight store for K x N: codes [N/16][K/128][1024], meta [N/16][K/128][16] with binary16
 * scales in [2^-10, 2^-6) and zero points 0..15. */
static void make_weights(int64_t K, int64_t N, uint8_t **codes, uint32_t **meta)
{
    size_t blocks = (size_t)(N / 16) * (size_t)(K / 128);
    *codes = (uint8_t *)alloc(blocks * 1024);
    *meta = (uint32_t *)alloc(blocks * 16 * sizeof(uint32_t));
    fill_bytes(*codes, blocks * 1024);
    for (size_t i = 0; i < blocks * 16; ++i) {
        uint32_t scale = ((5u + next_u32() % 4u) << 10) | (next_u32() & 1023u);
        (*meta)[i] = scale | ((next_u32() % 16u) << 16);
    }
}

static void linear_layers(int64_t M, int64_t K, int64_t N)
{
    uint8_t *codes;
    uint32_t *meta;
    make_weights(K, N, &codes, &meta);
    uint16_t *x = (uint16_t *)alloc((size_t)(M * K) * 2);
    fill_bf16(x, (size_t)(M * K));
    /* one all-zero group: the quantizer's a == 0 branch */
    memset(x, 0, 128 * sizeof(uint16_t));
    uint16_t *w_hat = (uint16_t *)alloc((size_t)(N * K) * 2);
    orc_dequant(codes, meta, K, N, w_hat);
    double *y = (double *)alloc((size_t)(M * N) * sizeof(double));
    orc_gemm_w4a16(x, M, codes, meta, K, N, y);
    uint8_t *a_codes = (uint8_t *)alloc((size_t)(M * K / 2));
    float *a_scales = (float *)alloc((size_t)(M * K / 128) * sizeof(float));
    orc_quantize_act(x, M, K, a_codes, a_scales);
    int64_t *D = (int64_t *)alloc((size_t)(K / 128 * M * N) * sizeof(int64_t));
    orc_gemm_w4a4(a_codes, a_scales, M, codes, meta, K, N, D, y);
    orc_gemm_w4a4(a_codes, a_scales, M, codes, meta, K, N, NULL, y);
    free(D);
    free(a_scales);
    free(a_codes);
    free(y);
    free(w_hat);
    free(x);
    free(meta);
    free(codes);
}

static void verification(int64_t B, int64_t gamma, int64_t V)
{
    float *t = (float *)alloc((size_t)(B * (gamma + 1) * V) * sizeof(float));
    float *d = (float *)alloc((size_t)(B * gamma * V) * sizeof(float));
    int32_t *tok = (int32_t *)alloc((size_t)(B * gamma) * sizeof(int32_t));
    float *u = (float *)alloc((size_t)(B * gamma) * sizeof(float));
    float *v = (float *)alloc((size_t)B * sizeof(float));
    int32_t *acc = (int32_t *)alloc((size_t)B * sizeof(int32_t));
    int32_t *out = (int32_t *)alloc((size_t)(B * (gamma + 1)) * sizeof(int32_t));
    double *diag = (double *)alloc((size_t)(B * (gamma + 1)) * sizeof(double));
    fill_logits(t, (size_t)(B * (gamma + 1) * V));
    fill_logits(d, (size_t)(B * gamma * V));
    for (int64_t i = 0; i < B * gamma; ++i) {
        uint32_t r = next_u32() % 8u;
        tok[i] = r == 0 ? -1 : r == 1 ? (int32_t)V : (int32_t)(next_u32() % (uint32_t)V);
        u[i] = uniform01();
    }
    for (int64_t b = 0; b < B; ++b) v[b] = b == 0 ? 0.0f : uniform01();
    orc_verify_greedy(t, tok, B, gamma, V, acc, out);
    orc_verify_sample(t, d, tok, u, v, B, gamma, V, acc, out, diag);
    orc_verify_sample(t, d, tok, u, v, B, gamma, V, acc, out, NULL);
    /* q == p: every rejection meets a zero residual (the fallback branch) */
    if (gamma > 0) {
        for (int64_t b = 0; b < B; ++b)
            memcpy(d + b * gamma * V, t + b * (gamma + 1) * V, (size_t)(gamma * V) * sizeof(float));
        orc_verify_sample(t, d, tok, u, v, B, gamma, V, acc, out, diag);
    }
    free(diag);
    free(out);
    free(acc);
    free(v);
    free(u);
    free(tok);
    free(d);
    free(t);
}

static void controller(int64_t R, int64_t V, int64_t max_gamma)
{
    const int64_t G1 = max_gamma + 1;
    float *logits = (float *)alloc((size_t)(R * V) * sizeof(float));
    float *w1 = (float *)alloc(64 * 3 * sizeof(float)), *b1 = (float *)alloc(64 * sizeof(float));
    float *w2 = (float *)alloc((size_t)(G1 * 64) * sizeof(float)), *b2 = (float *)alloc((size_t)G1 * sizeof(float));
    fill_logits(logits, (size_t)(R * V));
    fill_logits(w1, 64 * 3);
    fill_logits(b1, 64);
    fill_logits(w2, (size_t)(G1 * 64));
    fill_logits(b2, (size_t)G1);
    double *feat = (double *)alloc((size_t)(R * 2) * sizeof(double));
    int32_t *g = (int32_t *)alloc((size_t)R * sizeof(int32_t));
    double *lo = (double *)alloc((size_t)(R * G1) * sizeof(double));
    orc_speckv_gamma(logits, R, V, 0.5f, w1, b1, w2, b2, max_gamma, feat, g, lo);
    orc_speckv_gamma(logits, R, V, 1.0f, w1, b1, w2, b2, max_gamma, NULL, g, NULL);
    free(lo);
    free(g);
    free(feat);
    free(b2);
    free(w2);
    free(b1);
    free(w1);
    free(logits);
}

static void attention(int64_t B, int64_t Q, int64_t Hq, int64_t Hkv, int64_t T)
{
    const int64_t D = 128;
    uint16_t *q = (uint16_t *)alloc((size_t)(B * Q * Hq * D) * 2);
    uint16_t *cache = (uint16_t *)alloc((size_t)(B * 2 * Hkv * T * D) * 2);
    uint16_t *out = (uint16_t *)alloc((size_t)(B * Q * Hq * D) * 2);
    int32_t *pos = (int32_t *)alloc((size_t)B * sizeof(int32_t));
    fill_bf16(q, (size_t)(B * Q * Hq * D));
    fill_bf16(cache, (size_t)(B * 2 * Hkv * T * D));
    for (int64_t b = 0; b < B; ++b) pos[b] = b == 0 ? -3 : b == 1 ? (int32_t)(T + 5) : (int32_t)(next_u32() % (uint32_t)T);
    orc_attention(q, cache, pos, B, Q, Hq, Hkv, T, D, 0.0883883f, out);
    free(pos);
    free(out);
    free(cache);
    free(q);
}

static void kv(int64_t L, int64_t B, int64_t H, int64_t T, int64_t D, int64_t gamma)
{
    uint16_t *cache = (uint16_t *)alloc((size_t)(L * B * 2 * H * T * D) * 2);
    uint16_t *stage = (uint16_t *)alloc((size_t)(L * B * 2 * H * (gamma + 1) * D) * 2);
    int32_t *start = (int32_t *)alloc((size_t)B * sizeof(int32_t));
    int32_t *acc = (int32_t *)alloc((size_t)B * sizeof(int32_t));
    fill_bf16(cache, (size_t)(L * B * 2 * H * T * D));
    fill_bf16(stage, (size_t)(L * B * 2 * H * (gamma + 1) * D));
    for (int64_t b = 0; b < B; ++b) {
        start[b] = b == 0 ? -2 : b == 1 ? (int32_t)(T - 1) : (int32_t)(next_u32() % (uint32_t)T);
        acc[b] = b == 2 ? -4 : (int32_t)(next_u32() % (uint32_t)(gamma + 1));
    }
    /* the last sequence's rows end the staging buffer: an accept count past gamma must be clamped */
    start[B - 1] = 0;
    acc[B - 1] = (int32_t)(gamma + 9);
    orc_kv_overwrite(cache, stage, start, acc, L, B, H, T, D, gamma);
    free(acc);
    free(start);
    free(stage);
    free(cache);
}

/* the quantized cache: rows written by the FP8 overwrite (edge starts and accept counts as in kv),
 * then attention over one layer of it with the same causal edge positions as attention() */
static void kv_fp8(int64_t L, int64_t B, int64_t H, int64_t T, int64_t gamma, int64_t Q)
{
    const int64_t D = 128;
    uint8_t *codes = (uint8_t *)alloc((size_t)(L * B * 2 * H * T * D));
    float *scales = (float *)alloc((size_t)(L * B * 2 * H * T) * sizeof(float));
    uint16_t *stage = (uint16_t *)alloc((size_t)(L * B * 2 * H * (gamma + 1) * D) * 2);
    int32_t *start = (int32_t *)alloc((size_t)B * sizeof(int32_t));
    int32_t *acc = (int32_t *)alloc((size_t)B * sizeof(int32_t));
    fill_bytes(codes, (size_t)(L * B * 2 * H * T * D));
    for (int64_t i = 0; i < L * B * 2 * H * T * D; ++i)
        if ((codes[i] & 0x7F) == 0x7F) codes[i] ^= 1;   /* no NaN codes */
    for (int64_t i = 0; i < L * B * 2 * H * T; ++i) scales[i] = 0.01f * (float)(1 + i % 7);
    fill_bf16(stage, (size_t)(L * B * 2 * H * (gamma + 1) * D));
    for (int64_t i = 0; i < D; ++i) stage[i] = 0;          /* one all-zero row: s = 0, codes 0 */
    for (int64_t b = 0; b < B; ++b) {
        start[b] = b == 0 ? -2 : b == 1 ? (int32_t)(T - 1) : (int32_t)(next_u32() % (uint32_t)T);
        acc[b] = b == 2 ? -4 : (int32_t)(next_u32() % (uint32_t)(gamma + 1));
    }
    start[B - 1] = 0;
    acc[B - 1] = (int32_t)(gamma + 9);
    orc_kv_overwrite_fp8(codes, scales, stage, start, acc, L, B, H, T, D, gamma);
    /* attention over layer 0: its B sequences' codes and scales are contiguous */
    const int64_t Hq = 2 * H;
    uint16_t *q = (uint16_t *)alloc((size_t)(B * Q * Hq * D) * 2);
    uint16_t *out = (uint16_t *)alloc((size_t)(B * Q * Hq * D) * 2);
    int32_t *pos = (int32_t *)alloc((size_t)B * sizeof(int32_t));
    fill_bf16(q, (size_t)(B * Q * Hq * D));
    for (int64_t b = 0; b < B; ++b) pos[b] = b == 0 ? -3 : b == 1 ? (int32_t)(T + 5) : (int32_t)(next_u32() % (uint32_t)T);
    orc_attention_fp8(q, codes, scales, pos, B, Q, Hq, H, T, D, 0.0883883f, out);
    free(pos);
    free(out);
    free(q);
    free(acc);
    free(start);
    free(stage);
    free(scales);
    free(codes);
}

static void fp8(int64_t M, int64_t K, int64_t N)
{
    for (int c = 0; c < 256; ++c) {
        double v = orc_e4m3_to_double((uint8_t)c);
        if (v == v) (void)orc_double_to_e4m3(v);
    }
    (void)orc_double_to_e4m3(1e9);
    (void)orc_double_to_e4m3(-1e-9);
    uint16_t *x = (uint16_t *)alloc((size_t)(M * K) * 2);
    fill_bf16(x, (size_t)(M * K));
    memset(x, 0, (size_t)K * 2);                     /* a zero row */
    uint8_t *ac = (uint8_t *)alloc((size_t)(M * K));
    float *as = (float *)alloc((size_t)M * sizeof(float));
    orc_quantize_act_fp8(x, M, K, ac, as);
    uint16_t *w = (uint16_t *)alloc((size_t)(N * K) * 2);
    fill_bf16(w, (size_t)(N * K));
    uint8_t *wc = (uint8_t *)alloc((size_t)(N * K));
    float *ws = (float *)alloc((size_t)N * sizeof(float));
    orc_quantize_weights_fp8(w, K, N, wc, ws);
    uint8_t *store = (uint8_t *)alloc((size_t)(N * K));
    fill_bytes(store, (size_t)(N * K));
    for (int64_t i = 0; i < N * K; ++i)
        if ((store[i] & 0x7F) == 0x7F) store[i] ^= 1;   /* no NaN codes */
    double *y = (double *)alloc((size_t)(M * N) * sizeof(double));
    orc_gemm_w8a8(ac, as, M, store, ws, K, N, y);
    free(y);
    free(store);
    free(ws);
    free(wc);
    free(w);
    free(as);
    free(ac);
    free(x);
}

int main(void)
{
    for (uint32_t h = 0; h < 65536; ++h) {
        (void)orc_fp16_to_double((uint16_t)h);
        (void)orc_bf16_to_double((uint16_t)h);
    }
    (void)orc_double_to_bf16(1e300);
    (void)orc_double_to_bf16(-1e-300);
    (void)orc_double_to_bf16(0.0);
    for (int w = 0; w < 16; ++w)
        for (int z = 0; z < 16; ++z) (void)orc_dequant_one(0x3C00, w, z);
    linear_layers(1, 128, 16);
    linear_layers(5, 384, 48);
    linear_layers(17, 256, 32);
    verification(1, 0, 7);
    verification(3, 4, 33);
    verification(2, 1, 1);
    controller(3, 50, 8);
    controller(1, 1, 0);
    attention(3, 2, 4, 2, 37);
    attention(2, 1, 1, 1, 1);
    kv(2, 5, 2, 9, 8, 3);
    kv(1, 4, 1, 1, 4, 0);
    fp8(3, 256, 32);
    kv_fp8(2, 4, 2, 9, 3, 2);
    kv_fp8(1, 3, 1, 1, 0, 1);
    printf("oracle sanitizer driver: done\n");
    return 0;
}
