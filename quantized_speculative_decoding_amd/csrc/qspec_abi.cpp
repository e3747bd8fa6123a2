// The C ABI (include/qspec.h): host-side argument validation, then kernel launches on the
// caller's stream.  No allocation, no synchronization, no state.
#include "qspec.h"

#include <hip/hip_runtime.h>

#include "kernels.hpp"

#define QSPEC_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

inline int status_of(hipError_t e) { return e == hipSuccess ? QSPEC_OK : QSPEC_ERR_HIP; }

inline bool bad_k(int32_t K) { return K < QSPEC_GROUP || K % QSPEC_GROUP != 0; }

inline bool bad_n(int32_t N) { return N < 16 || N % 16 != 0; }

inline hipStream_t as_stream(qspec_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Largest M * N (or row count) whose flat indices stay far inside the int64 range and whose
// grids fit the launch limits; sizes are int32 on the interface.
constexpr long long kMaxElems = 1LL << 40;

// The shared-INT4 kernels address the activation rows one workgroup reads (at most 128 rows for
// W4A16, 64 codes rows for W4A4; all M rows below those) and one column tile's weight blocks
// (K / 128 kilobytes) through 32-bit buffer ranges and offsets.
inline bool w4a16_range_ok(int32_t M, int32_t K) {
    const long long rows = M < 128 ? M : 128;
    return rows * K * 2 < (1LL << 32) && (long long)K * 8 < (1LL << 32);
}
inline bool w4a4_range_ok(int32_t M, int32_t K) {
    const long long rows = M < 64 ? M : 64;
    return rows * (K / 2) < (1LL << 32) && (long long)K * 8 < (1LL << 32);
}

}  // namespace

QSPEC_EXPORT const char *qspec_status_string(int status) {
    switch (status) {
    case QSPEC_OK: return "ok";
    case QSPEC_ERR_NULL: return "null pointer argument";
    case QSPEC_ERR_SHAPE: return "invalid or inconsistent size";
    case QSPEC_ERR_UNSUPPORTED: return "unsupported dtype or mode";
    case QSPEC_ERR_HIP: return "HIP launch failure";
    case QSPEC_ERR_WORKSPACE: return "workspace missing or too small";
    case QSPEC_ERR_ALIGN: return "misaligned pointer";
    case QSPEC_ERR_TOO_LARGE: return "problem needs more scratch than the fixed buffer holds";
    default: return "unknown status";
    }
}

QSPEC_EXPORT int qspec_quantize_act(const uint16_t *x, int32_t M, int32_t K, uint8_t *codes,
                                    float *scales, qspec_stream_t stream) {
    if (!x || !codes || !scales) return QSPEC_ERR_NULL;
    if (M < 1 || bad_k(K)) return QSPEC_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(scales, 4)) return QSPEC_ERR_ALIGN;
    return status_of(qspec::launch_quantize_act(x, M, K, codes, scales, as_stream(stream)));
}

QSPEC_EXPORT int qspec_gemm_w4a4(const uint8_t *a_codes, const float *a_scales, int32_t M,
                                 const uint8_t *w_codes, const uint32_t *w_meta, int32_t K, int32_t N,
                                 void *y, int32_t y_dtype, int32_t *group_dots, qspec_stream_t stream) {
    if (!a_codes || !a_scales || !w_codes || !w_meta || !y) return QSPEC_ERR_NULL;
    if (M < 1 || bad_n(N) || bad_k(K)) return QSPEC_ERR_SHAPE;
    if ((long long)M * N > kMaxElems || !w4a4_range_ok(M, K)) return QSPEC_ERR_SHAPE;
    if (y_dtype != QSPEC_OUT_BF16 && y_dtype != QSPEC_OUT_F32) return QSPEC_ERR_UNSUPPORTED;
    if (!aligned(a_codes, 16) || !aligned(w_codes, 16) || !aligned(a_scales, 4) || !aligned(w_meta, 4) ||
        !aligned(y, 16) || !aligned(group_dots, 4))
        return QSPEC_ERR_ALIGN;
    return status_of(qspec::launch_gemm_w4a4(a_codes, a_scales, M, w_codes, w_meta, K, N, y,
                                             y_dtype == QSPEC_OUT_F32, group_dots, as_stream(stream)));
}

static bool w4a16_sizes_ok(int32_t M, int32_t K, int32_t N) {
    return M >= 1 && !bad_n(N) && !bad_k(K) && (long long)M * N <= kMaxElems && w4a16_range_ok(M, K);
}

QSPEC_EXPORT size_t qspec_gemm_w4a16_workspace_bytes(int32_t M, int32_t K, int32_t N) {
    if (!w4a16_sizes_ok(M, K, N)) return 0;
    return qspec::gemm_w4a16_workspace_bytes(M, K, N);
}

QSPEC_EXPORT int qspec_gemm_w4a16_tier(int32_t M, int32_t K, int32_t N, int32_t *m_first, int32_t *m_last) {
    if (!m_first || !m_last) return QSPEC_ERR_NULL;
    if (!w4a16_sizes_ok(M, K, N)) return QSPEC_ERR_SHAPE;
    int lo = 0, hi = 0;
    const int tier = qspec::gemm_w4a16_tier(M, K, N, &lo, &hi);
    *m_first = lo;
    *m_last = hi;
    return tier;
}

QSPEC_EXPORT int qspec_gemm_w4a4_tier(int32_t M, int32_t K, int32_t N, int32_t *m_first, int32_t *m_last) {
    if (!m_first || !m_last) return QSPEC_ERR_NULL;
    if (M < 1 || bad_n(N) || bad_k(K) || (long long)M * N > kMaxElems || !w4a4_range_ok(M, K))
        return QSPEC_ERR_SHAPE;
    int lo = 0, hi = 0;
    const int tier = qspec::gemm_w4a4_tier(M, K, N, &lo, &hi);
    *m_first = lo;
    *m_last = hi;
    return tier;
}

QSPEC_EXPORT int qspec_gemm_w4a16(const uint16_t *x, int32_t M, const uint8_t *w_codes,
                                  const uint32_t *w_meta, int32_t K, int32_t N, void *y, int32_t y_dtype,
                                  void *workspace, size_t workspace_bytes, qspec_stream_t stream) {
    if (!x || !w_codes || !w_meta || !y) return QSPEC_ERR_NULL;
    if (!w4a16_sizes_ok(M, K, N)) return QSPEC_ERR_SHAPE;
    if (y_dtype != QSPEC_OUT_BF16 && y_dtype != QSPEC_OUT_F32) return QSPEC_ERR_UNSUPPORTED;
    const size_t need = qspec::gemm_w4a16_workspace_bytes(M, K, N);
    if (need > 0 && (!workspace || workspace_bytes < need)) return QSPEC_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(w_codes, 16) || !aligned(w_meta, 4) ||
        !aligned(y, 16) || !aligned(workspace, 256))
        return QSPEC_ERR_ALIGN;
    return status_of(qspec::launch_gemm_w4a16(x, M, w_codes, w_meta, K, N, y, y_dtype == QSPEC_OUT_F32,
                                              workspace, as_stream(stream)));
}

static bool verify_sizes_ok(int32_t B, int32_t gamma, int32_t V) {
    if (B < 1 || gamma < 0 || V < 1) return false;
    // row-chunk grids are 1-D with at most 2^31 - 1 workgroups
    const long long rows = (long long)B * (2LL * gamma + 1);
    const long long chunks = (V + 8191) / 8192;
    return rows * chunks < (1LL << 31) && (long long)B * (gamma + 1) * V <= kMaxElems;
}

QSPEC_EXPORT size_t qspec_verify_workspace_bytes(int32_t mode, int32_t B, int32_t gamma, int32_t V) {
    if ((mode != QSPEC_GREEDY && mode != QSPEC_SAMPLE) || !verify_sizes_ok(B, gamma, V)) return 0;
    return qspec::verify_workspace_bytes(mode, B, gamma, V);
}

QSPEC_EXPORT int qspec_verify_accept(int32_t mode, const float *target_logits,
                                     const float *draft_logits, const int32_t *draft_tokens,
                                     const float *u_accept, const float *u_resample, int32_t B,
                                     int32_t gamma, int32_t V, int32_t *accept_count,
                                     int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                                     qspec_stream_t stream) {
    if (mode != QSPEC_GREEDY && mode != QSPEC_SAMPLE) return QSPEC_ERR_UNSUPPORTED;
    if (!target_logits || !accept_count || !out_tokens) return QSPEC_ERR_NULL;
    if (gamma > 0 && !draft_tokens) return QSPEC_ERR_NULL;
    if (mode == QSPEC_SAMPLE && (!u_resample || (gamma > 0 && (!draft_logits || !u_accept))))
        return QSPEC_ERR_NULL;
    if (!verify_sizes_ok(B, gamma, V)) return QSPEC_ERR_SHAPE;
    if (!workspace || workspace_bytes < qspec::verify_workspace_bytes(mode, B, gamma, V))
        return QSPEC_ERR_WORKSPACE;
    if (!aligned(target_logits, 4) || !aligned(draft_logits, 4) || !aligned(draft_tokens, 4) ||
        !aligned(u_accept, 4) || !aligned(u_resample, 4) || !aligned(accept_count, 4) ||
        !aligned(out_tokens, 4) || !aligned(workspace, 16))
        return QSPEC_ERR_ALIGN;
    return status_of(qspec::launch_verify_accept(mode, target_logits, draft_logits, draft_tokens,
                                                 u_accept, u_resample, B, gamma, V, accept_count,
                                                 out_tokens, workspace, as_stream(stream)));
}

QSPEC_EXPORT int qspec_verify_accept_noalloc(int32_t mode, const float *target_logits,
                                             const float *draft_logits, const int32_t *draft_tokens,
                                             const float *u_accept, const float *u_resample, int32_t B,
                                             int32_t gamma, int32_t V, int32_t *accept_count,
                                             int32_t *out_tokens, qspec_stream_t stream) {
    if (mode != QSPEC_GREEDY && mode != QSPEC_SAMPLE) return QSPEC_ERR_UNSUPPORTED;
    if (!target_logits || !accept_count || !out_tokens) return QSPEC_ERR_NULL;
    if (gamma > 0 && !draft_tokens) return QSPEC_ERR_NULL;
    if (mode == QSPEC_SAMPLE && (!u_resample || (gamma > 0 && (!draft_logits || !u_accept))))
        return QSPEC_ERR_NULL;
    if (!verify_sizes_ok(B, gamma, V)) return QSPEC_ERR_SHAPE;
    if (qspec::verify_workspace_bytes(mode, B, gamma, V) > QSPEC_VERIFY_SCRATCH_BYTES) return QSPEC_ERR_TOO_LARGE;
    if (!aligned(target_logits, 4) || !aligned(draft_logits, 4) || !aligned(draft_tokens, 4) ||
        !aligned(u_accept, 4) || !aligned(u_resample, 4) || !aligned(accept_count, 4) || !aligned(out_tokens, 4))
        return QSPEC_ERR_ALIGN;
    void *ws = nullptr;
    if (qspec::verify_scratch(&ws) != hipSuccess) return QSPEC_ERR_HIP;
    return status_of(qspec::launch_verify_accept(mode, target_logits, draft_logits, draft_tokens, u_accept,
                                                 u_resample, B, gamma, V, accept_count, out_tokens, ws,
                                                 as_stream(stream)));
}

static_assert(qspec::kVerifyScratchBytes == QSPEC_VERIFY_SCRATCH_BYTES, "scratch size");

static bool speckv_sizes_ok(int32_t R, int32_t V, int32_t max_gamma) {
    if (R < 1 || V < 1 || max_gamma < 0 || max_gamma > QSPEC_SPECKV_MAX_GAMMA) return false;
    return (long long)R * ((V + 8191) / 8192) < (1LL << 31) && (long long)R * V <= kMaxElems;
}

QSPEC_EXPORT size_t qspec_speckv_workspace_bytes(int32_t R, int32_t V) {
    if (!speckv_sizes_ok(R, V, 0)) return 0;
    return qspec::speckv_workspace_bytes(R, V);
}

QSPEC_EXPORT int qspec_speckv_gamma(const float *draft_logits, int32_t R, int32_t V, float quant_feature,
                                    const float *w1, const float *b1, const float *w2, const float *b2,
                                    int32_t max_gamma, double *features, int32_t *gamma_out, void *workspace,
                                    size_t workspace_bytes, qspec_stream_t stream) {
    if (!draft_logits || !w1 || !b1 || !w2 || !b2 || !gamma_out) return QSPEC_ERR_NULL;
    if (!speckv_sizes_ok(R, V, max_gamma)) return QSPEC_ERR_SHAPE;
    if (!workspace || workspace_bytes < qspec::speckv_workspace_bytes(R, V)) return QSPEC_ERR_WORKSPACE;
    if (!aligned(draft_logits, 4) || !aligned(w1, 4) || !aligned(b1, 4) || !aligned(w2, 4) || !aligned(b2, 4) ||
        !aligned(features, 8) || !aligned(gamma_out, 4) || !aligned(workspace, 16))
        return QSPEC_ERR_ALIGN;
    return status_of(qspec::launch_speckv_gamma(draft_logits, R, V, quant_feature, w1, b1, w2, b2, max_gamma,
                                                features, gamma_out, workspace, as_stream(stream)));
}

QSPEC_EXPORT int qspec_kv_overwrite(uint16_t *cache, const uint16_t *verify_kv,
                                    const int32_t *start_pos, const int32_t *accept_count,
                                    int32_t L, int32_t B, int32_t H, int32_t T, int32_t D,
                                    int32_t gamma, qspec_stream_t stream) {
    if (!cache || !verify_kv || !start_pos || !accept_count) return QSPEC_ERR_NULL;
    if (L < 1 || B < 1 || H < 1 || T < 1 || D < 1 || gamma < 0 || gamma + 1 > T)
        return QSPEC_ERR_SHAPE;
    if ((long long)L * B * 2 * H * (gamma + 1) * D >= (1LL << 32)) return QSPEC_ERR_SHAPE;   // 32-bit indices
    if (!aligned(cache, 2) || !aligned(verify_kv, 2) || !aligned(start_pos, 4) || !aligned(accept_count, 4))
        return QSPEC_ERR_ALIGN;
    return status_of(qspec::launch_kv_overwrite(cache, verify_kv, start_pos, accept_count, L, B, H, T,
                                                D, gamma, as_stream(stream)));
}

static bool attention_sizes_ok(int32_t B, int32_t Q, int32_t Hq, int32_t Hkv, int32_t T, int32_t D) {
    if (B < 1 || Q < 1 || Hq < 1 || Hkv < 1 || T < 1 || D != QSPEC_ATTN_HEAD_DIM) return false;
    if (Q > QSPEC_ATTN_MAX_QUERIES || Hq % Hkv != 0) return false;
    if ((long long)B * Hkv > 65535 || (long long)B * Q * Hq >= (1LL << 31)) return false;
    return (long long)B * 2 * Hkv * T * D <= kMaxElems && (long long)B * Q * Hq * T <= kMaxElems;
}

QSPEC_EXPORT size_t qspec_attention_workspace_bytes(int32_t B, int32_t Q, int32_t Hq, int32_t Hkv, int32_t T) {
    if (!attention_sizes_ok(B, Q, Hq, Hkv, T, QSPEC_ATTN_HEAD_DIM)) return 0;
    return qspec::attention_workspace_bytes(B, Q, Hq, T);
}

QSPEC_EXPORT int qspec_attention(const uint16_t *q, const uint16_t *cache, const int32_t *pos, int32_t B, int32_t Q,
                                 int32_t Hq, int32_t Hkv, int32_t T, int32_t D, float scale, uint16_t *out,
                                 void *workspace, size_t workspace_bytes, qspec_stream_t stream) {
    if (!q || !cache || !pos || !out) return QSPEC_ERR_NULL;
    if (!attention_sizes_ok(B, Q, Hq, Hkv, T, D)) return QSPEC_ERR_SHAPE;
    if (!workspace || workspace_bytes < qspec::attention_workspace_bytes(B, Q, Hq, T)) return QSPEC_ERR_WORKSPACE;
    if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(pos, 4) || !aligned(out, 2) || !aligned(workspace, 16))
        return QSPEC_ERR_ALIGN;
    return status_of(qspec::launch_attention(q, cache, pos, B, Q, Hq, Hkv, T, scale, out, workspace,
                                             as_stream(stream)));
}

QSPEC_EXPORT int qspec_kv_overwrite_fp8(uint8_t *cache_codes, float *cache_scales, const uint16_t *verify_kv,
                                        const int32_t *start_pos, const int32_t *accept_count, int32_t L, int32_t B,
                                        int32_t H, int32_t T, int32_t D, int32_t gamma, qspec_stream_t stream) {
    if (!cache_codes || !cache_scales || !verify_kv || !start_pos || !accept_count) return QSPEC_ERR_NULL;
    if (L < 1 || B < 1 || H < 1 || T < 1 || gamma < 0 || gamma + 1 > T || D != QSPEC_ATTN_HEAD_DIM)
        return QSPEC_ERR_SHAPE;
    if ((long long)L * B * 2 * H * T * D > kMaxElems || (long long)L * B * 2 * H * (gamma + 1) >= (1LL << 31) * 4)
        return QSPEC_ERR_SHAPE;
    if (!aligned(cache_codes, 2) || !aligned(cache_scales, 4) || !aligned(verify_kv, 4) || !aligned(start_pos, 4) ||
        !aligned(accept_count, 4))
        return QSPEC_ERR_ALIGN;
    return status_of(qspec::launch_kv_overwrite_fp8(cache_codes, cache_scales, verify_kv, start_pos, accept_count, L,
                                                    B, H, T, gamma, as_stream(stream)));
}

QSPEC_EXPORT int qspec_attention_fp8(const uint16_t *q, const uint8_t *cache_codes, const float *cache_scales,
                                     const int32_t *pos, int32_t B, int32_t Q, int32_t Hq, int32_t Hkv, int32_t T,
                                     int32_t D, float scale, uint16_t *out, void *workspace, size_t workspace_bytes,
                                     qspec_stream_t stream) {
    if (!q || !cache_codes || !cache_scales || !pos || !out) return QSPEC_ERR_NULL;
    if (!attention_sizes_ok(B, Q, Hq, Hkv, T, D)) return QSPEC_ERR_SHAPE;
    if (!workspace || workspace_bytes < qspec::attention_workspace_bytes(B, Q, Hq, T)) return QSPEC_ERR_WORKSPACE;
    if (!aligned(q, 16) || !aligned(cache_codes, 16) || !aligned(cache_scales, 4) || !aligned(pos, 4) ||
        !aligned(out, 2) || !aligned(workspace, 16))
        return QSPEC_ERR_ALIGN;
    return status_of(qspec::launch_attention_fp8(q, cache_codes, cache_scales, pos, B, Q, Hq, Hkv, T, scale, out,
                                                 workspace, as_stream(stream)));
}

// The W8A8 kernels address a_codes (M * K bytes) and the FP8 store (K * N bytes) through 32-bit
// buffer offsets.
static bool w8a8_sizes_ok(int32_t M, int32_t K, int32_t N) {
    if (M < 1 || bad_n(N) || bad_k(K) || (long long)M * N > kMaxElems) return false;
    return (long long)M * K < (1LL << 32) && (long long)K * N < (1LL << 32) && M < (1 << 30);
}

QSPEC_EXPORT int qspec_quantize_act_fp8(const uint16_t *x, int32_t M, int32_t K, uint8_t *codes, float *scales,
                                        qspec_stream_t stream) {
    if (!x || !codes || !scales) return QSPEC_ERR_NULL;
    if (M < 1 || bad_k(K)) return QSPEC_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return QSPEC_ERR_ALIGN;
    return status_of(qspec::launch_quantize_act_fp8(x, M, K, codes, scales, as_stream(stream)));
}

QSPEC_EXPORT size_t qspec_gemm_w8a8_workspace_bytes(int32_t M, int32_t K, int32_t N) {
    if (!w8a8_sizes_ok(M, K, N)) return 0;
    return qspec::gemm_w8a8_workspace_bytes(M, K, N);
}

QSPEC_EXPORT int qspec_gemm_w8a8(const uint8_t *a_codes, const float *a_scales, int32_t M, const uint8_t *w_store,
                                 const float *w_scales, int32_t K, int32_t N, void *y, int32_t y_dtype,
                                 void *workspace, size_t workspace_bytes, qspec_stream_t stream) {
    if (!a_codes || !a_scales || !w_store || !w_scales || !y) return QSPEC_ERR_NULL;
    if (!w8a8_sizes_ok(M, K, N)) return QSPEC_ERR_SHAPE;
    if (y_dtype != QSPEC_OUT_BF16 && y_dtype != QSPEC_OUT_F32) return QSPEC_ERR_UNSUPPORTED;
    const size_t need = qspec::gemm_w8a8_workspace_bytes(M, K, N);
    if (need > 0 && (!workspace || workspace_bytes < need)) return QSPEC_ERR_WORKSPACE;
    if (!aligned(a_codes, 16) || !aligned(w_store, 16) || !aligned(a_scales, 4) || !aligned(w_scales, 4) ||
        !aligned(y, 16) || !aligned(workspace, 256))
        return QSPEC_ERR_ALIGN;
    return status_of(qspec::launch_gemm_w8a8(a_codes, a_scales, M, w_store, w_scales, K, N, y,
                                             y_dtype == QSPEC_OUT_F32, workspace, as_stream(stream)));
}

QSPEC_EXPORT size_t qspec_draft_sample_workspace_bytes(int32_t mode, int32_t B, int32_t V) {
    if ((mode != QSPEC_GREEDY && mode != QSPEC_SAMPLE) || !verify_sizes_ok(B, 0, V)) return 0;
    return qspec::draft_sample_workspace_bytes(mode, B, V);
}

QSPEC_EXPORT int qspec_draft_sample(int32_t mode, const float *logits, int32_t B, int32_t V, int64_t row_stride,
                                    const float *u, int32_t *tokens, int32_t token_stride, void *workspace,
                                    size_t workspace_bytes, qspec_stream_t stream) {
    if (mode != QSPEC_GREEDY && mode != QSPEC_SAMPLE) return QSPEC_ERR_UNSUPPORTED;
    if (!logits || !tokens || (mode == QSPEC_SAMPLE && !u)) return QSPEC_ERR_NULL;
    if (!verify_sizes_ok(B, 0, V) || row_stride < V || token_stride < 1) return QSPEC_ERR_SHAPE;
    if ((long long)(B - 1) * row_stride + V > kMaxElems) return QSPEC_ERR_SHAPE;
    if (!workspace || workspace_bytes < qspec::draft_sample_workspace_bytes(mode, B, V)) return QSPEC_ERR_WORKSPACE;
    if (!aligned(logits, 4) || !aligned(u, 4) || !aligned(tokens, 4) || !aligned(workspace, 16))
        return QSPEC_ERR_ALIGN;
    return status_of(qspec::launch_draft_sample(mode, logits, (size_t)row_stride, u, B, V, tokens, token_stride,
                                                workspace, as_stream(stream)));
}

QSPEC_EXPORT size_t qspec_draft_sample_speckv_workspace_bytes(int32_t mode, int32_t B, int32_t V) {
    if ((mode != QSPEC_GREEDY && mode != QSPEC_SAMPLE) || !verify_sizes_ok(B, 0, V) || !speckv_sizes_ok(B, V, 0))
        return 0;
    return qspec::draft_speckv_workspace_bytes(mode, B, V);
}

QSPEC_EXPORT int qspec_draft_sample_speckv(int32_t mode, const float *logits, int32_t B, int32_t V,
                                           int64_t row_stride, const float *u, int32_t *tokens, int32_t token_stride,
                                           float quant_feature, const float *w1, const float *b1, const float *w2,
                                           const float *b2, int32_t max_gamma, double *features, int32_t *gamma_out,
                                           void *workspace, size_t workspace_bytes, qspec_stream_t stream) {
    if (mode != QSPEC_GREEDY && mode != QSPEC_SAMPLE) return QSPEC_ERR_UNSUPPORTED;
    if (!logits || !tokens || (mode == QSPEC_SAMPLE && !u)) return QSPEC_ERR_NULL;
    if (!w1 || !b1 || !w2 || !b2 || !gamma_out) return QSPEC_ERR_NULL;
    if (!verify_sizes_ok(B, 0, V) || !speckv_sizes_ok(B, V, max_gamma) || row_stride < V || token_stride < 1)
        return QSPEC_ERR_SHAPE;
    if ((long long)(B - 1) * row_stride + V > kMaxElems) return QSPEC_ERR_SHAPE;
    if (!workspace || workspace_bytes < qspec::draft_speckv_workspace_bytes(mode, B, V)) return QSPEC_ERR_WORKSPACE;
    if (!aligned(logits, 4) || !aligned(u, 4) || !aligned(tokens, 4) || !aligned(w1, 4) || !aligned(b1, 4) ||
        !aligned(w2, 4) || !aligned(b2, 4) || !aligned(features, 8) || !aligned(gamma_out, 4) ||
        !aligned(workspace, 16))
        return QSPEC_ERR_ALIGN;
    return status_of(qspec::launch_draft_speckv(mode, logits, (size_t)row_stride, u, B, V, tokens, token_stride,
                                                quant_feature, w1, b1, w2, b2, max_gamma, features, gamma_out,
                                                workspace, as_stream(stream)));
}
