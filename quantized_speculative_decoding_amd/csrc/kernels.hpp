// Host-side launchers of the gfx950 kernels (internal to the library; the public
// interface is include/qspec.h).  Each returns the status of its last launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qspec {

hipError_t launch_quantize_act(const uint16_t *x, int M, int K, uint8_t *codes, float *scales,
                               hipStream_t st);

hipError_t launch_gemm_w4a16(const uint16_t *x, int M, const uint8_t *codes, const uint32_t *meta, int K,
                             int N, void *y, int y_f32, void *workspace, hipStream_t st);

size_t gemm_w4a16_workspace_bytes(int M, int K, int N);

// Batch tier of M for (K, N): its index, and the range of M sharing its reduction order.
int gemm_w4a16_tier(int M, int K, int N, int *m_first, int *m_last);
int gemm_w4a4_tier(int M, int K, int N, int *m_first, int *m_last);

hipError_t launch_gemm_w4a4(const uint8_t *a_codes, const float *a_scales, int M, const uint8_t *codes,
                            const uint32_t *meta, int K, int N, void *y, int y_f32, int32_t *group_dots,
                            hipStream_t st);

size_t verify_workspace_bytes(int mode, int B, int gamma, int V);

// The fixed device scratch of the verification entry point that allocates nothing: its size, and
// its address on the current device (looked up once per device).
constexpr size_t kVerifyScratchBytes = (size_t)1 << 20;
hipError_t verify_scratch(void **ptr);

hipError_t launch_verify_accept(int mode, const float *target, const float *draft,
                                const int32_t *draft_tokens, const float *u_accept,
                                const float *u_resample, int B, int gamma, int V,
                                int32_t *accept_count, int32_t *out_tokens, void *workspace,
                                hipStream_t st);

size_t draft_sample_workspace_bytes(int mode, int B, int V);

hipError_t launch_draft_sample(int mode, const float *logits, size_t ldt, const float *u, int B, int V,
                               int32_t *tokens, int ldo, void *workspace, hipStream_t st);

size_t speckv_workspace_bytes(int R, int V);

// The draft-side head and the adaptive-gamma controller on one draft step's rows (SAMPLE shares
// the softmax statistics pass between them).
size_t draft_speckv_workspace_bytes(int mode, int B, int V);
hipError_t launch_draft_speckv(int mode, const float *logits, size_t ldt, const float *u, int B, int V,
                               int32_t *tokens, int ldo, float quant_feature, const float *w1, const float *b1,
                               const float *w2, const float *b2, int max_gamma, double *features,
                               int32_t *gamma_out, void *ws, hipStream_t st);

hipError_t launch_speckv_gamma(const float *logits, int R, int V, float quant_feature, const float *w1,
                               const float *b1, const float *w2, const float *b2, int max_gamma,
                               double *features, int32_t *gamma_out, void *workspace, hipStream_t st);

// y (bf16 or fp32) = the sum of S <= 16 fp32 partials [S][M][N], added in split order.
void launch_splitk_reduce(const float *partials, int S, int M, int N, void *y, int y_f32, hipStream_t st);

hipError_t launch_quantize_act_fp8(const uint16_t *x, int M, int K, uint8_t *codes, float *scales, hipStream_t st);

size_t gemm_w8a8_workspace_bytes(int M, int K, int N);

hipError_t launch_gemm_w8a8(const uint8_t *a_codes, const float *a_scales, int M, const uint8_t *w_store,
                            const float *w_scales, int K, int N, void *y, int y_f32, void *workspace,
                            hipStream_t st);

size_t attention_workspace_bytes(int B, int Q, int Hq, int T);

hipError_t launch_attention(const uint16_t *q, const uint16_t *cache, const int32_t *pos, int B, int Q, int Hq,
                            int Hkv, int T, float scale, uint16_t *out, void *workspace, hipStream_t st);

hipError_t launch_kv_overwrite(uint16_t *cache, const uint16_t *verify_kv, const int32_t *start_pos,
                               const int32_t *accept_count, int L, int B, int H, int T, int D,
                               int gamma, hipStream_t st);

// The quantized (FP8 E4M3, one scale per row of 128) cache: committed rows quantized as written,
// and attention over it.
hipError_t launch_kv_overwrite_fp8(uint8_t *codes, float *scales, const uint16_t *verify_kv,
                                   const int32_t *start_pos, const int32_t *accept_count, int L, int B, int H,
                                   int T, int gamma, hipStream_t st);
hipError_t launch_attention_fp8(const uint16_t *q, const uint8_t *codes, const float *scales, const int32_t *pos,
                                int B, int Q, int Hq, int Hkv, int T, float scale, uint16_t *out, void *workspace,
                                hipStream_t st);


}  // namespace qspec
