// Per-token, per-group symmetric INT4 activation quantizer on gfx950.
// (QSPEC notes, background terms: W4A4 quantizes the activations to 4 bits as well.)
//   a = max |x| over the 128-wide group, s_a = a / 7 (binary32 division, nearest-even),
//   q = clamp(nearest_even(x / s_a), -8, 7) with a binary32 division per element, q = 0 if a = 0.
// One wave per (token, group): each lane loads one dword (two bfloat16, k = 2l and 2l+1), the
// absmax is a wave max, and each lane writes the byte holding its two codes (even k low).
#include "common.hpp"
#include "kernels.hpp"

namespace qspec {

__device__ __forceinline__ int quant_code(float v, float s) {
    float t = __builtin_rintf(v / s);           // correctly rounded division, ties-to-even rint
    t = fminf(fmaxf(t, -8.0f), 7.0f);
    return (int)t;
}

__global__ void __launch_bounds__(256)
k_quantize_act(const uint16_t *__restrict__ x, int M, int K, uint8_t *__restrict__ codes,
               float *__restrict__ scales) {
    const int G = K / kGroup;
    const int lane = threadIdx.x & 63;
    const long long grp = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (grp >= (long long)M * G) return;        // uniform per wave
    const long long m = grp / G;
    const int g = (int)(grp % G);
    const uint32_t pair = *(const uint32_t *)(x + (size_t)m * K + (size_t)g * kGroup + 2 * lane);
    const float x0 = bf16_bits_to_float(pair & 0xFFFFu);
    const float x1 = bf16_bits_to_float(pair >> 16);
    const float a = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    const float s = a / 7.0f;
    int q0 = 0, q1 = 0;
    if (a != 0.0f) {
        q0 = quant_code(x0, s);
        q1 = quant_code(x1, s);
    }
    codes[(size_t)m * (K / 2) + (size_t)g * 64 + lane] = (uint8_t)((q0 & 15) | ((q1 & 15) << 4));
    if (lane == 0) scales[(size_t)m * G + g] = s;
}

hipError_t launch_quantize_act(const uint16_t *x, int M, int K, uint8_t *codes, float *scales,
                               hipStream_t st) {
    const long long groups = (long long)M * (K / kGroup);
    const unsigned blocks = (unsigned)((groups + 3) / 4);
    hipLaunchKernelGGL(k_quantize_act, dim3(blocks), dim3(256), 0, st, x, M, K, codes, scales);
    return hipGetLastError();
}

}  // namespace qspec
