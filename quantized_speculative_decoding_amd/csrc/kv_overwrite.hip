// Replacement of draft KV by verify KV for the committed positions, on gfx950.
// (QSPEC notes, QSPEC structure: for accepted tokens the W4A4 draft's KV is replaced with the
//  W4A16 verifier's KV.)  Rows r = 0..A_b of the verifier's gamma+1 rows land at positions
// start_pos[b] + r; nothing else is written.  One thread per 16-byte vector of a candidate row,
// with 32-bit index arithmetic (the staging rows hold fewer than 2^32 elements, checked at the
// boundary); the accept count is read on the device, so no host round trip separates this from
// the verification.
#include "common.hpp"
#include "kernels.hpp"

namespace qspec {

template <typename VecT>
__global__ void __launch_bounds__(256)
k_kv_overwrite(uint16_t *__restrict__ cache, const uint16_t *__restrict__ vkv,
               const int32_t *__restrict__ start_pos, const int32_t *__restrict__ accept,
               int B, int H, int T, int D, int gamma, long long total) {
    constexpr int EPV = sizeof(VecT) / sizeof(uint16_t);   // elements per vector
    const unsigned idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (unsigned)total) return;
    const unsigned DV = D / EPV;
    const unsigned v = idx % DV;
    const unsigned rest = idx / DV;
    const int r = (int)(rest % (unsigned)(gamma + 1));
    const unsigned head = rest / (unsigned)(gamma + 1);   // ((l * B + b) * 2 + kv) * H + h
    const int b = (int)((head / (2u * H)) % (unsigned)B);
    int A = accept[b];
    A = A < 0 ? 0 : (A > gamma ? gamma : A);
    if (r > A) return;
    const long long t = (long long)start_pos[b] + r;
    if (t < 0 || t >= T) return;
    VecT *dst = (VecT *)(cache + ((size_t)head * T + (size_t)t) * D) + v;
    const VecT *src = (const VecT *)(vkv + ((size_t)head * (gamma + 1) + r) * D) + v;
    *dst = *src;
}

hipError_t launch_kv_overwrite(uint16_t *cache, const uint16_t *verify_kv, const int32_t *start_pos,
                               const int32_t *accept_count, int L, int B, int H, int T, int D,
                               int gamma, hipStream_t st) {
    const long long heads = (long long)L * B * 2 * H;
    const bool vec = (D % 8 == 0) && (((uintptr_t)cache | (uintptr_t)verify_kv) % 16 == 0);
    const int epv = vec ? 8 : 1;
    const long long total = heads * (gamma + 1) * (D / epv);
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (vec)
        hipLaunchKernelGGL(k_kv_overwrite<uint4>, dim3(blocks), dim3(256), 0, st, cache, verify_kv,
                           start_pos, accept_count, B, H, T, D, gamma, total);
    else
        hipLaunchKernelGGL(k_kv_overwrite<uint16_t>, dim3(blocks), dim3(256), 0, st, cache, verify_kv,
                           start_pos, accept_count, B, H, T, D, gamma, total);
    return hipGetLastError();
}

// The quantized cache (FP8 E4M3 codes [L][B][2][H][T][128] with one binary32 scale per
// (position, head) row, [L][B][2][H][T]): a committed row is quantized as it is written, with the
// per-row quantizer of the FP8 variant (s = max |v| / 448, code = E4M3(v / s), nearest even,
// binary32 division; an all-zero row gets s = 0 and zero codes).  One wave per candidate row
// (head, r): lane l holds elements 2 l and 2 l + 1; the row's absmax is a wave max.  Rows past
// the accept count or outside [0, T) are skipped by the whole wave.
constexpr int kKvD = 128;

__global__ void __launch_bounds__(256)
k_kv_overwrite_fp8(uint8_t *__restrict__ codes, float *__restrict__ scales, const uint16_t *__restrict__ vkv,
                   const int32_t *__restrict__ start_pos, const int32_t *__restrict__ accept, int B, int H, int T,
                   int gamma, long long rows) {
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;                                   // uniform per wave
    const int lane = threadIdx.x & 63;
    const int r = (int)(row % (gamma + 1));
    const long long head = row / (gamma + 1);                  // ((l * B + b) * 2 + kv) * H + h
    const int b = (int)((head / (2LL * H)) % B);
    int A = accept[b];
    A = A < 0 ? 0 : (A > gamma ? gamma : A);
    if (r > A) return;
    const long long t = (long long)start_pos[b] + r;
    if (t < 0 || t >= T) return;
    const uint32_t pair = *(const uint32_t *)(vkv + (size_t)row * kKvD + 2 * lane);
    const float x0 = bf16_bits_to_float(pair & 0xFFFFu), x1 = bf16_bits_to_float(pair >> 16);
    const float a = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    const float s = a / 448.0f;
    uint32_t c = 0;
    if (a != 0.0f) c = f32_to_e4m3(x0 / s) | (f32_to_e4m3(x1 / s) << 8);
    *(uint16_t *)(codes + ((size_t)head * T + (size_t)t) * kKvD + 2 * lane) = (uint16_t)c;
    if (lane == 0) scales[(size_t)head * T + (size_t)t] = s;
}

hipError_t launch_kv_overwrite_fp8(uint8_t *codes, float *scales, const uint16_t *verify_kv,
                                   const int32_t *start_pos, const int32_t *accept_count, int L, int B, int H,
                                   int T, int gamma, hipStream_t st) {
    const long long rows = (long long)L * B * 2 * H * (gamma + 1);
    const unsigned blocks = (unsigned)((rows + 3) / 4);
    hipLaunchKernelGGL(k_kv_overwrite_fp8, dim3(blocks), dim3(256), 0, st, codes, scales, verify_kv, start_pos,
                       accept_count, B, H, T, gamma, rows);
    return hipGetLastError();
}

}  // namespace qspec

