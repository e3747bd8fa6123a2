/*
 * qspec.h -- C ABI of the shared-INT4 speculative-decoding hot path (gfx950).
 *
 * One set of 4-bit weight codes with a per-group scale s and zero point z is
 * read by two linear-layer kernels: a W4A4 draft layer (activations quantized to
 * 4 bits, exact integer group dot products, then rescaling) and a W4A16 verify
 * layer (W_hat = s (W - z) dequantized on the fly, bfloat16 activations).  They
 * are followed by the verification step and by the replacement of draft KV
 * with verify KV for the accepted positions.
 *
 * Source: the study-notes page "QSPEC 논문 요점 정리" on "QSPEC: Speculative
 * Decoding with Complementary Quantization Schemes" (Zhao, Lu, Wang, Kong, Wu).
 * Its sections are cited by content: "background terms" (weight-only vs
 * weight-activation quantization, INT32 accumulation then scaling, the
 * dequantization example), "speculative-decoding background" (acceptance rule,
 * greedy acceptance, first-reject cutoff, L = A + 1), "QSPEC structure" (draft
 * with W4A4, verify with W4A16 over gamma+1 positions, shared 4-bit weights,
 * KV replacement).
 *
 * Conventions for every call
 *   - Every pointer argument is DEVICE memory (hipMalloc'd or a torch CUDA
 *     tensor), allocated, owned and freed by the caller.  The library never
 *     allocates or frees memory and keeps no state between calls (workspaces
 *     are the caller's).
 *   - Calls are asynchronous: they validate their arguments on the host, enqueue
 *     kernels on `stream` (a hipStream_t; NULL = the legacy default stream) and
 *     return without synchronizing.  Results are visible after the caller
 *     synchronizes the stream or orders later work on it.
 *   - Argument errors (NULL pointers, non-positive or inconsistent sizes,
 *     unsupported shapes or dtypes, a too-small workspace) are detected before
 *     any launch and return a negative status with no side effects.
 *     QSPEC_ERR_HIP reports a launch failure.  Device-resident values (logits,
 *     token ids, positions, accept counts) are not inspected on the host;
 *     out-of-range values there never cause out-of-bounds accesses (see each
 *     call) but give unspecified results.
 *   - Outputs must not alias inputs.
 *   - Alignment: x / activation codes / weight codes 16 bytes (they are read with 16-byte
 *     loads; row starts stay aligned because K is a multiple of 128); the GEMM outputs y
 *     16 bytes (written with 16-byte stores; rows stay aligned because N is a multiple of 16);
 *     other fp32 / int32 / meta arrays 4 bytes; other bf16 arrays 2 bytes; the verify
 *     workspace 16 bytes and the W4A16 workspace 256 bytes.  Torch allocations satisfy all of
 *     these.  A violation returns QSPEC_ERR_ALIGN.
 *
 * Storage formats (the pages fix none of these; this library's choices)
 *   weight codes   u8  [N/16][K/128][1024]  the shared 4-bit store, tile-major.  Block (t, g)
 *                  holds columns n = 16t..16t+15 and k = 128g..128g+127 as
 *                  [quarter q = (k%128)/32][column c = n%16][16 bytes for k%32 = 0..31], two
 *                  unsigned codes (0..15) per byte, even k in the low nibble.  A wave reading a
 *                  block with lane l taking bytes 16l..16l+15 reads one contiguous kilobyte and
 *                  receives exactly its MFMA B fragments (lane l = column l%16, quarter l/16).
 *   weight meta    u32 [N/16][K/128][16]    per (column, group): binary16 scale s in bits
 *                  0..15, zero point z (0..15) in bits 16..23, bits 24..31 zero; entry (t, g, c)
 *                  belongs to column 16t + c.
 *   activations    u16 [M][K]       bfloat16 bit patterns, row-major
 *   act. codes     u8  [M][K/2]     4-bit two's complement, even k in the low nibble
 *   act. scales    f32 [M][K/128]
 *   K must be a positive multiple of QSPEC_GROUP (128); N a positive multiple of 16; M >= 1.
 *   Weight bytes per element: 0.5 (code) + 4/128 (meta) = 0.53125.
 */
#ifndef QSPEC_H
#define QSPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *qspec_stream_t; /* hipStream_t */

#define QSPEC_GROUP 128

enum qspec_status {
    QSPEC_OK = 0,
    QSPEC_ERR_NULL = -1,        /* a required pointer is NULL */
    QSPEC_ERR_SHAPE = -2,       /* a size is non-positive, too large or inconsistent */
    QSPEC_ERR_UNSUPPORTED = -3, /* unknown dtype or mode */
    QSPEC_ERR_HIP = -4,         /* a kernel launch failed */
    QSPEC_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than qspec_verify_workspace_bytes() */
    QSPEC_ERR_ALIGN = -6,       /* a pointer is not aligned as its call requires */
    QSPEC_ERR_TOO_LARGE = -7    /* the problem needs more than a fixed scratch buffer holds */
};

enum qspec_out_dtype { QSPEC_OUT_BF16 = 0, QSPEC_OUT_F32 = 1 };
enum qspec_verify_mode { QSPEC_GREEDY = 0, QSPEC_SAMPLE = 1 };

/* Largest gamma the adaptive-gamma controller may choose (its outputs are 0..max_gamma). */
#define QSPEC_SPECKV_MAX_GAMMA 63

/* qspec_attention: the head dimension it supports and the most query tokens per sequence. */
#define QSPEC_ATTN_HEAD_DIM 128
#define QSPEC_ATTN_MAX_QUERIES 64

/* Human-readable name of a status code (static string). */
const char *qspec_status_string(int status);

/*
 * qspec_quantize_act -- per-token, per-group symmetric INT4 activation codes.
 * [QSPEC notes, background terms: weight-activation (W4A4) quantization puts the
 * activations in 4 bits as well.]  The page fixes no quantizer; this one is, for
 * every row m and 128-wide group g:
 *     a = max |x|,  s_a = a / 7 (binary32 division, nearest-even),
 *     q = clamp(nearest_even(x / s_a), -8, 7)   (binary32 division), q = 0 when a = 0.
 * x        [in]  u16 [M][K] bfloat16 (finite values)
 * codes    [out] u8  [M][K/2]   (format above)
 * scales   [out] f32 [M][K/128] (s_a)
 * Errors: NULL pointer; M < 1; K < 128 or K % 128 != 0.
 */
int qspec_quantize_act(const uint16_t *x, int32_t M, int32_t K, uint8_t *codes, float *scales,
                       qspec_stream_t stream);

/*
 * qspec_gemm_w4a4 -- W4A4 draft linear layer over the shared 4-bit weights.
 * [QSPEC notes, background terms: the 4-bit MACs accumulate in INT32 and the
 * scale is applied afterwards; QSPEC structure: the draft runs W4A4 on the same
 * 4-bit weights as the verifier.]  With per-group scales:
 *     D[g][m][n] = sum_{k in g} q_a[m][k] * (w[k][n] - z[n][g])   (exact, int32)
 *     y[m][n]    = sum_g s_a[m][g] * s[n][g] * D[g][m][n]          (fp32 accumulation)
 * a_codes     [in]  u8  [M][K/2], a_scales [in] f32 [M][K/128]  (from qspec_quantize_act)
 * w_codes, w_meta [in] the shared weight store, formats above
 * y           [out] [M][N], bfloat16 (y_dtype = QSPEC_OUT_BF16, nearest-even) or f32
 * group_dots  [out, optional] i32 [K/128][M][N] -- the exact D; NULL to skip
 *             (diagnostic: slower).
 * Batch invariance: the reduction order of an output depends only on (K, N) and on the batch
 * tier of M -- [1, 16], [17, 64] or 65 and above (qspec_gemm_w4a4_tier reports it) -- so row m
 * of y is bit-identical for every M in the same tier.  D is exact, hence independent of M.
 * Errors: NULL pointer; M < 1; N < 1 or N % 16 != 0; K < 128 or K % 128 != 0; min(M, 64) * K / 2
 * or K * 8 of 2^32 or more (32-bit buffer ranges); bad y_dtype.
 */
int qspec_gemm_w4a4(const uint8_t *a_codes, const float *a_scales, int32_t M,
                    const uint8_t *w_codes, const uint32_t *w_meta, int32_t K, int32_t N, void *y,
                    int32_t y_dtype, int32_t *group_dots, qspec_stream_t stream);

/*
 * qspec_gemm_w4a4_tier -- the batch tier of M for (K, N): returns its index (0, 1 or 2) and sets
 * [*m_first, *m_last] to the batch sizes that share it (*m_last = INT32_MAX for the last tier).
 * Every M of one tier reduces each output of qspec_gemm_w4a4 in the same order; different tiers
 * may round differently.  The tiers are [1, 16], [17, 64] and [65, INT32_MAX] for every (K, N).
 * Host-only: launches nothing.
 * Errors (negative status): NULL pointer; the size errors of qspec_gemm_w4a4.
 */
int qspec_gemm_w4a4_tier(int32_t M, int32_t K, int32_t N, int32_t *m_first, int32_t *m_last);

/*
 * qspec_gemm_w4a16_tier -- the batch tier of M for (K, N) in qspec_gemm_w4a16, as
 * qspec_gemm_w4a4_tier reports it for the W4A4 layer.  The tiers are
 *   0: [1, D]       the decode kernel (one 16-row tile up to 16 rows, two above);
 *   1: [D + 1, V]   the verify kernel: two K parts (and K splits), ceil(M / 80) row blocks;
 *   2: [V + 1, INT32_MAX] the shared-activation kernel over 128-row blocks;
 * with D = 24 when N >= 65536 (vocabulary-sized heads: four column tiles per workgroup),
 * D = 32 when the decode grid has at most 256 workgroups and K * N <= 4096 * 6144 (small
 * projections), and otherwise: for N < 6144 (one-tile workgroups) D = 8 when K >= 8192 and 12
 * below; for 6144 <= N < 65536 (two-tile workgroups) D = 8 when K >= 12288, else D = 20 when
 * tier 1's workgroups W1 = ceil(N / 128) * S1 (S1: its K split count below) leave the last of
 * ceil(W1 / 256) generations of 256 under three quarters full (4 W1 < 3 * 256 * ceil(W1 / 256)),
 * and D = 12 otherwise.  The decode grid has N / 16 workgroups for N < 6144, ceil(N / 32) for
 * 6144 <= N < 65536.  With P = ceil(N / 256) * S2, the tier-2 workgroups per 128-row block (S2:
 * its K split count below), V = 384 for P <= 32, 256 for P <= 64, 160 for P <= 128 and 80
 * above.  Host-only: launches nothing.
 * Errors (negative status): NULL pointer; the size errors of qspec_gemm_w4a16.
 */
int qspec_gemm_w4a16_tier(int32_t M, int32_t K, int32_t N, int32_t *m_first, int32_t *m_last);

/*
 * qspec_gemm_w4a16_workspace_bytes -- device workspace qspec_gemm_w4a16 needs for (M, K, N); 0
 * when the shape needs none (M in tier 0 of qspec_gemm_w4a16_tier, or a shape whose K is not
 * split) or on invalid sizes.  K is split for tier-1 shapes with fewer than 192 blocks of 128
 * columns (S1 = max(1, min(256 / blocks, 16, K / 640)) splits, integer quotients) and for
 * tier-2 shapes with fewer than 64
 * blocks of 256 columns and at least 64 groups (S2, the largest power of two up to 8 with
 * S2 * blocks <= 128 and at least 32 groups per split); the split count depends on (K, N) and
 * the tier only, and the size is S * M * N * 4 bytes.
 */
size_t qspec_gemm_w4a16_workspace_bytes(int32_t M, int32_t K, int32_t N);

/*
 * qspec_gemm_w4a16 -- W4A16 verify linear layer over the shared 4-bit weights.
 * [QSPEC notes, background terms: dequantization example, Y = X W_hat with
 * W_hat = s (W_INT4 - z) in 16 bits; QSPEC structure: the verifier scores the
 * gamma+1 positions in one pass.]  W_hat[k][n] = bfloat16_nearest_even(s[n][g] *
 * (w[k][n] - z[n][g])) (the product is exact before that rounding);
 * y[m][n] = sum_k x[m][k] * W_hat[k][n] accumulated in fp32.
 * x   [in]  u16 [M][K] bfloat16
 * w_codes, w_meta [in] the shared weight store (the same arrays the W4A4 layer reads)
 * y   [out] [M][N], bfloat16 (nearest-even) or f32 per y_dtype
 * workspace [in/out] at least qspec_gemm_w4a16_workspace_bytes(M, K, N) bytes, 256-byte aligned
 *           (NULL allowed when that is 0).  It receives the fp32 partial sums of the K splits,
 *           [S][M][N], which a second kernel on the same stream adds in split order; its contents
 *           need no initialization.  Calls sharing a workspace must be ordered on one stream.
 * Batch invariance: the reduction order of an output depends only on (K, N) and on the
 * batch tier of M (qspec_gemm_w4a16_tier), so row m of y is bit-identical for every M in the
 * same tier; verifying gamma + 1 <= D positions of one sequence (D >= 8 for every shape, 24 or
 * 32 for some) therefore reproduces one-position decoding bit for bit.  Across tiers (say plain
 * decoding at M = B = 16 and verification at M = 5B = 80) rows agree to fp32 rounding, not bit
 * for bit.
 * Errors: NULL pointer; M < 1; N < 1 or N % 16 != 0; K < 128 or K % 128 != 0; min(M, 128) * K * 2
 * or K * 8 of 2^32 or more (32-bit buffer ranges); bad y_dtype; workspace missing or too small.
 */
int qspec_gemm_w4a16(const uint16_t *x, int32_t M, const uint8_t *w_codes, const uint32_t *w_meta,
                     int32_t K, int32_t N, void *y, int32_t y_dtype, void *workspace,
                     size_t workspace_bytes, qspec_stream_t stream);

/*
 * qspec_verify_workspace_bytes -- device workspace qspec_verify_accept needs
 * for (mode, B, gamma, V); 0 on invalid sizes.
 */
size_t qspec_verify_workspace_bytes(int32_t mode, int32_t B, int32_t gamma, int32_t V);

/*
 * qspec_verify_accept -- verification of gamma draft tokens per sequence.
 * [QSPEC notes, speculative-decoding background: greedy acceptance when the
 * target's most probable token equals the draft; otherwise acceptance with
 * probability min(1, p(x|h)/q(x|h)); the first rejection discards the rest; a
 * correction token follows a rejection and an extra target token follows full
 * acceptance, so L = A + 1 tokens are committed.  QSPEC structure: the verifier
 * outputs gamma+1 distributions p_{i+1..i+gamma+1}.]
 * GREEDY: t_j = argmax target[b][j] (ties -> lowest index); A = number of
 *   leading j with draft_tokens[b][j] == t_j; out = d_0..d_{A-1}, t_A.
 * SAMPLE: p_j = softmax(target[b][j]), q_j = softmax(draft[b][j]) (temperature 1);
 *   candidate j is accepted iff u_accept[b][j] < p_j(d_j) / q_j(d_j); A = index of
 *   the first rejection (gamma if none); the last token is drawn from the
 *   residual max(0, p_A - q_A) (or from p_A if that has no mass) when A < gamma,
 *   and from p_gamma when A == gamma, by inverse CDF at u_resample[b] times the
 *   total mass (first x whose running sum exceeds it).  Softmax normalizers,
 *   ratios and running sums are in fp64.
 * target_logits [in]  f32 [B][gamma+1][V]
 * draft_logits  [in]  f32 [B][gamma][V]  (SAMPLE only; may be NULL for GREEDY or gamma = 0)
 * draft_tokens  [in]  i32 [B][gamma]     (may be NULL when gamma = 0)
 * u_accept      [in]  f32 [B][gamma] in [0,1)  (SAMPLE only; may be NULL otherwise)
 * u_resample    [in]  f32 [B] in [0,1)         (SAMPLE only; may be NULL otherwise)
 * accept_count  [out] i32 [B]            A per sequence
 * out_tokens    [out] i32 [B][gamma+1]   committed tokens, -1 after position A
 * workspace     [in]  device scratch of at least qspec_verify_workspace_bytes(mode, B, gamma, V)
 *               bytes; contents on entry are ignored.
 * A draft token outside [0, V) counts as a mismatch / rejection.  Logits must be
 * finite.
 * Errors: NULL pointer; bad mode; B < 1; gamma < 0; V < 1; too many rows;
 * workspace too small.
 */
int qspec_verify_accept(int32_t mode, const float *target_logits, const float *draft_logits,
                        const int32_t *draft_tokens, const float *u_accept,
                        const float *u_resample, int32_t B, int32_t gamma, int32_t V,
                        int32_t *accept_count, int32_t *out_tokens, void *workspace,
                        size_t workspace_bytes, qspec_stream_t stream);

/*
 * qspec_verify_accept_noalloc -- qspec_verify_accept without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, arithmetic and results as
 * qspec_verify_accept; the chunk partials go to a fixed device scratch buffer of
 * QSPEC_VERIFY_SCRATCH_BYTES inside the library (one per GPU, held until the process ends; its
 * device address is looked up on the first call on each device).  The call allocates and frees
 * nothing.  The scratch needs no initialization and keeps the last call's contents.  Every call
 * on one GPU shares that GPU's buffer: calls that may overlap on one GPU (different streams, or
 * host threads without ordering) race and must not be issued.
 * Errors: those of qspec_verify_accept (no workspace errors); QSPEC_ERR_TOO_LARGE when
 * qspec_verify_workspace_bytes(mode, B, gamma, V) exceeds QSPEC_VERIFY_SCRATCH_BYTES (1 MiB:
 * e.g. B = 32, gamma = 4, V = 128256 in sampling mode needs about 90 KB); QSPEC_ERR_HIP when the
 * scratch address cannot be obtained or a launch fails.
 */
#define QSPEC_VERIFY_SCRATCH_BYTES (1u << 20)
int qspec_verify_accept_noalloc(int32_t mode, const float *target_logits, const float *draft_logits,
                                const int32_t *draft_tokens, const float *u_accept,
                                const float *u_resample, int32_t B, int32_t gamma, int32_t V,
                                int32_t *accept_count, int32_t *out_tokens, qspec_stream_t stream);

/*
 * qspec_draft_sample_workspace_bytes -- device workspace qspec_draft_sample needs; 0 on invalid
 * arguments.
 */
size_t qspec_draft_sample_workspace_bytes(int32_t mode, int32_t B, int32_t V);

/*
 * qspec_draft_sample -- the draft-side head of one draft step: one token per sequence from that
 * step's draft logits.
 * [QSPEC notes, QSPEC structure: the W4A4 draft proposes gamma tokens one step at a time; the
 * speculative-decoding background: a draft token x is drawn from the draft distribution q, which
 * verification later compares with p.]  GREEDY: tokens[b] = argmax logits[b] (lowest index on
 * ties).  SAMPLE: tokens[b] = the first x whose running sum of softmax(logits[b]) (temperature 1,
 * fp64) exceeds u[b] times the total mass -- exactly qspec_verify_accept's draw for gamma = 0.
 * The rows may be strided so that step j of a [B][gamma][V] draft-logit buffer (row_stride =
 * gamma * V) is read in place and its tokens land in column j of the [B][gamma] draft-token
 * buffer (token_stride = gamma) that qspec_verify_accept then reads.
 * logits     [in]  f32, row b at logits + b * row_stride, V values each (finite)
 * row_stride       elements between rows, >= V
 * u          [in]  f32 [B] uniforms in [0, 1) (SAMPLE; ignored and may be NULL for GREEDY)
 * tokens     [out] i32, token b at tokens + b * token_stride
 * workspace  [in/out] at least qspec_draft_sample_workspace_bytes(mode, B, V) bytes
 * Errors: bad mode; NULL pointer; B < 1; V < 1; row_stride < V; token_stride < 1; workspace missing
 * or too small.
 */
int qspec_draft_sample(int32_t mode, const float *logits, int32_t B, int32_t V, int64_t row_stride,
                       const float *u, int32_t *tokens, int32_t token_stride, void *workspace,
                       size_t workspace_bytes, qspec_stream_t stream);

/*
 * qspec_kv_overwrite -- replace draft KV with verify KV for committed positions.
 * [QSPEC notes, QSPEC structure: for accepted tokens the low-precision KV written
 * by the W4A4 draft is replaced with the KV computed by the W4A16 verifier.]
 * The verifier scores gamma+1 positions starting at start_pos[b] (the previous
 * round's last token, then the gamma drafts), so rows r = 0..A_b of verify_kv go
 * to positions start_pos[b] + r; nothing else in the cache changes.
 * cache        [in/out] u16 [L][B][2][H][T][D] bfloat16 (2 = key, value)
 * verify_kv    [in]     u16 [L][B][2][H][gamma+1][D]
 * start_pos    [in]     i32 [B]
 * accept_count [in]     i32 [B] (device; e.g. straight from qspec_verify_accept),
 *                       clamped to [0, gamma]; positions outside [0, T) are skipped.
 * Errors: NULL pointer; any size < 1 (gamma < 0); gamma + 1 > T; verify_kv of 2^32
 * elements or more (QSPEC_ERR_SHAPE).
 */
int qspec_kv_overwrite(uint16_t *cache, const uint16_t *verify_kv, const int32_t *start_pos,
                       const int32_t *accept_count, int32_t L, int32_t B, int32_t H, int32_t T,
                       int32_t D, int32_t gamma, qspec_stream_t stream);

/*
 * qspec_kv_overwrite_fp8 -- replace draft KV with verify KV in a quantized (FP8) cache.
 * [QSPEC notes: the opening summary speaks of quantized KV; QSPEC structure: for accepted tokens
 * the draft's low-precision KV is replaced with the verifier's.]  The page fixes no KV format;
 * this cache holds OCP FP8 E4M3 codes with one binary32 scale per (position, head) row of D = 128
 * values, the per-row quantizer of qspec_quantize_act_fp8: s = max |v| / 448 (binary32 division),
 * code = the nearest E4M3 value to v / s (ties to even, binary32 quotient, saturating), s = 0 and
 * codes 0 for an all-zero row; a value reads back as s * decoded code.  Rows r = 0..A_b of
 * verify_kv are quantized and written at positions start_pos[b] + r (as qspec_kv_overwrite:
 * A_b clamped to [0, gamma], positions outside [0, T) skipped); nothing else changes.
 * cache_codes  [in/out] u8  [L][B][2][H][T][D]
 * cache_scales [in/out] f32 [L][B][2][H][T]
 * verify_kv    [in]     u16 [L][B][2][H][gamma+1][D] bfloat16 (finite)
 * start_pos, accept_count [in] i32 [B] (device)
 * Errors: NULL pointer; any size < 1 (gamma < 0); gamma + 1 > T; D != QSPEC_ATTN_HEAD_DIM;
 * misaligned cache_codes (2 bytes), cache_scales / verify_kv / start_pos / accept_count (4).
 */
int qspec_kv_overwrite_fp8(uint8_t *cache_codes, float *cache_scales, const uint16_t *verify_kv,
                           const int32_t *start_pos, const int32_t *accept_count, int32_t L, int32_t B, int32_t H,
                           int32_t T, int32_t D, int32_t gamma, qspec_stream_t stream);

/*
 * qspec_attention_fp8 -- qspec_attention over one layer of the quantized (FP8) cache.
 * [QSPEC notes: quantized KV, read by the draft and the verifier alike.]  The arithmetic of
 * qspec_attention, with key and value t of a head read back as s_t * decoded code: the MFMAs take
 * the codes widened exactly to bfloat16, each score is multiplied by its key's scale and each
 * probability by its value's scale (the softmax normalizer keeps the unscaled probabilities).
 * Half the bytes of the bfloat16 cache are read.
 * q            [in]  u16 [B][Q][Hq][D] bfloat16
 * cache_codes  [in]  u8  [B][2][Hkv][T][D]: one layer of the [L][B][2][H][T][D] codes
 * cache_scales [in]  f32 [B][2][Hkv][T]:    the same layer's scales (finite)
 * pos, D, scale, out, workspace: as qspec_attention (workspace of
 *              qspec_attention_workspace_bytes bytes)
 * Errors: those of qspec_attention; cache_codes needs 16-byte and cache_scales 4-byte alignment.
 */
int qspec_attention_fp8(const uint16_t *q, const uint8_t *cache_codes, const float *cache_scales,
                        const int32_t *pos, int32_t B, int32_t Q, int32_t Hq, int32_t Hkv, int32_t T, int32_t D,
                        float scale, uint16_t *out, void *workspace, size_t workspace_bytes,
                        qspec_stream_t stream);

/*
 * qspec_speckv_workspace_bytes -- device workspace qspec_speckv_gamma needs for R rows of V
 * logits; 0 on invalid sizes.
 */
size_t qspec_speckv_workspace_bytes(int32_t R, int32_t V);

/*
 * qspec_speckv_gamma -- draft statistics and the adaptive-gamma controller.
 * [SpecKV notes, architecture and mechanism: how sure the draft is (its largest
 * softmax probability) and how spread its distribution is (its entropy), with
 * the compression level, feed a small MLP that picks gamma for the next step;
 * implementation guide: the controller is Linear(3 -> 64), ReLU,
 * Linear(64 -> max_gamma + 1), and gamma is the index of the largest output;
 * the entropy adds 1e-9 inside the logarithm.]  Per row r, in fp64:
 *     p = softmax(draft_logits[r])                          (temperature 1)
 *     confidence = max p,  entropy = -sum_x p(x) log(p(x) + 1e-9)
 *     h = relu(w1 [confidence, entropy, quant_feature] + b1)       (64 units)
 *     gamma_out[r] = argmax_j (w2 h + b2)_j   (lowest index among equal outputs)
 * Every dot product is summed in input order after its bias.
 * draft_logits  [in]  f32 [R][V] (finite values)
 * quant_feature [in]  the controller's third input, shared by all rows (the page feeds one column
 *                     of the compression-level one-hot)
 * w1 [in] f32 [64][3], b1 [in] f32 [64], w2 [in] f32 [max_gamma + 1][64], b2 [in] f32
 *                     [max_gamma + 1]: device copies of the controller's weights
 * max_gamma     [in]  0 .. QSPEC_SPECKV_MAX_GAMMA
 * features      [out] f64 [R][2] = (confidence, entropy), or NULL
 * gamma_out     [out] i32 [R]
 * workspace     [in/out] at least qspec_speckv_workspace_bytes(R, V) bytes (chunk partials; no
 *                     initialization needed)
 * Errors: NULL pointer (features may be NULL); R < 1; V < 1; max_gamma outside
 * [0, QSPEC_SPECKV_MAX_GAMMA]; workspace missing or too small.
 */
int qspec_speckv_gamma(const float *draft_logits, int32_t R, int32_t V, float quant_feature,
                       const float *w1, const float *b1, const float *w2, const float *b2,
                       int32_t max_gamma, double *features, int32_t *gamma_out, void *workspace,
                       size_t workspace_bytes, qspec_stream_t stream);

/*
 * qspec_draft_sample_speckv_workspace_bytes -- device workspace qspec_draft_sample_speckv needs;
 * 0 on invalid arguments.
 */
size_t qspec_draft_sample_speckv_workspace_bytes(int32_t mode, int32_t B, int32_t V);

/*
 * qspec_draft_sample_speckv -- the draft-side head and the adaptive-gamma controller of one draft
 * step, on the same draft rows.
 * [QSPEC notes, QSPEC structure: the draft proposes one token per step from its distribution;
 * SpecKV notes, architecture and mechanism: the draft's statistics at that step (its largest
 * probability and its entropy) pick gamma.]  tokens are exactly qspec_draft_sample's, and
 * gamma_out / features exactly qspec_speckv_gamma's on the rows (R = B): the same kernels.  With
 * SAMPLE the head's softmax statistics (per-chunk max and sum of exponentials) are the
 * controller's too, so one statistics pass over the rows serves both; GREEDY takes argmaxes and
 * runs the controller's statistics pass after them.
 * Arguments as qspec_draft_sample (mode, logits, B, V, row_stride, u, tokens, token_stride) and
 * qspec_speckv_gamma (quant_feature, w1, b1, w2, b2, max_gamma, features, gamma_out).
 * workspace  [in/out] at least qspec_draft_sample_speckv_workspace_bytes(mode, B, V) bytes
 * Errors: those of both calls.
 */
int qspec_draft_sample_speckv(int32_t mode, const float *logits, int32_t B, int32_t V, int64_t row_stride,
                              const float *u, int32_t *tokens, int32_t token_stride, float quant_feature,
                              const float *w1, const float *b1, const float *w2, const float *b2,
                              int32_t max_gamma, double *features, int32_t *gamma_out, void *workspace,
                              size_t workspace_bytes, qspec_stream_t stream);

/*
 * qspec_attention_workspace_bytes -- device workspace qspec_attention needs; 0 on invalid sizes
 * (the head dimension is QSPEC_ATTN_HEAD_DIM).
 */
size_t qspec_attention_workspace_bytes(int32_t B, int32_t Q, int32_t Hq, int32_t Hkv, int32_t T);

/*
 * qspec_attention -- one layer's attention over the shared KV cache.
 * [QSPEC notes, QSPEC structure: the W4A4 draft and the W4A16 verifier read and write one KV
 * cache, and the verifier's KV replaces the draft's for accepted tokens (qspec_kv_overwrite).]
 * The pages fix no attention arithmetic; this call is causal scaled dot-product attention with
 * grouped KV heads.  Query token j of sequence b sits at position pos[b] + j (a draft step has
 * Q = 1, a verify pass Q = gamma + 1) and attends to cached positions t = 0 .. min(pos[b] + j,
 * T - 1); query head h reads KV head h / (Hq / Hkv):
 *     out[b][j][h] = sum_t softmax_t(scale * q[b][j][h] . key[b][h'][t]) value[b][h'][t]
 * Scores, exponentials and sums are fp32; the output is rounded once to bfloat16.  The cache
 * entries of the query positions themselves are expected to be written before the call.
 * q          [in]  u16 [B][Q][Hq][D] bfloat16
 * cache      [in]  u16 [B][2][Hkv][T][D] bfloat16 (2 = key, value): one layer of the
 *                  [L][B][2][H][T][D] cache qspec_kv_overwrite updates, i.e. its base plus
 *                  layer * B * 2 * H * T * D elements
 * pos        [in]  i32 [B] (device); negative entries read as 0
 * D          QSPEC_ATTN_HEAD_DIM
 * scale      the score scale, typically 1 / sqrt(D)
 * out        [out] u16 [B][Q][Hq][D] bfloat16
 * workspace  [in/out] at least qspec_attention_workspace_bytes(B, Q, Hq, Hkv, T) bytes (chunk
 *            partials; no initialization needed)
 * Alignment: q, cache and workspace 16 bytes.
 * Errors: NULL pointer; B, Q, Hq, Hkv or T < 1; D other than QSPEC_ATTN_HEAD_DIM; Q above
 * QSPEC_ATTN_MAX_QUERIES; Hq not a multiple of Hkv; B * Hkv above 65535; workspace missing or
 * too small.
 */
int qspec_attention(const uint16_t *q, const uint16_t *cache, const int32_t *pos, int32_t B, int32_t Q,
                    int32_t Hq, int32_t Hkv, int32_t T, int32_t D, float scale, uint16_t *out,
                    void *workspace, size_t workspace_bytes, qspec_stream_t stream);

/*
 * The FP8 parent variant.
 * [SpecQuant notes, one-line summary, key contributions and approach: INT4, FP8 and FP16
 * variants of one model are made by post-training quantization with shared base weights; a
 * low-precision draft proposes and a parent variant verifies.  The recipe is not given.]
 * FP8 here is OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 fraction bits, no infinities,
 * 0x7F / 0xFF NaN, largest finite 448).  Codes are the nearest finite E4M3 value to the scaled
 * input (ties to the even code, saturating at +-448; the sign bit is the input's).
 *   FP8 weight store  u8 [N/16][K/128][2048]: block (t, g) holds columns 16t..16t+15 and
 *                     k = 128g..128g+127; byte h * 1024 + l * 16 + b, with lane l = c + 16 q, is
 *                     column 16t + c at k = 128g + 32q + 16h + b.  A wave reading a block half
 *                     with lane l taking 16 bytes at 16 l reads one contiguous kilobyte.
 *   weight scales     f32 [N], one per output column (absmax over K / 448 for a post-training
 *                     quantized FP16 weight; any positive values are accepted)
 *   FP8 act. codes    u8 [M][K] row-major;  act. scales f32 [M]
 * K must be a positive multiple of 128, N of 16; M * K and K * N must stay below 2^32.
 */

/*
 * qspec_quantize_act_fp8 -- per-token FP8 activation codes.
 * a = max_k |x[m][k]|, scales[m] = a / 448 (one binary32 division), codes[m][k] =
 * E4M3(x[m][k] / scales[m]) with the quotient a binary32 division; a row with a == 0 gets
 * scale 0 and all codes 0.
 * x [in] u16 [M][K] bfloat16 (finite values); codes [out] u8 [M][K]; scales [out] f32 [M]
 * Alignment: x and codes 16 bytes.
 * Errors: NULL pointer; M < 1; K < 128 or K % 128 != 0.
 */
int qspec_quantize_act_fp8(const uint16_t *x, int32_t M, int32_t K, uint8_t *codes, float *scales,
                           qspec_stream_t stream);

/*
 * qspec_gemm_w8a8_workspace_bytes -- device workspace qspec_gemm_w8a8 needs for (M, K, N); 0 when
 * K is not split or on invalid sizes.  The split count depends on (K, N) only; the size is
 * S * M * N * 4 bytes.
 */
size_t qspec_gemm_w8a8_workspace_bytes(int32_t M, int32_t K, int32_t N);

/*
 * qspec_gemm_w8a8 -- the FP8 parent's linear layer.
 * y[m][n] = a_scales[m] * w_scales[n] * sum_k E4M3(a_codes[m][k]) * E4M3(w[k][n]): every product
 * is exact, the sum is fp32 (FP8 MFMA), the scales are applied to the fp32 sum of each K split
 * and the splits are added in split order.
 * a_codes, a_scales [in] from qspec_quantize_act_fp8
 * w_store, w_scales [in] the FP8 weight store and its column scales
 * y   [out] [M][N], bfloat16 (nearest-even) or f32 per y_dtype
 * workspace [in/out] at least qspec_gemm_w8a8_workspace_bytes(M, K, N) bytes, 256-byte aligned
 *           (NULL allowed when that is 0); contents need no initialization; calls sharing a
 *           workspace must be ordered on one stream.
 * Batch invariance: the reduction order of an output depends only on (K, N), so row m of y is
 * bit-identical for every M.
 * Errors: NULL pointer; M < 1; N < 16 or N % 16 != 0; K < 128 or K % 128 != 0; M * K or K * N
 * of 2^32 or more; bad y_dtype; workspace missing or too small.
 */
int qspec_gemm_w8a8(const uint8_t *a_codes, const float *a_scales, int32_t M, const uint8_t *w_store,
                    const float *w_scales, int32_t K, int32_t N, void *y, int32_t y_dtype, void *workspace,
                    size_t workspace_bytes, qspec_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QSPEC_H */
