/*
 * tern.h -- C ABI of libtern.so, the ternary-weight matmul for AMD MI355X (gfx950).
 *
 * The operation (2kiu.com/news/5082861, "putting a ternary embedding model
 * into vLLM"):
 *   - weights W[N,K] take values in {-1, 0, +1}; each is a 2-bit code
 *     00 -> 0, 01 -> +1, 10 -> -1, 11 -> reserved, read as 0            (§3.1)
 *   - four codes per byte, little-endian: weight 4j+i of a row sits in
 *     bits 2i..2i+1 of byte j of that row; packed[N, K/4] uint8         (§2.2, §3.1)
 *   - every `group` = 128 consecutive weights of a row along K share one
 *     fp16 scale; scales[N, K/128]                                      (§1.1, §3.1)
 *   - Y[M,N] = X[M,K] . (T (*) S)^T, X fp16 or bf16, fp32 accumulation  (§4.2)
 *   - callers flatten activations to a contiguous 2-D [tokens, K]      (§4.4)
 *
 * Conventions shared by every entry point:
 *   - Every pointer is a DEVICE pointer the caller allocated and owns.  The
 *     library allocates no device memory, uses no scratch buffer and never
 *     frees or retains a caller buffer.  Its only state across calls is a
 *     per-process record, per device and kernel instantiation, that the
 *     kernel's dynamic-LDS limit has been raised (hipFuncSetAttribute, done
 *     once on first use); no call's result depends on an earlier call.
 *   - Every tensor is dense, row-major and contiguous.  Pointers to X, W, T
 *     and packed bytes must be 16-byte aligned (TERN_ERR_ALIGN otherwise);
 *     scales need 2-byte and Y its element alignment.
 *   - Calls are asynchronous on `stream` (NULL = the device's default
 *     stream) and never synchronize the host.
 *   - Arguments are validated before anything is launched.  A non-OK status
 *     means nothing was launched and no output byte was written, except
 *     TERN_ERR_HIP, which reports a failed launch.
 *   - Sizes of zero are valid: nothing is launched (tern_matmul with K = 0
 *     and M, N > 0 writes Y = 0, the empty sum).  A pointer may be NULL only
 *     when the buffer it stands for has zero elements.
 *   - The library never exits the process and never throws across the ABI.
 */
#ifndef TERN_H
#define TERN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TERN_OK = 0,
    TERN_ERR_NULL = 1,        /* a required pointer is NULL */
    TERN_ERR_SHAPE = 2,       /* negative size, K % 4 != 0, or a size beyond the limits below */
    TERN_ERR_GROUP = 3,       /* K is not a multiple of `group`, or group <= 0 */
    TERN_ERR_DTYPE = 4,       /* x or y dtype outside the supported set */
    TERN_ERR_ALIGN = 5,       /* a pointer lacks the alignment stated above */
    TERN_ERR_UNSUPPORTED = 6, /* a valid request this build does not implement (group != 128, forced path that cannot run) */
    TERN_ERR_HIP = 7          /* the HIP runtime reported an error at launch */
} tern_status;

typedef enum { TERN_F16 = 0, TERN_BF16 = 1, TERN_F32 = 2 } tern_dtype;

/* Which kernel family computes tern_matmul_path's result. */
typedef enum {
    TERN_PATH_AUTO = 0, /* choose by shape (what tern_matmul does): for M <= 4, GEMV_FP4 with
                           bf16 X (K <= 32768), else with fp16 X GEMV_MFMA for M = 3, 4 where
                           it fits and GEMV for M <= 2 or where GEMV_MFMA does not fit;
                           GEMV_B16 for 5 <= M <= 16 with N >= 16384 and K <= 8192;
                           MFMA for every other shape */
    TERN_PATH_GEMV = 1, /* VALU sign-select decode kernel; M <= TERN_GEMV_MAX_M */
    TERN_PATH_MFMA = 2, /* LDS-staged activations + in-register weight decode + MFMA; any M */
    TERN_PATH_GEMV_MFMA = 3, /* decode kernel whose sign-select sums run on the matrix cores
                                (v_mfma_f32_4x4x4_16b on +-2 / 0 operands); M <= 4, with
                                the activations X[M,K] staged whole in LDS */
    TERN_PATH_GEMV_FP4 = 4, /* decode kernel with the weights as 4-bit (e2m1 +-2 / 0) matrix-core
                               operands and each bf16 activation split exactly into two e4m3
                               terms with a power-of-two scale per 32 (v_mfma_scale_f32_
                               16x16x128_f8f6f4); bf16 X only, M <= 4, K <= 32768 */
    TERN_PATH_GEMV_B16 = 5  /* decode kernel for batches of up to 16 rows: +-2 / 0 weight
                               operands of v_mfma_f32_16x16x32 against activation fragments
                               held in registers, waves splitting K; M <= 16, K <= 2^20 */
} tern_path;

#define TERN_GROUP 128
#define TERN_GEMV_MAX_M 4
/* Size limits: M, N <= 2^31 - 1 and K <= 2^30; M*N, M*K and N*K <= 2^62. */

/* Human-readable name of a status code (a static string; never NULL). */
const char *tern_status_string(tern_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
int tern_version(void);

/*
 * tern_pack -- T[N,K] int8 -> packed[N,K/4] uint8.
 * Source: 2kiu.com/news/5082861 §3.1 (code map, four codes per byte, first
 * weight in the lowest two bits).  T holds -1, 0 or +1; any other value is
 * written as the reserved code 11, which every reader decodes as 0.
 * Requires K % 4 == 0 (TERN_ERR_SHAPE).  T and packed: 16-byte aligned.
 */
tern_status tern_pack(const int8_t *T, uint8_t *packed, int64_t N, int64_t K, hipStream_t stream);

/*
 * tern_unpack -- packed[N,K/4] uint8 -> T[N,K] int8 in {-1, 0, +1}.
 * Source: 2kiu.com/news/5082861 §3.1 (the unpack function that recovers the
 * integer matrix from the packed bytes).  Code 11 is written as 0.
 * Requires K % 4 == 0.  Both pointers 16-byte aligned.
 */
tern_status tern_unpack(const uint8_t *packed, int8_t *T, int64_t N, int64_t K, hipStream_t stream);

/*
 * tern_matmul -- Y[M,N] = X[M,K] . (T (*) S)^T with fp32 accumulation.
 * Source: 2kiu.com/news/5082861 §4.2 (the kernel contract x[M,K], w[N,K/4],
 * scale[N,K/128], out[M,N]) with §3.1 for the weight encoding.
 *   X        [M,K]      x_dtype TERN_F16 or TERN_BF16
 *   packed_W [N,K/4]    uint8, the encoding of tern_pack
 *   scales   [N,K/128]  fp16 bit patterns (little-endian), one per 128
 *                       consecutive weights of a row
 *   Y        [M,N]      y_dtype TERN_F32, TERN_BF16 or TERN_F16; overwritten
 *                       (never accumulated into); fp32 results are rounded
 *                       to nearest-even into bf16/fp16, overflow gives inf
 *   group    must be 128 (TERN_ERR_UNSUPPORTED otherwise) and divide K
 * Result accuracy: |Y - exact| <= 2e-3 * sum_k |X[m,k] * S[n,k/128]| + one
 * ulp of y_dtype, for finite inputs (every finite fp16 scale).
 */
tern_status tern_matmul(const void *X, tern_dtype x_dtype, const uint8_t *packed_W,
                        const uint16_t *scales, void *Y, tern_dtype y_dtype, int64_t M, int64_t N,
                        int64_t K, int32_t group, hipStream_t stream);

/*
 * tern_matmul_path -- tern_matmul with an explicit kernel choice.  Same
 * arguments, layouts and result contract as tern_matmul; `path` picks the
 * kernel family (for tests that compare the two, and for benchmarks).
 * TERN_PATH_GEMV, TERN_PATH_GEMV_MFMA or TERN_PATH_GEMV_FP4 with M >
 * TERN_GEMV_MAX_M, or with an activation block too large for on-chip staging,
 * TERN_PATH_GEMV_FP4 with fp16 activations, and TERN_PATH_GEMV_B16 with M > 16
 * or K > 2^20, return TERN_ERR_UNSUPPORTED.
 */
tern_status tern_matmul_path(const void *X, tern_dtype x_dtype, const uint8_t *packed_W,
                             const uint16_t *scales, void *Y, tern_dtype y_dtype, int64_t M,
                             int64_t N, int64_t K, int32_t group, tern_path path,
                             hipStream_t stream);

/*
 * tern_dequant -- W[N,K] = t * s, the dense 16-bit weight matrix.
 * Source: 2kiu.com/news/5082861 §4.1 (the first route: dequantise, then a
 * library GEMM; the pages measure their kernel against it in §4.3).  This
 * is the comparison route's first half, not part of tern_matmul.
 *   packed [N,K/4] uint8, scales [N,K/group] fp16 bits, W [N,K] in w_dtype
 *   (TERN_F16: exact; TERN_BF16: s rounded to bf16, nearest even).
 *   group must be 128 and divide K.  packed and W 16-byte aligned.
 */
tern_status tern_dequant(const uint8_t *packed, const uint16_t *scales, void *W, tern_dtype w_dtype,
                         int64_t N, int64_t K, int32_t group, hipStream_t stream);

/*
 * tern_block_map -- which 128-weight blocks hold a nonzero weight.
 * Source: 2kiu.com/news/5082861 §6 (next steps: skip blocks that are
 * entirely zero).  block_map[n, w] (uint32, row-major [N, ceil(K/4096)]) has
 * bit b set when block 32w + b of row n contains a code 01 or 10; blocks of
 * codes 00 and 11 only are clear, and so are the unused high bits of a row's
 * last word.  packed 16-byte aligned, block_map 4-byte aligned; group must
 * be 128.  Computed once per weight matrix, not per product.
 */
tern_status tern_block_map(const uint8_t *packed, uint32_t *block_map, int64_t N, int64_t K, int32_t group,
                           hipStream_t stream);

/*
 * tern_matmul_blockmap -- tern_matmul that skips the unmarked blocks.
 * Source: 2kiu.com/news/5082861 §6 (zero-block skipping), §4.2 otherwise.
 * Same arguments, layouts, result contract and errors as tern_matmul, plus
 * block_map in the layout of tern_block_map (4-byte aligned; NULL only when
 * M, N or K is 0).  Blocks whose bit is clear are not read (no code bytes,
 * no scale) and not computed, so the map must mark every block with a
 * nonzero weight; marking more blocks is harmless.  The skipping kernel is
 * the decode path for M <= 2 (where the GEMV is the faster kernel); other
 * calls are tern_matmul (the map is not read).
 */
tern_status tern_matmul_blockmap(const void *X, tern_dtype x_dtype, const uint8_t *packed_W,
                                 const uint16_t *scales, const uint32_t *block_map, void *Y, tern_dtype y_dtype,
                                 int64_t M, int64_t N, int64_t K, int32_t group, hipStream_t stream);

/*
 * tern_quantize_scales -- int8 scale codes for tern_matmul_s8.
 * Source: 2kiu.com/news/5082861 §6 (next steps: compress the fp16 block
 * scale further to INT8).  The pages do not fix the scheme; this library's
 * reading is a symmetric code per output row with one fp32 factor:
 *   row_factor[n]  = max_g |S[n,g]| / 127            (fp32 division)
 *   scales_q[n,g]  = round-to-nearest-even(S[n,g] / row_factor[n]),
 *                    clamped to [-127, 127]; 0 for a row whose scales are 0
 * so the effective scale is scales_q[n,g] * row_factor[n] (relative error
 * up to 1/254 of the row's largest scale).  Both divisions are IEEE fp32.
 *   scales [N,K/group] fp16 bits (2-byte aligned), scales_q [N,K/group]
 *   int8, row_factor [N] fp32 (4-byte aligned).  group must be 128.
 */
tern_status tern_quantize_scales(const uint16_t *scales, int8_t *scales_q, float *row_factor, int64_t N,
                                 int64_t K, int32_t group, hipStream_t stream);

/*
 * tern_matmul_s8 -- tern_matmul_path with int8 block scales:
 *   Y[m,n] = sum_g (scales_q[n,g] * row_factor[n]) * sum_{k in g} t[n,k] X[m,k]
 * Source: 2kiu.com/news/5082861 §6 (INT8 scales, halving the scale traffic:
 * 1 byte per 128 weights instead of 2), with §4.2 for everything else.
 * Arguments, layouts, paths and errors as tern_matmul_path, with the fp16
 * scales replaced by scales_q [N,K/128] int8 and row_factor [N] fp32
 * (4-byte aligned; NULL only when M, N or K is 0).  Each path runs the
 * kernels of tern_matmul_path, reading the int8 codes in place of the fp16
 * scales.  Accuracy: the tern_matmul bound with
 * S[n,g] = scales_q[n,g] * row_factor[n].
 */
tern_status tern_matmul_s8(const void *X, tern_dtype x_dtype, const uint8_t *packed_W, const int8_t *scales_q,
                           const float *row_factor, void *Y, tern_dtype y_dtype, int64_t M, int64_t N,
                           int64_t K, int32_t group, tern_path path, hipStream_t stream);

/*
 * tern_stream_copy -- calibration, not part of the method: stream `bytes`
 * bytes of src with 16-byte loads (one instruction reads 1 KB of
 * consecutive bytes, every load of a thread issued before any is used) and,
 * when dst is not NULL, write them to dst.  With dst NULL it only reads.
 * It gives the plain-read (and copy) ceiling the decode kernels are timed
 * against, and a kernel of known traffic for scaling the HBM byte counters.
 * bytes % 16 == 0 and bytes <= 2^40 (TERN_ERR_SHAPE); src and dst 16-byte
 * aligned (TERN_ERR_ALIGN); src NULL with bytes > 0 is TERN_ERR_NULL;
 * bytes == 0 launches nothing.  Asynchronous on `stream`.
 */
tern_status tern_stream_copy(const void *src, void *dst, uint64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TERN_H */
