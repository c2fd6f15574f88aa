// tern_kernels.h -- host-side launchers of the HIP kernels behind tern.h.
// Every launcher assumes its arguments were validated by tern_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tern {

struct GemmArgs {
    const void *X;       // [M,K] fp16/bf16
    int x_dtype;         // 0 = fp16, 1 = bf16
    const uint8_t *W;    // [N,K/4]
    const uint16_t *S;   // [N,K/128] fp16 bits (when Q is null)
    const int8_t *Q;     // int8 scale codes [N,K/128], or null
    const float *R;      // per-row factor [N] of the int8 codes (scale = Q * R)
    void *Y;             // [M,N]
    int y_dtype;         // 0 = fp16, 1 = bf16, 2 = fp32
    int64_t M, N, K;
    hipStream_t stream;
};

// Decode-path GEMV, 1 <= M <= 4.
hipError_t launch_gemv(const GemmArgs &a);
// LDS bytes the GEMV needs for this M, K (it stages X[M,K] on chip).
size_t gemv_lds_bytes(int64_t M, int64_t K);
// True when launch_gemv takes its short-step kernel (M <= 4, N <= 5120, and
// K <= 5120 at M = 1 or K <= 8192 at M = 2 .. 4; also M = 2, K <= 8192,
// N >= 12288).
bool gemv_short(int64_t M, int64_t N, int64_t K);

// Decode-path kernel with matrix-core sign selects, 1 <= M <= 4: weights
// decoded to +-2 / 0 operands of v_mfma_f32_4x4x4_16b.  fits() is false when
// the activations of the call do not fit the workgroup's LDS.
bool gemv_mfma_fits(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv_mfma(const GemmArgs &a);

// Decode-path kernel with 4-bit weight operands on the matrix cores (bf16
// activations split exactly into two e4m3 terms), 1 <= M <= 4.
bool gemv_fp4_fits(int64_t M, int64_t N, int64_t K, int x_dtype);
hipError_t launch_gemv_fp4(const GemmArgs &a);

// Decode-path kernel for batches of 1 <= M <= 16 rows: +-2 / 0 weight operands
// of v_mfma_f32_16x16x32 against activation fragments held in registers.
bool gemv_b16_fits(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv_b16(const GemmArgs &a);

// Decode-path GEMV that skips the blocks MAP does not mark (1 <= M <= 2).
hipError_t launch_gemv_skip(const GemmArgs &a, const uint32_t *map);
size_t gemv_skip_lds_bytes(int64_t M, int64_t K);

// MAP[n, w] bit b = block 32w + b of row n holds a nonzero weight.
hipError_t launch_block_map(const uint8_t *P, uint32_t *map, int64_t N, int64_t K, hipStream_t stream);

// Batched path: MFMA GEMM, any M >= 1.
hipError_t launch_gemm(const GemmArgs &a);
// Batched path for many rows with fp16 X (fp16 scales, or int8 codes with
// row factors): 256 x 256, 192 x 256 or 128 x 64 tiles, weights decoded once
// per workgroup into LDS.
hipError_t launch_gemm_big(const GemmArgs &a);

// Int8 scale codes: Q[n,g] = rint(S[n,g] / R[n]), R[n] = max_g |S[n,g]| / 127.
hipError_t launch_quantize_scales(const uint16_t *S, int8_t *Q, float *R, int64_t N, int64_t groups,
                                  hipStream_t stream);

// W[N,K] = t * s in fp16 (w_dtype 0) or bf16 (1).
hipError_t launch_dequant(const uint8_t *P, const uint16_t *S, void *W, int w_dtype, int64_t N, int64_t K,
                          hipStream_t stream);

// Y = 0 (K == 0).
hipError_t launch_fill_zero(void *Y, int64_t bytes, hipStream_t stream);

// Pack / unpack over n_bytes packed bytes (= N*K/4).
hipError_t launch_pack(const int8_t *T, uint8_t *P, int64_t n_bytes, hipStream_t stream);
hipError_t launch_unpack(const uint8_t *P, int8_t *T, int64_t n_bytes, hipStream_t stream);

}  // namespace tern
