// tern_api.hip -- the C ABI declared in include/tern.h: argument validation
// and kernel dispatch.  Validation never touches the GPU, so a rejected call
// launches nothing and writes nothing.
#include <hip/hip_runtime.h>

#include "../../include/tern.h"
#include "tern_kernels.h"

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxK = int64_t(1) << 30;
constexpr int64_t kMaxProduct = int64_t(1) << 62;
constexpr size_t kGemvLdsLimit = 152 * 1024;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool product_ok(int64_t a, int64_t b) { return a == 0 || b <= kMaxProduct / a; }

tern_status check_pack_args(const void *T, const void *P, int64_t N, int64_t K) {
    if (N < 0 || K < 0 || N > kMaxDim || K > kMaxK || K % 4 != 0) return TERN_ERR_SHAPE;
    if (!product_ok(N, K)) return TERN_ERR_SHAPE;
    if (N == 0 || K == 0) return TERN_OK;
    if (T == nullptr || P == nullptr) return TERN_ERR_NULL;
    if (!aligned(T, 16) || !aligned(P, 16)) return TERN_ERR_ALIGN;
    return TERN_OK;
}

size_t dtype_size(tern_dtype d) { return d == TERN_F32 ? 4 : 2; }

// S is the scale array (fp16 values, or int8 codes with s_align 1)
tern_status check_matmul_args(const void *X, tern_dtype x_dtype, const uint8_t *W, const void *S,
                              uintptr_t s_align, void *Y, tern_dtype y_dtype, int64_t M, int64_t N, int64_t K,
                              int32_t group) {
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxK) return TERN_ERR_SHAPE;
    if (!product_ok(M, N) || !product_ok(M, K) || !product_ok(N, K)) return TERN_ERR_SHAPE;
    if (K % 4 != 0) return TERN_ERR_SHAPE;
    if (group <= 0 || K % group != 0) return TERN_ERR_GROUP;
    if (x_dtype != TERN_F16 && x_dtype != TERN_BF16) return TERN_ERR_DTYPE;
    if (y_dtype != TERN_F16 && y_dtype != TERN_BF16 && y_dtype != TERN_F32) return TERN_ERR_DTYPE;
    if (group != TERN_GROUP) return TERN_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return TERN_OK;
    if (Y == nullptr) return TERN_ERR_NULL;
    if (!aligned(Y, dtype_size(y_dtype))) return TERN_ERR_ALIGN;
    if (K == 0) return TERN_OK;
    if (X == nullptr || W == nullptr || S == nullptr) return TERN_ERR_NULL;
    if (!aligned(X, 16) || !aligned(W, 16) || !aligned(S, s_align)) return TERN_ERR_ALIGN;
    return TERN_OK;
}

tern_status from_hip(hipError_t e) { return e == hipSuccess ? TERN_OK : TERN_ERR_HIP; }

// Kernel arguments of a validated product: fp16 scales S, or int8 codes Q with
// row factors R (exactly one of the two is set).
tern::GemmArgs make_args(const void *X, tern_dtype x_dtype, const uint8_t *W, const uint16_t *S, const int8_t *Q,
                         const float *R, void *Y, tern_dtype y_dtype, int64_t M, int64_t N, int64_t K,
                         hipStream_t stream) {
    tern::GemmArgs a;
    a.X = X;
    a.x_dtype = x_dtype == TERN_BF16 ? 1 : 0;
    a.W = W;
    a.S = S;
    a.Q = Q;
    a.R = R;
    a.Y = Y;
    a.y_dtype = y_dtype == TERN_F16 ? 0 : (y_dtype == TERN_BF16 ? 1 : 2);
    a.M = M;
    a.N = N;
    a.K = K;
    a.stream = stream;
    return a;
}

bool gemv_fits(int64_t M, int64_t K) {
    return M >= 1 && M <= TERN_GEMV_MAX_M && tern::gemv_lds_bytes(M, K) <= kGemvLdsLimit;
}

// The automatic choice: the VALU decode kernel for one or two activation
// rows; from three rows on, the MFMA kernel (16-row tiles: its time hardly
// changes up to M = 16) is faster.  Measured on the 5120 / 17408 decode
// shapes: M = 2 GEMV 4.6 / 12.5 / 13.6 us against MFMA 7.4 / 15.8 / 16.4;
// M = 3 GEMV 7.6 / 18.8 / 19.9 against MFMA 7.5 / 15.9 / 16.6.
constexpr int64_t kAutoGemvMaxM = 2;

// Up to M = 4 the decode kernel also wins where it takes its short-step form
// (N <= 5120, K <= 8192; bf16, graph-timed): 5120 -> 5120 at M = 3 / 4
// 5.3 / 6.1 us against MFMA 6.9 / 7.0, 5120 -> 1024 at M = 4 3.8 against
// 5.7, 6144 -> 5120 at M = 3 / 4 5.5 / 6.3 against 8.8 / 8.8.
bool auto_gemv(int64_t M, int64_t N, int64_t K) {
    return (M <= kAutoGemvMaxM && gemv_fits(M, K)) || tern::gemv_short(M, N, K);
}

// With bf16 activations the fp4 matrix-core decode kernel is the fastest of
// the decode kernels at every M <= 4 measured (graph-timed, weights rotated
// over 2 GB; M = 1: 5120 -> 5120 4.04 us against the VALU kernel's 4.16,
// 5120 -> 17408 7.34 against 8.28, 17408 -> 5120 8.51 against 9.08; M = 4:
// 5120 -> 17408 11.0 against 29.4 (VALU) and 13.4 (16-row MFMA tiles),
// 17408 -> 5120 12.7 against 23.9 and 15.9).  With fp16 activations the
// 4x4x4 matrix-core kernel takes M = 3, 4 (M = 4: 5120 -> 17408 11.3 us
// against 13.4, 5120 -> 5120 6.1 against the VALU kernel's 6.5).
//
// For 5 <= M <= 16 the 16-row decode kernel beats the MFMA tiles where
// there are many weight rows and K is not long (graph-timed, bf16, weights
// rotated over 2 GB; M = 16: 5120 -> 34816 23.0 us against 31.1, 8192 ->
// 28672 34.0 against 40.5, 5120 -> 17408 16.9 against 19.0; M = 8 / 5 at
// 5120 -> 17408 16.9 / 16.8 against 19.1 / 18.6).  With N <= 15360, or K =
// 17408 (17408 -> 5120: 19.7 against 18.8), the tiles are as fast or faster.
bool auto_b16(int64_t M, int64_t N, int64_t K) {
    return M >= 5 && M <= 16 && N >= 16384 && K <= 8192 && tern::gemv_b16_fits(M, N, K);
}

tern_path auto_path(const tern::GemmArgs &a) {
    if (a.M <= 4 && a.x_dtype == 1 && tern::gemv_fp4_fits(a.M, a.N, a.K, 1)) return TERN_PATH_GEMV_FP4;
    if (a.M >= 3 && a.M <= 4 && a.x_dtype == 0 && tern::gemv_mfma_fits(a.M, a.N, a.K)) return TERN_PATH_GEMV_MFMA;
    if (auto_b16(a.M, a.N, a.K)) return TERN_PATH_GEMV_B16;
    return auto_gemv(a.M, a.N, a.K) ? TERN_PATH_GEMV : TERN_PATH_MFMA;
}

// A forced path that cannot run this shape is TERN_ERR_UNSUPPORTED (checked
// before anything is launched).
tern_status check_path(tern_path path, tern_dtype x_dtype, int64_t M, int64_t N, int64_t K) {
    if (path != TERN_PATH_AUTO && path != TERN_PATH_GEMV && path != TERN_PATH_MFMA && path != TERN_PATH_GEMV_MFMA &&
        path != TERN_PATH_GEMV_FP4 && path != TERN_PATH_GEMV_B16)
        return TERN_ERR_UNSUPPORTED;
    if (M == 0 || N == 0 || K == 0) return TERN_OK;
    if (path == TERN_PATH_GEMV && !gemv_fits(M, K)) return TERN_ERR_UNSUPPORTED;
    if (path == TERN_PATH_GEMV_MFMA && !tern::gemv_mfma_fits(M, N, K)) return TERN_ERR_UNSUPPORTED;
    if (path == TERN_PATH_GEMV_FP4 && !tern::gemv_fp4_fits(M, N, K, x_dtype == TERN_BF16 ? 1 : 0))
        return TERN_ERR_UNSUPPORTED;
    if (path == TERN_PATH_GEMV_B16 && !tern::gemv_b16_fits(M, N, K)) return TERN_ERR_UNSUPPORTED;
    return TERN_OK;
}

hipError_t dispatch(const tern::GemmArgs &a, tern_path path) {
    switch (path) {
    case TERN_PATH_GEMV: return tern::launch_gemv(a);
    case TERN_PATH_MFMA: return tern::launch_gemm(a);
    case TERN_PATH_GEMV_MFMA: return tern::launch_gemv_mfma(a);
    case TERN_PATH_GEMV_FP4: return tern::launch_gemv_fp4(a);
    case TERN_PATH_GEMV_B16: return tern::launch_gemv_b16(a);
    default: {
        const tern_path p = auto_path(a);
        return p == TERN_PATH_AUTO ? hipErrorInvalidValue : dispatch(a, p);
    }
    }
}

}  // namespace

extern "C" {

const char *tern_status_string(tern_status status) {
    switch (status) {
    case TERN_OK: return "TERN_OK";
    case TERN_ERR_NULL: return "TERN_ERR_NULL: a required pointer is NULL";
    case TERN_ERR_SHAPE: return "TERN_ERR_SHAPE: invalid size (negative, K % 4 != 0, or beyond limits)";
    case TERN_ERR_GROUP: return "TERN_ERR_GROUP: K is not a multiple of group, or group <= 0";
    case TERN_ERR_DTYPE: return "TERN_ERR_DTYPE: unsupported x or y dtype";
    case TERN_ERR_ALIGN: return "TERN_ERR_ALIGN: pointer misaligned";
    case TERN_ERR_UNSUPPORTED: return "TERN_ERR_UNSUPPORTED: request not implemented by this build";
    case TERN_ERR_HIP: return "TERN_ERR_HIP: HIP launch error";
    }
    return "TERN_ERR_UNKNOWN: not a tern_status value";
}

int tern_version(void) { return 100; }

tern_status tern_pack(const int8_t *T, uint8_t *packed, int64_t N, int64_t K, hipStream_t stream) {
    const tern_status st = check_pack_args(T, packed, N, K);
    if (st != TERN_OK || N == 0 || K == 0) return st;
    return from_hip(tern::launch_pack(T, packed, N * (K / 4), stream));
}

tern_status tern_unpack(const uint8_t *packed, int8_t *T, int64_t N, int64_t K, hipStream_t stream) {
    const tern_status st = check_pack_args(T, packed, N, K);
    if (st != TERN_OK || N == 0 || K == 0) return st;
    return from_hip(tern::launch_unpack(packed, T, N * (K / 4), stream));
}

tern_status tern_matmul_path(const void *X, tern_dtype x_dtype, const uint8_t *packed_W,
                             const uint16_t *scales, void *Y, tern_dtype y_dtype, int64_t M,
                             int64_t N, int64_t K, int32_t group, tern_path path,
                             hipStream_t stream) {
    const tern_status st = check_matmul_args(X, x_dtype, packed_W, scales, 2, Y, y_dtype, M, N, K, group);
    if (st != TERN_OK) return st;
    const tern_status pst = check_path(path, x_dtype, M, N, K);
    if (pst != TERN_OK) return pst;
    if (M == 0 || N == 0) return TERN_OK;
    if (K == 0) return from_hip(tern::launch_fill_zero(Y, M * N * (int64_t)dtype_size(y_dtype), stream));

    const tern::GemmArgs a = make_args(X, x_dtype, packed_W, scales, nullptr, nullptr, Y, y_dtype, M, N, K, stream);
    return from_hip(dispatch(a, path));
}

tern_status tern_matmul(const void *X, tern_dtype x_dtype, const uint8_t *packed_W, const uint16_t *scales,
                        void *Y, tern_dtype y_dtype, int64_t M, int64_t N, int64_t K, int32_t group,
                        hipStream_t stream) {
    return tern_matmul_path(X, x_dtype, packed_W, scales, Y, y_dtype, M, N, K, group, TERN_PATH_AUTO,
                            stream);
}

tern_status tern_quantize_scales(const uint16_t *scales, int8_t *scales_q, float *row_factor, int64_t N,
                                 int64_t K, int32_t group, hipStream_t stream) {
    if (N < 0 || K < 0 || N > kMaxDim || K > kMaxK || !product_ok(N, K) || K % 4 != 0) return TERN_ERR_SHAPE;
    if (group <= 0 || K % group != 0) return TERN_ERR_GROUP;
    if (group != TERN_GROUP) return TERN_ERR_UNSUPPORTED;
    if (N == 0) return TERN_OK;
    if (row_factor == nullptr) return TERN_ERR_NULL;
    if (K > 0 && (scales == nullptr || scales_q == nullptr)) return TERN_ERR_NULL;
    if (!aligned(scales, 2) || !aligned(row_factor, 4)) return TERN_ERR_ALIGN;
    return from_hip(tern::launch_quantize_scales(scales, scales_q, row_factor, N, K / group, stream));
}

tern_status tern_matmul_s8(const void *X, tern_dtype x_dtype, const uint8_t *packed_W, const int8_t *scales_q,
                           const float *row_factor, void *Y, tern_dtype y_dtype, int64_t M, int64_t N,
                           int64_t K, int32_t group, tern_path path, hipStream_t stream) {
    const tern_status st = check_matmul_args(X, x_dtype, packed_W, scales_q, 1, Y, y_dtype, M, N, K, group);
    if (st != TERN_OK) return st;
    if (M > 0 && N > 0 && K > 0 && row_factor == nullptr) return TERN_ERR_NULL;
    if (!aligned(row_factor, 4)) return TERN_ERR_ALIGN;
    const tern_status pst = check_path(path, x_dtype, M, N, K);
    if (pst != TERN_OK) return pst;
    if (M == 0 || N == 0) return TERN_OK;
    if (K == 0) return from_hip(tern::launch_fill_zero(Y, M * N * (int64_t)dtype_size(y_dtype), stream));

    const tern::GemmArgs a =
        make_args(X, x_dtype, packed_W, nullptr, scales_q, row_factor, Y, y_dtype, M, N, K, stream);
    return from_hip(dispatch(a, path));
}

tern_status tern_block_map(const uint8_t *packed, uint32_t *block_map, int64_t N, int64_t K, int32_t group,
                           hipStream_t stream) {
    if (N < 0 || K < 0 || N > kMaxDim || K > kMaxK || !product_ok(N, K) || K % 4 != 0) return TERN_ERR_SHAPE;
    if (group <= 0 || K % group != 0) return TERN_ERR_GROUP;
    if (group != TERN_GROUP) return TERN_ERR_UNSUPPORTED;
    if (N == 0 || K == 0) return TERN_OK;
    if (packed == nullptr || block_map == nullptr) return TERN_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(block_map, 4)) return TERN_ERR_ALIGN;
    return from_hip(tern::launch_block_map(packed, block_map, N, K, stream));
}

tern_status tern_matmul_blockmap(const void *X, tern_dtype x_dtype, const uint8_t *packed_W,
                                 const uint16_t *scales, const uint32_t *block_map, void *Y, tern_dtype y_dtype,
                                 int64_t M, int64_t N, int64_t K, int32_t group, hipStream_t stream) {
    const tern_status st = check_matmul_args(X, x_dtype, packed_W, scales, 2, Y, y_dtype, M, N, K, group);
    if (st != TERN_OK) return st;
    if (M > 0 && N > 0 && K > 0 && block_map == nullptr) return TERN_ERR_NULL;
    if (!aligned(block_map, 4)) return TERN_ERR_ALIGN;
    const bool skip = M >= 1 && M <= kAutoGemvMaxM && K > 0 && tern::gemv_skip_lds_bytes(M, K) <= kGemvLdsLimit;
    if (!skip) return tern_matmul_path(X, x_dtype, packed_W, scales, Y, y_dtype, M, N, K, group, TERN_PATH_AUTO,
                                       stream);
    if (N == 0) return TERN_OK;

    const tern::GemmArgs a = make_args(X, x_dtype, packed_W, scales, nullptr, nullptr, Y, y_dtype, M, N, K, stream);
    return from_hip(tern::launch_gemv_skip(a, block_map));
}

tern_status tern_dequant(const uint8_t *packed, const uint16_t *scales, void *W, tern_dtype w_dtype,
                         int64_t N, int64_t K, int32_t group, hipStream_t stream) {
    if (N < 0 || K < 0 || N > kMaxDim || K > kMaxK || !product_ok(N, K) || K % 4 != 0) return TERN_ERR_SHAPE;
    if (group <= 0 || K % group != 0) return TERN_ERR_GROUP;
    if (w_dtype != TERN_F16 && w_dtype != TERN_BF16) return TERN_ERR_DTYPE;
    if (group != TERN_GROUP) return TERN_ERR_UNSUPPORTED;
    if (N == 0 || K == 0) return TERN_OK;
    if (packed == nullptr || scales == nullptr || W == nullptr) return TERN_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(W, 16) || !aligned(scales, 2)) return TERN_ERR_ALIGN;
    return from_hip(tern::launch_dequant(packed, scales, W, w_dtype == TERN_BF16 ? 1 : 0, N, K, stream));
}

}  // extern "C"
