// tern_gemm.hip -- batched-path kernel: Y[M,N] = X[M,K] . (T*S)^T on MFMA.
//
// Method (2kiu.com/news/5082861): weights stay packed in memory and are
// decoded on chip (§4.1, second route: decode inside the kernel, never a
// dequantised copy in memory); scales are read once per 128-weight block and
// kept in registers (§4.2, §4.3).  Here the decoded block feeds gfx950's
// matrix cores, because with many activation rows the work is a dense
// contraction.
//
// Tiling: a workgroup of 4 waves computes a (16*MB) x 256 tile of Y; wave w
// owns columns 64w..64w+63 (4 blocks of 16) and all 16*MB rows.  Per
// 128-wide K block (one scale group):
//   * X[rows, 128] goes global -> registers -> LDS, pair-interleaved (see
//     tern_device.h), row stride 272 bytes (bank-conflict-free 16-byte reads);
//   * each lane loads 8 bytes of codes (32 weights) for each of its 4
//     columns and decodes them in registers straight into MFMA B operands:
//     +-2 pairs (tern_device.h); with fp16 X they are multiplied by the fp16
//     scale (+-2s, exact); with bf16 X they stay +-2 and the scale is applied
//     in fp32 to the block's partial sum;
//   * v_mfma_f32_16x16x32_{f16,bf16}: lane l gives A[l%16][8(l/16)+e] and
//     B[8(l/16)+e][l%16]; the lane's 32 weights of a block are spread over
//     the 4 MFMA k-steps so that the activation fragment for step t is the
//     16-byte run X'[32g + 8t .. +8] of the pair-interleaved row.
#include <hip/hip_runtime.h>

#include "tern_device.h"
#include "tern_kernels.h"

namespace tern {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int BN = 256;              // columns per workgroup
constexpr int NB = 4;                // 16-column blocks per wave
constexpr int BK = 128;              // K per iteration (= one scale group)
constexpr int LDS_ROW = 272;         // bytes per staged activation row (256 + 16 pad)

template <bool BF16>
__device__ __forceinline__ float4_t mfma16x16x32(const uint4 &a, const uint4 &b, float4_t c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, a),
                                                       __builtin_bit_cast(bf168_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    }
}

__device__ __forceinline__ uint32_t mul_pair_f16(uint32_t p, half2_t s2) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p) * s2);
}

// The 4 B-operand words for k-step t from one lane's 8 code bytes.
template <int T>
__device__ __forceinline__ uint4 b_operand(uint32_t v_lo, uint32_t v_hi) {
    const uint32_t v = (T < 2) ? v_lo : v_hi;
    constexpr int H = T & 1;
    return make_uint4(weight_pair<4 * H + 0>(v), weight_pair<4 * H + 1>(v),
                      weight_pair<4 * H + 2>(v), weight_pair<4 * H + 3>(v));
}

template <int MB, bool XBF16, int YT>
__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t *__restrict__ X,
                                                    const uint8_t *__restrict__ P,
                                                    const uint16_t *__restrict__ S,
                                                    void *__restrict__ Y, int M, int N, int K,
                                                    int tiles_n) {
    constexpr int BM = 16 * MB;
    constexpr int A_UNITS = BM * (BK / 16) / 256;   // 16-element blocks per thread per K block
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[BM * LDS_ROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;   // row (A) / column (B) within a 16-block
    const int lg = lane >> 4;   // k-slot group
    const int tile_m = blockIdx.x / tiles_n;
    const int tile_n = blockIdx.x - tile_m * tiles_n;
    const int m0 = tile_m * BM;
    const int n0 = tile_n * BN + wave * 64;
    const int64_t row_bytes = K >> 2;
    const int groups = K >> 7;
    const int nk = K / BK;

    // activation prefetch registers
    uint4 a_reg[A_UNITS][2];
    // Loads are unconditional at clamped, in-bounds addresses: rows past M
    // and columns past N produce outputs that are never stored.  (A
    // conditional load with a zeroing else-branch would make every load wait
    // for the previous one.)
    auto load_a = [&](int kb) {
#pragma unroll
        for (int u = 0; u < A_UNITS; ++u) {
            const int b = tid + 256 * u;
            const int row = b >> 3;
            const int blk = b & 7;
            const int64_t m = min(m0 + row, M - 1);
            const uint4 *src = reinterpret_cast<const uint4 *>(X + m * K + (int64_t)kb * BK + blk * 16);
            a_reg[u][0] = src[0];
            a_reg[u][1] = src[1];
        }
    };
    auto store_a = [&]() {
#pragma unroll
        for (int u = 0; u < A_UNITS; ++u) {
            const int b = tid + 256 * u;
            const int row = b >> 3;
            const int blk = b & 7;
            uint32_t pr[8];
            interleave16(a_reg[u][0], a_reg[u][1], pr);
            uint4 *dst = reinterpret_cast<uint4 *>(a_lds + row * LDS_ROW + blk * 32);
            dst[0] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
            dst[1] = make_uint4(pr[4], pr[5], pr[6], pr[7]);
        }
    };

    // weight prefetch registers: 8 code bytes + one scale per column block
    uint2 w_reg[NB];
    uint16_t s_reg[NB];
    auto load_w = [&](int kb) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int64_t n = min(n0 + nb * 16 + li, N - 1);
            w_reg[nb] = *reinterpret_cast<const uint2 *>(P + n * row_bytes + (int64_t)kb * (BK / 4) + lg * 8);
            s_reg[nb] = S[n * groups + kb];
        }
    };

    float4_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

    load_a(0);
    load_w(0);
    for (int kb = 0; kb < nk; ++kb) {
        __syncthreads();                 // everyone is done reading the previous tile
        store_a();
        __syncthreads();
        uint2 w_cur[NB];
        uint16_t s_cur[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            w_cur[nb] = w_reg[nb];
            s_cur[nb] = s_reg[nb];
        }
        if (kb + 1 < nk) {               // next block's loads overlap this block's math
            load_a(kb + 1);
            load_w(kb + 1);
        }

        uint32_t v_lo[NB], v_hi[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            v_lo[nb] = sign_nz_fields(w_cur[nb].x);
            v_hi[nb] = sign_nz_fields(w_cur[nb].y);
        }

        float4_t part[XBF16 ? MB : 1][XBF16 ? NB : 1];
        if constexpr (XBF16) {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) part[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
        }

        auto kstep = [&](auto tc) {
            constexpr int T = decltype(tc)::value;
            uint4 bop[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                uint4 b = b_operand<T>(v_lo[nb], v_hi[nb]);
                if constexpr (!XBF16) {
                    const _Float16 sh = __builtin_bit_cast(_Float16, s_cur[nb]);
                    const half2_t s2 = {sh, sh};
                    b.x = mul_pair_f16(b.x, s2);
                    b.y = mul_pair_f16(b.y, s2);
                    b.z = mul_pair_f16(b.z, s2);
                    b.w = mul_pair_f16(b.w, s2);
                }
                bop[nb] = b;
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const uint4 a = *reinterpret_cast<const uint4 *>(a_lds + (mb * 16 + li) * LDS_ROW + (32 * lg + 8 * T) * 2);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if constexpr (XBF16)
                        part[mb][nb] = mfma16x16x32<true>(a, bop[nb], part[mb][nb]);
                    else
                        acc[mb][nb] = mfma16x16x32<false>(a, bop[nb], acc[mb][nb]);
                }
            }
        };
        kstep(std::integral_constant<int, 0>{});
        kstep(std::integral_constant<int, 1>{});
        kstep(std::integral_constant<int, 2>{});
        kstep(std::integral_constant<int, 3>{});

        if constexpr (XBF16) {           // block boundary: scale the block's sums
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float s = f16_bits_to_float(s_cur[nb]) * 0.5f;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    acc[mb][nb][0] = fmaf(s, part[mb][nb][0], acc[mb][nb][0]);
                    acc[mb][nb][1] = fmaf(s, part[mb][nb][1], acc[mb][nb][1]);
                    acc[mb][nb][2] = fmaf(s, part[mb][nb][2], acc[mb][nb][2]);
                    acc[mb][nb][3] = fmaf(s, part[mb][nb][3], acc[mb][nb][3]);
                }
            }
        }
    }

    // epilogue: lane l holds rows 4(l/16)+i, column l%16 of each 16x16 block
    const float post = XBF16 ? 1.0f : 0.5f;    // the +-2s operand counted each weight twice
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = n0 + nb * 16 + li;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + mb * 16 + lg * 4 + i;
                if (m < M) store_out<YT>(Y, (int64_t)m * N + n, acc[mb][nb][i] * post);
            }
        }
}

template <int MB, bool XBF16, int YT>
hipError_t launch_t(const GemmArgs &a) {
    const int64_t tiles_n = (a.N + BN - 1) / BN;
    const int64_t tiles_m = (a.M + 16 * MB - 1) / (16 * MB);
    if (tiles_n * tiles_m > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(tiles_n * tiles_m));
    hipLaunchKernelGGL((gemm_kernel<MB, XBF16, YT>), grid, dim3(256), 0, a.stream,
                       static_cast<const uint16_t *>(a.X), a.W, a.S, a.Y, (int)a.M, (int)a.N, (int)a.K,
                       (int)tiles_n);
    return hipGetLastError();
}

template <bool XBF16>
hipError_t launch_y(const GemmArgs &a) {
    constexpr int MB = XBF16 ? 4 : 8;
    switch (a.y_dtype) {
    case 0: return launch_t<MB, XBF16, 0>(a);
    case 1: return launch_t<MB, XBF16, 1>(a);
    default: return launch_t<MB, XBF16, 2>(a);
    }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs &a) {
    return a.x_dtype == 1 ? launch_y<true>(a) : launch_y<false>(a);
}

}  // namespace tern
