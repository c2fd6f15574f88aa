// tern_dequant.hip -- the comparison route's first half: W[N,K] = t * s.
//
// 2kiu.com/news/5082861 §4.1 describes the route this serves as a yardstick:
// dequantise the packed weights to a dense 16-bit matrix, then call a library
// GEMM.  The pages measure their fused kernel against it (§4.3); this kernel
// lets the same comparison be made here (a hipBLASLt GEMM through torch does
// the second half, outside this library).
//
// Each thread step turns one 32-bit code word (16 consecutive weights of a
// row, inside one 128-weight block) into 16 output values (two 16-byte
// stores): +s, -s or 0, where s is the block's fp16 scale (exact in fp16; for
// a bf16 output, s is rounded to bf16 once, to nearest even).
#include <hip/hip_runtime.h>

#include "tern_device.h"
#include "tern_kernels.h"

namespace tern {

namespace {

template <bool BF16OUT>
__global__ void dequant_kernel(const uint32_t *__restrict__ P, const uint16_t *__restrict__ S,
                               uint4 *__restrict__ W, int64_t words, int64_t words_per_row, int groups) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) {
        const int64_t n = i / words_per_row;
        const int64_t wrow = i - n * words_per_row;   // word index inside the row: weights 16*wrow ..
        const uint16_t sb = S[n * groups + (wrow >> 3)];  // 8 words per 128-weight block
        uint32_t pos;
        if constexpr (BF16OUT) {
            const __bf16 b = static_cast<__bf16>(f16_bits_to_float(sb));
            pos = __builtin_bit_cast(uint16_t, b);
        } else {
            pos = sb;
        }
        const uint32_t neg = pos ^ 0x8000u;
        const uint32_t w = P[i];
        uint32_t out[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            uint32_t half2 = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t c = (w >> (4 * h + 2 * e)) & 3u;
                const uint32_t v = c == 1u ? pos : (c == 2u ? neg : 0u);
                half2 |= v << (16 * e);
            }
            out[h] = half2;
        }
        W[2 * i] = make_uint4(out[0], out[1], out[2], out[3]);
        W[2 * i + 1] = make_uint4(out[4], out[5], out[6], out[7]);
    }
}

}  // namespace

hipError_t launch_dequant(const uint8_t *P, const uint16_t *S, void *W, int w_dtype, int64_t N, int64_t K,
                          hipStream_t stream) {
    const int64_t words = N * (K / 16);
    const int block = 256;
    int64_t grid = (words + block - 1) / block;
    if (grid > 65536) grid = 65536;
    if (grid < 1) grid = 1;
    if (w_dtype == 1)
        hipLaunchKernelGGL(dequant_kernel<true>, dim3((unsigned)grid), dim3(block), 0, stream,
                           reinterpret_cast<const uint32_t *>(P), S, static_cast<uint4 *>(W), words, K / 16,
                           (int)(K / 128));
    else
        hipLaunchKernelGGL(dequant_kernel<false>, dim3((unsigned)grid), dim3(block), 0, stream,
                           reinterpret_cast<const uint32_t *>(P), S, static_cast<uint4 *>(W), words, K / 16,
                           (int)(K / 128));
    return hipGetLastError();
}

}  // namespace tern
