// tern_scales.hip -- int8 scale codes for the int8-scale variant.
//
// 2kiu.com/news/5082861 §6 lists compressing the per-block fp16 scale
// further to INT8 as a next step, without fixing the scheme.  The reading
// taken here: per output row n, a symmetric code with one fp32 factor,
//   R[n]   = max_g |S[n,g]| / 127                (fp32 division)
//   Q[n,g] = round-to-nearest-even(S[n,g] / R[n]) in [-127, 127]
// (Q = 0 when the row's scales are all zero).  The effective scale is
// Q[n,g] * R[n].  One wave per row: the maximum is a wave reduction, then
// each lane codes its groups; every integer decision is an IEEE fp32
// division and rint, so it is reproducible.
#include <hip/hip_runtime.h>

#include "tern_device.h"
#include "tern_kernels.h"

namespace tern {

namespace {

constexpr int ROWS_PER_BLOCK = 4;   // one wave per row

__global__ __launch_bounds__(64 * ROWS_PER_BLOCK) void quantize_kernel(const uint16_t *__restrict__ S,
                                                                     int8_t *__restrict__ Q,
                                                                     float *__restrict__ R, int64_t N,
                                                                     int64_t groups) {
    const int lane = threadIdx.x & 63;
    const int64_t n = (int64_t)blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
    if (n >= N) return;   // whole waves leave together
    const uint16_t *s = S + n * groups;
    float amax = 0.f;
    for (int64_t g = lane; g < groups; g += 64) amax = fmaxf(amax, fabsf(f16_bits_to_float(s[g])));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const float r = amax / 127.0f;
    if (lane == 0) R[n] = r;
    int8_t *q = Q + n * groups;
    for (int64_t g = lane; g < groups; g += 64) {
        float t = 0.f;
        if (r > 0.f) t = rintf(f16_bits_to_float(s[g]) / r);
        t = fminf(fmaxf(t, -127.f), 127.f);
        q[g] = (int8_t)t;
    }
}

}  // namespace

hipError_t launch_quantize_scales(const uint16_t *S, int8_t *Q, float *R, int64_t N, int64_t groups,
                                  hipStream_t stream) {
    const int64_t blocks = (N + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(64 * ROWS_PER_BLOCK), 0, stream, S, Q, R, N,
                       groups);
    return hipGetLastError();
}

}  // namespace tern
