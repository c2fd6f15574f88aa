// tern_gemv.hip -- decode-path kernel (small M): Y[M,N] = X[M,K] . (T*S)^T.
//
// Method (2kiu.com/news/5082861): weights stay packed (§4.1, second route);
// inside a 128-weight block the signs are accumulated with add / subtract /
// skip and the block sum is multiplied by its fp16 scale at the block
// boundary (§1.1, §4.1 third route, §4.2); activations and scales are kept
// on chip, never re-read from memory in the inner loop (§4.2, §4.3).
//
// Work layout (one workgroup = 16 output rows x all of K):
//   * a wave "step" covers 4 rows x 1024 weights per load instruction:
//     lane = 16*r + kk; lane kk of row-group r loads 16 bytes (64 weights) of
//     row n0 + 4j + r (j = 0..3) at K offset step*1024 + 64*kk.  Each load
//     instruction reads four 256-byte contiguous row segments.
//   * the waves of the workgroup split the K steps; each wave keeps one fp32
//     partial per (row, m) per lane, reduces it over the 16 lanes of its DPP
//     row, and the waves' partials are summed through LDS in a fixed order
//     (deterministic; no atomics, no workspace).
//   * X is staged once per workgroup into LDS, pair-interleaved (see
//     tern_device.h) and swizzled so that the 16 lanes of a row-group read 16
//     consecutive 16-byte pieces (conflict-free; the 4 row-groups broadcast).
#include <hip/hip_runtime.h>

#include "tern_device.h"
#include "tern_kernels.h"

namespace tern {

namespace {

constexpr int ROWS = 16;          // output rows per workgroup
constexpr int STEP = 1024;        // weights of one row per wave step
constexpr int CHUNK = 64;         // weights per lane per row per step (16 bytes)

// LDS word offset (in 16-byte pieces) of piece q (0..7) of 64-weight chunk c
// of activation row m.
__device__ __forceinline__ int x_piece(int m, int c, int q, int pieces_per_row) {
    return m * pieces_per_row + ((c >> 4) * 8 + q) * 16 + (c & 15);
}

template <int M, bool XBF16, int YT>
__global__ __launch_bounds__(1024) void gemv_kernel(const uint16_t *__restrict__ X,
                                                     const uint8_t *__restrict__ P,
                                                     const uint16_t *__restrict__ S,
                                                     void *__restrict__ Y, int N, int K,
                                                     int steps_per_wave) {
    extern __shared__ uint4 lds[];
    const int nsteps = (K + STEP - 1) / STEP;
    const int pieces_per_row = nsteps * 128;  // 16 chunks x 8 pieces per step
    float *red = reinterpret_cast<float *>(lds + M * pieces_per_row);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int r = lane >> 4;
    const int kk = lane & 15;
    const int n0 = blockIdx.x * ROWS;
    const int64_t row_bytes = K >> 2;
    const int groups = K >> 7;

    // ---- this wave's weight loads go out first (they are the long pole) ----
    const int s_begin = wave * steps_per_wave;
    const int s_end = min(nsteps, s_begin + steps_per_wave);

    // ---- stage X into LDS: one 16-element block per thread iteration ----
    const int blocks_per_row = K >> 4;
    for (int b = tid; b < M * blocks_per_row; b += blockDim.x) {
        const int m = b / blocks_per_row;
        const int d = b - m * blocks_per_row;  // 16-element block along K
        const uint4 *src = reinterpret_cast<const uint4 *>(X + (int64_t)m * K + (int64_t)d * 16);
        const uint4 lo = src[0];
        const uint4 hi = src[1];
        uint32_t pr[8];
        interleave16(lo, hi, pr);
        const int c = d >> 2;              // 64-weight chunk
        const int q0 = (d & 3) * 2;        // first of its two 16-byte pieces
        lds[x_piece(m, c, q0, pieces_per_row)] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
        lds[x_piece(m, c, q0 + 1, pieces_per_row)] = make_uint4(pr[4], pr[5], pr[6], pr[7]);
    }
    __syncthreads();

    float acc[4][M];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[j][m] = 0.f;

    for (int s = s_begin; s < s_end; ++s) {
        const int c = s * 16 + kk;                 // this lane's 64-weight chunk
        const bool kact = c * CHUNK < K;
        uint4 code[4];
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + 4 * j + r;
            if (kact && n < N) {
                code[j] = *reinterpret_cast<const uint4 *>(P + (int64_t)n * row_bytes + (int64_t)c * 16);
                sc[j] = f16_bits_to_float(S[(int64_t)n * groups + (c >> 1)]) * 0.5f;
            } else {
                code[j] = make_uint4(0, 0, 0, 0);
                sc[j] = 0.f;
            }
        }
        if (!kact) continue;
        uint4 xq[M][8];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int q = 0; q < 8; ++q) xq[m][q] = lds[x_piece(m, c, q, pieces_per_row)];

#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float part[M];
#pragma unroll
            for (int m = 0; m < M; ++m) part[m] = 0.f;
            const uint32_t cw[4] = {code[j].x, code[j].y, code[j].z, code[j].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t v = sign_nz_fields(cw[d]);
                const uint32_t p0 = weight_pair<0>(v), p1 = weight_pair<1>(v);
                const uint32_t p2 = weight_pair<2>(v), p3 = weight_pair<3>(v);
                const uint32_t p4 = weight_pair<4>(v), p5 = weight_pair<5>(v);
                const uint32_t p6 = weight_pair<6>(v), p7 = weight_pair<7>(v);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const uint4 a = xq[m][2 * d];
                    const uint4 b = xq[m][2 * d + 1];
                    float t = part[m];
                    t = dot2<XBF16>(p0, a.x, t);
                    t = dot2<XBF16>(p1, a.y, t);
                    t = dot2<XBF16>(p2, a.z, t);
                    t = dot2<XBF16>(p3, a.w, t);
                    t = dot2<XBF16>(p4, b.x, t);
                    t = dot2<XBF16>(p5, b.y, t);
                    t = dot2<XBF16>(p6, b.z, t);
                    t = dot2<XBF16>(p7, b.w, t);
                    part[m] = t;
                }
            }
            // block boundary: this lane's 64 weights lie in one 128-block
#pragma unroll
            for (int m = 0; m < M; ++m) acc[j][m] = fmaf(sc[j], part[m], acc[j][m]);
        }
    }

    // ---- reduce over the 16 lanes of each DPP row, then across waves ----
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[j][m] = row16_sum(acc[j][m]);
    if (kk == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int m = 0; m < M; ++m) red[(wave * ROWS + 4 * j + r) * M + m] = acc[j][m];
    }
    __syncthreads();
    if (tid < ROWS * M) {
        const int row = tid % ROWS;
        const int m = tid / ROWS;
        float y = 0.f;
        for (int w = 0; w < nwaves; ++w) y += red[(w * ROWS + row) * M + m];
        const int n = n0 + row;
        if (n < N) store_out<YT>(Y, (int64_t)m * N + n, y);
    }
}

template <int M, bool XBF16, int YT>
hipError_t launch_gemv_t(const GemmArgs &a) {
    const int nsteps = (int)((a.K + STEP - 1) / STEP);
    const int spw = (nsteps + 15) / 16;
    const int nwaves = (nsteps + spw - 1) / spw;
    const size_t lds_bytes = (size_t)M * nsteps * 128 * 16 + (size_t)nwaves * ROWS * M * sizeof(float);
    auto kern = gemv_kernel<M, XBF16, YT>;
    if (lds_bytes > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)((a.N + ROWS - 1) / ROWS));
    const dim3 block((unsigned)(64 * nwaves));
    hipLaunchKernelGGL(kern, grid, block, lds_bytes, a.stream, static_cast<const uint16_t *>(a.X),
                       a.W, a.S, a.Y, (int)a.N, (int)a.K, spw);
    return hipGetLastError();
}

template <int M, bool XBF16>
hipError_t launch_gemv_y(const GemmArgs &a) {
    switch (a.y_dtype) {
    case 0: return launch_gemv_t<M, XBF16, 0>(a);
    case 1: return launch_gemv_t<M, XBF16, 1>(a);
    default: return launch_gemv_t<M, XBF16, 2>(a);
    }
}

template <int M>
hipError_t launch_gemv_m(const GemmArgs &a) {
    return a.x_dtype == 1 ? launch_gemv_y<M, true>(a) : launch_gemv_y<M, false>(a);
}

}  // namespace

size_t gemv_lds_bytes(int64_t M, int64_t K) {
    const int64_t nsteps = (K + STEP - 1) / STEP;
    const int64_t spw = (nsteps + 15) / 16;
    const int64_t nwaves = (nsteps + spw - 1) / spw;
    return (size_t)(M * nsteps * 128 * 16 + nwaves * ROWS * M * 4);
}

hipError_t launch_gemv(const GemmArgs &a) {
    switch (a.M) {
    case 1: return launch_gemv_m<1>(a);
    case 2: return launch_gemv_m<2>(a);
    case 3: return launch_gemv_m<3>(a);
    default: return launch_gemv_m<4>(a);
    }
}

}  // namespace tern
