// tern_gemv.hip -- decode-path kernel (small M): Y[M,N] = X[M,K] . (T*S)^T.
//
// Method (2kiu.com/news/5082861): weights stay packed (§4.1, second route);
// inside a 128-weight block the signs are accumulated with add / subtract /
// skip and the block sum is multiplied by its fp16 scale at the block
// boundary (§1.1, §4.1 third route, §4.2); activations and scales are kept
// on chip, never re-read from memory in the inner loop (§4.2, §4.3); wide
// vector loads of the packed bytes (§4.3, third version).
//
// Work layout (one workgroup = 4 JR output rows x all of K; JR = 2 or 3):
//   * a wave "step" covers 4 JR rows x 1024 weights: lane = 16*r + kk; for
//     j < JR the lane loads 16 bytes (64 weights) of row n0 + 4j + r at K
//     offset step*1024 + 64*kk, so every load instruction reads four
//     256-byte contiguous row segments;
//   * the waves of a workgroup (up to 16 for M = 1, 8 otherwise) split the K
//     steps.  Each wave first issues all of its loads (activations, then
//     weights and scales), stages the activations of its own steps into a
//     wave-private LDS slice
//     (pair-interleaved, see tern_device.h; the four lanes that share a
//     64-weight chunk stage a quarter each), then decodes and accumulates as
//     the loads land;
//   * each lane keeps one fp32 partial per (row, m); it is summed over the
//     16 lanes of its DPP row, then across the waves through LDS in a fixed
//     order (deterministic; no atomics, no workspace).
//   * small workgroups (8 rows, or 12 when K > 16384) spread a layer's rows
//     over many CUs, so no CU runs much more than its share.
// A short-step variant (gemv_short_kernel, below) serves M <= 4 when N is at
// most 5120 and K at most 5120 (M = 1) or 8192, and M = 2 with K <= 8192 on
// layers of 12288 rows or more: 512-weight steps and 8 code bytes per lane
// and row, each decoded pair feeding every activation row; workgroups of
// 4 ceil(N / 1024) <= 20 rows (at most 256 of them, one per CU) up to N =
// 5120, and of 20 rows over several rounds of workgroups on the wide M = 2
// layers.
#include <hip/hip_runtime.h>

#include <atomic>

#include "tern_device.h"
#include "tern_gemv_common.h"
#include "tern_kernels.h"

namespace tern {

namespace {

using namespace gemv;

template <int M, bool XBF16, int YT, int SPW, bool S8, int JR>
__global__ __launch_bounds__(M == 1 ? 1024 : 512) void gemv_kernel(const uint16_t *__restrict__ X,
                                                     const uint8_t *__restrict__ P,
                                                     const uint16_t *__restrict__ S,
                                                     const int8_t *__restrict__ Q,
                                                     const float *__restrict__ R,
                                                     void *__restrict__ Y, int N, int K) {
    constexpr int ROWS = 4 * JR;
    extern __shared__ uint4 lds[];
    const int nsteps = (K + STEP - 1) / STEP;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int r = lane >> 4;
    const int kk = lane & 15;
    const int n0 = blockIdx.x * ROWS;
    const int64_t row_bytes = K >> 2;
    const int groups = K >> 7;
    uint4 *xw = lds + wave * (SPW * M * PIECES);                          // this wave's activations
    float *red = reinterpret_cast<float *>(lds + nwaves * (SPW * M * PIECES));

    const int s_begin = wave * SPW;

    // ---- 1. activation loads first (they gate the staging), then every
    //         weight and scale load of this wave.  All loads are issued
    //         unconditionally at clamped, in-bounds addresses: a row past N is
    //         never stored, and a chunk past K is excluded when accumulating.
    //         (A conditional load with a zeroing else-branch would force a
    //         wait for every load before the next one is issued.)
    const int nchunks = K / CHUNK;
    uint4 xraw[SPW][M][2];
#pragma unroll
    for (int si = 0; si < SPW; ++si) {
        const int c = min((s_begin + si) * 16 + kk, nchunks - 1);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            // lane (r, kk) fetches 16-element block r of chunk c
            const uint4 *src = reinterpret_cast<const uint4 *>(X + (int64_t)m * K + (int64_t)c * CHUNK + r * 16);
            xraw[si][m][0] = src[0];
            xraw[si][m][1] = src[1];
        }
    }
    uint4 code[SPW][JR];
    uint32_t sbits[SPW][JR];     // fp16 scale bits, or the sign-extended int8 code
#pragma unroll
    for (int si = 0; si < SPW; ++si) {
        const int c = min((s_begin + si) * 16 + kk, nchunks - 1);
#pragma unroll
        for (int j = 0; j < JR; ++j) {
            const int64_t n = min(n0 + 4 * j + r, N - 1);
            code[si][j] = load_codes(P + n * row_bytes + (int64_t)c * 16);
            if constexpr (S8) sbits[si][j] = (uint32_t)(int32_t)Q[n * groups + (c >> 1)];
            else sbits[si][j] = S[n * groups + (c >> 1)];
        }
    }
    // S8: the row factor multiplies the finished row sum (sum_g q r p = r sum_g q p);
    // the threads that store rows fetch it now, off the critical path
    float rowf = 1.f;
    if constexpr (S8) {
        if (tid < ROWS * M) rowf = R[min(n0 + tid % ROWS, N - 1)];
    }

    // ---- 2. stage this wave's activations, pair-interleaved ----
#pragma unroll
    for (int si = 0; si < SPW; ++si) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            uint32_t pr[8];
            interleave16(xraw[si][m][0], xraw[si][m][1], pr);
            uint4 *dst = xw + (si * M + m) * PIECES;
            dst[(2 * r) * 16 + kk] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
            dst[(2 * r + 1) * 16 + kk] = make_uint4(pr[4], pr[5], pr[6], pr[7]);
        }
    }
    // the slice is private to this wave: a wave-level fence and barrier suffice
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- 3. decode + sign-select accumulate, scale at the block boundary ----
    float acc[JR][M];
#pragma unroll
    for (int j = 0; j < JR; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[j][m] = 0.f;

    // activation rows are taken MC at a time (a row's 32 activation words in
    // registers); each code word is decoded once per group of MC rows.  Two
    // rows per decode for even M (M = 2: 14-24% faster than one row at a
    // time on the decode shapes), one for odd M, which keeps the register
    // footprint of M = 1
    constexpr int MC = M % 2 == 0 ? 2 : 1;
#pragma unroll
    for (int si = 0; si < SPW; ++si) {
        const uint32_t kact = opaque_mask((s_begin + si) * 16 + kk < nchunks);   // this lane's chunk lies inside K
#pragma unroll
        for (int mb = 0; mb < M; mb += MC) {
            uint4 xq[MC][8];
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const uint4 *src = xw + (si * M + mb + m) * PIECES;
#pragma unroll
                for (int q = 0; q < 8; ++q) xq[m][q] = src[q * 16 + kk];
            }
#pragma unroll
            for (int j = 0; j < JR; ++j) {
                // this lane's 64 weights lie inside one 128-weight block; the +-2
                // operands double the sum and the 0.5 undoes it exactly
                float part[MC];
#pragma unroll
                for (int m = 0; m < MC; ++m) part[m] = 0.f;
                chunk_dot<MC, XBF16>(code[si][j], xq, part);
                const float s = (S8 ? (float)(int32_t)sbits[si][j]
                                    : f16_bits_to_float((uint16_t)sbits[si][j])) * 0.5f;
#pragma unroll
                for (int m = 0; m < MC; ++m)
                    acc[j][mb + m] = masked_fma(kact, s, part[m], acc[j][mb + m]);
                if constexpr (M > 1) __builtin_amdgcn_sched_barrier(0);   // one row's pairs live at a time
            }
        }
        // keep the scheduler from hoisting the next step's LDS reads into this
        // step (that would hold several steps' activations in registers)
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- 4. reduce over the 16 lanes of each DPP row, then across waves ----
#pragma unroll
    for (int j = 0; j < JR; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[j][m] = row16_sum(acc[j][m]);
    if (kk == 0) {
#pragma unroll
        for (int j = 0; j < JR; ++j)
#pragma unroll
            for (int m = 0; m < M; ++m) red[(wave * ROWS + 4 * j + r) * M + m] = acc[j][m];
    }
    __syncthreads();
    if (tid < ROWS * M) {
        const int row = tid % ROWS;
        const int m = tid / ROWS;
        float y = 0.f;
        for (int w = 0; w < nwaves; ++w) y += red[(w * ROWS + row) * M + m];
        if constexpr (S8) y *= rowf;
        const int n = n0 + row;
        if (n < N) store_out<YT>(Y, (int64_t)m * N + n, y);
    }
}

template <int M, bool XBF16, int YT, int SPW, bool S8, int JR>
hipError_t launch_gemv_t(const GemmArgs &a, const GemvShape &g) {
    constexpr int ROWS = 4 * JR;
    if (g.jr != JR) return hipErrorInvalidValue;   // the LDS size was computed for g.jr
    auto kern = gemv_kernel<M, XBF16, YT, SPW, S8, JR>;
    if (g.lds > 64 * 1024) {
        // raise the dynamic-LDS limit once per device (not a stream operation,
        // so it is kept out of any graph capture after the first call)
        static std::atomic<uint64_t> done_mask{0};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const uint64_t bit = 1ull << (dev & 63);
        if (!(done_mask.load(std::memory_order_acquire) & bit)) {
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
            if (e != hipSuccess) return e;
            done_mask.fetch_or(bit, std::memory_order_acq_rel);
        }
    }
    const dim3 grid((unsigned)((a.N + ROWS - 1) / ROWS));
    const dim3 block((unsigned)(64 * g.nwaves));
    hipLaunchKernelGGL(kern, grid, block, g.lds, a.stream, static_cast<const uint16_t *>(a.X), a.W, a.S,
                       a.Q, a.R, a.Y, (int)a.N, (int)a.K);
    return hipGetLastError();
}

template <int M, bool XBF16, int YT, bool S8>
hipError_t launch_gemv_s(const GemmArgs &a) {
    const GemvShape g = gemv_shape(M, a.K);
    if constexpr (M == 1) {   // gemv_lds_bytes admits at most two steps per wave for M = 1
        if (g.spw == 1) return launch_gemv_t<M, XBF16, YT, 1, S8, 2>(a, g);
        return launch_gemv_t<M, XBF16, YT, 2, S8, 3>(a, g);
    } else {
        switch (g.spw) {
        case 1: return launch_gemv_t<M, XBF16, YT, 1, S8, 2>(a, g);
        case 2: return launch_gemv_t<M, XBF16, YT, 2, S8, 3>(a, g);
        case 3: return launch_gemv_t<M, XBF16, YT, 3, S8, 3>(a, g);
        default: return launch_gemv_t<M, XBF16, YT, 4, S8, 3>(a, g);
        }
    }
}

template <int M, bool XBF16, bool S8>
hipError_t launch_gemv_y(const GemmArgs &a) {
    switch (a.y_dtype) {
    case 0: return launch_gemv_s<M, XBF16, 0, S8>(a);
    case 1: return launch_gemv_s<M, XBF16, 1, S8>(a);
    default: return launch_gemv_s<M, XBF16, 2, S8>(a);
    }
}

template <int M>
hipError_t launch_gemv_m(const GemmArgs &a) {
    if (a.Q != nullptr) return a.x_dtype == 1 ? launch_gemv_y<M, true, true>(a) : launch_gemv_y<M, false, true>(a);
    return a.x_dtype == 1 ? launch_gemv_y<M, true, false>(a) : launch_gemv_y<M, false, false>(a);
}


// ---- short-step variant: M <= 4, N <= 5120, K <= 5120 (M = 1) or 8192;
//      also M = 2, K <= 8192, N >= 12288 ----
// Up to N = 5120 the layer's rows fit in one workgroup per CU: a workgroup
// covers 4 JR rows with JR = ceil(N / 1024) <= 5, so there are at most 256
// workgroups and each CU gets the same share (8-row workgroups would leave
// half of the CUs with one workgroup more than the others).  On the wide
// M = 2 layers the workgroups keep 20 rows (JR = 5) and run in several
// rounds, N / 20 of them.  Each wave takes one 512-weight step,
// so a workgroup has ceil(K / 512) <= 16 waves, and lane (r, kk) reads the
// 8 code bytes (32 weights) of chunk kk of rows n0 + 4j + r.  The step's
// activations (32 blocks of 16) are staged pair-interleaved in the wave's
// LDS slice by lanes r = 0, 1; lanes r = 2, 3 write the same words again.
// Measured at M = 1, bf16 (graph-timed, weights rotated), against the kernel
// above: 5120 -> 5120 3.98 -> 3.94 us (4.22 -> 4.07 with bench.py's 2 GB
// of rotated weights), 5120 -> 3072 3.58 -> 3.32, 2048 -> 5120 3.01 -> 2.88;
// at K = 8192 or N = 6144 it was no better or slower.  From M = 2 it beat
// the 8-row kernel and the MFMA kernel on every shape tried up to K = 8192
// (e.g. M = 3, 6144 -> 5120: 8.77 -> 5.53 us), hence the longer K there.
constexpr int SHORT_STEP = 512;   // weights of one row per wave
constexpr int SHORT_CHUNK = 32;   // weights per lane per row (8 bytes)
constexpr int SHORT_PIECES = 64;  // 16-byte activation pieces per step
constexpr int64_t kShortMaxK = 5120;       // M = 1
constexpr int64_t kShortMaxKWide = 8192;   // M = 2 .. 4
constexpr int64_t kShortMaxN = 5120;
constexpr int64_t kShortMaxM = 4;
// M = 2 also takes it on layers of at least 12288 rows (2.4 or more rounds of
// 20-row workgroups over the CUs), against the 8-row kernel: 5120 -> 15360
// 10.53 -> 8.9 us, 5120 -> 17408 11.78 -> 10.7 us; with 1.2 rounds
// (5120 -> 6144) it was slower, 5.10 -> 6.45 us, and at M = 3, 4 it lost to
// the MFMA kernel at every N past 5120 tried.
constexpr int64_t kShortMinNRounds = 12288;

template <int M, bool XBF16, int YT, int JR, bool S8>
__global__ __launch_bounds__(64 * ((M == 1 ? kShortMaxK : kShortMaxKWide) / SHORT_STEP)) void gemv_short_kernel(
    const uint16_t *__restrict__ X, const uint8_t *__restrict__ P, const uint16_t *__restrict__ S,
    const int8_t *__restrict__ Q, const float *__restrict__ R, void *__restrict__ Y, int N, int K) {
    constexpr int ROWS = 4 * JR;
    extern __shared__ uint4 lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int r = lane >> 4;
    const int kk = lane & 15;
    const int n0 = blockIdx.x * ROWS;
    const int64_t row_bytes = K >> 2;
    const int groups = K >> 7;
    const int nchunks = K / SHORT_CHUNK;
    uint4 *xw = lds + wave * (M * SHORT_PIECES);
    float *red = reinterpret_cast<float *>(lds + nwaves * (M * SHORT_PIECES));

    // ---- 1. loads, all unconditional at clamped in-bounds addresses: the
    //         activation block this lane stages first, then codes and scales
    //         (the scheduling barriers keep that order, so the staging waits
    //         for the activations alone) ----
    const int blk = 2 * kk + (r & 1);   // 16-element block of this step
    const int64_t xoff = min((int64_t)wave * SHORT_STEP + blk * 16, (int64_t)K - 16);
    uint4 xraw[M][2];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const uint4 *xs = reinterpret_cast<const uint4 *>(X + (int64_t)m * K + xoff);
        xraw[m][0] = xs[0];
        xraw[m][1] = xs[1];
    }
    __builtin_amdgcn_sched_barrier(0);
    const int c = min(wave * 16 + kk, nchunks - 1);
    uint2 code[JR];
    uint32_t sbits[JR];
#pragma unroll
    for (int j = 0; j < JR; ++j) {
        const int64_t n = min(n0 + 4 * j + r, N - 1);
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(P + n * row_bytes + (int64_t)c * 8));
        code[j] = make_uint2(v[0], v[1]);
        if constexpr (S8) sbits[j] = (uint32_t)(int32_t)Q[n * groups + (c >> 2)];
        else sbits[j] = S[n * groups + (c >> 2)];
    }
    __builtin_amdgcn_sched_barrier(0);
    // S8: the row factor multiplies the finished row sum; the threads that
    // store rows fetch it now, off the critical path
    float rowf = 1.f;
    if constexpr (S8) {
        if (tid < ROWS * M) rowf = R[min(n0 + tid % ROWS, N - 1)];
    }

    // ---- 2. stage the step's activations, pair-interleaved ----
#pragma unroll
    for (int m = 0; m < M; ++m) {
        uint32_t pr[8];
        interleave16(xraw[m][0], xraw[m][1], pr);
        uint4 *dst = xw + m * SHORT_PIECES;
        dst[(2 * (r & 1)) * 16 + kk] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
        dst[(2 * (r & 1) + 1) * 16 + kk] = make_uint4(pr[4], pr[5], pr[6], pr[7]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- 3. decode + sign-select accumulate; the chunk lies inside one
    //         128-weight block, whose scale (halved: the operands are +-2)
    //         multiplies the chunk's sum ----
    const uint32_t kact = opaque_mask(wave * 16 + kk < nchunks);
    uint4 xq[M][4];   // per row m: blocks 2 kk (pieces 0, 1) and 2 kk + 1 (pieces 2, 3)
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) xq[m][q] = xw[m * SHORT_PIECES + q * 16 + kk];
    float acc[JR][M];
#pragma unroll
    for (int j = 0; j < JR; ++j) {
        const uint64_t v = sign_nz_fields64((uint64_t)code[j].x | ((uint64_t)code[j].y << 32));
        float part[M];
#pragma unroll
        for (int m = 0; m < M; ++m) part[m] = 0.f;
        auto pair = [&](auto ic) {
            constexpr int I = decltype(ic)::value;
            uint32_t lo, hi;
            weight_pairs2<I>(v, lo, hi);   // code word 0 -> block 2 kk, word 1 -> block 2 kk + 1
#pragma unroll
            for (int m = 0; m < M; ++m) {   // each decoded pair feeds every activation row
                part[m] = dot2<XBF16>(lo, (&xq[m][I >> 2].x)[I & 3], part[m]);
                part[m] = dot2<XBF16>(hi, (&xq[m][2 + (I >> 2)].x)[I & 3], part[m]);
            }
        };
        pair(std::integral_constant<int, 0>{});
        pair(std::integral_constant<int, 1>{});
        pair(std::integral_constant<int, 2>{});
        pair(std::integral_constant<int, 3>{});
        pair(std::integral_constant<int, 4>{});
        pair(std::integral_constant<int, 5>{});
        pair(std::integral_constant<int, 6>{});
        pair(std::integral_constant<int, 7>{});
        const float s = (S8 ? (float)(int32_t)sbits[j] : f16_bits_to_float((uint16_t)sbits[j])) * 0.5f;
#pragma unroll
        for (int m = 0; m < M; ++m) acc[j][m] = masked_fma(kact, s, part[m], 0.f);
    }

    // ---- 4. reduce over the 16 lanes of each DPP row, then across waves ----
#pragma unroll
    for (int j = 0; j < JR; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[j][m] = row16_sum(acc[j][m]);
    if (kk == 0) {
#pragma unroll
        for (int j = 0; j < JR; ++j)
#pragma unroll
            for (int m = 0; m < M; ++m) red[(wave * ROWS + 4 * j + r) * M + m] = acc[j][m];
    }
    __syncthreads();
    auto finish = [&](int o, float f) {   // output o = m * ROWS + row, row factor f
        const int row = o % ROWS;
        const int m = o / ROWS;
        float y = 0.f;
        for (int w = 0; w < nwaves; ++w) y += red[(w * ROWS + row) * M + m];
        if constexpr (S8) y *= f;
        const int n = n0 + row;
        if (n < N) store_out<YT>(Y, (int64_t)m * N + n, y);
    };
    if constexpr (ROWS * M <= 64) {
        if (tid < ROWS * M) finish(tid, rowf);
    } else {
        // more outputs than one wave has threads (M = 4, 20 rows, K <= 512)
        for (int o = tid; o < ROWS * M; o += blockDim.x)
            finish(o, o == tid ? rowf : (S8 ? R[min(n0 + o % ROWS, N - 1)] : 1.f));
    }
}

template <int M, bool XBF16, int YT, int JR, bool S8>
hipError_t launch_short_t(const GemmArgs &a) {
    constexpr int ROWS = 4 * JR;
    const int nwaves = (int)((a.K + SHORT_STEP - 1) / SHORT_STEP);
    const size_t lds = (size_t)nwaves * M * SHORT_PIECES * 16 + (size_t)nwaves * ROWS * M * sizeof(float);
    if (lds > 64 * 1024) {   // M = 4 with K > 7168: raise the dynamic-LDS limit once per device
        static std::atomic<uint64_t> done_mask{0};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const uint64_t bit = 1ull << (dev & 63);
        if (!(done_mask.load(std::memory_order_acquire) & bit)) {
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(gemv_short_kernel<M, XBF16, YT, JR, S8>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
            if (e != hipSuccess) return e;
            done_mask.fetch_or(bit, std::memory_order_acq_rel);
        }
    }
    hipLaunchKernelGGL((gemv_short_kernel<M, XBF16, YT, JR, S8>), dim3((unsigned)((a.N + ROWS - 1) / ROWS)),
                       dim3((unsigned)(64 * nwaves)), lds, a.stream, static_cast<const uint16_t *>(a.X), a.W,
                       a.S, a.Q, a.R, a.Y, (int)a.N, (int)a.K);
    return hipGetLastError();
}

template <int M, bool XBF16, int YT, bool S8>
hipError_t launch_short_j(const GemmArgs &a) {
    switch ((a.N + 1023) / 1024) {
    case 1: return launch_short_t<M, XBF16, YT, 1, S8>(a);
    case 2: return launch_short_t<M, XBF16, YT, 2, S8>(a);
    case 3: return launch_short_t<M, XBF16, YT, 3, S8>(a);
    case 4: return launch_short_t<M, XBF16, YT, 4, S8>(a);
    default: return launch_short_t<M, XBF16, YT, 5, S8>(a);
    }
}

template <int M, bool S8>
hipError_t launch_short_s(const GemmArgs &a) {
    const bool bf = a.x_dtype == 1;
    switch (a.y_dtype) {
    case 0: return bf ? launch_short_j<M, true, 0, S8>(a) : launch_short_j<M, false, 0, S8>(a);
    case 1: return bf ? launch_short_j<M, true, 1, S8>(a) : launch_short_j<M, false, 1, S8>(a);
    default: return bf ? launch_short_j<M, true, 2, S8>(a) : launch_short_j<M, false, 2, S8>(a);
    }
}

template <int M>
hipError_t launch_short_m(const GemmArgs &a) {
    return a.Q != nullptr ? launch_short_s<M, true>(a) : launch_short_s<M, false>(a);
}

hipError_t launch_short(const GemmArgs &a) {
    switch (a.M) {
    case 1: return launch_short_m<1>(a);
    case 2: return launch_short_m<2>(a);
    case 3: return launch_short_m<3>(a);
    default: return launch_short_m<4>(a);
    }
}
}  // namespace

size_t gemv_lds_bytes(int64_t M, int64_t K) {
    const GemvShape g = gemv_shape(M, K);
    // more steps per wave than the register budget holds (M = 1: K > 32768;
    // M > 1: K > 32768 as well, with 8 waves of up to 4 steps): not this kernel
    if (g.spw > (M == 1 ? 2 : 4)) return (size_t)-1;
    return g.lds;
}

bool gemv_short(int64_t M, int64_t N, int64_t K) {
    if (M == 2 && K <= kShortMaxKWide && N >= kShortMinNRounds) return true;
    return M >= 1 && M <= kShortMaxM && K <= (M == 1 ? kShortMaxK : kShortMaxKWide) && N <= kShortMaxN;
}

hipError_t launch_gemv(const GemmArgs &a) {
    if (gemv_short(a.M, a.N, a.K)) return launch_short(a);
    switch (a.M) {
    case 1: return launch_gemv_m<1>(a);
    case 2: return launch_gemv_m<2>(a);
    case 3: return launch_gemv_m<3>(a);
    default: return launch_gemv_m<4>(a);
    }
}

}  // namespace tern
