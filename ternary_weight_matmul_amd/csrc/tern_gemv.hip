// tern_gemv.hip -- decode-path kernel (small M): Y[M,N] = X[M,K] . (T*S)^T.
//
// Method (2kiu.com/news/5082861): weights stay packed (§4.1, second route);
// inside a 128-weight block the signs are accumulated with add / subtract /
// skip and the block sum is multiplied by its fp16 scale at the block
// boundary (§1.1, §4.1 third route, §4.2); activations and scales are kept
// on chip, never re-read from memory in the inner loop (§4.2, §4.3); wide
// vector loads of the packed bytes (§4.3, third version).
//
// Work layout (one workgroup = 4 JR output rows x all of K; JR = 1 or 2):
//   * a wave "step" covers 4 JR rows x 1024 weights: lane = 16*r + kk; for
//     j < JR the lane loads 16 bytes (64 weights) of row n0 + 4j + r at K
//     offset step*1024 + 64*kk, so every load instruction reads four
//     256-byte contiguous row segments;
//   * the waves of a workgroup (up to 16 for M = 1, 8 otherwise) split the K
//     steps.  Each wave first issues all of its weight and scale loads, then
//     stages the activations of its own steps into a wave-private LDS slice
//     (pair-interleaved, see tern_device.h; the four lanes that share a
//     64-weight chunk stage a quarter each), then decodes and accumulates as
//     the loads land;
//   * each lane keeps one fp32 partial per (row, m); it is summed over the
//     16 lanes of its DPP row, then across the waves through LDS in a fixed
//     order (deterministic; no atomics, no workspace).
//   * small workgroups (8 rows, or 4 when K > 16384 at M = 1) spread a
//     layer's rows over many CUs, so no CU runs much more than its share.
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "tern_device.h"
#include "tern_kernels.h"

namespace tern {

namespace {

constexpr int SKIP_ROWS = 16;     // rows per workgroup of the zero-block skipping kernel
constexpr int STEP = 1024;        // weights of one row per wave step
constexpr int CHUNK = 64;         // weights per lane per row per step (16 bytes)
constexpr int PIECES = 128;       // 16-byte activation pieces per (step, m): 16 chunks x 8

// 16 code bytes that are read exactly once per product: a non-temporal load
// (the weights stream through; nothing else reuses their cache lines).
__device__ __forceinline__ uint4 load_codes(const uint8_t *p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Sums of 2t*x over one lane's 64 weights (one 16-byte code vector) against
// the pair-interleaved activation pieces xq[m][0..7] of the same chunk, for
// every activation row m: each decoded pair feeds M packed dots.
template <int M, bool BF16>
__device__ __forceinline__ void chunk_dot(const uint4 &code, const uint4 (&xq)[M][8], float (&part)[M]) {
    const uint64_t a = sign_nz_fields64((uint64_t)code.x | ((uint64_t)code.y << 32));
    const uint64_t b = sign_nz_fields64((uint64_t)code.z | ((uint64_t)code.w << 32));
    auto step = [&](auto ic) {
        constexpr int I = decltype(ic)::value;
        constexpr int q = I >> 2;
        constexpr int e = I & 3;
        uint32_t p0, p1, p2, p3;
        weight_pairs2<I>(a, p0, p1);   // words 0, 1
        weight_pairs2<I>(b, p2, p3);   // words 2, 3
#pragma unroll
        for (int m = 0; m < M; ++m) {
            part[m] = dot2<BF16>(p0, (&xq[m][0 + q].x)[e], part[m]);
            part[m] = dot2<BF16>(p1, (&xq[m][2 + q].x)[e], part[m]);
            part[m] = dot2<BF16>(p2, (&xq[m][4 + q].x)[e], part[m]);
            part[m] = dot2<BF16>(p3, (&xq[m][6 + q].x)[e], part[m]);
        }
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    step(std::integral_constant<int, 4>{});
    step(std::integral_constant<int, 5>{});
    step(std::integral_constant<int, 6>{});
    step(std::integral_constant<int, 7>{});
}

// S8: scales are int8 codes Q[N,K/128] times a per-row fp32 factor R[N]
// (the int8-scale variant) instead of fp16 values S[N,K/128].
// JR: rows per 16-lane team; a workgroup covers ROWS = 4 JR rows.
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

    // activation rows are taken one at a time (a row's 32 activation words in
    // registers); for M > 1 each code word is decoded once per row, which
    // keeps the register footprint of M = 1
    constexpr int MC = 1;
#pragma unroll
    for (int si = 0; si < SPW; ++si) {
        const bool kact = (s_begin + si) * 16 + kk < nchunks;   // this lane's chunk lies inside K
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
                    acc[j][mb + m] = kact ? fmaf(s, part[m], acc[j][mb + m]) : acc[j][mb + m];
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

// ---------------------------------------------------------------------------
// Zero-block skipping (2kiu.com/news/5082861 §6 proposes skipping blocks that
// are entirely zero to save bandwidth and compute).  MAP[n, w] bit b marks
// block 32w + b of row n as holding a nonzero weight (tern_block_map).  The
// work layout is the kernel above; per wave step, each 16-lane team (rows
// n0 + 4j + r, j = 0..3, chunks kk = 0..15) lists the (row, chunk) pairs whose
// block is marked, in (j, chunk) order, through a wave-private LDS slot, and
// lane kk then takes items kk, kk+16, kk+32, kk+48 of the list.  Only listed
// chunks load codes and scales, and a pass that no lane of the wave needs is
// not executed: zero blocks cost neither bytes nor decode work.  Each lane
// still accumulates per row j, so the reduction is the dense kernel's.
template <int M, bool XBF16, int YT, int SPW>
__global__ __launch_bounds__(M == 1 ? 1024 : 512) void gemv_skip_kernel(const uint16_t *__restrict__ X,
                                                                      const uint8_t *__restrict__ P,
                                                                      const uint16_t *__restrict__ S,
                                                                      const uint32_t *__restrict__ MAP,
                                                                      void *__restrict__ Y, int N, int K) {
    extern __shared__ uint4 lds[];
    const int nsteps = (K + STEP - 1) / STEP;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int r = lane >> 4;
    const int kk = lane & 15;
    const int n0 = blockIdx.x * SKIP_ROWS;
    const int64_t row_bytes = K >> 2;
    const int groups = K >> 7;
    const int mapw = (groups + 31) >> 5;
    uint4 *xw = lds + wave * (SPW * M * PIECES);
    float *red = reinterpret_cast<float *>(lds + nwaves * (SPW * M * PIECES));
    uint8_t *slots = reinterpret_cast<uint8_t *>(red + nwaves * SKIP_ROWS * M) + wave * (SPW * 4 * 64);
    const int s_begin = wave * SPW;
    const int nchunks = K / CHUNK;

    // ---- 1. activation loads and the map words of this wave's steps ----
    uint4 xraw[SPW][M][2];
    uint32_t mw[SPW][4];
#pragma unroll
    for (int si = 0; si < SPW; ++si) {
        const int c = min((s_begin + si) * 16 + kk, nchunks - 1);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint4 *src = reinterpret_cast<const uint4 *>(X + (int64_t)m * K + (int64_t)c * CHUNK + r * 16);
            xraw[si][m][0] = src[0];
            xraw[si][m][1] = src[1];
        }
        const int st = min(s_begin + si, nsteps - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) mw[si][j] = MAP[(int64_t)min(n0 + 4 * j + r, N - 1) * mapw + (st >> 2)];
    }

    // ---- 2. stage the activations (as the dense kernel) ----
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

    // ---- 3. list each team's marked (row, chunk) pairs: item byte = 16 j + chunk ----
    int count[SPW];
#pragma unroll
    for (int si = 0; si < SPW; ++si) {
        const int st = s_begin + si;
        const bool chunk_ok = st < nsteps && st * 16 + kk < nchunks;
        int base = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool act = chunk_ok && n0 + 4 * j + r < N &&
                             ((mw[si][j] >> (((st & 3) << 3) + (kk >> 1))) & 1u);
            const uint32_t tb = (uint32_t)(__ballot(act) >> (16 * r)) & 0xFFFFu;
            if (act) slots[(si * 4 + r) * 64 + base + __popc(tb & ((1u << kk) - 1u))] = (uint8_t)(16 * j + kk);
            base += __popc(tb);
        }
        count[si] = base;
    }
    // activations and lists are private to this wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- 4. codes and scales of the listed chunks only ----
    uint4 code[SPW][4];
    uint32_t sbits[SPW][4];
    uint32_t item[SPW][4];
    bool pass[SPW][4];
#pragma unroll
    for (int si = 0; si < SPW; ++si) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bool mine = kk + 16 * t < count[si];
            pass[si][t] = __ballot(mine) != 0;   // uniform: does any lane of the wave need pass t?
            item[si][t] = mine ? slots[(si * 4 + r) * 64 + kk + 16 * t] : 0u;
            if (mine) {
                const int j = item[si][t] >> 4;
                const int c = (s_begin + si) * 16 + (item[si][t] & 15);
                const int64_t n = n0 + 4 * j + r;
                code[si][t] = *reinterpret_cast<const uint4 *>(P + n * row_bytes + (int64_t)c * 16);
                sbits[si][t] = S[n * groups + (c >> 1)];
            }
        }
    }

    // ---- 5. decode + accumulate the listed chunks into their rows ----
    float acc[4][M];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[j][m] = 0.f;
#pragma unroll
    for (int si = 0; si < SPW; ++si) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (!pass[si][t]) continue;
            const bool mine = kk + 16 * t < count[si];
            const int j = item[si][t] >> 4;
            const int cl = item[si][t] & 15;
            const float s = f16_bits_to_float((uint16_t)sbits[si][t]) * 0.5f;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                uint4 xq[1][8];
                const uint4 *src = xw + (si * M + m) * PIECES;
#pragma unroll
                for (int q = 0; q < 8; ++q) xq[0][q] = src[q * 16 + cl];
                float part[1] = {0.f};
                chunk_dot<1, XBF16>(code[si][t], xq, part);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    acc[jj][m] = (mine && j == jj) ? fmaf(s, part[0], acc[jj][m]) : acc[jj][m];
                if constexpr (M > 1) __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- 6. reduce as the dense kernel ----
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[j][m] = row16_sum(acc[j][m]);
    if (kk == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int m = 0; m < M; ++m) red[(wave * SKIP_ROWS + 4 * j + r) * M + m] = acc[j][m];
    }
    __syncthreads();
    if (tid < SKIP_ROWS * M) {
        const int row = tid % SKIP_ROWS;
        const int m = tid / SKIP_ROWS;
        float y = 0.f;
        for (int w = 0; w < nwaves; ++w) y += red[(w * SKIP_ROWS + row) * M + m];
        const int n = n0 + row;
        if (n < N) store_out<YT>(Y, (int64_t)m * N + n, y);
    }
}

struct GemvShape {
    int nsteps, spw, nwaves, jr;
    size_t lds;
};

GemvShape gemv_shape(int64_t M, int64_t K) {
    GemvShape g;
    g.nsteps = (int)((K + STEP - 1) / STEP);
    const int max_waves = M == 1 ? 16 : 8;  // (M > 1 needs the 256-register budget of <= 512 threads)
    g.spw = (g.nsteps + max_waves - 1) / max_waves;
    if (g.spw < 1) g.spw = 1;
    g.nwaves = (g.nsteps + g.spw - 1) / g.spw;
    // rows per team: 2 (8-row workgroups); 1 when one row's K already gives
    // every wave two steps (M = 1, K > 16384).  Measured on the decode shapes:
    // fewer rows per workgroup spread the rows of a layer over more CUs.
    g.jr = (M == 1 && g.spw >= 2) ? 1 : 2;
    g.lds = (size_t)g.nwaves * g.spw * M * PIECES * 16 + (size_t)g.nwaves * 4 * g.jr * M * sizeof(float);
    return g;
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
        return launch_gemv_t<M, XBF16, YT, 2, S8, 1>(a, g);
    } else {
        switch (g.spw) {
        case 1: return launch_gemv_t<M, XBF16, YT, 1, S8, 2>(a, g);
        case 2: return launch_gemv_t<M, XBF16, YT, 2, S8, 2>(a, g);
        case 3: return launch_gemv_t<M, XBF16, YT, 3, S8, 2>(a, g);
        default: return launch_gemv_t<M, XBF16, YT, 4, S8, 2>(a, g);
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

// LDS of the skipping kernel: staged activations, its 16-row reduction
// buffer and the per-wave item lists
size_t skip_lds(const GemvShape &g, int64_t M) {
    return (size_t)g.nwaves * g.spw * M * PIECES * 16 + (size_t)g.nwaves * SKIP_ROWS * M * sizeof(float) +
           (size_t)g.nwaves * g.spw * 4 * 64;
}

template <int M, bool XBF16, int YT, int SPW>
hipError_t launch_skip_t(const GemmArgs &a, const uint32_t *map, const GemvShape &g) {
    auto kern = gemv_skip_kernel<M, XBF16, YT, SPW>;
    const size_t lds = skip_lds(g, M);
    if (lds > 64 * 1024) {
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
    const dim3 grid((unsigned)((a.N + SKIP_ROWS - 1) / SKIP_ROWS));
    const dim3 block((unsigned)(64 * g.nwaves));
    hipLaunchKernelGGL(kern, grid, block, lds, a.stream, static_cast<const uint16_t *>(a.X), a.W, a.S, map, a.Y,
                       (int)a.N, (int)a.K);
    return hipGetLastError();
}

template <int M, bool XBF16, int YT>
hipError_t launch_skip_s(const GemmArgs &a, const uint32_t *map) {
    const GemvShape g = gemv_shape(M, a.K);
    if constexpr (M == 1) {
        if (g.spw == 1) return launch_skip_t<M, XBF16, YT, 1>(a, map, g);
        return launch_skip_t<M, XBF16, YT, 2>(a, map, g);
    } else {
        switch (g.spw) {
        case 1: return launch_skip_t<M, XBF16, YT, 1>(a, map, g);
        case 2: return launch_skip_t<M, XBF16, YT, 2>(a, map, g);
        case 3: return launch_skip_t<M, XBF16, YT, 3>(a, map, g);
        default: return launch_skip_t<M, XBF16, YT, 4>(a, map, g);
        }
    }
}

template <int M, bool XBF16>
hipError_t launch_skip_y(const GemmArgs &a, const uint32_t *map) {
    switch (a.y_dtype) {
    case 0: return launch_skip_s<M, XBF16, 0>(a, map);
    case 1: return launch_skip_s<M, XBF16, 1>(a, map);
    default: return launch_skip_s<M, XBF16, 2>(a, map);
    }
}

template <int M>
hipError_t launch_skip_m(const GemmArgs &a, const uint32_t *map) {
    return a.x_dtype == 1 ? launch_skip_y<M, true>(a, map) : launch_skip_y<M, false>(a, map);
}

}  // namespace

size_t gemv_skip_lds_bytes(int64_t M, int64_t K) {
    if (gemv_lds_bytes(M, K) == (size_t)-1) return (size_t)-1;
    return skip_lds(gemv_shape(M, K), M);
}

hipError_t launch_gemv_skip(const GemmArgs &a, const uint32_t *map) {
    switch (a.M) {
    case 1: return launch_skip_m<1>(a, map);
    case 2: return launch_skip_m<2>(a, map);
    case 3: return launch_skip_m<3>(a, map);
    default: return launch_skip_m<4>(a, map);
    }
}

size_t gemv_lds_bytes(int64_t M, int64_t K) {
    const GemvShape g = gemv_shape(M, K);
    // more steps per wave than the register budget holds (M = 1: K > 32768;
    // M > 1: K > 32768 as well, with 8 waves of up to 4 steps): not this kernel
    if (g.spw > (M == 1 ? 2 : 4)) return (size_t)-1;
    return g.lds;
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
