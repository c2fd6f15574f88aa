// tern_gemv_skip.hip -- decode path that skips all-zero 128-weight blocks.
//
// 2kiu.com/news/5082861 §6 proposes skipping blocks whose weights are all
// zero, to save bandwidth and compute.  tern_block_map marks each (row,
// block) holding a nonzero weight; this kernel follows the layout of
// tern_gemv.hip but loads and decodes only the marked blocks.
#include <hip/hip_runtime.h>

#include <atomic>

#include "tern_device.h"
#include "tern_gemv_common.h"
#include "tern_kernels.h"

namespace tern {

namespace {

using namespace gemv;

constexpr int SKIP_ROWS = 16;     // most rows per workgroup of the zero-block skipping kernel (JS = 4 per team)

// MAP[n, w] bit b marks block 32w + b of row n as holding a nonzero weight
// (tern_block_map).  The work layout is that of the dense decode kernel in
// tern_gemv.hip, with 4 JS rows per workgroup (JS = 2 or 4); per wave step,
// each 16-lane team (rows n0 + 4j + r, j = 0..JS-1, chunks kk = 0..15) lists
// the (row, chunk) pairs whose block is marked, in (j, chunk) order, through
// a wave-private LDS slot, and lane kk then takes items kk, kk+16, ... of the
// list (JS passes).  Only listed chunks load codes and scales, and a pass
// that no lane of the wave needs is not executed: zero blocks cost neither
// bytes nor decode work.  Each lane still accumulates per row j, so the
// reduction is the dense kernel's.
template <int M, bool XBF16, int YT, int SPW, int JS>
__global__ __launch_bounds__(M == 1 ? 1024 : 512) void gemv_skip_kernel(const uint16_t *__restrict__ X,
                                                                      const uint8_t *__restrict__ P,
                                                                      const uint16_t *__restrict__ S,
                                                                      const uint32_t *__restrict__ MAP,
                                                                      void *__restrict__ Y, int N, int K) {
    extern __shared__ uint4 lds[];
    constexpr int ROWS = 4 * JS;      // JS rows per 16-lane team
    static_assert(ROWS <= SKIP_ROWS, "rows per workgroup");
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
    const int mapw = (groups + 31) >> 5;
    uint4 *xw = lds + wave * (SPW * M * PIECES);
    float *red = reinterpret_cast<float *>(lds + nwaves * (SPW * M * PIECES));
    uint8_t *slots = reinterpret_cast<uint8_t *>(red + nwaves * ROWS * M) + wave * (SPW * 4 * 64);
    const int s_begin = wave * SPW;
    const int nchunks = K / CHUNK;

    // ---- 1. activation loads and the map words of this wave's steps ----
    uint4 xraw[SPW][M][2];
    uint32_t mw[SPW][JS];
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
        for (int j = 0; j < JS; ++j) mw[si][j] = MAP[(int64_t)min(n0 + 4 * j + r, N - 1) * mapw + (st >> 2)];
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
        for (int j = 0; j < JS; ++j) {
            // a bit operation on an opaque mask: a short-circuit condition let
            // the compiler move the map load into a branch, behind the staging
            const uint32_t ok = opaque_mask(chunk_ok && n0 + 4 * j + r < N);
            const bool act = ((mw[si][j] >> (((st & 3) << 3) + (kk >> 1))) & ok & 1u) != 0u;
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
    // Every lane issues its loads of every pass: a lane without an item reads
    // the first bytes of P and S instead, one cache line the whole GPU
    // shares, so it adds no HBM traffic.  (Loads under a per-lane condition
    // made the compiler wait for each pass's loads before issuing the next
    // pass's: one memory round trip per pass.)
    uint4 code[SPW][JS];
    uint32_t sbits[SPW][JS];
    uint32_t item[SPW][JS];
    bool pass[SPW][JS];
#pragma unroll
    for (int si = 0; si < SPW; ++si) {
#pragma unroll
        for (int t = 0; t < JS; ++t) {
            const bool mine = kk + 16 * t < count[si];
            pass[si][t] = __ballot(mine) != 0;   // uniform: does any lane of the wave need pass t?
            item[si][t] = mine ? slots[(si * 4 + r) * 64 + kk + 16 * t] : 0u;
            const int j = item[si][t] >> 4;
            const int c = (s_begin + si) * 16 + (item[si][t] & 15);
            const int64_t n = n0 + 4 * j + r;
            const uint8_t *pa = mine ? P + n * row_bytes + (int64_t)c * 16 : P;
            const uint16_t *sa = mine ? S + n * groups + (c >> 1) : S;
            code[si][t] = *reinterpret_cast<const uint4 *>(pa);
            sbits[si][t] = *sa;
        }
    }

    // ---- 5. decode + accumulate the listed chunks into their rows ----
    float acc[JS][M];
#pragma unroll
    for (int j = 0; j < JS; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[j][m] = 0.f;
#pragma unroll
    for (int si = 0; si < SPW; ++si) {
#pragma unroll
        for (int t = 0; t < JS; ++t) {
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
                for (int jj = 0; jj < JS; ++jj)
                    acc[jj][m] = (mine && j == jj) ? fmaf(s, part[0], acc[jj][m]) : acc[jj][m];
                if constexpr (M > 1) __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- 6. reduce as the dense kernel ----
#pragma unroll
    for (int j = 0; j < JS; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[j][m] = row16_sum(acc[j][m]);
    if (kk == 0) {
#pragma unroll
        for (int j = 0; j < JS; ++j)
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

// LDS of the skipping kernel: staged activations, its 16-row reduction
// buffer and the per-wave item lists
size_t skip_lds(const GemvShape &g, int64_t M) {
    return (size_t)g.nwaves * g.spw * M * PIECES * 16 + (size_t)g.nwaves * SKIP_ROWS * M * sizeof(float) +
           (size_t)g.nwaves * g.spw * 4 * 64;
}

template <int M, bool XBF16, int YT, int SPW, int JS>
hipError_t launch_skip_t(const GemmArgs &a, const uint32_t *map, const GemvShape &g) {
    auto kern = gemv_skip_kernel<M, XBF16, YT, SPW, JS>;
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
    const dim3 grid((unsigned)((a.N + 4 * JS - 1) / (4 * JS)));
    const dim3 block((unsigned)(64 * g.nwaves));
    hipLaunchKernelGGL(kern, grid, block, lds, a.stream, static_cast<const uint16_t *>(a.X), a.W, a.S, map, a.Y,
                       (int)a.N, (int)a.K);
    return hipGetLastError();
}

template <int M, bool XBF16, int YT, int JS>
hipError_t launch_skip_j(const GemmArgs &a, const uint32_t *map, const GemvShape &g) {
    if constexpr (M == 1) {
        if (g.spw == 1) return launch_skip_t<M, XBF16, YT, 1, JS>(a, map, g);
        return launch_skip_t<M, XBF16, YT, 2, JS>(a, map, g);
    } else {
        switch (g.spw) {
        case 1: return launch_skip_t<M, XBF16, YT, 1, JS>(a, map, g);
        case 2: return launch_skip_t<M, XBF16, YT, 2, JS>(a, map, g);
        case 3: return launch_skip_t<M, XBF16, YT, 3, JS>(a, map, g);
        default: return launch_skip_t<M, XBF16, YT, 4, JS>(a, map, g);
        }
    }
}

template <int M, bool XBF16, int YT>
hipError_t launch_skip_s(const GemmArgs &a, const uint32_t *map) {
    const GemvShape g = gemv_shape(M, a.K);
    // 16-row workgroups when there are at least 1024 of them, else 8-row
    // ones (more workgroups to spread over the CUs).  At 50% zero blocks,
    // skip / dense: 5120 -> 5120 1.30 (16 rows) / 1.15 (8 rows), 17408 ->
    // 5120 1.44 / 1.23, 5120 -> 17408 1.10 / 1.23.
    if (a.N >= 1024 * 16) return launch_skip_j<M, XBF16, YT, 4>(a, map, g);
    return launch_skip_j<M, XBF16, YT, 2>(a, map, g);
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
    default: return hipErrorInvalidValue;   // the skipping kernel serves M <= 2
    }
}

}  // namespace tern
