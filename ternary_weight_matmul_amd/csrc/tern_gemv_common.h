// tern_gemv_common.h -- pieces shared by the decode-path kernels
// (tern_gemv.hip, tern_gemv_skip.hip): the step geometry, the code-byte load,
// the per-chunk sign-select dot and the launch shape.  Layout and method:
// see tern_gemv.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "tern_device.h"

namespace tern {
namespace gemv {

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

// All ones where c holds, else zero, hidden from the optimiser: a select on
// it stays a bit select instead of becoming a branch (the compiler would move
// the scale load into that branch, after the activation staging, which puts a
// second memory round trip on the kernel's critical path).
__device__ __forceinline__ uint32_t opaque_mask(bool c) {
    uint32_t m = c ? ~0u : 0u;
    asm("" : "+v"(m));
    return m;
}

// fmaf(s, p, acc) where mask is all ones, acc where it is zero.
__device__ __forceinline__ float masked_fma(uint32_t mask, float s, float p, float acc) {
    const uint32_t r = __builtin_bit_cast(uint32_t, fmaf(s, p, acc));
    const uint32_t a = __builtin_bit_cast(uint32_t, acc);
    return __builtin_bit_cast(float, (r & mask) | (a & ~mask));
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

// Launch shape of a decode-path product: K steps per wave (spw), waves per
// workgroup, rows per 16-lane team of the dense kernel (jr; its workgroups
// cover 4 jr rows) and the dynamic LDS bytes (activation slices plus the
// cross-wave reduction of the dense kernel).
struct GemvShape {
    int nsteps, spw, nwaves, jr;
    size_t lds;
};

inline GemvShape gemv_shape(int64_t M, int64_t K) {
    GemvShape g;
    g.nsteps = (int)((K + STEP - 1) / STEP);
    const int max_waves = M == 1 ? 16 : 8;  // (M > 1 needs the 256-register budget of <= 512 threads)
    g.spw = (g.nsteps + max_waves - 1) / max_waves;
    if (g.spw < 1) g.spw = 1;
    g.nwaves = (g.nsteps + g.spw - 1) / g.spw;
    // rows per team: 2 (8-row workgroups); 3 when each wave takes two or more
    // steps (K > 16384 at M = 1), where the activation slice every workgroup
    // stages is large enough that sharing it over 12 rows pays for the less
    // even spread of rows over the CUs.  Measured on the decode shapes, with
    // every load issued before the activation staging: 4-row workgroups were
    // slower everywhere, 16-row ones at N = 5120.
    g.jr = g.spw >= 2 ? 3 : 2;
    g.lds = (size_t)g.nwaves * g.spw * M * PIECES * 16 + (size_t)g.nwaves * 4 * g.jr * M * sizeof(float);
    return g;
}

}  // namespace gemv
}  // namespace tern
