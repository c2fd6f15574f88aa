// tern_gemv_b16.hip -- decode-path kernel for batches of up to 16 activation
// rows, on the 16x16x32 matrix-core instruction.
//
// Method (2kiu.com/news/5082861): the weights stay packed in memory and are
// decoded on chip (§4.1); each code selects add, subtract or skip of its
// activation (§3.1), here as a +-2 / 0 operand of a matrix-core product; the
// scale of a 128-weight block is applied once, at the block boundary, in fp32
// (§4.2, §4.3).
//
// Why a kernel of its own.  With 5 to 16 activation rows every weight meets
// several rows, so the sign-select sums are a small dense contraction, but
// the weights are still read once and dominate the bytes.  The 16-row tiles
// of the batched kernel stage the activations through LDS behind a
// workgroup barrier per iteration and re-stage them for every 32 output
// columns; here each wave stages its own activations, one group at a time,
// and uses them for up to 64 output columns, and the only workgroup
// barriers are the two of the final reduction.
//
// Layout.  A workgroup owns NB column blocks (16 NB consecutive weight rows)
// over all of K.  Its waves split K in steps of 512 weights (128 code bytes of
// a row): wave w takes steps w, w + nw, w + 2 nw, ...  Per step:
//   * codes: per column block two 16-byte loads per lane, each instruction
//     reading 8 rows x 128 contiguous bytes (whole lines), stored into the
//     wave's own LDS image of the block (16 rows x 128 bytes, 16-byte pieces
//     XOR-swizzled by the row) in a transposed order: the 8-byte unit (K
//     slice u, group b) of a row sits at unit index 4u + b, so lane l reads,
//     for group b, the 8 code bytes of its MFMA column (row l%16) and its K
//     slice (weights 32(l/16) .. +32 of the group) as one 8-byte LDS read;
//   * activations, per group: four loads per lane, each instruction reading
//     4 rows x 256 contiguous bytes (rows past M read row M-1 again and feed
//     only output rows that are never stored), one group ahead of their use,
//     staged in the wave's activation tile (16 rows x 256 bytes, 16-byte
//     chunks XOR-swizzled by the row); lane l reads back the K slice of its
//     MFMA row l%16 (weights 32(l/16) .. +32 of the group) and
//     pair-interleaves it; the words serve all NB column blocks.  Loaded
//     straight into each lane's fragment instead (16 rows x four 16-byte
//     pieces per instruction), the kernel took 21.3 against 16.9 us at
//     M = 16, 5120 -> 17408;
//   * decode, per column block and group: the 8 code bytes become 16 words of
//     +-2 / 0 pairs (weights i, i+8 of each 16; tern_device.h), the B
//     operands of 4 MFMAs whose A operands are the matching interleaved
//     activation pairs; their fp32 sum is scaled by the group's scale;
//   * v_mfma_f32_16x16x32_{bf16,f16}: lane l gives A[l%16][8(l/16)+e] and
//     B[8(l/16)+e][l%16] and receives D[4(l/16)+i][l%16].
// All loads are issued unconditionally, in the order their data is used, so
// the compiler can count the loads in flight; a load with nothing to fetch
// (past a workgroup's rows, past K, or the prefetch after a wave's last
// step) gets an offset past its buffer and returns zero without reading
// memory, so a step's groups past K get a zero scale and zero activations.
// Finally each wave writes its partial tiles to LDS and the workgroup sums
// them over the waves in a fixed order, halves (the weights were +-2),
// applies the int8 row factor if any, and rounds once.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "tern_device.h"
#include "tern_kernels.h"

namespace tern {

namespace {

constexpr int B_STEP = 512;            // weights of a row per step
constexpr int B_MAX_WAVES = 12;
constexpr int B_MAX_NB = 4;
constexpr int B_ROW = 128;             // LDS bytes of a staged code row
constexpr int B_TILE = 16 * B_ROW;     // one column block's codes of one step
constexpr int B_XTILE = 16 * 256;      // one group's activations, 16 rows x 128 (bf16/fp16)

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

template <int AUX>
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Byte offset, in a staged code row image, of logical byte `byte` (0..127) of
// row `row`: the 16-byte pieces are XOR-swizzled by row / 2, so the 16 rows a
// fragment read touches (rows 2i and 2i + 1 share a 256-byte bank line) fall
// on 16 distinct 16-byte bank slots.
__device__ __forceinline__ int b_off(int row, int byte) {
    return row * B_ROW + ((((byte >> 4) ^ (row >> 1)) & 7) << 4) + (byte & 15);
}

// Byte offset of 16-byte chunk c (0..15) of row r in an activation tile:
// chunks XOR-swizzled by the row, so both the row-wise writes and the
// column-wise fragment reads touch 16 distinct bank slots per 16 lanes.
__device__ __forceinline__ int x_off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

template <bool BF16>
__device__ __forceinline__ float4_t mfma16(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t b0,
                                           uint32_t b1, uint32_t b2, uint32_t b3, float4_t c) {
    const uint4 a = make_uint4(a0, a1, a2, a3), b = make_uint4(b0, b1, b2, b3);
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, a),
                                                       __builtin_bit_cast(bf168_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    }
}

template <bool XBF16, bool S8, int NB>
__global__ __launch_bounds__(64 * B_MAX_WAVES) void gemv_b16_kernel(const uint16_t *__restrict__ X,
                                                                 const uint8_t *__restrict__ P,
                                                                 const uint16_t *__restrict__ S,
                                                                 const int8_t *__restrict__ Qs,
                                                                 const float *__restrict__ Rf,
                                                                 void *__restrict__ Y, int y_dtype, int M, int N,
                                                                 int K) {
    extern __shared__ uint4 lds[];
    char *ldsb = reinterpret_cast<char *>(lds);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = blockDim.x >> 6;
    const int j = lane & 15;    // MFMA column (weight row of the block), activation row of A
    const int g = lane >> 4;    // K slice: weights 32 g .. 32 g + 31 of a group
    const int steps = (K + B_STEP - 1) / B_STEP;
    const int groups = K >> 7;
    const int row_bytes = K >> 2;
    const int n0 = blockIdx.x * 16 * NB;
    const int rows = min(16 * NB, N - n0);
    char *cimg = ldsb + wave * (NB * B_TILE + B_XTILE);
    char *ximg = cimg + NB * B_TILE;

    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(X, (uint32_t)(M * K * 2));
    const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(P + (int64_t)n0 * row_bytes, (uint32_t)(rows * row_bytes));
    constexpr int SB = S8 ? 1 : 2;
    const char *sbase = S8 ? reinterpret_cast<const char *>(Qs + (int64_t)n0 * groups)
                           : reinterpret_cast<const char *>(S + (int64_t)n0 * groups);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(sbase, (uint32_t)(rows * groups * SB));

    // code loads: lane -> row crow (and crow + 8) of a block, 16-byte piece cp
    // of the row's 128 bytes = group cp / 2, K slices 2 (cp % 2) and + 1
    const int crow = lane >> 3;
    const int cp = lane & 7;
    const int cu = 2 * (cp & 1), cg = cp >> 1;
    const int wofs[2][2] = {{b_off(crow, 8 * (cu * 4 + cg)), b_off(crow, 8 * ((cu + 1) * 4 + cg))},
                            {b_off(crow + 8, 8 * (cu * 4 + cg)), b_off(crow + 8, 8 * ((cu + 1) * 4 + cg))}};

    // Loads are issued in the order their data is used (the wait counter
    // counts them in order): for step s, the codes and scales of the step
    // come first, then the activations of group 0, 1, 2, 3, each group's
    // issued while the previous group computes; the next step's codes go out
    // right after the step's last activation load and its first activations
    // while group 3 computes.  A load with nothing to fetch (a step or group
    // past K) gets an offset past its buffer: it returns zero and reads no
    // memory.
    constexpr int OOB = 0x7FFFFFF0;
    uint4 cr[NB][2];
    uint32_t sr[NB][4];   // scale bits of the step's 4 groups (fp16, or sign-extended int8)
    auto load_codes = [&](int s, bool live) {
        const int base = live ? s * (B_STEP / 4) + 16 * cp : OOB;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int i = 0; i < 2; ++i) cr[nb][i] = load16<2 /* nt */>(rp, (16 * nb + crow + 8 * i) * row_bytes + base);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int soff = live && 4 * s + b < groups ? ((16 * nb + j) * groups + 4 * s + b) * SB : OOB;
                if constexpr (S8)
                    sr[nb][b] = (uint32_t)(int32_t)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(rs, soff, 0, 0);
                else
                    sr[nb][b] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff, 0, 0);
            }
        }
    };
    // activations of a group: 4 loads of 4 rows x 256 contiguous bytes
    // (lane -> row 4 q + l / 16, 16-byte chunk l % 16), staged in the wave's
    // activation tile and read back as each lane's K slice
    const int xr = lane >> 4, xc = lane & 15;
    uint4 xa[4];
    auto load_a = [&](int s, int b, bool live) {
        const int k = s * B_STEP + b * 128;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = min(4 * q + xr, M - 1);
            xa[q] = load16<0>(rx, live && k < K ? (row * K + k) * 2 + 16 * xc : OOB);
        }
    };

    float4_t acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = float4_t{0.f, 0.f, 0.f, 0.f};

    int s = wave;   // the host launches at most `steps` waves
    load_codes(s, true);
    load_a(s, 0, true);
    for (; s < steps; s += nw) {
        const int sn = s + nw;
        const bool more = sn < steps;   // wave-uniform
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            char *t = cimg + nb * B_TILE;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                *reinterpret_cast<uint2 *>(t + wofs[i][0]) = make_uint2(cr[nb][i].x, cr[nb][i].y);
                *reinterpret_cast<uint2 *>(t + wofs[i][1]) = make_uint2(cr[nb][i].z, cr[nb][i].w);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        uint32_t scur[NB][4];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int b = 0; b < 4; ++b) scur[nb][b] = sr[nb][b];
        // this wave's images are written before its own reads below
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4 *>(ximg + x_off(4 * q + xr, xc)) = xa[q];
            __builtin_amdgcn_sched_barrier(0);
            if (b < 3) load_a(s, b + 1, true);
            if (b == 2) load_codes(sn, more);
            if (b == 3) load_a(sn, 0, more);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            uint4 xs[4];   // row j, weights 32 g .. 32 g + 31 of the group
#pragma unroll
            for (int q = 0; q < 4; ++q) xs[q] = *reinterpret_cast<const uint4 *>(ximg + x_off(j, 4 * g + q));
            uint32_t a01[8], a23[8];
            interleave16(xs[0], xs[1], a01);   // {x[i], x[i+8]}, x = weights 32g .. +15 of the group
            interleave16(xs[2], xs[3], a23);   // the same for weights 32g + 16 .. +31
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const uint2 c = *reinterpret_cast<const uint2 *>(cimg + nb * B_TILE + b_off(j, 8 * (4 * g + b)));
                const uint64_t v = sign_nz_fields64<true>((uint64_t)c.x | ((uint64_t)c.y << 32));
                uint32_t lo[8], hi[8];
                weight_pairs2<0, true>(v, lo[0], hi[0]);
                weight_pairs2<1, true>(v, lo[1], hi[1]);
                weight_pairs2<2, true>(v, lo[2], hi[2]);
                weight_pairs2<3, true>(v, lo[3], hi[3]);
                weight_pairs2<4, true>(v, lo[4], hi[4]);
                weight_pairs2<5, true>(v, lo[5], hi[5]);
                weight_pairs2<6, true>(v, lo[6], hi[6]);
                weight_pairs2<7, true>(v, lo[7], hi[7]);
                float4_t d = mfma16<XBF16>(a01[0], a01[1], a01[2], a01[3], lo[0], lo[1], lo[2], lo[3],
                                           float4_t{0.f, 0.f, 0.f, 0.f});
                d = mfma16<XBF16>(a01[4], a01[5], a01[6], a01[7], lo[4], lo[5], lo[6], lo[7], d);
                d = mfma16<XBF16>(a23[0], a23[1], a23[2], a23[3], hi[0], hi[1], hi[2], hi[3], d);
                d = mfma16<XBF16>(a23[4], a23[5], a23[6], a23[7], hi[4], hi[5], hi[6], hi[7], d);
                // a group past K has scale 0 (its load read nothing)
                const float sc = S8 ? (float)(int32_t)scur[nb][b] : f16_bits_to_float((uint16_t)scur[nb][b]);
                acc[nb][0] = fmaf(sc, d[0], acc[nb][0]);
                acc[nb][1] = fmaf(sc, d[1], acc[nb][1]);
                acc[nb][2] = fmaf(sc, d[2], acc[nb][2]);
                acc[nb][3] = fmaf(sc, d[3], acc[nb][3]);
            }
        }
    }
    // keep the prefetches after the last step (they read nothing) from being
    // dropped, which would change the load counts the waits rely on
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) asm volatile("" ::"v"(cr[nb][0].x), "v"(cr[nb][1].x), "v"(sr[nb][0]), "v"(sr[nb][3]));
    asm volatile("" ::"v"(xa[0].x), "v"(xa[3].x));

    // ---- the waves' partial tiles, summed in wave order ----
    __syncthreads();   // every wave is done with its code images
    float4_t *red = reinterpret_cast<float4_t *>(ldsb);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) red[(wave * NB + nb) * 64 + lane] = acc[nb];
    __syncthreads();
    for (int o = tid; o < NB * 64; o += blockDim.x) {
        const int nb = o >> 6;
        const int l = o & 63;
        float4_t y = red[nb * 64 + l];
        for (int w = 1; w < nw; ++w) y += red[(w * NB + nb) * 64 + l];
        const int n = n0 + 16 * nb + (l & 15);
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * (l >> 4) + i;
            if (m >= M) continue;
            float v = y[i] * 0.5f;   // the weights were +-2
            if constexpr (S8) v *= Rf[n];
            if (y_dtype == 2) store_out<2>(Y, (int64_t)m * N + n, v);
            else if (y_dtype == 1) store_out<1>(Y, (int64_t)m * N + n, v);
            else store_out<0>(Y, (int64_t)m * N + n, v);
        }
    }
}

struct B16Shape {
    int nb, nw, grid;
    size_t lds;
};

// Waves: about three steps each (at most 12 waves), so each wave's loads
// for the next step overlap its work on the current one.  Column blocks
// per workgroup: the busiest CU takes ceil(grid / CUs) workgroups of NB
// blocks, plus about one block's worth of per-workgroup work (activation
// loads, reduction); the NB with the least of that, the larger NB on ties.
// Measured against a sweep of 1 .. 12 waves and NB 1 .. 4 at M = 16
// (graph-timed, weights rotated over 2 GB): 5120 -> 17408 best at 4 waves
// and NB 3 (16.9 us), 17408 -> 5120 at 12 waves and NB 2 (19.7 us), the
// rule's choices.
B16Shape b16_shape(int64_t N, int64_t K) {
    B16Shape g{};
    const int64_t steps = (K + B_STEP - 1) / B_STEP;
    g.nw = (int)std::min<int64_t>(B_MAX_WAVES, (steps + 2) / 3);
    const int64_t per_wave = (steps + g.nw - 1) / g.nw;
    g.nw = (int)((steps + per_wave - 1) / per_wave);
    constexpr int64_t kCUs = 256;
    const int64_t blocks = (N + 15) / 16;
    int64_t best = -1;
    for (int nb = 1; nb <= B_MAX_NB; ++nb) {
        if ((size_t)g.nw * (nb * B_TILE + B_XTILE) > 160 * 1024) continue;
        const int64_t grid = (blocks + nb - 1) / nb;
        const int64_t cost = (grid + kCUs - 1) / kCUs * (nb + 1);
        if (best < 0 || cost <= best) {
            best = cost;
            g.nb = nb;
        }
    }
    if (best < 0) return g;   // nb = 0: nothing fits
    g.grid = (int)((blocks + g.nb - 1) / g.nb);
    g.lds = (size_t)g.nw * (g.nb * B_TILE + B_XTILE);
    return g;
}

template <bool XBF16, bool S8, int NB>
hipError_t launch_b16t(const GemmArgs &a, const B16Shape &g) {
    auto kern = gemv_b16_kernel<XBF16, S8, NB>;
    if (g.lds > 64 * 1024) {
        // raise the dynamic-LDS limit once per device and instantiation (a
        // per-process attribute cache; not a stream operation)
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
    hipLaunchKernelGGL(kern, dim3((unsigned)g.grid), dim3(64 * g.nw), g.lds, a.stream,
                       static_cast<const uint16_t *>(a.X), a.W, a.S, a.Q, a.R, a.Y, a.y_dtype, (int)a.M, (int)a.N,
                       (int)a.K);
    return hipGetLastError();
}

template <bool XBF16, bool S8>
hipError_t launch_b16s(const GemmArgs &a, const B16Shape &g) {
    switch (g.nb) {
    case 1: return launch_b16t<XBF16, S8, 1>(a, g);
    case 2: return launch_b16t<XBF16, S8, 2>(a, g);
    case 3: return launch_b16t<XBF16, S8, 3>(a, g);
    case 4: return launch_b16t<XBF16, S8, 4>(a, g);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool gemv_b16_fits(int64_t M, int64_t N, int64_t K) {
    // K: 32-bit buffer offsets over a workgroup's 16 NB code rows and over X
    if (M < 1 || M > 16 || N < 1 || K < 128 || K > (1 << 20)) return false;
    return b16_shape(N, K).nb > 0;
}

hipError_t launch_gemv_b16(const GemmArgs &a) {
    if (!gemv_b16_fits(a.M, a.N, a.K)) return hipErrorInvalidValue;
    const B16Shape g = b16_shape(a.N, a.K);
    if (a.x_dtype == 1) return a.Q != nullptr ? launch_b16s<true, true>(a, g) : launch_b16s<true, false>(a, g);
    return a.Q != nullptr ? launch_b16s<false, true>(a, g) : launch_b16s<false, false>(a, g);
}

}  // namespace tern
