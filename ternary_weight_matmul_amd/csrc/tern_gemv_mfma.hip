// tern_gemv_mfma.hip -- decode-path kernel (M <= 4) whose sign-select sums
// run on the matrix cores: Y[M,N] = X[M,K] . (T*S)^T.
//
// Method (2kiu.com/news/5082861): the weights stay packed and stream once
// (§4.1, second route); inside each 128-weight block the ternary signs add,
// subtract or skip activations, and the block sum is multiplied by the
// block's fp16 scale at the block boundary (§1.1, §4.1 third route, §4.2);
// activations and scales stay on chip (§4.2, §4.3); the code bytes arrive in
// wide vector loads (§4.3, third version).
//
// Why matrix cores at M <= 4.  The weights are decoded, as in the VALU GEMV,
// into pairs of 16-bit values +-2 / 0 (tern_device.h), one shift and one AND
// per pair.  Those pairs are exactly representable operands of
// v_mfma_f32_4x4x4_16b_{bf16,f16}, so the add / subtract / skip sums (exact
// products, fp32 accumulation) can run on the matrix pipe instead of as packed
// dots on the VALU.  That takes about a third of the decode kernel's VALU
// work away; the VALU is the nearer limit of the decode shapes, not HBM.
//
// The 4x4x4_16b shape fits the decode layout: its 16 blocks are 16
// independent 4x4x4 products, lane 4b + j holding row j of block b's A and
// column j of its B (4 K values each), and D VGPR i of that lane is
// D_b[i][j].  Here block b is a 64-weight segment of K, B column j is weight
// row j of a 4-row quad and A row i is activation row i, so
//   D_b[i][j] = sum over the segment of X[i,k] * 2t[4q+j,k]
// and each lane owns complete partial sums for its (segment, row): no lane of
// the block mixes weights of two scale blocks, the scale is applied per lane,
// and the matrix pipe never sums across segments.
//
// Work layout.
//   * unit = (quad q, step s): rows 4q..4q+3 x K range [1024 s, 1024 s + 1024);
//     lane 4b + j loads the 16 code bytes of row 4q + j at K offset
//     1024 s + 64 b (one 16-byte load; each row's 16 lanes read 256 contiguous
//     bytes), then runs 16 MFMAs (4 code words x 4 pairs of pairs);
//   * one workgroup of 16 waves per CU takes a contiguous range of quads (so
//     N = 5120 and 17408 give every CU exactly 5 or 17 quads); its units are
//     numbered quad-major and wave w takes units [UPW w, UPW w + UPW);
//   * all 16 waves first stage the workgroup's activations, X[0..M)[0..K),
//     pair-interleaved (tern_device.h) into LDS, with every code and scale
//     load of the wave already issued behind them;
//   * per unit: D = 16 MFMAs (two accumulator chains), acc += s * D per lane;
//     when the wave leaves a quad, acc is summed over the 4 segments of each
//     16-lane row (DPP row rotations) and the 4 row sums are written to LDS;
//     after a barrier each output adds its quad's row sums and wave partials
//     in a fixed order (deterministic; no atomics, no workspace), halves the
//     sum (the operands are +-2) and rounds it to the output type.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "tern_device.h"
#include "tern_kernels.h"

namespace tern {

namespace {

constexpr int QSTEP = 1024;            // weights of a row per unit
constexpr int QSEG = 64;               // weights per lane per unit (16 code bytes)
constexpr int QSEGS = QSTEP / QSEG;    // segments per step (= MFMA blocks)
constexpr int QWAVES = 16;             // waves per workgroup
constexpr int QTHREADS = 64 * QWAVES;
constexpr int QMAX_UPW = 8;            // units per wave at most
constexpr int QCHUNKS = QSEG * 2 / 16; // 16-byte LDS chunks per segment and row (8)

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// D += A * B over the 16 blocks of a 4x4x4 product: A = {a0, a1}, B = {b0, b1},
// four 16-bit values each.
template <bool BF16>
__device__ __forceinline__ float4_t mfma4x4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, float4_t c) {
    const uint64_t a = (uint64_t)a0 | ((uint64_t)a1 << 32);
    const uint64_t b = (uint64_t)b0 | ((uint64_t)b1 << 32);
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(short4_t, a), __builtin_bit_cast(short4_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, a), __builtin_bit_cast(half4_t, b), c,
                                                  0, 0, 0);
}

// LDS layout of the staged activations: [row m][step s][chunk c][segment b]
// x 16 bytes.  Chunk c (0..7) of a 64-weight segment holds pair-interleaved
// words 4c..4c+3 of its 128 bytes.  The 16 segments an A read covers (lanes
// 4b + j, same c) are 256 contiguous bytes: no bank conflict whatever the
// bank count.  Chunk c sits at the lane's base plus the immediate 256 c, a
// step at +2048 s.  Rows are 64 bytes further apart than their size, so the 4
// rows of M = 4 fall on different banks too.
constexpr int QSTEP_BYTES = QCHUNKS * QSEGS * 16;   // 2048
__device__ __forceinline__ int row_pitch(int steps) { return steps * QSTEP_BYTES + 64; }

// Range-checked buffer resource over [base, base + bytes): loads past the end
// return zeros (gfx9 raw buffer, stride 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// All ones where c holds, else zero, hidden from the optimiser so that a
// mask built from it stays a bit operation instead of becoming a branch.
__device__ __forceinline__ uint32_t opaque_lanes(bool c) {
    uint32_t m = c ? ~0u : 0u;
    asm("" : "+v"(m));
    return m;
}

// Sum of x over the 4 segments b of each 16-lane row that share j = lane & 3
// (lane 4b + j, b = 4 row + b'): two DPP row rotations.  The 4 rows' sums are
// added in LDS by the output pass.
__device__ __forceinline__ float row_segment_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true));
    return x;
}

// UPW: units per wave; BPT: 16-element activation blocks staged per thread.
template <int M, bool XBF16, bool S8, int UPW, int BPT>
__global__ __launch_bounds__(QTHREADS) void gemv_mfma_kernel(const uint16_t *__restrict__ X,
                                                             const uint8_t *__restrict__ P,
                                                             const uint16_t *__restrict__ S,
                                                             const int8_t *__restrict__ Q,
                                                             const float *__restrict__ R, void *__restrict__ Y,
                                                             int y_dtype, int N, int K, int nquads, int kmax) {
    extern __shared__ uint4 lds[];
    const int steps = (K + QSTEP - 1) / QSTEP;
    const int nseg = steps * QSEGS;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: unit arithmetic on the scalar unit
    const int b = lane >> 2;   // segment of the step (MFMA block)
    const int j = lane & 3;    // weight row within the quad (B column), activation row of A
    const int G = gridDim.x;
    const int qa = (int)((int64_t)blockIdx.x * nquads / G);
    const int qb = (int)((int64_t)(blockIdx.x + 1) * nquads / G);
    const int U = (qb - qa) * steps;          // units of this workgroup, quad-major
    const int ufirst = wave * UPW;            // this wave's units: [ufirst, ufirst + UPW) below U
    const int64_t row_bytes = K >> 2;
    const int groups = K >> 7;
    const int pitch = row_pitch(steps);
    char *ldsb = reinterpret_cast<char *>(lds);
    float4_t *red = reinterpret_cast<float4_t *>(ldsb + M * pitch);   // [QWAVES][kmax][4 lane rows][4 j]

    // ---- 1. loads.  Activation blocks first (they gate the staging), then
    //         the wave's code and scale loads.  All are unconditional: units
    //         past U repeat the last unit (their results are never used).
    //         Codes and scales are buffer loads over this workgroup's rows;
    //         each unit rebases the resource on the scalar unit, so a lane's
    //         offset is the same for every unit, and rows past N read zeros
    //         (range check).  Segments past K read whatever bytes follow
    //         (finite codes and scales): their activations are zero. ----
    const int xblocks = K >> 4;                 // 16-element blocks per activation row
    const int pblocks = nseg * (QSEG / 16);     // ... including the zero padding up to whole steps
    uint4 xraw[BPT][2];
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int t = tid + i * QTHREADS;
        const int m = min(t / pblocks, M - 1);
        const int blk = min(t % pblocks, xblocks - 1);
        const uint4 *src = reinterpret_cast<const uint4 *>(X + (int64_t)m * K + (int64_t)blk * 16);
        xraw[i][0] = src[0];
        xraw[i][1] = src[1];
    }
    // keep the activation loads ahead of the code loads: the staging waits for them alone
    __builtin_amdgcn_sched_barrier(0);
    const int wg_rows = min(4 * qb, N) - 4 * qa;
    const uint8_t *Pwg = P + (int64_t)4 * qa * row_bytes;
    const uint32_t pbytes = (uint32_t)(wg_rows * row_bytes);
    const char *Swg = S8 ? reinterpret_cast<const char *>(Q + (int64_t)4 * qa * groups)
                         : reinterpret_cast<const char *>(S + (int64_t)4 * qa * groups);
    constexpr int SB = S8 ? 1 : 2;              // bytes per scale
    const uint32_t sbytes = (uint32_t)(wg_rows * groups * SB);
    const int pofs = j * (int)row_bytes + b * 16;                 // this lane's code bytes within a unit
    const int sofs = (j * groups + (b >> 1)) * SB;               // this lane's scale within a unit
    uint4 code[UPW];
    uint32_t sbits[UPW];
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
        const int u = min(ufirst + i, U - 1);
        const int ql = u / steps;                 // scalar (u is wave-uniform)
        const int s = u - ql * steps;
        const uint32_t pu = (uint32_t)(4 * ql * row_bytes + s * (QSTEP / 4));
        const uint32_t su = (uint32_t)((4 * ql * groups + s * (QSTEP / 128)) * SB);
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(buffer_rsrc(Pwg + pu, pbytes - pu), pofs, 0, 2 /* nt */));
        code[i] = make_uint4(v[0], v[1], v[2], v[3]);
        if constexpr (S8)
            sbits[i] = (uint32_t)(int32_t)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(buffer_rsrc(Swg + su, sbytes - su),
                                                                                     sofs, 0, 0);
        else
            sbits[i] = __builtin_amdgcn_raw_buffer_load_b16(buffer_rsrc(Swg + su, sbytes - su), sofs, 0, 0);
    }

    // ---- 2. stage the activations pair-interleaved; the padding past K up to
    //         whole steps is zero, so segments past K add nothing ----
    //         (written without a branch: a conditional store would let the
    //         compiler sink the activation loads behind the code loads, and
    //         the staging would then wait for every code load; threads past
    //         the last block write a spare LDS slot instead)
    const int spare = M * pitch + QWAVES * kmax * 256;   // two chunks past the reduction area
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int t = tid + i * QTHREADS;
        const bool valid = t < M * pblocks;
        const int m = min(t / pblocks, M - 1);
        const int blk = t % pblocks;
        const uint32_t keep = opaque_lanes(blk < xblocks);   // zero padding past K
        uint32_t pr[8];
        interleave16(xraw[i][0], xraw[i][1], pr);
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] &= keep;
        const int st = blk >> 6;           // step
        const int sg = (blk >> 2) & 15;    // segment within the step
        const int w = blk & 3;             // 16-element block within the segment: chunks 2w, 2w + 1
        const int base = m * pitch + st * QSTEP_BYTES + (2 * w) * 256 + sg * 16;
        const int c0 = valid ? base : spare;
        const int c1 = valid ? base + 256 : spare + 16;
        *reinterpret_cast<uint4 *>(ldsb + c0) = make_uint4(pr[0], pr[1], pr[2], pr[3]);
        *reinterpret_cast<uint4 *>(ldsb + c1) = make_uint4(pr[4], pr[5], pr[6], pr[7]);
    }
    __syncthreads();

    // ---- 3. units: decode, 16 MFMAs, scale per lane; flush per quad ----
    // Lanes j >= M feed A rows whose outputs are never stored; they read row
    // M - 1 again (the same addresses as lane j = M - 1 of their segment, so
    // no extra bank conflict).
    const char *abase = ldsb + min(j, M - 1) * pitch + b * 16;   // + 2048 s + 256 c
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;
    const int u0 = min(ufirst, U - 1);
    const int qfirst = u0 / steps;   // local quad of the wave's first unit
    int ql = qfirst;                 // (quad, step) of unit i, advanced without divisions
    int s = u0 - qfirst * steps;
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
        const int u = ufirst + i;
        if (i > 0) {
            if (++s == steps) {
                s = 0;
                ++ql;
            }
        }
        if (u < U) {
            uint4 a[QCHUNKS];
            const char *src = abase + s * QSTEP_BYTES;
#pragma unroll
            for (int c = 0; c < QCHUNKS; ++c) a[c] = *reinterpret_cast<const uint4 *>(src + c * 256);
            const uint64_t v01 = sign_nz_fields64<true>((uint64_t)code[i].x | ((uint64_t)code[i].y << 32));
            const uint64_t v23 = sign_nz_fields64<true>((uint64_t)code[i].z | ((uint64_t)code[i].w << 32));
            float4_t d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
            // pairs 2t', 2t'+1 of code word w against activation words 2t', 2t'+1 of block w
            auto quarter = [&](auto tc) {
                constexpr int T = decltype(tc)::value;   // t' = 0..3
                uint32_t p0a, p1a, p2a, p3a, p0b, p1b, p2b, p3b;
                weight_pairs2<2 * T, true>(v01, p0a, p1a);
                weight_pairs2<2 * T + 1, true>(v01, p0b, p1b);
                weight_pairs2<2 * T, true>(v23, p2a, p3a);
                weight_pairs2<2 * T + 1, true>(v23, p2b, p3b);
                constexpr int cc = T >> 1;            // chunk within the block
                constexpr int e = (T & 1) * 2;        // first word within the chunk
                d0 = mfma4x4<XBF16>((&a[0 + cc].x)[e], (&a[0 + cc].x)[e + 1], p0a, p0b, d0);
                d1 = mfma4x4<XBF16>((&a[4 + cc].x)[e], (&a[4 + cc].x)[e + 1], p2a, p2b, d1);
                d0 = mfma4x4<XBF16>((&a[2 + cc].x)[e], (&a[2 + cc].x)[e + 1], p1a, p1b, d0);
                d1 = mfma4x4<XBF16>((&a[6 + cc].x)[e], (&a[6 + cc].x)[e + 1], p3a, p3b, d1);
            };
            quarter(std::integral_constant<int, 0>{});
            quarter(std::integral_constant<int, 1>{});
            quarter(std::integral_constant<int, 2>{});
            quarter(std::integral_constant<int, 3>{});
            const float sc = S8 ? (float)(int32_t)sbits[i] : f16_bits_to_float((uint16_t)sbits[i]);
#pragma unroll
            for (int m = 0; m < M; ++m) acc[m] = fmaf(sc, d0[m] + d1[m], acc[m]);
            // leave the quad: the next unit belongs to another quad, or this is the wave's last
            if (i == UPW - 1 || u + 1 >= U || s == steps - 1) {
                float4_t r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < M; ++m) r[m] = row_segment_sum(acc[m]);
                if ((lane & 12) == 0) red[((wave * kmax + (ql - qfirst)) * 4 + (lane >> 4)) * 4 + j] = r;
#pragma unroll
                for (int m = 0; m < M; ++m) acc[m] = 0.f;
            }
        }
    }
    // every code and scale register is read again here, so the compiler
    // cannot sink a load into its unit's conditional block (behind the
    // staging barrier); it stays among the loads issued at the start
#pragma unroll
    for (int i = 0; i < UPW; ++i) asm volatile("" ::"v"(code[i].x), "v"(sbits[i]));
    __syncthreads();

    // ---- 4. outputs: sum the wave partials of each row in wave order ----
    const int nrows = 4 * (qb - qa);
    for (int o = tid; o < nrows * M; o += QTHREADS) {
        const int m = o / nrows;
        const int rl = o % nrows;
        const int qo = rl >> 2;
        const int n = 4 * qa + rl;
        if (n >= N) continue;
        const int w0 = (qo * steps) / UPW;
        const int w1 = (qo * steps + steps - 1) / UPW;
        float y = 0.f;
        for (int w = w0; w <= w1; ++w) {
            const int qf = min(w * UPW, U - 1) / steps;   // first local quad of wave w
            const float4_t *p = red + (w * kmax + (qo - qf)) * 16 + (rl & 3);
            y += ((p[0][m] + p[4][m]) + (p[8][m] + p[12][m]));   // the 4 lane rows (segments 0-3, ..., 12-15)
        }
        y *= 0.5f;   // the operands were +-2
        if constexpr (S8) y *= R[n];
        if (y_dtype == 2) store_out<2>(Y, (int64_t)m * N + n, y);
        else if (y_dtype == 1) store_out<1>(Y, (int64_t)m * N + n, y);
        else store_out<0>(Y, (int64_t)m * N + n, y);
    }
}

struct QuadShape {
    int steps, grid, upw, bpt, kmax;
    size_t lds;
};

QuadShape quad_shape(int64_t M, int64_t N, int64_t K) {
    QuadShape g{};
    g.steps = (int)((K + QSTEP - 1) / QSTEP);
    const int64_t nquads = (N + 3) / 4;
    // one workgroup per CU (256), more rounds of them only when a workgroup
    // would hold more than QWAVES * QMAX_UPW units
    int64_t grid = 256;
    while ((nquads + grid - 1) / grid * g.steps > (int64_t)QWAVES * QMAX_UPW && grid < nquads) grid += 256;
    g.grid = (int)(grid < nquads ? grid : nquads);
    const int64_t qmax = (nquads + g.grid - 1) / g.grid;      // quads of the largest workgroup
    const int64_t units = qmax * g.steps;
    int upw = (int)((units + QWAVES - 1) / QWAVES);
    if (upw > QMAX_UPW) upw = 0;                              // does not fit (K too long)
    else if (upw == 5) upw = 6;
    else if (upw == 7) upw = 8;
    g.upw = upw;
    const int64_t blocks = M * g.steps * (QSTEP / 16);
    const int64_t bpt = (blocks + QTHREADS - 1) / QTHREADS;
    g.bpt = bpt <= 1 ? 1 : bpt <= 2 ? 2 : bpt <= 4 ? 4 : bpt <= 6 ? 6 : 0;   // 8 would spill
    // quads a wave touches at most: its units span ceil(upw / steps) + 1 quads
    g.kmax = upw == 0 ? 0 : (int)std::min<int64_t>(upw, (upw + g.steps - 1) / g.steps + 1);
    g.lds = (size_t)M * (g.steps * QSTEP_BYTES + 64) + (size_t)QWAVES * g.kmax * 16 * 16 + 2 * 16;
    return g;
}

template <int M, bool XBF16, bool S8, int UPW, int BPT>
hipError_t launch_qt(const GemmArgs &a, const QuadShape &g) {
    auto kern = gemv_mfma_kernel<M, XBF16, S8, UPW, BPT>;
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
    hipLaunchKernelGGL(kern, dim3((unsigned)g.grid), dim3(QTHREADS), g.lds, a.stream,
                       static_cast<const uint16_t *>(a.X), a.W, a.S, a.Q, a.R, a.Y, a.y_dtype, (int)a.N, (int)a.K,
                       (int)((a.N + 3) / 4), g.kmax);
    return hipGetLastError();
}

template <int M, bool XBF16, bool S8, int UPW>
hipError_t launch_qb(const GemmArgs &a, const QuadShape &g) {
    switch (g.bpt) {
    case 1: return launch_qt<M, XBF16, S8, UPW, 1>(a, g);
    case 2: return launch_qt<M, XBF16, S8, UPW, 2>(a, g);
    case 4: return launch_qt<M, XBF16, S8, UPW, 4>(a, g);
    default: return launch_qt<M, XBF16, S8, UPW, 6>(a, g);
    }
}

template <int M, bool XBF16, bool S8>
hipError_t launch_qu(const GemmArgs &a, const QuadShape &g) {
    switch (g.upw) {
    case 1: return launch_qb<M, XBF16, S8, 1>(a, g);
    case 2: return launch_qb<M, XBF16, S8, 2>(a, g);
    case 3: return launch_qb<M, XBF16, S8, 3>(a, g);
    case 4: return launch_qb<M, XBF16, S8, 4>(a, g);
    case 6: return launch_qb<M, XBF16, S8, 6>(a, g);
    default: return launch_qb<M, XBF16, S8, 8>(a, g);
    }
}

template <int M>
hipError_t launch_qm(const GemmArgs &a, const QuadShape &g) {
    const bool bf = a.x_dtype == 1;
    if (a.Q != nullptr) return bf ? launch_qu<M, true, true>(a, g) : launch_qu<M, false, true>(a, g);
    return bf ? launch_qu<M, true, false>(a, g) : launch_qu<M, false, false>(a, g);
}

}  // namespace

bool gemv_mfma_fits(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || M > 4 || N < 1 || K < QSEG) return false;
    const QuadShape g = quad_shape(M, N, K);
    return g.upw > 0 && g.bpt > 0 && g.lds <= 160 * 1024;
}

hipError_t launch_gemv_mfma(const GemmArgs &a) {
    const QuadShape g = quad_shape(a.M, a.N, a.K);
    if (g.upw == 0 || g.bpt == 0 || g.lds > 160 * 1024) return hipErrorInvalidValue;
    switch (a.M) {
    case 1: return launch_qm<1>(a, g);
    case 2: return launch_qm<2>(a, g);
    case 3: return launch_qm<3>(a, g);
    default: return launch_qm<4>(a, g);
    }
}

}  // namespace tern
