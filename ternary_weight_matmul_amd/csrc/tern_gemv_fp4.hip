// tern_gemv_fp4.hip -- decode-path kernel (M <= 4, bf16 activations) whose
// sign-select sums run on the matrix cores with 4-bit weight operands:
// Y[M,N] = X[M,K] . (T*S)^T.
//
// Method (2kiu.com/news/5082861): the weights stay packed and stream once
// (§4.1, second route); inside each 128-weight block the ternary signs add,
// subtract or skip activations, and the block sum is multiplied by the
// block's fp16 scale at the block boundary (§1.1, §4.1 third route, §4.2);
// activations and scales stay on chip (§4.2, §4.3).
//
// Operands (tern_fp4.h): the weights as e2m1 +-2 / 0 (B; 10 VALU operations
// per 32 weights, about a third of a lane-op per weight against 0.9 for
// 16-bit +-2 pairs, which is what lets the decode keep up with HBM), each
// bf16 activation split exactly into two e4m3 terms with a power-of-two scale
// per 32-run (A) of v_mfma_scale_f32_16x16x128_f8f6f4.  Here both terms
// enter one MFMA as separate A rows where M <= 2.  With the fp4 decode, A
// slice s carries the activations of weights 16s..16s+15 (bytes 0..15) and
// 64+16s..79+16s (bytes 16..31) of the 128-weight block, evens first, then
// odds.
//
// Work layout.
//   * B column j = 4 r + c is (row r of a 4-row quad, block c of a 512-weight
//     step): lane (p, j) loads the 8 code bytes of slice p of that block, so
//     one load instruction reads 4 rows x 128 contiguous bytes (whole cache
//     lines; measured: loads that cover only half of each row's line, as in
//     a 16-row x 64-byte pattern, stream 25-50% slower).  A row i = 4 c' +
//     2 h + m (M <= 2: one MFMA, term h and row m in it) or 4 c' + m (M = 3,
//     4: one MFMA per term, chained) carries the activations of block c', so
//     only the entries with c' = c are used: lanes with p = c, VGPR 2 h + m
//     (or m).  Each such lane multiplies them by the scale of its own (row,
//     block) and keeps a running sum.
//   * A workgroup takes Q quads (4 Q rows) and all of K; its waves split K
//     into 512-weight steps, SPW consecutive steps per wave, and each wave
//     loops over the Q quads of its steps with every code and scale load
//     issued at the start.
//   * Each wave splits and stages only its own steps' activations into a
//     wave-private LDS area laid out as the A registers (8 M images of 4
//     lanes x 32 bytes per step, then their block-scale bytes): no
//     workgroup barrier before the products, and one step's A registers
//     serve all Q quads.
//   * At the end the used lanes write their sums to LDS, the 4 blocks of a
//     row side by side; after one barrier each output adds its blocks (one
//     16-byte read per wave) and the waves in a fixed order (a rotation sum
//     over a row of 16 lanes where the rows fit the workgroup, else in wave
//     order), halves the sum (the weights are +-2) and rounds it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "tern_device.h"
#include "tern_fp4.h"
#include "tern_kernels.h"

namespace tern {

namespace {

constexpr int F_STEP = 512;          // weights of a row per step
constexpr int F_MAX_WAVES = 16;
constexpr int F_MAX_SPW = 4;
constexpr int F_IMG = 128;           // one A image: 4 lanes x 32 bytes

typedef int int8v_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// All ones where c holds, else zero, hidden from the optimiser.
__device__ __forceinline__ uint32_t opaque_lanes(bool c) {
    uint32_t m = c ? ~0u : 0u;
    asm("" : "+v"(m));
    return m;
}

// Max over the 4 lanes of a DPP quad.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
    return v;
}

// (steps per wave, quads per workgroup) pairs that are instantiated.
#define TERN_F4_TABLE(X)                                                                                       \
    X(1, 1) X(1, 2) X(1, 3) X(1, 4) X(1, 5) X(1, 6) X(1, 8) X(1, 9) X(1, 10) X(1, 12) X(1, 17) X(2, 1) X(2, 2) X(2, 3) \
    X(2, 4) X(2, 5) X(2, 6) X(2, 8) X(3, 1) X(3, 2) X(3, 3) X(3, 4) X(3, 5) X(4, 1) X(4, 2) X(4, 3) X(4, 4)

// LDS bytes of one wave's step: 8 M A images, then their scale bytes.
template <int M>
constexpr int step_lds() {
    return 8 * M * (F_IMG + 4);
}

template <int M, bool S8, int Q, int SPW>
__global__ __launch_bounds__(64 * F_MAX_WAVES) void gemv_fp4_kernel(const uint16_t *__restrict__ X,
                                                                  const uint8_t *__restrict__ P,
                                                                  const uint16_t *__restrict__ S,
                                                                  const int8_t *__restrict__ Qs,
                                                                  const float *__restrict__ Rf, void *__restrict__ Y,
                                                                  int y_dtype, int N, int K) {
    constexpr int IMGS = 8 * M;
    constexpr int SL = step_lds<M>();
    constexpr bool ONE = M <= 2;   // hi and lo terms in one MFMA
    extern __shared__ uint4 lds[];
    char *ldsb = reinterpret_cast<char *>(lds);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // waves of the workgroup, as the host sizes it (from K and SPW rather
    // than the block size, whose hidden-argument load would sit before the
    // address arithmetic of every wave)
    const int nw = ((K + F_STEP - 1) / F_STEP + SPW - 1) / SPW;
    const int p = lane >> 4;        // K slice of the lane (A and B)
    const int col = lane & 15;      // B column: 4 r + c
    const int r = col >> 2;
    const int c = col & 3;
    const int steps = (K + F_STEP - 1) / F_STEP;
    const int groups = K >> 7;
    const int row_bytes = K >> 2;
    const int n0 = blockIdx.x * 4 * Q;
    const int rows = min(4 * Q, N - n0);
    char *wimg = ldsb + wave * SL;   // one step's images, reused step after step
    // [M][nw][4 Q rows][4 blocks], then 64 + 16 Q spare words (a lane that
    // holds no used sum stores into one of them), then spare bytes
    float *red = reinterpret_cast<float *>(ldsb + nw * SL);
    char *spare_byte = reinterpret_cast<char *>(red + nw * Q * 16 * M + 64 + 16 * Q);

    // ---- 1. loads: this lane's activation octets first, then every code and
    //         scale load of the wave (rows past N read zeros; bytes past K
    //         meet zero activations, and their scales are dropped) ----
    uint4 xq[SPW][M];
#pragma unroll
    for (int st = 0; st < SPW; ++st) {
        const int k0 = min((wave * SPW + st) * F_STEP + 8 * lane, K - 8);
#pragma unroll
        for (int m = 0; m < M; ++m) xq[st][m] = *reinterpret_cast<const uint4 *>(X + (int64_t)m * K + k0);
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int SB = S8 ? 1 : 2;
    const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(P + (int64_t)n0 * row_bytes, (uint32_t)(rows * row_bytes));
    const char *sbase = S8 ? reinterpret_cast<const char *>(Qs + (int64_t)n0 * groups)
                           : reinterpret_cast<const char *>(S + (int64_t)n0 * groups);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(sbase, (uint32_t)(rows * groups * SB));
    // per step, the scales go out before the codes: the wait counter counts
    // loads in order, so quad q's MFMA then waits for code q alone, not for
    // every code load issued before a later scale
    uint2 code[SPW][Q];
    uint32_t sbits[SPW][Q];
#pragma unroll
    for (int st = 0; st < SPW; ++st) {
        const int s = min(wave * SPW + st, steps - 1);
        const int blk = min(4 * s + c, groups - 1);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int soff = ((4 * q + r) * groups + blk) * SB;
            if constexpr (S8)
                sbits[st][q] = (uint32_t)(int32_t)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(rs, soff, 0, 0);
            else
                sbits[st][q] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int off = (4 * q + r) * row_bytes + s * (F_STEP / 4) + c * 32 + p * 8;
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rp, off, 0, 2 /* nt */));
            code[st][q] = make_uint2(v[0], v[1]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- 2. per step: split the wave's activations and stage them as A
    //         images, then read this lane's A registers and run the quads.
    //         Staging: lane t holds octet t of the step: block g = t / 16,
    //         32-run u = (t / 4) % 4 of the block (its weights 32 u .. 32 u +
    //         31, the K slots of B lane group u), octet o = t % 4 of the run.
    //         Run u's 32 slots are A lanes 2 (u % 2) and 2 (u % 2) + 1, bytes
    //         16 (u / 2) .. +15: the octet's evens at byte 4 (o % 2) of lane
    //         2 (u % 2) + o / 2, its odds 8 bytes further.  The run's scale is
    //         byte u of the image's scale word.  A DPP quad holds one run.
    //         Products: A lane (p, i) takes image (c', h, m) of its row i, the
    //         32 bytes of lane p; rows m >= M read row M - 1's image (MFMA
    //         rows are independent, and those result rows are never used). ----
    const int sg = lane >> 4;
    const int su = (lane >> 2) & 3;
    const int so = lane & 3;
    const int loff = (2 * (su & 1) + (so >> 1)) * 32 + 16 * (su >> 1) + 4 * (so & 1);
    const int ca = col >> 2;                       // A block of the lane's row
    const int ha = ONE ? (col >> 1) & 1 : 0;
    const int ma = ONE ? (col & 1) : (col & 3);
    const int mc = min(ma, M - 1);
    float acc[Q][M];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[q][m] = 0.f;
#pragma unroll
    for (int st = 0; st < SPW; ++st) {
        const int s = wave * SPW + st;
        if (SPW > 1 && s >= steps) break;   // wave-uniform
        if (st > 0) {
            // the previous step's A reads are done before its images are overwritten
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        const uint32_t keep = opaque_lanes(s * F_STEP + 8 * lane < K);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            uint4 xv = xq[st][m];
            xv.x &= keep;
            xv.y &= keep;
            xv.z &= keep;
            xv.w &= keep;
            uint32_t eh, el;   // the 32-run's hi and lo scale exponents
            split_exponents(quad_max(max_mag8(xv)), eh, el);
            uint32_t he, ho, le, lo;
            split8(xv, eh, el, he, ho, le, lo);
            const int ih = (sg * 2 + 0) * M + m;
            const int il = (sg * 2 + 1) * M + m;
            *reinterpret_cast<uint32_t *>(wimg + ih * F_IMG + loff) = he;
            *reinterpret_cast<uint32_t *>(wimg + ih * F_IMG + loff + 8) = ho;
            *reinterpret_cast<uint32_t *>(wimg + il * F_IMG + loff) = le;
            *reinterpret_cast<uint32_t *>(wimg + il * F_IMG + loff + 8) = lo;
            // one lane of the quad writes the run's scale bytes (the others a
            // spare byte: no branch around the stores)
            *(so == 0 ? wimg + IMGS * F_IMG + ih * 4 + su : spare_byte) = (char)eh;
            *(so == 0 ? wimg + IMGS * F_IMG + il * 4 + su : spare_byte) = (char)el;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        int8v_t a[2];
        uint32_t sa[2];
#pragma unroll
        for (int h = 0; h < (ONE ? 1 : 2); ++h) {
            const int img = (ca * 2 + (ONE ? ha : h)) * M + mc;
            const uint4 d0 = *reinterpret_cast<const uint4 *>(wimg + img * F_IMG + p * 32);
            const uint4 d1 = *reinterpret_cast<const uint4 *>(wimg + img * F_IMG + p * 32 + 16);
            a[h] = (int8v_t){(int)d0.x, (int)d0.y, (int)d0.z, (int)d0.w, (int)d1.x, (int)d1.y, (int)d1.z, (int)d1.w};
            sa[h] = (unsigned char)wimg[IMGS * F_IMG + img * 4 + p];
        }
        const bool blk_ok = 4 * s + c < groups;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const float4_t z = {0.f, 0.f, 0.f, 0.f};
            const uint4 bw = fp4_weights(code[st][q].x, code[st][q].y);
            float4_t d = mfma_f8f4(a[0], bw, z, sa[0]);
            if constexpr (!ONE) d = mfma_f8f4(a[1], bw, d, sa[1]);
            float sc = S8 ? (float)(int32_t)sbits[st][q] : f16_bits_to_float((uint16_t)sbits[st][q]);
            sc = blk_ok ? sc : 0.f;
#pragma unroll
            for (int m = 0; m < M; ++m) acc[q][m] = fmaf(sc, ONE ? d[m] + d[2 + m] : d[m], acc[q][m]);
        }
    }
#pragma unroll
    for (int st = 0; st < SPW; ++st)
#pragma unroll
        for (int q = 0; q < Q; ++q) asm volatile("" ::"v"(code[st][q].x), "v"(sbits[st][q]));

    // ---- 4. the used sums sit in the lanes with p = c (block c of row r,
    //         column 4 r + c): each writes its sum to LDS at [m][wave][row][c]
    //         (the other lanes into a spare word, so every lane stores and no
    //         MFMA sits under a partial EXEC mask); after the barrier each
    //         output reads its 4 blocks as one 16-byte word per wave ----
    // (the index is chosen with a mask the compiler cannot see through, so
    // the store stays one branch-free instruction)
    const int hmask = (int)opaque_lanes(p == c);
    const int spare_at = nw * Q * 16 * M + lane;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        // one select per activation row; the quads then store at constant offsets
        const int base = spare_at + ((((m * nw + wave) * Q * 4 + r) * 4 + c - spare_at) & hmask);
#pragma unroll
        for (int q = 0; q < Q; ++q) red[base + 16 * q] = acc[q][m];
    }
    __syncthreads();
    // Each output's partials (one float4 of 4 block sums per wave) are summed
    // in a fixed order.  When a row of 16 lanes per output fits the
    // workgroup in one pass, lane w of the row reads wave w's float4 and the
    // row adds by rotation, the row's first lane storing; otherwise one lane
    // per output adds the waves in turn.  Measured: the rows took 5120 ->
    // 5120 from 3.82 to 3.69 us at M = 1; with many outputs (M = 4, 17 quads:
    // 7 passes) they were 10% slower than one lane per output.
    auto finish = [&](int m, int rr, float y) {
        const int n = n0 + rr;
        if (n >= N) return;
        y *= 0.5f;   // the weights were +-2
        if constexpr (S8) y *= Rf[n];
        if (y_dtype == 2) store_out<2>(Y, (int64_t)m * N + n, y);
        else if (y_dtype == 1) store_out<1>(Y, (int64_t)m * N + n, y);
        else store_out<0>(Y, (int64_t)m * N + n, y);
    };
    const float4_t *red4 = reinterpret_cast<const float4_t *>(red);
    if (Q * M <= nw) {   // uniform: 4 Q M outputs x 16 lanes fit the 64 nw lanes
        const int o = tid >> 4;      // a row of 16 lanes shares o
        const int w = tid & 15;
        const int m = o / (4 * Q);
        const int rr = o - m * 4 * Q;
        float y = 0.f;
        if (o < 4 * Q * M && w < nw) {
            const float4_t v = red4[(m * nw + w) * 4 * Q + rr];
            y = (v[0] + v[1]) + (v[2] + v[3]);
        }
        y = row16_sum(y);
        if (o < 4 * Q * M && w == 0) finish(m, rr, y);
    } else {
        for (int o = tid; o < 4 * Q * M; o += 64 * nw) {
            const int m = o / (4 * Q);
            const int rr = o - m * 4 * Q;
            const float4_t *pp = red4 + m * nw * 4 * Q + rr;
            float y = 0.f;
            for (int w = 0; w < nw; ++w) {
                const float4_t v = pp[w * 4 * Q];
                y += (v[0] + v[1]) + (v[2] + v[3]);
            }
            finish(m, rr, y);
        }
    }
}

struct F4Shape {
    int steps, spw, nw, q, grid;
    size_t lds;
};

// Instantiated (steps per wave, quads) pairs, minus the two that spill
// registers at this M, 9 quads (one step per wave) where M > 1, and 12 quads
// (one step per wave) at M = 1: measured slower than 9 or 8 quads on every
// width tried (M = 1, K = 5120: 8.76 / 8.64 / 13.2 us at 17408 / 15360 /
// 34816 rows, against 6.71 / 6.21 / 11.0), though the tile model prefers it
// at 34816.
bool f4_instantiated(int64_t M, int spw, int q) {
    bool in = false;
#define TERN_F4_CASE(SP, QQ) in = in || (spw == SP && q == QQ);
    TERN_F4_TABLE(TERN_F4_CASE)
#undef TERN_F4_CASE
    return in && !(M == 1 && spw == 1 && (q == 17 || q == 12)) && !(M == 4 && spw == 2 && q == 8) && !(M > 1 && q == 9);
}

size_t f4_lds(int64_t M, int nw, int q) {
    return (size_t)nw * 8 * M * (F_IMG + 4) + (size_t)nw * q * 16 * M * 4 + (64 + 16 * (size_t)q) * 4 + 16;
}

F4Shape f4_shape(int64_t M, int64_t N, int64_t K) {
    F4Shape g{};
    g.steps = (int)((K + F_STEP - 1) / F_STEP);
    g.spw = (g.steps + F_MAX_WAVES - 1) / F_MAX_WAVES;
    g.nw = (g.steps + g.spw - 1) / g.spw;
    // Quads per workgroup.  The busiest CU runs ceil(grid / CUs) workgroups
    // of Q quads each, plus about one quad's worth of per-workgroup work
    // (staging, reduction): pick the Q with the least of that, the larger Q
    // on ties.  Measured at M = 1 (rows 5120 / 17408): the best Q of a sweep
    // over 2..16 was also the model's choice, 5 / 6 (4.16 / 7.35 us); at
    // 17408 -> 5120, 5 (7.04 us against 9.7 for 2).  Nine quads, added
    // later, put 5120 -> 17408 in two rounds of workgroups instead of three:
    // 6.88 -> 6.78 us at M = 1 (in-process A/B); at M = 3 it was 1% slower,
    // so it serves M = 1 only.
    constexpr int64_t kCUs = 256;
    const int64_t quads = (N + 3) / 4;
    int64_t best = -1;
    for (int q = 1; q <= 17; ++q) {
        if (!f4_instantiated(M, g.spw, q) || f4_lds(M, g.nw, q) > 160 * 1024) continue;
        const int64_t grid = (quads + q - 1) / q;
        const int64_t cost = (grid + kCUs - 1) / kCUs * (q + 1);
        if (best < 0 || cost <= best) {
            best = cost;
            g.q = q;
        }
    }
    if (best < 0) return g;   // q = 0: nothing fits
    g.grid = (int)((quads + g.q - 1) / g.q);
    g.lds = f4_lds(M, g.nw, g.q);
    return g;
}

template <int M, bool S8, int Q, int SPW>
hipError_t launch_f4t(const GemmArgs &a, const F4Shape &g) {
    auto kern = gemv_fp4_kernel<M, S8, Q, SPW>;
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
                       static_cast<const uint16_t *>(a.X), a.W, a.S, a.Q, a.R, a.Y, a.y_dtype, (int)a.N, (int)a.K);
    return hipGetLastError();
}

template <int M, bool S8>
hipError_t launch_f4s(const GemmArgs &a, const F4Shape &g) {
#define TERN_F4_CASE(SP, QQ) \
    if (g.spw == SP && g.q == QQ) return launch_f4t<M, S8, QQ, SP>(a, g);
    TERN_F4_TABLE(TERN_F4_CASE)
#undef TERN_F4_CASE
    return hipErrorInvalidValue;
}

template <int M>
hipError_t launch_f4m(const GemmArgs &a, const F4Shape &g) {
    return a.Q != nullptr ? launch_f4s<M, true>(a, g) : launch_f4s<M, false>(a, g);
}

}  // namespace

bool gemv_fp4_fits(int64_t M, int64_t N, int64_t K, int x_dtype) {
    if (x_dtype != 1 || M < 1 || M > 4 || N < 1 || K < 128) return false;
    const F4Shape g = f4_shape(M, N, K);
    return g.spw <= F_MAX_SPW && g.q > 0;
}

hipError_t launch_gemv_fp4(const GemmArgs &a) {
    if (!gemv_fp4_fits(a.M, a.N, a.K, a.x_dtype)) return hipErrorInvalidValue;
    const F4Shape g = f4_shape(a.M, a.N, a.K);
    switch (a.M) {
    case 1: return launch_f4m<1>(a, g);
    case 2: return launch_f4m<2>(a, g);
    case 3: return launch_f4m<3>(a, g);
    default: return launch_f4m<4>(a, g);
    }
}

}  // namespace tern
