// tern_gemm_big.hip -- batched-path kernel for many activation rows (fp16 X).
//
// Same product as tern_gemm.hip, Y[M,N] = X[M,K] . (T*S)^T with the weights
// kept packed in memory and decoded on chip, one fp16 scale per 128-weight
// block (2kiu.com/news/5082861 §3.1 for the codes, §4.1-§4.3 for decoding in
// the kernel and reading each scale once per block).  With many activation
// rows the weight decode can be shared by a large tile, so this kernel is an
// LDS-staged MFMA GEMM:
//   * a workgroup of WM x WN waves computes a BM x BN tile of Y, BM = 16 MB WM,
//     BN = 16 NB WN; wave (wm, wn) owns an (16 MB) x (16 NB) sub-tile (MB x NB
//     blocks of 16 x 16, fp32 accumulators);
//   * per 64-wide K step both operands are staged in LDS in natural k order:
//     X[BM rows, 64] as read, and W[BN columns, 64] decoded once per
//     workgroup into exact fp16 products t*s (the scale with the code's sign
//     where the code is nonzero, +0 elsewhere) -- exact for every finite
//     scale, so the MFMA sums the pages' products directly;
//   * LDS rows are 128 bytes with their eight 16-byte chunks XOR-swizzled by
//     (row / 2) mod 8: the 16 lanes reading one MFMA fragment touch 64
//     distinct banks, and each 8 lanes writing (16-byte writes go 8 lanes at
//     a time) write 8 distinct chunks: 8 chunks of one X row, or one chunk of
//     8 weight columns 2 i (+1) (in the 128 x 64 tile, 4 columns, 2-way);
//   * both tiles are double-buffered in LDS, one barrier per step; an
//     iteration writes step s+1 (held in registers) to LDS, issues the global
//     loads of step s+2 (or s+3, with two register sets of staged loads) and
//     runs the MFMAs of step s, with no branches, so the decode can
//     interleave with the MFMAs and each load has one step (two) to land;
//     each group of 8 lanes reads one 128-byte row segment of X (coalesced);
//   * v_mfma_f32_16x16x32_f16: lane l supplies A[l%16][8(l/16)+e] and
//     B[8(l/16)+e][l%16], e = 0..7: one 16-byte chunk of an LDS row.
// With fewer tiles than CUs, a workgroup holds two such groups of waves
// (KG = 2), each over one half of K with its own LDS buffers; the second
// group's accumulators are added to the first's through LDS at the end.
// Workgroups are renumbered so that each XCD gets a contiguous run of tiles
// (tile_n fastest): workgroups resident on one XCD share activation rows in
// its L2.
#include <hip/hip_runtime.h>

#include "tern_device.h"
#include "tern_kernels.h"

namespace tern {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int KS = 64;       // K per step
constexpr int ROWB = 128;    // bytes per LDS row (KS fp16)

// byte offset of 16-byte chunk c of row r inside a tile
__device__ __forceinline__ int swz(int r, int c) { return r * ROWB + ((c ^ ((r >> 1) & 7)) << 4); }

template <int WM, int WN, int MB, int NB, int SETS, int KG, int YT, bool S8>
__global__ __launch_bounds__(64 * WM * WN * KG) void gemm_big_kernel(const uint16_t *__restrict__ X,
                                                                 const uint8_t *__restrict__ P,
                                                                 const uint16_t *__restrict__ S,
                                                                 const int8_t *__restrict__ Q,
                                                                 const float *__restrict__ R,
                                                                 void *__restrict__ Y, int M, int N, int K,
                                                                 int tiles_m, int tiles_n) {
    constexpr int NT = 64 * WM * WN;          // threads of one K group
    constexpr int BM = 16 * MB * WM;
    constexpr int BN = 16 * NB * WN;
    constexpr int A_TILE = BM * ROWB;
    constexpr int W_TILE = BN * ROWB;
    constexpr int AP = BM * 8 / NT;          // 16-byte X chunks per thread per step
    constexpr int RSTEP = NT / 8;            // rows between a thread's chunks
    static_assert(AP * NT == BM * 8 && AP >= 2 && AP <= 4, "two to four X chunks per thread (kept in scalars)");
    static_assert(RSTEP % 16 == 0, "swizzle must not depend on the chunk index");
    static_assert(2 * BN <= NT, "one thread per 32 decoded weights");
    static_assert(SETS == 1 || SETS == 2, "one or two register sets of staged loads");
    static_assert(KG == 1 || KG == 2, "one or two K groups");
    // per K group: [A buffer 0][A buffer 1][W buffer 0][W buffer 1]
    constexpr int GROUP_LDS = 2 * A_TILE + 2 * W_TILE;
    __shared__ __attribute__((aligned(16))) uint8_t lds_all[KG * GROUP_LDS];

    // KG = 2: two groups of WM x WN waves take the two halves of K, each with
    // its own LDS buffers; their tiles are summed through LDS at the end
    const int kg = KG == 1 ? 0 : (int)(threadIdx.x / NT);
    const int tid = KG == 1 ? (int)threadIdx.x : (int)(threadIdx.x % NT);
    uint8_t *const lds = lds_all + kg * GROUP_LDS;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave - wm * WN;
    const int li = lane & 15;
    const int lg = lane >> 4;

    const int ntiles = tiles_m * tiles_n;
    int tile = blockIdx.x;
    if (ntiles % 8 == 0) tile = (blockIdx.x % 8) * (ntiles / 8) + blockIdx.x / 8;
    const int tile_m = tile / tiles_n;
    const int tile_n = tile - tile_m * tiles_n;
    const int m0 = tile_m * BM;
    const int n0 = tile_n * BN;
    const int64_t row_bytes = K >> 2;
    const int groups = K >> 7;
    const int nsteps = K / KS / KG;  // steps of this K group (>= 2: the launcher requires K >= 128 KG)
    const int s_base = kg * nsteps;  // its first step

    // X loader: chunk j of this thread is row RSTEP j + tid/8, chunk tid%8 of the step;
    // rows past M are clamped to M-1 (read, never stored)
    const int xr = tid >> 3;
    const int xc = tid & 7;
    const uint16_t *x_src0 = X + (int64_t)min(m0 + xr, M - 1) * K + xc * 8;
    const uint16_t *x_src1 = X + (int64_t)min(m0 + RSTEP + xr, M - 1) * K + xc * 8;
    const uint16_t *x_src2 = X + (int64_t)min(m0 + (AP > 2 ? 2 : 1) * RSTEP + xr, M - 1) * K + xc * 8;
    const uint16_t *x_src3 = X + (int64_t)min(m0 + (AP > 3 ? 3 : 2) * RSTEP + xr, M - 1) * K + xc * 8;
    const int x_dst = swz(xr, xc);    // + RSTEP*ROWB j (same swizzle)

    // W loader: thread t < 2 BN decodes one column's weights 32 h .. 32 h + 31 of
    // the step.  LDS takes 16-byte writes 8 lanes (128 bytes) at a time, so
    // with BN >= 128 each 8 consecutive threads take columns 2 i (+1), i =
    // 0..7, of one 16-column block and one h: their chunks differ under the
    // row swizzle, where columns 2 i and 2 i + 1 share one.  Measured at
    // M = 2048, 5120 -> 17408: SQ_LDS_BANK_CONFLICT 15.3 M -> 0 cycles per
    // dispatch, 355.7 -> 348.1 us; the 128 x 64 tile keeps columns t / 2
    // (it was 2.7% slower remapped at M = 256).
    const bool w_role = (2 * BN == NT) || tid < 2 * BN;
    const int wc_col = BN >= 128 ? (16 * (tid >> 5) + 2 * (tid & 7) + ((tid >> 3) & 1)) % BN : (tid >> 1) % BN;
    const int wc_h = BN >= 128 ? (tid >> 4) & 1 : tid & 1;
    const int64_t wn_g = min(n0 + wc_col, N - 1);                           // clamped: never stored
    const uint8_t *w_src = P + wn_g * row_bytes + 8 * wc_h;
    const uint16_t *s_src = S + wn_g * groups;   // (S8: Q + wn_g * groups)
    const int8_t *q_src = Q + wn_g * groups;
    const int w_dst0 = swz(wc_col, 4 * wc_h + 0);
    const int w_dst1 = swz(wc_col, 4 * wc_h + 1);
    const int w_dst2 = swz(wc_col, 4 * wc_h + 2);
    const int w_dst3 = swz(wc_col, 4 * wc_h + 3);

    // staged global loads: one register set (A), or two (A, B) when SETS = 2,
    // used alternately so that each load has two iterations to land; plain
    // scalars rather than an array or struct, so that they stay in registers
    uint4 xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3;
    uint2 wca, wcb;
    uint32_t sba, sbb;
    auto load_into = [&](uint4 &x0, uint4 &x1, uint4 &x2, uint4 &x3, uint2 &wc, uint32_t &sb, int s) {
        s += s_base;
        const int64_t o = (int64_t)s * KS;
        x0 = *reinterpret_cast<const uint4 *>(x_src0 + o);
        x1 = *reinterpret_cast<const uint4 *>(x_src1 + o);
        if constexpr (AP > 2) x2 = *reinterpret_cast<const uint4 *>(x_src2 + o);
        if constexpr (AP > 3) x3 = *reinterpret_cast<const uint4 *>(x_src3 + o);
        wc = *reinterpret_cast<const uint2 *>(w_src + (int64_t)s * (KS / 4));
        if constexpr (S8) sb = (uint32_t)(int32_t)q_src[s >> 1];
        else sb = s_src[s >> 1];
    };
    auto store_x = [&](const uint4 &x0, const uint4 &x1, const uint4 &x2, const uint4 &x3, int buf) {
        uint8_t *a_t = lds + buf * A_TILE + x_dst;
        *reinterpret_cast<uint4 *>(a_t) = x0;
        *reinterpret_cast<uint4 *>(a_t + RSTEP * ROWB) = x1;
        if constexpr (AP > 2) *reinterpret_cast<uint4 *>(a_t + 2 * RSTEP * ROWB) = x2;
        if constexpr (AP > 3) *reinterpret_cast<uint4 *>(a_t + 3 * RSTEP * ROWB) = x3;
    };
    auto store_w = [&](int buf, uint2 wc, uint32_t sb) {
        if (w_role) {
            const uint64_t v = sign_nz_fields64<true>((uint64_t)wc.x | ((uint64_t)wc.y << 32));
            // S8: the block's int8 code q as an fp16 value (exact: |q| <= 127);
            // the row factor multiplies the finished sums in the epilogue
            const uint32_t sh = S8 ? (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(int32_t)sb) : sb;
            const uint32_t s2 = sh | (sh << 16);
            // products of weights (i, i+8) of code word 0 (a*) and word 1 (b*)
            uint32_t a0, a1, a2, a3, a4, a5, a6, a7, b0, b1, b2, b3, b4, b5, b6, b7;
            scaled_pairs2<0, true>(v, s2, a0, b0);
            scaled_pairs2<1, true>(v, s2, a1, b1);
            scaled_pairs2<2, true>(v, s2, a2, b2);
            scaled_pairs2<3, true>(v, s2, a3, b3);
            scaled_pairs2<4, true>(v, s2, a4, b4);
            scaled_pairs2<5, true>(v, s2, a5, b5);
            scaled_pairs2<6, true>(v, s2, a6, b6);
            scaled_pairs2<7, true>(v, s2, a7, b7);
            uint8_t *w_t = lds + 2 * A_TILE + buf * W_TILE;
            // natural order: chunk 4h = weights 0..7 of word 0, 4h+1 = 8..15, 4h+2/3 from word 1
            *reinterpret_cast<uint4 *>(w_t + w_dst0) =
                make_uint4(pair_lo(a0, a1), pair_lo(a2, a3), pair_lo(a4, a5), pair_lo(a6, a7));
            *reinterpret_cast<uint4 *>(w_t + w_dst1) =
                make_uint4(pair_hi(a0, a1), pair_hi(a2, a3), pair_hi(a4, a5), pair_hi(a6, a7));
            *reinterpret_cast<uint4 *>(w_t + w_dst2) =
                make_uint4(pair_lo(b0, b1), pair_lo(b2, b3), pair_lo(b4, b5), pair_lo(b6, b7));
            *reinterpret_cast<uint4 *>(w_t + w_dst3) =
                make_uint4(pair_hi(b0, b1), pair_hi(b2, b3), pair_hi(b4, b5), pair_hi(b6, b7));
        }
    };

    float4_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

    // fragment offsets: row li of a 16-row block, chunk 4t + lg; the swizzle
    // term depends on li only because every block starts at a multiple of 16
    const int a_off = (16 * MB * wm + li) * ROWB;
    const int b_off = 2 * A_TILE + (16 * NB * wn + li) * ROWB;
    const int f0 = ((0 + lg) ^ (li >> 1)) << 4;
    const int f1 = ((4 + lg) ^ (li >> 1)) << 4;
    // one half of a step (32 of its 64 k): fragment reads, then MB x NB MFMAs
    half8_t af[MB], bf[NB];
    auto read_frags = [&](int buf, int f) {
        const uint8_t *a_t = lds + buf * A_TILE + a_off + f;
        const uint8_t *b_t = lds + buf * W_TILE + b_off + f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bf[nb] = *reinterpret_cast<const half8_t *>(b_t + nb * 16 * ROWB);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) af[mb] = *reinterpret_cast<const half8_t *>(a_t + mb * 16 * ROWB);
    };
    auto mfmas = [&]() {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mb], bf[nb], acc[mb][nb], 0, 0, 0);
    };

    constexpr int DIST = SETS + 1;   // steps between a load and the MFMAs that use it
    load_into(xa0, xa1, xa2, xa3, wca, sba, 0);
    store_x(xa0, xa1, xa2, xa3, 0);
    store_w(0, wca, sba);
    load_into(xa0, xa1, xa2, xa3, wca, sba, 1);
    if constexpr (SETS == 2) load_into(xb0, xb1, xb2, xb3, wcb, sbb, min(2, nsteps - 1));
    __syncthreads();
    // iteration s (steps 0 .. nsteps-2): the set given holds step s+1; write it
    // to the other LDS buffer, refill the set with step s+DIST (past the end
    // it repeats step nsteps-1: in bounds, unused), then decode step s+1's
    // weights while the MFMAs of step s run: decode instructions are spread
    // between the MFMAs
    auto iter = [&](int s, uint4 &x0, uint4 &x1, uint4 &x2, uint4 &x3, uint2 &wcr, uint32_t &sbr) {
        const int buf = s & 1;
        store_x(x0, x1, x2, x3, buf ^ 1);
        const uint2 wc = wcr;
        const uint32_t sb = sbr;
        load_into(x0, x1, x2, x3, wcr, sbr, min(s + DIST, nsteps - 1));
        // first half's fragments are read before the decode writes to LDS, so
        // its MFMAs do not wait for them
        read_frags(buf, f0);
        __builtin_amdgcn_sched_barrier(0);
        store_w(buf ^ 1, wc, sb);
        mfmas();
        // spread the decode between the first half's MFMAs (they read only
        // fragments loaded above), so the SIMD's other wave can issue its
        // MFMAs while this one decodes, and vice versa
#pragma unroll
        for (int i = 0; i < MB * NB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
        read_frags(buf, f1);
        mfmas();
        __syncthreads();
    };
    int s = 0;
    if constexpr (SETS == 2) {
        for (; s + 1 < nsteps - 1; s += 2) {
            iter(s, xa0, xa1, xa2, xa3, wca, sba);
            iter(s + 1, xb0, xb1, xb2, xb3, wcb, sbb);
        }
    }
    for (; s < nsteps - 1; ++s) iter(s, xa0, xa1, xa2, xa3, wca, sba);
    read_frags((nsteps - 1) & 1, f0);
    mfmas();
    read_frags((nsteps - 1) & 1, f1);
    mfmas();

    if constexpr (KG == 2) {
        // the second K group's tile goes through LDS (its buffers are free
        // after this barrier) and the first group adds it in a fixed order
        static_assert((size_t)NT * MB * NB * 4 * sizeof(float) <= (size_t)GROUP_LDS, "reduction buffer");
        float *red = reinterpret_cast<float *>(lds_all + GROUP_LDS);
        __syncthreads();
        if (kg == 1) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) red[((mb * NB + nb) * 4 + i) * NT + tid] = acc[mb][nb][i];
        }
        __syncthreads();
        if (kg == 1) return;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mb][nb][i] += red[((mb * NB + nb) * 4 + i) * NT + tid];
    }

    // epilogue: lane l holds rows 4(l/16)+i, column l%16 of each 16 x 16 block
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = n0 + 16 * NB * wn + 16 * nb + li;
            if (n >= N) continue;
            const float rowf = S8 ? R[n] : 1.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + 16 * MB * wm + 16 * mb + 4 * lg + i;
                if (m < M) store_out<YT>(Y, (int64_t)m * N + n, S8 ? acc[mb][nb][i] * rowf : acc[mb][nb][i]);
            }
        }
}

template <int WM, int WN, int MB, int NB, int SETS, int KG = 1>
struct Tile {
    static constexpr int BM = 16 * MB * WM, BN = 16 * NB * WN;
    static int64_t count(const GemmArgs &a) { return ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN); }
    template <int YT, bool S8>
    static hipError_t launch(const GemmArgs &a) {
        const int64_t tiles_n = (a.N + BN - 1) / BN;
        const int64_t tiles_m = (a.M + BM - 1) / BM;
        if (tiles_n * tiles_m > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((gemm_big_kernel<WM, WN, MB, NB, SETS, KG, YT, S8>), dim3((unsigned)(tiles_n * tiles_m)),
                           dim3(64 * WM * WN * KG), 0, a.stream, static_cast<const uint16_t *>(a.X), a.W, a.S, a.Q, a.R, a.Y,
                           (int)a.M, (int)a.N, (int)a.K, (int)tiles_m, (int)tiles_n);
        return hipGetLastError();
    }
};

// Two load sets where the registers allow (the 256 x 256 tile would spill):
// M=256, 5120 -> 7168 runs 20% faster with them, M=2048, 5120 -> 17408 5%.
using Tile256 = Tile<2, 4, 8, 4, 1>;   // 256 x 256, 8 waves of 128 x 64, one workgroup per CU
using Tile192 = Tile<2, 4, 6, 4, 2>;   // 192 x 256, 8 waves of 96 x 64, one workgroup per CU
using Tile64 = Tile<2, 2, 4, 2, 2>;    // 128 x 64, 4 waves of 64 x 32, three workgroups per CU
using Tile64K2 = Tile<2, 2, 4, 2, 2, 2>;  // the same tile with K split over two groups of 4 waves
using Tile128K2 = Tile<2, 2, 4, 4, 2, 2>; // 128 x 128, two groups of 4 waves of 64 x 64 splitting K

// Pick the tile with the least estimated time: rounds of resident workgroups
// times the output area a CU covers per round, divided by the CU throughput
// measured for that tile (1.0, 0.95, 0.55 relative; 256 CUs).  Quantisation
// decides most shapes: e.g. 2048 x 17408 is 544 tiles of 256 x 256 (three
// rounds, the last 71% idle) but 748 of 192 x 256 (three rounds, 97% full).
template <int YT, bool S8>
hipError_t launch_big_y(const GemmArgs &a) {

    constexpr int64_t kCUs = 256;
    auto cost = [&](int64_t tiles, int64_t area, int64_t per_cu, double thr) {
        const int64_t rounds = (tiles + kCUs * per_cu - 1) / (kCUs * per_cu);
        return (double)rounds * (double)(area * per_cu) / thr;
    };
    const double c256 = cost(Tile256::count(a), 256 * 256, 1, 1.0);
    const double c192 = cost(Tile192::count(a), 192 * 256, 1, 0.95);
    const double c64 = cost(Tile64::count(a), 128 * 64, 3, 0.55);
    if (c64 <= c256 && c64 <= c192) {
        // fewer 128 x 64 tiles than CUs: each CU would run one 4-wave
        // workgroup (one wave per SIMD); two K groups give it eight.
        // M=256, 5120 -> 7168: 50.1 -> 40.0 us.  With more tiles than CUs
        // the 96 KB of LDS per workgroup costs more than it gains (M=256,
        // 5120 -> 17408: 87 -> 115 us), so those keep one group.
        if (Tile64::count(a) <= kCUs && a.K >= 256) return Tile64K2::launch<YT, S8>(a);
        // more 128 x 64 tiles than CUs, but 128 x 128 tiles fill 3/4 to all
        // of the CUs in one round: those, with two K groups (one 8-wave
        // workgroup per CU).  M=4096, 1024 -> 1024: 19.4 -> 17.3 us; 3072 ->
        // 1024: 46.2 -> 38.1 us.  Elsewhere they lost (e.g. 1024 -> 3072,
        // 768 tiles: 36.1 -> 45.5 us).
        const int64_t t128 = Tile128K2::count(a);
        if (t128 <= kCUs && 4 * t128 >= 3 * kCUs && a.K >= 256) return Tile128K2::launch<YT, S8>(a);
        return Tile64::launch<YT, S8>(a);
    }
    if (c192 < c256) return Tile192::launch<YT, S8>(a);
    return Tile256::launch<YT, S8>(a);
}

}  // namespace

hipError_t launch_gemm_big(const GemmArgs &a) {
    const bool s8 = a.Q != nullptr;
    switch (a.y_dtype) {
    case 0: return s8 ? launch_big_y<0, true>(a) : launch_big_y<0, false>(a);
    case 1: return s8 ? launch_big_y<1, true>(a) : launch_big_y<1, false>(a);
    default: return s8 ? launch_big_y<2, true>(a) : launch_big_y<2, false>(a);
    }
}

}  // namespace tern
