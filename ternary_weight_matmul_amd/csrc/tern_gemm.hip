// tern_gemm.hip -- batched-path kernel: Y[M,N] = X[M,K] . (T*S)^T on MFMA.
//
// Method (2kiu.com/news/5082861): weights stay packed in memory and are
// decoded on chip (§4.1, second route: decode inside the kernel, never a
// dequantised copy in memory); scales are read once per 128-weight block and
// kept in registers (§4.2, §4.3).  Here the decoded block feeds gfx950's
// matrix cores, because with many activation rows the work is a dense
// contraction.
//
// Tiling.  A workgroup has WN x WK waves and computes a (16*MB) x (16*NB*WN)
// tile of Y.  Wave (wn, wk) owns columns 16*NB*wn .. +16*NB of the tile and
// the K blocks kb = it*WK + wk (128-wide, one scale group each); with WK > 1
// the waves' partial tiles are summed through LDS at the end (fixed order).
// Per iteration:
//   * X[rows, WK K blocks] goes global -> registers -> LDS, pair-interleaved
//     (tern_device.h); the LDS tile is double-buffered (one barrier per
//     iteration) and the global loads run two iterations ahead.  16-row
//     tiles stage only the XR rows that can exist (4, 8 or 16);
//   * codes: in the 16 x 32 tiles (WK = 8) the workgroup loads the tile's
//     code bytes together, 32 threads per row, so each row's 256 bytes of
//     the iteration are one contiguous run, and stages them in LDS beside
//     the activations; in the 64 x 256 tiles each lane loads the 8 code
//     bytes (32 weights) of its column per column block, prefetched two
//     iterations ahead in a ring of two register sets;
//   * each lane decodes its 8 code bytes per column block straight into
//     MFMA B operands: +-2 pairs (tern_device.h), exact in fp16 and bf16;
//     the block's fp32 partial sum is then scaled by s/2 in fp32 (the pages'
//     scale-at-the-block-boundary step), so no scale is ever rounded or
//     overflowed into the 16-bit operand;
//   * v_mfma_f32_16x16x32_{f16,bf16}: lane l gives A[l%16][8(l/16)+e] and
//     B[8(l/16)+e][l%16]; the lane's 32 weights of a block are spread over the
//     4 MFMA k-steps so that the activation fragment of step t is the 16-byte
//     run X'[32g + 8t .. +8] of the pair-interleaved row;
//   * every global load is issued unconditionally, at a clamped in-bounds
//     address, so the compiler can count the loads in flight.
// Staged rows are padded (64 x 256 tiles) or XOR-swizzled (16-row tiles, see
// x_chunk) so the fragment reads are free of bank conflicts.
// Workgroups are numbered so that each XCD (workgroups go round-robin over
// the 8 XCDs) gets a contiguous run of tiles, which share activation rows in
// that XCD's L2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tern_device.h"
#include "tern_kernels.h"

namespace tern {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 128;              // K per block (= one scale group)
// A staged activation row (one K block, 256 bytes) either is padded to 272
// bytes (SWZ = false) or keeps 256 bytes with its 16-byte chunks XOR-swizzled
// by the row (SWZ = true); either way the 16 rows one MFMA operand read
// touches fall in distinct banks.  The swizzle saves the LDS that lets two
// 16 x 32 workgroups share a CU; the 64 x 256 tile runs faster padded
// (M=64, 5120 -> 17408: 70.6 against 77.3 us).
template <bool SWZ>
__device__ __forceinline__ int x_chunk(int row, int c) {
    return SWZ ? row * 256 + ((c ^ (row & 15)) << 4) : row * 272 + c * 16;
}
// Staged code rows (256 bytes, 32 pieces of 8 bytes), swizzled the same way.
__device__ __forceinline__ int c_piece_off(int row, int p) { return row * 256 + ((p ^ ((row & 15) << 1)) << 3); }

template <bool BF16>
__device__ __forceinline__ float4_t mfma16x16x32(const uint4 &a, const uint4 &b, float4_t c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, a),
                                                       __builtin_bit_cast(bf168_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    }
}

// S8: scales are int8 codes Q[N,K/128] times a per-row fp32 factor R[N].
// XR: activation rows of a tile that are loaded and staged (a power of two,
// XR = BM or, with one 16-row block, 4 or 8 when M <= XR).
// TWO: registers are capped for 8 waves per SIMD, so that two 16-wave
// workgroups fit on a CU (the LDS of a 16 x 32 tile is at most 80 KB).
template <int MB, int NB, int WN, int WK, int XR, bool TWO, bool XBF16, int YT, bool S8>
__global__ __launch_bounds__(64 * WN * WK, TWO ? 8 : 1) void gemm_kernel(const uint16_t *__restrict__ X,
                                                             const uint8_t *__restrict__ P,
                                                             const uint16_t *__restrict__ S,
                                                             const int8_t *__restrict__ Q,
                                                             const float *__restrict__ R,
                                                             void *__restrict__ Y, int M, int N, int K,
                                                             int tiles_m, int tiles_n) {
    constexpr int BM = 16 * MB;
    constexpr int BN = 16 * NB * WN;
    constexpr int NT = 64 * WN * WK;
    static_assert(XR == BM || (MB == 1 && (XR == 4 || XR == 8)), "rows staged per tile");
    constexpr int A_UNITS_TOTAL = WK * XR * (BK / 16);   // 16-element units per iteration
    constexpr int A_UNITS = (A_UNITS_TOTAL + NT - 1) / NT;
    constexpr bool SWZ = MB == 1;                         // 16-row tiles: swizzled, unpadded rows
    constexpr int A_TILE = XR * (SWZ ? 256 : 272);        // bytes of one K block's activations
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[2 * WK * A_TILE];
    // CT: the workgroup loads its code tile (BN rows x WK K blocks) together,
    // 32 threads per row, each 8 bytes, so each row's WK*32 bytes are read as
    // one contiguous run; the tile is staged in LDS (double-buffered beside
    // the activations) and each wave reads its MFMA operand bytes from there.
    // Without it, a load instruction reads 32 bytes from each of 16 rows.
    constexpr bool CT = WK == 8 && NT == BN * 4 * WK;     // 256-byte code rows of 32 pieces
    __shared__ __attribute__((aligned(16))) uint8_t c_lds[CT ? 2 * BN * 256 : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave % WN;
    const int wk = wave / WN;
    const int li = lane & 15;   // row (A) / column (B) within a 16-block
    const int lg = lane >> 4;   // k-slot group

    // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a
    // contiguous range of tiles (tile_n fastest), so neighbours share rows.
    const int ntiles = tiles_m * tiles_n;
    int tile = blockIdx.x;
    if (ntiles % 8 == 0) tile = (blockIdx.x % 8) * (ntiles / 8) + blockIdx.x / 8;
    const int tile_m = tile / tiles_n;
    const int tile_n = tile - tile_m * tiles_n;
    const int m0 = tile_m * BM;
    const int n0 = tile_n * BN + wn * (16 * NB);
    const int64_t row_bytes = K >> 2;
    const int groups = K >> 7;
    const int nkb = K / BK;
    const int niter = (nkb + WK - 1) / WK;

    // ---- activation tile: global -> registers (clamped addresses) ----
    // Every load is issued unconditionally, at a clamped in-bounds address
    // (rows past M read row M - 1 again; K blocks past the end read the last
    // one).  A load under a condition would leave the compiler unable to
    // count the loads in flight, and it would then wait for all of them,
    // including the prefetch two iterations ahead, at the top of every
    // iteration.  Rows at or past M are not staged: their LDS rows hold
    // stale values, which reach only output rows that are never stored (row
    // i of an MFMA result depends on row i of A alone).
    uint4 a_reg[A_UNITS][2];
    auto load_a = [&](int it) {
#pragma unroll
        for (int u = 0; u < A_UNITS; ++u) {
            const int b = min(tid + NT * u, A_UNITS_TOTAL - 1);   // past the last unit: load it again
            const int w = b / (XR * 8);              // which of the WK K blocks
            const int rem = b - w * (XR * 8);
            const int row = rem >> 3;
            const int blk = rem & 7;
            const int kb = min(it * WK + w, nkb - 1);
            const int64_t m = min(m0 + row, M - 1);
            const uint4 *src = reinterpret_cast<const uint4 *>(X + m * K + (int64_t)kb * BK + blk * 16);
            a_reg[u][0] = src[0];
            a_reg[u][1] = src[1];
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int u = 0; u < A_UNITS; ++u) {
            const int b = tid + NT * u;
            const int rowb = (b - (b / (XR * 8)) * (XR * 8)) >> 3;
            if ((A_UNITS * NT == A_UNITS_TOTAL || b < A_UNITS_TOTAL) && m0 + rowb < M) {
                const int w = b / (XR * 8);
                const int rem = b - w * (XR * 8);
                const int row = rem >> 3;
                const int blk = rem & 7;
                uint32_t pr[8];
                interleave16(a_reg[u][0], a_reg[u][1], pr);
                uint8_t *dst = a_lds + (buf * WK + w) * A_TILE;
                *reinterpret_cast<uint4 *>(dst + x_chunk<SWZ>(row, 2 * blk)) = make_uint4(pr[0], pr[1], pr[2], pr[3]);
                *reinterpret_cast<uint4 *>(dst + x_chunk<SWZ>(row, 2 * blk + 1)) = make_uint4(pr[4], pr[5], pr[6], pr[7]);
            }
        }
    };

    // ---- CT: the workgroup's code tile, thread t -> row t / (4 WK), 8-byte piece t % (4 WK) ----
    const int c_row = tid / (4 * WK);
    const int c_piece = tid - c_row * (4 * WK);
    const uint8_t *c_src = P + (int64_t)min(tile_n * BN + c_row, N - 1) * row_bytes;   // clamped: never stored
    uint2 c_reg = make_uint2(0u, 0u);
    auto load_c = [&](int it) {
        if constexpr (CT) {
            // past the last K block: the row's last 8 bytes (in bounds, unused)
            const int64_t o = min((int64_t)it * (WK * 32) + c_piece * 8, row_bytes - 8);
            c_reg = *reinterpret_cast<const uint2 *>(c_src + o);
        }
    };
    auto store_c = [&](int buf) {
        if constexpr (CT) *reinterpret_cast<uint2 *>(c_lds + buf * BN * 256 + c_piece_off(c_row, c_piece)) = c_reg;
    };

    // ---- weights: 8 code bytes (unless CT) + one scale per column block (clamped) ----
    auto load_w = [&](int it, uint2 (&w)[NB], uint32_t (&s)[NB]) {
        const int kb = min(it * WK + wk, nkb - 1);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int64_t n = min(n0 + nb * 16 + li, N - 1);
            if constexpr (!CT) w[nb] = *reinterpret_cast<const uint2 *>(P + n * row_bytes + (int64_t)kb * (BK / 4) + lg * 8);
            if constexpr (S8) s[nb] = (uint32_t)(int32_t)Q[n * groups + kb];
            else s[nb] = S[n * groups + kb];
        }
    };

    float4_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

    // weight loads of iterations it and it + 1: a ring of two sets, each
    // reloaded (for it + 2) by the iteration that used it, so no register
    // copy has to wait for a load in flight
    uint2 wa[NB], wb[NB];
    uint32_t sa[NB], sb[NB];    // fp16 scale bits, or the sign-extended int8 code
    float rowf[NB];             // S8: the row factor of this lane's column, applied in the epilogue
    if constexpr (S8) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) rowf[nb] = R[min(n0 + nb * 16 + li, N - 1)];
    }
    load_a(0);
    load_c(0);
    load_w(0, wa, sa);
    store_a(0);
    store_c(0);
    load_a(1);            // clamped: iteration 1 need not exist
    load_c(1);
    load_w(1, wb, sb);
    __syncthreads();

    auto iteration = [&](const int it, uint2 (&w0)[NB], uint32_t (&s0)[NB]) {
        const int buf = it & 1;
        if (it * WK + wk < nkb) {             // this wave's K block exists (uniform per wave)
            // decode: field transform of the lane's two code words per column block
            uint64_t v[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                uint2 wv = w0[nb];
                if constexpr (CT)
                    wv = *reinterpret_cast<const uint2 *>(c_lds + buf * BN * 256 +
                                                          c_piece_off(16 * (NB * wn + nb) + li, wk * 4 + lg));
                v[nb] = sign_nz_fields64<true>((uint64_t)wv.x | ((uint64_t)wv.y << 32));
            }

            float4_t part[MB][NB];
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) part[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
            // rows past XR (only when M <= XR) read a staged row: they feed
            // output rows that are never stored
            const int arow0 = li & (XR - 1);
            const uint8_t *a_tile = a_lds + (buf * WK + wk) * A_TILE;

            // k-steps H and H+2 use pairs 4H..4H+3 of word 0 and of word 1:
            // one 64-bit shift per pair index gives both (low and high half)
            auto kstep2 = [&](auto hc) {
                constexpr int H = decltype(hc)::value;
                uint4 blo[NB], bhi[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    uint32_t lo0, hi0, lo1, hi1, lo2, hi2, lo3, hi3;
                    weight_pairs2<4 * H + 0, true>(v[nb], lo0, hi0);
                    weight_pairs2<4 * H + 1, true>(v[nb], lo1, hi1);
                    weight_pairs2<4 * H + 2, true>(v[nb], lo2, hi2);
                    weight_pairs2<4 * H + 3, true>(v[nb], lo3, hi3);
                    blo[nb] = make_uint4(lo0, lo1, lo2, lo3);
                    bhi[nb] = make_uint4(hi0, hi1, hi2, hi3);
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    // this lane's 32 activations of the block: chunks 4 lg .. 4 lg + 3
                    const int r = arow0 + 16 * mb;
                    const uint4 al = *reinterpret_cast<const uint4 *>(a_tile + x_chunk<SWZ>(r, 4 * lg + H));       // k-step H
                    const uint4 ah = *reinterpret_cast<const uint4 *>(a_tile + x_chunk<SWZ>(r, 4 * lg + H + 2));   // k-step H+2
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        part[mb][nb] = mfma16x16x32<XBF16>(al, blo[nb], part[mb][nb]);
                        part[mb][nb] = mfma16x16x32<XBF16>(ah, bhi[nb], part[mb][nb]);
                    }
                }
            };
            kstep2(std::integral_constant<int, 0>{});
            kstep2(std::integral_constant<int, 1>{});

            // block boundary: scale the block's sums (s/2: the operands were +-2)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float s = (S8 ? (float)(int32_t)s0[nb] : f16_bits_to_float((uint16_t)s0[nb])) * 0.5f;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    acc[mb][nb][0] = fmaf(s, part[mb][nb][0], acc[mb][nb][0]);
                    acc[mb][nb][1] = fmaf(s, part[mb][nb][1], acc[mb][nb][1]);
                    acc[mb][nb][2] = fmaf(s, part[mb][nb][2], acc[mb][nb][2]);
                    acc[mb][nb][3] = fmaf(s, part[mb][nb][3], acc[mb][nb][3]);
                }
            }
        }
        // next tile into the other buffer; loads two iterations ahead, issued
        // whether or not that iteration exists (clamped, see load_a)
        if (it + 1 < niter) {
            store_a(buf ^ 1);
            store_c(buf ^ 1);
        }
        load_a(it + 2);
        load_c(it + 2);
        load_w(it + 2, w0, s0);
        __syncthreads();
    };
    // both halves of the loop body run on every trip (a conditional second
    // half would make the compiler assume, at the top of the loop, that the
    // first half's loads were the last ones issued, and wait for them)
    int it = 0;
    for (; it + 1 < niter; it += 2) {
        iteration(it, wa, sa);
        iteration(it + 1, wb, sb);
    }
    if (it < niter) iteration(it, wa, sa);

    // ---- waves that split K: sum their partial tiles through LDS ----
    if constexpr (WK > 1) {
        float *red = reinterpret_cast<float *>(a_lds);   // reuse the tile buffer
        constexpr int PER_WAVE = MB * NB * 4 * 64;        // floats
        static_assert((size_t)(WK - 1) * WN * PER_WAVE * 4 <= sizeof(a_lds), "reduction buffer");
        if (wk > 0) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        red[(((wk - 1) * WN + wn) * MB * NB * 4 + (mb * NB + nb) * 4 + i) * 64 + lane] =
                            acc[mb][nb][i];
        }
        __syncthreads();
        if (wk > 0) return;
        for (int w = 1; w < WK; ++w) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[mb][nb][i] += red[(((w - 1) * WN + wn) * MB * NB * 4 + (mb * NB + nb) * 4 + i) * 64 + lane];
        }
    }

    // ---- epilogue: lane l holds rows 4(l/16)+i, column l%16 of each 16x16 block ----
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = n0 + nb * 16 + li;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + mb * 16 + lg * 4 + i;
                if (m < M) store_out<YT>(Y, (int64_t)m * N + n, S8 ? acc[mb][nb][i] * rowf[nb] : acc[mb][nb][i]);
            }
        }
}

template <int MB, int NB, int WN, int WK, int XR, bool TWO, bool XBF16, int YT, bool S8>
hipError_t launch_t(const GemmArgs &a) {
    constexpr int BM = 16 * MB, BN = 16 * NB * WN;
    const int64_t tiles_n = (a.N + BN - 1) / BN;
    const int64_t tiles_m = (a.M + BM - 1) / BM;
    if (tiles_n * tiles_m > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_kernel<MB, NB, WN, WK, XR, TWO, XBF16, YT, S8>), dim3((unsigned)(tiles_n * tiles_m)),
                       dim3(64 * WN * WK), 0, a.stream, static_cast<const uint16_t *>(a.X), a.W, a.S, a.Q, a.R, a.Y,
                       (int)a.M, (int)a.N, (int)a.K, (int)tiles_m, (int)tiles_n);
    return hipGetLastError();
}

template <bool XBF16, int YT, bool S8>
hipError_t launch_shape(const GemmArgs &a) {
    // M <= 16: 16 x 32 tiles of two 16-column waves, K split over 8 waves
    // each (16 waves).  Measured on the 5120 <-> 17408 decode shapes against
    // one 32-column wave x 8 (the previous choice): M = 4 19.2 / 19.0 us
    // against 19.7 / 19.9, M = 16 22.1 / 22.7 against 22.7 / 23.7; 64-column
    // tiles, or K split over 2 or 4 waves, were 5-90% slower.
    // K <= 8192 (at most 8 iterations): two workgroups share a CU, so one's
    // pipeline fill overlaps the other's work; with M <= 8 only the 4 or 8
    // rows that exist are staged.  Measured, FFN up (K=5120): M = 4 18.5 ->
    // 16.1 us, M = 8 18.7 -> 16.6 us, M = 16 20.0 -> 19.1 us.  With longer K
    // it was 3-4% slower (FFN down, K=17408: the register cap of two
    // workgroups per CU spills a few registers), so those keep one
    // workgroup per CU.
    // M <= 4: 16-column workgroups of 8 waves (twice as many; four per CU
    // with the register cap at K <= 8192, two without it beyond): FFN up
    // 16.0 -> 15.0 us, 5120 -> 5120 7.6 -> 7.3 us, FFN down 16.6 -> 16.1 us,
    // 12288 -> 4096 13.7 -> 10.8 us.  At M = 8 no change or slower, at
    // M = 16 slower.
    if (a.M <= 4 && a.K <= 8192) return launch_t<1, 1, 1, 8, 4, true, XBF16, YT, S8>(a);
    if (a.M <= 4) return launch_t<1, 1, 1, 8, 4, false, XBF16, YT, S8>(a);
    if (a.M <= 8 && a.K <= 8192) return launch_t<1, 1, 2, 8, 8, true, XBF16, YT, S8>(a);
    if (a.M <= 16 && a.K <= 8192) return launch_t<1, 1, 2, 8, 16, true, XBF16, YT, S8>(a);
    if (a.M <= 16) return launch_t<1, 1, 2, 8, 16, false, XBF16, YT, S8>(a);
    return launch_t<4, 4, 4, 1, 64, false, XBF16, YT, S8>(a);            // 64 x 256
}

template <bool XBF16, bool S8>
hipError_t launch_y(const GemmArgs &a) {
    switch (a.y_dtype) {
    case 0: return launch_shape<XBF16, 0, S8>(a);
    case 1: return launch_shape<XBF16, 1, S8>(a);
    default: return launch_shape<XBF16, 2, S8>(a);
    }
}

}  // namespace

// fp16 X with at least this many rows goes to the LDS-staged kernel of
// tern_gemm_big.hip, which shares each weight decode across the rows of a
// large tile.  Its operand is the exact fp16 product t*s (t*q for int8
// scales), which needs fp16 activations beside it; bf16 X stays here.
constexpr int64_t kBigMinM = 128;

hipError_t launch_gemm(const GemmArgs &a) {
    if (a.x_dtype == 0 && a.M >= kBigMinM) return launch_gemm_big(a);
    if (a.Q != nullptr) return a.x_dtype == 1 ? launch_y<true, true>(a) : launch_y<false, true>(a);
    return a.x_dtype == 1 ? launch_y<true, false>(a) : launch_y<false, false>(a);
}

}  // namespace tern
