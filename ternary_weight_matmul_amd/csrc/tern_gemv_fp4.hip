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
// Weight operand.  After the field transform of tern_device.h each 2-bit
// field is [sign, nonzero].  Read as a 4-bit e2m1 value with the field in
// bits 3..2 of its nibble, that is -2, +2 or +-0: one AND turns the 8 odd
// fields of a code word into 8 fp4 weights in place, and a shift by 2 plus an
// AND the 8 even ones.  Decoding 32 weights costs 10 VALU operations (about a
// third of a lane-op per weight, against 0.9 for 16-bit +-2 pairs), which is
// what lets the decode keep up with HBM.
//
// Activation operand.  v_mfma_scale_f32_16x16x128_f8f6f4 multiplies e4m3
// activations (A) by the e2m1 weights (B), each A row carrying a power-of-two
// scale per 32 consecutive K.  Every bf16 activation is split exactly into two
// e4m3 terms sharing its 32-block: hi = RNE(x / 2^e) with 2^e = 2^(E - 7) for
// the block's largest exponent E (|x / 2^e| < 256 <= 448), and
// lo = RNE((x - hi 2^e) / 2^(e - 4)).  The residual x - hi 2^e is a multiple
// of the bf16 ulp of x and smaller than half the e4m3 ulp of hi, so it has at
// most 4 significant bits: lo is exact whenever that ulp is at least the
// smallest e4m3 subnormal, i.e. for every element within 2^13 of its block's
// largest magnitude.  Smaller elements keep an absolute error below 2^-21 of
// the block maximum, far inside the product's 2e-3 * sum |x s| bound.  Both
// terms enter one MFMA as separate A rows; products of e4m3 and e2m1 values
// are exact, sums are fp32.
//
// Operand layout (gfx950, measured): B lane l = column l%16, true K
// 32 (l/16) + nibble; A lane l = row l%16, true K 16 (l/16) + byte for bytes
// 0..15 and 64 + 16 (l/16) + byte - 16 for bytes 16..31; the A scale of lane
// l is the one of true-K block l/16; D VGPR v of lane l is row 4 (l/16) + v,
// column l%16.  With the fp4 decode above, true K (32p + 8d + t) holds weight
// 32p + 16 (d/2) + 2t + (d%2) of the 128-weight block, so A slice s carries
// the activations of weights 16s..16s+15 (bytes 0..15) and 64+16s..79+16s
// (bytes 16..31), evens first, then odds.
//
// Work layout.
//   * unit = (quad q, step s): rows 4q..4q+3 x 512 weights (4 blocks g0..g0+3,
//     g0 = 4s).  B column j = 4r + c is (row 4q + r, block g0 + c); lane l
//     loads the 8 code bytes of slice l/16 of its column (each row's 16 lanes
//     read 128 contiguous bytes).  A row i = 4c + 2h + m (M <= 2: one MFMA,
//     term h and row m both in it) or i = 4c + m (M = 3, 4: one MFMA per
//     term): only D entries with A block c = B block c are used -- lanes l
//     with l/16 = l%4, VGPR 2h + m (or m).
//   * one workgroup of 16 waves per CU takes a contiguous range of quads;
//     units are numbered quad-major; wave w takes units [UPW w, UPW w + UPW);
//   * all waves first split and stage the workgroup's activations in LDS,
//     with every code and scale load of the wave already issued behind them;
//   * per unit: 1 or 2 MFMAs, acc += s * (D_hi + D_lo) on the 16 lanes that
//     hold same-block entries; when the wave leaves a quad these write their
//     sums to LDS; after a barrier each output adds its 4 blocks' and waves'
//     partials in a fixed order (deterministic), halves the sum (the weights
//     are +-2) and rounds it to the output type.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "tern_device.h"
#include "tern_kernels.h"

namespace tern {

namespace {

constexpr int F_STEP = 512;          // weights of a row per unit
constexpr int F_BPU = F_STEP / 128;  // 128-weight blocks per unit (4)
constexpr int F_WAVES = 16;
constexpr int F_THREADS = 64 * F_WAVES;
constexpr int F_MAX_UPW = 12;

typedef int int8v_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef short short2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// All ones where c holds, else zero, hidden from the optimiser.
__device__ __forceinline__ uint32_t opaque_lanes(bool c) {
    uint32_t m = c ? ~0u : 0u;
    asm("" : "+v"(m));
    return m;
}

// A block (128 bytes: 4 slices of 32) of activation row m, term h (0 = hi,
// 1 = lo), weight block g: index k = (2 g + h) M + m.  Slice p sits at
// 32 ((p + (k >> 1)) & 3) inside the block, which spreads the A reads of the
// 16 lanes of one slice over the banks; for a lane the rotation does not
// depend on the unit (the blocks of a unit start at a multiple of 4).
__device__ __forceinline__ int ablock(int M, int g, int h, int m) { return (2 * g + h) * M + m; }
__device__ __forceinline__ int aslice(int k, int p) { return k * 128 + 32 * ((p + (k >> 1)) & 3); }

// Largest of the 8 bf16 magnitudes in q (as integers: same order as values).
__device__ __forceinline__ uint32_t max_mag8(const uint4 &q) {
    typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
    auto mag = [](uint32_t v) { return __builtin_bit_cast(ushort2_t, v & 0x7FFF7FFFu); };
    ushort2_t a = __builtin_elementwise_max(mag(q.x), mag(q.y));
    ushort2_t b = __builtin_elementwise_max(mag(q.z), mag(q.w));
    a = __builtin_elementwise_max(a, b);
    return a[0] > a[1] ? a[0] : a[1];
}

// Max over the 4 lanes of a DPP quad.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
    return v;
}

// Exact two-term e4m3 split of 8 bf16 activations q (scales 2^(eh - 127),
// 2^(el - 127)): hi and lo bytes in the A order of a half chunk, evens first
// (even[i] = element 2i, odd[i] = element 2i + 1).
__device__ __forceinline__ void split8(const uint4 &q, uint32_t eh, uint32_t el, uint32_t &hi_even,
                                       uint32_t &hi_odd, uint32_t &lo_even, uint32_t &lo_odd) {
    const float sh = __builtin_bit_cast(float, eh << 23);
    const float sl = __builtin_bit_cast(float, el << 23);
    const short2_t z = {0, 0};
    // hi bytes: elements 0..3 in h01, 4..7 in h23 (one pair per 16-bit half)
    short2_t h01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(z, __builtin_bit_cast(bf162v_t, q.x), sh, false);
    h01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(h01, __builtin_bit_cast(bf162v_t, q.y), sh, true);
    short2_t h23 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(z, __builtin_bit_cast(bf162v_t, q.z), sh, false);
    h23 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(h23, __builtin_bit_cast(bf162v_t, q.w), sh, true);
    const uint32_t hb01 = __builtin_bit_cast(uint32_t, h01), hb23 = __builtin_bit_cast(uint32_t, h23);
    // residuals x - hi (exact in fp32), then their e4m3 bytes at the lo scale
    auto res = [](uint32_t w, float2_t hf, int half) {
        const float x = __builtin_bit_cast(float, half ? (w & 0xFFFF0000u) : (w << 16));
        return x - hf[half];
    };
    const float2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hb01, sh, false);
    const float2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hb01, sh, true);
    const float2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hb23, sh, false);
    const float2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hb23, sh, true);
    short2_t l01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, res(q.x, f0, 0), res(q.x, f0, 1), sl, false);
    l01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l01, res(q.y, f1, 0), res(q.y, f1, 1), sl, true);
    short2_t l23 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, res(q.z, f2, 0), res(q.z, f2, 1), sl, false);
    l23 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l23, res(q.w, f3, 0), res(q.w, f3, 1), sl, true);
    const uint32_t lb01 = __builtin_bit_cast(uint32_t, l01), lb23 = __builtin_bit_cast(uint32_t, l23);
    hi_even = __builtin_amdgcn_perm(hb23, hb01, 0x06040200u);
    hi_odd = __builtin_amdgcn_perm(hb23, hb01, 0x07050301u);
    lo_even = __builtin_amdgcn_perm(lb23, lb01, 0x06040200u);
    lo_odd = __builtin_amdgcn_perm(lb23, lb01, 0x07050301u);
}

// D = A * B on the matrix cores: A e4m3 with per-lane block scale sa (E8M0),
// B e2m1 (scale 1).
__device__ __forceinline__ float4_t mfma_f8f4(const uint4 &a0, const uint4 &a1, const uint4 &b, uint32_t sa) {
    const int8v_t av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const int8v_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    const float4_t z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z, 0 /* A e4m3 */, 4 /* B e2m1 */, 0,
                                                            (int)sa, 0, 127);
}

// UPW: units per wave; OPT: 8-activation octets staged per thread.
template <int M, bool S8, int UPW, int OPT>
__global__ __launch_bounds__(F_THREADS) void gemv_fp4_kernel(const uint16_t *__restrict__ X,
                                                             const uint8_t *__restrict__ P,
                                                             const uint16_t *__restrict__ S,
                                                             const int8_t *__restrict__ Q,
                                                             const float *__restrict__ R, void *__restrict__ Y,
                                                             int y_dtype, int N, int K, int nquads, int kmax) {
    constexpr int TERMS_PER_MFMA = M <= 2 ? 2 : 1;   // hi and lo rows in one MFMA, or one MFMA per term
    extern __shared__ uint4 lds[];
    char *ldsb = reinterpret_cast<char *>(lds);
    const int groups = K >> 7;
    const int steps = (groups + F_BPU - 1) / F_BPU;
    const int g4 = steps * F_BPU;                    // blocks staged (zero padded to whole units)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = lane >> 4;        // K slice of the lane (A and B)
    const int col = lane & 15;      // B column: 4 r + c
    const int r = col >> 2;         // weight row within the quad
    const int c = col & 3;          // weight block within the unit
    const int G = gridDim.x;
    const int qa = (int)((int64_t)blockIdx.x * nquads / G);
    const int qb = (int)((int64_t)(blockIdx.x + 1) * nquads / G);
    const int U = (qb - qa) * steps;
    const int ufirst = wave * UPW;
    const int64_t row_bytes = K >> 2;
    const int abytes = M * 2 * g4 * 128;             // staged activations
    const int sbytes_lds = M * 2 * g4 * 4;           // their block scales (E8M0)
    char *ascale = ldsb + abytes;
    float4_t *red = reinterpret_cast<float4_t *>(ldsb + abytes + sbytes_lds);   // [F_WAVES][kmax][16 (r, c)], then 64 lane spares

    // ---- 1. loads: activation octets first, then every code and scale load
    //         of the wave (buffer loads rebased per unit on the scalar unit;
    //         rows past N read zeros; blocks past K read finite bytes that meet
    //         zero activations) ----
    const int octs = M * g4 * 16;                    // 8-activation octets, padding included
    uint4 xq[OPT];
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
        const int t = tid + i * F_THREADS;
        const int m = min(t / (g4 * 16), M - 1);
        const int o = t % (g4 * 16);                 // octet within the row
        const int oc = min(o, (K >> 3) - 1);
        xq[i] = *reinterpret_cast<const uint4 *>(X + (int64_t)m * K + (int64_t)oc * 8);
    }
    // keep the activation loads ahead of the code loads: the staging waits for them alone
    __builtin_amdgcn_sched_barrier(0);
    const int wg_rows = min(4 * qb, N) - 4 * qa;
    const uint8_t *Pwg = P + (int64_t)4 * qa * row_bytes;
    const uint32_t pbytes = (uint32_t)(wg_rows * row_bytes);
    constexpr int SB = S8 ? 1 : 2;
    const char *Swg = S8 ? reinterpret_cast<const char *>(Q + (int64_t)4 * qa * groups)
                         : reinterpret_cast<const char *>(S + (int64_t)4 * qa * groups);
    const uint32_t sbytes = (uint32_t)(wg_rows * groups * SB);
    const int pofs = r * (int)row_bytes + c * 32 + p * 8;   // this lane's 8 code bytes within a unit
    const int sofs = (r * groups + c) * SB;                // this lane's block scale within a unit
    uint2 code[UPW];
    uint32_t sbits[UPW];
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
        const int u = min(ufirst + i, U - 1);
        const int ql = u / steps;
        const int s = u - ql * steps;
        const uint32_t pu = (uint32_t)(4 * ql * row_bytes + s * (F_STEP / 4));
        const uint32_t su = (uint32_t)((4 * ql * groups + s * F_BPU) * SB);
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(buffer_rsrc(Pwg + pu, pbytes - pu), pofs, 0, 2 /* nt */));
        code[i] = make_uint2(v[0], v[1]);
        if constexpr (S8)
            sbits[i] = (uint32_t)(int32_t)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(buffer_rsrc(Swg + su, sbytes - su),
                                                                                     sofs, 0, 0);
        else
            sbits[i] = __builtin_amdgcn_raw_buffer_load_b16(buffer_rsrc(Swg + su, sbytes - su), sofs, 0, 0);
    }

    // ---- 2. split and stage the activations.  Octet o of block g (elements
    //         128 g + 8 o ..) is quarter o % 4 of 32-block o / 4: the 4 lanes of
    //         a DPP quad hold one 32-block and share its maximum.  Written
    //         without branches (threads past the last octet write a spare
    //         slot), so the activation loads stay ahead of the code loads. ----
    const int spare = abytes + sbytes_lds + F_WAVES * kmax * 256 + 64 * 16;   // after the per-lane flush spares
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
        const int t = tid + i * F_THREADS;
        const bool valid = t < octs;
        const int m = min(t / (g4 * 16), M - 1);
        const int o = t % (g4 * 16);
        const int g = o >> 4;                        // 128-weight block
        const int ob = o & 15;                       // octet within the block
        uint4 q = xq[i];
        const uint32_t keep = opaque_lanes(o < (K >> 3));   // zero padding past K
        q.x &= keep;
        q.y &= keep;
        q.z &= keep;
        q.w &= keep;
        const uint32_t mx = quad_max(max_mag8(q));   // largest magnitude of the 32-block
        const uint32_t eb = mx >> 7;                 // its biased exponent
        const uint32_t eh = eb > 8 ? eb - 7 : 1;     // hi scale 2^(E - 7), at least 2^-126
        const uint32_t el = eh > 5 ? eh - 4 : 1;     // lo scale 2^(E - 11)
        uint32_t he, ho, le, lo;
        split8(q, eh, el, he, ho, le, lo);
        // the 16-element chunk ob / 2 of the block goes to A slice (ob / 2) % 4,
        // half (ob / 2) / 4; this octet is half ob % 2 of the chunk's evens and odds
        const int ch = ob >> 1;
        const int sl = ch & 3;
        const int off = 16 * (ch >> 2) + 4 * (ob & 1);
        const int kh = ablock(M, g, 0, m), kl = ablock(M, g, 1, m);
        const int ah = valid ? aslice(kh, sl) + off : spare;
        const int al = valid ? aslice(kl, sl) + off : spare + 16;
        *reinterpret_cast<uint32_t *>(ldsb + ah) = he;
        *reinterpret_cast<uint32_t *>(ldsb + ah + 8) = ho;
        *reinterpret_cast<uint32_t *>(ldsb + al) = le;
        *reinterpret_cast<uint32_t *>(ldsb + al + 8) = lo;
        // block scales: A scale of slice p covers weights 32p..32p+31 of the block
        if ((ob & 3) == 0) {
            const int sb = ob >> 2;
            ascale[valid ? kh * 4 + sb : sbytes_lds] = (char)eh;
            ascale[valid ? kl * 4 + sb : sbytes_lds] = (char)el;
        }
    }
    __syncthreads();

    // ---- 3. units ----
    // A row of this lane: M <= 2: i = 4 ci + 2 h + m; M = 3, 4: i = 4 ci + m
    // (ci is the A block, the lane's row within the MFMA is col = lane & 15)
    const int ci = col >> 2;
    int ka[2];
    if constexpr (M <= 2) {
        const int h = (col >> 1) & 1;
        const int m = min(col & 1, M - 1);
        ka[0] = ablock(M, ci, h, m);
        ka[1] = ka[0];
    } else {
        const int m = min(col & 3, M - 1);
        ka[0] = ablock(M, ci, 0, m);
        ka[1] = ablock(M, ci, 1, m);
    }
    const char *abase0 = ldsb + aslice(ka[0], p);
    const char *abase1 = ldsb + aslice(ka[1], p);
    const unsigned char *sbase0 = reinterpret_cast<const unsigned char *>(ascale) + ka[0] * 4 + p;
    const unsigned char *sbase1 = reinterpret_cast<const unsigned char *>(ascale) + ka[1] * 4 + p;
    const int ustride_a = F_BPU * 2 * M * 128;       // A bytes per unit step
    const int ustride_s = F_BPU * 2 * M * 4;
    const bool holder = p == c;                      // lane holds same-block D entries
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;
    const int u0 = min(ufirst, U - 1);
    const int qfirst = u0 / steps;
    int ql = qfirst;
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
            // decode: 32 fp4 weights, K order 32p + 8d + t <-> weight 16 (d/2) + 2t + (d%2)
            const uint64_t v = sign_nz_fields64((uint64_t)code[i].x | ((uint64_t)code[i].y << 32));
            const uint64_t e = shl64<2>(v);
            const uint4 bw = make_uint4((uint32_t)e & 0xCCCCCCCCu, (uint32_t)v & 0xCCCCCCCCu,
                                        (uint32_t)(e >> 32) & 0xCCCCCCCCu, (uint32_t)(v >> 32) & 0xCCCCCCCCu);
            const uint4 a0 = *reinterpret_cast<const uint4 *>(abase0 + s * ustride_a);
            const uint4 a1 = *reinterpret_cast<const uint4 *>(abase0 + s * ustride_a + 16);
            const uint32_t sa0 = sbase0[s * ustride_s];
            const float4_t d0 = mfma_f8f4(a0, a1, bw, sa0);
            const float sc = S8 ? (float)(int32_t)sbits[i] : f16_bits_to_float((uint16_t)sbits[i]);
            if constexpr (TERMS_PER_MFMA == 2) {
#pragma unroll
                for (int m = 0; m < M; ++m) acc[m] = fmaf(sc, d0[m] + d0[2 + m], acc[m]);
            } else {
                const uint4 b0 = *reinterpret_cast<const uint4 *>(abase1 + s * ustride_a);
                const uint4 b1 = *reinterpret_cast<const uint4 *>(abase1 + s * ustride_a + 16);
                const uint32_t sa1 = sbase1[s * ustride_s];
                const float4_t d1 = mfma_f8f4(b0, b1, bw, sa1);
#pragma unroll
                for (int m = 0; m < M; ++m) acc[m] = fmaf(sc, d0[m] + d1[m], acc[m]);
            }
            if (i == UPW - 1 || u + 1 >= U || s == steps - 1) {
                // every lane stores (the other lanes into a private spare
                // slot): a store only the holder lanes made would let the
                // compiler sink the MFMA into that divergent branch, and a
                // matrix instruction run under a partial EXEC mask does not
                // see the operands of the masked lanes
                float4_t rr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < M; ++m) rr[m] = acc[m];
                red[holder ? (wave * kmax + (ql - qfirst)) * 16 + col : F_WAVES * kmax * 16 + lane] = rr;
#pragma unroll
                for (int m = 0; m < M; ++m) acc[m] = 0.f;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < UPW; ++i) asm volatile("" ::"v"(code[i].x), "v"(sbits[i]));
    __syncthreads();

    // ---- 4. outputs: the 4 blocks and the wave partials of each row, in order ----
    const int nrows = 4 * (qb - qa);
    for (int o = tid; o < nrows * M; o += F_THREADS) {
        const int m = o / nrows;
        const int rl = o % nrows;
        const int qo = rl >> 2;
        const int n = 4 * qa + rl;
        if (n >= N) continue;
        const int w0 = (qo * steps) / UPW;
        const int w1 = (qo * steps + steps - 1) / UPW;
        float y = 0.f;
        for (int w = w0; w <= w1; ++w) {
            const int qf = min(w * UPW, U - 1) / steps;
            const float4_t *pp = red + (w * kmax + (qo - qf)) * 16 + 4 * (rl & 3);
            y += (pp[0][m] + pp[1][m]) + (pp[2][m] + pp[3][m]);
        }
        y *= 0.5f;   // the weights were +-2
        if constexpr (S8) y *= R[n];
        if (y_dtype == 2) store_out<2>(Y, (int64_t)m * N + n, y);
        else if (y_dtype == 1) store_out<1>(Y, (int64_t)m * N + n, y);
        else store_out<0>(Y, (int64_t)m * N + n, y);
    }
}

struct F4Shape {
    int steps, grid, upw, opt, kmax;
    size_t lds;
};

F4Shape f4_shape(int64_t M, int64_t N, int64_t K) {
    F4Shape g{};
    const int64_t groups = K / 128;
    g.steps = (int)((groups + F_BPU - 1) / F_BPU);
    const int64_t nquads = (N + 3) / 4;
    int64_t grid = 256;
    while ((nquads + grid - 1) / grid * g.steps > (int64_t)F_WAVES * F_MAX_UPW && grid < nquads) grid += 256;
    g.grid = (int)std::min<int64_t>(grid, nquads);
    const int64_t qmax = (nquads + g.grid - 1) / g.grid;
    const int64_t units = qmax * g.steps;
    int upw = (int)((units + F_WAVES - 1) / F_WAVES);
    if (upw > F_MAX_UPW) upw = 0;
    else if (upw == 5) upw = 6;
    else if (upw == 7) upw = 8;
    else if (upw > 8) upw = 12;
    g.upw = upw;
    const int64_t octs = M * g.steps * F_BPU * 16;
    const int64_t opt = (octs + F_THREADS - 1) / F_THREADS;
    g.opt = opt <= 1 ? 1 : opt <= 2 ? 2 : opt <= 4 ? 4 : opt <= 6 ? 6 : opt <= 9 ? 9 : 0;
    g.kmax = upw == 0 ? 0 : (int)std::min<int64_t>(upw, (upw + g.steps - 1) / g.steps + 1);
    const int64_t g4 = (int64_t)g.steps * F_BPU;
    g.lds = (size_t)(M * 2 * g4 * 128 + M * 2 * g4 * 4) + (size_t)F_WAVES * g.kmax * 256 + 64 * 16 + 32;
    return g;
}

template <int M, bool S8, int UPW, int OPT>
hipError_t launch_f4t(const GemmArgs &a, const F4Shape &g) {
    auto kern = gemv_fp4_kernel<M, S8, UPW, OPT>;
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
    hipLaunchKernelGGL(kern, dim3((unsigned)g.grid), dim3(F_THREADS), g.lds, a.stream,
                       static_cast<const uint16_t *>(a.X), a.W, a.S, a.Q, a.R, a.Y, a.y_dtype, (int)a.N, (int)a.K,
                       (int)((a.N + 3) / 4), g.kmax);
    return hipGetLastError();
}

template <int M, bool S8, int UPW>
hipError_t launch_f4o(const GemmArgs &a, const F4Shape &g) {
    switch (g.opt) {
    case 1: return launch_f4t<M, S8, UPW, 1>(a, g);
    case 2: return launch_f4t<M, S8, UPW, 2>(a, g);
    case 4: return launch_f4t<M, S8, UPW, 4>(a, g);
    case 6: return launch_f4t<M, S8, UPW, 6>(a, g);
    default: return launch_f4t<M, S8, UPW, 9>(a, g);
    }
}

template <int M, bool S8>
hipError_t launch_f4u(const GemmArgs &a, const F4Shape &g) {
    switch (g.upw) {
    case 1: return launch_f4o<M, S8, 1>(a, g);
    case 2: return launch_f4o<M, S8, 2>(a, g);
    case 3: return launch_f4o<M, S8, 3>(a, g);
    case 4: return launch_f4o<M, S8, 4>(a, g);
    case 6: return launch_f4o<M, S8, 6>(a, g);
    case 8: return launch_f4o<M, S8, 8>(a, g);
    default: return launch_f4o<M, S8, 12>(a, g);
    }
}

template <int M>
hipError_t launch_f4m(const GemmArgs &a, const F4Shape &g) {
    return a.Q != nullptr ? launch_f4u<M, true>(a, g) : launch_f4u<M, false>(a, g);
}

}  // namespace

bool gemv_fp4_fits(int64_t M, int64_t N, int64_t K, int x_dtype) {
    if (x_dtype != 1 || M < 1 || M > 4 || N < 1 || K < 128) return false;
    const F4Shape g = f4_shape(M, N, K);
    return g.upw > 0 && g.opt > 0 && g.lds <= 160 * 1024;
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
