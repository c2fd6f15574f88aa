// tern_fp4.h -- operands of v_mfma_scale_f32_16x16x128_f8f6f4 for the decode
// kernels that run the sign-select sums with 4-bit weights.
//
// Weight operand (B, e2m1).  After the field transform of tern_device.h each
// 2-bit field is [sign, nonzero].  Read as a 4-bit e2m1 value with the field
// in bits 3..2 of its nibble, that is -2, +2 or +-0 (2kiu.com/news/5082861
// §3.1 for the codes): one AND turns the 8 odd fields of a code word into 8
// fp4 weights in place, and a shift by 2 plus an AND the 8 even ones.
//
// Activation operand (A, e4m3 with a power-of-two scale per 32 K).  Every
// bf16 activation is split exactly into two e4m3 terms sharing its 32-run:
// hi = RNE(x / 2^e) with 2^e = 2^(E - 7) for the run's largest exponent E
// (|x / 2^e| < 256 <= 448), and lo = RNE((x - hi 2^e) / 2^(e - 4)).  The
// residual x - hi 2^e is a multiple of the bf16 ulp of x and smaller than half
// the e4m3 ulp of hi, so it has at most 4 significant bits: lo is exact
// whenever that ulp is at least the smallest e4m3 subnormal, i.e. for every
// element within 2^13 of its run's largest magnitude.  Smaller elements keep
// an absolute error below 2^-21 of the run maximum, far inside the product's
// 2e-3 * sum |x s| bound.  Products of e4m3 and e2m1 values are exact; sums
// are fp32.
//
// Operand layout (gfx950, measured): B lane l = column l%16, true K
// 32 (l/16) + nibble; A lane l = row l%16, true K 16 (l/16) + byte for bytes
// 0..15 and 64 + 16 (l/16) + byte - 16 for bytes 16..31; the A scale of lane
// l is the one of true-K block l/16; D VGPR v of lane l is row 4 (l/16) + v,
// column l%16.  With the fp4 decode above, true K (32p + 8d + t) holds weight
// 32p + 16 (d/2) + 2t + (d%2) of the 128-weight block: 8 code bytes of slice p
// (weights 32p .. 32p + 31) give the B registers of lane p, evens first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tern_device.h"

namespace tern {

typedef int fp4_int8v_t __attribute__((ext_vector_type(8)));
typedef float fp4_float4_t __attribute__((ext_vector_type(4)));
typedef float fp4_float2_t __attribute__((ext_vector_type(2)));
typedef short fp4_short2_t __attribute__((ext_vector_type(2)));
typedef __bf16 fp4_bf162_t __attribute__((ext_vector_type(2)));

// Largest of the 8 bf16 magnitudes in q (as integers: same order as values).
__device__ __forceinline__ uint32_t max_mag8(const uint4 &q) {
    typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
    auto mag = [](uint32_t v) { return __builtin_bit_cast(ushort2_t, v & 0x7FFF7FFFu); };
    ushort2_t a = __builtin_elementwise_max(mag(q.x), mag(q.y));
    ushort2_t b = __builtin_elementwise_max(mag(q.z), mag(q.w));
    a = __builtin_elementwise_max(a, b);
    return a[0] > a[1] ? a[0] : a[1];
}

// Biased E8M0 exponents of a 32-run's two terms from its largest bf16
// magnitude mx: hi scale 2^(E - 7) (at least 2^-126), lo scale 2^(E - 11).
__device__ __forceinline__ void split_exponents(uint32_t mx, uint32_t &eh, uint32_t &el) {
    const uint32_t eb = mx >> 7;   // biased exponent of the largest magnitude
    eh = eb > 8 ? eb - 7 : 1;
    el = eh > 5 ? eh - 4 : 1;
}

// Exact two-term e4m3 split of 8 bf16 activations q (scales 2^(eh - 127),
// 2^(el - 127)): hi and lo bytes, evens first (even[i] = element 2i,
// odd[i] = element 2i + 1).
__device__ __forceinline__ void split8(const uint4 &q, uint32_t eh, uint32_t el, uint32_t &hi_even,
                                       uint32_t &hi_odd, uint32_t &lo_even, uint32_t &lo_odd) {
    const float sh = __builtin_bit_cast(float, eh << 23);
    const float sl = __builtin_bit_cast(float, el << 23);
    const fp4_short2_t z = {0, 0};
    // hi bytes: elements 0..3 in h01, 4..7 in h23 (one pair per 16-bit half)
    fp4_short2_t h01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(z, __builtin_bit_cast(fp4_bf162_t, q.x), sh, false);
    h01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(h01, __builtin_bit_cast(fp4_bf162_t, q.y), sh, true);
    fp4_short2_t h23 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(z, __builtin_bit_cast(fp4_bf162_t, q.z), sh, false);
    h23 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(h23, __builtin_bit_cast(fp4_bf162_t, q.w), sh, true);
    const uint32_t hb01 = __builtin_bit_cast(uint32_t, h01), hb23 = __builtin_bit_cast(uint32_t, h23);
    // residuals x - hi (exact in fp32), then their e4m3 bytes at the lo scale
    auto res = [](uint32_t w, fp4_float2_t hf, int half) {
        const float x = __builtin_bit_cast(float, half ? (w & 0xFFFF0000u) : (w << 16));
        return x - hf[half];
    };
    const fp4_float2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hb01, sh, false);
    const fp4_float2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hb01, sh, true);
    const fp4_float2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hb23, sh, false);
    const fp4_float2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hb23, sh, true);
    fp4_short2_t l01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, res(q.x, f0, 0), res(q.x, f0, 1), sl, false);
    l01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l01, res(q.y, f1, 0), res(q.y, f1, 1), sl, true);
    fp4_short2_t l23 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, res(q.z, f2, 0), res(q.z, f2, 1), sl, false);
    l23 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l23, res(q.w, f3, 0), res(q.w, f3, 1), sl, true);
    const uint32_t lb01 = __builtin_bit_cast(uint32_t, l01), lb23 = __builtin_bit_cast(uint32_t, l23);
    hi_even = __builtin_amdgcn_perm(hb23, hb01, 0x06040200u);
    hi_odd = __builtin_amdgcn_perm(hb23, hb01, 0x07050301u);
    lo_even = __builtin_amdgcn_perm(lb23, lb01, 0x06040200u);
    lo_odd = __builtin_amdgcn_perm(lb23, lb01, 0x07050301u);
}

// D = A * B + C on the matrix cores: A e4m3 with per-lane block scale sa
// (E8M0), B e2m1 (scale 1).
__device__ __forceinline__ fp4_float4_t mfma_f8f4(const fp4_int8v_t &av, const uint4 &b, const fp4_float4_t &c,
                                                  uint32_t sa) {
    const fp4_int8v_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0 /* A e4m3 */, 4 /* B e2m1 */, 0,
                                                            (int)sa, 0, 127);
}

// 8 code bytes -> 32 e2m1 weights (+-2 / 0) in the K order above.
__device__ __forceinline__ uint4 fp4_weights(uint32_t w0, uint32_t w1) {
    const uint64_t v = sign_nz_fields64<true>((uint64_t)w0 | ((uint64_t)w1 << 32));
    const uint64_t e = shl64<2, true>(v);
    return make_uint4((uint32_t)e & 0xCCCCCCCCu, (uint32_t)v & 0xCCCCCCCCu, (uint32_t)(e >> 32) & 0xCCCCCCCCu,
                      (uint32_t)(v >> 32) & 0xCCCCCCCCu);
}

}  // namespace tern
