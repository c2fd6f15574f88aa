// tern_device.h -- device-side helpers shared by the HIP kernels of libtern.
//
// Weight decode (2kiu.com/news/5082861 §3.1): a 32-bit word read from a
// packed row holds 16 consecutive weights, weight i in bits 2i..2i+1, codes
// 00 -> 0, 01 -> +1, 10 -> -1, 11 -> 0.
//
// The kernels never build the integer weight.  They turn the code word into
// pairs of 16-bit floats whose value is 2t (t in {-1,0,+1}):
//   1. v = w ^ ((w >> 1) & 0x5555...): each 2-bit field becomes
//      [sign = bit1, nonzero = bit0 ^ bit1]; code 11 turns into [1, 0].
//   2. pair i (0..7) = (v << (14 - 2i)) & 0xC000C000 places the field of
//      weight i at bits 15..14 and the field of weight i+8 at bits 31..30.
//      A 16-bit value whose only set bits are 15 (sign) and 14 is +-2.0 in
//      both fp16 and bf16, and +-0 when bit 14 is clear.
// A packed dot (v_dot2_f32_f16 / _bf16) of such a pair with the activation
// pair {x[i], x[i+8]} then adds +2x, subtracts 2x or skips, in fp32: the
// pages' add / subtract / skip, two weights per instruction.  The factor two
// is removed with the scale (exact: a power of two).
//
// Activations are stored "pair-interleaved" so the pair {x[16c+i], x[16c+i+8]}
// is one 32-bit word: within each block of 16 elements, position 2i holds
// element i and position 2i+1 holds element i+8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tern {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

// Field transform: [bit1, bit0] -> [sign, nonzero] for all 16 fields.
__device__ __forceinline__ uint32_t sign_nz_fields(uint32_t w) {
    return w ^ ((w >> 1) & 0x55555555u);
}

// 64-bit shifts of a register pair.  On gfx950 v_lshlrev_b64 issues at the
// same rate as a 32-bit shift, so one instruction moves the fields of two
// code words; the compiler would split it into two 32-bit operations.
//
// MC = true (kernels that issue matrix-core instructions) takes the plain C++
// shift instead.  The inline-asm form hides the instruction from the
// compiler's hazard recognizer, which then does not keep it away from an
// MFMA still in flight: an MFMA writes its result registers many cycles
// after it issues, and the register allocator may hand a result register
// the program never reads (an unused D row) to the asm output, which the
// MFMA then overwrites.  Measured on the fp4 decode kernel: the even-weight
// nibbles of one operand, written by the asm shift three instructions after
// an MFMA whose unused D rows shared their registers, came out zero.
template <int S, bool MC = false>
__device__ __forceinline__ uint64_t shl64(uint64_t v) {
    if constexpr (S == 0 || MC) {
        return v << S;
    } else {
        uint64_t r;
        asm("v_lshlrev_b64 %0, %1, %2" : "=v"(r) : "i"(S), "v"(v));
        return r;
    }
}
template <bool MC = false>
__device__ __forceinline__ uint64_t shr64_1(uint64_t v) {
    if constexpr (MC) {
        return v >> 1;
    } else {
        uint64_t r;
        asm("v_lshrrev_b64 %0, 1, %1" : "=v"(r) : "v"(v));
        return r;
    }
}

// Field transform of two code words at once (bits that cross between the
// words are cleared by the 0x5555... mask).
template <bool MC = false>
__device__ __forceinline__ uint64_t sign_nz_fields64(uint64_t w) {
    return w ^ (shr64_1<MC>(w) & 0x5555555555555555ull);
}

// +-2 / 0 pairs for weights (i, i+8) of both words of a transformed pair:
// after a 64-bit shift by 14 - 2i, the bits that cross from the low word
// into the high word land below bit 14 and are masked away.
template <int I, bool MC = false>
__device__ __forceinline__ void weight_pairs2(uint64_t v, uint32_t &lo, uint32_t &hi) {
    const uint64_t t = shl64<14 - 2 * I, MC>(v);
    lo = (uint32_t)t & 0xC000C000u;
    hi = (uint32_t)(t >> 32) & 0xC000C000u;
}

// 0xFFFF in each 16-bit half whose bit 15 is set, 0 elsewhere.
__device__ __forceinline__ uint32_t half_masks(uint32_t u) {
    typedef short short2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(short2_t, u) >> (short2_t){15, 15});
}

// Exact fp16 products t*s for weights (i, i+8) of both words of a transformed
// pair, s2 = the scale's bits in both halves: s with the code's sign where the
// field is nonzero, +0 where it is zero (codes 00 and 11).  No arithmetic, so
// every finite scale gives its exact product.
template <int I, bool MC = false>
__device__ __forceinline__ void scaled_pairs2(uint64_t v, uint32_t s2, uint32_t &lo, uint32_t &hi) {
    const uint64_t t = shl64<14 - 2 * I, MC>(v);   // signs at bits 15, 31 (and 47, 63)
    const uint64_t u = shl64<15 - 2 * I, MC>(v);   // nonzero flags at bits 15, 31 (and 47, 63)
    lo = (((uint32_t)t & 0x80008000u) ^ s2) & half_masks((uint32_t)u);
    hi = (((uint32_t)(t >> 32) & 0x80008000u) ^ s2) & half_masks((uint32_t)(u >> 32));
}

// +-2 / 0 pair for weights (i, i+8) of a transformed word.
template <int I>
__device__ __forceinline__ uint32_t weight_pair(uint32_t v) {
    static_assert(I >= 0 && I < 8, "pair index");
    return (v << (14 - 2 * I)) & 0xC000C000u;
}

// acc + a.lo*b.lo + a.hi*b.hi with fp16 or bf16 operands, fp32 accumulate.
template <bool BF16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    if constexpr (BF16) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                               __builtin_bit_cast(bf162_t, b), acc, false);
    } else {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a),
                                      __builtin_bit_cast(half2_t, b), acc, false);
    }
}

// Pair {lo16(a), lo16(b)} and {hi16(a), hi16(b)}.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// 16 consecutive activations (two 16-byte vectors lo = x[0..7], hi = x[8..15])
// -> 8 pair-interleaved words {x[i], x[i+8]}, i = 0..7.
__device__ __forceinline__ void interleave16(const uint4 &lo, const uint4 &hi, uint32_t out[8]) {
    out[0] = pair_lo(lo.x, hi.x);
    out[1] = pair_hi(lo.x, hi.x);
    out[2] = pair_lo(lo.y, hi.y);
    out[3] = pair_hi(lo.y, hi.y);
    out[4] = pair_lo(lo.z, hi.z);
    out[5] = pair_hi(lo.z, hi.z);
    out[6] = pair_lo(lo.w, hi.w);
    out[7] = pair_hi(lo.w, hi.w);
}

__device__ __forceinline__ float f16_bits_to_float(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// fp32 -> output element, round to nearest even (overflow -> inf).
template <int YT>
__device__ __forceinline__ void store_out(void *Y, int64_t idx, float v) {
    if constexpr (YT == 2) {
        static_cast<float *>(Y)[idx] = v;
    } else if constexpr (YT == 1) {
        static_cast<__bf16 *>(Y)[idx] = static_cast<__bf16>(v);
    } else {
        static_cast<_Float16 *>(Y)[idx] = static_cast<_Float16>(v);
    }
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
// The rotated operand is written as an update_dpp with old = 0 and every
// lane valid (row rotations never leave a row), which lets the compiler fold
// each move into its add (one v_add_f32 with a DPP source per step).
__device__ __forceinline__ float row16_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xF, 0xF, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xF, 0xF, true));
    return x;
}

}  // namespace tern
