// tern_pack.hip -- packed-layout utilities: pack, unpack, block map, zero fill.
//
// Layout (2kiu.com/news/5082861 §3.1): weight 4j+i of a row lives in bits
// 2i..2i+1 of byte j of that row, codes 00 -> 0, 01 -> +1, 10 -> -1,
// 11 -> reserved (read as 0).  Because K % 4 == 0, byte j of the whole
// packed matrix always comes from the four int8 weights 4j..4j+3 of the
// flattened T, so both kernels run over the flat arrays.
#include <hip/hip_runtime.h>

#include "tern_kernels.h"

namespace tern {

namespace {

// Code of one int8 weight: -1, 0, +1 -> 10, 00, 01; anything else -> 11.
__device__ __forceinline__ uint32_t code_of(uint32_t byte) {
    const int t = static_cast<int8_t>(byte & 0xFFu);
    return t == 0 ? 0u : (t == 1 ? 1u : (t == -1 ? 2u : 3u));
}

// Four int8 weights (one 32-bit word) -> one packed byte.
__device__ __forceinline__ uint32_t pack_word(uint32_t w) {
    return code_of(w) | (code_of(w >> 8) << 2) | (code_of(w >> 16) << 4) | (code_of(w >> 24) << 6);
}

// One packed byte -> four int8 weights (one 32-bit word): t = bit0 - bit1.
__device__ __forceinline__ uint32_t unpack_byte(uint32_t b) {
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t c = (b >> (2 * i)) & 3u;
        const int t = static_cast<int>(c & 1u) - static_cast<int>(c >> 1);
        out |= (static_cast<uint32_t>(t) & 0xFFu) << (8 * i);
    }
    return out;
}

// Each vector step: 16 int8 in (one 16-byte load) -> 4 packed bytes out.
__global__ void pack_kernel(const int8_t *__restrict__ T, uint8_t *__restrict__ P, int64_t n_bytes) {
    const int64_t n_vec = n_bytes >> 2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec; i += stride) {
        const uint4 w = reinterpret_cast<const uint4 *>(T)[i];
        const uint32_t out = pack_word(w.x) | (pack_word(w.y) << 8) | (pack_word(w.z) << 16) |
                             (pack_word(w.w) << 24);
        reinterpret_cast<uint32_t *>(P)[i] = out;
    }
    // tail: the last n_bytes % 4 packed bytes
    for (int64_t j = (n_vec << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_bytes; j += stride) {
        const uint32_t w = static_cast<uint32_t>(static_cast<uint8_t>(T[4 * j])) |
                           (static_cast<uint32_t>(static_cast<uint8_t>(T[4 * j + 1])) << 8) |
                           (static_cast<uint32_t>(static_cast<uint8_t>(T[4 * j + 2])) << 16) |
                           (static_cast<uint32_t>(static_cast<uint8_t>(T[4 * j + 3])) << 24);
        P[j] = static_cast<uint8_t>(pack_word(w));
    }
}

// Each vector step: 4 packed bytes in (one 4-byte load) -> 16 int8 out.
__global__ void unpack_kernel(const uint8_t *__restrict__ P, int8_t *__restrict__ T, int64_t n_bytes) {
    const int64_t n_vec = n_bytes >> 2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec; i += stride) {
        const uint32_t w = reinterpret_cast<const uint32_t *>(P)[i];
        uint4 out;
        out.x = unpack_byte(w & 0xFFu);
        out.y = unpack_byte((w >> 8) & 0xFFu);
        out.z = unpack_byte((w >> 16) & 0xFFu);
        out.w = unpack_byte(w >> 24);
        reinterpret_cast<uint4 *>(T)[i] = out;
    }
    for (int64_t j = (n_vec << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_bytes; j += stride) {
        const uint32_t o = unpack_byte(P[j]);
        T[4 * j] = static_cast<int8_t>(o & 0xFFu);
        T[4 * j + 1] = static_cast<int8_t>((o >> 8) & 0xFFu);
        T[4 * j + 2] = static_cast<int8_t>((o >> 16) & 0xFFu);
        T[4 * j + 3] = static_cast<int8_t>(o >> 24);
    }
}

// Block map: one thread per map word (32 blocks of 128 weights = 32 x 32
// bytes of one row).  A code is a nonzero weight exactly when its two bits
// differ (01 or 10), so a block is marked when (w ^ (w >> 1)) & 0x5555...
// is nonzero for any of its eight 32-bit words.
__global__ void block_map_kernel(const uint8_t *__restrict__ P, uint32_t *__restrict__ map, int64_t N,
                                 int64_t groups, int64_t words) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t row_bytes = groups * 32;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < N * words; i += stride) {
        const int64_t n = i / words;
        const int64_t g0 = (i - n * words) * 32;
        const int64_t g1 = min(g0 + 32, groups);
        uint32_t bits = 0;
        for (int64_t g = g0; g < g1; ++g) {
            const uint4 *src = reinterpret_cast<const uint4 *>(P + n * row_bytes + g * 32);
            const uint4 a = src[0];
            const uint4 b = src[1];
            const uint32_t any = ((a.x ^ (a.x >> 1)) | (a.y ^ (a.y >> 1)) | (a.z ^ (a.z >> 1)) |
                                  (a.w ^ (a.w >> 1)) | (b.x ^ (b.x >> 1)) | (b.y ^ (b.y >> 1)) |
                                  (b.z ^ (b.z >> 1)) | (b.w ^ (b.w >> 1))) & 0x55555555u;
            if (any) bits |= 1u << (g - g0);
        }
        map[i] = bits;
    }
}

__global__ void fill_zero_kernel(uint8_t *__restrict__ Y, int64_t bytes) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < bytes; i += stride) Y[i] = 0;
}

unsigned grid_for(int64_t items, int block) {
    int64_t g = (items + block - 1) / block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;  // grid-stride loops cover the rest
    return (unsigned)g;
}

}  // namespace

hipError_t launch_pack(const int8_t *T, uint8_t *P, int64_t n_bytes, hipStream_t stream) {
    const int block = 256;
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for((n_bytes >> 2) + 1, block)), dim3(block), 0, stream, T, P,
                       n_bytes);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *P, int8_t *T, int64_t n_bytes, hipStream_t stream) {
    const int block = 256;
    hipLaunchKernelGGL(unpack_kernel, dim3(grid_for((n_bytes >> 2) + 1, block)), dim3(block), 0, stream, P, T,
                       n_bytes);
    return hipGetLastError();
}

hipError_t launch_block_map(const uint8_t *P, uint32_t *map, int64_t N, int64_t K, hipStream_t stream) {
    const int block = 256;
    const int64_t groups = K / 128;
    const int64_t words = (groups + 31) / 32;
    hipLaunchKernelGGL(block_map_kernel, dim3(grid_for(N * words, block)), dim3(block), 0, stream, P, map, N,
                       groups, words);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *Y, int64_t bytes, hipStream_t stream) {
    const int block = 256;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(bytes, block)), dim3(block), 0, stream,
                       static_cast<uint8_t *>(Y), bytes);
    return hipGetLastError();
}

}  // namespace tern
