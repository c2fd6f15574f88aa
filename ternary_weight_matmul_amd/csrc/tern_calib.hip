// tern_calib.hip -- calibration kernel: a plain streaming read (or copy) of a
// device buffer, the ceiling the decode kernels are measured against.  It is
// no part of the product: it computes nothing of the method.
//
// Layout: 32 KB per workgroup of 512 threads; each thread issues four
// 16-byte loads at lane-contiguous offsets (one instruction reads 1 KB of
// consecutive bytes) before using any of them, non-temporal.  Measured on
// MI355X among the fastest of the plain-read layouts tried (1 KB contiguous,
// 4 rows x 128 or 256 bytes, 8 rows x 128 bytes, 8-byte loads; 256 to 1024
// threads; 1 to 16 loads per thread): 22.3 MB in 4.68-4.78 us, 6.55 MB in
// 2.36-2.5 us, graph-timed over rotated regions.  A read-only call folds the
// bytes into one word per thread and stores it only under a condition that
// never holds, so the loads cannot be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tern.h"

namespace {

constexpr int C_THREADS = 512;
constexpr int C_UNROLL = 4;
constexpr uint32_t C_CHUNK = C_THREADS * C_UNROLL * 16;   // bytes per workgroup

__device__ __forceinline__ __amdgpu_buffer_rsrc_t calib_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__global__ __launch_bounds__(C_THREADS) void stream_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                          uint64_t bytes, uint32_t *__restrict__ sink) {
    const uint64_t base = (uint64_t)blockIdx.x * C_CHUNK;
    const uint32_t n = (uint32_t)min<uint64_t>(C_CHUNK, bytes - base);   // bytes past n read as zero
    const __amdgpu_buffer_rsrc_t rs = calib_rsrc(src + base, n);
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    u32x4 v[C_UNROLL];
#pragma unroll
    for (int i = 0; i < C_UNROLL; ++i)
        v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (i * C_THREADS + threadIdx.x) * 16,
                                                                              0, 2 /* nt */));
    if (dst != nullptr) {
        const __amdgpu_buffer_rsrc_t rd = calib_rsrc(dst + base, n);   // stores past n are dropped
#pragma unroll
        for (int i = 0; i < C_UNROLL; ++i)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v[i]),
                                                   rd, (i * C_THREADS + threadIdx.x) * 16, 0, 2);
    } else {
        uint32_t acc = 0;
#pragma unroll
        for (int i = 0; i < C_UNROLL; ++i) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
        if (acc == 0x9E3779B9u + threadIdx.x && bytes == 0) sink[blockIdx.x & 1023] = acc;   // never taken
    }
}

__device__ uint32_t g_calib_sink[1024];

}  // namespace

extern "C" tern_status tern_stream_copy(const void *src, void *dst, uint64_t bytes, hipStream_t stream) {
    if (bytes == 0) return TERN_OK;
    if (src == nullptr) return TERN_ERR_NULL;
    if (bytes % 16 != 0 || bytes > (uint64_t(1) << 40)) return TERN_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0) return TERN_ERR_ALIGN;
    uint32_t *sink = nullptr;
    if (hipGetSymbolAddress(reinterpret_cast<void **>(&sink), HIP_SYMBOL(g_calib_sink)) != hipSuccess)
        return TERN_ERR_HIP;
    const uint64_t grid = (bytes + C_CHUNK - 1) / C_CHUNK;
    hipLaunchKernelGGL(stream_kernel, dim3((unsigned)grid), dim3(C_THREADS), 0, stream,
                       static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst), bytes, sink);
    return hipGetLastError() == hipSuccess ? TERN_OK : TERN_ERR_HIP;
}
