// Attainable-peak probes for gfx950 (measurement support, not part of the
// IndexShare path): dense MFMA throughput in bf16, fp8 and int8, LDS read
// bandwidth, and the HBM streaming-read rate.  bench.py times each probe with
// HIP events and reports the rates beside the published peaks its roofline
// fractions use.  Every probe writes a value derived from all its work to a
// sink so that nothing is removed as dead code.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef long v2l __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int PK_THREADS = 512;     // 8 waves per workgroup: 2 per SIMD
constexpr int PK_CHAINS = 4;        // independent accumulators per wave

__global__ __launch_bounds__(PK_THREADS) void mfma_bf16_kernel(float* sink, int iters, float seed) {
    v8bf a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
        b[i] = (__bf16)(seed * (float)(i - (int)threadIdx.x));
    }
    v16f acc[PK_CHAINS];
    for (int c = 0; c < PK_CHAINS; ++c)
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < PK_CHAINS; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
    for (int c = 0; c < PK_CHAINS; ++c)
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[blockIdx.x * PK_THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(PK_THREADS) void mfma_fp8_kernel(float* sink, int iters, int seed) {
    const long x = (long)seed * (threadIdx.x + 1);
    const v2l a = {x, x ^ 0x3C3C3C3C3C3C3C3CL}, b = {~x, x * 3};
    v16f acc[PK_CHAINS];
    for (int c = 0; c < PK_CHAINS; ++c)
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    // v_mfma_f32_32x32x64_f8f6f4 with both operands e4m3 (format code 0)
    typedef int v8i __attribute__((ext_vector_type(8)));
    v8i av = {(int)a[0], (int)(a[0] >> 32), (int)a[1], (int)(a[1] >> 32), 0, 0, 0, 0};
    v8i bv = {(int)b[0], (int)(b[0] >> 32), (int)b[1], (int)(b[1] >> 32), 0, 0, 0, 0};
    av[4] = av[0] ^ 0x11; av[5] = av[1]; av[6] = av[2]; av[7] = av[3];
    bv[4] = bv[0] ^ 0x22; bv[5] = bv[1]; bv[6] = bv[2]; bv[7] = bv[3];
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < PK_CHAINS; ++c)
            acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[c], 0, 0, 0, 127,
                                                                     0, 127);
    }
    float s = 0.0f;
    for (int c = 0; c < PK_CHAINS; ++c)
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[blockIdx.x * PK_THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(PK_THREADS) void mfma_i8_kernel(float* sink, int iters, int seed) {
    const int x = seed * (threadIdx.x + 1);
    const v4i a = {x, x ^ 0x5A5A5A5A, x * 7, x + 11}, b = {~x, x * 3, x ^ 0x0F0F0F0F, x - 5};
    v16i acc[PK_CHAINS];
    for (int c = 0; c < PK_CHAINS; ++c)
        for (int r = 0; r < 16; ++r) acc[c][r] = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < PK_CHAINS; ++c)
            acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
    }
    int s = 0;
    for (int c = 0; c < PK_CHAINS; ++c)
        for (int r = 0; r < 16; ++r) s ^= acc[c][r];
    sink[blockIdx.x * PK_THREADS + threadIdx.x] = (float)s;
}

// Every thread reads 16 bytes per step from a 64 KiB LDS array; the 64 lanes
// of a wave read 1 KiB of consecutive bytes (no bank conflicts).
constexpr int LDS_BYTES = 65536;
__global__ __launch_bounds__(1024) void lds_read_kernel(float* sink, int iters) {
    __shared__ __attribute__((aligned(16))) v4u lds[LDS_BYTES / 16];
    for (int i = threadIdx.x; i < LDS_BYTES / 16; i += 1024) lds[i] = v4u{(unsigned)i, 1u, 2u, 3u};
    __syncthreads();
    v4u acc = {0u, 0u, 0u, 0u};
    int p = threadIdx.x;
    for (int it = 0; it < iters; ++it) {
        // eight distinct 16-byte words per thread per step (offsets 512 words
        // apart inside the 4096-word array), a new set every step
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            acc ^= lds[(p + u * 512) & (LDS_BYTES / 16 - 1)];
        }
        p += 64 + (acc[0] & 0);
    }
    sink[blockIdx.x * 1024 + threadIdx.x] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

// Streaming read of n16 16-byte words, grid-stride, 4 loads in flight per thread.
__global__ __launch_bounds__(256) void hbm_read_kernel(const v4u* __restrict__ src, size_t n16,
                                                       float* sink) {
    v4u acc = {0u, 0u, 0u, 0u};
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const v4u a = __builtin_nontemporal_load(src + i);
        const v4u b = __builtin_nontemporal_load(src + i + stride);
        const v4u c = __builtin_nontemporal_load(src + i + 2 * stride);
        const v4u d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= src[i];
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9E3779B9u) sink[threadIdx.x] = 1.0f;
}

}  // namespace

extern "C" {

// Each launcher enqueues one probe on `stream` and returns the hipError_t.
// sink: device float array of at least grid * 1024 entries (grid <= 4096).
// Work: bf16 / fp8 / int8 probes do grid * 8 waves * iters * 4 MFMAs of
// 32x32x16 (32768 FLOP), 32x32x64 (131072 FLOP) and 32x32x32 (65536 OP);
// the LDS probe reads grid * 1024 threads * iters * 8 * 16 bytes.
int peaks_mfma_bf16(float* sink, int grid, int iters, void* stream) {
    hipLaunchKernelGGL(mfma_bf16_kernel, dim3(grid), dim3(PK_THREADS), 0, (hipStream_t)stream,
                       sink, iters, 0.001f);
    return (int)hipGetLastError();
}
int peaks_mfma_fp8(float* sink, int grid, int iters, void* stream) {
    hipLaunchKernelGGL(mfma_fp8_kernel, dim3(grid), dim3(PK_THREADS), 0, (hipStream_t)stream,
                       sink, iters, 12345);
    return (int)hipGetLastError();
}
int peaks_mfma_i8(float* sink, int grid, int iters, void* stream) {
    hipLaunchKernelGGL(mfma_i8_kernel, dim3(grid), dim3(PK_THREADS), 0, (hipStream_t)stream,
                       sink, iters, 12345);
    return (int)hipGetLastError();
}
int peaks_lds_read(float* sink, int grid, int iters, void* stream) {
    hipLaunchKernelGGL(lds_read_kernel, dim3(grid), dim3(1024), 0, (hipStream_t)stream, sink, iters);
    return (int)hipGetLastError();
}
// src: device buffer of n16 * 16 bytes, 16-byte aligned; sink: >= 256 floats
int peaks_hbm_read(const void* src, size_t n16, float* sink, int grid, void* stream) {
    hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const v4u*)src, n16, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
