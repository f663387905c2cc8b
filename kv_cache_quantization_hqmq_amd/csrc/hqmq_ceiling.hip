// Measured machine ceilings (declared in include/hqmq_ceiling.h): plain
// streaming loops over HBM and arithmetic loops on the VALU and the matrix
// cores, for the benchmark's context figures.  Not part of the codec.
#include <hip/hip_runtime.h>

#include "hqmq.h"
#include "hqmq_ceiling.h"
#include "hqmq_device.h"

namespace {

using hqmq::f16x4;
using hqmq::f32x16;
using hqmq::f32x4;
using hqmq::u32x4;

constexpr int kCeilThreads = 256;
constexpr uint32_t kNever = 0x9E3779B9u;    // a result the loops are not expected to produce

// Streaming loops shaped like the codec's bandwidth-bound kernels: every
// thread issues kStreamUnroll independent 16-byte accesses before using any,
// and a block covers kStreamUnroll * 256 consecutive 16-byte elements
// (element u * 256 + thread of the block's range, so each access
// instruction of a wave touches 1 KB of consecutive bytes).  One pass, no
// grid-stride loop: the grid has one block per range.
constexpr int kStreamUnroll = 8;
constexpr size_t kStreamBlockElems = static_cast<size_t>(kStreamUnroll) * kCeilThreads;

__global__ __launch_bounds__(kCeilThreads) void ceil_read_kernel(const u32x4 *a, size_t n, uint32_t *out) {
    const size_t base = static_cast<size_t>(blockIdx.x) * kStreamBlockElems + threadIdx.x;
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
        const size_t i = base + static_cast<size_t>(u) * kCeilThreads;
        v[u] = i < n ? __builtin_nontemporal_load(a + i) : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 acc = v[0];
#pragma unroll
    for (int u = 1; u < kStreamUnroll; ++u) acc ^= v[u];
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == kNever) out[0] = 1u;
}

__global__ __launch_bounds__(kCeilThreads) void ceil_write_kernel(u32x4 *b, size_t n) {
    const size_t base = static_cast<size_t>(blockIdx.x) * kStreamBlockElems + threadIdx.x;
    const u32x4 v = {threadIdx.x, blockIdx.x, 1u, 2u};
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
        const size_t i = base + static_cast<size_t>(u) * kCeilThreads;
        if (i < n) __builtin_nontemporal_store(v, b + i);
    }
}

__global__ __launch_bounds__(kCeilThreads) void ceil_copy_kernel(const u32x4 *a, u32x4 *b, size_t n) {
    const size_t base = static_cast<size_t>(blockIdx.x) * kStreamBlockElems + threadIdx.x;
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
        const size_t i = base + static_cast<size_t>(u) * kCeilThreads;
        v[u] = i < n ? __builtin_nontemporal_load(a + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
        const size_t i = base + static_cast<size_t>(u) * kCeilThreads;
        if (i < n) __builtin_nontemporal_store(v[u], b + i);
    }
}

// 16 independent FMA chains per lane (32 flops per lane per round).
__global__ __launch_bounds__(kCeilThreads) void ceil_fma_kernel(int64_t iters, float *sink) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 1.0f + 1e-3f * static_cast<float>(threadIdx.x + i);
    const float b = 0.999f + 1e-7f * static_cast<float>(blockIdx.x & 7), c = 1e-3f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = __builtin_fmaf(v[i], b, c);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += v[i];
    if (__float_as_uint(s) == kNever) sink[0] = s;
}

// 4 independent 16x16x4 fp32 accumulators per wave (4 x 2048 flops per round).
__global__ __launch_bounds__(kCeilThreads) void ceil_mfma_f32_kernel(int64_t iters, float *sink) {
    const float av = 1e-3f * static_cast<float>(threadIdx.x & 63), bv = 1e-3f;
    f32x4 d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, d[j], 0, 0, 0);
    }
    const float s = d[0][0] + d[1][1] + d[2][2] + d[3][3];
    if (__float_as_uint(s) == kNever) sink[0] = s;
}

// 2 independent 32x32x8 f16 accumulators per wave (2 x 16384 flops per round).
__global__ __launch_bounds__(kCeilThreads) void ceil_mfma_f16_kernel(int64_t iters, float *sink) {
    const _Float16 h = static_cast<_Float16>(1e-3f * static_cast<float>(threadIdx.x & 63));
    const f16x4 av = {h, h, h, h}, bv = {h, h, h, h};
    f32x16 d[2] = {};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 2; ++j) d[j] = __builtin_amdgcn_mfma_f32_32x32x8f16(av, bv, d[j], 0, 0, 0);
    }
    const float s = d[0][0] + d[1][15];
    if (__float_as_uint(s) == kNever) sink[0] = s;
}

}  // namespace

extern "C" int hqmq_ceiling_stream(int kind, const void *src, void *dst, size_t bytes, hipStream_t stream) {
    if (bytes == 0 || bytes % 16 != 0) return HQMQ_EINVAL;
    if (kind != HQMQ_CEIL_READ && kind != HQMQ_CEIL_WRITE && kind != HQMQ_CEIL_COPY) return HQMQ_EINVAL;
    if (kind != HQMQ_CEIL_WRITE && (src == nullptr || reinterpret_cast<uintptr_t>(src) % 16 != 0)) return HQMQ_EINVAL;
    if (dst == nullptr || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return HQMQ_EINVAL;
    const size_t n = bytes / 16;
    const size_t blocks = (n + kStreamBlockElems - 1) / kStreamBlockElems;
    if (blocks >= (size_t{1} << 31)) return HQMQ_EINVAL;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (kind == HQMQ_CEIL_READ)
        hipLaunchKernelGGL(ceil_read_kernel, grid, dim3(kCeilThreads), 0, stream, static_cast<const u32x4 *>(src), n,
                           static_cast<uint32_t *>(dst));
    else if (kind == HQMQ_CEIL_WRITE)
        hipLaunchKernelGGL(ceil_write_kernel, grid, dim3(kCeilThreads), 0, stream, static_cast<u32x4 *>(dst), n);
    else
        hipLaunchKernelGGL(ceil_copy_kernel, grid, dim3(kCeilThreads), 0, stream, static_cast<const u32x4 *>(src),
                           static_cast<u32x4 *>(dst), n);
    return hipGetLastError() == hipSuccess ? HQMQ_OK : HQMQ_EHIP;
}

extern "C" int hqmq_ceiling_compute(int kind, int64_t iterations, float *sink, hipStream_t stream, double *flops) {
    if (iterations < 1 || sink == nullptr || flops == nullptr) return HQMQ_EINVAL;
    if (kind != HQMQ_CEIL_FMA_F32 && kind != HQMQ_CEIL_MFMA_F32 && kind != HQMQ_CEIL_MFMA_F16) return HQMQ_EINVAL;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return HQMQ_EHIP;
    // 8 blocks of 4 waves per CU: 8 waves on each SIMD
    const int64_t blocks = static_cast<int64_t>(cus) * 8;
    const int64_t waves = blocks * (kCeilThreads / 64);
    const dim3 grid(static_cast<unsigned>(blocks));
    if (kind == HQMQ_CEIL_FMA_F32) {
        hipLaunchKernelGGL(ceil_fma_kernel, grid, dim3(kCeilThreads), 0, stream, iterations, sink);
        *flops = static_cast<double>(blocks) * kCeilThreads * static_cast<double>(iterations) * 32.0;
    } else if (kind == HQMQ_CEIL_MFMA_F32) {
        hipLaunchKernelGGL(ceil_mfma_f32_kernel, grid, dim3(kCeilThreads), 0, stream, iterations, sink);
        *flops = static_cast<double>(waves) * static_cast<double>(iterations) * 4.0 * 2048.0;
    } else {
        hipLaunchKernelGGL(ceil_mfma_f16_kernel, grid, dim3(kCeilThreads), 0, stream, iterations, sink);
        *flops = static_cast<double>(waves) * static_cast<double>(iterations) * 2.0 * 16384.0;
    }
    return hipGetLastError() == hipSuccess ? HQMQ_OK : HQMQ_EHIP;
}
