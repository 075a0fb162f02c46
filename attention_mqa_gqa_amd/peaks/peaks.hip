// Attainable-peak probes for MI355X (gfx950): the ceilings the attention
// kernels are compared against, measured on the machine they run on.
//   * MFMA: back-to-back v_mfma_f32_32x32x16_bf16 (the prefill / MLA MFMA),
//     eight independent accumulators per wave, one or two waves per SIMD;
//     one wave also reads the shader clock counter (s_memtime) and the
//     constant 100 MHz counter (s_memrealtime) around its loop, which gives
//     the clock the MFMA loop actually ran at.
//   * HBM read: a streaming 16-byte-per-lane read of a large buffer (the
//     shape of a decode KV-cache scan).
//   * HBM copy: read one buffer, write another (a plain device copy).
//   * LDS read: ds_read_b128 from a 64 KB workgroup array.
// Each launch is timed by the caller (HIP events); the kernels write a
// checksum to `sink` so that no work is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mqa_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512) void peak_mfma_kernel(int iters, float* __restrict__ sink,
                                                        unsigned long long* __restrict__ clocks) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(lane + i));
        b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    f32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x16{};
    const bool timer = blockIdx.x == 0 && threadIdx.x < 64;
    unsigned long long t0 = 0, r0 = 0;
    if (timer) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[j][i];
    if (timer) {
        const unsigned long long t1 = __builtin_amdgcn_s_memtime();
        const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
        if (lane == 0) {
            clocks[0] = t1 - t0;
            clocks[1] = r1 - r0;
        }
    }
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each workgroup streams its own contiguous chunk of the buffer: four 16-byte
// non-temporal loads per lane in flight, so every wave instruction reads 1 KB
// of consecutive addresses (measured faster than a grid-stride loop over the
// whole buffer, 7.0 against 6.1 TB/s, and than plain loads, 5.9 TB/s).
__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                        float* __restrict__ sink) {
    const size_t chunk = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t beg = (size_t)blockIdx.x * chunk;
    const size_t end = beg + chunk < n16 ? beg + chunk : n16;
    uint32_t x = 0;
    size_t i = beg + threadIdx.x;
    for (; i + 3 * 256 < end; i += 4 * 256) {
        const u32x4 v0 = __builtin_nontemporal_load(src + i);
        const u32x4 v1 = __builtin_nontemporal_load(src + i + 256);
        const u32x4 v2 = __builtin_nontemporal_load(src + i + 512);
        const u32x4 v3 = __builtin_nontemporal_load(src + i + 768);
        x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
        x ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
    }
    for (; i < end; i += 256) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[blockIdx.x * blockDim.x + threadIdx.x] = (float)x;
}

// dst <- src, each workgroup over its own contiguous chunk, non-temporal
__global__ __launch_bounds__(256) void peak_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        size_t n16) {
    const size_t chunk = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t beg = (size_t)blockIdx.x * chunk;
    const size_t end = beg + chunk < n16 ? beg + chunk : n16;
    size_t i = beg + threadIdx.x;
    for (; i + 256 < end; i += 2 * 256) {
        const u32x4 v0 = __builtin_nontemporal_load(src + i);
        const u32x4 v1 = __builtin_nontemporal_load(src + i + 256);
        __builtin_nontemporal_store(v0, dst + i);
        __builtin_nontemporal_store(v1, dst + i + 256);
    }
    for (; i < end; i += 256) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Every lane reads 16 bytes per ds_read_b128; a wave's 64 reads cover 1 KB
// of consecutive addresses (no bank conflicts).
__global__ __launch_bounds__(1024) void peak_lds_kernel(int iters, float* __restrict__ sink) {
    __shared__ __attribute__((aligned(16))) u32x4 buf[4096];          // 64 KB
    for (int i = threadIdx.x; i < 4096; i += blockDim.x) buf[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    uint32_t x = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const u32x4 v = buf[((it * 8 + j + w) & 63) * 64 + lane];
            x += v.x ^ v.w;
        }
    }
    sink[blockIdx.x * blockDim.x + threadIdx.x] = (float)x;
}

int cus() {
    static const int n = [] {
        int dev = 0, c = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        return c;
    }();
    return n;
}

int status(hipError_t e) { return e == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" {

int mqa_peak_compute_units(void) { return cus(); }

size_t mqa_peak_sink_floats(int kind, int waves_per_simd) {
    const int n = cus();
    if (n <= 0) return 0;
    switch (kind) {
        case MQA_PEAK_MFMA: return (size_t)n * 256 * (waves_per_simd == 2 ? 2 : 1);
        case MQA_PEAK_READ: return (size_t)n * 8 * 256;
        case MQA_PEAK_LDS: return (size_t)n * 1024;
        default: return 0;
    }
}

int mqa_peak_mfma_bf16(int waves_per_simd, int iters, float* sink, unsigned long long* clocks, void* stream) {
    if ((waves_per_simd != 1 && waves_per_simd != 2) || iters <= 0 || !sink || !clocks) return -1;
    const int n = cus();
    if (n <= 0) return -4;
    hipLaunchKernelGGL(peak_mfma_kernel, dim3(n), dim3(256 * waves_per_simd), 0, (hipStream_t)stream, iters, sink,
                       clocks);
    return status(hipGetLastError());
}

int mqa_peak_hbm_read(const void* src, size_t bytes, float* sink, void* stream) {
    if (!src || !sink || bytes < 16 || ((uintptr_t)src & 15u)) return -1;
    const int n = cus();
    if (n <= 0) return -4;
    hipLaunchKernelGGL(peak_read_kernel, dim3(n * 4), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                       bytes / 16, sink);
    return status(hipGetLastError());
}

int mqa_peak_hbm_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || bytes < 16 || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return -1;
    const int n = cus();
    if (n <= 0) return -4;
    hipLaunchKernelGGL(peak_copy_kernel, dim3(n * 8), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                       (u32x4*)dst, bytes / 16);
    return status(hipGetLastError());
}

int mqa_peak_lds_read(int waves_per_cu, int iters, float* sink, void* stream) {
    if (waves_per_cu < 1 || waves_per_cu > 16 || iters <= 0 || !sink) return -1;
    const int n = cus();
    if (n <= 0) return -4;
    hipLaunchKernelGGL(peak_lds_kernel, dim3(n), dim3(64 * waves_per_cu), 0, (hipStream_t)stream, iters, sink);
    return status(hipGetLastError());
}

}  // extern "C"
