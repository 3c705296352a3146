// gen_device.hip -- seeded synthetic inputs on the GPU (twin of gen_host.c).
//
// Holds none of the optimizer's arithmetic: it only draws numbers, so that
// shards of hundreds of GB can be filled in HBM without a host round trip.
// The definition is the one stated in gen_host.c (SplitMix64 of Steele, Lea
// and Flood, used counter-style; Irwin-Hall sum of twelve 16-bit fields;
// one binary32 multiply by the caller's scale; bf16 by truncation; zero past
// valid_end).  This file implements it independently of the host twin.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t output(uint64_t key, uint64_t i) {
    return mix64(key + (i + 1u) * kGamma);
}

__device__ __forceinline__ float variate(uint64_t key, uint64_t hkey, uint64_t gi, float scale,
                                         uint32_t heavy_thresh, float heavy_scale) {
    int32_t s = 0;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const uint64_t x = output(key, 3u * gi + (uint64_t)q);
        s += (int32_t)(x & 0xffffu) + (int32_t)((x >> 16) & 0xffffu) +
             (int32_t)((x >> 32) & 0xffffu) + (int32_t)(x >> 48);
    }
    float sc = scale;
    if (heavy_thresh != 0u && (uint32_t)(output(hkey, gi) >> 32) < heavy_thresh) sc = heavy_scale;
    return (float)(s - 393210) * sc;
}

__global__ __launch_bounds__(256) void fill_f32(float *out, int64_t n, uint64_t key,
                                                uint64_t hkey, int64_t index0, int64_t valid_end,
                                                float scale, uint32_t heavy_thresh,
                                                float heavy_scale) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int64_t gi = index0 + i;
        out[i] = gi < valid_end
                     ? variate(key, hkey, (uint64_t)gi, scale, heavy_thresh, heavy_scale)
                     : 0.0f;
    }
}

__global__ __launch_bounds__(256) void fill_bf16(uint16_t *out, int64_t n, uint64_t key,
                                                 uint64_t hkey, int64_t index0,
                                                 int64_t valid_end, float scale,
                                                 uint32_t heavy_thresh, float heavy_scale) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int64_t gi = index0 + i;
        uint32_t u = 0;
        if (gi < valid_end)
            u = __float_as_uint(
                variate(key, hkey, (uint64_t)gi, scale, heavy_thresh, heavy_scale));
        out[i] = (uint16_t)(u >> 16);
    }
}

__global__ __launch_bounds__(256) void fill_q8(int8_t *out, int64_t n, uint64_t key,
                                               int64_t index0, int64_t valid_end) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int64_t gi = index0 + i;
        int32_t q = 0;
        if (gi < valid_end) {
            int32_t s = 0;
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const uint64_t x = output(key, 3u * (uint64_t)gi + (uint64_t)r);
                s += (int32_t)(x & 0xffffu) + (int32_t)((x >> 16) & 0xffffu) +
                     (int32_t)((x >> 32) & 0xffffu) + (int32_t)(x >> 48);
            }
            q = (s - 393210) / 1560;
            q = q > 127 ? 127 : (q < -127 ? -127 : q);
        }
        out[i] = (int8_t)q;
    }
}

__global__ __launch_bounds__(256) void fill_scales(float *out, int64_t nblocks, uint64_t skey,
                                                   int64_t block0, float base) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += stride) {
        const uint64_t h = output(skey, (uint64_t)(block0 + b));
        const float f = (float)(1024u + (uint32_t)(h & 1023u)) * 0.0009765625f;
        out[b] = base * f;
    }
}

unsigned grid_for(int64_t n) {
    int64_t b = (n + 255) / 256;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return (unsigned)b;
}

}  // namespace

extern "C" {

// Both return a hipError_t (0 on success).  out is a device pointer of n
// elements; nothing is launched for n <= 0.
int synth_dev_normal_f32(float *out, int64_t n, uint64_t key, uint64_t hkey, int64_t index0,
                         int64_t valid_end, float scale, uint32_t heavy_thresh,
                         float heavy_scale, void *stream) {
    if (n <= 0) return 0;
    if (!out) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(fill_f32, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, out, n,
                       key, hkey, index0, valid_end, scale, heavy_thresh, heavy_scale);
    return (int)hipGetLastError();
}

int synth_dev_normal_bf16(uint16_t *out, int64_t n, uint64_t key, uint64_t hkey, int64_t index0,
                          int64_t valid_end, float scale, uint32_t heavy_thresh,
                          float heavy_scale, void *stream) {
    if (n <= 0) return 0;
    if (!out) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(fill_bf16, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, out, n,
                       key, hkey, index0, valid_end, scale, heavy_thresh, heavy_scale);
    return (int)hipGetLastError();
}

// Int8 partials and their block scales (definition in gen_host.c).
int synth_dev_q8(int8_t *out, int64_t n, uint64_t key, int64_t index0, int64_t valid_end,
                 void *stream) {
    if (n <= 0) return 0;
    if (!out) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(fill_q8, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, out, n, key,
                       index0, valid_end);
    return (int)hipGetLastError();
}

int synth_dev_q8_scales(float *out, int64_t nblocks, uint64_t skey, int64_t block0, float base,
                        void *stream) {
    if (nblocks <= 0) return 0;
    if (!out) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(fill_scales, dim3(grid_for(nblocks)), dim3(256), 0, (hipStream_t)stream,
                       out, nblocks, skey, block0, base);
    return (int)hipGetLastError();
}

}  // extern "C"
