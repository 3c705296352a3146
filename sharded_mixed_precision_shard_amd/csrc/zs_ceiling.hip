// zs_ceiling.hip -- a plain streaming copy for gfx950, the in-run bandwidth
// ceiling that bench.py measures beside the shard step (measurement only;
// the step never calls it).
//
// Same access pattern as the step: 256-thread workgroups, each lane moving
// one 16-byte quad per sub-window, every instruction of a wavefront one
// dense 1 KB run, non-temporal loads and stores, one 4 KB tile per
// workgroup.  It reads each byte once and writes each byte once, so its
// rate is the best a one-read-one-write stream reaches on the same box and
// allocation pattern.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
// A dispatch packet holds the grid size in work-items as a 32-bit number.
constexpr int64_t kMaxBlocks = 0xffffffffLL / kThreads;

// quads [q0, q1) of src -> dst, one quad per thread per tile, tiles strided
// by the grid.
__global__ __launch_bounds__(kThreads) void stream_copy(const f32x4 *__restrict__ src,
                                                        f32x4 *__restrict__ dst, int64_t nq) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nq; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

extern "C" {

// Copy `bytes` bytes (a multiple of 16; both pointers 16-byte aligned DEVICE
// memory, not overlapping) on `stream`.  Returns 0, -1 on a bad argument
// (nothing enqueued) or the hipError_t of the launch.
int zs_ceiling_copy(const void *src, void *dst, int64_t bytes, void *stream) {
    if (bytes < 0 || bytes % 16 || (!src && bytes) || (!dst && bytes)) return -1;
    if (((uintptr_t)src | (uintptr_t)dst) & 15u) return -1;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (bytes && s0 < d0 + (uintptr_t)bytes && d0 < s0 + (uintptr_t)bytes) return -1;
    const int64_t nq = bytes / 16;
    if (nq == 0) return 0;
    int64_t blocks = (nq + kThreads - 1) / kThreads;
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    hipLaunchKernelGGL(stream_copy, dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, (const f32x4 *)src, (f32x4 *)dst, nq);
    return (int)hipGetLastError();
}

}  // extern "C"
