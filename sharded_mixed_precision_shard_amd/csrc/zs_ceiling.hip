// zs_ceiling.hip -- bandwidth ceilings for gfx950 that bench.py measures
// beside the shard step (measurement only; the step never calls them).
//
//  * zs_ceiling_copy: a plain streaming copy (one read stream, one write
//    stream), 16-byte non-temporal accesses, every wavefront instruction one
//    dense 1 KB run.
//  * zs_ceiling_twin: the step's own memory traffic with no arithmetic, on
//    the step's own buffers and in the step's own launch (grid, chunk, chunk
//    order, occupancy cap): every stream the step reads is read with the
//    same instruction shape and every stream it writes is written, in the
//    same order per wavefront.  Three modes: the whole step's traffic (each
//    state array is written back with the bits just read, so the state is
//    left as it was; the output arrays get arbitrary bytes), the read streams
//    alone, or the write streams alone (which overwrites the state).  Its
//    rate is what the memory system delivers for exactly this traffic on
//    this machine and this physical placement of the arrays.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWave = 64;
constexpr int kQuad = 4;                  // elements per lane per sub-window
constexpr int kSub = kWave * kQuad;       // 256 elements per wavefront window
constexpr int kTile = kSub * (kThreads / kWave);
constexpr int kMaxK = 16;
constexpr int kBlock = 256;               // int8 quantization block
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

// Stream layouts of the step's entry points.
constexpr int kLayoutBase = 0;    // f32 master/m/v, bf16 partials, bf16 param
constexpr int kLayoutQ8Out = 1;   // + int8 parameter copy and one f32 scale per block
constexpr int kLayoutQ8Grad = 2;  // int8 partials with one f32 scale per block each
constexpr int kLayoutBf16Mv = 4;  // bf16 m and v
constexpr int kLayoutPacked = 8;  // master, m, v packed per 256-element block in one array
                                  // (with kLayoutBf16Mv: fp32 master, then bf16 m and v)

// Modes: 0 = the step's reads and writes, then
constexpr int kModeRead = 1;   // its reads only
constexpr int kModeWrite = 2;  // its writes only

struct TwinArgs {
    float *master;
    void *m;
    void *v;
    uint16_t *param;
    int8_t *q8;
    float *q8_scale;
    const void *grads[kMaxK];
    const float *qscales[kMaxK];
    uint32_t *sink;   // one word, written only if a read-only pass meets a sentinel
    int64_t n;
    int64_t chunk;    // elements per workgroup, a multiple of kTile
    int32_t xcds;     // > 1: XCD-contiguous chunk order
    int32_t mode;
};

template <typename T>
__device__ __forceinline__ T ld(const void *p, int64_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const T *>(p) + i);
}
template <typename T>
__device__ __forceinline__ void st(void *p, int64_t i, T x) {
    __builtin_nontemporal_store(x, reinterpret_cast<T *>(p) + i);
}
// Hide a value from the optimizer so that a store of it is kept as it is.
template <typename T>
__device__ __forceinline__ void opaque(T &x) {
    asm volatile("" : "+v"(x));
}

// kQ: 256-element sub-windows each wave takes per tile, as the step's kernel
// in that launch (zs_launch_info.window_quads).
template <int K, int L, int kQ>
__global__ __launch_bounds__(kThreads) void twin_kernel(const TwinArgs a) {
    constexpr bool kMv16 = (L & kLayoutBf16Mv) != 0;
    constexpr bool kG8 = (L & kLayoutQ8Grad) != 0;
    constexpr bool kOut8 = (L & kLayoutQ8Out) != 0;
    constexpr bool kPk = (L & kLayoutPacked) != 0;
    constexpr int64_t kTileQ = (int64_t)kTile * kQ;
    const int lane = (int)(threadIdx.x % kWave);
    const int wave = (int)(threadIdx.x / kWave);
    int64_t b = blockIdx.x;
    if (a.xcds > 1) {
        const int64_t nb = gridDim.x, q = nb / a.xcds, r = nb % a.xcds;
        const int64_t x = b % a.xcds, y = b / a.xcds;
        b = x * q + (x < r ? x : r) + y;
    }
    const int64_t c0 = b * a.chunk;
    const int64_t c1 = (c0 + a.chunk < a.n) ? c0 + a.chunk : a.n;
    for (int64_t t0 = c0; t0 < c1; t0 += kTileQ) {
        const int64_t wv0 = t0 + (int64_t)wave * kSub * kQ;
        if (wv0 + kSub * kQ > c1) continue;  // whole windows only; the host sizes n to match
        int64_t qi[kQ];  // this lane's quad of each sub-window
        int64_t iw[kQ], im[kQ], iv[kQ];  // its master, m and v quads
#pragma unroll
        for (int qd = 0; qd < kQ; ++qd) {
            qi[qd] = (wv0 + (int64_t)qd * kSub) / kQuad + lane;
            if constexpr (kPk && kMv16) {
                // 2 KB per block: 1 KB of fp32 quads, then 512 B each of bf16 m, v quads
                const int64_t blk = (wv0 + (int64_t)qd * kSub) / kSub;
                iw[qd] = blk * (2 * kWave) + lane;
                im[qd] = blk * (4 * kWave) + 2 * kWave + lane;
                iv[qd] = im[qd] + kWave;
            } else if constexpr (kPk) {
                iw[qd] = (wv0 + (int64_t)qd * kSub) / kSub * (3 * kWave) + lane;
                im[qd] = iw[qd] + kWave;
                iv[qd] = iw[qd] + 2 * kWave;
            } else {
                iw[qd] = im[qd] = iv[qd] = qi[qd];
            }
        }
        void *const pm = kPk ? (void *)a.master : a.m;
        void *const pv = kPk ? (void *)a.master : a.v;
        if (a.mode == kModeWrite) {
            const f32x4 z = {1.0f, 2.0f, 3.0f, 4.0f};
            const u32x2 h = {0x3f803f80u, 0x3f803f80u};
#pragma unroll
            for (int qd = 0; qd < kQ; ++qd) {
                st<f32x4>(a.master, iw[qd], z);
                if constexpr (kMv16) {
                    st<u32x2>(pm, im[qd], h);
                    st<u32x2>(pv, iv[qd], h);
                } else {
                    st<f32x4>(pm, im[qd], z);
                    st<f32x4>(pv, iv[qd], z);
                }
                st<u32x2>(a.param, qi[qd], h);
                if constexpr (kOut8) {
                    st<uint32_t>(a.q8, qi[qd], 0x01010101u);
                    if (lane == 0) a.q8_scale[(wv0 + (int64_t)qd * kSub) / kBlock] = 1.0f;
                }
            }
            continue;
        }
        // every sub-window's loads first, as the step issues them
        f32x4 w[kQ], m[kQ], v[kQ];
        u32x2 mh[kQ], vh[kQ];
        u32x2 g[kQ][K];
        uint32_t g8[kQ][K];
        float s[kQ][K];
#pragma unroll
        for (int qd = 0; qd < kQ; ++qd) {
            w[qd] = ld<f32x4>(a.master, iw[qd]);
            if constexpr (kMv16) {
                mh[qd] = ld<u32x2>(pm, im[qd]);
                vh[qd] = ld<u32x2>(pv, iv[qd]);
            } else {
                m[qd] = ld<f32x4>(pm, im[qd]);
                v[qd] = ld<f32x4>(pv, iv[qd]);
            }
#pragma unroll
            for (int j = 0; j < K; ++j) {
                if constexpr (kG8) {
                    g8[qd][j] = ld<uint32_t>(a.grads[j], qi[qd]);
                    s[qd][j] = a.qscales[j][(wv0 + (int64_t)qd * kSub) / kBlock];
                } else {
                    g[qd][j] = ld<u32x2>(a.grads[j], qi[qd]);
                }
            }
        }
        if (a.mode == kModeRead) {
            uint32_t acc = 0;
#pragma unroll
            for (int qd = 0; qd < kQ; ++qd) {
                acc ^= __float_as_uint(w[qd][0]) ^ __float_as_uint(w[qd][1]) ^
                       __float_as_uint(w[qd][2]) ^ __float_as_uint(w[qd][3]);
                if constexpr (kMv16) {
                    acc ^= mh[qd][0] ^ mh[qd][1] ^ vh[qd][0] ^ vh[qd][1];
                } else {
                    acc ^= __float_as_uint(m[qd][0]) ^ __float_as_uint(m[qd][1]) ^
                           __float_as_uint(m[qd][2]) ^ __float_as_uint(m[qd][3]) ^
                           __float_as_uint(v[qd][0]) ^ __float_as_uint(v[qd][1]) ^
                           __float_as_uint(v[qd][2]) ^ __float_as_uint(v[qd][3]);
                }
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    if constexpr (kG8) acc ^= g8[qd][j] ^ __float_as_uint(s[qd][j]);
                    else acc ^= g[qd][j][0] ^ g[qd][j][1];
                }
            }
            if (acc == 0x9e3779b9u) a.sink[0] = acc;
            continue;
        }
        // The whole step's traffic: state written back bit for bit.  Every
        // value loaded is pinned, so that no load can be dropped as unused.
#pragma unroll
        for (int qd = 0; qd < kQ; ++qd) {
#pragma unroll
            for (int j = 0; j < K; ++j) {
                if constexpr (kG8) {
                    opaque(g8[qd][j]);
                    opaque(s[qd][j]);
                } else {
                    opaque(g[qd][j]);
                }
            }
            opaque(w[qd]);
            st<f32x4>(a.master, iw[qd], w[qd]);
            if constexpr (kMv16) {
                opaque(mh[qd]);
                opaque(vh[qd]);
                st<u32x2>(pm, im[qd], mh[qd]);
                st<u32x2>(pv, iv[qd], vh[qd]);
            } else {
                opaque(m[qd]);
                opaque(v[qd]);
                st<f32x4>(pm, im[qd], m[qd]);
                st<f32x4>(pv, iv[qd], v[qd]);
            }
            u32x2 p;
            if constexpr (kG8) {
                p[0] = g8[qd][0];
                p[1] = __float_as_uint(s[qd][0]);
            } else {
                p = g[qd][0];
            }
            opaque(p);
            st<u32x2>(a.param, qi[qd], p);
            if constexpr (kOut8) {
                st<uint32_t>(a.q8, qi[qd], p[0]);
                if (lane == 0) a.q8_scale[(wv0 + (int64_t)qd * kSub) / kBlock] = __uint_as_float(p[1]);
            }
        }
    }
}

typedef void (*twin_fn)(const TwinArgs);

template <int K, int Q>
twin_fn pick_layout(int layout) {
    switch (layout) {
        case kLayoutBase: return twin_kernel<K, kLayoutBase, Q>;
        case kLayoutQ8Out: return twin_kernel<K, kLayoutQ8Out, Q>;
        case kLayoutQ8Grad: return twin_kernel<K, kLayoutQ8Grad, Q>;
        case kLayoutBf16Mv: return twin_kernel<K, kLayoutBf16Mv, Q>;
        case kLayoutPacked: return twin_kernel<K, kLayoutPacked, Q>;
        case kLayoutPacked | kLayoutQ8Out: return twin_kernel<K, kLayoutPacked | kLayoutQ8Out, Q>;
        case kLayoutPacked | kLayoutQ8Grad: return twin_kernel<K, kLayoutPacked | kLayoutQ8Grad, Q>;
        case kLayoutPacked | kLayoutBf16Mv: return twin_kernel<K, kLayoutPacked | kLayoutBf16Mv, Q>;
        default: return nullptr;
    }
}

template <int K>
twin_fn pick_quads(int layout, int quads) {
    // two sub-windows per wave only where the step has such a kernel
    if (quads == 2) return (layout & kLayoutBf16Mv) ? pick_layout<K, 2>(layout) : nullptr;
    return quads == 1 ? pick_layout<K, 1>(layout) : nullptr;
}

twin_fn pick_twin(int k, int layout, int quads) {
    switch (k) {
        case 1: return pick_quads<1>(layout, quads);
        case 2: return pick_quads<2>(layout, quads);
        case 3: return pick_quads<3>(layout, quads);
        case 4: return pick_quads<4>(layout, quads);
        case 5: return pick_quads<5>(layout, quads);
        case 6: return pick_quads<6>(layout, quads);
        case 7: return pick_quads<7>(layout, quads);
        case 8: return pick_quads<8>(layout, quads);
        case 9: return pick_quads<9>(layout, quads);
        case 10: return pick_quads<10>(layout, quads);
        case 11: return pick_quads<11>(layout, quads);
        case 12: return pick_quads<12>(layout, quads);
        case 13: return pick_quads<13>(layout, quads);
        case 14: return pick_quads<14>(layout, quads);
        case 15: return pick_quads<15>(layout, quads);
        case 16: return pick_quads<16>(layout, quads);
        default: return nullptr;
    }
}

// Per device: one word the read-only mode may write, and the properties the
// launch needs (queried once; measurement code, not thread-safe).
struct DevState {
    uint32_t *sink;
    int cus;
    int64_t lds_per_cu, lds_per_group;
};
DevState g_dev[64];

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

// The step's traffic without its arithmetic (see the top of this file), on
// the calling thread's current device and `stream`.
//   mode: 0 = the step's reads and writes (state left bit for bit as it
//         was; param and the int8 copy receive arbitrary bytes), 1 = its
//         reads only, 2 = its writes only (state overwritten).
//   layout: 0 = zs_shard_step, 1 = zs_shard_step_q8ag, 2 = zs_shard_step_q8grad,
//         4 = zs_shard_step_bf16mv, 8 = zs_shard_step_packed, 9 and 10 = its
//         int8-payload and int8-partial forms, 12 = zs_shard_step_packed_bf16mv
//         (the streams and element sizes that entry point moves; with layouts
//         8-12 master is the packed state and m, v are unused).  grads holds
//         k device pointers (int8 with bit 2, bf16 otherwise); qscales (bit
//         2) k device pointers to one f32 per 256 elements; q8 and q8_scale
//         (bit 1) the int8 copy and its scales.
//   n: elements; a multiple of chunk and of the tile (1024 elements per
//         sub-window of a wave: the twin covers whole windows only, so the host
//         rounds a shard down to that).
//   chunk, block_order (1 linear, 2 XCD-contiguous), groups_per_cu (0 =
//         none), quads (sub-windows per wave: 1, or 2 with layouts 4 and 12): the
//         launch zs_launch_plan reports for the step.
// Every pointer is DEVICE memory sized for n elements, 16-byte aligned (the
// scale arrays 4-byte).  Returns 0, -1 on a bad argument (nothing enqueued),
// or a hipError_t.
int zs_ceiling_twin(int mode, int layout, float *master, void *m, void *v, uint16_t *param,
                    int8_t *q8, float *q8_scale, const void *const *grads,
                    const float *const *qscales, int k, int64_t n, int64_t chunk,
                    int block_order, int groups_per_cu, int quads, void *stream) {
    if (mode < 0 || mode > 2 || k < 1 || k > kMaxK || n < 0 || !grads) return -1;
    if (layout != kLayoutBase && layout != kLayoutQ8Out && layout != kLayoutQ8Grad &&
        layout != kLayoutBf16Mv && layout != kLayoutPacked &&
        layout != (kLayoutPacked | kLayoutQ8Out) && layout != (kLayoutPacked | kLayoutQ8Grad) &&
        layout != (kLayoutPacked | kLayoutBf16Mv))
        return -1;
    if (quads != 1 && quads != 2) return -1;
    const int64_t tile = (int64_t)kTile * quads;
    if (n % tile || chunk < tile || chunk % tile || (n && n % chunk)) return -1;
    if (block_order != 1 && block_order != 2) return -1;
    if (groups_per_cu < 0 || groups_per_cu > 32) return -1;
    const twin_fn fn = pick_twin(k, layout, quads);
    if (!fn) return -1;
    if (!master || !param || (!(layout & kLayoutPacked) && (!m || !v))) return -1;
    if ((layout & kLayoutQ8Out) && (!q8 || !q8_scale)) return -1;
    if ((layout & kLayoutQ8Grad) && !qscales) return -1;
    for (int j = 0; j < k; ++j)
        if (!grads[j] || ((layout & kLayoutQ8Grad) && !qscales[j])) return -1;
    if (n == 0) return 0;
    const int64_t blocks = n / chunk;
    if (blocks > kMaxBlocks) return -1;

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= 64) return -1;
    DevState &ds = g_dev[dev];
    if (!ds.sink) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return (int)e;
        ds.cus = prop.multiProcessorCount;
        ds.lds_per_cu = (int64_t)prop.maxSharedMemoryPerMultiProcessor;
        ds.lds_per_group = (int64_t)prop.sharedMemPerBlock;
        e = hipMalloc((void **)&ds.sink, sizeof(uint32_t));
        if (e != hipSuccess) return (int)e;
    }
    TwinArgs a = {};
    a.master = master;
    a.m = m;
    a.v = v;
    a.param = param;
    a.q8 = q8;
    a.q8_scale = q8_scale;
    for (int j = 0; j < k; ++j) {
        a.grads[j] = grads[j];
        a.qscales[j] = (layout & kLayoutQ8Grad) ? qscales[j] : nullptr;
    }
    a.sink = ds.sink;
    a.n = n;
    a.chunk = chunk;
    // as the step: the XCD count is the CU count over 32 on a whole part
    const int cus = ds.cus;
    a.xcds = (block_order == 2 && cus % 32 == 0 && cus >= 32) ? cus / 32 : 1;
    a.mode = mode;
    // as the step: a cap reserves 1/groups_per_cu of the CU's LDS per workgroup
    size_t dyn_lds = 0;
    if (groups_per_cu > 0) {
        const int64_t share = ds.lds_per_cu / groups_per_cu / 1024 * 1024;
        if (share > ds.lds_per_group) return -1;
        dyn_lds = (size_t)share;
    }
    void *args[] = {&a};
    e = hipLaunchKernel((const void *)fn, dim3((unsigned)blocks), dim3(kThreads), args, dyn_lds,
                        (hipStream_t)stream);
    return (int)e;
}

}  // extern "C"
