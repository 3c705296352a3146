// zs_step.hip -- fused reduce + AdamW + bf16-cast shard step for gfx950,
// and the C ABI declared in include/zs.h.
//
// One rank's share of the ZeRO-1 optimizer step ("Chapter 9: Distributed
// Training and Data Parallelism", section 9.4.2; "Lecture 7: Parallelism I",
// section 8.1): sum the k bf16 gradient partials the reduce-scatter delivers
// for this rank's chunk, run mixed-precision AdamW (section 9.2.2 of the
// first page) on the fp32 master, m and v, and write the bf16 parameter copy
// that the all-gather would broadcast.
//
// The work is purely elementwise and bandwidth bound (about 0.5 flop per HBM
// byte), so there is no MFMA here.  Design for CDNA4:
//   * a wavefront's window is Q sub-windows of 256 elements (Q = 1 for one
//     or two partials, 4 for more; a workgroup tile is four windows); lane
//     l owns elements 4l..4l+3 of each sub-window.  Every load and store
//     instruction of a wavefront is then one dense, contiguous run (1 KB per
//     fp32 array, 512 B per bf16 array) of 16-byte (fp32) or 8-byte (bf16)
//     accesses, and every byte is read once and written once;
//   * a workgroup owns a contiguous chunk of tiles (one tile by default: the
//     resident workgroups then sweep memory as one compact front);
//   * every wavefront resolves the weight-decay flags of its own window, with
//     no workgroup barrier and after issuing its loads (so the lookup
//     overlaps them): a 64-way search of the device table finds the entry
//     covering the window (two dependent loads for up to 4096 entries); a
//     window inside one segment takes that segment's flag, a window with
//     segment boundaries stages the 64 entries around it in the wave's LDS
//     slot and each lane walks them for its own elements;
//   * 64-bit element indices throughout (shards exceed 2^31 elements).
//
// Numerics follow the header: binary32, no contraction, correctly rounded
// divide and square root, denormals kept, bf16 round-to-nearest-even with
// NaN -> 0x7FC0.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "zs.h"

namespace {

constexpr int kThreads = 256;                 // 4 wavefronts of 64 lanes
constexpr int kWave = 64;
constexpr int kQuad = 4;                      // contiguous elements per lane per sub-window
constexpr int kSub = kWave * kQuad;           // 256: one dense instruction per array per wave

// Sub-windows (quads per lane) a wave handles per tile.  Measured on MI355X:
// with one or two partials the fewest bytes in flight per wave streamed best
// (one quad); with three or more partials each lane already has many loads
// in flight and four quads per lane streamed best.
constexpr int quads_for(int k) { return k <= 2 ? 1 : 4; }
constexpr int tile_for(int k) { return (kThreads / kWave) * quads_for(k) * kSub; }
constexpr int kMaxChunkTiles = 4096;
constexpr int64_t kNoStart = INT64_MAX;       // sentinel past the table end

static_assert(tile_for(1) == 1024 && tile_for(8) == 4096, "tile sizes");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct StepArgs {
    float *master;
    void *m;         // fp32 [n], or bf16 [n] in the bf16-moment variant
    void *v;
    uint16_t *param;
    int8_t *q8;      // quantized parameter copy (variant with an int8 payload)
    float *q8_scale;
    const uint16_t *grads[ZS_MAX_K];   // bf16 partials
    const int8_t *qgrads[ZS_MAX_K];    // int8 partials (block-quantized variant)
    const float *qscales[ZS_MAX_K];
    const zs_segment *segs;
    int64_t n;
    int64_t chunk;  // elements per workgroup, a multiple of kTile
    int32_t nseg;
    float lr, b1, b2, c1, c2, bc1, bc2, eps, df, gscale;
};

template <int NT, typename T>
__device__ __forceinline__ T load(const T *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int NT, typename T>
__device__ __forceinline__ void store(T *p, T x) {
    if constexpr (NT) __builtin_nontemporal_store(x, p);
    else *p = x;
}

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xffff0000u); }

// Round to nearest even by adding 0x7fff plus the lowest kept bit, then
// dropping 16 bits; NaN is mapped to the canonical quiet NaN.
__device__ __forceinline__ uint32_t to_bf16(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7fffffffu) > 0x7f800000u) ? 0x7fc0u : r;
}

// One element of the update: g is the reduced, scaled gradient.
__device__ __forceinline__ void adamw(float &w, float &m, float &v, float g, bool decay,
                                      const StepArgs &a) {
#pragma clang fp contract(off)
    const float m1 = a.b1 * m + a.c1 * g;
    const float v1 = a.b2 * v + a.c2 * (g * g);
    const float mh = m1 / a.bc1;
    const float vh = v1 / a.bc2;
    const float u = mh / (sqrtf(vh) + a.eps);
    const float wd = decay ? w * a.df : w;
    w = wd - a.lr * u;
    m = m1;
    v = v1;
}

// Largest s with segs[s].start <= e (0 if none); reads stay in [0, nseg).
__device__ int32_t last_le(const zs_segment *segs, int32_t nseg, int64_t e) {
    int32_t lo = 0, hi = nseg - 1;
    while (lo < hi) {
        const int32_t mid = lo + (hi - lo + 1) / 2;
        if (segs[mid].start <= e) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Per-wavefront LDS slot: the 64 table entries around a window that holds
// segment boundaries.
struct WaveSlot {
    int64_t start[kWave];
    uint8_t flag[kWave];
};

// Decay flags of this lane's elements in the window [w0, w1) (w0 < w1, both
// wave-uniform): bit q belongs to element q of the lane, whose index is
// elem(q), increasing in q; elements at or past w1 get no bit.  Done by the
// wavefront alone, with no workgroup barrier.  A 64-way search finds the
// entry covering w0: each round probes 64 entries at once and narrows the
// range 64-fold, and the last round loads 64 consecutive entries (two
// dependent loads in all for tables of up to 4096 entries).  A window inside
// one segment takes that segment's flag; a window that holds boundaries stages
// the 64 loaded entries in the wave's LDS slot and every lane walks them for
// its own elements; a window with more boundaries than the slot holds looks
// each element up in the table.  All 64 lanes must call this; every read
// stays inside segs[0 .. nseg-1] and the slot, sorted table or not.
template <typename ElemFn>
__device__ uint32_t window_mask(const StepArgs &a, int64_t w0, int64_t w1, int nelem,
                                ElemFn elem, WaveSlot &slot) {
    const int lane = (int)(threadIdx.x % kWave);
    int32_t lo = 0, hi = a.nseg;  // the entry covering w0 lies in [lo, hi)
    while (hi - lo > kWave) {
        const int32_t step = (hi - lo + kWave - 1) / kWave;
        const int64_t idx = (int64_t)lo + (int64_t)lane * step;
        const bool le = idx < hi && a.segs[idx].start <= w0;
        const uint64_t b = __ballot(le);
        const int top = b ? 63 - __clzll(b) : 0;
        lo = lo + top * step;
        hi = (lo + step < hi) ? lo + step : hi;
    }
    const int64_t idx = (int64_t)lo + lane;
    int64_t st = kNoStart;
    uint32_t fl = 0;
    if (idx < a.nseg) {
        st = a.segs[idx].start;
        fl = a.segs[idx].wd_on != 0;
    }
    const uint64_t b = __ballot(st <= w0);
    const int cov = b ? 63 - __clzll(b) : 0;  // lane holding the covering entry
    const uint32_t cov_flag = (uint32_t)__shfl((int)fl, cov, kWave);
    int64_t next;
    if (cov < kWave - 1) {
        next = __shfl(st, cov + 1, kWave);
    } else {
        next = lo + kWave < a.nseg ? a.segs[lo + kWave].start : kNoStart;
    }
    const uint32_t all = (nelem >= 32) ? 0xffffffffu : ((1u << nelem) - 1u);
    if (next >= w1) return cov_flag ? all : 0u;

    uint32_t mask = 0;
    if (__shfl(st, kWave - 1, kWave) >= w1) {
        // every entry the window needs is among the 64 loaded ones
        slot.start[lane] = st;
        slot.flag[lane] = (uint8_t)fl;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        int c = cov;
        for (int q = 0; q < nelem; ++q) {
            const int64_t eq = elem(q);
            if (eq >= w1) break;
            while (c + 1 < kWave && slot.start[c + 1] <= eq) ++c;
            mask |= (uint32_t)slot.flag[c] << q;
        }
        __builtin_amdgcn_wave_barrier();
    } else {
        for (int q = 0; q < nelem; ++q) {
            const int64_t eq = elem(q);
            if (eq >= w1) break;
            const int32_t s = last_le(a.segs, a.nseg, eq);
            mask |= (uint32_t)(a.segs[s].wd_on != 0) << q;
        }
    }
    return mask;
}

// Variants of the step, chosen at compile time (bit mask):
//   kOutQ8  - also write the block-quantized int8 copy of the new parameters
//             with one fp32 scale per kQ8Block elements (the payload of a
//             quantized all-gather);
//   kGradQ8 - the k partials arrive as int8 with one fp32 scale per
//             kQ8Block elements each (a block-quantized reduce-scatter) and
//             are dequantized inside the reduce;
//   kMvBf16 - the moments m and v are stored as bf16 (12 bytes per parameter
//             of optimizer state plus weight instead of 16).
constexpr int kOutQ8 = 1;
constexpr int kGradQ8 = 2;
constexpr int kMvBf16 = 4;
constexpr int kQ8Block = ZS_Q8_BLOCK;
static_assert(kQ8Block == kSub, "a quantization block is one sub-window of a wave");

__device__ __forceinline__ f32x4 bf16x4_to_f32x4(u32x2 d) {
    f32x4 r;
    r[0] = bf16_lo(d[0]);
    r[1] = bf16_hi(d[0]);
    r[2] = bf16_lo(d[1]);
    r[3] = bf16_hi(d[1]);
    return r;
}

__device__ __forceinline__ u32x2 f32x4_to_bf16x4(f32x4 x) {
    u32x2 r;
    r[0] = to_bf16(x[0]) | (to_bf16(x[1]) << 16);
    r[1] = to_bf16(x[2]) | (to_bf16(x[3]) << 16);
    return r;
}

__device__ __forceinline__ float i8_at(uint32_t word, int byte) {
    return (float)(int32_t)(int8_t)(uint8_t)(word >> (8 * byte));
}

// The four reduced gradients of one lane's quad (elements 4 * qi .. +3).
template <int K, int V, int NT>
struct QuadGrads {
    u32x2 bf[(V & kGradQ8) ? 1 : K];   // bf16 partials
    uint32_t q[(V & kGradQ8) ? K : 1]; // int8 partials (4 per word)
    float s[(V & kGradQ8) ? K : 1];    // their block scales

    __device__ __forceinline__ void load_from(const StepArgs &a, int64_t qi) {
        if constexpr (V & kGradQ8) {
            const int64_t blk = (qi * kQuad) / kQ8Block;
#pragma unroll
            for (int j = 0; j < K; ++j) {
                q[j] = load<NT>(reinterpret_cast<const uint32_t *>(a.qgrads[j]) + qi);
                s[j] = a.qscales[j][blk];
            }
        } else {
#pragma unroll
            for (int j = 0; j < K; ++j)
                bf[j] = load<NT>(reinterpret_cast<const u32x2 *>(a.grads[j]) + qi);
        }
    }

    // Left fold over the partials of element e (0..3 of the quad), then the scale.
    __device__ __forceinline__ float reduced(int e, const StepArgs &a) const {
#pragma clang fp contract(off)
        float g;
        if constexpr (V & kGradQ8) {
            g = i8_at(q[0], e) * s[0];
#pragma unroll
            for (int j = 1; j < K; ++j) {
                const float t = i8_at(q[j], e) * s[j];
                g = g + t;
            }
        } else {
            const int d = e >> 1;
            g = (e & 1) ? bf16_hi(bf[0][d]) : bf16_lo(bf[0][d]);
#pragma unroll
            for (int j = 1; j < K; ++j) g = g + ((e & 1) ? bf16_hi(bf[j][d]) : bf16_lo(bf[j][d]));
        }
        return g * a.gscale;
    }
};

// Reduced gradient of one element in the scalar (ragged tail) path.
template <int K, int V>
__device__ __forceinline__ float scalar_grad(const StepArgs &a, int64_t i) {
#pragma clang fp contract(off)
    float g;
    if constexpr (V & kGradQ8) {
        const int64_t blk = i / kQ8Block;
        g = (float)a.qgrads[0][i] * a.qscales[0][blk];
#pragma unroll
        for (int j = 1; j < K; ++j) {
            const float t = (float)a.qgrads[j][i] * a.qscales[j][blk];
            g = g + t;
        }
    } else {
        g = __uint_as_float((uint32_t)a.grads[0][i] << 16);
#pragma unroll
        for (int j = 1; j < K; ++j) g = g + __uint_as_float((uint32_t)a.grads[j][i] << 16);
    }
    return g * a.gscale;
}

// Maximum over the 64 lanes of a wavefront (every lane gets it).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
        const uint32_t y = (uint32_t)__shfl_xor((int)x, off, kWave);
        x = x > y ? x : y;
    }
    return x;
}

// Quantize one block (one half window: 64 lanes x 4 bf16 values) to int8.
// `bits` are the lane's four bf16 values widened to fp32 bit patterns;
// `valid` marks which of them lie inside the shard.  The block maximum of
// |x| is taken on the bit patterns (integer order of |x| bits = order of
// |x|, and every NaN pattern sorts above infinity, so a NaN wins).  All 64
// lanes must call this together.  Returns the four int8 codes packed in a
// word; lane 0 stores the scale when the block exists.
__device__ __forceinline__ uint32_t quantize_block(const uint32_t bits[4], uint32_t valid,
                                                   const StepArgs &a, int64_t block,
                                                   bool block_exists) {
    uint32_t amax = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t ab = bits[e] & 0x7fffffffu;
        if (((valid >> e) & 1u) && ab > amax) amax = ab;
    }
    amax = wave_max_u32(amax);
    const float scale = __uint_as_float(amax) / 127.0f;
    const bool usable = scale > 0.0f && scale <= 3.40282347e+38f;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        int32_t q = 0;
        if (usable) {
            float r = __builtin_rintf(__uint_as_float(bits[e]) / scale);
            r = r > 127.0f ? 127.0f : r;
            r = r < -127.0f ? -127.0f : r;
            q = (int32_t)r;
        }
        word |= ((uint32_t)q & 0xffu) << (8 * e);
    }
    if (block_exists && (threadIdx.x % kWave) == 0) a.q8_scale[block] = scale;
    return word;
}

// Reduce, update and pack one lane's quad.  mask bit e = decay of element e.
template <int K, int V, int NT>
__device__ __forceinline__ void quad_update(f32x4 &w, f32x4 &m, f32x4 &v,
                                            const QuadGrads<K, V, NT> &gr, uint32_t mask,
                                            const StepArgs &a, u32x2 &pout) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float g = gr.reduced(e, a);
        float we = w[e], me = m[e], ve = v[e];
        adamw(we, me, ve, g, (mask >> e) & 1u, a);
        w[e] = we;
        m[e] = me;
        v[e] = ve;
    }
    pout = f32x4_to_bf16x4(w);
}

template <int K, int V, int NT>
__global__ __launch_bounds__(kThreads) void shard_step_kernel(const StepArgs a) {
    constexpr int kQuads = quads_for(K);      // sub-windows per wave per tile
    constexpr int kWindow = kQuads * kSub;    // elements per wave per tile
    constexpr int kTile = tile_for(K);        // elements per workgroup tile
    __shared__ WaveSlot s_slot[kThreads / kWave];

    const int tid = (int)threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int64_t c0 = (int64_t)blockIdx.x * a.chunk;
    const int64_t c1 = (c0 + a.chunk < a.n) ? c0 + a.chunk : a.n;

    // Every wavefront works on its own windows; there is no workgroup barrier.
    for (int64_t t0 = c0; t0 < c1; t0 += kTile) {
        const int64_t w0 = t0 + (int64_t)wave * kWindow;
        if (w0 >= c1) continue;  // wave-uniform
        const int64_t w1 = (w0 + kWindow < c1) ? w0 + kWindow : c1;
        // This lane's quads: elements e[qd] .. e[qd]+3 of sub-window qd.
        int64_t e[kQuads];
#pragma unroll
        for (int qd = 0; qd < kQuads; ++qd) e[qd] = w0 + (int64_t)qd * kSub + (int64_t)lane * kQuad;
        auto elem = [&](int q) { return e[q / kQuad] + (q % kQuad); };

        if (w0 + kWindow <= a.n) {
            // Whole window in range: dense vector traffic only.  The loads are
            // issued first, so the segment search below overlaps them.
            f32x4 *pw = reinterpret_cast<f32x4 *>(a.master);
            f32x4 wv[kQuads], mv[kQuads], vv[kQuads];
            QuadGrads<K, V, NT> gq[kQuads];
#pragma unroll
            for (int qd = 0; qd < kQuads; ++qd) {
                const int64_t qi = e[qd] / kQuad;
                wv[qd] = load<NT>(pw + qi);
                if constexpr (V & kMvBf16) {
                    mv[qd] = bf16x4_to_f32x4(load<NT>(reinterpret_cast<const u32x2 *>(a.m) + qi));
                    vv[qd] = bf16x4_to_f32x4(load<NT>(reinterpret_cast<const u32x2 *>(a.v) + qi));
                } else {
                    mv[qd] = load<NT>(reinterpret_cast<const f32x4 *>(a.m) + qi);
                    vv[qd] = load<NT>(reinterpret_cast<const f32x4 *>(a.v) + qi);
                }
                gq[qd].load_from(a, qi);
            }
            // Decay flags: bit 4*qd + j for element e[qd] + j.
            const uint32_t mask = window_mask(a, w0, w1, kQuads * kQuad, elem, s_slot[wave]);
#pragma unroll
            for (int qd = 0; qd < kQuads; ++qd) {
                const int64_t qi = e[qd] / kQuad;
                u32x2 pq;
                quad_update<K, V, NT>(wv[qd], mv[qd], vv[qd], gq[qd], (mask >> (kQuad * qd)) & 0xfu,
                                      a, pq);
                store<NT>(pw + qi, wv[qd]);
                if constexpr (V & kMvBf16) {
                    store<NT>(reinterpret_cast<u32x2 *>(a.m) + qi, f32x4_to_bf16x4(mv[qd]));
                    store<NT>(reinterpret_cast<u32x2 *>(a.v) + qi, f32x4_to_bf16x4(vv[qd]));
                } else {
                    store<NT>(reinterpret_cast<f32x4 *>(a.m) + qi, mv[qd]);
                    store<NT>(reinterpret_cast<f32x4 *>(a.v) + qi, vv[qd]);
                }
                store<NT>(reinterpret_cast<u32x2 *>(a.param) + qi, pq);
                if constexpr (V & kOutQ8) {
                    const uint32_t bits[4] = {pq[0] << 16, pq[0] & 0xffff0000u, pq[1] << 16,
                                              pq[1] & 0xffff0000u};
                    const int64_t blk = (w0 + (int64_t)qd * kSub) / kQ8Block;
                    const uint32_t word = quantize_block(bits, 0xfu, a, blk, true);
                    store<NT>(reinterpret_cast<uint32_t *>(a.q8) + qi, word);
                }
            }
        } else {
            // The shard's last, partial window: element by element (the whole
            // wavefront stays here together, for the search and block maxima).
            const uint32_t mask = window_mask(a, w0, w1, kQuads * kQuad, elem, s_slot[wave]);
            uint32_t pbits[kQuads * kQuad];
            uint32_t valid = 0;
            for (int q = 0; q < kQuads * kQuad; ++q) {
                pbits[q] = 0;
                const int64_t i = e[q / kQuad] + (q % kQuad);
                if (i >= a.n) continue;
                valid |= 1u << q;
                const float g = scalar_grad<K, V>(a, i);
                float wv = a.master[i], mvv, vvv;
                if constexpr (V & kMvBf16) {
                    mvv = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(a.m)[i] << 16);
                    vvv = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(a.v)[i] << 16);
                } else {
                    mvv = reinterpret_cast<const float *>(a.m)[i];
                    vvv = reinterpret_cast<const float *>(a.v)[i];
                }
                adamw(wv, mvv, vvv, g, (mask >> q) & 1u, a);
                a.master[i] = wv;
                if constexpr (V & kMvBf16) {
                    reinterpret_cast<uint16_t *>(a.m)[i] = (uint16_t)to_bf16(mvv);
                    reinterpret_cast<uint16_t *>(a.v)[i] = (uint16_t)to_bf16(vvv);
                } else {
                    reinterpret_cast<float *>(a.m)[i] = mvv;
                    reinterpret_cast<float *>(a.v)[i] = vvv;
                }
                const uint32_t pbf = to_bf16(wv);
                a.param[i] = (uint16_t)pbf;
                pbits[q] = pbf << 16;
            }
            if constexpr (V & kOutQ8) {
#pragma unroll
                for (int qd = 0; qd < kQuads; ++qd) {
                    const int64_t sub0 = w0 + (int64_t)qd * kSub;
                    const uint32_t word = quantize_block(pbits + kQuad * qd,
                                                         (valid >> (kQuad * qd)) & 0xfu, a,
                                                         sub0 / kQ8Block, sub0 < a.n);
                    for (int j = 0; j < kQuad; ++j) {
                        const int q = kQuad * qd + j;
                        if ((valid >> q) & 1u)
                            a.q8[e[qd] + j] = (int8_t)(uint8_t)(word >> (8 * j));
                    }
                }
            }
        }
    }
}

typedef void (*kernel_fn)(const StepArgs);

template <int K>
kernel_fn pick_variant(int variant, int nt) {
    switch (variant) {
        case 0: return nt ? shard_step_kernel<K, 0, 1> : shard_step_kernel<K, 0, 0>;
        case kOutQ8: return shard_step_kernel<K, kOutQ8, 1>;
        case kGradQ8: return shard_step_kernel<K, kGradQ8, 1>;
        case kMvBf16: return shard_step_kernel<K, kMvBf16, 1>;
        default: return nullptr;
    }
}

kernel_fn pick_kernel(int k, int variant, int nt) {
    switch (k) {
        case 1: return pick_variant<1>(variant, nt);
        case 2: return pick_variant<2>(variant, nt);
        case 3: return pick_variant<3>(variant, nt);
        case 4: return pick_variant<4>(variant, nt);
        case 5: return pick_variant<5>(variant, nt);
        case 6: return pick_variant<6>(variant, nt);
        case 7: return pick_variant<7>(variant, nt);
        case 8: return pick_variant<8>(variant, nt);
        case 9: return pick_variant<9>(variant, nt);
        case 10: return pick_variant<10>(variant, nt);
        case 11: return pick_variant<11>(variant, nt);
        case 12: return pick_variant<12>(variant, nt);
        case 13: return pick_variant<13>(variant, nt);
        case 14: return pick_variant<14>(variant, nt);
        case 15: return pick_variant<15>(variant, nt);
        case 16: return pick_variant<16>(variant, nt);
        default: return nullptr;
    }
}

// ---------------------------------------------------------------- host side

constexpr int kMaxDevices = 64;

struct DeviceInfo {
    int ready;
    int cus;
};

DeviceInfo g_dev[kMaxDevices];
int g_initialized = 0;
thread_local int t_last_hip_error = 0;

int device_error(hipError_t e) {
    t_last_hip_error = (int)e;
    return ZS_ERR_DEVICE;
}

bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    const uintptr_t a1 = a0 + (uintptr_t)abytes, b1 = b0 + (uintptr_t)bbytes;
    return a0 < b1 && b0 < a1;
}

int pick_chunk_tiles(int64_t n, int cus) {
    // One tile per workgroup: the resident workgroups then cover one compact
    // stretch of every array and sweep through memory together, which
    // measured best on MI355X for every shard size (longer chunks spread the
    // active front over more DRAM pages).  The per-workgroup segment search
    // is two dependent table loads and hides behind the other workgroups.
    (void)n;
    (void)cus;
    return 1;
}

// One call, whatever the variant: the buffers it reads and writes.
struct Request {
    float *master = nullptr;
    void *m = nullptr;
    void *v = nullptr;
    uint16_t *param = nullptr;
    int8_t *q8 = nullptr;
    float *q8_scale = nullptr;
    const uint16_t *const *grads = nullptr;
    const int8_t *const *qgrads = nullptr;
    const float *const *qscales = nullptr;
    int k = 0;
    int64_t n = 0;
    const zs_seg_table *st = nullptr;
    const zs_hparams *hp = nullptr;
    int64_t step = 0;
    void *stream = nullptr;
    const zs_launch_cfg *cfg = nullptr;
    int variant = 0;
};

struct Span {
    const void *p;
    int64_t bytes;
    uintptr_t align;
};

int validate_and_launch(const Request &r) {
    if (!g_initialized) return ZS_ERR_NOT_INITIALIZED;
    const bool gq = (r.variant & kGradQ8) != 0;
    if (r.k < 1 || r.k > ZS_MAX_K || r.n < 0 || r.step < 1 || !r.st || !r.hp)
        return ZS_ERR_INVALID_ARGUMENT;
    if (gq ? (!r.qgrads || !r.qscales) : !r.grads) return ZS_ERR_INVALID_ARGUMENT;
    const zs_hparams *hp = r.hp;
    if (!std::isfinite(hp->lr) || !std::isfinite(hp->beta1) || !std::isfinite(hp->beta2) ||
        !std::isfinite(hp->eps) || !std::isfinite(hp->weight_decay) ||
        !std::isfinite(hp->grad_scale))
        return ZS_ERR_INVALID_ARGUMENT;
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f) ||
        hp->eps < 0.0f)
        return ZS_ERR_INVALID_ARGUMENT;
    if (r.st->count < 1) return ZS_ERR_INVALID_ARGUMENT;
    if (r.st->count > ZS_MAX_SEGMENTS) return ZS_ERR_TOO_MANY_SEGMENTS;
    // Streaming (non-temporal) loads and stores by default: nothing is
    // reused, and on MI355X they measured 5-10 % faster than cached access.
    int chunk_tiles = 0, nt = 1;
    if (r.cfg) {
        if (r.cfg->chunk_tiles < 0 || r.cfg->chunk_tiles > kMaxChunkTiles)
            return ZS_ERR_INVALID_ARGUMENT;
        if (r.cfg->nontemporal < 0 || r.cfg->nontemporal > 2) return ZS_ERR_INVALID_ARGUMENT;
        chunk_tiles = r.cfg->chunk_tiles;
        nt = r.cfg->nontemporal == 2 ? 0 : 1;
    }
    if (r.n == 0) return ZS_OK;
    if (r.n > INT64_MAX / 8) return ZS_ERR_INVALID_ARGUMENT;
    if (!r.st->segs) return ZS_ERR_INVALID_ARGUMENT;
    if ((uintptr_t)r.st->segs & 7u) return ZS_ERR_MISALIGNED;

    const int64_t n = r.n;
    const int64_t nblocks = (n + kQ8Block - 1) / kQ8Block;
    const int64_t mv_bytes = (r.variant & kMvBf16) ? 2 * n : 4 * n;
    Span outs[6];
    int nouts = 0;
    outs[nouts++] = {r.master, 4 * n, 16};
    outs[nouts++] = {r.m, mv_bytes, 16};
    outs[nouts++] = {r.v, mv_bytes, 16};
    outs[nouts++] = {r.param, 2 * n, 16};
    if (r.variant & kOutQ8) {
        outs[nouts++] = {r.q8, n, 16};
        outs[nouts++] = {r.q8_scale, 4 * nblocks, 4};
    }
    Span ins[2 * ZS_MAX_K];
    int nins = 0;
    for (int j = 0; j < r.k; ++j) {
        if (gq) {
            ins[nins++] = {r.qgrads[j], n, 16};
            ins[nins++] = {r.qscales[j], 4 * nblocks, 4};
        } else {
            ins[nins++] = {r.grads[j], 2 * n, 16};
        }
    }
    for (int x = 0; x < nouts; ++x)
        if (!outs[x].p) return ZS_ERR_INVALID_ARGUMENT;
    for (int x = 0; x < nins; ++x)
        if (!ins[x].p) return ZS_ERR_INVALID_ARGUMENT;
    for (int x = 0; x < nouts; ++x)
        if ((uintptr_t)outs[x].p & (outs[x].align - 1)) return ZS_ERR_MISALIGNED;
    for (int x = 0; x < nins; ++x)
        if ((uintptr_t)ins[x].p & (ins[x].align - 1)) return ZS_ERR_MISALIGNED;
    for (int x = 0; x < nouts; ++x) {
        for (int y = x + 1; y < nouts; ++y)
            if (overlaps(outs[x].p, outs[x].bytes, outs[y].p, outs[y].bytes)) return ZS_ERR_ALIASING;
        for (int y = 0; y < nins; ++y)
            if (overlaps(outs[x].p, outs[x].bytes, ins[y].p, ins[y].bytes)) return ZS_ERR_ALIASING;
    }

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_error(e);
    if (dev < 0 || dev >= kMaxDevices || !g_dev[dev].ready) return ZS_ERR_NOT_INITIALIZED;

    StepArgs a;
    a.master = r.master;
    a.m = r.m;
    a.v = r.v;
    a.param = r.param;
    a.q8 = r.q8;
    a.q8_scale = r.q8_scale;
    for (int j = 0; j < ZS_MAX_K; ++j) {
        a.grads[j] = (!gq && j < r.k) ? r.grads[j] : nullptr;
        a.qgrads[j] = (gq && j < r.k) ? r.qgrads[j] : nullptr;
        a.qscales[j] = (gq && j < r.k) ? r.qscales[j] : nullptr;
    }
    a.segs = r.st->segs;
    a.nseg = r.st->count;
    a.n = n;
    a.lr = hp->lr;
    a.b1 = hp->beta1;
    a.b2 = hp->beta2;
    a.c1 = 1.0f - hp->beta1;
    a.c2 = 1.0f - hp->beta2;
    a.bc1 = (float)(1.0 - std::pow((double)hp->beta1, (double)r.step));
    a.bc2 = (float)(1.0 - std::pow((double)hp->beta2, (double)r.step));
    a.eps = hp->eps;
    {
        const float lrwd = hp->lr * hp->weight_decay;
        a.df = 1.0f - lrwd;
    }
    a.gscale = hp->grad_scale;

    if (chunk_tiles == 0) chunk_tiles = pick_chunk_tiles(n, g_dev[dev].cus);
    int64_t chunk = (int64_t)chunk_tiles * tile_for(r.k);
    int64_t blocks = (n + chunk - 1) / chunk;
    while (blocks > 0x7fffffffLL) {  // keep the grid inside the 32-bit limit
        chunk *= 2;
        blocks = (n + chunk - 1) / chunk;
    }
    a.chunk = chunk;

    kernel_fn fn = pick_kernel(r.k, r.variant, nt);
    if (!fn) return ZS_ERR_INVALID_ARGUMENT;
    void *args[] = {&a};
    e = hipLaunchKernel((const void *)fn, dim3((unsigned)blocks), dim3(kThreads), args, 0,
                        (hipStream_t)r.stream);
    if (e != hipSuccess) return device_error(e);
    return ZS_OK;
}

Request base_request(float *master, void *m, void *v, uint16_t *param, int k, int64_t n,
                     const zs_seg_table *st, const zs_hparams *hp, int64_t step, void *stream) {
    Request r;
    r.master = master;
    r.m = m;
    r.v = v;
    r.param = param;
    r.k = k;
    r.n = n;
    r.st = st;
    r.hp = hp;
    r.step = step;
    r.stream = stream;
    return r;
}

}  // namespace

extern "C" {

int zs_init(int device_ordinal) {
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess) return device_error(e);
    if (device_ordinal < 0 || device_ordinal >= count || device_ordinal >= kMaxDevices)
        return ZS_ERR_INVALID_ARGUMENT;
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, device_ordinal);
    if (e != hipSuccess) return device_error(e);
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return ZS_ERR_DEVICE;
    g_dev[device_ordinal].cus = prop.multiProcessorCount;
    g_dev[device_ordinal].ready = 1;
    g_initialized = 1;
    return ZS_OK;
}

int zs_shard_step(float *master, float *m, float *v, uint16_t *param_bf16,
                  const uint16_t *const *grads, int k, int64_t n,
                  const zs_seg_table *seg_table, const zs_hparams *hparams,
                  int64_t step, void *stream) {
    Request r = base_request(master, m, v, param_bf16, k, n, seg_table, hparams, step, stream);
    r.grads = grads;
    return validate_and_launch(r);
}

int zs_shard_step_cfg(float *master, float *m, float *v, uint16_t *param_bf16,
                      const uint16_t *const *grads, int k, int64_t n,
                      const zs_seg_table *seg_table, const zs_hparams *hparams,
                      int64_t step, void *stream, const zs_launch_cfg *cfg) {
    Request r = base_request(master, m, v, param_bf16, k, n, seg_table, hparams, step, stream);
    r.grads = grads;
    r.cfg = cfg;
    return validate_and_launch(r);
}

int zs_shard_step_q8ag(float *master, float *m, float *v, uint16_t *param_bf16,
                       int8_t *param_q8, float *param_q8_scale,
                       const uint16_t *const *grads, int k, int64_t n,
                       const zs_seg_table *seg_table, const zs_hparams *hparams,
                       int64_t step, void *stream) {
    Request r = base_request(master, m, v, param_bf16, k, n, seg_table, hparams, step, stream);
    r.grads = grads;
    r.q8 = param_q8;
    r.q8_scale = param_q8_scale;
    r.variant = kOutQ8;
    return validate_and_launch(r);
}

int zs_shard_step_q8grad(float *master, float *m, float *v, uint16_t *param_bf16,
                         const int8_t *const *qgrads, const float *const *qscales, int k,
                         int64_t n, const zs_seg_table *seg_table, const zs_hparams *hparams,
                         int64_t step, void *stream) {
    Request r = base_request(master, m, v, param_bf16, k, n, seg_table, hparams, step, stream);
    r.qgrads = qgrads;
    r.qscales = qscales;
    r.variant = kGradQ8;
    return validate_and_launch(r);
}

int zs_shard_step_bf16mv(float *master, uint16_t *m_bf16, uint16_t *v_bf16,
                         uint16_t *param_bf16, const uint16_t *const *grads, int k, int64_t n,
                         const zs_seg_table *seg_table, const zs_hparams *hparams,
                         int64_t step, void *stream) {
    Request r = base_request(master, m_bf16, v_bf16, param_bf16, k, n, seg_table, hparams, step,
                             stream);
    r.grads = grads;
    r.variant = kMvBf16;
    return validate_and_launch(r);
}

int zs_fini(void) {
    for (int d = 0; d < kMaxDevices; ++d) g_dev[d].ready = 0;
    g_initialized = 0;
    return ZS_OK;
}

const char *zs_status_string(int status) {
    switch (status) {
        case ZS_OK: return "ok";
        case ZS_ERR_NOT_INITIALIZED: return "library not initialized for this device";
        case ZS_ERR_INVALID_ARGUMENT: return "invalid argument";
        case ZS_ERR_MISALIGNED: return "buffer not aligned";
        case ZS_ERR_TOO_MANY_SEGMENTS: return "segment table too large";
        case ZS_ERR_DEVICE: return "HIP runtime error";
        case ZS_ERR_ALIASING: return "output buffers overlap";
        default: return "unknown status";
    }
}

int zs_last_device_error(void) { return t_last_hip_error; }

int64_t zs_algorithmic_bytes(int k, int64_t n) {
    if (k < 1 || n < 0) return 0;
    return n * (int64_t)(12 + 2 * k) + n * 14;
}

}  // extern "C"
