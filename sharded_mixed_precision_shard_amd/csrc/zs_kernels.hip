// zs_kernels.hip -- fused reduce + AdamW + bf16-cast shard step kernels for
// gfx950 (the C ABI that launches them is in zs_api.hip).
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
//   * a wavefront's window is Q sub-windows of 256 elements (Q = 1; Q = 2
//     for the bf16-moment kernel on shards of 2^32 elements and more; a
//     workgroup tile is four windows); lane l owns elements
//     4l..4l+3 of each sub-window.  Every load and store instruction of a
//     wavefront is then one dense, contiguous run (1 KB per fp32 array, 512 B
//     per bf16 array) of 16-byte (fp32) or 8-byte (bf16) accesses, and every
//     byte is read once and written once;
//   * a workgroup owns a contiguous chunk of tiles (one tile by default); on
//     large grids the chunks are ordered so that the workgroups the
//     dispatcher deals to one XCD take one contiguous run, giving each XCD's
//     L2 a sequential stream (eight fronts sweep the arrays), on small grids
//     linearly (one front);
//   * every wavefront resolves the weight-decay flags of its own window, with
//     no workgroup barrier and after issuing its loads (so the lookup
//     overlaps them): a 64-way search of the device table finds the entry
//     covering the window (up to 4096 entries: a six-step scalar search,
//     then one vector load of 64 consecutive entries); a
//     window inside one segment takes that segment's flag, a window with
//     segment boundaries stages the 64 entries around it in the wave's LDS
//     slot and each lane walks them for its own elements;
//   * the optimizer state may instead be packed per 256-element block in one
//     array (master, then m, then v: one 3 KB run per wavefront, or 2 KB with
//     bf16 moments); the arithmetic is the same;
//   * 64-bit element indices throughout (shards exceed 2^31 elements).
//
// Numerics follow the header: binary32, no contraction, correctly rounded
// divide and square root, denormals kept, bf16 round-to-nearest-even with
// NaN -> 0x7FC0.

#include <type_traits>

#include "zs_kernels.h"

namespace zs_detail {
namespace {

constexpr int64_t kNoStart = INT64_MAX;       // sentinel past the table end

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// One element of the update: g is the reduced, scaled gradient.  U1 (U2)
// says that bc1 (bc2) is exactly 1.0f, which it is once beta^t is at most
// 2^-25 (1 - 2^-25 is a tie that rounds to the even 1.0f): x / 1.0f == x for
// every x, so the division is left out and the result is bit for bit the same.
template <bool U1 = false, bool U2 = false>
__device__ __forceinline__ void adamw(float &w, float &m, float &v, float g, bool decay,
                                      const StepArgs &a) {
#pragma clang fp contract(off)
    const float m1 = a.b1 * m + a.c1 * g;
    const float v1 = a.b2 * v + a.c2 * (g * g);
    const float mh = U1 ? m1 : m1 / a.bc1;
    const float vh = U2 ? v1 : v1 / a.bc2;
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
// entry covering w0: each round probes 64 entries and narrows the range
// 64-fold, and the last round loads 64 consecutive entries.  A window inside
// one segment takes that segment's flag; a window that holds boundaries stages
// the 64 loaded entries in the wave's LDS slot and every lane walks them for
// its own elements; a window with more boundaries than the slot holds looks
// each element up in the table.  All 64 lanes must call this; every read
// stays inside segs[0 .. nseg-1] and the slot, sorted table or not.
//
// The first round (tables of more than 64 entries) is a binary search over
// its 64 probe entries j * step with wave-uniform indices, so that it runs on
// scalar loads: the scalar cache holds the few probe entries every window
// visits, and the scalar loads' counter is apart from the vector loads', so
// waiting for them does not wait for the window's data (a vector probe here
// made each wave wait for its data and then for two table loads in turn).  On
// a sorted table it finds the probe a 64-lane compare would, the highest whose
// start is <= w0 (0 if none).  Further rounds (tables of more than 4096
// entries) probe 64 entries at once with vector loads.
template <typename ElemFn>
__device__ uint32_t window_mask(const StepArgs &a, int64_t w0, int64_t w1, int nelem,
                                ElemFn elem, WaveSlot &slot) {
    const int lane = (int)(threadIdx.x % kWave);
    int32_t lo = 0, hi = a.nseg;  // the entry covering w0 lies in [lo, hi)
    if (hi > kWave) {
        const int32_t step = (hi + kWave - 1) / kWave;
        int32_t jlo = 0, jhi = (hi - 1) / step;  // probes j * step < nseg, j < 64
        // the table is read-only for the kernel: read it as constant memory
        typedef const __attribute__((address_space(4))) zs_segment ConstSegment;
        ConstSegment *cs = (ConstSegment *)a.segs;
        while (jlo < jhi) {
            const int32_t mid = jlo + (jhi - jlo + 1) / 2;
            if (cs[(int64_t)mid * step].start <= w0) jlo = mid;
            else jhi = mid - 1;
        }
        lo = jlo * step;
        hi = (lo + step < hi) ? lo + step : hi;
    }
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

__device__ __forceinline__ f32x4 bf16x4_to_f32x4(u32x2 d) {
    f32x4 r;
    r[0] = bf16_lo(d[0]);
    r[1] = bf16_hi(d[0]);
    r[2] = bf16_lo(d[1]);
    r[3] = bf16_hi(d[1]);
    return r;
}

// Two values to packed bf16 with gfx950's v_cvt_pk_bf16_f32, which rounds to
// nearest even and keeps denormals exactly as to_bf16 does but carries a NaN's
// payload into the result; every NaN is therefore replaced by the canonical
// quiet NaN first, which converts to 0x7FC0.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const uint32_t qnan = 0x7fc00000u;
    const f32x2 x = {__uint_as_float(__builtin_isnan(a) ? qnan : __float_as_uint(a)),
                     __uint_as_float(__builtin_isnan(b) ? qnan : __float_as_uint(b))};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

__device__ __forceinline__ u32x2 f32x4_to_bf16x4(f32x4 x) {
    u32x2 r;
    r[0] = pack_bf16x2(x[0], x[1]);
    r[1] = pack_bf16x2(x[2], x[3]);
    return r;
}

// Stochastic fp32 -> bf16 with the 16 random bits r: adding r below the
// kept bits and dropping them rounds the magnitude up with probability
// (dropped bits) / 2^16 (the carry stays inside the magnitude; the largest
// finite value can round up to infinity); NaN -> 0x7FC0, infinities stay.
__device__ __forceinline__ uint32_t to_bf16_sr(float x, uint32_t r) {
    const uint32_t u = __float_as_uint(x);
    return ((u & 0x7fffffffu) > 0x7f800000u) ? 0x7fc0u : ((u + r) >> 16);
}

// A moment quad (elements 4 qi .. 4 qi + 3) to bf16: to nearest even, or
// stochastically (kSR) with the 64-bit word qi of the stream `key`, 16 bits
// per element, the lowest for the first.
template <int V>
__device__ __forceinline__ u32x2 moment_bf16x4(f32x4 x, uint64_t key, int64_t qi) {
    if constexpr ((V & kSR) != 0) {
        const uint64_t w = sr_word(key, (uint64_t)qi);
        u32x2 r;
        r[0] = to_bf16_sr(x[0], (uint32_t)w & 0xffffu) |
               (to_bf16_sr(x[1], (uint32_t)(w >> 16) & 0xffffu) << 16);
        r[1] = to_bf16_sr(x[2], (uint32_t)(w >> 32) & 0xffffu) |
               (to_bf16_sr(x[3], (uint32_t)(w >> 48)) << 16);
        return r;
    } else {
        return f32x4_to_bf16x4(x);
    }
}

// One moment element i to bf16, as moment_bf16x4 does it for its quad.
template <int V>
__device__ __forceinline__ uint32_t moment_bf16(float x, uint64_t key, int64_t i) {
    if constexpr ((V & kSR) != 0) {
        const uint64_t w = sr_word(key, (uint64_t)(i / kQuad));
        return to_bf16_sr(x, (uint32_t)(w >> (16 * (i % kQuad))) & 0xffffu);
    } else {
        return to_bf16(x);
    }
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

// Quantize one block (one sub-window: 64 lanes x 4 bf16 values) to int8.
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
    if (usable) {
        // q = rint(x / scale) with the quotient correctly rounded.  y = x * rcp(scale)
        // (hardware reciprocal within 1 ulp, product rounded) is within
        // 1.5 * 2^-23 * |y| of x / scale, and the rounded quotient within half an
        // ulp of it: 1.75 * 2^-16 apart for |y| < 128 (1.75 * 2^-15 below 256), so
        // wherever y lies more than 2^-14 from a half-integer both round to the
        // same integer; the rare other elements (and any non-finite or larger y)
        // take the correctly rounded division.
        const float rs = __builtin_amdgcn_rcpf(scale);
        float r[4];
        uint32_t slow = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float y = __uint_as_float(bits[e]) * rs;
            r[e] = __builtin_rintf(y);
            const bool near_half = !(__builtin_fabsf(y - r[e]) < 0.5f - 0x1p-14f);
            const bool big = !(__builtin_fabsf(y) < 256.0f);
            slow |= (uint32_t)(near_half | big) << e;
        }
        if (slow) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if ((slow >> e) & 1u) r[e] = __builtin_rintf(__uint_as_float(bits[e]) / scale);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float c = __builtin_fminf(__builtin_fmaxf(r[e], -127.0f), 127.0f);
            word |= ((uint32_t)(int32_t)c & 0xffu) << (8 * e);
        }
    }
    if (block_exists && (threadIdx.x % kWave) == 0) a.q8_scale[block] = scale;
    return word;
}

// Where element e's optimizer state lives.  Separate arrays: index e of
// master, m and v (m, v fp32, or bf16 with kMvBf16).  Packed (kPacked): in
// the one state array, the block of e holds its kSub master values, then its
// kSub m and its kSub v (fp32, or bf16 with kMvBf16).  For a quad's first
// element (e a multiple of kQuad) the pointers are also the quad's.
template <int V>
struct StateAt {
    static constexpr bool kMv16 = (V & kMvBf16) != 0;
    typedef typename std::conditional<kMv16, uint16_t, float>::type Moment;
    float *w;
    Moment *m;
    Moment *v;

    __device__ __forceinline__ StateAt(const StepArgs &a, int64_t e) {
        if constexpr ((V & kPacked) && kMv16) {
            w = a.master + packed16_master(e);
            m = reinterpret_cast<uint16_t *>(a.master) + packed16_m(e);
            v = m + kSub;
        } else if constexpr ((V & kPacked) != 0) {
            w = a.master + packed_index(e);
            m = w + kSub;
            v = w + 2 * kSub;
        } else {
            w = a.master + e;
            m = reinterpret_cast<Moment *>(a.m) + e;
            v = reinterpret_cast<Moment *>(a.v) + e;
        }
    }

    // A moment quad widened to fp32, and stored back (bf16: rounded as the
    // variant says, moment_bf16x4).
    template <int NT>
    __device__ __forceinline__ static f32x4 load_quad(const Moment *p) {
        if constexpr (kMv16) return bf16x4_to_f32x4(load<NT>(reinterpret_cast<const u32x2 *>(p)));
        else return load<NT>(reinterpret_cast<const f32x4 *>(p));
    }
    template <int NT>
    __device__ __forceinline__ static void store_quad(Moment *p, f32x4 x, uint64_t key,
                                                      int64_t qi) {
        if constexpr (kMv16) store<NT>(reinterpret_cast<u32x2 *>(p), moment_bf16x4<V>(x, key, qi));
        else store<NT>(reinterpret_cast<f32x4 *>(p), x);
    }
    // One moment element, the same way.
    __device__ __forceinline__ static float load_one(const Moment *p) {
        if constexpr (kMv16) return __uint_as_float((uint32_t)*p << 16);
        else return *p;
    }
    __device__ __forceinline__ static void store_one(Moment *p, float x, uint64_t key, int64_t i) {
        if constexpr (kMv16) *p = (uint16_t)moment_bf16<V>(x, key, i);
        else *p = x;
    }
};

// Reduce, update and pack one lane's quad.  mask bit e = decay of element e.
template <int K, int V, int NT, bool U1, bool U2>
__device__ __forceinline__ void quad_update(f32x4 &w, f32x4 &m, f32x4 &v,
                                            const QuadGrads<K, V, NT> &gr, uint32_t mask,
                                            const StepArgs &a, u32x2 &pout) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float g = gr.reduced(e, a);
        float we = w[e], me = m[e], ve = v[e];
        adamw<U1, U2>(we, me, ve, g, (mask >> e) & 1u, a);
        w[e] = we;
        m[e] = me;
        v[e] = ve;
    }
    pout = f32x4_to_bf16x4(w);
}

// U: bit 0 leaves out the division by bc1, bit 1 the division by bc2 (the
// host picks these kernels only when that correction is exactly 1.0f).
template <int K, int V, int NT, int U>
__global__ __launch_bounds__(kThreads) void shard_step_kernel(const StepArgs a) {
    constexpr int kQuads = quads_for(V);      // sub-windows per wave per tile
    constexpr int kWindow = kQuads * kSub;    // elements per wave per tile
    constexpr int kTile = tile_for(V);        // elements per workgroup tile
    __shared__ WaveSlot s_slot[kThreads / kWave];

    const int tid = (int)threadIdx.x;
    const int lane = tid % kWave;
    // wave-uniform, so that window starts (and the segment search) are scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    // Chunk order.  The dispatcher deals workgroup b to XCD b % xcds; with
    // xcds > 1 each XCD is given one contiguous run of the nb = xcds*q + r
    // chunks (XCD x: q or q + 1 chunks from x*q + min(x, r)), so its L2 sees
    // a sequential stream; the map is a bijection onto [0, nb).
    int64_t b = blockIdx.x;
    if (a.xcds > 1) {
        const int64_t nb = gridDim.x, q = nb / a.xcds, r = nb % a.xcds;
        const int64_t x = b % a.xcds, y = b / a.xcds;
        b = x * q + (x < r ? x : r) + y;
    }
    const int64_t c0 = b * a.chunk;
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
            // (packed: the wave's state is one run, 3 KB, or 2 KB with bf16 moments)
            typedef StateAt<V> S;
            f32x4 wv[kQuads], mv[kQuads], vv[kQuads];
            QuadGrads<K, V, NT> gq[kQuads];
#pragma unroll
            for (int qd = 0; qd < kQuads; ++qd) {
                const int64_t qi = e[qd] / kQuad;
                const S st(a, e[qd]);
                wv[qd] = load<NT>(reinterpret_cast<const f32x4 *>(st.w));
                mv[qd] = S::template load_quad<NT>(st.m);
                vv[qd] = S::template load_quad<NT>(st.v);
                gq[qd].load_from(a, qi);
            }
            // Decay flags: bit 4*qd + j for element e[qd] + j.
            const uint32_t mask = window_mask(a, w0, w1, kQuads * kQuad, elem, s_slot[wave]);
#pragma unroll
            for (int qd = 0; qd < kQuads; ++qd) {
                const int64_t qi = e[qd] / kQuad;
                u32x2 pq;
                quad_update<K, V, NT, (U & 1) != 0, (U & 2) != 0>(
                    wv[qd], mv[qd], vv[qd], gq[qd], (mask >> (kQuad * qd)) & 0xfu, a, pq);
                const S st(a, e[qd]);
                store<NT>(reinterpret_cast<f32x4 *>(st.w), wv[qd]);
                S::template store_quad<NT>(st.m, mv[qd], a.sr_key_m, qi);
                S::template store_quad<NT>(st.v, vv[qd], a.sr_key_v, qi);
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
                typedef StateAt<V> S;
                const S st(a, i);
                float wv = *st.w, mvv = S::load_one(st.m), vvv = S::load_one(st.v);
                adamw<(U & 1) != 0, (U & 2) != 0>(wv, mvv, vvv, g, (mask >> q) & 1u, a);
                *st.w = wv;
                S::store_one(st.m, mvv, a.sr_key_m, i);
                S::store_one(st.v, vvv, a.sr_key_v, i);
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

static_assert(sizeof(WaveSlot) * (kThreads / kWave) == kStaticLds, "LDS per workgroup");

// Quad q of the element space (elements 4q .. 4q+3, the last block's padding
// included) between the separate arrays and its three quads in the packed
// state; a quad that reaches past n goes element by element.
__global__ __launch_bounds__(kThreads) void layout_kernel(int dir, float *master, float *m,
                                                          float *v, float *state, int64_t n) {
    const int64_t nq = packed_floats(n) / 3 / kQuad;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    f32x4 *const st4 = reinterpret_cast<f32x4 *>(state);
    for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < nq; q += stride) {
        const int64_t i = q * kQuad;
        const int64_t s = packed_index(i) / kQuad;
        if (i + kQuad <= n) {
            if (dir == kLayoutPack) {
                st4[s] = reinterpret_cast<const f32x4 *>(master)[q];
                st4[s + kWave] = reinterpret_cast<const f32x4 *>(m)[q];
                st4[s + 2 * kWave] = reinterpret_cast<const f32x4 *>(v)[q];
            } else {
                reinterpret_cast<f32x4 *>(master)[q] = st4[s];
                reinterpret_cast<f32x4 *>(m)[q] = st4[s + kWave];
                reinterpret_cast<f32x4 *>(v)[q] = st4[s + 2 * kWave];
            }
            continue;
        }
        for (int j = 0; j < kQuad; ++j) {
            const int64_t e = i + j;
            const int64_t ps = packed_index(e);
            if (dir == kLayoutPack) {
                state[ps] = e < n ? master[e] : 0.0f;
                state[ps + kSub] = e < n ? m[e] : 0.0f;
                state[ps + 2 * kSub] = e < n ? v[e] : 0.0f;
            } else if (e < n) {
                master[e] = state[ps];
                m[e] = state[ps + kSub];
                v[e] = state[ps + 2 * kSub];
            }
        }
    }
}

// The same between fp32 master, bf16 m and v and the packed state with bf16
// moments (packed16 layout): per quad, one 16-byte and two 8-byte moves.
__global__ __launch_bounds__(kThreads) void layout16_kernel(int dir, float *master, uint16_t *m,
                                                            uint16_t *v, float *state,
                                                            int64_t n) {
    const int64_t nq = packed16_floats(n) / 2 / kQuad;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    f32x4 *const st4 = reinterpret_cast<f32x4 *>(state);
    u32x2 *const st2 = reinterpret_cast<u32x2 *>(state);
    uint16_t *const s16 = reinterpret_cast<uint16_t *>(state);
    for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < nq; q += stride) {
        const int64_t i = q * kQuad;
        const int64_t sw = packed16_master(i) / kQuad;
        const int64_t sm = packed16_m(i) / kQuad;
        if (i + kQuad <= n) {
            if (dir == kLayoutPack) {
                st4[sw] = reinterpret_cast<const f32x4 *>(master)[q];
                st2[sm] = reinterpret_cast<const u32x2 *>(m)[q];
                st2[sm + kWave] = reinterpret_cast<const u32x2 *>(v)[q];
            } else {
                reinterpret_cast<f32x4 *>(master)[q] = st4[sw];
                reinterpret_cast<u32x2 *>(m)[q] = st2[sm];
                reinterpret_cast<u32x2 *>(v)[q] = st2[sm + kWave];
            }
            continue;
        }
        for (int j = 0; j < kQuad; ++j) {
            const int64_t e = i + j;
            const int64_t pw = packed16_master(e), pm = packed16_m(e);
            if (dir == kLayoutPack) {
                state[pw] = e < n ? master[e] : 0.0f;
                s16[pm] = e < n ? m[e] : (uint16_t)0;
                s16[pm + kSub] = e < n ? v[e] : (uint16_t)0;
            } else if (e < n) {
                master[e] = state[pw];
                m[e] = s16[pm];
                v[e] = s16[pm + kSub];
            }
        }
    }
}

}  // namespace

hipError_t launch_layout16(int dir, float *master, uint16_t *m, uint16_t *v, float *state,
                           int64_t n, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(layout16_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, dir,
                       master, m, v, state, n);
    return hipGetLastError();
}

hipError_t launch_layout(int dir, float *master, float *m, float *v, float *state, int64_t n,
                         int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(layout_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, dir,
                       master, m, v, state, n);
    return hipGetLastError();
}

template <int K, int V>
kernel_fn pick_unit(int unit) {
    switch (unit) {
        case 3: return shard_step_kernel<K, V, 1, 3>;
        case 1: return shard_step_kernel<K, V, 1, 1>;
        default: return shard_step_kernel<K, V, 1, 0>;
    }
}

template <int K>
kernel_fn pick_variant(int variant, int nt, int unit) {
    switch (variant) {
        case 0: return nt ? pick_unit<K, 0>(unit) : shard_step_kernel<K, 0, 0, 0>;
        case kOutQ8: return pick_unit<K, kOutQ8>(unit);
        case kGradQ8: return pick_unit<K, kGradQ8>(unit);
        case kMvBf16: return pick_unit<K, kMvBf16>(unit);
        case kPacked: return nt ? pick_unit<K, kPacked>(unit) : nullptr;
        case kPacked | kOutQ8: return nt ? pick_unit<K, kPacked | kOutQ8>(unit) : nullptr;
        case kPacked | kGradQ8: return nt ? pick_unit<K, kPacked | kGradQ8>(unit) : nullptr;
        case kPacked | kMvBf16: return nt ? pick_unit<K, kPacked | kMvBf16>(unit) : nullptr;
        case kMvBf16 | kWide:
            if constexpr (K <= kWideMaxK) return pick_unit<K, kMvBf16 | kWide>(unit);
            return nullptr;
        case kPacked | kMvBf16 | kWide:
            if constexpr (K <= kWideMaxK)
                return nt ? pick_unit<K, kPacked | kMvBf16 | kWide>(unit) : nullptr;
            return nullptr;
        case kMvBf16 | kSR: return pick_unit<K, kMvBf16 | kSR>(unit);
        case kMvBf16 | kSR | kWide:
            if constexpr (K <= kWideMaxK) return pick_unit<K, kMvBf16 | kSR | kWide>(unit);
            return nullptr;
        case kPacked | kMvBf16 | kSR:
            return nt ? pick_unit<K, kPacked | kMvBf16 | kSR>(unit) : nullptr;
        case kPacked | kMvBf16 | kSR | kWide:
            if constexpr (K <= kWideMaxK)
                return nt ? pick_unit<K, kPacked | kMvBf16 | kSR | kWide>(unit) : nullptr;
            return nullptr;
        default: return nullptr;
    }
}

kernel_fn pick_kernel(int k, int variant, int nt, int unit_bc) {
    // kernels without the bc1 division, or without both; otherwise the
    // general one (bc2 reaching 1.0f before bc1 needs beta2 < beta1)
    const int unit = unit_bc == 3 ? 3 : (unit_bc & 1);
    switch (k) {
        case 1: return pick_variant<1>(variant, nt, unit);
        case 2: return pick_variant<2>(variant, nt, unit);
        case 3: return pick_variant<3>(variant, nt, unit);
        case 4: return pick_variant<4>(variant, nt, unit);
        case 5: return pick_variant<5>(variant, nt, unit);
        case 6: return pick_variant<6>(variant, nt, unit);
        case 7: return pick_variant<7>(variant, nt, unit);
        case 8: return pick_variant<8>(variant, nt, unit);
        case 9: return pick_variant<9>(variant, nt, unit);
        case 10: return pick_variant<10>(variant, nt, unit);
        case 11: return pick_variant<11>(variant, nt, unit);
        case 12: return pick_variant<12>(variant, nt, unit);
        case 13: return pick_variant<13>(variant, nt, unit);
        case 14: return pick_variant<14>(variant, nt, unit);
        case 15: return pick_variant<15>(variant, nt, unit);
        case 16: return pick_variant<16>(variant, nt, unit);
        default: return nullptr;
    }
}

}  // namespace zs_detail
