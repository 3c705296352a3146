// zs_host.cpp -- the ZeRO-Offload form of the shard step: the same fused
// reduce + AdamW + bf16 cast, run by the host CPU over state kept in host
// memory ("Chapter 9: Distributed Training and Data Parallelism", section
// 9.4.3: ZeRO-Offload keeps the optimizer state in CPU memory, the GPU sends
// the gradients over PCIe, the CPU runs the Adam update and the updated
// parameters go back to the GPU).  C ABI in include/zs_host.h.
//
// Bandwidth-bound like the GPU kernel (about 0.5 flop per byte of DRAM
// traffic), so the design is: one pass over each element, 16 elements per
// AVX-512 vector, OpenMP threads over contiguous chunks (each thread walks
// its own segment cursor), and the weight-decay flag resolved once per
// vector (one broadcast when the vector lies inside a segment).  Numerics
// are those of the GPU path and of include/zs.h: binary32 one operation at a
// time, no fused multiply-add (built with -ffp-contract=off and written
// without FMA intrinsics), IEEE divide and square root, bf16 round to
// nearest even with NaN -> 0x7FC0.  Denormals are kept: the library clears
// the flush-to-zero and denormals-are-zero bits of MXCSR for the duration of
// a call, on every thread it uses, and restores them afterwards.

#include <immintrin.h>
#include <omp.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "zs_host.h"

namespace {

constexpr int64_t kChunk = 1 << 16;  // elements per scheduling unit (multiple of 16)
constexpr unsigned kMxcsrDaz = 1u << 6;
constexpr unsigned kMxcsrFtz = 1u << 15;

struct Consts {
    float lr, b1, b2, c1, c2, bc1, bc2, eps, df, gscale;
};

inline float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

inline uint16_t f32_to_bf16(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

inline void adamw_scalar(float &w, float &m, float &v, float g, bool decay, const Consts &c) {
    const float a = c.b1 * m;
    const float b = c.c1 * g;
    const float m1 = a + b;
    const float gg = g * g;
    const float cc = c.b2 * v;
    const float d = c.c2 * gg;
    const float v1 = cc + d;
    const float mh = m1 / c.bc1;
    const float vh = v1 / c.bc2;
    const float den = std::sqrt(vh) + c.eps;
    const float u = mh / den;
    const float wd = decay ? w * c.df : w;
    const float st = c.lr * u;
    w = wd - st;
    m = m1;
    v = v1;
}

// Decay flags of elements [e, e + cnt) as a bit mask, advancing the cursor.
inline uint32_t decay_bits(const zs_segment *segs, int32_t nseg, int32_t &cur, int64_t e,
                           int cnt) {
    while (cur + 1 < nseg && segs[cur + 1].start <= e) ++cur;
    const int64_t next = cur + 1 < nseg ? segs[cur + 1].start : INT64_MAX;
    if (next >= e + cnt) return segs[cur].wd_on ? (cnt == 32 ? 0xffffffffu : ((1u << cnt) - 1u)) : 0u;
    uint32_t bits = 0;
    int32_t c = cur;
    for (int q = 0; q < cnt; ++q) {
        while (c + 1 < nseg && segs[c + 1].start <= e + q) ++c;
        if (segs[c].wd_on) bits |= 1u << q;
    }
    return bits;
}

void range_scalar(float *w, float *m, float *v, uint16_t *p, const uint16_t *const *g, int k,
                  int64_t lo, int64_t hi, const zs_segment *segs, int32_t nseg, const Consts &c) {
    int32_t cur = 0;
    for (int64_t i = lo; i < hi; ++i) {
        const bool decay = decay_bits(segs, nseg, cur, i, 1) != 0;
        float gs = bf16_to_f32(g[0][i]);
        for (int j = 1; j < k; ++j) gs = gs + bf16_to_f32(g[j][i]);
        gs = gs * c.gscale;
        adamw_scalar(w[i], m[i], v[i], gs, decay, c);
        p[i] = f32_to_bf16(w[i]);
    }
}

__attribute__((target("avx512f,avx512bw"))) inline __m512 widen_bf16(const uint16_t *src) {
    const __m256i h = _mm256_loadu_si256(reinterpret_cast<const __m256i *>(src));
    return _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(h), 16));
}

__attribute__((target("avx512f,avx512bw"))) void range_avx512(
    float *w, float *m, float *v, uint16_t *p, const uint16_t *const *g, int k, int64_t lo,
    int64_t hi, const zs_segment *segs, int32_t nseg, const Consts &c) {
    const __m512 b1 = _mm512_set1_ps(c.b1), b2 = _mm512_set1_ps(c.b2);
    const __m512 c1 = _mm512_set1_ps(c.c1), c2 = _mm512_set1_ps(c.c2);
    const __m512 bc1 = _mm512_set1_ps(c.bc1), bc2 = _mm512_set1_ps(c.bc2);
    const __m512 eps = _mm512_set1_ps(c.eps), df = _mm512_set1_ps(c.df);
    const __m512 lr = _mm512_set1_ps(c.lr), gsc = _mm512_set1_ps(c.gscale);
    const __m512i bias = _mm512_set1_epi32(0x7fff), one = _mm512_set1_epi32(1);
    const __m512i absm = _mm512_set1_epi32(0x7fffffff), inf = _mm512_set1_epi32(0x7f800000);
    const __m512i qnan = _mm512_set1_epi32(0x7fc0);
    int32_t cur = 0;
    int64_t i = lo;
    for (; i + 16 <= hi; i += 16) {
        const __mmask16 dec = (__mmask16)decay_bits(segs, nseg, cur, i, 16);
        __m512 gs = widen_bf16(g[0] + i);
        for (int j = 1; j < k; ++j) gs = _mm512_add_ps(gs, widen_bf16(g[j] + i));
        gs = _mm512_mul_ps(gs, gsc);
        const __m512 w0 = _mm512_loadu_ps(w + i);
        const __m512 m0 = _mm512_loadu_ps(m + i);
        const __m512 v0 = _mm512_loadu_ps(v + i);
        const __m512 m1 = _mm512_add_ps(_mm512_mul_ps(b1, m0), _mm512_mul_ps(c1, gs));
        const __m512 v1 =
            _mm512_add_ps(_mm512_mul_ps(b2, v0), _mm512_mul_ps(c2, _mm512_mul_ps(gs, gs)));
        const __m512 mh = _mm512_div_ps(m1, bc1);
        const __m512 vh = _mm512_div_ps(v1, bc2);
        const __m512 u = _mm512_div_ps(mh, _mm512_add_ps(_mm512_sqrt_ps(vh), eps));
        const __m512 wd = _mm512_mask_mul_ps(w0, dec, w0, df);
        const __m512 w1 = _mm512_sub_ps(wd, _mm512_mul_ps(lr, u));
        _mm512_storeu_ps(w + i, w1);
        _mm512_storeu_ps(m + i, m1);
        _mm512_storeu_ps(v + i, v1);
        const __m512i ub = _mm512_castps_si512(w1);
        const __m512i lsb = _mm512_and_si512(_mm512_srli_epi32(ub, 16), one);
        __m512i r = _mm512_srli_epi32(_mm512_add_epi32(_mm512_add_epi32(ub, bias), lsb), 16);
        const __mmask16 isnan = _mm512_cmpgt_epu32_mask(_mm512_and_si512(ub, absm), inf);
        r = _mm512_mask_mov_epi32(r, isnan, qnan);
        _mm256_storeu_si256(reinterpret_cast<__m256i *>(p + i), _mm512_cvtepi32_epi16(r));
    }
    if (i < hi) range_scalar(w, m, v, p, g, k, i, hi, segs, nseg, c);
}

bool have_avx512() {
    static const bool ok = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw");
    return ok;
}

bool overlaps(const void *a, int64_t ab, const void *b, int64_t bb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bb && b0 < a0 + (uintptr_t)ab;
}

}  // namespace

extern "C" {

int zs_host_shard_step(float *master, float *m, float *v, uint16_t *param_bf16,
                       const uint16_t *const *grads, int k, int64_t n, const zs_segment *segs,
                       int32_t nseg, const zs_hparams *hp, int64_t step, int nthreads) {
    if (k < 1 || k > ZS_MAX_K || n < 0 || step < 1 || !hp || !grads || nthreads < 0)
        return ZS_ERR_INVALID_ARGUMENT;
    if (!std::isfinite(hp->lr) || !std::isfinite(hp->beta1) || !std::isfinite(hp->beta2) ||
        !std::isfinite(hp->eps) || !std::isfinite(hp->weight_decay) ||
        !std::isfinite(hp->grad_scale))
        return ZS_ERR_INVALID_ARGUMENT;
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f) ||
        hp->eps < 0.0f)
        return ZS_ERR_INVALID_ARGUMENT;
    if (nseg < 1 || !segs) return ZS_ERR_INVALID_ARGUMENT;
    if (nseg > ZS_MAX_SEGMENTS) return ZS_ERR_TOO_MANY_SEGMENTS;
    // The table is in host memory here, so its order is checked.
    if (segs[0].start != 0) return ZS_ERR_INVALID_ARGUMENT;
    for (int32_t s = 1; s < nseg; ++s)
        if (segs[s].start < segs[s - 1].start) return ZS_ERR_INVALID_ARGUMENT;
    if (n == 0) return ZS_OK;
    if (!master || !m || !v || !param_bf16) return ZS_ERR_INVALID_ARGUMENT;
    for (int j = 0; j < k; ++j)
        if (!grads[j]) return ZS_ERR_INVALID_ARGUMENT;
    if (n > INT64_MAX / 4) return ZS_ERR_INVALID_ARGUMENT;
    const void *outs[4] = {master, m, v, param_bf16};
    const int64_t ob[4] = {4 * n, 4 * n, 4 * n, 2 * n};
    for (int x = 0; x < 4; ++x) {
        for (int y = x + 1; y < 4; ++y)
            if (overlaps(outs[x], ob[x], outs[y], ob[y])) return ZS_ERR_ALIASING;
        for (int j = 0; j < k; ++j)
            if (overlaps(outs[x], ob[x], grads[j], 2 * n)) return ZS_ERR_ALIASING;
    }

    Consts c;
    c.lr = hp->lr;
    c.b1 = hp->beta1;
    c.b2 = hp->beta2;
    c.c1 = 1.0f - hp->beta1;
    c.c2 = 1.0f - hp->beta2;
    c.bc1 = (float)(1.0 - std::pow((double)hp->beta1, (double)step));
    c.bc2 = (float)(1.0 - std::pow((double)hp->beta2, (double)step));
    c.eps = hp->eps;
    const float lrwd = hp->lr * hp->weight_decay;
    c.df = 1.0f - lrwd;
    c.gscale = hp->grad_scale;

    const int threads = nthreads > 0 ? nthreads : omp_get_max_threads();
    const int64_t nchunks = (n + kChunk - 1) / kChunk;
    const bool wide = have_avx512();
#pragma omp parallel num_threads(threads)
    {
        const unsigned saved = _mm_getcsr();
        _mm_setcsr(saved & ~(kMxcsrDaz | kMxcsrFtz));
#pragma omp for schedule(static)
        for (int64_t ch = 0; ch < nchunks; ++ch) {
            const int64_t lo = ch * kChunk;
            const int64_t hi = lo + kChunk < n ? lo + kChunk : n;
            // first segment of the chunk: binary search, then the cursor walks
            int32_t a = 0, b = nseg - 1;
            while (a < b) {
                const int32_t mid = a + (b - a + 1) / 2;
                if (segs[mid].start <= lo) a = mid;
                else b = mid - 1;
            }
            const zs_segment *s0 = segs + a;
            const int32_t ns = nseg - a;
            // the chunk sees a table rebased so that its first entry covers lo
            if (wide) range_avx512(master, m, v, param_bf16, grads, k, lo, hi, s0, ns, c);
            else range_scalar(master, m, v, param_bf16, grads, k, lo, hi, s0, ns, c);
        }
        _mm_setcsr(saved);
    }
    return ZS_OK;
}

int zs_host_max_threads(void) { return omp_get_max_threads(); }

const char *zs_host_isa(void) { return have_avx512() ? "avx512" : "scalar"; }

}  // extern "C"
