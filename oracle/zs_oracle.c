/*
 * zs_oracle.c -- plain, slow, obviously correct CPU oracle for one rank's
 * share of the sharded mixed-precision AdamW step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library) never calls it and shares no code with it.
 *
 * Sources (page titles as printed on the pages):
 *  - "Chapter 9: Distributed Training and Data Parallelism", section 9.2.2
 *    (Adam): first moment, second moment, bias correction, update with the
 *    epsilon added after the square root.
 *  - same page, section 9.2.1 and 9.4.2: fp32 master copy plus two fp32
 *    moments per parameter (12 bytes), low-precision parameter and gradient.
 *  - same page, section 9.3.5 (reduce-scatter: rank r receives the sum over
 *    ranks of chunk r) and section 9.4.2 (ZeRO-1/2 training step:
 *    reduce-scatter the gradients, update only the owned shard, all-gather).
 *  - "Lecture 7: Parallelism I -- collectives, data parallelism and ZeRO"
 *    (CS336 notes), section 7 (16 bytes per parameter under mixed-precision
 *    AdamW: bf16 parameter, bf16 gradient, fp32 master, fp32 m, fp32 v) and
 *    section 8.1 (FlatZeRO1: all parameters concatenated into one flat
 *    vector, split evenly; exercise 1(e): pad with zeros until divisible).
 *
 * Every floating-point operation is IEEE-754 binary32 with round-to-nearest-
 * even, evaluated one operation at a time in the order written below.  Build
 * with -ffp-contract=off and without fast-math so that no multiply-add is
 * fused and denormals are kept.  The bias-correction denominators are formed
 * once per call in binary64 and rounded once to binary32.
 *
 * Readings taken where the pages are silent (each is listed with its reason
 * in the design notes of the repository):
 *  - "AdamW" is named but its decay is not written out: decoupled decay
 *    coupled to the learning rate, w <- w*(1 - lr*wd) on decayed elements,
 *    then w <- w - lr*u, both using the pre-step w.
 *  - the k gradient partials are SUMMED (reduce-scatter delivers a sum), in
 *    a fixed left fold j = 0..k-1, then multiplied by grad_scale.
 *  - the step counter t starts at 1.
 *  - fp32 -> bf16 is round-to-nearest-even on the 16 dropped bits; every NaN
 *    becomes the canonical quiet NaN 0x7FC0.
 *  - element i takes the weight-decay flag of the LAST segment-table entry
 *    whose start is <= i (entries sorted non-decreasing, first start 0).
 *
 * Parity pins (all in the CPU test suite): page examples for the reduce
 * (reduce-scatter exercise, ring demo), closed forms for step 1, constant
 * and zero gradients, the t -> infinity limit of bias correction, exact
 * power-of-two scaling, the library AdamW of torch (CPU, float64) for the
 * update formula, torch's bf16 conversion over all 2^32 inputs, and the
 * sharding invariant against the unsharded routine.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* Same field layout as the product's segment and hyper-parameter structs
 * (an interface both sides must agree on), declared here independently. */
typedef struct {
    int64_t start;   /* element offset inside the buffer the call covers */
    int32_t wd_on;   /* non-zero: decoupled weight decay applies */
    int32_t reserved;
} zo_segment;

typedef struct {
    float lr, beta1, beta2, eps, weight_decay, grad_scale;
} zo_hparams;

enum { ZO_OK = 0, ZO_ERR_INVALID = 2 };

static float bf16_to_f32(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even, done by looking at the 16
 * bits that are dropped.  NaN -> 0x7FC0.  Finite values whose rounding
 * carries past the largest bf16 become infinity (the carry walks into the
 * exponent field), which is what round-to-nearest requires. */
uint16_t zs_oracle_bf16_rne(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)0x7FC0u;
    uint32_t hi = u >> 16;
    uint32_t lo = u & 0xffffu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))
        hi += 1u;
    return (uint16_t)hi;
}

void zs_oracle_bf16_rne_array(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = zs_oracle_bf16_rne(x[i]);
}

/* Per-call scalars of the update, shared by both routines below. */
typedef struct {
    float c1, c2, bc1, bc2, df;
} zo_scalars;

static int hparams_ok(const zo_hparams *hp)
{
    if (!hp) return 0;
    if (!isfinite(hp->lr) || !isfinite(hp->beta1) || !isfinite(hp->beta2) ||
        !isfinite(hp->eps) || !isfinite(hp->weight_decay) ||
        !isfinite(hp->grad_scale))
        return 0;
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f)) return 0;
    if (!(hp->beta2 >= 0.0f && hp->beta2 < 1.0f)) return 0;
    if (hp->eps < 0.0f) return 0;
    return 1;
}

static zo_scalars make_scalars(const zo_hparams *hp, int64_t t)
{
    zo_scalars s;
    s.c1 = 1.0f - hp->beta1;
    s.c2 = 1.0f - hp->beta2;
    s.bc1 = (float)(1.0 - pow((double)hp->beta1, (double)t));
    s.bc2 = (float)(1.0 - pow((double)hp->beta2, (double)t));
    float lrwd = hp->lr * hp->weight_decay;
    s.df = 1.0f - lrwd;
    return s;
}

/* Moments, bias correction, update and decay for one element.  g is the
 * already-reduced fp32 gradient. */
static void adamw_element(float *w, float *m, float *v, float g, int decay,
                          const zo_hparams *hp, const zo_scalars *s)
{
    float m_prev = *m, v_prev = *v, w_prev = *w;

    float a = hp->beta1 * m_prev;
    float b = s->c1 * g;
    float m_new = a + b;

    float gg = g * g;
    float c = hp->beta2 * v_prev;
    float d = s->c2 * gg;
    float v_new = c + d;

    float m_hat = m_new / s->bc1;
    float v_hat = v_new / s->bc2;
    float denom = sqrtf(v_hat) + hp->eps;
    float u = m_hat / denom;

    float w_dec = decay ? (w_prev * s->df) : w_prev;
    float step = hp->lr * u;
    float w_new = w_dec - step;

    *m = m_new;
    *v = v_new;
    *w = w_new;
}

/*
 * One rank's shard step.  Host pointers, n elements of the shard:
 *   master, m, v : fp32 [n], updated in place
 *   param_bf16   : bf16 [n] (raw 16-bit patterns), written only
 *   grads[j]     : bf16 [n] for j < k, the k partial gradients
 *   segs[nseg]   : weight-decay segment table of this shard
 * Returns 0 on success, 2 on an invalid argument (nothing written).
 */
int zs_oracle_shard_step(float *master, float *m, float *v, uint16_t *param_bf16,
                         const uint16_t *const *grads, int k, int64_t n,
                         const zo_segment *segs, int32_t nseg,
                         const zo_hparams *hp, int64_t step)
{
    if (k < 1 || n < 0 || step < 1 || !hparams_ok(hp)) return ZO_ERR_INVALID;
    if (nseg < 1 || !segs || segs[0].start != 0) return ZO_ERR_INVALID;
    for (int32_t s = 1; s < nseg; ++s)
        if (segs[s].start < segs[s - 1].start) return ZO_ERR_INVALID;
    if (n == 0) return ZO_OK;
    if (!master || !m || !v || !param_bf16 || !grads) return ZO_ERR_INVALID;
    for (int j = 0; j < k; ++j)
        if (!grads[j]) return ZO_ERR_INVALID;

    zo_scalars sc = make_scalars(hp, step);

    int32_t seg = 0;
    for (int64_t i = 0; i < n; ++i) {
        while (seg + 1 < nseg && segs[seg + 1].start <= i)
            ++seg;
        int decay = segs[seg].wd_on != 0;

        /* reduce: left fold of the k partials, then the scale */
        float g = bf16_to_f32(grads[0][i]);
        for (int j = 1; j < k; ++j)
            g = g + bf16_to_f32(grads[j][i]);
        g = g * hp->grad_scale;

        adamw_element(&master[i], &m[i], &v[i], g, decay, hp, &sc);
        param_bf16[i] = zs_oracle_bf16_rne(master[i]);
    }
    return ZO_OK;
}

/*
 * AdamW over an unsharded buffer with an already-reduced fp32 gradient and a
 * per-element decay mask (one byte per element, non-zero = decay).  This is
 * the plain optimizer the sharded step must reproduce: the concatenation of
 * every rank's shard step equals this routine run over the whole padded
 * buffer on the fold-summed gradient.
 */
int zs_oracle_adamw_unsharded(float *w, float *m, float *v, uint16_t *param_bf16,
                              const float *g, const uint8_t *decay_mask,
                              int64_t n, const zo_hparams *hp, int64_t step)
{
    if (n < 0 || step < 1 || !hparams_ok(hp)) return ZO_ERR_INVALID;
    if (n == 0) return ZO_OK;
    if (!w || !m || !v || !param_bf16 || !g || !decay_mask) return ZO_ERR_INVALID;
    zo_scalars sc = make_scalars(hp, step);
    for (int64_t i = 0; i < n; ++i) {
        float gi = g[i] * hp->grad_scale;
        adamw_element(&w[i], &m[i], &v[i], gi, decay_mask[i] != 0, hp, &sc);
        param_bf16[i] = zs_oracle_bf16_rne(w[i]);
    }
    return ZO_OK;
}

/* The four per-call scalars, exposed so that tests can pin them to the
 * closed forms (c1 = 1-b1, bias corrections, decay factor). */
void zs_oracle_scalars(const zo_hparams *hp, int64_t step, float out[5])
{
    zo_scalars s = make_scalars(hp, step);
    out[0] = s.c1;
    out[1] = s.c2;
    out[2] = s.bc1;
    out[3] = s.bc2;
    out[4] = s.df;
}

/*
 * Block-wise symmetric int8 quantization of bf16 values: the payload of a
 * quantized all-gather ("Chapter 9: Distributed Training and Data
 * Parallelism", section 9.4.3, ZeRO++: weights converted from 16-bit to INT8
 * before the all-gather and dequantized after it; block-wise quantization to
 * limit the loss).  The pages give neither the block size nor the scale
 * rule; the reading is the plainest one:
 *   blocks of `block` consecutive elements from element 0 (the last block may
 *   be shorter); a = max |x| over the block (NaN if any element is NaN);
 *   scale = a / 127 in binary32; q = clamp(round_half_even(x / scale),
 *   -127, 127), except that every q of a block whose scale is 0 or not finite
 *   is 0.  The receiver reconstructs q * scale.
 */
int zs_oracle_q8_blocks(const uint16_t *x_bf16, int64_t n, int32_t block, int8_t *q,
                        float *scale)
{
    if (n < 0 || block < 1) return ZO_ERR_INVALID;
    if (n == 0) return ZO_OK;
    if (!x_bf16 || !q || !scale) return ZO_ERR_INVALID;
    int64_t nblocks = (n + block - 1) / block;
    for (int64_t b = 0; b < nblocks; ++b) {
        int64_t lo = b * block;
        int64_t hi = lo + block < n ? lo + block : n;
        float a = 0.0f;
        int has_nan = 0;
        for (int64_t i = lo; i < hi; ++i) {
            float x = bf16_to_f32(x_bf16[i]);
            if (isnan(x)) has_nan = 1;
            else if (fabsf(x) > a) a = fabsf(x);
        }
        if (has_nan) a = NAN;
        float s = a / 127.0f;
        scale[b] = s;
        int usable = isfinite(s) && s > 0.0f;
        for (int64_t i = lo; i < hi; ++i) {
            if (!usable) {
                q[i] = 0;
                continue;
            }
            float r = rintf(bf16_to_f32(x_bf16[i]) / s);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[i] = (int8_t)r;
        }
    }
    return ZO_OK;
}

/* Receiver side of the quantized all-gather: x = q * scale (binary32). */
void zs_oracle_q8_dequant(const int8_t *q, const float *scale, int64_t n, int32_t block,
                          float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)q[i] * scale[i / block];
}

static int segs_ok(const zo_segment *segs, int32_t nseg)
{
    if (nseg < 1 || !segs || segs[0].start != 0) return 0;
    for (int32_t s = 1; s < nseg; ++s)
        if (segs[s].start < segs[s - 1].start) return 0;
    return 1;
}

/*
 * Shard step whose k partials arrive block-quantized to int8 (the quantized
 * reduce-scatter of "Chapter 9", section 9.4.3): partial j of element i is
 * q[j][i] * scale[j][i / block], one binary32 rounding; the partials are then
 * summed in the left fold j = 0..k-1 and multiplied by grad_scale, and the
 * rest is the ordinary step.
 */
int zs_oracle_shard_step_q8grad(float *master, float *m, float *v, uint16_t *param_bf16,
                                const int8_t *const *q, const float *const *scale, int k,
                                int64_t n, int32_t block, const zo_segment *segs,
                                int32_t nseg, const zo_hparams *hp, int64_t step)
{
    if (k < 1 || n < 0 || block < 1 || step < 1 || !hparams_ok(hp)) return ZO_ERR_INVALID;
    if (!segs_ok(segs, nseg)) return ZO_ERR_INVALID;
    if (n == 0) return ZO_OK;
    if (!master || !m || !v || !param_bf16 || !q || !scale) return ZO_ERR_INVALID;
    for (int j = 0; j < k; ++j)
        if (!q[j] || !scale[j]) return ZO_ERR_INVALID;
    zo_scalars sc = make_scalars(hp, step);
    int32_t seg = 0;
    for (int64_t i = 0; i < n; ++i) {
        while (seg + 1 < nseg && segs[seg + 1].start <= i)
            ++seg;
        int64_t b = i / block;
        float g = (float)q[0][i] * scale[0][b];
        for (int j = 1; j < k; ++j) {
            float t = (float)q[j][i] * scale[j][b];
            g = g + t;
        }
        g = g * hp->grad_scale;
        adamw_element(&master[i], &m[i], &v[i], g, segs[seg].wd_on != 0, hp, &sc);
        param_bf16[i] = zs_oracle_bf16_rne(master[i]);
    }
    return ZO_OK;
}

/*
 * Shard step with the moments kept in bf16 ("Lecture 7: Parallelism I",
 * section 8.4: everything in BF16 except the fp32 master weights).  m and v
 * are widened to binary32, updated as in the ordinary step (the weight
 * update uses the unrounded new moments), then stored rounded to nearest
 * even (reading: the page does not say how they are rounded).
 */
int zs_oracle_shard_step_bf16mv(float *master, uint16_t *m, uint16_t *v, uint16_t *param_bf16,
                                const uint16_t *const *grads, int k, int64_t n,
                                const zo_segment *segs, int32_t nseg, const zo_hparams *hp,
                                int64_t step)
{
    if (k < 1 || n < 0 || step < 1 || !hparams_ok(hp)) return ZO_ERR_INVALID;
    if (!segs_ok(segs, nseg)) return ZO_ERR_INVALID;
    if (n == 0) return ZO_OK;
    if (!master || !m || !v || !param_bf16 || !grads) return ZO_ERR_INVALID;
    for (int j = 0; j < k; ++j)
        if (!grads[j]) return ZO_ERR_INVALID;
    zo_scalars sc = make_scalars(hp, step);
    int32_t seg = 0;
    for (int64_t i = 0; i < n; ++i) {
        while (seg + 1 < nseg && segs[seg + 1].start <= i)
            ++seg;
        float g = bf16_to_f32(grads[0][i]);
        for (int j = 1; j < k; ++j)
            g = g + bf16_to_f32(grads[j][i]);
        g = g * hp->grad_scale;
        float mf = bf16_to_f32(m[i]);
        float vf = bf16_to_f32(v[i]);
        adamw_element(&master[i], &mf, &vf, g, segs[seg].wd_on != 0, hp, &sc);
        m[i] = zs_oracle_bf16_rne(mf);
        v[i] = zs_oracle_bf16_rne(vf);
        param_bf16[i] = zs_oracle_bf16_rne(master[i]);
    }
    return ZO_OK;
}

/*
 * Stochastic rounding of the bf16 moments: the other reading of "Lecture 7:
 * Parallelism I", section 8.4 (bf16 m and v), whose text does not say how
 * the moments are rounded.  A value is rounded down to the bf16 below it in
 * magnitude or up to the one above with probability equal to its distance
 * from the lower one, so that the expectation of the rounded value is the
 * value itself.  The 16 random bits per rounding come from SplitMix64
 * (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014), used counter-style: output i of the stream with key K is
 * mix64(K + (i + 1) * 0x9E3779B97F4A7C15).
 */
static uint64_t sm64_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t zs_oracle_splitmix64(uint64_t key, uint64_t i)
{
    return sm64_mix(key + (i + 1u) * 0x9E3779B97F4A7C15ull);
}

/* fp32 -> bf16 with the 16 random bits r: adding r below the kept bits and
 * dropping them rounds the magnitude up exactly when r >= 65536 - (dropped
 * bits), i.e. with probability (dropped bits) / 65536.  The sign bit is not
 * touched (the carry stays inside the magnitude; the largest finite value
 * can round up to infinity).  NaN -> 0x7FC0; infinities stay. */
uint16_t zs_oracle_bf16_sr(float x, uint32_t r)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)0x7FC0u;
    return (uint16_t)((u + (r & 0xffffu)) >> 16);
}

void zs_oracle_bf16_sr_array(const float *x, const uint32_t *r, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = zs_oracle_bf16_sr(x[i], r[i]);
}

/* The random bits of element i for moment `which` (0 = m, 1 = v) at step
 * t: the stream key is output 2t + which of the caller's seed; word i / 4 of
 * that stream holds the bits of elements 4(i/4) .. 4(i/4) + 3, 16 each, the
 * lowest for the first. */
uint32_t zs_oracle_sr_bits(uint64_t seed, int64_t step, int which, int64_t i)
{
    uint64_t key = zs_oracle_splitmix64(seed, 2u * (uint64_t)step + (uint64_t)which);
    uint64_t word = zs_oracle_splitmix64(key, (uint64_t)i / 4u);
    return (uint32_t)((word >> (16 * (i % 4))) & 0xffffu);
}

/*
 * Shard step with bf16 moments rounded stochastically: exactly
 * zs_oracle_shard_step_bf16mv except that the new m and v are stored with
 * zs_oracle_bf16_sr, each with its own random bits (the parameter copy is
 * still rounded to nearest even).  `seed` selects the random streams; a
 * rank would pass its own.  The arrays hold shard elements index0 ..
 * index0 + n - 1 (a window of the shard; index0 = 0 for the whole shard),
 * whose random bits are those of their place in the shard.
 */
int zs_oracle_shard_step_bf16mv_sr(float *master, uint16_t *m, uint16_t *v, uint16_t *param_bf16,
                                   const uint16_t *const *grads, int k, int64_t n,
                                   const zo_segment *segs, int32_t nseg, const zo_hparams *hp,
                                   int64_t step, uint64_t seed, int64_t index0)
{
    if (index0 < 0) return ZO_ERR_INVALID;
    if (k < 1 || n < 0 || step < 1 || !hparams_ok(hp)) return ZO_ERR_INVALID;
    if (!segs_ok(segs, nseg)) return ZO_ERR_INVALID;
    if (n == 0) return ZO_OK;
    if (!master || !m || !v || !param_bf16 || !grads) return ZO_ERR_INVALID;
    for (int j = 0; j < k; ++j)
        if (!grads[j]) return ZO_ERR_INVALID;
    zo_scalars sc = make_scalars(hp, step);
    int32_t seg = 0;
    for (int64_t i = 0; i < n; ++i) {
        while (seg + 1 < nseg && segs[seg + 1].start <= i)
            ++seg;
        float g = bf16_to_f32(grads[0][i]);
        for (int j = 1; j < k; ++j)
            g = g + bf16_to_f32(grads[j][i]);
        g = g * hp->grad_scale;
        float mf = bf16_to_f32(m[i]);
        float vf = bf16_to_f32(v[i]);
        adamw_element(&master[i], &mf, &vf, g, segs[seg].wd_on != 0, hp, &sc);
        m[i] = zs_oracle_bf16_sr(mf, zs_oracle_sr_bits(seed, step, 0, index0 + i));
        v[i] = zs_oracle_bf16_sr(vf, zs_oracle_sr_bits(seed, step, 1, index0 + i));
        param_bf16[i] = zs_oracle_bf16_rne(master[i]);
    }
    return ZO_OK;
}
