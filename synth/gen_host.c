/*
 * gen_host.c -- seeded synthetic inputs on the host (twin of gen_device.hip).
 *
 * Holds none of the optimizer's arithmetic: it only draws numbers.  The
 * device twin implements the same definition independently; tests check that
 * both produce bit-identical arrays.
 *
 * Definition.  SplitMix64 (Steele, Lea and Flood, "Fast Splittable
 * Pseudorandom Number Generators", OOPSLA 2014): the i-th output (i >= 0) of
 * the stream with seed s is mix64(s + (i + 1) * G), G = 0x9E3779B97F4A7C15,
 * with the published 64-bit finaliser
 *     z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 *     z ^= z >> 27; z *= 0x94D049BB133111EB;
 *     z ^= z >> 31.
 * Streams are keyed by (seed, role, j, t):
 *     key = mix64(seed ^ mix64(role << 56 | j << 40 | t))
 * and element gi (its index in the whole flat model buffer) uses outputs
 * 3*gi, 3*gi+1, 3*gi+2 of that stream.  Their twelve 16-bit fields h_q are
 * summed (Irwin-Hall with 12 terms): S = sum h_q, and
 *     z = S - 393210    (an exact integer, |z| <= 393210)
 * has mean 0 and variance ~ 65536^2.  The variate is the single binary32
 * product  (float)z * scale,  scale = sigma * 2^-16 rounded to binary32 on
 * the caller side.  A heavy-tail mixture draws output gi of the stream keyed
 * with role HEAVY: if its top 32 bits are below `heavy_thresh` the element
 * uses `heavy_scale` instead.  bf16 outputs keep the top 16 bits of the
 * binary32 variate (truncation).  Elements with gi >= valid_end are zero
 * (the zero padding of a flat buffer split evenly across ranks).
 */
#include <stdint.h>
#include <string.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ull

static uint64_t mix64(uint64_t z)
{
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

uint64_t synth_stream_key(uint64_t seed, uint32_t role, uint32_t j, uint64_t t)
{
    uint64_t sid = ((uint64_t)(role & 0xffu) << 56) | ((uint64_t)(j & 0xffffu) << 40) |
                   (t & 0xffffffffffull);
    return mix64(seed ^ mix64(sid));
}

uint64_t synth_output(uint64_t key, uint64_t i)
{
    return mix64(key + (i + 1u) * SM_GAMMA);
}

static int32_t irwin_hall_z(uint64_t key, uint64_t gi)
{
    int32_t s = 0;
    for (int q = 0; q < 3; ++q) {
        uint64_t x = synth_output(key, 3u * gi + (uint64_t)q);
        for (int b = 0; b < 4; ++b)
            s += (int32_t)((x >> (16 * b)) & 0xffffu);
    }
    return s - 393210;
}

static float variate(uint64_t key, uint64_t hkey, uint64_t gi, float scale,
                     uint32_t heavy_thresh, float heavy_scale)
{
    float sc = scale;
    if (heavy_thresh != 0u) {
        uint64_t h = synth_output(hkey, gi);
        if ((uint32_t)(h >> 32) < heavy_thresh)
            sc = heavy_scale;
    }
    float zf = (float)irwin_hall_z(key, gi); /* exact: |z| < 2^24 */
    return zf * sc;
}

/* out[i] for i < n is the variate of element gi = index0 + i. */
void synth_normal_f32(float *out, int64_t n, uint64_t key, uint64_t hkey, int64_t index0,
                      int64_t valid_end, float scale, uint32_t heavy_thresh, float heavy_scale)
{
    for (int64_t i = 0; i < n; ++i) {
        int64_t gi = index0 + i;
        out[i] = gi < valid_end ? variate(key, hkey, (uint64_t)gi, scale, heavy_thresh,
                                          heavy_scale)
                                : 0.0f;
    }
}

void synth_normal_bf16(uint16_t *out, int64_t n, uint64_t key, uint64_t hkey, int64_t index0,
                       int64_t valid_end, float scale, uint32_t heavy_thresh, float heavy_scale)
{
    for (int64_t i = 0; i < n; ++i) {
        int64_t gi = index0 + i;
        uint32_t u = 0;
        if (gi < valid_end) {
            float f = variate(key, hkey, (uint64_t)gi, scale, heavy_thresh, heavy_scale);
            memcpy(&u, &f, sizeof u);
        }
        out[i] = (uint16_t)(u >> 16);
    }
}

/*
 * Int8 block-quantized partials, drawn directly (no quantizer involved):
 * q[i] = clamp(z / 1560, -127, 127) with z the Irwin-Hall integer of element
 * gi = index0 + i (C division, truncating toward zero; |q| has standard
 * deviation about 42), 0 past valid_end.  Block b's scale is
 *   base * ((1024 + (h & 1023)) * 2^-10),  h = output b of the stream keyed
 * `skey` (one binary32 multiply by an exact factor in [1, 2)).  Blocks are
 * counted from the shard start (block0 = index of its first block).
 */
void synth_q8(int8_t *out, int64_t n, uint64_t key, int64_t index0, int64_t valid_end)
{
    for (int64_t i = 0; i < n; ++i) {
        int64_t gi = index0 + i;
        int32_t q = 0;
        if (gi < valid_end) {
            q = irwin_hall_z(key, (uint64_t)gi) / 1560;
            if (q > 127) q = 127;
            if (q < -127) q = -127;
        }
        out[i] = (int8_t)q;
    }
}

void synth_q8_scales(float *out, int64_t nblocks, uint64_t skey, int64_t block0, float base)
{
    for (int64_t b = 0; b < nblocks; ++b) {
        uint64_t h = synth_output(skey, (uint64_t)(block0 + b));
        float f = (float)(1024u + (uint32_t)(h & 1023u)) * 0.0009765625f;
        out[b] = base * f;
    }
}
