/*
 * Drives every routine of oracle/zs_oracle.c over exactly-sized heap buffers
 * (ragged n, one- to seven-element segments, 1..16 partials, several
 * quantization blocks, the argument errors), for a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer: any read or write outside a buffer, or any
 * undefined operation, aborts the run.  Test infrastructure only.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct { int64_t start; int32_t wd_on; int32_t reserved; } seg_t;
typedef struct { float lr, beta1, beta2, eps, weight_decay, grad_scale; } hp_t;

int zs_oracle_shard_step(float *, float *, float *, uint16_t *, const uint16_t *const *, int,
                         int64_t, const seg_t *, int32_t, const hp_t *, int64_t);
int zs_oracle_adamw_unsharded(float *, float *, float *, uint16_t *, const float *,
                              const uint8_t *, int64_t, const hp_t *, int64_t);
void zs_oracle_scalars(const hp_t *, int64_t, float out[5]);
uint16_t zs_oracle_bf16_rne(float);
void zs_oracle_bf16_rne_array(const float *, uint16_t *, int64_t);
int zs_oracle_q8_blocks(const uint16_t *, int64_t, int32_t, int8_t *, float *);
void zs_oracle_q8_dequant(const int8_t *, const float *, int64_t, int32_t, float *);
int zs_oracle_shard_step_q8grad(float *, float *, float *, uint16_t *, const int8_t *const *,
                                const float *const *, int, int64_t, int32_t, const seg_t *,
                                int32_t, const hp_t *, int64_t);
int zs_oracle_shard_step_bf16mv(float *, uint16_t *, uint16_t *, uint16_t *,
                                const uint16_t *const *, int, int64_t, const seg_t *, int32_t,
                                const hp_t *, int64_t);
int zs_oracle_shard_step_bf16mv_sr(float *, uint16_t *, uint16_t *, uint16_t *,
                                   const uint16_t *const *, int, int64_t, const seg_t *, int32_t,
                                   const hp_t *, int64_t, uint64_t, int64_t);
void zs_oracle_bf16_sr_array(const float *, const uint32_t *, uint16_t *, int64_t);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 11);
}
static float rndf(float scale) { return ((float)(rnd() % 20001) - 10000.0f) * scale * 1e-4f; }
static uint16_t rnd_bf16(float scale)
{
    float f = rndf(scale);
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}
static void *xmalloc(size_t bytes) { void *p = malloc(bytes ? bytes : 1); if (!p) abort(); return p; }

static int32_t make_segments(seg_t **out, int64_t n)
{
    int32_t cap = (int32_t)(n + 2), c = 0;
    seg_t *s = xmalloc(sizeof(seg_t) * (size_t)cap);
    int64_t a = 0;
    while (a < n && c < cap - 1) {
        s[c].start = a; s[c].wd_on = (int32_t)(rnd() & 1); s[c].reserved = 0; ++c;
        a += 1 + (int64_t)(rnd() % 7);
    }
    if (c == 0) { s[0].start = 0; s[0].wd_on = 1; s[0].reserved = 0; c = 1; }
    s[c].start = n + 3; s[c].wd_on = 1; s[c].reserved = 0; ++c;  /* an entry past n */
    *out = s;
    return c;
}

int main(void)
{
    const int64_t sizes[] = {0, 1, 2, 7, 15, 16, 17, 255, 256, 257, 1000, 4099};
    const int ks[] = {1, 2, 3, 8, 16};
    hp_t hp = {1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f};
    int failures = 0;
    for (size_t si = 0; si < sizeof sizes / sizeof sizes[0]; ++si) {
        const int64_t n = sizes[si];
        for (size_t ki = 0; ki < sizeof ks / sizeof ks[0]; ++ki) {
            const int k = ks[ki];
            float *w = xmalloc(4 * (size_t)n), *m = xmalloc(4 * (size_t)n);
            float *v = xmalloc(4 * (size_t)n);
            uint16_t *p = xmalloc(2 * (size_t)n), *mb = xmalloc(2 * (size_t)n);
            uint16_t *vb = xmalloc(2 * (size_t)n);
            uint16_t *g[16];
            int8_t *q[16];
            const int32_t block = (int32_t)(1 + rnd() % 300);
            const int64_t nb = n ? (n + block - 1) / block : 0;
            float *sc[16];
            for (int64_t i = 0; i < n; ++i) {
                w[i] = rndf(0.02f); m[i] = 0.0f; v[i] = 0.0f; mb[i] = 0; vb[i] = 0;
            }
            for (int j = 0; j < k; ++j) {
                g[j] = xmalloc(2 * (size_t)n);
                q[j] = xmalloc((size_t)n);
                sc[j] = xmalloc(4 * (size_t)nb);
                for (int64_t i = 0; i < n; ++i) {
                    g[j][i] = rnd_bf16(0.01f);
                    q[j][i] = (int8_t)((int)(rnd() % 255) - 127);
                }
                for (int64_t b = 0; b < nb; ++b) sc[j][b] = 1e-4f * (float)(1 + rnd() % 100);
            }
            seg_t *segs;
            const int32_t nseg = make_segments(&segs, n);
            for (int64_t t = 1; t <= 3; ++t) {
                failures += zs_oracle_shard_step(w, m, v, p, (const uint16_t *const *)g, k, n,
                                                 segs, nseg, &hp, t) != 0;
                failures += zs_oracle_shard_step_q8grad(w, m, v, p, (const int8_t *const *)q,
                                                        (const float *const *)sc, k, n, block,
                                                        segs, nseg, &hp, t) != 0;
                failures += zs_oracle_shard_step_bf16mv(w, mb, vb, p,
                                                        (const uint16_t *const *)g, k, n, segs,
                                                        nseg, &hp, t) != 0;
                failures += zs_oracle_shard_step_bf16mv_sr(w, mb, vb, p,
                                                           (const uint16_t *const *)g, k, n,
                                                           segs, nseg, &hp, t, 77u + t,
                                                           (int64_t)(t * 3)) != 0;
            }
            /* argument errors touch nothing */
            failures += zs_oracle_shard_step(w, m, v, p, (const uint16_t *const *)g, k, n, segs,
                                             nseg, &hp, 0) == 0;
            failures += zs_oracle_shard_step(w, m, v, p, (const uint16_t *const *)g, 0, n, segs,
                                             nseg, &hp, 1) == 0;
            /* quantized payload of the new parameters and its receiver side */
            int8_t *pq = xmalloc((size_t)n);
            float *ps = xmalloc(4 * (size_t)nb), *back = xmalloc(4 * (size_t)n);
            failures += zs_oracle_q8_blocks(p, n, block, pq, ps) != 0;
            zs_oracle_q8_dequant(pq, ps, n, block, back);
            /* unsharded routine and the array cast */
            uint8_t *mask = xmalloc((size_t)n);
            float *gf = xmalloc(4 * (size_t)n);
            for (int64_t i = 0; i < n; ++i) { mask[i] = (uint8_t)(rnd() & 1); gf[i] = rndf(0.01f); }
            failures += zs_oracle_adamw_unsharded(w, m, v, p, gf, mask, n, &hp, 1) != 0;
            zs_oracle_bf16_rne_array(w, p, n);
            uint32_t *rb = xmalloc(4 * (size_t)n);
            for (int64_t i = 0; i < n; ++i) rb[i] = rnd();
            zs_oracle_bf16_sr_array(w, rb, p, n);
            free(rb);
            float s5[5];
            zs_oracle_scalars(&hp, 10000, s5);
            free(pq); free(ps); free(back); free(mask); free(gf); free(segs);
            for (int j = 0; j < k; ++j) { free(g[j]); free(q[j]); free(sc[j]); }
            free(w); free(m); free(v); free(p); free(mb); free(vb);
        }
    }
    /* special values through the cast */
    const float specials[] = {0.0f, -0.0f, 1.0f / 0.0f, -1.0f / 0.0f, 3.4028235e38f, 1e-45f};
    for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i)
        (void)zs_oracle_bf16_rne(specials[i]);
    if (failures) {
        fprintf(stderr, "%d unexpected status codes\n", failures);
        return 1;
    }
    printf("oracle driver: clean\n");
    return 0;
}
