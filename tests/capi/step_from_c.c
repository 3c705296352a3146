/*
 * The C ABI used from plain C: device memory from the HIP runtime, three
 * shard steps through libzs.so on a stream, the same steps through the C
 * oracle (test infrastructure), and a bitwise comparison.  Exit status 0 and
 * "C ABI: bitwise equal" on success.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zs.h"

/* the oracle's own declarations (it has no header; same field layout) */
int zs_oracle_shard_step(float *, float *, float *, uint16_t *, const uint16_t *const *, int,
                         int64_t, const zs_segment *, int32_t, const zs_hparams *, int64_t);
int zs_oracle_shard_step_bf16mv_sr(float *, uint16_t *, uint16_t *, uint16_t *,
                                   const uint16_t *const *, int, int64_t, const zs_segment *,
                                   int32_t, const zs_hparams *, int64_t, uint64_t, int64_t);

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));            \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

static uint64_t st_ = 0x853C49E6748FEA9Bull;
static uint32_t rnd(void) {
    st_ ^= st_ << 13;
    st_ ^= st_ >> 7;
    st_ ^= st_ << 17;
    return (uint32_t)(st_ >> 11);
}
static float rndf(float s) { return ((float)(rnd() % 20001) - 10000.0f) * s * 1e-4f; }

int main(void) {
    const int64_t n = 1000003;
    const int k = 3;
    zs_segment segs[4] = {{0, 1, 0}, {1000, 0, 0}, {1001, 1, 0}, {500000, 0, 0}};
    zs_hparams hp = {1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f};

    float *w = malloc(4 * n), *m = calloc(n, 4), *v = calloc(n, 4);
    uint16_t *p = calloc(n, 2), *g[3];
    float *wr = malloc(4 * n), *mr = calloc(n, 4), *vr = calloc(n, 4);
    uint16_t *pr = calloc(n, 2);
    for (int64_t i = 0; i < n; ++i) wr[i] = w[i] = rndf(0.02f);

    if (zs_init(0) != ZS_OK) { fprintf(stderr, "zs_init failed\n"); return 1; }
    hipStream_t s;
    CHECK_HIP(hipStreamCreate(&s));
    float *dw, *dm, *dv;
    uint16_t *dp, *dg[3];
    zs_segment *dsegs;
    CHECK_HIP(hipMalloc((void **)&dw, 4 * n));
    CHECK_HIP(hipMalloc((void **)&dm, 4 * n));
    CHECK_HIP(hipMalloc((void **)&dv, 4 * n));
    CHECK_HIP(hipMalloc((void **)&dp, 2 * n));
    CHECK_HIP(hipMalloc((void **)&dsegs, sizeof segs));
    CHECK_HIP(hipMemcpy(dw, w, 4 * n, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dm, m, 4 * n, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dv, v, 4 * n, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dsegs, segs, sizeof segs, hipMemcpyHostToDevice));
    for (int j = 0; j < k; ++j) {
        g[j] = malloc(2 * n);
        CHECK_HIP(hipMalloc((void **)&dg[j], 2 * n));
    }
    zs_seg_table table = {dsegs, 4, 0};

    /* the same steps on the packed state (master, m, v per 256-element block) */
    float *dstate, *du[3];
    uint16_t *dpp;
    CHECK_HIP(hipMalloc((void **)&dstate, 4 * ZS_PACKED_FLOATS(n)));
    CHECK_HIP(hipMalloc((void **)&dpp, 2 * n));
    for (int x = 0; x < 3; ++x) CHECK_HIP(hipMalloc((void **)&du[x], 4 * n));
    if (zs_pack_state(dw, dm, dv, dstate, n, s) != ZS_OK) {
        fprintf(stderr, "zs_pack_state failed\n");
        return 1;
    }

    for (int64_t t = 1; t <= 3; ++t) {
        for (int j = 0; j < k; ++j) {
            for (int64_t i = 0; i < n; ++i) {
                float f = rndf(0.01f);
                uint32_t u;
                memcpy(&u, &f, 4);
                g[j][i] = (uint16_t)(u >> 16);
            }
            CHECK_HIP(hipMemcpy(dg[j], g[j], 2 * n, hipMemcpyHostToDevice));
        }
        const uint16_t *const dgs[3] = {dg[0], dg[1], dg[2]};
        int rc = zs_shard_step(dw, dm, dv, dp, dgs, k, n, &table, &hp, t, s);
        if (rc != ZS_OK) { fprintf(stderr, "zs_shard_step: %s\n", zs_status_string(rc)); return 1; }
        rc = zs_shard_step_packed(dstate, dpp, dgs, k, n, &table, &hp, t, s);
        if (rc != ZS_OK) {
            fprintf(stderr, "zs_shard_step_packed: %s\n", zs_status_string(rc));
            return 1;
        }
        CHECK_HIP(hipStreamSynchronize(s));
        const uint16_t *const hgs[3] = {g[0], g[1], g[2]};
        if (zs_oracle_shard_step(wr, mr, vr, pr, hgs, k, n, segs, 4, &hp, t) != 0) {
            fprintf(stderr, "oracle refused the step\n");
            return 1;
        }
    }
    CHECK_HIP(hipMemcpy(w, dw, 4 * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(m, dm, 4 * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(v, dv, 4 * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(p, dp, 2 * n, hipMemcpyDeviceToHost));
    int bad = memcmp(w, wr, 4 * n) != 0 || memcmp(m, mr, 4 * n) != 0 ||
              memcmp(v, vr, 4 * n) != 0 || memcmp(p, pr, 2 * n) != 0;
    /* the packed state, unpacked on the device, against the oracle too */
    if (zs_unpack_state(dstate, du[0], du[1], du[2], n, s) != ZS_OK) bad = 1;
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(w, du[0], 4 * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(m, du[1], 4 * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(v, du[2], 4 * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(p, dpp, 2 * n, hipMemcpyDeviceToHost));
    if (memcmp(w, wr, 4 * n) != 0 || memcmp(m, mr, 4 * n) != 0 || memcmp(v, vr, 4 * n) != 0 ||
        memcmp(p, pr, 2 * n) != 0) {
        fprintf(stderr, "C ABI: the packed step differs from the oracle\n");
        bad = 1;
    }
    /* bf16 moments rounded stochastically, with a full 64-bit seed */
    {
        const uint64_t seed = 0xFEDCBA9876543210ull;
        float *w2 = malloc(4 * n), *dw2;
        uint16_t *mb = calloc(n, 2), *vb = calloc(n, 2), *pb = calloc(n, 2);
        uint16_t *mbr = calloc(n, 2), *vbr = calloc(n, 2), *pbr = calloc(n, 2);
        uint16_t *dmb, *dvb, *dpb;
        float *wr2 = malloc(4 * n);
        for (int64_t i = 0; i < n; ++i) wr2[i] = w2[i] = rndf(0.02f);
        CHECK_HIP(hipMalloc((void **)&dw2, 4 * n));
        CHECK_HIP(hipMalloc((void **)&dmb, 2 * n));
        CHECK_HIP(hipMalloc((void **)&dvb, 2 * n));
        CHECK_HIP(hipMalloc((void **)&dpb, 2 * n));
        CHECK_HIP(hipMemcpy(dw2, w2, 4 * n, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(dmb, mb, 2 * n, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(dvb, vb, 2 * n, hipMemcpyHostToDevice));
        for (int64_t t = 1; t <= 3; ++t) {
            for (int j = 0; j < k; ++j) {
                for (int64_t i = 0; i < n; ++i) {
                    float f = rndf(0.001f);
                    uint32_t u;
                    memcpy(&u, &f, 4);
                    g[j][i] = (uint16_t)(u >> 16);
                }
                CHECK_HIP(hipMemcpy(dg[j], g[j], 2 * n, hipMemcpyHostToDevice));
            }
            const uint16_t *const dgs2[3] = {dg[0], dg[1], dg[2]};
            int rc = zs_shard_step_bf16mv_sr(dw2, dmb, dvb, dpb, dgs2, k, n, &table, &hp, t, seed,
                                             s);
            if (rc != ZS_OK) {
                fprintf(stderr, "zs_shard_step_bf16mv_sr: %s\n", zs_status_string(rc));
                return 1;
            }
            CHECK_HIP(hipStreamSynchronize(s));
            const uint16_t *const hgs[3] = {g[0], g[1], g[2]};
            if (zs_oracle_shard_step_bf16mv_sr(wr2, mbr, vbr, pbr, hgs, k, n, segs, 4, &hp, t, seed,
                                               0) != 0) {
                fprintf(stderr, "oracle refused the stochastic step\n");
                return 1;
            }
        }
        CHECK_HIP(hipMemcpy(w2, dw2, 4 * n, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(mb, dmb, 2 * n, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(vb, dvb, 2 * n, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(pb, dpb, 2 * n, hipMemcpyDeviceToHost));
        if (memcmp(w2, wr2, 4 * n) != 0 || memcmp(mb, mbr, 2 * n) != 0 ||
            memcmp(vb, vbr, 2 * n) != 0 || memcmp(pb, pbr, 2 * n) != 0) {
            fprintf(stderr, "C ABI: the stochastic step differs from the oracle\n");
            bad = 1;
        }
        hipFree(dw2); hipFree(dmb); hipFree(dvb); hipFree(dpb);
        free(w2); free(wr2); free(mb); free(vb); free(pb); free(mbr); free(vbr); free(pbr);
    }
    /* an argument error is reported synchronously, nothing enqueued */
    const uint16_t *const dgs[3] = {dg[0], dg[1], dg[2]};
    if (zs_shard_step(dw, dm, dv, dp, dgs, k, n, &table, &hp, 0, s) != ZS_ERR_INVALID_ARGUMENT)
        bad = 1;
    for (int j = 0; j < k; ++j) { hipFree(dg[j]); free(g[j]); }
    hipFree(dw); hipFree(dm); hipFree(dv); hipFree(dp); hipFree(dsegs);
    hipFree(dstate); hipFree(dpp);
    for (int x = 0; x < 3; ++x) hipFree(du[x]);
    hipStreamDestroy(s);
    zs_fini();
    if (bad) { fprintf(stderr, "C ABI: results differ from the oracle\n"); return 1; }
    printf("C ABI: bitwise equal (separate and packed state, stochastic bf16 moments)\n");
    return 0;
}
