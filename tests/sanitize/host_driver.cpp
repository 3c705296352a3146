// Drives zs_host_shard_step (csrc/zs_host.cpp) over exactly-sized heap
// buffers -- ragged n around the 16-wide vector and the 64K-element thread
// chunk, one- to seven-element segments, 1..16 partials, several thread
// counts, the argument errors -- for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer.  Test infrastructure only.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "zs_host.h"

namespace {

uint64_t g_state = 0x243F6A8885A308D3ull;
uint32_t rnd() {
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (uint32_t)(g_state >> 11);
}
float rndf(float s) { return ((float)(rnd() % 20001) - 10000.0f) * s * 1e-4f; }

template <typename T> T *alloc(int64_t n) {
    void *p = std::malloc(n ? (size_t)n * sizeof(T) : 1);
    if (!p) std::abort();
    return static_cast<T *>(p);
}

}  // namespace

int main() {
    const int64_t sizes[] = {0, 1, 15, 16, 17, 31, 65535, 65536, 65537, 200003};
    const int ks[] = {1, 2, 5, 16};
    const int threads[] = {1, 3, 0};
    zs_hparams hp = {1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f};
    int failures = 0;
    for (int64_t n : sizes) {
        for (int k : ks) {
            float *w = alloc<float>(n), *m = alloc<float>(n), *v = alloc<float>(n);
            uint16_t *p = alloc<uint16_t>(n);
            std::vector<uint16_t *> g(k);
            for (int64_t i = 0; i < n; ++i) {
                w[i] = rndf(0.02f);
                m[i] = v[i] = 0.0f;
            }
            for (int j = 0; j < k; ++j) {
                g[j] = alloc<uint16_t>(n);
                for (int64_t i = 0; i < n; ++i) {
                    float f = rndf(0.01f);
                    uint32_t u;
                    std::memcpy(&u, &f, 4);
                    g[j][i] = (uint16_t)(u >> 16);
                }
            }
            std::vector<zs_segment> segs;
            for (int64_t a = 0; a < n || segs.empty(); a += 1 + rnd() % (n > 1000 ? 5000 : 7))
                segs.push_back({a, (int32_t)(rnd() & 1), 0});
            segs.push_back({n + 5, 1, 0});
            for (int th : threads)
                for (int64_t t = 1; t <= 2; ++t)
                    failures += zs_host_shard_step(w, m, v, p, g.data(), k, n, segs.data(),
                                                   (int32_t)segs.size(), &hp, t, th) != ZS_OK;
            // errors: nothing is touched
            failures += zs_host_shard_step(w, m, v, p, g.data(), k, n, segs.data(),
                                           (int32_t)segs.size(), &hp, 0, 1) == ZS_OK;
            if (n > 0)
                failures += zs_host_shard_step(w, w, v, p, g.data(), k, n, segs.data(),
                                               (int32_t)segs.size(), &hp, 1, 1) == ZS_OK;
            for (int j = 0; j < k; ++j) std::free(g[j]);
            std::free(w);
            std::free(m);
            std::free(v);
            std::free(p);
        }
    }
    if (failures) {
        std::fprintf(stderr, "%d unexpected status codes\n", failures);
        return 1;
    }
    std::printf("host driver: clean (%s)\n", zs_host_isa());
    return 0;
}
