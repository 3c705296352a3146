// zs_api.hip -- the C ABI declared in include/zs.h: argument checks, launch
// geometry and the launch of the shard step kernels (zs_kernels.hip).
//
// Errors are found on the host before anything is enqueued; the library
// allocates nothing and keeps no pointer after a call returns.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "zs.h"
#include "zs_kernels.h"

namespace {

using namespace zs_detail;

constexpr int kMaxChunkTiles = 4096;

constexpr int kMaxDevices = 64;

struct DeviceInfo {
    int ready;
    int cus;
    int64_t lds_per_cu;     // bytes of LDS one compute unit holds
    int64_t lds_per_group;  // most LDS bytes one workgroup may take
    int xcds;               // accelerator complex dies the device's CUs sit on
};

// Shards of at least this many elements default to the XCD-contiguous chunk
// order (on MI355X it measured 0-3 % faster on shards of 10^8-10^10 elements
// and slower on shards that fit the 256 MB last-level cache).
constexpr int64_t kXcdOrderMinElems = int64_t(1) << 26;

// Default occupancy cap for shards of at least kXcdOrderMinElems elements:
// 5 resident workgroups per CU.  On MI355X it measured 0-8 % faster on shards
// of 0.8-3 x 10^9 elements (most on placements where DRAM queues congest) and
// 1.3-1.6 % faster for every entry point on the 8 x 10^9-element 70B shard
// (same process, two machines; 4 is as good, 6 and more or none slower).  The
// bf16-moment step with one sub-window per wavefront keeps no default cap
// (0-1 % slower under it below 2^32 elements, 9-11 % above).
constexpr int kDefaultCap = 5;
// From this many elements the bf16-moment step with k <= kWideMaxK takes two
// 256-element sub-windows per wavefront (kWide), which gains 0.5-1.9 % under
// the cap there.
constexpr int64_t kWideMinElems = int64_t(1) << 32;
constexpr int kCusPerXcd = 32;  // gfx950

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

// One tile per workgroup by default: the resident workgroups then cover one
// compact stretch of every array and sweep through memory together, which
// measured best on MI355X for every shard size (longer chunks spread the
// active front over more DRAM pages).
constexpr int kDefaultChunkTiles = 1;

// A dispatch packet holds the grid size in work-items as a 32-bit number.
constexpr int64_t kMaxBlocks = 0xffffffffLL / kThreads;

// Elements per workgroup and workgroup count for n elements: chunk_tiles
// tiles of the variant's kernel per workgroup (0 = default), doubled until
// the grid fits.
void launch_geometry(int variant, int64_t n, int chunk_tiles, int64_t *chunk_out,
                     int64_t *blocks_out) {
    if (chunk_tiles == 0) chunk_tiles = kDefaultChunkTiles;
    int64_t chunk = (int64_t)chunk_tiles * tile_for(variant);
    int64_t blocks = (n + chunk - 1) / chunk;
    while (blocks > kMaxBlocks) {
        chunk *= 2;
        blocks = (n + chunk - 1) / chunk;
    }
    *chunk_out = chunk;
    *blocks_out = blocks;
}

// The launch of one call: the geometry, chunk order, occupancy cap and cache
// policy its cfg and the defaults resolve to (device-independent; the XCD
// count and the LDS sizes are applied at launch).
int resolve_launch(int k, int64_t n, int variant, const zs_launch_cfg *cfg,
                   zs_launch_info *out, int *kernel_variant = nullptr) {
    if (k < 1 || k > ZS_MAX_K || n < 0 || n > INT64_MAX / 8) return ZS_ERR_INVALID_ARGUMENT;
    if (variant != 0 && variant != kOutQ8 && variant != kGradQ8 && variant != kMvBf16 &&
        variant != kPacked && variant != (kPacked | kOutQ8) && variant != (kPacked | kGradQ8) &&
        variant != (kPacked | kMvBf16) && variant != (kMvBf16 | kSR) &&
        variant != (kPacked | kMvBf16 | kSR))
        return ZS_ERR_INVALID_ARGUMENT;
    // Streaming (non-temporal) loads and stores by default: nothing is
    // reused, and on MI355X they measured 5-10 % faster than cached access.
    int chunk_tiles = 0, nt = 1, groups_per_cu = 0, block_order = 0;
    if (cfg) {
        if (cfg->chunk_tiles < 0 || cfg->chunk_tiles > kMaxChunkTiles)
            return ZS_ERR_INVALID_ARGUMENT;
        if (cfg->nontemporal < 0 || cfg->nontemporal > 2) return ZS_ERR_INVALID_ARGUMENT;
        if (cfg->groups_per_cu < 0 || cfg->groups_per_cu > ZS_MAX_GROUPS_PER_CU)
            return ZS_ERR_INVALID_ARGUMENT;
        if (cfg->block_order < 0 || cfg->block_order > 2) return ZS_ERR_INVALID_ARGUMENT;
        chunk_tiles = cfg->chunk_tiles;
        nt = cfg->nontemporal == 2 ? 0 : 1;
        groups_per_cu = cfg->groups_per_cu;
        block_order = cfg->block_order;
    }
    const bool mv16 = (variant & kMvBf16) != 0;
    const bool wide = mv16 && n >= kWideMinElems && k <= kWideMaxK;
    const int kv = wide ? (variant | kWide) : variant;
    int64_t chunk = 0, blocks = 0;
    if (n > 0) launch_geometry(kv, n, chunk_tiles, &chunk, &blocks);
    const bool xcd_order = block_order == 2 || (block_order == 0 && n >= kXcdOrderMinElems);
    // the default cap (negative: dropped where the device cannot hold it)
    const int cap = (mv16 && !wide) ? 0 : kDefaultCap;
    if (groups_per_cu == 0 && n >= kXcdOrderMinElems && cap) groups_per_cu = -cap;
    out->workgroups = blocks;
    out->chunk_elements = chunk;
    out->block_order = xcd_order ? 2 : 1;
    out->groups_per_cu = groups_per_cu;
    out->nontemporal = nt;
    out->window_quads = quads_for(kv);
    if (kernel_variant) *kernel_variant = kv;
    return ZS_OK;
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
    uint64_t seed = 0;  // kSR: the caller's seed of the random streams
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
    zs_launch_info plan;
    int kernel_variant = r.variant;
    const int pst = resolve_launch(r.k, r.n, r.variant, r.cfg, &plan, &kernel_variant);
    if (pst != ZS_OK) return pst;
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
    if (r.n == 0) return ZS_OK;
    if (r.n > ((r.variant & kPacked) ? INT64_MAX / 16 : INT64_MAX / 8))
        return ZS_ERR_INVALID_ARGUMENT;
    if (!r.st->segs) return ZS_ERR_INVALID_ARGUMENT;
    if ((uintptr_t)r.st->segs & 7u) return ZS_ERR_MISALIGNED;

    const int64_t n = r.n;
    const int64_t nblocks = (n + kQ8Block - 1) / kQ8Block;
    const int64_t mv_bytes = (r.variant & kMvBf16) ? 2 * n : 4 * n;
    Span outs[6];
    int nouts = 0;
    if (r.variant & kPacked) {
        // the packed state
        const int64_t floats = (r.variant & kMvBf16) ? packed16_floats(n) : packed_floats(n);
        outs[nouts++] = {r.master, 4 * floats, 16};
    } else {
        outs[nouts++] = {r.master, 4 * n, 16};
        outs[nouts++] = {r.m, mv_bytes, 16};
        outs[nouts++] = {r.v, mv_bytes, 16};
    }
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
    // kSR: the stream keys of this step's m and v roundings
    a.sr_key_m = sr_word(r.seed, 2u * (uint64_t)r.step);
    a.sr_key_v = sr_word(r.seed, 2u * (uint64_t)r.step + 1u);

    const int64_t blocks = plan.workgroups;
    a.chunk = plan.chunk_elements;
    a.xcds = plan.block_order == 2 ? g_dev[dev].xcds : 1;
    const bool default_cap = plan.groups_per_cu < 0;
    const int groups_per_cu = default_cap ? -plan.groups_per_cu : plan.groups_per_cu;

    // Occupancy cap: each workgroup reserves 1/groups_per_cu of the unit's
    // LDS (rounded down to 1 KB), so at most groups_per_cu of them fit.  The
    // kernels never touch the reserved bytes.
    // A cap the caller asked for and cannot be met is an error; the default
    // cap is simply dropped on a device where it does not fit.
    size_t dyn_lds = 0;
    if (groups_per_cu > 0) {
        const int64_t share = g_dev[dev].lds_per_cu / groups_per_cu / 1024 * 1024;
        if (share <= g_dev[dev].lds_per_group && share >= kStaticLds)
            dyn_lds = (size_t)(share - kStaticLds);
        else if (!default_cap)
            return ZS_ERR_INVALID_ARGUMENT;
    }

    const int unit_bc = (a.bc1 == 1.0f ? 1 : 0) | (a.bc2 == 1.0f ? 2 : 0);
    kernel_fn fn = pick_kernel(r.k, kernel_variant, plan.nontemporal, unit_bc);
    if (!fn) return ZS_ERR_INVALID_ARGUMENT;
    void *args[] = {&a};
    e = hipLaunchKernel((const void *)fn, dim3((unsigned)blocks), dim3(kThreads), args, dyn_lds,
                        (hipStream_t)r.stream);
    if (e != hipSuccess) return device_error(e);
    return ZS_OK;
}

// zs_pack_state / zs_unpack_state: validate, then one grid-stride launch.
int layout_call(int dir, bool mv16, float *master, void *m, void *v, float *state, int64_t n,
                void *stream) {
    if (!g_initialized) return ZS_ERR_NOT_INITIALIZED;
    if (n < 0 || n > INT64_MAX / 16) return ZS_ERR_INVALID_ARGUMENT;
    if (n == 0) return ZS_OK;
    const int64_t mv_bytes = mv16 ? 2 * n : 4 * n;
    const int64_t floats = mv16 ? packed16_floats(n) : packed_floats(n);
    const Span spans[4] = {{master, 4 * n, 16}, {m, mv_bytes, 16}, {v, mv_bytes, 16},
                           {state, 4 * floats, 16}};
    for (const Span &x : spans)
        if (!x.p) return ZS_ERR_INVALID_ARGUMENT;
    for (const Span &x : spans)
        if ((uintptr_t)x.p & (x.align - 1)) return ZS_ERR_MISALIGNED;
    for (int x = 0; x < 4; ++x)
        for (int y = x + 1; y < 4; ++y)
            if (overlaps(spans[x].p, spans[x].bytes, spans[y].p, spans[y].bytes))
                return ZS_ERR_ALIASING;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_error(e);
    if (dev < 0 || dev >= kMaxDevices || !g_dev[dev].ready) return ZS_ERR_NOT_INITIALIZED;
    // enough workgroups to fill the device; each loops over its share
    const int64_t quads = (n + kSub - 1) / kSub * (kSub / kQuad);
    const int64_t want = (quads + kThreads - 1) / kThreads;
    const int64_t fill = (int64_t)g_dev[dev].cus * 16;
    const int blocks = (int)(want < fill ? want : fill);
    e = mv16 ? launch_layout16(dir, master, (uint16_t *)m, (uint16_t *)v, state, n, blocks,
                               (hipStream_t)stream)
             : launch_layout(dir, master, (float *)m, (float *)v, state, n, blocks,
                             (hipStream_t)stream);
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
    g_dev[device_ordinal].lds_per_cu = (int64_t)prop.maxSharedMemoryPerMultiProcessor;
    g_dev[device_ordinal].lds_per_group = (int64_t)prop.sharedMemPerBlock;
    // A whole MI355X has 8 XCDs of 32 CUs; a partition holds fewer.
    g_dev[device_ordinal].xcds =
        prop.multiProcessorCount % kCusPerXcd == 0 && prop.multiProcessorCount >= kCusPerXcd
            ? prop.multiProcessorCount / kCusPerXcd
            : 1;
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

int zs_shard_step_packed(float *state, uint16_t *param_bf16, const uint16_t *const *grads,
                         int k, int64_t n, const zs_seg_table *seg_table,
                         const zs_hparams *hparams, int64_t step, void *stream) {
    Request r = base_request(state, nullptr, nullptr, param_bf16, k, n, seg_table, hparams, step,
                             stream);
    r.grads = grads;
    r.variant = kPacked;
    return validate_and_launch(r);
}

int zs_shard_step_packed_q8ag(float *state, uint16_t *param_bf16, int8_t *param_q8,
                              float *param_q8_scale, const uint16_t *const *grads, int k,
                              int64_t n, const zs_seg_table *seg_table,
                              const zs_hparams *hparams, int64_t step, void *stream) {
    Request r = base_request(state, nullptr, nullptr, param_bf16, k, n, seg_table, hparams, step,
                             stream);
    r.grads = grads;
    r.q8 = param_q8;
    r.q8_scale = param_q8_scale;
    r.variant = kPacked | kOutQ8;
    return validate_and_launch(r);
}

int zs_shard_step_packed_q8grad(float *state, uint16_t *param_bf16, const int8_t *const *qgrads,
                                const float *const *qscales, int k, int64_t n,
                                const zs_seg_table *seg_table, const zs_hparams *hparams,
                                int64_t step, void *stream) {
    Request r = base_request(state, nullptr, nullptr, param_bf16, k, n, seg_table, hparams, step,
                             stream);
    r.qgrads = qgrads;
    r.qscales = qscales;
    r.variant = kPacked | kGradQ8;
    return validate_and_launch(r);
}

int zs_shard_step_packed_bf16mv(float *state, uint16_t *param_bf16,
                                const uint16_t *const *grads, int k, int64_t n,
                                const zs_seg_table *seg_table, const zs_hparams *hparams,
                                int64_t step, void *stream) {
    Request r = base_request(state, nullptr, nullptr, param_bf16, k, n, seg_table, hparams, step,
                             stream);
    r.grads = grads;
    r.variant = kPacked | kMvBf16;
    return validate_and_launch(r);
}

int zs_shard_step_bf16mv_sr(float *master, uint16_t *m_bf16, uint16_t *v_bf16,
                            uint16_t *param_bf16, const uint16_t *const *grads, int k, int64_t n,
                            const zs_seg_table *seg_table, const zs_hparams *hparams,
                            int64_t step, uint64_t seed, void *stream) {
    Request r = base_request(master, m_bf16, v_bf16, param_bf16, k, n, seg_table, hparams, step,
                             stream);
    r.grads = grads;
    r.variant = kMvBf16 | kSR;
    r.seed = seed;
    return validate_and_launch(r);
}

int zs_shard_step_packed_bf16mv_sr(float *state, uint16_t *param_bf16,
                                   const uint16_t *const *grads, int k, int64_t n,
                                   const zs_seg_table *seg_table, const zs_hparams *hparams,
                                   int64_t step, uint64_t seed, void *stream) {
    Request r = base_request(state, nullptr, nullptr, param_bf16, k, n, seg_table, hparams, step,
                             stream);
    r.grads = grads;
    r.variant = kPacked | kMvBf16 | kSR;
    r.seed = seed;
    return validate_and_launch(r);
}

int zs_pack_state(const float *master, const float *m, const float *v, float *state, int64_t n,
                  void *stream) {
    return layout_call(kLayoutPack, false, const_cast<float *>(master), const_cast<float *>(m),
                       const_cast<float *>(v), state, n, stream);
}

int zs_unpack_state(const float *state, float *master, float *m, float *v, int64_t n,
                    void *stream) {
    return layout_call(kLayoutUnpack, false, master, m, v, const_cast<float *>(state), n, stream);
}

int zs_pack_state_bf16mv(const float *master, const uint16_t *m_bf16, const uint16_t *v_bf16,
                         float *state, int64_t n, void *stream) {
    return layout_call(kLayoutPack, true, const_cast<float *>(master),
                       const_cast<uint16_t *>(m_bf16), const_cast<uint16_t *>(v_bf16), state, n,
                       stream);
}

int zs_unpack_state_bf16mv(const float *state, float *master, uint16_t *m_bf16, uint16_t *v_bf16,
                           int64_t n, void *stream) {
    return layout_call(kLayoutUnpack, true, master, m_bf16, v_bf16, const_cast<float *>(state), n,
                       stream);
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

int zs_launch_geometry(int k, int64_t n, const zs_launch_cfg *cfg, int64_t *workgroups,
                       int64_t *chunk_elements) {
    if (k < 1 || k > ZS_MAX_K || n < 0 || n > INT64_MAX / 8 || !workgroups || !chunk_elements)
        return ZS_ERR_INVALID_ARGUMENT;
    int chunk_tiles = 0;
    if (cfg) {
        if (cfg->chunk_tiles < 0 || cfg->chunk_tiles > kMaxChunkTiles)
            return ZS_ERR_INVALID_ARGUMENT;
        chunk_tiles = cfg->chunk_tiles;
    }
    if (n == 0) {
        *workgroups = 0;
        *chunk_elements = 0;
        return ZS_OK;
    }
    launch_geometry(0, n, chunk_tiles, chunk_elements, workgroups);
    return ZS_OK;
}

int zs_launch_plan(int k, int64_t n, int variant, const zs_launch_cfg *cfg,
                   zs_launch_info *out) {
    if (!out || (cfg && variant != 0)) return ZS_ERR_INVALID_ARGUMENT;
    const int st = resolve_launch(k, n, variant, cfg, out);
    if (st != ZS_OK) return st;
    if (out->groups_per_cu < 0) out->groups_per_cu = -out->groups_per_cu;
    return ZS_OK;
}

int64_t zs_algorithmic_bytes(int k, int64_t n) {
    if (k < 1 || n < 0) return 0;
    return n * (int64_t)(12 + 2 * k) + n * 14;
}

}  // extern "C"
