// zs_kernels.h -- what the C ABI layer (zs_api.hip) and the kernels
// (zs_kernels.hip) share: the launch geometry, the kernel argument block, the
// variant bits and the kernel table.  Private to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "zs.h"

namespace zs_detail {

constexpr int kThreads = 256;                 // 4 wavefronts of 64 lanes
constexpr int kWave = 64;
constexpr int kQuad = 4;                      // contiguous elements per lane per sub-window
constexpr int kSub = kWave * kQuad;           // 256: one dense instruction per array per wave

// Variants of the step, chosen at compile time (bit mask):
//   kOutQ8  - also write the block-quantized int8 copy of the new parameters
//             with one fp32 scale per kQ8Block elements (the payload of a
//             quantized all-gather);
//   kGradQ8 - the k partials arrive as int8 with one fp32 scale per
//             kQ8Block elements each (a block-quantized reduce-scatter) and
//             are dequantized inside the reduce;
//   kMvBf16 - the moments m and v are stored as bf16 (12 bytes per parameter
//             of optimizer state plus weight instead of 16).
//   kWide   - two sub-windows per wave instead of one (launch-time choice for
//             the bf16-moment step on the largest shards, see quads_for);
//   kSR     - with kMvBf16: m and v are rounded to bf16 stochastically (the
//             magnitude rounds up with probability equal to the dropped
//             bits over 2^16), with 16 random bits per rounding from
//             SplitMix64 streams keyed per step and moment (see sr_word);
//   kPacked - master, m and v live in one array, packed per kSub-element
//             block: block b holds the master values of elements kSub*b ..
//             kSub*b + kSub-1, then their m, then their v (ZS packed layout;
//             with kMvBf16 the m and v runs are bf16, 2 KB per block).
constexpr int kOutQ8 = 1;
constexpr int kGradQ8 = 2;
constexpr int kMvBf16 = 4;
constexpr int kWide = 8;
constexpr int kPacked = 16;
constexpr int kSR = 32;

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014) used counter-style: output i of the stream with
// key `key`.  The stochastic step's stream for moment w (0 = m, 1 = v) at
// step t has key sr_word(seed, 2t + w); element i takes the 16 bits
// 16 (i mod 4) .. 16 (i mod 4) + 15 of its output i / 4.
__host__ __device__ constexpr uint64_t sr_word(uint64_t key, uint64_t i) {
    uint64_t z = key + (i + 1u) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static_assert(sr_word(0, 0) == 0xE220A8397B1DCDAFull, "SplitMix64's first output for seed 0");

// Packed layout: index of element i's master value (its m is kSub further,
// its v 2*kSub further), and floats the packed state holds for n elements.
__host__ __device__ constexpr int64_t packed_index(int64_t i) {
    return (i / kSub) * (3 * kSub) + i % kSub;
}
constexpr int64_t packed_floats(int64_t n) { return 3 * kSub * ((n + kSub - 1) / kSub); }

// Packed layout with bf16 moments (kPacked | kMvBf16): block b holds kSub
// fp32 master values, then their m and their v as bf16.  Float index of
// element i's master value, 16-bit index of its m (its v is kSub further),
// and floats the state holds for n elements.
__host__ __device__ constexpr int64_t packed16_master(int64_t i) {
    return (i / kSub) * (2 * kSub) + i % kSub;
}
__host__ __device__ constexpr int64_t packed16_m(int64_t i) {
    return (i / kSub) * (4 * kSub) + 2 * kSub + i % kSub;
}
constexpr int64_t packed16_floats(int64_t n) { return 2 * kSub * ((n + kSub - 1) / kSub); }
static_assert(packed16_m(kSub) == 2 * packed16_master(kSub) + 2 * kSub, "bf16 runs follow master");

// Sub-windows (quads per lane) a wave handles per tile.  Measured on MI355X
// with the per-wavefront segment lookup: one quad per lane, i.e. the fewest
// bytes in flight per wave and the most waves, streams as fast as or faster
// than two or four quads for every partial count and entry point in the
// default launches (even on the eight-partial 7B shard; 5-12 % faster on small
// shards, which get four times the workgroups; two quads lost 0.2-0.6 % on the
// 70B- and 175B-shaped shards for the base and bf16-moment steps, same
// process).  The exception is kWide: on shards of 2^32 elements and more the
// bf16-moment step with two quads per lane under an occupancy cap of 5 moved
// 1.3-1.9 % more than with one quad uncapped (same process, three machines),
// while one quad under that cap lost 9-11 %: fewer waves, each with twice
// the loads in flight across its arithmetic.
constexpr int quads_for(int variant) { return (variant & kWide) ? 2 : 1; }
constexpr int tile_for(int variant) { return (kThreads / kWave) * quads_for(variant) * kSub; }

static_assert(tile_for(0) == 1024 && tile_for(kMvBf16 | kWide) == 2048, "tile sizes");

struct StepArgs {
    float *master;   // fp32 [n], or the packed state (kPacked; bf16 moments inside with kMvBf16)
    void *m;         // fp32 [n], or bf16 [n] in the bf16-moment variant; unused with kPacked
    void *v;
    uint16_t *param;
    int8_t *q8;      // quantized parameter copy (variant with an int8 payload)
    float *q8_scale;
    const uint16_t *grads[ZS_MAX_K];   // bf16 partials
    const int8_t *qgrads[ZS_MAX_K];    // int8 partials (block-quantized variant)
    const float *qscales[ZS_MAX_K];
    const zs_segment *segs;
    int64_t n;
    int64_t chunk;  // elements per workgroup, a multiple of tile_for(variant)
    int32_t nseg;
    int32_t xcds;   // XCDs the dispatcher deals workgroups to in turn; 1 = linear order
    float lr, b1, b2, c1, c2, bc1, bc2, eps, df, gscale;
    uint64_t sr_key_m, sr_key_v;  // kSR: the step's stream keys for m and v
};

constexpr int kQ8Block = ZS_Q8_BLOCK;
static_assert(kQ8Block == kSub, "a quantization block is one sub-window of a wave");

// LDS each workgroup of every kernel declares: one boundary slot per
// wavefront, 64 eight-byte segment starts and 64 one-byte flags.
constexpr int64_t kStaticLds = (int64_t)(8 + 1) * kWave * (kThreads / kWave);

typedef void (*kernel_fn)(const StepArgs);

// Conversion between separate master, m, v arrays [n] and the packed state
// (kPacked layout, packed_floats(n) floats): dir 0 packs (the padding past n
// is written as +0), dir 1 unpacks (nothing past n is written).  A
// grid-stride loop over `blocks` workgroups of kThreads.
constexpr int kLayoutPack = 0;
constexpr int kLayoutUnpack = 1;
hipError_t launch_layout(int dir, float *master, float *m, float *v, float *state, int64_t n,
                         int blocks, hipStream_t stream);
// The same between fp32 master, bf16 m and v [n] and the packed state with
// bf16 moments (packed16_floats(n) floats).
hipError_t launch_layout16(int dir, float *master, uint16_t *m, uint16_t *v, float *state,
                           int64_t n, int blocks, hipStream_t stream);

// Most partials the wide (kWide) kernels are built for.
constexpr int kWideMaxK = 4;

// The kernel for k partials, a variant (0 or one of the bits above; kWide
// only with kMvBf16 and k <= kWideMaxK; kPacked only streaming),
// streaming (nt = 1) or cached (nt = 0) access and the bias corrections that
// are exactly 1.0f (unit_bc bit 0: bc1, bit 1: bc2; a streaming kernel then
// leaves out that division); nullptr if there is none.
kernel_fn pick_kernel(int k, int variant, int nt, int unit_bc);

}  // namespace zs_detail
