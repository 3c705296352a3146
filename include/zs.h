/*
 * zs.h -- C ABI of libzs: one rank's share of the sharded mixed-precision
 * AdamW step (ZeRO-1 "update only my shard"), fused into one HBM pass on
 * AMD Instinct MI355X (gfx950).
 *
 * What one call computes, for every element i of the rank's shard [0, n):
 *
 *   g   = (((f32(G[0][i]) + f32(G[1][i])) + ...) + f32(G[k-1][i])) * grad_scale
 *   m'  = beta1*m + (1-beta1)*g
 *   v'  = beta2*v + (1-beta2)*(g*g)
 *   u   = (m'/bc1) / (sqrt(v'/bc2) + eps),   bc1 = 1-beta1^t, bc2 = 1-beta2^t
 *   w'  = (decay(i) ? w*(1 - lr*wd) : w) - lr*u
 *   master[i] = w', m[i] = m', v[i] = v', param_bf16[i] = bf16_rne(w')
 *
 * Sources (page titles as printed):
 *  - "Chapter 9: Distributed Training and Data Parallelism", section 9.2.2
 *    (Adam moments, bias correction, update with epsilon outside the root);
 *    section 9.3.5 (reduce-scatter hands rank r the SUM of chunk r over all
 *    ranks); section 9.4.2 (ZeRO-1/2 step: reduce-scatter the gradients,
 *    update the owned shard of optimizer state and parameters, all-gather
 *    the parameters).
 *  - "Lecture 7: Parallelism I -- collectives, data parallelism and ZeRO"
 *    (CS336 notes), section 7 (mixed-precision AdamW keeps 16 bytes per
 *    parameter: bf16 weight, bf16 gradient, fp32 master, fp32 m, fp32 v) and
 *    section 8.1 (FlatZeRO1: one flat buffer split evenly across ranks; the
 *    rank's k partials are the inputs of its reduce-scatter chunk).
 *
 * Numerics: IEEE binary32, round to nearest even, one operation at a time in
 * the order above (no fused multiply-add), correctly rounded divide and
 * square root, denormals kept.  bc1, bc2 are formed on the host in binary64
 * as 1 - pow(beta, t) and rounded once; (1-beta1), (1-beta2) and
 * (1 - lr*wd) are formed in binary32.  bf16_rne is round-to-nearest-even on
 * the 16 dropped bits; every NaN becomes 0x7FC0.  "AdamW" decay is read as
 * decoupled and lr-coupled, applied to the pre-step weight.
 *
 * Threading: zs_init/zs_fini must not race with other calls.  After
 * zs_init the library holds no mutable state, so zs_shard_step may be
 * called concurrently from several threads and on several streams.
 *
 * Graph capture: a step call enqueues one kernel and nothing else (no
 * allocation, memset or synchronisation), so it may be recorded into a HIP
 * graph.  The arguments are checked and the bias corrections formed when the
 * call is made, i.e. at capture: every replay repeats the captured call with
 * the same step t and the same buffers.
 */
#ifndef ZS_H_
#define ZS_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZS_MAX_K 16           /* most gradient partials one call sums */
#define ZS_MAX_SEGMENTS 65536 /* most entries in one segment table */
#define ZS_Q8_BLOCK 256       /* elements per int8 quantization block */
#define ZS_MAX_GROUPS_PER_CU 32 /* largest zs_launch_cfg.groups_per_cu */

typedef enum {
    ZS_OK = 0,
    ZS_ERR_NOT_INITIALIZED = 1, /* zs_init not called, or zs_fini called */
    ZS_ERR_INVALID_ARGUMENT = 2,/* bad pointer, size, k, step or hparams */
    ZS_ERR_MISALIGNED = 3,      /* a buffer base is not aligned as documented */
    ZS_ERR_TOO_MANY_SEGMENTS = 4,
    ZS_ERR_DEVICE = 5,          /* a HIP call failed; see zs_last_device_error */
    ZS_ERR_ALIASING = 6         /* output ranges overlap each other or an input */
} zs_status;

/* Optimizer hyper-parameters.  beta1, beta2 in [0, 1); eps >= 0; all finite.
 * grad_scale multiplies the summed gradient (1.0 = plain sum). */
typedef struct {
    float lr, beta1, beta2, eps, weight_decay, grad_scale;
} zs_hparams;

/* One entry of a weight-decay segment table.  start is an element offset
 * inside the shard.  Element i takes wd_on of the LAST entry whose
 * start <= i.  Entries must be sorted by start (non-decreasing) and the
 * first must have start == 0.  Entries with start >= n are ignored.
 * 16 bytes per entry, 8-byte aligned. */
typedef struct {
    int64_t start;
    int32_t wd_on;    /* non-zero: decoupled weight decay applies */
    int32_t reserved; /* must be 0 */
} zs_segment;

/* segs is a DEVICE pointer (device memory the caller owns) to count
 * entries; the table is read by the kernel and never written.  Because it
 * lives on the device the library does not check its order: an unsorted
 * table gives unspecified decay flags but every read stays inside
 * segs[0 .. count-1]. */
typedef struct {
    const zs_segment *segs;
    int32_t count;
    int32_t reserved;
} zs_seg_table;

/* Launch geometry override, for tuning and for determinism tests.  Zero in a
 * field selects the library default.  Results never depend on it. */
typedef struct {
    int32_t chunk_tiles;  /* tiles per workgroup (1..4096); a tile is 1024 elements */
    int32_t nontemporal;  /* 0 = default (streaming), 1 = streaming (non-temporal)
                             loads/stores, 2 = ordinary cached loads/stores */
    int32_t groups_per_cu; /* 1..ZS_MAX_GROUPS_PER_CU caps resident workgroups per
                              compute unit by reserving that share of the unit's LDS
                              per workgroup; ZS_MAX_GROUPS_PER_CU never binds (no
                              cap).  Fewer requests in flight relieve DRAM
                              congestion on many physical placements of the arrays.
                              0 = default: none below 2^26 elements, a cap of 5
                              from 2^26 elements on, except for
                              zs_shard_step_bf16mv (and its packed and
                              stochastic forms) below 2^32 elements or with
                              k > 4 (no cap); from 2^32 elements with k <= 4
                              it takes two 256-element sub-windows per
                              wavefront.
                              A cap whose LDS share exceeds the per-workgroup
                              limit returns ZS_ERR_INVALID_ARGUMENT. */
    int32_t block_order;  /* 0 = default, 1 = linear (workgroup b takes chunk b),
                             2 = XCD-contiguous (the workgroups the dispatcher deals to
                             one XCD take one contiguous run of chunks).  The default
                             is XCD-contiguous for shards of at least 2^26 elements
                             on a part with several XCDs, linear otherwise. */
} zs_launch_cfg;

/* Prepare the library for one device: records its compute-unit count, its
 * LDS sizes and its XCD count (compute units / 32), and checks that it is a
 * gfx950 part.  Idempotent for the same ordinal.
 * Returns ZS_OK, ZS_ERR_INVALID_ARGUMENT (no such device) or
 * ZS_ERR_DEVICE (HIP error, or the device is not gfx950). */
int zs_init(int device_ordinal);

/*
 * Enqueue one shard step on `stream` (a hipStream_t; NULL = the null
 * stream).  The step runs on the calling thread's current device, which
 * zs_init must have prepared; the stream and every buffer must belong to it.
 * Asynchronous: returns once the kernel is enqueued; faults during execution
 * surface at the caller's next synchronisation of the stream.
 *
 *   master, m, v : DEVICE fp32 [n], read and updated in place
 *   param_bf16   : DEVICE bf16 [n] (raw 16-bit patterns), written only
 *   grads        : HOST array of k DEVICE pointers, each bf16 [n], read only;
 *                  partial j is added in the order j = 0, 1, ..., k-1
 *   k            : 1 .. ZS_MAX_K
 *   n            : elements in the shard, >= 0 (n == 0: ZS_OK, nothing enqueued)
 *   seg_table    : HOST struct describing the device-resident table above
 *   hparams      : HOST struct, read during the call only
 *   step         : the optimizer step t >= 1 used in the bias correction
 *
 * All buffers are owned by the caller; the library allocates nothing and
 * keeps no pointer after returning.  Every base pointer (master, m, v,
 * param_bf16, each grads[j]) must be 16-byte aligned, and the segment table
 * 8-byte aligned.  The byte ranges of master, m, v and param_bf16 must not
 * overlap each other or any grads[j] (partials may alias one another).
 *
 * Errors are reported synchronously with nothing enqueued:
 * ZS_ERR_NOT_INITIALIZED, ZS_ERR_INVALID_ARGUMENT (null pointer, k or n out
 * of range, step < 1, non-finite or out-of-range hparams, count < 1),
 * ZS_ERR_TOO_MANY_SEGMENTS, ZS_ERR_MISALIGNED, ZS_ERR_ALIASING.  A launch
 * failure returns ZS_ERR_DEVICE.
 */
int zs_shard_step(float *master, float *m, float *v, uint16_t *param_bf16,
                  const uint16_t *const *grads, int k, int64_t n,
                  const zs_seg_table *seg_table, const zs_hparams *hparams,
                  int64_t step, void *stream);

/* zs_shard_step with an explicit launch geometry (cfg may be NULL).  Same
 * arguments, results and errors; a cfg field out of range returns
 * ZS_ERR_INVALID_ARGUMENT.  Outputs are bitwise identical for every cfg. */
int zs_shard_step_cfg(float *master, float *m, float *v, uint16_t *param_bf16,
                      const uint16_t *const *grads, int k, int64_t n,
                      const zs_seg_table *seg_table, const zs_hparams *hparams,
                      int64_t step, void *stream, const zs_launch_cfg *cfg);

/*
 * zs_shard_step that also writes the block-quantized int8 copy of the new
 * parameters: the payload of a quantized all-gather ("Chapter 9: Distributed
 * Training and Data Parallelism", section 9.4.3, ZeRO++: 16-bit weights are
 * converted to INT8 before the all-gather, halving its volume, and
 * dequantized after it; quantization is block-wise).  The pages give no
 * block size or scale rule; the reading used:
 *   blocks of ZS_Q8_BLOCK consecutive shard elements from element 0 (the
 *   last block may be shorter); x = the new bf16 parameter as fp32;
 *   a = max |x| over the block (NaN if any x is NaN); scale = a / 127
 *   (binary32); q = clamp(round_half_even(x / scale), -127, 127), and q = 0
 *   for every element of a block whose scale is 0 or not finite.
 *   The receiver reconstructs x ~ q * scale, |x - q*scale| <= scale / 2.
 *
 *   param_q8       : DEVICE int8 [n], written only, 16-byte aligned
 *   param_q8_scale : DEVICE fp32 [ceil(n / ZS_Q8_BLOCK)], written only,
 *                    4-byte aligned
 * Every other argument, the other outputs and the errors are those of
 * zs_shard_step; the two new ranges must not overlap any other buffer.
 * Extra HBM traffic: n + 4 * ceil(n / 256) bytes written.
 */
int zs_shard_step_q8ag(float *master, float *m, float *v, uint16_t *param_bf16,
                       int8_t *param_q8, float *param_q8_scale,
                       const uint16_t *const *grads, int k, int64_t n,
                       const zs_seg_table *seg_table, const zs_hparams *hparams,
                       int64_t step, void *stream);

/*
 * zs_shard_step whose k partials arrive block-quantized to int8, as a
 * quantized reduce-scatter would deliver them ("Chapter 9", section 9.4.3,
 * ZeRO++: gradients of the reduce-scatter quantized block-wise).  Partial j
 * of element i is qgrads[j][i] * qscales[j][i / ZS_Q8_BLOCK], each product
 * rounded once in binary32; the partials are then summed in the same left
 * fold j = 0 .. k-1 as zs_shard_step and multiplied by grad_scale.
 *
 *   qgrads  : HOST array of k DEVICE pointers, int8 [n], 16-byte aligned
 *   qscales : HOST array of k DEVICE pointers, fp32 [ceil(n / ZS_Q8_BLOCK)],
 *             4-byte aligned
 * Everything else as zs_shard_step.  HBM traffic per element:
 * 12 + k (1 + 4/256) bytes read, 14 written.
 */
int zs_shard_step_q8grad(float *master, float *m, float *v, uint16_t *param_bf16,
                         const int8_t *const *qgrads, const float *const *qscales, int k,
                         int64_t n, const zs_seg_table *seg_table, const zs_hparams *hparams,
                         int64_t step, void *stream);

/*
 * zs_shard_step with the moments m and v stored as bf16: the "everything in
 * BF16 except the fp32 master weights" state of "Lecture 7: Parallelism I",
 * section 8.4 (12 bytes per parameter instead of 16).  Each element's m and
 * v are widened to fp32, updated exactly as in zs_shard_step (the weight
 * update uses the unrounded new moments), and stored back rounded to nearest
 * even (reading: the page does not say how the moments are rounded).
 *
 *   m_bf16, v_bf16 : DEVICE bf16 [n], read and updated in place, 16-byte
 *                    aligned
 * Everything else as zs_shard_step.  HBM traffic per element: 8 + 2k bytes
 * read, 10 written.
 */
int zs_shard_step_bf16mv(float *master, uint16_t *m_bf16, uint16_t *v_bf16,
                         uint16_t *param_bf16, const uint16_t *const *grads, int k, int64_t n,
                         const zs_seg_table *seg_table, const zs_hparams *hparams,
                         int64_t step, void *stream);

/*
 * zs_shard_step on optimizer state packed in one fp32 array.  The fp32
 * master weights and the two moments ("Chapter 9: Distributed Training and
 * Data Parallelism", section 9.2.1: 12 bytes of fp32 state per parameter)
 * belong to the rank's optimizer alone (section 9.4.2: each rank keeps and
 * updates only its shard of them, and no collective moves them), so their
 * layout is the library's to choose.  Packed, block b of 256 elements holds
 * the master values of elements 256b .. 256b + 255, then their m, then
 * their v:
 *   state[768 b + j]       = master[256 b + j]
 *   state[768 b + 256 + j] = m[256 b + j]
 *   state[768 b + 512 + j] = v[256 b + j]        (0 <= j < 256)
 * ZS_PACKED_FLOATS(n) floats in all; the slots past n in the last block are
 * padding, which the step neither reads nor writes.  Each wavefront then
 * moves its state as one 3 KB run instead of three 1 KB runs in three
 * arrays: on MI355X about 2 % faster on average on the 70B-shaped shard,
 * though a single run can go either way (the placement of the arrays in
 * physical memory alone moves either layout by up to 3 %), and 2-7 % on
 * the smaller shards measured.  The arithmetic and every output bit are
 * zs_shard_step's.
 *
 *   state : DEVICE fp32 [ZS_PACKED_FLOATS(n)], read and updated in place,
 *           16-byte aligned
 * Everything else as zs_shard_step (ZS_ERR_ALIASING when param_bf16 or a
 * partial overlaps the state).  HBM traffic: that of zs_shard_step.
 */
#define ZS_PACKED_FLOATS(n) (768 * (((int64_t)(n) + 255) / 256))
int zs_shard_step_packed(float *state, uint16_t *param_bf16, const uint16_t *const *grads,
                         int k, int64_t n, const zs_seg_table *seg_table,
                         const zs_hparams *hparams, int64_t step, void *stream);

/*
 * zs_shard_step_q8ag and zs_shard_step_q8grad on the packed state: the same
 * outputs (the int8 parameter copy and its scales; the int8 partials and
 * their scales read as there), bit for bit, with master, m and v in `state`
 * as for zs_shard_step_packed.  Everything else as those entry points.
 */
int zs_shard_step_packed_q8ag(float *state, uint16_t *param_bf16, int8_t *param_q8,
                              float *param_q8_scale, const uint16_t *const *grads, int k,
                              int64_t n, const zs_seg_table *seg_table,
                              const zs_hparams *hparams, int64_t step, void *stream);
int zs_shard_step_packed_q8grad(float *state, uint16_t *param_bf16, const int8_t *const *qgrads,
                                const float *const *qscales, int k, int64_t n,
                                const zs_seg_table *seg_table, const zs_hparams *hparams,
                                int64_t step, void *stream);

/*
 * zs_shard_step_bf16mv on packed state: the bf16-moment state of "Lecture 7:
 * Parallelism I", section 8.4 (fp32 master weights, bf16 m and v) in one
 * array, the rank's own to lay out as for zs_shard_step_packed.  Block b of
 * 256 elements takes 2 KB: the fp32 master values of elements 256b .. 256b +
 * 255, then their m and then their v as bf16.  In 16-bit units (state viewed
 * as uint16_t, j = 0 .. 255):
 *   state as fp32    [512 b + j]        = master[256 b + j]
 *   state as uint16_t[1024 b + 512 + j] = m_bf16[256 b + j]
 *   state as uint16_t[1024 b + 768 + j] = v_bf16[256 b + j]
 * ZS_PACKED_BF16MV_FLOATS(n) floats in all (the last block's slots past n
 * are padding the step neither reads nor writes).  The arithmetic and every
 * output bit are zs_shard_step_bf16mv's.
 *
 *   state : DEVICE [ZS_PACKED_BF16MV_FLOATS(n) floats], read and updated in
 *           place, 16-byte aligned
 * Everything else as zs_shard_step_bf16mv.  HBM traffic: that of
 * zs_shard_step_bf16mv.
 */
#define ZS_PACKED_BF16MV_FLOATS(n) (512 * (((int64_t)(n) + 255) / 256))
int zs_shard_step_packed_bf16mv(float *state, uint16_t *param_bf16,
                                const uint16_t *const *grads, int k, int64_t n,
                                const zs_seg_table *seg_table, const zs_hparams *hparams,
                                int64_t step, void *stream);

/*
 * zs_shard_step_bf16mv (and its packed form) with the new m and v rounded to
 * bf16 stochastically instead of to nearest: the other reading of "Lecture 7:
 * Parallelism I", section 8.4, which keeps the moments in bf16 without saying
 * how they are rounded.  Each moment's magnitude is rounded up to the next
 * bf16 with probability (its 16 dropped bits) / 2^16 and down otherwise, so
 * the stored moment equals the exact one in expectation; NaN -> 0x7FC0,
 * infinities stay, the largest finite value may round up to infinity.  The
 * master update uses the unrounded moments and the parameter copy is rounded
 * to nearest even, as in zs_shard_step_bf16mv.
 *
 * Random bits: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used counter-style, output i
 * of key K being mix64(K + (i + 1) * 0x9E3779B97F4A7C15).  At step t the key
 * of m's stream is output 2t of `seed`, that of v's output 2t + 1; element i
 * (shard-local) takes bits 16 (i mod 4) .. 16 (i mod 4) + 15 of output i / 4
 * of the stream.  The result is a function of (inputs, step, seed) alone,
 * whatever the launch; ranks should pass different seeds.
 *
 * Arguments, layout, errors and traffic as zs_shard_step_bf16mv and
 * zs_shard_step_packed_bf16mv, plus `seed`.
 */
int zs_shard_step_bf16mv_sr(float *master, uint16_t *m_bf16, uint16_t *v_bf16,
                            uint16_t *param_bf16, const uint16_t *const *grads, int k, int64_t n,
                            const zs_seg_table *seg_table, const zs_hparams *hparams,
                            int64_t step, uint64_t seed, void *stream);
int zs_shard_step_packed_bf16mv_sr(float *state, uint16_t *param_bf16,
                                   const uint16_t *const *grads, int k, int64_t n,
                                   const zs_seg_table *seg_table, const zs_hparams *hparams,
                                   int64_t step, uint64_t seed, void *stream);

/*
 * Convert, on `stream`, between separate master, m and v arrays (DEVICE fp32
 * [n] each) and the packed state of zs_shard_step_packed (DEVICE fp32
 * [ZS_PACKED_FLOATS(n)]).  zs_pack_state writes every slot of the state, the
 * padding past n as +0; zs_unpack_state writes master, m and v [0, n) and
 * nothing else.  Every pointer 16-byte aligned; the state must not overlap
 * the arrays, nor the arrays each other.  Asynchronous like a step; errors
 * are reported synchronously with nothing enqueued (ZS_ERR_NOT_INITIALIZED,
 * ZS_ERR_INVALID_ARGUMENT, ZS_ERR_MISALIGNED, ZS_ERR_ALIASING, ZS_ERR_DEVICE);
 * n == 0 does nothing.
 */
int zs_pack_state(const float *master, const float *m, const float *v, float *state, int64_t n,
                  void *stream);
int zs_unpack_state(const float *state, float *master, float *m, float *v, int64_t n,
                    void *stream);

/*
 * The same conversions for the bf16-moment state: fp32 master [n] and bf16
 * m_bf16, v_bf16 [n] (DEVICE) to and from the packed state of
 * zs_shard_step_packed_bf16mv (DEVICE, ZS_PACKED_BF16MV_FLOATS(n) floats).
 * Padding past n is written as zero bits.  Everything else as zs_pack_state.
 */
int zs_pack_state_bf16mv(const float *master, const uint16_t *m_bf16, const uint16_t *v_bf16,
                         float *state, int64_t n, void *stream);
int zs_unpack_state_bf16mv(const float *state, float *master, uint16_t *m_bf16, uint16_t *v_bf16,
                           int64_t n, void *stream);

/* Release what zs_init recorded.  Later calls return ZS_ERR_NOT_INITIALIZED
 * until zs_init is called again.  Always returns ZS_OK. */
int zs_fini(void);

/* Static, NUL-terminated description of a status code. */
const char *zs_status_string(int status);

/* The last hipError_t seen by the library on the calling thread (0 = none). */
int zs_last_device_error(void);

/* The grid a step over n elements with k partials would launch (cfg may be
 * NULL; only its chunk_tiles matters): *workgroups of 256 threads, each
 * owning *chunk_elements consecutive elements (the last one fewer).  The
 * chunk is chunk_tiles tiles of 1024 elements (default 1), doubled as often
 * as needed to keep workgroups * 256 below 2^32, the largest grid a dispatch
 * can describe.  Host-only; needs no device and no zs_init.  n == 0 gives 0
 * and 0.  Returns ZS_OK or ZS_ERR_INVALID_ARGUMENT (k or n out of range,
 * null output, chunk_tiles out of range). */
int zs_launch_geometry(int k, int64_t n, const zs_launch_cfg *cfg, int64_t *workgroups,
                       int64_t *chunk_elements);

/* Entry points, as zs_launch_plan names them. */
#define ZS_VARIANT_BASE 0   /* zs_shard_step, zs_shard_step_cfg */
#define ZS_VARIANT_Q8AG 1   /* zs_shard_step_q8ag */
#define ZS_VARIANT_Q8GRAD 2 /* zs_shard_step_q8grad */
#define ZS_VARIANT_BF16MV 4 /* zs_shard_step_bf16mv */
#define ZS_VARIANT_PACKED 16 /* zs_shard_step_packed */
#define ZS_VARIANT_PACKED_Q8AG 17   /* zs_shard_step_packed_q8ag */
#define ZS_VARIANT_PACKED_Q8GRAD 18 /* zs_shard_step_packed_q8grad */
#define ZS_VARIANT_PACKED_BF16MV 20 /* zs_shard_step_packed_bf16mv */
#define ZS_VARIANT_BF16MV_SR 36     /* zs_shard_step_bf16mv_sr */
#define ZS_VARIANT_PACKED_BF16MV_SR 52 /* zs_shard_step_packed_bf16mv_sr */

/* The launch a step call resolves its defaults to. */
typedef struct {
    int64_t workgroups;     /* workgroups of 256 threads (0 when n == 0) */
    int64_t chunk_elements; /* consecutive elements each workgroup owns (the last fewer) */
    int32_t block_order;    /* 1 = linear, 2 = XCD-contiguous (a part with a single XCD
                               runs the linear order either way) */
    int32_t groups_per_cu;  /* resident-workgroup cap per compute unit the launch asks
                               for, 0 = none (a default cap the device cannot hold is
                               dropped at launch) */
    int32_t nontemporal;    /* 1 = streaming loads and stores, 0 = cached */
    int32_t window_quads;   /* 256-element sub-windows each wavefront takes per tile
                               (1, or 2 for zs_shard_step_bf16mv and its packed and
                               stochastic forms on shards of at least 2^32 elements
                               with k <= 4) */
} zs_launch_info;

/* The launch a call of entry point `variant` (ZS_VARIANT_*) over n elements
 * with k partials and the override cfg (NULL = defaults, the only choice for
 * the variants other than ZS_VARIANT_BASE) would make: grid, chunk, chunk
 * order, occupancy cap and cache policy.  These decide the kernel's memory
 * traffic pattern; its arithmetic does not depend on them.  Host-only; needs
 * no device and no zs_init.  Returns ZS_OK or ZS_ERR_INVALID_ARGUMENT (k, n,
 * variant or a cfg field out of range, a cfg with a variant other than
 * ZS_VARIANT_BASE, or a null out). */
int zs_launch_plan(int k, int64_t n, int variant, const zs_launch_cfg *cfg,
                   zs_launch_info *out);

/* Bytes one zs_shard_step call moves through HBM, by the algorithm:
 * n * (12 + 2k) read + n * 14 written.  For reporting only. */
int64_t zs_algorithmic_bytes(int k, int64_t n);

#ifdef __cplusplus
}
#endif

#endif /* ZS_H_ */
