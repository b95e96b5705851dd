/*
 * zs.h - one data-parallel rank's ZeRO-1/2 optimizer step on MI355X (gfx950).
 *
 * The operation (CS336 lecture 8 notes "Parallelism basics", section "Code
 * example: ZeRO-1"; podcast summary of N. Tazi's "Training at thousands of
 * GPUs", section "ZeRO optimizer"): reduce-scatter the gradients so that
 * each rank holds the summed gradient of its own slice, update only that
 * slice with AdamW on rank-local fp32 state, then all-gather the updated
 * parameters.  Mixed precision follows the 16 bytes per parameter of the
 * same notes ("Core concepts"): bf16 parameter, bf16 gradient, fp32 master
 * weight and two fp32 Adam moments.  Gradients travel in buckets of
 * bucket_cap_mb = 25 (podcast summary, section "Data parallelism";
 * DDP-to-ZeRO blog, section 2.1).
 *
 * On one GPU the W ranks' gradient slices for this rank's shard are W
 * resident bf16 arrays; the library performs the arithmetic of the
 * reduce-scatter (sum in fp32 in rank order 0..W-1, then divide by W), the
 * AdamW update and the bf16 copy in one pass, and places the bf16 result
 * where the all-gather reads or writes it.
 *
 * Conventions for every call:
 *  - Return 0 on success or a negative ZS_E* code; nothing aborts and no
 *    exception crosses this interface.  zs_last_error() gives a text for the
 *    last failure on the calling thread.
 *  - Device pointers are HIP device memory on the current device, owned by
 *    the caller.  The library never allocates device memory.
 *  - Device calls are asynchronous on the given hipStream_t (passed as
 *    void*, NULL = the null stream).  Faults surface at the caller's next
 *    synchronisation.  Calls that touch the same arrays must be ordered by
 *    the caller (same stream or events).
 *  - bf16 values are passed as their 16-bit patterns (uint16_t).
 *  - NaN and Inf propagate element by element: no clipping, loss scaling or
 *    step skipping (the pages describe none).
 */
#ifndef ZS_H
#define ZS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZS_OK        0
#define ZS_EINVAL  (-1)  /* null pointer, bad count, W < 1, rank >= W, t < 1 */
#define ZS_EALIGN  (-2)  /* device pointer or stride not 16-byte aligned    */
#define ZS_ERANGE  (-3)  /* id out of range, size overflow, short stride    */
#define ZS_ENOMEM  (-4)  /* host allocation failed                          */
#define ZS_EDEVICE (-5)  /* HIP launch error                                */
#define ZS_EIO     (-6)  /* file cannot be opened, read or written; not a
                            checkpoint, truncated, or its checksum fails    */
#define ZS_EMISMATCH (-7) /* checkpoint written for another layout         */

/* Opaque host-side layout of one rank.  Created by zs_layout_build, released
 * by zs_layout_free; read-only afterwards, so it may be shared by threads. */
typedef struct zs_layout zs_layout;

/* One bucket: flat window [flat_off, flat_off + numel) of the flat bf16
 * buffer; rank r owns [flat_off + r*slice_numel, + slice_numel), which sits
 * at [shard_off, shard_off + slice_numel) of the rank's shard.  In the tiled
 * layouts below the slice occupies ceil(slice_numel / ZS_TILE) tiles from
 * tile tile_off on. */
typedef struct {
    int64_t flat_off;
    int64_t numel;
    int64_t slice_numel;
    int64_t shard_off;
    int64_t tile_off;
} zs_bucket;

/* One chunk: a maximal run of the rank's shard inside one tensor.
 * Elements [tensor_off, tensor_off + numel) of tensor tensor_id are shard
 * elements [shard_off, shard_off + numel), all inside bucket bucket_id. */
typedef struct {
    int32_t tensor_id;
    int32_t bucket_id;
    int64_t tensor_off;
    int64_t numel;
    int64_t shard_off;
} zs_chunk;

/* AdamW hyper-parameters (DDP-to-ZeRO blog, section 3.3: the optimizer is
 * AdamW).  Decoupled weight decay multiplies the master by (1 - lr*wd). */
typedef struct {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;
} zs_adamw;

/* ---- layout (host only) ------------------------------------------------ */

/* Build the layout of rank `rank` of `world` for a parameter list of
 * n_tensors tensors with tensor_numel[k] >= 0 elements, in list order.
 *
 * Flattening (podcast summary, "ZeRO optimizer": FSDP1 flattens before it
 * shards; DDP-to-ZeRO blog 3.3: contiguous_gradients): tensor k starts at
 * the first multiple of align_bytes/2 elements at or after the end of
 * tensor k-1.  Bucketing: a full bucket is the largest multiple of
 * world*align_bytes/2 elements whose bf16 size is <= bucket_cap_bytes
 * (25<<20 for bucket_cap_mb = 25); buckets are consecutive windows of the
 * flat buffer and may cut through tensors; the last bucket is the rest,
 * rounded up to world*align_bytes/2 with zero padding.  bucket_cap_bytes
 * <= 0 means one bucket (the single reduce_scatter_tensor of the sketch).
 * Ownership: rank r owns slice r of every bucket; its shard is those
 * slices in bucket order.
 *
 * align_bytes: positive multiple of 16 (256 recommended).  n_tensors may be
 * 0 (empty layout, every device call is then a no-op).
 * Errors: ZS_EINVAL for null out/tensor_numel (when n_tensors > 0),
 * n_tensors < 0, numel < 0, world < 1, rank outside [0, world),
 * bad align_bytes, or 0 < bucket_cap_bytes < world*align_bytes;
 * ZS_ERANGE on int64 overflow or a bucket slice above 2^21 - 1 tiles
 * (17.2 G elements, the most one kernel launch covers); ZS_ENOMEM. */
int zs_layout_build(const int64_t* tensor_numel, int32_t n_tensors,
                    int32_t world, int32_t rank, int64_t bucket_cap_bytes,
                    int32_t align_bytes, zs_layout** out);

/* Whole-tensor shard assignment (podcast summary, "ZeRO optimizer": an
 * optimizer that needs whole tensors, such as Muon, cannot work on
 * flattened slices, so the shards are assigned at whole-tensor granularity,
 * as FSDP2 keeps whole tensors per rank).
 *
 * Every tensor belongs entirely to one rank, assigned greedily longest
 * first: in order of decreasing padded size (numel rounded up to
 * align_bytes/2 elements; ties by list index), each tensor goes to the rank
 * with the least padded load so far (ties to the lowest rank).  Rank
 * `rank`'s shard is its tensors in list order, each padded; each owned
 * non-empty tensor is one bucket {flat_off = the tensor's flat offset,
 * numel = slice_numel = its padded size, shard_off, tile_off} whose whole
 * extent is this rank's slice, and one chunk.  The flat buffer is the same
 * aligned flattening as zs_layout_build, rounded up to align_bytes/2
 * elements; the padded tensors partition it.  The gradient exchange becomes
 * a reduce of each tensor to its owner (the W source ranks' gradients of
 * the owned tensors arrive as the [W][...] slices of this shard) and the
 * all-gather a broadcast from the owner: zs_step, zs_step_bf16, the bucket
 * steps, the conversions, zs_pack and zs_gather all accept such a layout.
 * Errors as zs_layout_build (the 2^21 - 1 tile limit applies to each
 * tensor). */
int zs_layout_build_tensors(const int64_t* tensor_numel, int32_t n_tensors,
                            int32_t world, int32_t rank, int32_t align_bytes,
                            zs_layout** out);

/* Whole-tensor layouts only: owner rank of every tensor and the tensor's
 * offset in its owner's shard, into caller memory of `cap` entries each.
 * Returns the tensor count, ZS_ERANGE if cap is short, ZS_EINVAL for a
 * flat-mode layout. */
int zs_layout_owners(const zs_layout* layout, int32_t* owner,
                     int64_t* owner_shard_off, int32_t cap);

/* Sizes: flat buffer elements (padding included), this rank's shard
 * elements, bucket count, this rank's chunk count.  Null outputs skipped. */
int zs_layout_info(const zs_layout* layout, int64_t* flat_numel,
                   int64_t* shard_numel, int32_t* n_buckets,
                   int32_t* n_chunks);

/* Number of tiles of this rank's shard: sum over buckets of
 * ceil(slice_numel / ZS_TILE).  The tiled state holds n_tiles*3*ZS_TILE
 * floats, tiled gradients n_tiles*W*ZS_TILE bf16 values. */
int zs_layout_tiles(const zs_layout* layout, int64_t* n_tiles);

/* Copy the bucket table / chunk table / tensor start offsets (flat element
 * index of each tensor's first element) into caller memory holding `cap`
 * entries.  Return the number of entries, or ZS_ERANGE if cap is short. */
int zs_layout_buckets(const zs_layout* layout, zs_bucket* out, int32_t cap);
int zs_layout_chunks(const zs_layout* layout, zs_chunk* out, int32_t cap);
int zs_layout_tensor_offsets(const zs_layout* layout, int64_t* out,
                             int32_t cap);

/* world and rank the layout was built for. */
int zs_layout_rank(const zs_layout* layout, int32_t* world, int32_t* rank);

void zs_layout_free(zs_layout* layout);

/* ---- HBM layouts of the step's operands --------------------------------- */

/* A tile is ZS_TILE consecutive elements of one bucket's slice: slice
 * element j of bucket b lies in tile b.tile_off + j / ZS_TILE at position
 * j % ZS_TILE; a slice's last tile is padded when slice_numel is not a
 * multiple of ZS_TILE.  The step works tile by tile (one workgroup, or a
 * fixed set of workgroups, per tile), and the tiled layouts keep everything
 * a tile reads or writes in a few long contiguous runs, which is what keeps
 * a read/write stream of this mix near the HBM peak on MI355X. */
#define ZS_TILE 8192

/* Optimizer state, tiled (the layout zs_step works on): fp32
 * [n_tiles][3][ZS_TILE]; in tile i, row 0 holds the fp32 master weights,
 * row 1 the first moment m, row 2 the second moment v (CS336 notes, "Core
 * concepts": fp32 master plus two fp32 Adam moments per parameter; "Code
 * example: ZeRO-1": this state lives only on the owning rank).  Padding
 * positions of a tile are never read or written by the step.  Use
 * zs_state_pack / zs_state_unpack to convert from / to three plain
 * [shard_numel] arrays (set-up, checkpoints). */

/* Gradient layouts: the W source ranks' bf16 slices of this rank's shard,
 * i.e. what the reduce-scatter delivers before it reduces (CS336 notes,
 * "Code example: ZeRO-1"). */
#define ZS_GRADS_SLICES 0  /* [W][grad_stride]: element i of the shard from
                              source rank s at s*grad_stride + i */
#define ZS_GRADS_TILED  1  /* [n_tiles][W][ZS_TILE]: position j of tile i
                              from source rank s at (i*W + s)*ZS_TILE + j */

/* ---- device calls -------------------------------------------------------- */

/* One optimizer step over the whole shard of `layout`'s rank: one rank's
 * ZeRO-1/2 step (CS336 lecture 8 notes, "Code example: ZeRO-1": the
 * reduce-scatter leaves each rank the summed gradient of its own slice, the
 * rank updates only that slice with its own fp32 optimizer state, and the
 * all-gather concatenates the updated slices; "Core concepts": bf16
 * parameter and gradient, fp32 master and two fp32 Adam moments; the
 * optimizer is AdamW, DDP-to-ZeRO blog section 3.3).  On one GPU the W
 * slices are resident, the sum over them is the local arithmetic of the
 * reduce-scatter, and full_flat is this rank's part of the all-gather.
 *
 * grads, grad_layout, grad_stride: the W gradient slices in one of the two
 *   layouts above.  ZS_GRADS_SLICES: grad_stride >= shard_numel and a
 *   multiple of 8.  ZS_GRADS_TILED: grad_stride is ignored.
 * state: the tiled fp32 state [n_tiles][3][ZS_TILE], updated in place.
 * param_shard: bf16 [shard_numel] output, or NULL.
 * full_flat: bf16 [flat_numel] all-gather buffer, or NULL; when given, the
 *   updated bf16 values are also written to this rank's positions
 *   (bucket.flat_off + rank*slice_numel + j); no other element is touched.
 *   At least one of param_shard and full_flat must be non-NULL.
 * step: the 1-based AdamW step counter t (bias corrections 1 - beta^t).
 *
 * Per element, with one fp32 rounding per operation and no contraction:
 *   g = (G0 + G1 + ... + G_{W-1}) / W          (sum in rank order)
 *   m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*(g*g)
 *   master = master*(1-lr*wd) - (lr/(1-b1^t)) * (m / (sqrt(v)/sqrt(1-b2^t)
 *            + eps))
 *   param = bf16(master), round to nearest even
 * where the constants are computed in double on the host and rounded to
 * fp32 once.  Shard padding (all-zero inputs) stays exactly zero.
 * All device pointers must be 16-byte aligned (ZS_EALIGN otherwise);
 * ZS_EINVAL for an unknown grad_layout.
 *
 * Launches: at W = 1, 2, 4, 8, 16, 32 or 64 the step's one-wave
 * workgroups reserve LDS they do not use, so that only a few of them share
 * a CU: 5 to 16 by W and launch size (at W = 8, 12, each holding 1/12 of
 * the CU's LDS; at W = 64, 5), which keeps fewer tiles in flight, measured
 * faster on MI355X (the workgroups of plain slices at W >= 32, of bucket
 * groups of 4096 tiles or more at W >= 32, and of every other W reserve
 * none).  Kernels of other streams running at the same time share the
 * CU's LDS with them.  The same holds for zs_step_plain, zs_bucket_step,
 * zs_buckets_step and zs_step_bf16. */
int zs_step(const zs_layout* layout, const uint16_t* grads,
            int32_t grad_layout, int64_t grad_stride, float* state,
            uint16_t* param_shard, uint16_t* full_flat, const zs_adamw* hp,
            int64_t step, void* hip_stream);

/* Turn the step launches' LDS reservation (the residency cap described at
 * zs_step) on (on != 0, the default) or off for the whole process; returns
 * the previous setting (1 or 0).  Off, the step's workgroups reserve no
 * LDS and fill the CUs as far as their registers allow.  Measured on
 * MI355X the cap pays alone (the 8B-shaped W = 8 step 6.2 against 6.5 ms)
 * and beside bf16 GEMMs on another stream (10 steps and 55 8192^3 GEMMs
 * together 104.0 against 106.4-107.0 ms); the switch is for callers who
 * measure their own mix of concurrent kernels.  Applies to every step
 * entry point, for launches issued after the call; results are the same
 * bits either way.  No device call, no error. */
int32_t zs_set_residency_cap(int32_t on);

/* zs_step on three plain fp32 arrays instead of the tiled state: master, m
 * and v are [shard_numel] each, element i the shard's element i (padding
 * included), updated in place; everything else as zs_step, with the same
 * arithmetic and the same results bit for bit.  For callers that keep the
 * optimizer state as plain arrays; the tiled state of zs_step reaches a
 * higher bandwidth on MI355X (its three rows of a tile are adjacent), and
 * zs_state_pack / zs_state_unpack convert between the two.  Errors as
 * zs_step; ZS_EINVAL when master, m or v is NULL, ZS_EALIGN when one is not
 * 16-byte aligned. */
int zs_step_plain(const zs_layout* layout, const uint16_t* grads,
                  int32_t grad_layout, int64_t grad_stride, float* master,
                  float* m, float* v, uint16_t* param_shard,
                  uint16_t* full_flat, const zs_adamw* hp, int64_t step,
                  void* hip_stream);

/* The same step over one bucket's part of the shard, for the ZeRO-2
 * streaming mode in which buckets arrive one by one (podcast summary, "Data
 * parallelism": a bucket's collective starts as soon as backward fills it;
 * "ZeRO optimizer": ZeRO-2 drops the gradients it does not own once they are
 * reduced).
 *
 * grads: bucket bucket_id's W slices only (a staging buffer):
 *   ZS_GRADS_SLICES [W][grad_stride], grad_stride >= slice_numel and a
 *   multiple of 8; ZS_GRADS_TILED [tiles_b][W][ZS_TILE] with
 *   tiles_b = ceil(slice_numel / ZS_TILE).
 * state, param_shard: the SHARD base pointers (the call finds the bucket's
 *   tiles and elements itself); full_flat: as in zs_step.
 * Buckets may be processed in any order, on any stream; the result equals
 * zs_step bit for bit once every bucket has been stepped once. */
int zs_bucket_step(const zs_layout* layout, int32_t bucket_id,
                   const uint16_t* grads, int32_t grad_layout,
                   int64_t grad_stride, float* state, uint16_t* param_shard,
                   uint16_t* full_flat, const zs_adamw* hp, int64_t step,
                   void* hip_stream);

/* Up to ZS_MAX_GROUP buckets in one launch: the bucket steps of the
 * streaming mode, batched when several buckets have landed, so that launch
 * and synchronisation costs are paid once per group.  Member i is bucket
 * bucket_ids[i] (all distinct) with its own staging buffer grads[i], laid
 * out as zs_bucket_step takes it; bucket_ids and grads are HOST arrays of
 * count entries, read during the call.  The result equals count
 * zs_bucket_step calls.  Errors: ZS_EINVAL for count outside
 * [1, ZS_MAX_GROUP], a repeated bucket or NULL arrays; otherwise as
 * zs_bucket_step, checked per member. */
#define ZS_MAX_GROUP 16
int zs_buckets_step(const zs_layout* layout, int32_t count,
                    const int32_t* bucket_ids, const uint16_t* const* grads,
                    int32_t grad_layout, int64_t grad_stride, float* state,
                    uint16_t* param_shard, uint16_t* full_flat,
                    const zs_adamw* hp, int64_t step, void* hip_stream);

/* Plain [shard_numel] fp32 master / m / v -> tiled state [n_tiles][3]
 * [ZS_TILE].  m or v may be NULL: that row is set to zero (a fresh
 * optimizer).  Padding positions of the tiles are set to zero.  master must
 * not be NULL. */
int zs_state_pack(const zs_layout* layout, const float* master,
                  const float* m, const float* v, float* state,
                  void* hip_stream);

/* Tiled state -> plain [shard_numel] arrays; NULL outputs are skipped. */
int zs_state_unpack(const zs_layout* layout, const float* state,
                    float* master, float* m, float* v, void* hip_stream);

/* ---- gradient accumulation -------------------------------------------------
 *
 * The step before the path: the global batch is split into k micro-batches
 * whose gradients are added up one after another before one optimizer step
 * (podcast summary, "Motivation" and the glossary; DDP-to-ZeRO blog 3.3,
 * gradient_accumulation_steps).  Per element, over the bf16 gradients
 * g_0 .. g_{k-1} of the k micro-batches, in order:
 *   ZS_ACC_FIRST  acc = f32(g_0)
 *   ZS_ACC_ADD    acc = acc + f32(g_j)            (j = 1 .. k-2)
 *   ZS_ACC_LAST   out = bf16((acc + f32(g_{k-1})) / k), nearest even
 * so out is the bf16 mean of the micro-batch gradients, summed in fp32 in
 * order: the local gradient bucket the reduce-scatter sends.  acc: fp32
 * [n] accumulator (not written by ZS_ACC_LAST); grad: bf16 [n]; out: bf16
 * [n] (ZS_ACC_LAST only, may alias grad).  n: a multiple of 4; acc
 * 16-byte aligned, grad and out 8-byte aligned; k >= 2 for ZS_ACC_LAST.
 * Errors: ZS_EINVAL (mode, pointers, k), ZS_EALIGN (alignment, n),
 * ZS_ERANGE (n above 2^34 - 2^8, more than one launch covers). */
#define ZS_ACC_FIRST 0
#define ZS_ACC_ADD   1
#define ZS_ACC_LAST  2
int zs_accumulate(int32_t mode, float* acc, const uint16_t* grad,
                  uint16_t* out, int64_t n, int32_t k, void* hip_stream);

/* ---- pure-bf16 variant ----------------------------------------------------
 *
 * Training in pure bf16 keeps 12 bytes per parameter: the bf16 parameter,
 * the bf16 gradient and two fp32 Adam moments, with no fp32 master copy
 * (CS336 notes, "Core concepts", and the fit table of "Code example:
 * FSDP", both at 12 bytes per parameter).  The optimizer state is then
 * tiled as fp32 [n_tiles][2][ZS_TILE]: row 0 = m, row 1 = v. */

/* One pure-bf16 step over the whole shard: the same reduction and AdamW
 * statements as zs_step, with the parameter read from its bf16 value and
 * the result rounded back to bf16 (nearest even) in place, so updates under
 * half a bf16 ulp are lost.  params: the bf16 parameters, read and written
 * at this rank's positions: params_flat = 0: the bf16 shard [shard_numel];
 * params_flat = 1: the flat bf16 buffer [flat_numel] (bucket.flat_off +
 * rank*slice_numel + j), i.e. the all-gather buffer updated in place.
 * grads, grad_layout, grad_stride, hp, step: as zs_step.  2W + 20 bytes per
 * element.  Errors as zs_step; ZS_EINVAL for params_flat not 0 or 1. */
int zs_step_bf16(const zs_layout* layout, const uint16_t* grads,
                 int32_t grad_layout, int64_t grad_stride, float* state_mv,
                 uint16_t* params, int32_t params_flat, const zs_adamw* hp,
                 int64_t step, void* hip_stream);

/* Plain fp32 m / v [shard_numel] -> tiled [n_tiles][2][ZS_TILE] (NULL
 * rows are set to zero; padding positions to zero), and back (NULL outputs
 * skipped). */
int zs_state_mv_pack(const zs_layout* layout, const float* m, const float* v,
                     float* state_mv, void* hip_stream);
int zs_state_mv_unpack(const zs_layout* layout, const float* state_mv,
                       float* m, float* v, void* hip_stream);

/* Gradient slices [W][stride] -> tiled [tiles][W][ZS_TILE]; padding
 * positions of the tiles are set to zero.  bucket_id < 0: the whole shard
 * (stride >= shard_numel, output n_tiles tiles); otherwise bucket
 * bucket_id's slices (stride >= its slice_numel, output tiles_b tiles),
 * the staging form zs_bucket_step takes.  stride: a multiple of 8. */
int zs_grads_tile(const zs_layout* layout, int32_t bucket_id,
                  const uint16_t* slices, int64_t stride, uint16_t* tiled,
                  void* hip_stream);

/* ZeRO-3 / FSDP parameter gather (podcast summary, "ZeRO optimizer": a
 * layer's full weight is all-gathered from the shards right before it is
 * used, the next layer's gather overlaps the current layer's compute, and
 * the full weight is dropped afterwards; CS336 notes, "Code example: FSDP").
 *
 * Writes flat positions [flat_lo, flat_hi) of the bf16 parameter buffer to
 * out[0 .. flat_hi - flat_lo), pulling each position from the rank that
 * owns it: shards is a HOST array of W device pointers, shards[r] = rank
 * r's bf16 shard [shard_numel] (as zs_step writes it to param_shard; on one
 * GPU the ranks' shards are W resident buffers).  Use a tensor's flat
 * offset and numel (zs_layout_tensor_offsets) to gather one tensor or a
 * run of tensors (a layer); padding positions are copied like the rest.
 * Any rank's layout works: the bucket table is the same for every rank.
 *
 * flat_lo must be a multiple of 8 (tensor starts are); flat_hi is free.
 * Errors: ZS_EINVAL for NULL pointers or W above ZS_GATHER_MAX_WORLD;
 * ZS_ERANGE for a range outside [0, flat_numel]; ZS_EALIGN for a pointer
 * not 16-byte aligned or a misaligned flat_lo.  An empty range is a no-op. */
#define ZS_GATHER_MAX_WORLD 64
int zs_gather(const zs_layout* layout, const uint16_t* const* shards,
              int64_t flat_lo, int64_t flat_hi, uint16_t* out,
              void* hip_stream);

/* Local part of the all-gather (CS336 notes, "Code example: ZeRO-1": the
 * all-gather concatenates the updated slices in rank order; "Code example:
 * FSDP": per-layer weights are views of the gathered parameters).
 *
 * param_shard: bf16 [shard_numel] input.
 * full_flat: bf16 [flat_numel] or NULL: this rank's slice of every bucket
 *   is written at bucket.flat_off + rank*slice_numel.
 * dev_chunks / n_chunks / dev_tensor_ptrs, all or none: a DEVICE copy of
 *   the layout's chunk table (n_chunks entries, as zs_layout_chunks writes
 *   it) and a DEVICE array of per-tensor bf16 base pointers indexed by
 *   tensor_id; every chunk's elements are written to its tensor.  Tensor
 *   pointers need only 2-byte alignment (16-byte aligned ones go faster).
 * At least one destination must be given. */
int zs_pack(const zs_layout* layout, const uint16_t* param_shard,
            uint16_t* full_flat, const zs_chunk* dev_chunks,
            int32_t n_chunks, uint16_t* const* dev_tensor_ptrs,
            void* hip_stream);

/* zs_pack for callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * flat and per-tensor writes, but the chunk table and the tensor pointer
 * array are staged by the library in a static device array of its own
 * (ZS_PACK_NOALLOC_MAX_CHUNKS 32-byte chunk records plus
 * ZS_PACK_NOALLOC_MAX_TENSORS pointers, 1.25 MiB, held on every device the
 * library runs on until the process ends).  It calls no hipMalloc, hipFree
 * or other allocating routine.
 *
 * param_shard, full_flat: as zs_pack.
 * tensor_ptrs / n_tensors: a HOST array of the layout's n_tensors per-tensor
 *   bf16 base pointers (device memory) indexed by tensor_id, or NULL for the
 *   flat output alone.  Every tensor with a chunk in this rank's shard needs
 *   a non-NULL pointer.  The array is copied on the stream; from pageable
 *   host memory that copy completes before the call returns, from pinned
 *   host memory it runs later, so keep a pinned array unchanged until the
 *   stream has passed the call.
 * hip_stream must belong to the current device.
 * Under stream capture the flat output alone records kernel launches only
 * (a test replays it in a graph); with tensor_ptrs the two table copies are
 * recorded as copies from the host arrays (the layout's chunk table and
 * tensor_ptrs), which then must stay valid and unchanged for as long as the
 * graph can run (that case is not tested).
 * Every call on one device shares the staging and overwrites it: calls
 * whose work can overlap on one device (on streams with no order between
 * them, or from several host threads at once) race.  Calls on one stream
 * are ordered.
 * Errors: ZS_ERANGE for a layout with more than ZS_PACK_NOALLOC_MAX_CHUNKS
 * chunks or ZS_PACK_NOALLOC_MAX_TENSORS tensors (checked before anything
 * else, nothing written); ZS_EINVAL (NULL layout or destinations, n_tensors
 * other than the layout's, a NULL pointer for a tensor the shard writes, a
 * stream of another device); ZS_EALIGN as zs_pack; ZS_EDEVICE. */
#define ZS_PACK_NOALLOC_MAX_CHUNKS 32768
#define ZS_PACK_NOALLOC_MAX_TENSORS 32768
int zs_pack_noalloc(const zs_layout* layout, const uint16_t* param_shard,
                    uint16_t* full_flat, uint16_t* const* tensor_ptrs,
                    int32_t n_tensors, void* hip_stream);

/* ---- ZeRO-3 / FSDP prefetch -----------------------------------------------
 *
 * Schedules the per-unit parameter gathers of ZeRO-3 / FSDP: a unit's full
 * weights are gathered right before it runs, the next unit's gather
 * overlaps the current unit's compute, and a unit's buffer is reused once
 * its compute is done (podcast summary, "ZeRO optimizer"; CS336 lecture 8
 * notes, "Code example: FSDP").  A host object on caller streams; it
 * allocates no device memory (only HIP events).
 *
 * zs_prefetch_create: shards[world] (device, read through zs_gather; the
 * array is copied), a ring of n_buffers caller-owned device unit buffers
 * (1..64, 16-byte aligned) of buffer_elems bf16 elements each, and the
 * gather stream.  The layout and the shards must outlive the object.
 * zs_prefetch_issue: gathers flat range [flat_lo, flat_hi) (as zs_gather)
 * into the next buffer of the ring on the gather stream, after the compute
 * that last released that buffer; *slot receives the buffer index.
 * zs_prefetch_acquire: makes compute_stream wait for that gather; *buffer
 * (may be NULL) receives the buffer's address.
 * zs_prefetch_release: compute_stream's use of the buffer ends here (an
 * event on it), so a later issue may overwrite the buffer.
 * A buffer goes issue -> acquire -> release -> issue ...; calls out of
 * that order fail with ZS_EINVAL (the next buffer is not released yet, or
 * the slot is not issued / acquired).  Errors also: ZS_ERANGE (range
 * outside [0, flat_numel] or longer than buffer_elems, slot index), those
 * of zs_gather, ZS_EDEVICE. */
typedef struct zs_prefetch zs_prefetch;
int zs_prefetch_create(const zs_layout* layout, const uint16_t* const* shards,
                       uint16_t* const* buffers, int32_t n_buffers,
                       int64_t buffer_elems, void* gather_stream,
                       zs_prefetch** out);
int zs_prefetch_issue(zs_prefetch* prefetch, int64_t flat_lo,
                      int64_t flat_hi, int32_t* slot);
int zs_prefetch_acquire(zs_prefetch* prefetch, int32_t slot,
                        void* compute_stream, uint16_t** buffer);
int zs_prefetch_release(zs_prefetch* prefetch, int32_t slot,
                        void* compute_stream);
void zs_prefetch_free(zs_prefetch* prefetch);

/* ---- ZeRO-2 streaming engine ----------------------------------------------
 *
 * Steps each bucket as soon as its gradients have arrived, while later
 * buckets are still being produced (podcast summary, "Data parallelism" and
 * "ZeRO optimizer": per-bucket reduce-scatter overlapped with backward;
 * DDP-to-ZeRO blog 3.3: overlap_comm).  A host object that schedules work
 * on caller streams; it allocates no device memory (only HIP events).
 *
 * zs_stream_create: `slots` is a ring of n_slots caller-owned device staging
 * buffers (n_slots >= group, 16-byte aligned) of slot_elems bf16 elements
 * each, at least the tiled size of every bucket (ceil(slice_numel /
 * ZS_TILE) * world * ZS_TILE); 2 * group slots let a group's copies run
 * while the previous group steps.  upload_stream carries the copies;
 * step_streams (1..8 of them, an array read during the call) take the
 * group launches in turn.  group: buckets per zs_buckets_step launch,
 * 1..ZS_MAX_GROUP.  The layout must outlive the engine.
 * zs_stream_step_begin: opens one optimizer step t (>= 1) on the tiled
 * state and the outputs (param_shard and/or full_flat, as zs_step).
 * zs_stream_arrive: bucket bucket_id's gradients have arrived at src, in
 * the tiled staging form of zs_bucket_step ([tiles][world][ZS_TILE] bf16,
 * as zs_grads_tile writes it for that bucket), in device memory or in
 * pinned host memory.  The engine copies them into the next slot on the
 * upload stream (after the step that last read the slot), and when `group`
 * buckets are pending it launches zs_buckets_step on the next step stream,
 * ordered after the copies.  src must stay valid until the copy has run.
 * Each bucket arrives at most once per step, in any order.
 * zs_stream_step_end: steps the pending partial group and closes the step.
 * Returns the number of buckets stepped in the step (>= 0) or an error.
 * The work is then queued on the caller's streams; synchronise them (or
 * wait on an event recorded on each step stream) before reading results.
 * Steps may be queued back to back with no host synchronisation: each
 * zs_stream_step_begin after the first orders every step stream after the
 * work already queued on the others, so a bucket's launch in step t+1 runs
 * after its launch in step t whichever step streams they use.
 * Errors: ZS_EINVAL (NULL arguments, counts, a step not open or already
 * open, a bucket arriving twice), ZS_EALIGN, ZS_ERANGE (bucket id, slot too
 * small), ZS_EDEVICE (a HIP call failed), and those of zs_buckets_step.
 * An argument error has no effect and the step stays usable.  A failed
 * copy or launch abandons the step: its pending group is dropped, later
 * arrivals are refused, and zs_stream_step_end closes it and returns
 * ZS_EINVAL; the step's results are then undefined.  Abandoning waits on
 * the host for the copies of the dropped group.  One host thread at a time
 * per engine. */
typedef struct zs_stream zs_stream;
int zs_stream_create(const zs_layout* layout, int32_t group,
                     uint16_t* const* slots, int32_t n_slots,
                     int64_t slot_elems, void* upload_stream,
                     void* const* step_streams, int32_t n_step_streams,
                     zs_stream** out);
/* The same engine with several upload streams (an array of
 * n_upload_streams, 1..8, read during the call): arrival i is copied on
 * upload stream i mod n_upload_streams, for hosts where one stream's copies
 * do not fill the host link; each group launch waits for the copies of
 * its buckets on every upload stream they used.  zs_stream_create is this
 * call with one upload stream.  Errors as zs_stream_create, and ZS_EINVAL
 * for n_upload_streams outside [1, 8] or a NULL array. */
int zs_stream_create_multi(const zs_layout* layout, int32_t group,
                           uint16_t* const* slots, int32_t n_slots,
                           int64_t slot_elems, void* const* upload_streams,
                           int32_t n_upload_streams,
                           void* const* step_streams, int32_t n_step_streams,
                           zs_stream** out);
int zs_stream_step_begin(zs_stream* stream, float* state,
                         uint16_t* param_shard, uint16_t* full_flat,
                         const zs_adamw* hp, int64_t step);
int zs_stream_arrive(zs_stream* stream, int32_t bucket_id,
                     const uint16_t* src);
int zs_stream_step_end(zs_stream* stream);
void zs_stream_free(zs_stream* stream);

/* ---- checkpoint and resume ------------------------------------------------
 *
 * A rank's optimizer state means something only together with the layout
 * that placed it: which tensors, in which order, cut into which buckets,
 * and which rank's slices.  A checkpoint restored under another layout
 * pairs moments and master weights with the wrong parameters, and nothing
 * in the numbers shows it (the DDP-to-ZeRO blog, section 3.3, warns that a
 * ZeRO checkpoint saved without the right gathering step is unusable).  A
 * checkpoint therefore carries the layout's fingerprint, and loading refuses
 * any other layout. */

/* 64-bit FNV-1a (offset basis 0xcbf29ce484222325, prime 0x100000001b3) over
 * the bytes of these little-endian int64 values, in order: the mode (0 flat,
 * 1 whole-tensor), world, rank, the alignment in elements, the full bucket
 * size in elements (0 in the whole-tensor mode), the tensor count, then every
 * tensor's numel.  Two layouts with equal fingerprints place every element
 * alike. */
int zs_layout_fingerprint(const zs_layout* layout, uint64_t* out);

/* Write this rank's tiled optimizer state and the step counter to `path`.
 *
 * state: rows = 3, the [n_tiles][3][ZS_TILE] state of zs_step (master, m,
 *   v); rows = 2, the [n_tiles][2][ZS_TILE] state of zs_step_bf16 (m, v).
 * step: the counter t of the last completed step (>= 0).
 * Synchronises hip_stream first (the state must be final), then copies the
 * state to the file through two pinned host staging buffers of 64 MiB
 * (allocated for the call), overlapping the device copies with the file
 * writes.  The file is written as path + ".tmp", flushed to disk and then
 * renamed over `path`, so an interrupted save leaves an earlier checkpoint
 * at `path` intact.
 * Format (little-endian): a 64-byte header {char magic[8] = "ZSCKPT01";
 * uint32 version = 1; uint32 rows; uint64 fingerprint; int64 step;
 * int64 n_tiles; int64 shard_numel; int32 world; int32 rank; uint64 payload
 * bytes}, the payload (the tiled state as it sits in device memory), then a
 * uint64 checksum of the payload: h = 0xcbf29ce484222325, and for each
 * little-endian 64-bit word w of it, h = (h ^ w) * 0x100000001b3 (mod 2^64).
 * Errors: ZS_EINVAL (NULL layout, path or state, rows not 2 or 3, step < 0),
 * ZS_EALIGN, ZS_EIO, ZS_ENOMEM, ZS_EDEVICE. */
int zs_checkpoint_save(const zs_layout* layout, const char* path,
                       const float* state, int32_t rows, int64_t step,
                       void* hip_stream);

/* Restore a checkpoint written by zs_checkpoint_save into `state` (tiled,
 * `rows` rows, device memory of the layout's size) and its counter into
 * *step.  Before any device access it checks the header: ZS_EIO for a file
 * that cannot be read or is not a checkpoint, ZS_EMISMATCH for one written
 * for another layout (fingerprint, world, rank, sizes) or another row
 * count; the state is then untouched.  The payload is copied through pinned
 * staging on hip_stream and the call returns when the copies are done; the
 * checksum is checked as the payload streams in, so a truncated or corrupt
 * payload returns ZS_EIO after the state has been overwritten (restore
 * another checkpoint).  Errors also: ZS_EINVAL (NULLs, rows), ZS_EALIGN,
 * ZS_ENOMEM, ZS_EDEVICE. */
int zs_checkpoint_load(const zs_layout* layout, const char* path,
                       float* state, int32_t rows, int64_t* step,
                       void* hip_stream);

/* ---- errors --------------------------------------------------------------- */

/* Static text of a ZS_E* code. */
const char* zs_strerror(int code);

/* Text describing the last failure on the calling thread ("" if none). */
const char* zs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZS_H */
