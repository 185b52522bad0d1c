/*
 * zds.h - C ABI of the ZeRO-sharded mixed-precision optimizer-step library
 * for AMD Instinct MI355X (gfx950).
 *
 * One data-parallel rank's share of the ZeRO optimizer step, on the rank's
 * contiguous shard of the flat parameter buffer:
 *
 *   per micro-batch   zds_grad_accumulate     flatten / accumulate grads
 *   per step          zds_overflow_and_norm   inf/NaN flag, global L2 norm, clip
 *                     zds_adam_step           fused AdamW + unscale/clip + cast
 *                     zds_loss_scaler_update  dynamic loss-scale state machine
 *
 * Pages the operations are taken from (cited by title and section):
 *   [algomooc] algomooc.com interview answer on the DeepSpeed framework
 *   [aidhplus] aidhplus.com "DeepSpeed" overview
 *   [csdn]     devpress.csdn.net DeepSpeed distributed-training tutorial
 *   [aiqz]     aiqz.cc "DeepSpeed ZeRO引擎深入"
 *   [ch01]     jwzheng96.github.io llm-train-tutorials, DeepSpeed chapter 1
 * The training loop of [csdn] §3.3 replaces loss.backward() by
 * engine.backward(loss) and optimizer.step() by engine.step(); here
 * engine.backward's gradient handling is zds_grad_accumulate and
 * engine.step is the other three calls, in the order listed above, on one
 * stream.
 *
 * Conventions for every function:
 *  - Plain C types only. Pointers documented as "device" are HIP device
 *    pointers the caller allocated and owns; the library never frees them.
 *    "host" pointers are read (or written) before the call returns.
 *  - `stream` is a hipStream_t (NULL selects the null stream). Hot calls only
 *    enqueue work on it and never synchronise the host; the caller keeps the
 *    buffers alive until the stream has run the work.
 *  - Arguments are checked before anything is launched. On failure nothing is
 *    enqueued, a status other than ZDS_OK is returned and zds_last_error()
 *    holds a message (thread-local, valid until the next call on that thread).
 *  - Zero-length inputs return ZDS_OK and launch nothing, except
 *    zds_overflow_and_norm, which still writes the scalars of an empty shard.
 *  - No C++ exception crosses this interface.
 */
#ifndef ZDS_H
#define ZDS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZDS_ABI_VERSION 3

typedef enum zds_status {
  ZDS_OK = 0,
  ZDS_EINVAL = 1, /* bad argument: null pointer, bad enum, size, range */
  ZDS_EALIGN = 2, /* a pointer is not aligned to its element size */
  ZDS_ENOMEM = 3, /* the library could not allocate its own memory */
  ZDS_EHIP = 4,   /* a HIP runtime call or kernel launch failed */
  ZDS_EIO = 5     /* a file could not be opened, read or written, or is not a
                     valid, intact checkpoint of this library */
} zds_status;

/* The *_RANGE_ enumerators of the enums below are not valid arguments: they
 * make every int32 value a value of the type, so that a call with any other
 * integer is well defined and rejected with ZDS_EINVAL. */
typedef enum zds_dtype {
  ZDS_FP16 = 0,
  ZDS_BF16 = 1,
  ZDS_FP32 = 2,
  ZDS_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  ZDS_DTYPE_RANGE_MAX_ = 2147483647
} zds_dtype;

typedef enum zds_accum_mode {
  ZDS_COPY = 0,       /* dst[j]  = src[j]          16-bit -> same 16-bit type */
  ZDS_OVERWRITE = 1,  /* dst[j]  = fp32(src[j])    first micro-batch          */
  ZDS_ACCUMULATE = 2, /* dst[j] += fp32(src[j])    later micro-batches        */
  ZDS_ACCUM_MODE_RANGE_MIN_ = -2147483647 - 1,
  ZDS_ACCUM_MODE_RANGE_MAX_ = 2147483647
} zds_accum_mode;

/* AdamW hyperparameters ([csdn] §3.2 optimizer block: lr, betas, eps,
 * weight_decay). Used as fp32 values. */
typedef struct zds_adamw_hparams {
  float lr;
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
} zds_adamw_hparams;

/* Loss-scaler configuration ([csdn] §3.2 fp16 block: loss_scale 0 selects the
 * dynamic scaler; loss_scale_window, initial_scale_power, hysteresis,
 * min_loss_scale). With dynamic == 0 the scale stays at static_scale (the
 * bf16 case). */
typedef struct zds_scaler_config {
  int32_t dynamic;
  int32_t initial_scale_power; /* initial scale = 2^power (dynamic)        */
  int32_t window;              /* clean steps before the scale doubles     */
  int32_t hysteresis;          /* overflows in a row before it halves (>=1) */
  float min_scale;
  float static_scale;
} zds_scaler_config;

/* Device-resident step state, 64 bytes. Written only by
 * zds_step_state_init / zds_loss_scaler_update (or their host twins). */
typedef struct zds_step_state {
  float scale;            /* loss scale S in force for the next step        */
  int32_t good_steps;     /* clean steps since the scale last changed       */
  int32_t hyst_left;      /* overflows still tolerated before a halving     */
  int32_t window;
  int32_t hysteresis;
  float min_scale;
  int32_t dynamic;
  uint32_t last_skip;     /* 1 if the last step was skipped (overflow)      */
  int64_t t;              /* Adam steps applied                             */
  double beta1_pow;       /* beta1^t (float64 running product)              */
  double beta2_pow;       /* beta2^t                                        */
  uint32_t steps_seen;    /* steps taken, skipped ones included             */
  uint32_t steps_skipped;
} zds_step_state;

/* Device-resident per-step scalars, 64 bytes. The first 32 bytes are written
 * by zds_overflow_and_norm; zds_adam_step fills the step constants of its
 * update (from its hyperparameters and the step state) before its main
 * kernel runs; zds_loss_scaler_update reads the overflow flag. */
typedef struct zds_step_scalars {
  uint32_t overflow;   /* 1 if any gradient element is inf or NaN           */
  int32_t accum_steps; /* K used for the mean over micro-batches            */
  double sumsq;        /* sum of x^2 over the raw (scaled, summed) grads    */
  float norm;          /* sqrt(sumsq) / (S * K), before clipping            */
  float clip_coef;     /* max_norm / (norm + 1e-6) if norm > max_norm, else 1 */
  float grad_scale;    /* clip_coef / (S * K), the factor Adam applies      */
  float scale_used;    /* S read from the step state                        */
  /* written by zds_adam_step: its step constants and the fp32 hyperparameters
   * it applies (the update kernel reads all of its scalars from here) */
  double inv_bc2_sqrt; /* 1 / bc2_sqrt in float64 (correctly rounded)       */
  float step_size;     /* lr / (1 - beta1^t)                                */
  float bc2_sqrt;      /* sqrt(1 - beta2^t)                                 */
  float decay;         /* 1 - lr * weight_decay                             */
  float beta1;         /* the update forms 1 - beta1 and 1 - beta2 in fp32  */
  float beta2;
  float eps;
} zds_step_scalars;

/* ---------------------------------------------------------------------------
 * Host-only geometry (no GPU needed).
 * Flat layout: tensor i starts at the next multiple of flat_align elements
 * after tensor i-1 ends; the total is padded to flat_align too ([csdn] §3.2
 * contiguous_gradients; [aiqz] 通信优化, grads packed into buckets).
 * ------------------------------------------------------------------------- */

/* offsets_out (host, num_tensors entries, may be NULL) receives each tensor's
 * flat offset; *total_out the padded flat length. flat_align >= 1. */
zds_status zds_flat_layout(const int64_t *numel, int32_t num_tensors, int32_t flat_align,
                           int64_t *offsets_out, int64_t *total_out);

/* Stage-1 shard of `rank` among `world` ranks ([csdn] §2.1 and §2.4: each rank
 * keeps and updates only its part of the optimizer state): the flat buffer is
 * padded to a multiple of world * flat_align and cut into `world` equal
 * contiguous slices; [*lo, *hi) is rank's slice. */
zds_status zds_shard_range(int64_t flat_total, int32_t world, int32_t rank, int32_t flat_align,
                           int64_t *lo, int64_t *hi);

/* The pieces of tensors that lie inside flat range [lo, hi): for entry e,
 * out[4e..4e+3] = {tensor index, start inside the tensor, length, destination
 * offset relative to lo}. out (host) holds room for max_entries entries;
 * *count receives the number of entries (even when it exceeds max_entries,
 * in which case ZDS_EINVAL is returned and out holds the first max_entries). */
zds_status zds_shard_entries(const int64_t *numel, int32_t num_tensors, int32_t flat_align,
                             int64_t lo, int64_t hi, int64_t *out, int32_t max_entries,
                             int32_t *count);

/* ---------------------------------------------------------------------------
 * Gradient plan: the tensor table of one flat range, kept on the device so
 * that one launch covers all tensors ([aiqz] 通信优化: a fixed cost per call
 * dominates when there are hundreds of small grad tensors).
 * ------------------------------------------------------------------------- */

typedef struct zds_plan zds_plan;

/* Builds the plan for flat range [lo, hi) of the layout of numel[0..T) with
 * flat_align. Allocates the plan's device table and a small pinned staging
 * ring for per-call source pointers on the current device. Not called on the
 * hot path. */
zds_status zds_plan_create(zds_plan **out, const int64_t *numel, int32_t num_tensors,
                           int32_t flat_align, int64_t lo, int64_t hi);
void zds_plan_destroy(zds_plan *plan);
int32_t zds_plan_num_entries(const zds_plan *plan);
/* Entry e as {tensor, start, length, dst_offset}; see zds_shard_entries. */
zds_status zds_plan_entry(const zds_plan *plan, int32_t e, int64_t *out4);

/* Row a1. One micro-batch's grads into the rank's flat buffer, one launch.
 *   src_ptrs  host array of num_tensors device pointers; src_ptrs[t] points at
 *             element 0 of tensor t (only tensors with plan entries are read;
 *             others may be NULL). Element size alignment required.
 *   src_dtype ZDS_FP16 / ZDS_BF16 (ZDS_FP32 allowed for the fp32 modes).
 *   dst       device, hi - lo elements of dst_dtype: a 16-bit bucket of
 *             src_dtype for ZDS_COPY, an fp32 accumulator otherwise.
 *             Padding elements between tensors are never written.
 * Definition: [csdn] §2.3, micro-batch grads summed in memory before one
 * update; the fp32 add rounds to nearest even. The source pointers are
 * copied to the device through the plan's pinned staging ring (8 slots), so
 * calls can be issued back to back without waiting; a call with the same
 * pointers as the previous one reuses that upload (on another stream than
 * the previous call's, after a stream wait on it). A plan must not be used
 * from two host threads at once.
 * HIP graphs: a call on a stream under capture records only its kernel. It
 * must use the previous call's source pointers, after that eager call has
 * completed (EINVAL otherwise); the slot holding them is then kept for the
 * graph's replays and never refilled (a plan has 8 slots; the grads must
 * stay at those addresses while the graph is used). */
zds_status zds_grad_accumulate(zds_plan *plan, const void *const *src_ptrs, zds_dtype src_dtype,
                               void *dst, zds_dtype dst_dtype, zds_accum_mode mode, void *stream);

/* Rows a1 + a2 fused, for the micro-batch that completes the step's grads:
 * the same as zds_grad_accumulate followed by zds_overflow_and_norm over
 * dst (dst_dtype, hi - lo elements), except that the sum of squares is
 * formed from the values as the kernel stores them, so the flat buffer is
 * not read a second time. Padding elements of dst between tensors are not
 * visited and must be zero (as they stay when the buffer was zeroed once).
 * The sum is accumulated in float64 per block in a fixed order, then the
 * block partials in index order, so it is run-to-run identical for the plan;
 * it may differ from zds_overflow_and_norm's sum of the same data in the
 * last bits (another order). Arguments as for the two calls; ws holds at
 * least zds_plan_norm_workspace_bytes(plan) bytes. */
size_t zds_plan_norm_workspace_bytes(const zds_plan *plan);
zds_status zds_grad_accumulate_norm(zds_plan *plan, const void *const *src_ptrs, zds_dtype src_dtype,
                                    void *dst, zds_dtype dst_dtype, zds_accum_mode mode,
                                    int32_t accum_steps, float max_norm,
                                    const zds_step_state *state_dev, zds_step_scalars *out_dev,
                                    void *ws, size_t ws_bytes, void *stream);

/* Row a2. Size in bytes of the workspace zds_overflow_and_norm needs for n
 * elements: one float64 partial sum per 2048 elements and the levels that
 * fold them (about 8 bytes per 2048 elements; it stops growing where the
 * first stage's grid reaches its cap, past 2^34 elements). */
size_t zds_workspace_bytes(int64_t n);

/* Row a2. Overflow flag and global L2 norm of n grads (device, dtype), and the
 * clip/unscale factor for the step.
 *   accum_steps K >= 1: the grads are the sum of K micro-batches; the step
 *               uses their mean ([csdn] §2.3: the accumulated grad stands for
 *               the big batch's grad).
 *   max_norm    clip threshold; <= 0 disables clipping.
 *   state_dev   device, supplies the loss scale S ([csdn] §2.2 loss scaling).
 *   out_dev     device, receives zds_step_scalars.
 *   ws, ws_bytes device workspace of at least zds_workspace_bytes(n).
 * overflow = 1 iff some element is inf or NaN ([csdn] §2.2: overflow under the
 * loss scale is detected). sumsq = sum of float64(x)^2 in a fixed order
 * (run-to-run identical for the same n). norm, clip_coef and grad_scale are
 * computed in float64 and rounded once to fp32. On overflow the step is
 * skipped: norm = inf, clip_coef = 1 and grad_scale = 0. */
zds_status zds_overflow_and_norm(const void *grads, zds_dtype dtype, int64_t n,
                                 int32_t accum_steps, float max_norm,
                                 const zds_step_state *state_dev, zds_step_scalars *out_dev,
                                 void *ws, size_t ws_bytes, void *stream);

/* Row a2 for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): zds_overflow_and_norm
 * with the same kernels and results, its partial sums kept in a fixed 4 MiB
 * device array of the library instead of a caller workspace. The array
 * exists once per GPU and stays allocated until the process ends; the first
 * call on a device resolves its address there (no stream operation). Calls
 * on one GPU share it, so calls that overlap in time on one GPU (different
 * streams, or host threads) race and must not be issued; calls in order on
 * one stream are safe (nothing needs clearing between calls: every partial
 * is written before it is read). Arguments as for zds_overflow_and_norm
 * without ws / ws_bytes; n may be at most 1,073,217,536 (the largest n whose
 * partial sums fit the array; EINVAL beyond). Allocates nothing. */
zds_status zds_overflow_and_norm_noalloc(const void *grads, zds_dtype dtype, int64_t n,
                                         int32_t accum_steps, float max_norm,
                                         const zds_step_state *state_dev, zds_step_scalars *out_dev,
                                         void *stream);

/* Row a4. Fused AdamW on the fp32 master shard with unscale/clip and the cast
 * back to 16 bits ([csdn] §2.2 and [aiqz] 混合精度: the update runs on the
 * fp32 master copy; [csdn] §3.2 AdamW; [aiqz] Python 演示: the moment
 * recurrences). Per element, in fp32 with one rounding per operation:
 *   g = x * grad_scale; m = b1*m + (1-b1)*g; v = b2*v + (1-b2)*(g*g);
 *   denom = sqrt(v)/sqrt(1-b2^t) + eps; p = p*(1-lr*wd);
 *   p = p - (lr/(1-b1^t))*(m/denom); params_out = round_nearest_even(p)
 * with t = state.t + 1 and the step scalars derived in float64, each rounded
 * once to fp32. If scalars_dev->overflow is set every element is left
 * untouched (the step is skipped on the device; no host sync).
 * The step constants are derived once per call by a single-wave kernel and
 * stored in scalars_dev (inv_bc2_sqrt .. eps); the update kernel reads them
 * from there. The division sqrt(v)/sqrt(1-b2^t) is carried out
 * as float64(sqrt(v)) * inv_bc2_sqrt rounded to fp32, which is the correctly
 * rounded quotient for every input (the float64 product is within 2^-52 of
 * it, relatively, and the quotient of two fp32 numbers is never that close
 * to a point halfway between two fp32 numbers).
 *   grads       device, n elements of grad_dtype (16-bit, or the fp32 accumulator)
 *   master, exp_avg, exp_avg_sq   device fp32, n elements, updated in place
 *   params_out  device, n elements of param_dtype (FP16/BF16), write-only;
 *               NULL skips the cast.
 *   n           below 2^40 (EINVAL otherwise; tile indices are 32-bit).
 * The state is read, not advanced: zds_loss_scaler_update commits t. */
zds_status zds_adam_step(const zds_adamw_hparams *hp, const void *grads, zds_dtype grad_dtype,
                         float *master, float *exp_avg, float *exp_avg_sq, void *params_out,
                         zds_dtype param_dtype, int64_t n, zds_step_scalars *scalars_dev,
                         const zds_step_state *state_dev, void *stream);

/* Stage-2 reduce-scatter intake (a next row). Under Stage 2 the grads are
 * reduce-scattered rather than all-reduced ([aidhplus] ZeRO-2 section; [ch01]
 * §1.2 table): each rank sums the N peers' copies of its own slice. This call
 * is that sum on one rank:
 *   dst  = sum_k fp32(peer_ptrs[k][j])        (ZDS_OVERWRITE)
 *   dst += sum_k fp32(peer_ptrs[k][j])        (ZDS_ACCUMULATE)
 * for j < n, the sum formed in fp32 in peer order 0..N-1 (one round-to-
 * nearest add per peer), the previous destination added last, a 16-bit
 * destination rounded once at the end.
 *   peer_ptrs  host array of num_peers (1..16) device pointers, n fp16/bf16
 *              elements each (the slices received from the peers)
 *   dst        device, n elements of fp32 or of the peers' dtype
 * No mean is taken: to average over peers, give the step accum_steps = K * N.
 * 2N + 4 (fp32 out) bytes of HBM traffic per element, +4 when accumulating. */
zds_status zds_reduce_peer_slices(const void *const *peer_ptrs, int32_t num_peers, zds_dtype src_dtype,
                                  int64_t n, void *dst, zds_dtype dst_dtype, zds_accum_mode mode,
                                  void *stream);

/* The Stage-2 intake with the step's row a2 fused in: the same as
 * zds_reduce_peer_slices followed by zds_overflow_and_norm over dst
 * (dst_dtype, n elements), except that the sum of squares is formed from the
 * values as the kernel stores them (for a 16-bit dst, the rounded values), so
 * the shard gradient is not read a second time. The overflow flag, norm and
 * clip scalars are those row a2 defines for dst. The sum is accumulated in
 * float64 per block in a fixed order, then the block partials in index
 * order, so it is run-to-run identical for n and the pointers' alignment; it
 * may differ from zds_overflow_and_norm's sum of the same data in the last
 * bits (another order). n == 0 writes the scalars of an empty shard. Other
 * arguments as for the two calls; ws holds at least
 * zds_reduce_norm_workspace_bytes(n) bytes (8-byte aligned). */
size_t zds_reduce_norm_workspace_bytes(int64_t n);
zds_status zds_reduce_peer_slices_norm(const void *const *peer_ptrs, int32_t num_peers, zds_dtype src_dtype,
                                       int64_t n, void *dst, zds_dtype dst_dtype, zds_accum_mode mode,
                                       int32_t accum_steps, float max_norm, const zds_step_state *state_dev,
                                       zds_step_scalars *out_dev, void *ws, size_t ws_bytes, void *stream);

/* 1-bit compression with error compensation (a next row): the rank-local
 * encode / decode of a sign-compressed exchange. 1-bit Adam sends only the
 * sign of each element and compensates the compression error afterwards
 * ([csdn] §4.2 通信压缩). The page gives no more; readings: a chunk of `chunk`
 * consecutive elements (the last one may be shorter) sends one fp32 scale,
 * its root mean square, with its signs; the error is fed back, i.e. added to
 * the next input before it is encoded.
 *
 * zds_onebit_compress, all device pointers, enqueued on stream:
 *   x        n fp32 values to encode (16-byte aligned)
 *   error    n fp32, read and updated in place, or NULL (no error feedback:
 *            encode x alone). With c = x + error: bit = c >= 0 (-0 is +),
 *            s = fp32(sqrt(sum over the chunk of c^2 / its length)), squares
 *            summed in float64; the new error is c - s (bit 1) or c + s.
 *   chunk    1024, 2048, 4096, 8192 or 16384
 *   words    64 * ceil(n / 2048) uint32, 4-byte aligned: bit 4r + i of
 *            word 64u + l is element 2048u + 256r + 4l + i (r < 8, l < 64,
 *            i < 4): word l of a 2048-element unit holds the signs of the
 *            l-th quad of each of its eight 256-element groups; bits past n
 *            are 0
 *   scales   ceil(n / chunk) fp32
 * Non-finite inputs give non-finite scales (check for overflow first).
 * HBM-bound: 12 B/element + the payload (1/8 B + 4/chunk B). */
zds_status zds_onebit_compress(const float *x, float *error, int64_t n, int32_t chunk, uint32_t *words,
                               float *scales, void *stream);

/* Decode of num_peers (1..16) payloads of n elements each, all made with the
 * same chunk: dst[i] (+)= sum over peers k = 0.. in that order of
 * +-scales_k[i / chunk] (fp32, one rounding per add; with ZDS_ACCUMULATE the
 * previous dst is added last). The mean over peers is left to the caller
 * (pass K * N as accum_steps to the step). Words 4-byte aligned; dst: n
 * fp32, 16-byte aligned, not overlapping any payload.
 * Moves N/8 + 4N/chunk B of payload + 4 B (8 B accumulating) per element.
 * The first 8 peers cost a table lookup per element whatever their number;
 * each peer past 8 adds a select and an add per element. */
zds_status zds_onebit_decompress(const uint32_t *const *peer_words, const float *const *peer_scales,
                                 int32_t num_peers, int64_t n, int32_t chunk, float *dst, zds_accum_mode mode,
                                 void *stream);

/* Offloaded optimizer shard (a next row). ZeRO-Offload keeps the optimizer
 * state, and runs its update, in host memory ([aiqz] 卸载策略; [csdn] §4.3):
 * this is zds_adam_step on host buffers, bit-identical to the device kernel
 * (same constants from hp and state, same fp32 operation order, IEEE divide
 * and square root, round-to-nearest-even casts).
 *   grads, master, exp_avg, exp_avg_sq, params_out   HOST pointers, n elements
 *              (params_out may be NULL); pinned memory lets the caller overlap
 *              the grad download and param upload with the update
 *   scalars, state   HOST copies of the step scalars / state (the norm pass
 *              runs on the device; copy the 64-byte structs down first); an
 *              overflow flag skips the update
 *   num_threads      host threads (0: the CPUs of the process's affinity
 *                    mask)
 * Returns when the update is done. Host-memory bound, 28 B/param. */
zds_status zds_cpu_adam_step(const zds_adamw_hparams *hp, const void *grads, zds_dtype grad_dtype,
                             float *master, float *exp_avg, float *exp_avg_sq, void *params_out,
                             zds_dtype param_dtype, int64_t n, const zds_step_scalars *scalars,
                             const zds_step_state *state, int32_t num_threads);

/* ---------------------------------------------------------------------------
 * Sharded checkpoint / resume and consolidation (a next row). The engine saves
 * and loads per-rank shard checkpoints to resume training when the library
 * version, the topology and the configuration (world size, ZeRO stage,
 * offload, format) match; merging the shards into one full fp32 state is a
 * separate export step that resuming does not need ([algomooc] 训练与恢复边界
 * and the checkpoint paragraph of the spoken answer).
 * A rank's file holds its fp32 master / exp_avg / exp_avg_sq shard, its step
 * state, the tensor table, a 64-bit hash per section and one over the header
 * (meta, step state, section hashes); a save goes to
 * "<path>.tmp" and is renamed over <path> only once complete. The save does
 * not fsync: the rename protects <path> against a crash of the process, not
 * of the machine (a load then finds a torn file by its hashes and fails with
 * ZDS_EIO). A caller that needs the save to survive a power loss fsyncs the
 * file and its directory after the call.
 * ------------------------------------------------------------------------- */

#define ZDS_CHECKPOINT_FORMAT 2

/* Where the arrays and the step state of a save / load live. */
typedef enum zds_location {
  ZDS_ON_DEVICE = 0,
  ZDS_ON_HOST = 1,
  ZDS_LOCATION_RANGE_MIN_ = -2147483647 - 1,
  ZDS_LOCATION_RANGE_MAX_ = 2147483647
} zds_location;

/* The partition a shard belongs to. lo, hi and flat_total must be what
 * zds_flat_layout and zds_shard_range give for the tensor table, world,
 * rank and flat_align; stage (1..3) and offload (0/1) record the run's
 * configuration and must match on load. 48 bytes. */
typedef struct zds_checkpoint_meta {
  int32_t world;
  int32_t rank;
  int32_t flat_align;
  int32_t stage;
  int32_t offload;
  int32_t num_tensors;
  int64_t flat_total;
  int64_t lo, hi;
} zds_checkpoint_meta;

/* Writes rank meta->rank's shard to `path`.
 *   numel      host, meta->num_tensors entries: the tensor table
 *   master, exp_avg, exp_avg_sq   hi - lo fp32 elements each, device or host
 *              memory as `loc` says (with the state)
 *   state      the 64-byte step state (device or host as `loc` says)
 *   stream     ZDS_ON_DEVICE: the save first waits for the work already
 *              enqueued on it, so it records the state that work leaves
 * Synchronous: returns once the file is complete (written through the page
 * cache, not synced to disk). The arrays move in 32 MiB pieces on up to 8
 * host threads with their own pinned buffers and streams. EINVAL if meta
 * does not match the tensor table's partition, EIO on a file error. */
zds_status zds_checkpoint_save(const char *path, const zds_checkpoint_meta *meta, const int64_t *numel,
                               const float *master, const float *exp_avg, const float *exp_avg_sq,
                               const zds_step_state *state, zds_location loc, void *stream);

/* Reads a file's meta and step state (host; state may be NULL) and, when
 * numel_out is not NULL, up to max_tensors entries of its tensor table
 * (EINVAL when the table has more). EIO for a file that is not an intact
 * checkpoint of this format. */
zds_status zds_checkpoint_read_meta(const char *path, zds_checkpoint_meta *meta, zds_step_state *state,
                                    int64_t *numel_out, int32_t max_tensors);

/* Restores rank expect->rank's shard from `path` into master / exp_avg /
 * exp_avg_sq and the step state, in device or host memory as `loc` says. The
 * file's meta must equal *expect field by field and its tensor table must
 * equal numel (EINVAL otherwise: a different world size, rank, stage,
 * offload setting or model); the header and every section are checked
 * against their hashes (EIO on a mismatch). The arrays are filled piece by
 * piece as the file is read and its hashes are only known at the end, so
 * after EIO from a section hash they hold an undefined mix of their previous
 * contents and the file's; the step state is written only after every check
 * has passed. Synchronous;
 * the transfer runs on up to 8 host threads with their own pinned buffers
 * and streams. */
zds_status zds_checkpoint_load(const char *path, const zds_checkpoint_meta *expect, const int64_t *numel,
                               float *master, float *exp_avg, float *exp_avg_sq, zds_step_state *state,
                               zds_location loc, void *stream);

/* Consolidation: the world's num_files shard files (any order; ranks 0 ..
 * world-1 of one run at one step) merged into full per-tensor fp32 state:
 * out (host, out_numel = sum of the tensor table) receives the tensors one
 * after another, unpadded, in table order. section 0 = master weights (the
 * full fp32 state dict), 1 = exp_avg, 2 = exp_avg_sq. */
zds_status zds_consolidate_fp32(const char *const *paths, int32_t num_files, int32_t section, float *out,
                                int64_t out_numel);

/* Row a3. Initialise the device step state from cfg with Adam step count t0
 * and powers beta1^t0, beta2^t0 (1, 1 for a fresh optimizer). */
zds_status zds_step_state_init(zds_step_state *state_dev, const zds_scaler_config *cfg, int64_t t0,
                               double beta1_pow0, double beta2_pow0, void *stream);

/* Row a3. Advance the state after a step ([csdn] §2.2: lower the scale on
 * overflow, raise it once stable; [csdn] §3.2 fp16 fields; [aidhplus] dynamic
 * loss scaling). Dynamic mode, with the flag from scalars_dev:
 *   overflow: skip; good_steps = 0; if hyst_left <= 1 the scale halves (not
 *             below min_scale) and hyst_left = hysteresis, else hyst_left -= 1.
 *   clean:    t += 1; beta powers *= (double)beta (fp32 hp values);
 *             hyst_left = hysteresis; good_steps += 1 and when it reaches
 *             window the scale doubles and good_steps = 0.
 * Static mode: the scale never changes; an overflow still skips the step. */
zds_status zds_loss_scaler_update(zds_step_state *state_dev, const zds_step_scalars *scalars_dev,
                                  const zds_adamw_hparams *hp, void *stream);

/* Host twins of the two state functions above, on a host struct; the same
 * code as the device path. */
zds_status zds_step_state_init_host(zds_step_state *state, const zds_scaler_config *cfg,
                                    int64_t t0, double beta1_pow0, double beta2_pow0);
zds_status zds_loss_scaler_update_host(zds_step_state *state, uint32_t overflow,
                                       const zds_adamw_hparams *hp);

/* The fp32 step constants zds_adam_step derives for the step after `state`:
 * out5 (host) = {step_size, bc2_sqrt, decay, 1-beta1, 1-beta2}. Host code path
 * shared with the kernel. */
zds_status zds_adam_constants_host(const zds_adamw_hparams *hp, const zds_step_state *state,
                                   float *out5);

/* Clip arithmetic of zds_overflow_and_norm on the host: from sumsq, S, K and
 * max_norm fill out (overflow, norm, clip_coef, grad_scale, scale_used). */
zds_status zds_clip_scalars_host(double sumsq, float scale, int32_t accum_steps, float max_norm,
                                 zds_step_scalars *out);

const char *zds_last_error(void);
const char *zds_status_string(zds_status status);
int32_t zds_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZDS_H */
