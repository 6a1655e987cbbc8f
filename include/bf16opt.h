/*
 * bf16opt.h -- C ABI of the MI355X (gfx950) mixed-precision AdamW step.
 *
 * The step has three parts and runs over one ZeRO-1 shard of a flat buffer
 * that holds many tensors back to back:
 *   1. grad_global_norm: a deterministic L2 norm of the bf16 gradients and
 *      the clip scale derived from it;
 *   2. adamw_sr_step: one fused pass per element -- AdamW with lerp-form
 *      moments, bias correction, decoupled weight decay on flagged (2-D)
 *      tensors only, an fp32 master update and a bf16 write-back by
 *      stochastic rounding keyed on (global element index, seed);
 *   3. master_to_bf16_sr: the resume-time rebuild of the bf16 weights from
 *      the fp32 master with the same rounding draws.
 *
 * Pages defining each operation (title, section):
 *   "04 · 多 GPU 与混合精度" (llm.c multi-GPU and mixed precision):
 *     §2.1 precision roles, §2.2 AdamW kernel, §2.3 stochastic rounding,
 *     §3.2 ZeRO-1 sharding, §4 grad norm and clip, §5.2 bit-perfect resume.
 *   "第 13 讲：扩大 LLM——优化与并行训练": §1.7 bias correction and AdamW,
 *     §2.3 fp32 master weights.
 *   "LLM 分布式训练实战：CUDA/ROCm 多卡并行优化详解": §3.1 sharded update.
 *
 * Conventions shared by every entry point
 *   - Shards.  A table describes one rank's shard of the flat buffer, in one
 *     of two layouts.  BFO_LAYOUT_FLAT: the contiguous global range
 *     [begin, end) = [r*n/N, (r+1)*n/N) (see shard_range).  BFO_LAYOUT_PER_TENSOR:
 *     rank r's 1/N slice of every tensor, concatenated in table order (the
 *     llm.c rule that every tensor size divides by the process count).  The
 *     shard holds S elements either way; shard-local element j maps to one
 *     global index i of the flat buffer (bfo_table_runs lists the mapping).
 *   - Arrays.  master, m and v are shard-local: element j of the array
 *     belongs to shard element j; they hold S fp32 values.  params and grads
 *     (bf16 patterns, uint16_t) are addressed differently per layout: FLAT --
 *     shard-local too (element j; pass the full buffer + begin); PER_TENSOR --
 *     the full n-element buffers (element i).
 *   - Memory.  Array arguments are device pointers on the device the table
 *     was created on.  master, m and v must be 16-byte aligned; params and
 *     grads 2-byte aligned (16-byte aligned pointers take the fastest path).
 *     The arrays of one call must not overlap one another (BFO_EINVAL): the
 *     kernels read and write them as distinct buffers.  Scalars and the
 *     hyperparameter struct are host memory.  The caller owns every buffer;
 *     the library keeps no pointer after a call returns.
 *   - Asynchrony.  GPU work is queued on `stream` (a hipStream_t; NULL means
 *     the null stream) and the call returns without waiting for it.  Argument
 *     errors are reported synchronously and queue no work.  Apart from the
 *     checkpoint calls (which move state through files, and so wait for their
 *     copies and use a pinned host stage for the call's length), nothing here
 *     synchronises the host or allocates memory per call; device memory is
 *     allocated only when a table or an outlier detector is created.
 *   - Errors.  Every function returns BFO_OK (0) or a negative BFO_E* code;
 *     bfo_status_string() names it.  BFO_EHIP means a HIP runtime call
 *     failed; bfo_last_hip_error() gives its hipError_t code for the calling
 *     thread.  The library never prints and never exits.
 *   - Concurrency.  A table may be used from several threads and streams;
 *     the one shared buffer is the norm workspace a table holds for callers
 *     that pass none (see grad_global_norm).
 *
 * A step, as a ZeRO-1 rank runs it (error checks left out):
 *   bfo_table tb;  bfo_table_create(tensors, count, world, rank, &tb);   once
 *   bfo_norm_result *res;  (16-byte aligned device memory)              once
 *   void *workspace;  (bfo_norm_workspace_bytes(tb) bytes of device memory) once
 *   per step t = 1, 2, ...:
 *     grad_global_norm(tb, grads + begin, 1.0f, workspace, res, stream);
 *     adamw_sr_step(tb, params + begin, grads + begin, master, m, v, &hp,
 *                   &res->scale, NULL, t, seed_t, BFO_ROUND_SR, stream);
 *   (the all-gather of params and the reduce-scatter of grads around it are
 *   the caller's; every array here is already resident on the device.)
 */
#ifndef BF16OPT_H
#define BF16OPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    BFO_OK = 0,
    BFO_EINVAL = -1,        /* null pointer, overlapping arrays, world == 0, t == 0, unknown rounding mode */
    BFO_ENOTDIVISIBLE = -2, /* n (or, per tensor, a tensor's size) is not a multiple of world */
    BFO_ERANGE = -3,        /* rank >= world */
    BFO_EMISALIGNED = -4,   /* pointer not aligned as required (see Memory above) */
    BFO_ETABLE = -5,        /* table not contiguous from 0, or undefined flag bits set */
    BFO_EHIP = -6,          /* a HIP runtime call failed */
    BFO_EDEVICE = -7,       /* called with a different current device than the table's */
    BFO_EIO = -8,           /* a checkpoint file could not be created, written or read */
    BFO_EFORMAT = -9,       /* a checkpoint file does not match the table, or is truncated */
    BFO_ENOTFOUND = -10     /* no such checkpoint (file or DONE marker) */
};

enum { BFO_ROUND_SR = 0, BFO_ROUND_RNE = 1 };

enum { BFO_LAYOUT_FLAT = 0, BFO_LAYOUT_PER_TENSOR = 1 };

/* bfo_tensor.flags bit 0: the tensor takes weight decay.  The pages apply
 * decay to 2-D tensors (embeddings, weight matrices) and not to 1-D ones
 * (LayerNorm / RMSNorm weights, biases): "04 · 多 GPU 与混合精度" §2.2. */
#define BFO_FLAG_DECAY 1u

/* One tensor of the flat buffer: global elements [offset, offset + numel).
 * A table lists the tensors in buffer order; tensor k must start where
 * tensor k-1 ends, the first at 0; numel may be 0; `reserved` must be 0. */
typedef struct {
    uint64_t offset;
    uint64_t numel;
    uint32_t flags;
    uint32_t reserved;
} bfo_tensor;

/* AdamW hyperparameters ("04 · 多 GPU 与混合精度" §4: lr, beta1 = 0.9,
 * beta2 = 0.95, eps, weight decay; "第 13 讲" §1.7: bias correction). */
typedef struct {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;     /* used for BFO_FLAG_DECAY tensors; others use 0 */
    int32_t bias_correction;/* nonzero: divide m by 1 - beta1^t and v by 1 - beta2^t */
} bfo_adamw_hparams;

/* Output of grad_global_norm, written to device memory (16 bytes). */
typedef struct {
    double sumsq;  /* sum of squares of the shard's widened bf16 grads, binary64 */
    float norm;    /* (float)sqrt(sumsq) */
    float scale;   /* max_norm / norm if norm > max_norm, else 1 */
} bfo_norm_result;

/* Opaque handle: a validated tensor table intersected with one shard, plus
 * the small device-side lookup it needs (created once, reused every step). */
typedef struct bfo_table_s *bfo_table;

/* One run of a shard plan: shard-local elements [local, local + length) are
 * params/grads positions [addr, addr + length) and global indices
 * [global, global + length) of the flat buffer, all in one tensor-flag
 * class (flags bit 0 = decay).  addr equals local for FLAT tables and global
 * for PER_TENSOR tables.  Consecutive pieces with the same flag that continue
 * one another are merged into one run. */
typedef struct {
    uint64_t local;
    uint64_t addr;
    uint64_t global;
    uint64_t length;
    uint32_t flags;
    uint32_t reserved;
} bfo_run;

/* ZeRO-1 shard of an n-element buffer over `world` ranks
 * ("04 · 多 GPU 与混合精度" §3.2: shard = parameter count / process count,
 * which must divide exactly; "LLM 分布式训练实战" §3.1: rank r starts at
 * r * (n / world)).  Writes [*begin, *end) = [r*n/world, (r+1)*n/world).
 * Errors: BFO_EINVAL (world == 0 or null output), BFO_ERANGE (rank >= world),
 * BFO_ENOTDIVISIBLE (n % world != 0).  Host only; touches no GPU. */
int shard_range(uint64_t n, uint32_t world, uint32_t rank, uint64_t *begin, uint64_t *end);

/* Validates `tensors` (count entries, host memory, copied), takes rank
 * `rank`'s BFO_LAYOUT_FLAT shard of the buffer they describe and uploads the
 * shard plan to the current device.  Errors: as shard_range, BFO_ETABLE,
 * BFO_EINVAL (null out, or null tensors with count > 0), BFO_EHIP.  The
 * handle holds device memory until bfo_table_destroy. */
int bfo_table_create(const bfo_tensor *tensors, uint32_t count, uint32_t world, uint32_t rank,
                     bfo_table *out);

/* As bfo_table_create with an explicit layout (BFO_LAYOUT_FLAT or
 * BFO_LAYOUT_PER_TENSOR).  PER_TENSOR ("04 · 多 GPU 与混合精度" §3.2 and §6:
 * each tensor's size must divide by the process count) gives rank r
 * elements [offset + r*numel/N, offset + (r+1)*numel/N) of every tensor;
 * BFO_ENOTDIVISIBLE if any numel % world != 0.  Unknown layout: BFO_EINVAL. */
int bfo_table_create_layout(const bfo_tensor *tensors, uint32_t count, uint32_t world, uint32_t rank,
                            int layout, bfo_table *out);

/* Frees the handle and its device memory.  No call queued on the handle may
 * still be running.  NULL is accepted. */
int bfo_table_destroy(bfo_table table);

/* Buffer length n and the shard of a table: FLAT -> [begin, end); PER_TENSOR
 * -> begin = 0, end = S (the shard length). */
int bfo_table_info(bfo_table table, uint64_t *n, uint64_t *begin, uint64_t *end);

/* The table's shard plan: *count = number of runs; when out is not NULL,
 * copies them (BFO_ERANGE if capacity < *count).  Host only. */
int bfo_table_runs(bfo_table table, bfo_run *out, uint32_t capacity, uint32_t *count);

/* The shard plan bfo_table_create_layout would build, computed on the host
 * with no device and no table ("04 · 多 GPU 与混合精度" §3.2 for both layouts;
 * "LLM 分布式训练实战" §3.1 for the flat offset): the same validation and
 * status codes, *nruns = number of runs, *shard_elems (if not NULL) = S; when
 * out is not NULL, copies the runs (BFO_ERANGE if capacity < *nruns). */
int bfo_plan_runs(const bfo_tensor *tensors, uint32_t count, uint32_t world, uint32_t rank, int layout,
                  bfo_run *out, uint32_t capacity, uint32_t *nruns, uint64_t *shard_elems);

/* *bytes = the device workspace grad_global_norm needs for this table: one
 * binary64 partial per 8,192-element tile of the shard, plus one per 4,096
 * tiles above 32,768 tiles; 0 for shards of at most 8 tiles (65,536
 * elements), whose norm runs in one workgroup.  Host only. */
int bfo_norm_workspace_bytes(bfo_table table, uint64_t *bytes);

/* Deterministic global grad norm of one shard ("04 · 多 GPU 与混合精度" §4:
 * grad_norm, then grad_scale = min(1, 1/grad_norm), i.e. clip to 1.0; under
 * ZeRO-1 this is the shard's part, which ranks would add before the root).
 * grads: as in Arrays above.  out: device bfo_norm_result.  Every
 * square is formed and summed in binary64 over a fixed partition that
 * depends only on the shard length, so repeated calls give identical bits.
 * scale = max_norm / norm when norm > max_norm, else 1.0f (an infinite norm
 * gives 0, a NaN norm gives 1: non-finite grads are not sanitised, check
 * norm).  An empty shard gives {0, 0, 1}.  max_norm must be > 0 (+inf
 * turns clipping off); zero, negative or NaN -> BFO_EINVAL.
 * workspace: device memory of at least bfo_norm_workspace_bytes bytes,
 * 8-byte aligned, owned by the caller, written and read by this call only
 * (its contents before and after mean nothing); calls with separate
 * workspaces may run at the same time on different streams.  NULL uses a
 * buffer the table holds, so calls on one table with a NULL workspace must
 * not overlap in time. */
int grad_global_norm(bfo_table table, const uint16_t *grads, float max_norm, void *workspace,
                     bfo_norm_result *out, void *stream);

/* grad_global_norm for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, partition and bits, with the partials kept in
 * a fixed 8 MiB device array of the library instead of a workspace.  Every
 * GPU the library runs on holds its own copy of that array until the process
 * ends; its address is looked up on the first call on each device.  The call
 * allocates nothing.  Shards of up to 8,587,837,440 elements (1,048,320
 * norm tiles); larger ones -> BFO_ERANGE.  The array keeps the last call's
 * partials, which nothing reads (each call writes every partial it reads),
 * but all calls on one GPU share it: calls whose GPU work overlaps in time
 * on one GPU (different streams without ordering, or several threads) race
 * and give wrong norms.  Other arguments and errors as grad_global_norm. */
int grad_global_norm_noalloc(bfo_table table, const uint16_t *grads, float max_norm, bfo_norm_result *out,
                             void *stream);

/* One AdamW step over the shard ("04 · 多 GPU 与混合精度" §2.2, with the
 * lerp computed as two fused multiply-adds; "第 13 讲" §1.7 for bias
 * correction and decoupled decay).  Per element i (global) / j (local):
 *   g   = scale * f32(grads[j])
 *   m1  = fma(b1, m[j], fma(-b1, g, g));  v1 = fma(b2, v[j], fma(-b2, g*g, g*g))
 *   mh  = m1 / bc1;  vh = v1 / bc2;  u = mh / (sqrt(vh) + eps)
 *   old = master ? master[j] : f32(params[j])
 *   p   = old - lr * (u + w_i * old),  w_i = weight_decay if i's tensor has
 *         BFO_FLAG_DECAY else 0
 *   m[j] = m1; v[j] = v1; master[j] = p (when master != NULL);
 *   params[j] = SR(p, r16(i, seed)) or RNE(p)
 * each a single binary32 operation in that order.  bc1/bc2 =
 * (float)(1 - pow(beta, t)) in binary64, or 1 when bias correction is off.
 * SR rounds to the next bf16 away from zero when the 16 discarded bits of p
 * exceed r16, else truncates; r16 is a 16-bit draw of Philox4x32-10 (Salmon
 * et al., SC'11) with counter (lo32(i>>3), hi32(i>>3), 0, 0) and key
 * (lo32(seed), hi32(seed)); element i takes output word (i>>1)&3, low half
 * for even i.  RNE rounds to nearest, ties to even.  NaN stays NaN.
 * i is element j's global index (its run's global + offset), so every
 * layout and shard count draws the same r16 for the same parameter.
 * master == NULL selects the no-master path (old weights read from params).
 * scale: device float (e.g. &out->scale of grad_global_norm), or NULL for 1.
 * skip: device int32 (e.g. written by bfo_outlier_update), or NULL; when it
 * holds a nonzero value at run time the step changes nothing (every
 * workgroup exits after reading it).
 * t: 1-based step number (0 -> BFO_EINVAL).  rounding: BFO_ROUND_SR/RNE. */
int adamw_sr_step(bfo_table table, uint16_t *params, const uint16_t *grads, float *master, float *m,
                  float *v, const bfo_adamw_hparams *hp, const float *scale, const int32_t *skip, uint64_t t,
                  uint64_t seed, int rounding, void *stream);

/* grad_global_norm and then adamw_sr_step with that norm's clip scale, in
 * one call ("04 · 多 GPU 与混合精度" §4 for the norm and clip, §2.2 for the
 * update): the result -- *out, params, master, m, v -- is bit for bit that
 * of the two calls.  For shards of at most 65,536 elements (8 norm tiles)
 * both run in one kernel launch: every workgroup of the update forms the
 * whole shard's sum of squares itself, in the norm's partition and order,
 * so a small step pays one launch instead of two (workspace is then not
 * used); larger shards take the two calls' launches.  skip: as in
 * adamw_sr_step (the norm is still written).  Arguments and errors as the
 * two calls; out and workspace must not overlap the arrays. */
int adamw_sr_step_with_norm(bfo_table table, uint16_t *params, const uint16_t *grads, float *master, float *m,
                            float *v, const bfo_adamw_hparams *hp, float max_norm, void *workspace,
                            bfo_norm_result *out, const int32_t *skip, uint64_t t, uint64_t seed, int rounding,
                            void *stream);

/* The per-step scalars of adamw_sr_step, for a step whose launches are
 * recorded once (HIP graph capture) and replayed every step: they are read
 * from device memory when the step runs instead of being passed by value.
 * ("04 · 多 GPU 与混合精度" §4: the learning rate and the step number change
 * every step; "第 13 讲" §1.7: bias correction.)  32 bytes. */
typedef struct {
    float lr;
    float bc1;          /* 1 - beta1^t as adamw_sr_step forms it (1 when correction is off) */
    float bc2;          /* 1 - beta2^t, likewise */
    uint32_t reserved;  /* 0 */
    uint64_t t;         /* the 1-based step number these were formed for */
    uint64_t seed;      /* the step's rounding seed */
} bfo_step_scalars;

/* Host only: *out = the scalars adamw_sr_step(hp with lr, t, seed) uses --
 * bc1 and bc2 exactly as documented there.  hp->lr is ignored (lr is the
 * step's rate, e.g. from bfo_lr_at).  BFO_EINVAL for a null pointer or
 * t == 0. */
int bfo_step_scalars_fill(const bfo_adamw_hparams *hp, uint64_t t, float lr, uint64_t seed,
                          bfo_step_scalars *out);

/* adamw_sr_step with its per-step scalars taken on the device at run time:
 * the step uses steps[*cursor], where steps is a device array of `count`
 * bfo_step_scalars (16-byte aligned) and cursor a device uint64 (8-byte
 * aligned).  hp supplies beta1, beta2, eps and weight_decay; its lr and
 * bias_correction are ignored (the scalars carry them).  A cursor at or past
 * `count` makes the step change nothing, as a set skip flag does.  Every
 * other argument is as in adamw_sr_step, and for the same scalars the result
 * is the same bit for bit.  No argument varies from step to step, so a graph
 * recorded from grad_global_norm, this call and bfo_cursor_advance replays
 * step after step, the caller changing only the grads (and, if it likes,
 * the steps array) between replays. */
int adamw_sr_step_scheduled(bfo_table table, uint16_t *params, const uint16_t *grads, float *master, float *m,
                            float *v, const bfo_adamw_hparams *hp, const bfo_step_scalars *steps,
                            uint64_t count, const uint64_t *cursor, const float *scale, const int32_t *skip,
                            int rounding, void *stream);

/* *cursor += 1, on the device (one work-item), queued on stream. */
int bfo_cursor_advance(uint64_t *cursor, void *stream);

/* Resume-time rebuild ("04 · 多 GPU 与混合精度" §5.2): params at element j's
 * position = SR(master[j], r16(i, seed)) with the draws of adamw_sr_step, so
 * passing the seed of the update that produced `master` reproduces its
 * bf16 output bit for bit. */
int master_to_bf16_sr(bfo_table table, const float *master, uint16_t *params, uint64_t seed,
                      void *stream);

/* The same rebuild with a rounding mode: BFO_ROUND_SR as master_to_bf16_sr,
 * BFO_ROUND_RNE params = RNE(master[j]) (seed unused), which reproduces an
 * update made with round-to-nearest.  Unknown rounding: BFO_EINVAL. */
int master_to_bf16(bfo_table table, const float *master, uint16_t *params, uint64_t seed, int rounding,
                   void *stream);

/* Test export: out[k] = r16(first + k, seed) for k < count (device array,
 * 2-byte aligned).  Any first and count. */
int bfo_rng_dump(uint64_t first, uint64_t count, uint64_t seed, uint16_t *out, void *stream);

/* Test export: out[j] = 1 if shard element j's tensor has BFO_FLAG_DECAY,
 * else 0, as the update kernel sees it (device array of S bytes). */
int bfo_decay_mask_dump(bfo_table table, uint8_t *out, void *stream);

/* Measurement export: the update's memory traffic with none of its
 * arithmetic, for an achievable-bandwidth ceiling measured the same way as
 * the update, in the update's workgroup and lane plan (4-element quads:
 * 16-byte fp32 and 8-byte bf16 accesses) and with its cache policies.  For
 * j < count (device arrays of count elements):
 *   BFO_MIX_BOTH -- with a master: m[j], v[j], master[j] ^= key (as 32-bit
 *     patterns) and params[j] = grads[j] ^ (key & 0xFFFF): 14 bytes read and
 *     14 written per element, as the master update; master == NULL: m[j],
 *     v[j] ^= key and params[j] ^= grads[j] ^ (key & 0xFFFF): 12 read and 10
 *     written, as the no-master update.  key 0 leaves m, v and master
 *     unchanged;
 *   BFO_MIX_READS -- the same reads and no writes (14 or 12 bytes per
 *     element); nothing changes;
 *   BFO_MIX_WRITES -- the same writes and no reads (14 or 10 bytes per
 *     element) of words made from key and j: m, v, master and params are
 *     overwritten.
 * READS and WRITES time the two directions of the mix on their own.  Every
 * non-null pointer 16-byte aligned (else BFO_EMISALIGNED); unknown mode
 * BFO_EINVAL; count 0 is a no-op. */
enum { BFO_MIX_BOTH = 0, BFO_MIX_READS = 1, BFO_MIX_WRITES = 2 };
int bfo_stream_mix(uint16_t *params, const uint16_t *grads, float *master, float *m, float *v, uint64_t count,
                   uint32_t key, int mode, void *stream);

/* Learning-rate schedules ("04 · 多 GPU 与混合精度" §4 names cosine, linear,
 * constant and wsd; the formulas are this library's reading).  For 0-based
 * step s, lr_min = final_frac * lr_max, W = warmup_steps, T = total_steps:
 *   s < W: lr_max * (s + 1) / W (every kind);
 *   then, with p = min(1, (s - W) / (T - W)) (p = 1 when T == W):
 *   CONSTANT lr_max; LINEAR lr_max - (lr_max - lr_min) * p;
 *   COSINE lr_min + (lr_max - lr_min) * (1 + cos(pi * p)) / 2;
 *   WSD lr_max until s >= T - D with D = decay_frac * T, then linear from
 *   lr_max to lr_min over those last D steps.
 * Evaluated in binary64, rounded once to binary32.  Host only. */
enum { BFO_LR_CONSTANT = 0, BFO_LR_LINEAR = 1, BFO_LR_COSINE = 2, BFO_LR_WSD = 3 };
typedef struct {
    int32_t kind;
    uint32_t reserved;
    uint64_t warmup_steps;
    uint64_t total_steps;   /* >= warmup_steps */
    float lr_max;
    float final_frac;
    float decay_frac;       /* WSD only */
    uint32_t reserved2;
} bfo_lr_schedule;

/* *lr = the schedule's learning rate at step `step`.  BFO_EINVAL for a null
 * argument, an unknown kind or total_steps < warmup_steps. */
int bfo_lr_at(const bfo_lr_schedule *schedule, uint64_t step, float *lr);

/* Outlier detector ("04 · 多 GPU 与混合精度" §4: z-score of the grad norm
 * over a window of 128 values; the update is skipped when it exceeds a
 * threshold).  State lives in device memory so the decision never leaves
 * the GPU.  bfo_outlier_update reads *value (device float, e.g.
 * &norm_out->norm), and writes, on `stream`:
 *   *z    = (value - mean) / sqrt(variance) of the previous `window` finite
 *           values (binary64, population variance, summed oldest to newest),
 *           NaN until `window` values have been seen;
 *   *skip = 1 if value is not finite, or threshold > 0 and z > threshold;
 *           else 0 (pass skip to adamw_sr_step);
 * then appends value to the window if it is finite.  window: 1..4096. */
typedef struct bfo_outlier_s *bfo_outlier;
int bfo_outlier_create(uint32_t window, float threshold, bfo_outlier *out);
int bfo_outlier_destroy(bfo_outlier detector);
/* Empties the window (queued on `stream`). */
int bfo_outlier_reset(bfo_outlier detector, void *stream);
int bfo_outlier_update(bfo_outlier detector, const float *value, float *z, int32_t *skip, void *stream);

/* Checkpoints ("04 · 多 GPU 与混合精度" §5.1-5.2).  Each rank saves its own
 * optimizer state; a DONE marker written after every rank has saved makes
 * the checkpoint count; resume takes the newest step with a marker.  With a
 * master, the bf16 weights need not be saved: loading rebuilds them from the
 * master with the saved seed and rounding mode, bit-identical to the ones
 * the saved step produced, and because only the master is needed the same
 * state can also resume a run without a master (the page's precision switch
 * at resume).
 *
 * bfo_checkpoint_save writes <dir>/state_<step:08>_<rank:05>.bin: a 128-byte
 * header (magic "BFOSTATE", version 2, step, seed, n, S, world, rank,
 * layout, whether a master and whether params are stored, a fingerprint of
 * the tensor table, the rounding mode, a checksum of each payload array and
 * one of the header) and the payload: master (S fp32) when master is not
 * NULL, the shard's bf16 params in shard-local order when params is not NULL
 * (params addressed as in adamw_sr_step), then m and v (S fp32 each).  At
 * least one of master and params must be given.  step is the last step the
 * state includes; seed and rounding (BFO_ROUND_SR / BFO_ROUND_RNE) are those
 * of the last update that changed the state.  Pass params too when that
 * update is not known for sure -- e.g. when a device skip flag may have
 * dropped it: the stored params are then restored as they are.  The
 * checksums are bfo_checksum64 of each array's bytes as stored.  Device
 * arrays are copied through a pinned buffer on `stream` after the work
 * already queued there; the call returns when the file is on disk (written
 * under a temporary name, synced, renamed into place, directory synced).
 * Errors: BFO_EINVAL, BFO_EIO, BFO_EHIP. */
int bfo_checkpoint_save(const char *dir, bfo_table table, const uint16_t *params, const float *master,
                        const float *m, const float *v, uint64_t step, uint64_t seed, int rounding, void *stream);

/* Creates the empty marker <dir>/DONE_<step:08> and syncs it and the
 * directory to disk. */
int bfo_checkpoint_done(const char *dir, uint64_t step);

/* *step = the largest step with a DONE marker in dir; BFO_ENOTFOUND if none. */
int bfo_checkpoint_latest(const char *dir, uint64_t *step);

/* Reads this rank's state of `step`; *seed (if not NULL) gets the saved seed.
 * m and v are always read.  master not NULL: the stored master is read into
 * it (BFO_EFORMAT if the file has none).  params not NULL: the shard's
 * positions of params get the stored params if the file has them, else they
 * are rebuilt from the stored master as master_to_bf16 does with the saved
 * seed and rounding mode -- also when master is NULL, which resumes a
 * master checkpoint in a run without one (v's buffer then holds the master
 * while the params are rebuilt, before v is read).  master and params may
 * not both be NULL.  BFO_ENOTFOUND if the file is missing; BFO_EFORMAT if
 * its header does not match the table (sizes, world, rank, layout,
 * fingerprint), the file is truncated, or a checksum does not match (the
 * arrays then hold partly loaded data and must not be used). */
int bfo_checkpoint_load(const char *dir, uint64_t step, bfo_table table, uint16_t *params, float *master,
                        float *m, float *v, uint64_t *seed, void *stream);

/* The 64-bit checksum stored in checkpoint headers, of `bytes` bytes of host
 * memory: four lanes h[0..3] (h[l] starting at the 64-bit FNV-1a offset
 * basis + l) take the data in 32-byte blocks (the last one padded with
 * zeros), lane l folding the block's l-th little-endian 8-byte word w in as
 * h[l] = (h[l] ^ w) * 1099511628211; then x = basis ^ bytes and, for each
 * lane in order, x = (x ^ h[l]) * 1099511628211, x ^= x >> 29.  A change
 * that stays within one 8-byte word always changes the result.  Host only. */
uint64_t bfo_checksum64(const void *data, uint64_t bytes);

/* Placement of the step's arrays in device memory (a measured property of
 * MI355X, not of the method).  The update streams five arrays at the same
 * element index -- params, grads, master, m, v -- and it moves its bytes
 * about 15% faster (6.1 against 5.3 TB/s on the 1.5B model's shard) when
 * every pair of them lies in different 16 GiB-aligned regions of physical
 * device memory, i.e. their physical addresses differ in bit 34 or above;
 * sharing a region, even at gigabytes' distance, gives the lower rate.  The
 * library does not allocate these arrays; a caller can get the placement by
 * carving them from one allocation that covers most of the device (whose
 * physical backing then follows its virtual layout) at the offsets below,
 * and fill the gaps with its other buffers.  Placement changes no result.
 *
 * Which regions also matters, a little for five arrays and a lot for four:
 * four arrays in the four regions of one 64 GiB-aligned block run at the
 * lower rate again, so the layout below starts no array in the fourth
 * region of a block.
 *
 * bfo_spread_layout: for `count` arrays of bytes[k] bytes (in that order),
 * offsets[k] = the first multiple of BFO_REGION_BYTES at or after the end
 * of array k-1 that is not the fourth region of a 64 GiB-aligned block
 * (offsets[0] = 0); *total = offsets[count-1] + bytes[count-1] (0 when
 * count is 0).  BFO_EINVAL for null pointers with count > 0 and BFO_ERANGE
 * if an offset or the total does not fit in 64 bits.  Host only. */
#define BFO_REGION_BYTES (1ull << 34)
int bfo_spread_layout(const uint64_t *bytes, uint32_t count, uint64_t *offsets, uint64_t *total);

/* Static string naming a status code. */
const char *bfo_status_string(int status);

/* hipError_t code of the last HIP failure seen by the calling thread (0 if none). */
int bfo_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BF16OPT_H */
