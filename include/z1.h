/*
 * z1.h -- C ABI of the ZeRO-1 shard optimizer step for one data-parallel
 * rank on one AMD Instinct MI355X (gfx950).
 *
 * The step (per optimizer step t, on this rank's shard of every parameter):
 *   1. shard plan      each tensor's numel split evenly over dp_size ranks,
 *                      rank r owning one contiguous slice
 *                      ("ZeRO-1 风格的 Distributed Optimizer", §6.3 shard
 *                      划分策略; §6.2: optimizer state only for the local
 *                      slice)
 *   2. accumulation    fp32 sum of K bf16 micro-batch gradients
 *                      ("Distributed Training", How it works, §2 Gradient
 *                      accumulation; tutorial §6.7; Nanotron Guide config
 *                      accumulate_grad_in_fp32)
 *   3. grad norm       S = sum of acc^2 over the shard, clip coefficient
 *                      c = min(1, clip / (sqrt(S) + 1e-6)) (tutorial §6.6
 *                      clip_grad: 1.0; the formula is torch's
 *                      clip_grad_norm_, the pages give only the key)
 *   4. AdamW           decoupled weight decay and bias-corrected moments on
 *                      the fp32 master / m / v shard (tutorial §6.6
 *                      adam_beta1 0.9, adam_beta2 0.95, adam_eps 1e-8,
 *                      weight_decay 0.1; Nanotron Guide, ZeRO-1 Optimizer
 *                      State Partitioning: fp32 master, m and v per parameter)
 *   5. bf16 weights    round-to-nearest-even of the new master into this
 *                      rank's slice of the full bf16 weight, which the
 *                      all-gather would then distribute (tutorial §6.2 step
 *                      4 and §6.3)
 *
 * Conventions
 *   - "device pointer" means memory on the GPU that is current when the plan
 *     is created (hipMalloc / PyTorch).  "host pointer" means ordinary CPU
 *     memory.  The caller owns every buffer it passes; the library never
 *     frees or reallocates caller memory.
 *   - The library owns only what z1_plan_create allocates (the chunk table,
 *     pointer tables and norm partials) and frees it in z1_plan_destroy.
 *     z1_accum_grads(_range), z1_grad_norm_sq, z1_adamw_step and
 *     z1_adamw_step_scheduled allocate nothing (z1_schedule_create owns its
 *     table until z1_schedule_destroy).
 *   - Work is enqueued on the given stream and the calls return without
 *     waiting for it; none of the step calls synchronises with the host.
 *     A kernel fault surfaces at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued: a
 *     call that returns Z1_EINVAL, Z1_EALIGN or Z1_ESTATE has enqueued no
 *     work.  Z1_EHIP means a launch failed (see each call).
 *   - A plan (or schedule, or pack) belongs to the GPU that is current when
 *     it is created; its calls take a stream of that GPU, with that GPU
 *     current.  A call that would enqueue work with another GPU current, or
 *     on a stream of another GPU, returns Z1_EINVAL and enqueues nothing;
 *     so does a scheduled step whose schedule and plan belong to different
 *     GPUs.  The destroy and query calls make the owning GPU current for
 *     their duration and restore the caller's.
 *   - A plan is used from one host thread and one stream at a time.
 *   - No C++ exception crosses this interface: a host allocation that fails
 *     while a call builds its tables returns Z1_ENOMEM.
 */
#ifndef Z1_H
#define Z1_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Z1_ABI_VERSION 10

typedef enum z1_status {
    Z1_OK = 0,
    Z1_EINVAL = 1, /* bad size, rank, micro-batch index, hyperparameter or null pointer */
    Z1_EALIGN = 2, /* a device base pointer is not 16-byte aligned (8 for d_S) */
    Z1_ENOMEM = 3, /* a library-owned allocation failed (device or host) */
    Z1_EHIP = 4,   /* the HIP runtime reported an error (launch or copy) */
    Z1_ESTATE = 5  /* calls made out of order (see z1_accum_grads) */
} z1_status;

/* A hipStream_t (struct ihipStream_t*); NULL is the null stream. */
typedef struct ihipStream_t *z1_stream;

/* Opaque plan: the shard geometry of one parameter list on one rank, bound
 * to the caller's device buffers. */
typedef struct z1_plan z1_plan;

/* Version of this interface (Z1_ABI_VERSION of the built library). */
int32_t z1_abi_version(void);

/* Static text for a status code; never NULL. */
const char *z1_strerror(z1_status status);

/* ------------------------------------------------------------------------
 * z1_shard_plan -- host-only shard plan (no device work).
 *
 * For each tensor i with numel[i] = q*dp_size + rho (0 <= rho < dp_size):
 *   len[i]   = q + (rank < rho ? 1 : 0)
 *   start[i] = rank*q + min(rank, rho)
 * so the dp_size slices of a tensor are contiguous, in rank order, cover it
 * exactly and differ in size by at most one element, the first rho ranks
 * holding the extra element ("ZeRO-1 风格的 Distributed Optimizer", §6.3:
 * every parameter is split on its own, its numel divided evenly over the
 * ranks; which ranks take the remainder is not on the page).
 *
 * arena_off[i] is where slice i lives in the fp32 arenas (master, m, v,
 * acc): offsets increase with i, slices do not overlap, and
 * arena_off[i] == start[i] (mod 64), so that element e of a slice sits at
 * the same position within a 128-byte cache line of a bf16 tensor (or
 * packed bf16 shard) and within a 256-byte block of an fp32 arena: the
 * pieces the step cuts at multiples of its work unit inside a tensor start
 * on whole lines of every buffer.  *arena_elems is the arena length in
 * elements (the shard size plus at most 63 padding elements per tensor).
 * (Before ABI version 7 the residue was taken mod 8.)
 *
 *   n_tensors   >= 0 (0 gives *arena_elems = 0)
 *   numel       host [n_tensors], each >= 0
 *   dp_size     >= 1;  rank in [0, dp_size)
 *   start, len, arena_off   host [n_tensors], written by the call
 *   arena_elems host, written by the call
 * Errors: Z1_EINVAL for a negative count or numel, a bad dp_size or rank,
 * or a null pointer (numel/start/len/arena_off may be NULL only when
 * n_tensors == 0).  Deterministic: same inputs, same outputs.
 * ------------------------------------------------------------------------ */
z1_status z1_shard_plan(int32_t n_tensors, const int64_t *numel, int32_t dp_size,
                        int32_t rank, int64_t *start, int64_t *len, int64_t *arena_off,
                        int64_t *arena_elems);

/* How a tensor list is cut into per-rank slices.  Every kind gives each
 * tensor one contiguous slice [start, start+len) per rank (possibly empty),
 * so the step itself is the same for all of them. */
typedef enum z1_plan_kind {
    /* each tensor split evenly on its own (z1_shard_plan above; nanotron,
     * "ZeRO-1 风格的 Distributed Optimizer" §6.3) */
    Z1_PLAN_PER_TENSOR = 0,
    /* all tensors concatenated in order and the concatenation split evenly,
     * first (total mod dp_size) ranks one element longer; a tensor's slice is
     * its overlap with the rank's range (the flatten-first layout §6.3
     * contrasts nanotron with) */
    Z1_PLAN_FLAT = 1,
    /* each tensor's rows (dimension 0) split like torch.chunk: ceil(rows /
     * dp_size) rows per rank in rank order, the last ranks possibly short or
     * empty ("TorchTitan 生产级预训练方案", appendix B.1: FSDP2 shards every
     * parameter on dimension 0; the rounding is not on the page) */
    Z1_PLAN_DIM0 = 2
} z1_plan_kind;

/* ------------------------------------------------------------------------
 * z1_shard_plan_kind -- z1_shard_plan for any z1_plan_kind.
 *
 * rows: host [n_tensors] dimension-0 sizes, read only for Z1_PLAN_DIM0
 * (numel[i] must be a multiple of rows[i]; rows[i] == 0 requires
 * numel[i] == 0); may be NULL otherwise.  Empty slices report start 0.
 * Arena offsets follow the same rule as z1_shard_plan.
 * Errors: as z1_shard_plan, plus Z1_EINVAL for an unknown kind or bad rows.
 * ------------------------------------------------------------------------ */
z1_status z1_shard_plan_kind(int32_t kind, int32_t n_tensors, const int64_t *numel,
                             const int64_t *rows, int32_t dp_size, int32_t rank,
                             int64_t *start, int64_t *len, int64_t *arena_off,
                             int64_t *arena_elems);

/* Buffers and geometry bound to a plan.  All device buffers are caller-owned
 * and must stay allocated until z1_plan_destroy. */
typedef struct z1_bind {
    int32_t n_tensors;      /* number of parameter tensors, >= 0            */
    int32_t dp_size;        /* >= 1                                         */
    int32_t rank;           /* in [0, dp_size)                              */
    int32_t n_micro;        /* K, bf16 micro-batch gradients per step, >= 1 */
    const int64_t *numel;   /* host [n_tensors]                             */
    /* bf16 working weights.  layout Z1_LAYOUT_FULL: host array [n_tensors]
     * of device pointers, each to element 0 of the FULL tensor (numel[i]
     * bf16 values); the step writes only elements [start[i],
     * start[i]+len[i]).  Z1_LAYOUT_PACKED: host array [1] holding one device
     * pointer to a packed bf16 shard of arena_elems values in arena order
     * (element e of slice i at arena_off[i] + e, as in the fp32 arenas);
     * padding elements are never written.                                  */
    void *const *weights;
    /* bf16 micro-batch gradients.  Z1_LAYOUT_FULL: host array
     * [n_micro * n_tensors] of device pointers; grads[k*n_tensors + i]
     * points to element 0 of the FULL gradient of tensor i for micro-batch
     * k, of which only this rank's slice is read.  Z1_LAYOUT_PACKED: host
     * array [n_micro], grads[k] one packed bf16 shard of arena_elems values
     * (the value z1_shard_plan returns) in arena order (for example the
     * output of an equal-count reduce-scatter); its padding may be read,
     * as the fp32 arenas' may.                                             */
    const void *const *grads;
    /* fp32 arenas, device, arena_elems floats each (see z1_shard_plan).
     * master holds the fp32 master weights, exp_avg / exp_avg_sq the Adam
     * moments (zero before the first step), acc receives the accumulated
     * gradient.  Padding elements are never written; the arena walks
     * (packed plans) may read them, in a tile that holds a slice boundary,
     * and discard what they read.                                          */
    float *master;
    float *exp_avg;
    float *exp_avg_sq;
    float *acc;
    int64_t arena_elems;    /* length the caller allocated; must be >= the
                               value z1_shard_plan returns                  */
    int64_t chunk_elems;    /* work unit in elements; 0 = library default
                               (4096); otherwise a multiple of 1024 in
                               [1024, 1048576]                              */
    int32_t max_blocks;     /* 0 = one workgroup per chunk; otherwise the
                               grid size of the accumulation kernels, and
                               4 x max_blocks one-wave workgroups for AdamW
                               (each workgroup loops over its work)        */
    int32_t plan_kind;      /* z1_plan_kind (0 = per tensor)                */
    const int64_t *rows;    /* host [n_tensors] dim-0 sizes for
                               Z1_PLAN_DIM0, else NULL                      */
    /* Per-tensor multipliers, host [n_tensors] each, NULL = all 1.0:
     * tensor i steps with lr*lr_scale[i] and weight_decay*wd_scale[i]
     * (Nanotron Guide, Spectral muTransfer: eta_hidden = eta_0 / d_model;
     * wd_scale 0 keeps a tensor out of weight decay).  Copied at creation;
     * must be finite, wd_scale >= 0.                                       */
    const double *lr_scale;
    const double *wd_scale;
    int32_t layout;         /* z1_layout of weights and grads (0 = full)    */
    int32_t walk;           /* z1_walk: how the AdamW step walks the shard
                               (0 = the library's choice)                   */
} z1_bind;

/* Where the bf16 weights and gradients live (z1_bind.layout).  The packed
 * form is the shard as the collectives around the step exchange it: with the
 * arena offsets residue-matched to the slice starts, a packed bf16 shard has
 * the same 16-byte alignment per element as the full tensor, so the kernels
 * are the same for both. */
typedef enum z1_layout {
    Z1_LAYOUT_FULL = 0,
    Z1_LAYOUT_PACKED = 1
} z1_layout;

/* How the AdamW step walks the shard (z1_bind.walk); the arithmetic and the
 * bits stored are the same either way.  AdamW runs one-wave workgroups of 256
 * elements (one 4-element vector per lane), at most 14 resident per compute
 * unit on either walk.
 *   Z1_WALK_CHUNKS       chunk_elems / 256 workgroups per entry of the chunk
 *                        table.  (The walk also decides the accumulation:
 *                        passes of one slot or of 8-16 slots take the
 *                        arena tiles when the plan has them; passes of 2-7
 *                        slots and the norm of a given acc always walk the
 *                        chunk table.)
 *   Z1_WALK_ARENA_TILES  one workgroup per 256-element tile of the arena;
 *                        every fp32 stream is addressed by arena position,
 *                        so a tile's loads depend on nothing fetched first.
 *                        A tile inside one slice takes its tensor from a
 *                        per-tile tag read after its loads are issued (with
 *                        full-size bf16 tensors, also the tensor's entry of
 *                        a per-tensor table for its bf16 store); a tile that
 *                        crosses a slice boundary (or the arena's end) runs
 *                        its slice segments one by one (padding is never
 *                        written).
 *   Z1_WALK_AUTO         arena tiles for a plan (either layout) with at
 *                        most 1% of its tiles crossing a slice boundary (the
 *                        loads of such a tile are issued before its tag is
 *                        known and then discarded), otherwise the chunk
 *                        table.
 * The arena walk runs one workgroup per tile, so AUTO keeps the chunk table
 * when max_blocks caps the grid.  Z1_WALK_ARENA_TILES with max_blocks > 0,
 * or any other value, is Z1_EINVAL at plan creation. */
typedef enum z1_walk {
    Z1_WALK_AUTO = 0,
    Z1_WALK_CHUNKS = 1,
    Z1_WALK_ARENA_TILES = 2
} z1_walk;

/* Geometry of a created plan. */
typedef struct z1_plan_info {
    int32_t n_tensors;
    int32_t n_micro;
    int64_t shard_elems;    /* L = sum of len[i]                          */
    int64_t arena_elems;    /* arena length required                      */
    int64_t chunk_elems;    /* work unit in elements                      */
    int64_t n_chunks;       /* entries of the device chunk table          */
    int64_t adamw_tiles;    /* 256-element arena tiles the AdamW step
                               walks (Z1_WALK_ARENA_TILES), 0 when it
                               walks the chunk table                      */
    int64_t boundary_tiles; /* of those, tiles that cross a slice boundary
                               or the arena's end                         */
} z1_plan_info;

/* ------------------------------------------------------------------------
 * z1_plan_create -- validate the binding, compute the shard plan, build the
 * chunk table (one entry per piece of a slice of at most chunk_elems
 * elements, split at multiples of chunk_elems within the tensor; empty
 * slices produce no entry) and upload it to the device once.
 *
 * Copies the pointer arrays; the caller may free bind's host arrays after
 * the call.  The upload is enqueued on `stream` and the call waits for it
 * (plan creation is not part of the step), so the plan is ready on return.
 * Errors: Z1_EINVAL (bad geometry, null pointers, arena too small,
 * bad chunk_elems, bad plan_kind / rows / multipliers / layout, reserved not 0), Z1_EALIGN
 * (a weight, gradient or arena pointer not 16-byte aligned), Z1_ENOMEM, Z1_EHIP.  *out is
 * NULL on error.
 * ------------------------------------------------------------------------ */
z1_status z1_plan_create(z1_plan **out, const z1_bind *bind, z1_stream stream);

/* Frees the plan's device and host memory (waits for the device to finish
 * using it).  NULL is accepted and ignored. */
z1_status z1_plan_destroy(z1_plan *plan);

/* Fills *info.  Z1_EINVAL on NULL. */
z1_status z1_plan_query(const z1_plan *plan, z1_plan_info *info);

/* Copies the plan's start / len / arena_off arrays (host [n_tensors] each,
 * any may be NULL).  Z1_EINVAL on a NULL plan. */
z1_status z1_plan_layout(const z1_plan *plan, int64_t *start, int64_t *len,
                         int64_t *arena_off);

/* ------------------------------------------------------------------------
 * z1_accum_grads -- fp32 accumulation of micro-batch k into the acc arena.
 *
 * k == 0:     acc[e] = (float)g_0[e]          (overwrites; may be called at
 *                                              any time and restarts a step)
 * 0 < k < K:  acc[e] = acc[e] + (float)g_k[e] (binary32 add, in order)
 * where g_k[e] is element start[i]+e of gradient (k, i).  The sum is a sum,
 * not a mean ("Distributed Training", §2: grad += backward(...) for each of
 * the K micro-batches, one optimizer step after them).  When k == K-1 the
 * same pass also writes, per chunk, the binary64 sum of acc^2 (a
 * double-double pair), which z1_grad_norm_sq reduces.
 *
 * Order: k must be 0 or one more than the previous accumulation call of this
 * step, else Z1_ESTATE.  Z1_EINVAL for k outside [0, K) or a NULL plan.
 * ------------------------------------------------------------------------ */
z1_status z1_accum_grads(z1_plan *plan, int32_t k, z1_stream stream);

/* ------------------------------------------------------------------------
 * z1_accum_grads_range -- micro-batches k_begin .. k_end-1 in one call.
 *
 * Stores exactly what z1_accum_grads(plan, k) for k = k_begin, ..., k_end-1
 * stores, in that order, bit for bit: the same binary32 additions in the
 * same order ("Distributed Training", §2: the gradients of the K micro-batches
 * are summed, one optimizer step after them).  It is for callers that hold
 * several micro-batch gradients in device memory at once (K full-size bf16
 * gradient sets, 2 bytes per parameter each): the range is split into
 * passes of at most 16 slots, as even as possible (20 slots: two passes of
 * 10), so the fp32 acc arena is read and written once per pass instead of
 * once per slot.  For K = 4 that is 12 bytes per shard element instead of 36;
 * for K = 16, 36 instead of 132.  (Before ABI version 9 a pass read at most
 * 8 slots.)
 * A range that ends at K also writes the norm partials, as the k == K-1 pass
 * of z1_accum_grads does.  A range may follow single-slot calls and be
 * followed by them.
 *
 * Order: k_begin must be 0 or one more than the last micro-batch already
 * accumulated in this step, else Z1_ESTATE.  Z1_EINVAL for a NULL plan or
 * unless 0 <= k_begin < k_end <= K (nothing enqueued).  Z1_EHIP if a launch
 * fails; the passes before it may already be enqueued, and the plan then
 * expects the step to restart at k = 0.
 * ------------------------------------------------------------------------ */
z1_status z1_accum_grads_range(z1_plan *plan, int32_t k_begin, int32_t k_end,
                               z1_stream stream);

/* ------------------------------------------------------------------------
 * z1_grad_norm_sq -- S = sum over the shard of acc^2.
 *
 * Writes S, the exact sum rounded to binary64 (double-double partials per
 * chunk, reduced in a fixed order, so the value does not depend on the grid
 * size or on timing), to the DEVICE double *d_S.  On more than one rank the
 * caller would all-reduce S before z1_adamw_step; on one rank S is the
 * global squared norm.
 * Errors: Z1_ESTATE unless all K accumulation passes of this step have been
 * enqueued; Z1_EINVAL for NULL; Z1_EALIGN if d_S is not 8-byte aligned.
 * ------------------------------------------------------------------------ */
z1_status z1_grad_norm_sq(z1_plan *plan, double *d_S, z1_stream stream);

/* ------------------------------------------------------------------------
 * The norm exchanged between ranks without rounding.  On D ranks the clip
 * coefficient needs the global S = sum over ranks of S_r; adding rounded
 * S_r values makes S depend on how it was split.  Instead each rank takes
 * its S_r as the unevaluated pair (hi, lo) the reduction ends with:
 *
 * z1_grad_norm_sq_pair writes d_pair[0] = hi, d_pair[1] = lo (DEVICE, 16-byte
 * aligned), S_r = hi + lo to about 2^-106 relative.  Same call order and
 * errors as z1_grad_norm_sq; afterwards z1_adamw_step may follow.
 *
 * The ranks all-gather the D pairs (16 bytes each, rank order) and each one
 * calls z1_norm_combine on the gathered [D][2] array (DEVICE, 16-byte
 * aligned): the pairs are added in index order in the same double-double
 * arithmetic and the sum is rounded once into d_S (DEVICE double).  Every
 * rank then holds the same S, equal to what one rank holding the whole
 * model computes unless the exact sum lies within about D * 2^-106 of a
 * binary64 rounding boundary.  With D = 1 it equals z1_grad_norm_sq.
 * No plan owns z1_norm_combine: the GPU current at the call must own the
 * stream and both buffers (device memory of that GPU, as the HIP runtime
 * records it), else Z1_EINVAL and nothing is enqueued.
 * Errors: Z1_EINVAL (NULL, n < 1, host memory, another GPU's memory or
 * stream), Z1_EALIGN, Z1_EHIP (no GPU current, launch failure).
 * ------------------------------------------------------------------------ */
z1_status z1_grad_norm_sq_pair(z1_plan *plan, double *d_pair, z1_stream stream);
z1_status z1_norm_combine(const double *d_pairs, int32_t n, double *d_S, z1_stream stream);

/* AdamW hyperparameters of one step (binary64, passed by value to the
 * kernel; the library derives 1 - lr*wd, 1 - beta1, 1 - beta2 and the bias
 * corrections 1 - beta^t on the host in binary64). */
typedef struct z1_adamw_hp {
    double lr;            /* > 0 is not required; finite                      */
    double beta1;         /* in [0, 1)                                         */
    double beta2;         /* in [0, 1)                                         */
    double eps;           /* > 0                                               */
    double weight_decay;  /* >= 0                                              */
    double clip;          /* max global norm; <= 0 disables clipping (c = 1)   */
    int64_t step;         /* t >= 1: this is the t-th optimizer step           */
} z1_adamw_hp;

/* ------------------------------------------------------------------------
 * z1_adamw_step -- clip coefficient, AdamW and the bf16 cast, in one pass.
 *
 * Reads S from the DEVICE pointer d_S_global (no host round trip), forms
 * c = min(1, clip / (sqrt(S) + 1e-6)) (c = 1 when clip <= 0), then for every
 * shard element of tensor i, in binary64 from the stored fp32 values, with
 * lr = hp->lr * lr_scale[i] and wd = hp->weight_decay * wd_scale[i]:
 *   g = c*acc;  p = p*(1 - lr*wd);  m = beta1*m + (1-beta1)*g;
 *   v = beta2*v + (1-beta2)*g*g;  mhat = m/(1-beta1^t);  vhat = v/(1-beta2^t);
 *   p = p - lr*mhat/(sqrt(vhat) + eps)
 * stores p, m, v rounded to fp32 (nearest-even) and writes the bf16
 * round-to-nearest-even of the new fp32 master into the weight slice.
 * Decoupled decay, eps outside the square root and t starting at 1 follow
 * torch.optim.AdamW; the pages give only the hyperparameter values.
 *
 * d_S_global may be NULL only when hp->clip <= 0.
 * Errors: Z1_ESTATE unless all K accumulation passes have been enqueued
 * since the last step and, when clipping is on, z1_grad_norm_sq as well;
 * Z1_EINVAL for bad hyperparameters or NULL; Z1_EALIGN for a misaligned
 * d_S_global.  After a successful call the plan expects k == 0 next.
 * ------------------------------------------------------------------------ */
z1_status z1_adamw_step(z1_plan *plan, const z1_adamw_hp *hp, const double *d_S_global,
                        z1_stream stream);

/* Learning-rate schedule (host only).  Nanotron Guide, config.yaml:
 * learning_rate (peak), lr_warmup_steps, lr_decay_steps, min_decay_lr; the
 * decay shape is not on the page. */
typedef enum z1_decay_style {
    Z1_DECAY_NONE = 0,    /* peak after warmup                              */
    Z1_DECAY_LINEAR = 1,  /* straight line from peak to minimum             */
    Z1_DECAY_COSINE = 2   /* half cosine from peak to minimum               */
} z1_decay_style;

typedef struct z1_lr_schedule {
    double lr_max;          /* peak learning rate                           */
    double lr_min;          /* learning rate after the decay                */
    int64_t warmup_steps;   /* >= 0                                         */
    int64_t decay_steps;    /* >= 0, counted from the end of warmup         */
    int32_t decay_style;    /* z1_decay_style                               */
    int32_t reserved;       /* must be 0                                    */
} z1_lr_schedule;

/* ------------------------------------------------------------------------
 * z1_lr_at -- learning rate of step t (t >= 0), in binary64:
 *   t <= warmup_steps (warmup > 0):  lr_max * t / warmup_steps
 *   after warmup, d = t - warmup_steps:
 *     NONE: lr_max;  d >= decay_steps: lr_min;  else tau = d / decay_steps,
 *     LINEAR: lr_max + (lr_min - lr_max) * tau,
 *     COSINE: lr_min + (lr_max - lr_min) * 0.5 * (1 + cos(pi * tau)).
 * The caller passes the result as z1_adamw_hp.lr.
 * Errors: Z1_EINVAL for NULL, negative counts, unknown style, t < 0.
 * ------------------------------------------------------------------------ */
z1_status z1_lr_at(const z1_lr_schedule *schedule, int64_t step, double *lr);

/* ------------------------------------------------------------------------
 * Per-step schedule for replayed steps.  z1_adamw_step bakes its step t and
 * lr into the launch, so a captured graph would repeat one step.  A
 * schedule holds, on the device, the binary64 constants z1_adamw_step would
 * derive for each of n_steps consecutive steps t = hp->step, hp->step + 1,
 * ... (lr from z1_lr_at(lr, t) when lr is not NULL, else hp->lr every step;
 * beta1, beta2, eps, weight_decay and clip from hp), plus a device counter
 * of the next row.  z1_adamw_step_scheduled applies the constants of that
 * row and then advances the counter, both as kernels on the stream, so
 * [accumulate, norm, z1_adamw_step_scheduled] captured once and replayed
 * once per step trains with the schedule ("Nanotron Guide", config.yaml:
 * warmup and decay of the learning rate).  Each replayed step stores the
 * bits z1_adamw_step stores for the same t and lr.
 *
 * Ownership: the schedule owns its table (80 bytes per step) and counter;
 * z1_schedule_destroy waits for the device and frees them.  A schedule
 * steps one plan at a time (its counter is shared by every caller).
 * z1_schedule_create errors: Z1_EINVAL (NULL, a hyperparameter z1_adamw_step
 * would reject, n_steps outside [1, Z1_SCHEDULE_MAX_STEPS], a bad lr
 * schedule), Z1_ENOMEM, Z1_EHIP; it waits for its upload on `stream`.
 * ------------------------------------------------------------------------ */
#define Z1_SCHEDULE_MAX_STEPS (1LL << 24)
typedef struct z1_schedule z1_schedule;
z1_status z1_schedule_create(z1_schedule **out, const z1_adamw_hp *hp,
                             const z1_lr_schedule *lr, int64_t n_steps, z1_stream stream);
z1_status z1_schedule_destroy(z1_schedule *schedule);

/* The step the next scheduled launch applies (t of its row) and how many
 * scheduled launches found the table exhausted (those changed nothing).
 * A blocking copy of the device counter: synchronise the stream the
 * scheduled steps were enqueued on first.  Either output may be NULL.
 * Errors: Z1_EINVAL, Z1_EHIP. */
z1_status z1_schedule_query(const z1_schedule *schedule, int64_t *next_step, int64_t *overrun);

/* z1_adamw_step with the constants of the schedule's current row; then the
 * row advances.  With the table exhausted nothing is updated and the
 * overrun count grows.  d_S_global and call order as z1_adamw_step (the
 * order is checked when the call is made, not when a graph is replayed).
 * Errors: Z1_EINVAL, Z1_EALIGN, Z1_ESTATE, Z1_EHIP. */
z1_status z1_adamw_step_scheduled(z1_plan *plan, z1_schedule *schedule,
                                  const double *d_S_global, z1_stream stream);

/* ------------------------------------------------------------------------
 * z1_grad_norm_sq_acc -- S from an acc arena the caller filled itself.
 *
 * For the order in which every micro-batch is first accumulated into full
 * fp32 gradients and reduced over DP once ("ZeRO-1 风格的 Distributed
 * Optimizer", §6.7), the reduce-scatter delivers this rank's summed
 * gradient straight into the plan's acc arena (see z1_pack_*): this call
 * reads it once, writes the same per-chunk double-double partials as the
 * last accumulation pass and reduces them to the DEVICE double *d_S.  It
 * marks the accumulation complete, so z1_adamw_step may follow.
 * Errors: Z1_EINVAL for NULL; Z1_EALIGN if d_S is not 8-byte aligned.
 * ------------------------------------------------------------------------ */
z1_status z1_grad_norm_sq_acc(z1_plan *plan, double *d_S, z1_stream stream);

/* ------------------------------------------------------------------------
 * z1_grad_norm_sq_flat_noalloc -- z1_grad_norm_sq_acc for a contiguous fp32
 * gradient shard, with no plan and no allocation.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It needs
 * no plan (whose creation allocates) and calls no hipMalloc / hipFree: its
 * per-tile partials, the second-level stage and the arrival counter live in
 * a fixed device array inside the library (4 MiB + 4.25 KiB per GPU, held
 * until the process ends).  The first call on a GPU resolves that array's
 * address there (hipGetSymbolAddress); make one call before capturing.
 *
 * Writes S = sum over e < n of acc[e]^2, the exact sum of the binary64
 * squares rounded once to binary64 (the same value z1_grad_norm_sq_acc gives
 * for a plan whose shard is these n elements in this order), to the DEVICE
 * double *d_S.
 *   acc    DEVICE, n floats, 16-byte aligned (may be NULL when n == 0)
 *   n      0 <= n <= Z1_NORM_FLAT_MAX_ELEMS (2^30)
 *   d_S    DEVICE, 8-byte aligned
 * Every call on a GPU uses that GPU's one array: calls that overlap on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller; calls on different GPUs are independent.
 * Errors: Z1_EINVAL (n out of range, NULL, host memory, another GPU's memory
 * or stream), Z1_EALIGN, Z1_EHIP (no GPU current, launch failure).
 * ------------------------------------------------------------------------ */
#define Z1_NORM_FLAT_MAX_ELEMS (1LL << 30)
z1_status z1_grad_norm_sq_flat_noalloc(const float *acc, int64_t n, double *d_S,
                                       z1_stream stream);

/* ------------------------------------------------------------------------
 * The step before the shard path: full-tensor accumulation into the
 * reduce-scatter send buffer.
 *
 * Nanotron adds each micro-batch's gradient into full fp32 gradients and
 * reduces over DP after the last one ([T6] §6.7); under ZeRO-1 that is a
 * reduce-scatter ([NG] ZeRO-1 section; [T6] §6.3).  Here the accumulation
 * itself writes the send buffer: segment r (seg_elems floats at r*seg_elems)
 * holds rank r's slice of every tensor at rank r's arena offsets
 * (z1_shard_plan_kind for that rank), so an equal-count reduce-scatter of
 * `send` leaves each rank its acc arena, ready for z1_grad_norm_sq_acc and
 * z1_adamw_step.  Padding elements of the segments are never written.
 * ------------------------------------------------------------------------ */
typedef struct z1_pack z1_pack;

/* Segment length: the largest arena of any rank, rounded up to a multiple of
 * 64 elements (so every segment starts on a 256-byte boundary).  Errors as
 * z1_shard_plan_kind. */
z1_status z1_pack_layout(int32_t kind, int32_t n_tensors, const int64_t *numel,
                         const int64_t *rows, int32_t dp_size, int64_t *seg_elems);

typedef struct z1_pack_bind {
    int32_t n_tensors;
    int32_t dp_size;
    int32_t n_micro;        /* K >= 1                                        */
    int32_t plan_kind;      /* z1_plan_kind                                  */
    const int64_t *numel;   /* host [n_tensors]                              */
    const int64_t *rows;    /* host [n_tensors] for Z1_PLAN_DIM0, else NULL  */
    /* host [n_micro * n_tensors] device pointers to FULL bf16 gradients,
     * 16-byte aligned; every element is read                               */
    const void *const *grads;
    float *send;            /* device, 16-byte aligned, send_elems floats    */
    int64_t send_elems;     /* >= dp_size * seg_elems                        */
    int64_t chunk_elems;    /* 0 = default; else multiple of 1024 in
                               [1024, 1048576]                               */
    int32_t divide;         /* nonzero: the last pass divides by dp_size in
                               binary32 ("TorchTitan 生产级预训练方案",
                               appendix B.1: one division of the fp32
                               gradients by the world size)                  */
    int32_t reserved;       /* must be 0                                     */
} z1_pack_bind;

/* Validates, builds and uploads the chunk table (all ranks' slices); waits
 * for the upload.  Errors: Z1_EINVAL, Z1_EALIGN, Z1_ENOMEM, Z1_EHIP. */
z1_status z1_pack_create(z1_pack **out, const z1_pack_bind *bind, z1_stream stream);
z1_status z1_pack_destroy(z1_pack *pack);

/* Micro-batch k: send = (k == 0 ? 0 : send) + (float)g_k in binary32, in
 * order; the last pass (k == K-1) divides by dp_size when divide is set.
 * Order as z1_accum_grads (k == 0 restarts; otherwise k must follow the
 * previous call), else Z1_ESTATE.  No norm is computed here. */
z1_status z1_pack_accum(z1_pack *pack, int32_t k, z1_stream stream);

/* Micro-batches k_begin .. k_end-1 in one call: bit for bit what
 * z1_pack_accum(pack, k) for each k in order stores, reading up to 16 slots
 * per pass (see z1_accum_grads_range).  Order and errors as
 * z1_accum_grads_range. */
z1_status z1_pack_accum_range(z1_pack *pack, int32_t k_begin, int32_t k_end, z1_stream stream);

/* ------------------------------------------------------------------------
 * Measurement aid (not part of the step): a streaming copy of n_bytes
 * (a multiple of 16, both pointers 16-byte aligned, non-overlapping) from
 * device src to device dst with 16-byte loads and stores (one per lane, one
 * 256-lane workgroup per 4 KB), used to measure the achievable HBM bandwidth
 * and to calibrate byte counters.
 * Errors: Z1_EINVAL, Z1_EALIGN, Z1_EHIP.
 * ------------------------------------------------------------------------ */
z1_status z1_probe_copy(const void *src, void *dst, int64_t n_bytes, z1_stream stream);

/* ------------------------------------------------------------------------
 * Measurement aid (not part of the step): streaming kernels with a step
 * kernel's traffic and no arithmetic, for the bandwidth this machine reaches
 * with each traffic mix.  n_vec counts 16-byte vectors per fp32 stream;
 * half-width (bf16) streams hold n_vec 8-byte vectors.  Every buffer is
 * device memory, 16-byte aligned, large enough for its stream.
 *   Z1_PROBE_READ           bufs[0] read (n_vec x 16 B); bufs[1] >= 4 bytes
 *                           (never written in practice)
 *   Z1_PROBE_WRITE          bufs[0] written
 *   Z1_PROBE_ADAMW_TRAFFIC  read bufs[0..3] (acc, p, m, v), write bufs[1..3]
 *                           and the half-width bufs[4]: 30 B per element
 *   Z1_PROBE_ACCUM_TRAFFIC  read the half-width bufs[0] and bufs[1], write
 *                           bufs[1]: 10 B per element
 *   Z1_PROBE_SLOTS_TRAFFIC  read the half-width bufs[0..G-1], write bufs[G]
 *                           (G = n_bufs - 1 in [2, 16]): 2G + 4 B per element,
 *                           the first resident-slot accumulation pass
 *   Z1_PROBE_ADAMW_TRAFFIC_WAVE  as Z1_PROBE_ADAMW_TRAFFIC, in one-wave (64-lane)
 *                           workgroups of one vector per lane, at most 12 of
 *                           them resident per compute unit: the shape at
 *                           which this mix streams fastest without arithmetic
 *   Z1_PROBE_SLOTS_TRAFFIC_ONE   as Z1_PROBE_SLOTS_TRAFFIC, in one-wave (64-lane)
 *                           workgroups of one vector per lane
 * The default shape is the accumulation kernels': 256-lane workgroups with 4
 * vectors per lane.  The contents written are meaningless.  Z1_EINVAL also
 * when n_vec needs more than 2^31 - 1 workgroups of 64 vectors.  Errors:
 * Z1_EINVAL, Z1_EALIGN, Z1_EHIP.
 * ------------------------------------------------------------------------ */
enum {
    Z1_PROBE_READ = 0,
    Z1_PROBE_WRITE = 1,
    Z1_PROBE_ADAMW_TRAFFIC = 2,
    Z1_PROBE_ACCUM_TRAFFIC = 3,
    Z1_PROBE_SLOTS_TRAFFIC = 4,
    Z1_PROBE_ADAMW_TRAFFIC_WAVE = 5,
    Z1_PROBE_SLOTS_TRAFFIC_ONE = 6
};
z1_status z1_probe(int32_t kind, void *const *bufs, int32_t n_bufs, int64_t n_vec,
                   z1_stream stream);

/* ------------------------------------------------------------------------
 * Measurement aid (not part of the step): Z1_PROBE_PLAN_ADAMW runs the AdamW
 * kernel's chunk walk over the plan's own buffers -- the same loads of acc,
 * master, exp_avg and exp_avg_sq and the same stores of master, exp_avg,
 * exp_avg_sq and the bf16 weight slices -- with the update replaced by an
 * add.  Its duration next to z1_adamw_step's, in the same process, is the
 * cost of the arithmetic on exactly the step's memory.  It OVERWRITES the
 * master, exp_avg, exp_avg_sq arenas and the weight slices with meaningless
 * values; call it only on buffers whose contents are no longer needed.
 * Call order is not checked and not changed.
 * Errors: Z1_EINVAL (NULL plan, unknown kind), Z1_EHIP.
 * ------------------------------------------------------------------------ */
enum { Z1_PROBE_PLAN_ADAMW = 0 };
z1_status z1_probe_plan(z1_plan *plan, int32_t kind, z1_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* Z1_H */
