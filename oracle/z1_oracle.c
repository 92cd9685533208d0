/*
 * z1_oracle.c -- plain CPU oracle for one data-parallel rank's ZeRO-1
 * mixed-precision optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the HIP library is checked against.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never does.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * Everything works on the rank's shard in *packed* order: the slices
 * [start_i, start_i + len_i) of every tensor, concatenated in tensor order.
 * Floating-point work is done in binary64 unless the method itself fixes the
 * precision (the binary32 gradient accumulation and the bf16 weights).
 *
 * Sources (web pages on ZeRO-1 mixed-precision training):
 *   [T6]  "ZeRO-1 风格的 Distributed Optimizer" (nanotron tutorial, ch. 6)
 *   [NG]  "Nanotron Guide: Minimalist 3D-Parallelism LLM Training"
 *   [DT]  "Distributed Training" (atlas wiki library article)
 * Readings where the pages are silent are marked READING and follow
 * PyTorch's clip_grad_norm_ / AdamW conventions.
 *
 * Parallelism: the element-wise loops may use OpenMP; every element is
 * computed independently, so thread count never changes a result.  The norm
 * is a single sequential compensated binary64 sum.
 */
#define _GNU_SOURCE
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <string.h>

#define Z1O_EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------ */
/* O1  shard plan                                                      */
/* ------------------------------------------------------------------ */
/* [T6] §6.3: each parameter is split on its own (not flattened), its
 * total numel divided evenly over dp_size ranks; each rank keeps its 1/N.
 * READING: when dp_size does not divide numel, the first (numel mod dp_size)
 * ranks hold one extra element; slices are contiguous and in rank order. */
Z1O_EXPORT int z1o_shard_plan(int32_t n_tensors, const int64_t *numel,
                              int32_t dp_size, int32_t rank,
                              int64_t *start, int64_t *len)
{
    if (n_tensors < 0 || dp_size < 1 || rank < 0 || rank >= dp_size)
        return -1;
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (numel[i] < 0)
            return -1;
        int64_t q = numel[i] / dp_size;   /* every rank gets q ...        */
        int64_t rho = numel[i] % dp_size; /* ... and rho ranks get one more */
        len[i] = q + (rank < rho ? 1 : 0);
        start[i] = (int64_t)rank * q + (rank < rho ? rank : rho);
    }
    return 0;
}

/* Flatten-then-split (the DeepSpeed layout [T6] §6.3 contrasts with
 * nanotron's): all tensors concatenated in order form one vector of
 * total = sum(numel) elements, split evenly like a single tensor (first
 * total mod dp_size ranks one element longer); a tensor's slice is the
 * intersection of its range in the concatenation with the rank's range.
 * Tensors that miss the rank's range get len 0 (start 0). */
Z1O_EXPORT int z1o_shard_plan_flat(int32_t n_tensors, const int64_t *numel,
                                   int32_t dp_size, int32_t rank,
                                   int64_t *start, int64_t *len)
{
    if (n_tensors < 0 || dp_size < 1 || rank < 0 || rank >= dp_size)
        return -1;
    int64_t total = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (numel[i] < 0)
            return -1;
        total += numel[i];
    }
    int64_t q = total / dp_size, rho = total % dp_size;
    int64_t lo = (int64_t)rank * q + (rank < rho ? rank : rho);
    int64_t hi = lo + q + (rank < rho ? 1 : 0);
    int64_t base = 0; /* first element of tensor i in the concatenation */
    for (int32_t i = 0; i < n_tensors; ++i) {
        int64_t a = lo > base ? lo : base;
        int64_t b = hi < base + numel[i] ? hi : base + numel[i];
        if (a < b) {
            start[i] = a - base;
            len[i] = b - a;
        } else {
            start[i] = 0;
            len[i] = 0;
        }
        base += numel[i];
    }
    return 0;
}

/* Dim-0 sharding of every tensor ("TorchTitan 生产级预训练方案", appendix
 * B.1: FSDP2 represents each parameter as a DTensor sharded on dimension 0).
 * READING: the rows are cut like torch.chunk -- every rank takes
 * ceil(rows / dp_size) rows in rank order, so the last ranks may hold fewer
 * rows or none; a rank's slice is its rows times the row length. */
Z1O_EXPORT int z1o_shard_plan_dim0(int32_t n_tensors, const int64_t *numel,
                                   const int64_t *rows, int32_t dp_size, int32_t rank,
                                   int64_t *start, int64_t *len)
{
    if (n_tensors < 0 || dp_size < 1 || rank < 0 || rank >= dp_size)
        return -1;
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (numel[i] < 0 || rows[i] < 0 || (rows[i] == 0 && numel[i] != 0) ||
            (rows[i] > 0 && numel[i] % rows[i] != 0))
            return -1;
        int64_t row_len = rows[i] ? numel[i] / rows[i] : 0;
        int64_t per = (rows[i] + dp_size - 1) / dp_size;
        int64_t r0 = (int64_t)rank * per;
        int64_t r1 = r0 + per;
        if (r0 > rows[i])
            r0 = rows[i];
        if (r1 > rows[i])
            r1 = rows[i];
        start[i] = r0 * row_len;
        len[i] = (r1 - r0) * row_len;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* bf16 <-> fp32                                                       */
/* ------------------------------------------------------------------ */
static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16; /* bf16 is the top half of binary32 */
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* O2e: round-to-nearest-even of a binary32 value to bfloat16 (8-bit
 * exponent, 7-bit fraction).  The low 16 bits are the discarded part; round
 * up when they exceed half an ulp, or equal half and the kept part is odd.
 * NaN stays NaN (quiet bit set, sign kept); Inf stays Inf; a finite value
 * that rounds past the largest bf16 becomes Inf (the carry runs into the
 * exponent); subnormals round like any other value (no flush). */
Z1O_EXPORT uint16_t z1o_bf16_rne(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u); /* NaN: keep sign, force quiet */
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;
    return (uint16_t)kept;
}

Z1O_EXPORT void z1o_bf16_rne_array(int64_t n, const float *x, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e)
        out[e] = z1o_bf16_rne(x[e]);
}

/* ------------------------------------------------------------------ */
/* O2a  fp32 gradient accumulation                                     */
/* ------------------------------------------------------------------ */
/* [DT] "Gradient accumulation": run K micro-batches, summing gradients,
 * then step once.  [T6] §6.7: gradients of every micro-batch are added into
 * .grad before the DP reduction; [NG] config: accumulate_grad_in_fp32.
 * The sum is the in-order binary32 sum: acc = g_0, acc = acc + g_k for
 * k = 1..K-1, each add rounded to binary32 (the file is built with
 * SSE arithmetic and -ffp-contract=off, so no wider intermediate exists).
 * g is [K][L] packed bf16. */
Z1O_EXPORT void z1o_accumulate(int64_t L, int32_t K, const uint16_t *g, float *acc)
{
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < L; ++e) {
        float a = bf16_to_f32(g[e]);
        for (int32_t k = 1; k < K; ++k) {
            float gk = bf16_to_f32(g[(int64_t)k * L + e]);
            a = a + gk;
        }
        acc[e] = a;
    }
}

/* ------------------------------------------------------------------ */
/* O2b  squared global gradient norm                                   */
/* ------------------------------------------------------------------ */
/* [T6] §6.6 clip_grad: 1.0 -- clipping by the global L2 norm of the
 * accumulated gradient.  S is the sum over the shard of acc^2.  Each square
 * of a binary32 value is exact in binary64, so S has one exact value; the
 * oracle returns it rounded once to binary64.  It gets there with Neumaier's
 * compensated summation (the running sum plus a running sum of the rounding
 * error of every addition), whose error (about n * 2^-106 relative for the
 * non-negative terms here) is far below half an ulp of S.  On one rank the
 * global S is this rank's S. */
Z1O_EXPORT double z1o_norm_sq(int64_t L, const float *acc)
{
    double s = 0.0;   /* running sum                          */
    double err = 0.0; /* sum of the errors of every s + x     */
    for (int64_t e = 0; e < L; ++e) {
        double a = (double)acc[e];
        double x = a * a;
        double t = s + x;
        if (fabs(s) >= fabs(x))
            err += (s - t) + x;
        else
            err += (x - t) + s;
        s = t;
    }
    /* a non-finite term leaves the error sum meaningless (Inf - Inf): the
     * exact sum is then the plain one, +Inf or NaN */
    return isfinite(s) ? s + err : s;
}

/* ------------------------------------------------------------------ */
/* The step before the shard path: the reduce-scatter send buffer      */
/* ------------------------------------------------------------------ */
/* [T6] §6.7: nanotron adds every micro-batch's gradient into the full
 * .grad tensors and reduces over DP only after the last one; under ZeRO-1
 * that reduction is a reduce-scatter ([NG] ZeRO-1 section; [T6] §6.3).  Its
 * send buffer holds, for every rank r in order, rank r's slice of every
 * tensor (the rank's packed shard order).  acc_full is the in-order fp32 sum
 * of the full tensors (z1o_accumulate over the concatenation of all
 * tensors); start/len are [dp_size][n_tensors] slices (any plan kind).  With
 * divide != 0 every value is divided by dp_size in binary32 ("TorchTitan
 * 生产级预训练方案", appendix B.1: a single division of the fp32 gradients by
 * the world size).  out receives sum_r sum_i len[r][i] values. */
Z1O_EXPORT void z1o_pack_send(int32_t n_tensors, const int64_t *numel, int32_t dp_size,
                              const int64_t *start, const int64_t *len,
                              const float *acc_full, int32_t divide, float *out)
{
    int64_t o = 0;
    for (int32_t r = 0; r < dp_size; ++r) {
        int64_t base = 0;
        for (int32_t i = 0; i < n_tensors; ++i) {
            const int64_t s0 = start[(int64_t)r * n_tensors + i];
            const int64_t ln = len[(int64_t)r * n_tensors + i];
            for (int64_t e = 0; e < ln; ++e) {
                float x = acc_full[base + s0 + e];
                out[o++] = divide ? x / (float)dp_size : x;
            }
            base += numel[i];
        }
    }
}

/* ------------------------------------------------------------------ */
/* O2c  clip coefficient                                               */
/* ------------------------------------------------------------------ */
/* READING: c = min(1, clip / (sqrt(S) + 1e-6)) as torch's clip_grad_norm_;
 * clip <= 0 disables clipping (c = 1). */
Z1O_EXPORT double z1o_clip_coef(double S, double clip)
{
    if (!(clip > 0.0))
        return 1.0;
    double c = clip / (sqrt(S) + 1e-6);
    return c >= 1.0 ? 1.0 : c; /* a clamp at 1: a NaN norm gives a NaN coefficient */
}

/* ------------------------------------------------------------------ */
/* O2d + O2e  AdamW on the fp32 shard, then the bf16 cast              */
/* ------------------------------------------------------------------ */
typedef struct z1o_hp {
    double lr, beta1, beta2, eps, weight_decay, clip;
    int64_t step; /* t, starting at 1 */
} z1o_hp;

/* [NG] ZeRO-1 section and [T6] §6.1: the optimizer keeps an fp32 master
 * copy and fp32 first/second moments per parameter; [T6] §6.6 and the [NG]
 * config give AdamW with beta1 0.9, beta2 0.95, eps 1e-8 and weight decay.
 * READING (PyTorch AdamW): the decay multiplies the previous master by
 * (1 - lr*wd); bias corrections use 1 - beta^t; eps is added outside the
 * square root.  Each element is computed in binary64 from the stored fp32
 * values and stored back rounded to binary32 (C's double->float conversion
 * rounds to nearest-even).  [T6] §6.3 / [NG]: the updated master is cast to
 * the bf16 working weight that the all-gather later distributes.
 *
 * Per-tensor multipliers: the packed shard is n_seg consecutive segments
 * (seg_len[j] elements each, summing to L); segment j uses
 * lr_j = lr * lr_scale[j] and wd_j = weight_decay * wd_scale[j]
 * ([NG] Spectral muP: eta_hidden = eta_0 / d_model; a zero wd_scale keeps a
 * tensor out of weight decay).  n_seg == 0 means one segment with both
 * multipliers 1. */
Z1O_EXPORT void z1o_adamw_seg(int64_t L, const float *acc, float *p, float *m, float *v,
                              uint16_t *w, double c, const z1o_hp *hp, int32_t n_seg,
                              const int64_t *seg_len, const double *lr_scale,
                              const double *wd_scale)
{
    const double t = (double)hp->step;
    const double bc1 = 1.0 - pow(hp->beta1, t);
    const double bc2 = 1.0 - pow(hp->beta2, t);
    int64_t seg_start = 0;
    for (int32_t j = 0; j < (n_seg > 0 ? n_seg : 1); ++j) {
        const int64_t seg_end = n_seg > 0 ? seg_start + seg_len[j] : L;
        const double lr = hp->lr * (n_seg > 0 ? lr_scale[j] : 1.0);
        const double wd = hp->weight_decay * (n_seg > 0 ? wd_scale[j] : 1.0);
#pragma omp parallel for schedule(static)
        for (int64_t e = seg_start; e < seg_end; ++e) {
            double g = c * (double)acc[e];
            double pe = (double)p[e];
            double me = (double)m[e];
            double ve = (double)v[e];
            pe = pe * (1.0 - lr * wd);
            me = hp->beta1 * me + (1.0 - hp->beta1) * g;
            ve = hp->beta2 * ve + (1.0 - hp->beta2) * g * g;
            double mhat = me / bc1;
            double vhat = ve / bc2;
            pe = pe - lr * mhat / (sqrt(vhat) + hp->eps);
            p[e] = (float)pe;
            m[e] = (float)me;
            v[e] = (float)ve;
            if (w)
                w[e] = z1o_bf16_rne(p[e]);
        }
        seg_start = seg_end;
    }
}

Z1O_EXPORT void z1o_adamw(int64_t L, const float *acc, float *p, float *m, float *v,
                          uint16_t *w, double c, const z1o_hp *hp)
{
    z1o_adamw_seg(L, acc, p, m, v, w, c, hp, 0, 0, 0, 0);
}

/* ------------------------------------------------------------------ */
/* Learning-rate schedule                                              */
/* ------------------------------------------------------------------ */
/* [NG] config: learning_rate (peak), lr_warmup_steps, lr_decay_steps,
 * min_decay_lr.  READING (the decay shape is not on the page): a linear
 * warmup reaching the peak at t = warmup, then over decay_steps a linear or
 * half-cosine decay to the minimum, then the minimum.  style: 0 none (peak
 * after warmup), 1 linear, 2 cosine. */
Z1O_EXPORT double z1o_lr_at(double lr_max, double lr_min, int64_t warmup, int64_t decay,
                            int32_t style, int64_t t)
{
    if (warmup > 0 && t <= warmup)
        return lr_max * (double)t / (double)warmup;
    if (style == 0)
        return lr_max;
    int64_t d = t - (warmup > 0 ? warmup : 0);
    if (d >= decay)
        return lr_min;
    double tau = (double)d / (double)decay;
    if (style == 1)
        return lr_max + (lr_min - lr_max) * tau;
    return lr_min + (lr_max - lr_min) * 0.5 * (1.0 + cos(M_PI * tau));
}

/* ------------------------------------------------------------------ */
/* One whole step: O2a -> O2b -> O2c -> O2d -> O2e                      */
/* ------------------------------------------------------------------ */
/* Returns S (before clipping); *c_out receives the clip coefficient. */
Z1O_EXPORT double z1o_step_seg(int64_t L, int32_t K, const uint16_t *g, float *acc,
                               float *p, float *m, float *v, uint16_t *w,
                               const z1o_hp *hp, double *c_out, int32_t n_seg,
                               const int64_t *seg_len, const double *lr_scale,
                               const double *wd_scale)
{
    z1o_accumulate(L, K, g, acc);
    double S = z1o_norm_sq(L, acc);
    double c = z1o_clip_coef(S, hp->clip);
    z1o_adamw_seg(L, acc, p, m, v, w, c, hp, n_seg, seg_len, lr_scale, wd_scale);
    if (c_out)
        *c_out = c;
    return S;
}

Z1O_EXPORT double z1o_step(int64_t L, int32_t K, const uint16_t *g, float *acc,
                           float *p, float *m, float *v, uint16_t *w,
                           const z1o_hp *hp, double *c_out)
{
    return z1o_step_seg(L, K, g, acc, p, m, v, w, hp, c_out, 0, 0, 0, 0);
}

Z1O_EXPORT int z1o_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
