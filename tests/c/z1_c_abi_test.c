/*
 * z1_c_abi_test.c -- drives libz1 from plain C (no Python, no torch): two
 * tiny optimizer steps through the C ABI, compared bit for bit with the CPU
 * oracle (test infrastructure, linked only here).  Exit status 0 = pass.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "z1.h"

/* oracle entry points (oracle/z1_oracle.c) */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay, clip;
    int64_t step;
} z1o_hp;
int z1o_shard_plan(int32_t, const int64_t *, int32_t, int32_t, int64_t *, int64_t *);
double z1o_step(int64_t, int32_t, const uint16_t *, float *, float *, float *, float *,
                uint16_t *, const z1o_hp *, double *);

#define CHECK_HIP(x)                                                              \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);      \
            return 2;                                                             \
        }                                                                         \
    } while (0)
#define CHECK_Z1(x)                                                               \
    do {                                                                          \
        z1_status s_ = (x);                                                       \
        if (s_ != Z1_OK) {                                                        \
            fprintf(stderr, "z1 error %s at line %d\n", z1_strerror(s_), __LINE__); \
            return 3;                                                             \
        }                                                                         \
    } while (0)

static uint64_t lcg = 88172645463325252ull;
static double uniform(void)
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return ((lcg >> 11) + 0.5) / 9007199254740992.0;
}
static float normal(double sigma)
{
    double u1 = uniform(), u2 = uniform();
    return (float)(sigma * sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}
static uint16_t bf16_trunc(float f) /* input generation only: any bf16 pattern will do */
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

enum { NT = 5, K = 3, D = 3, RANK = 2 };

int main(void)
{
    if (z1_abi_version() != Z1_ABI_VERSION) {
        fprintf(stderr, "library ABI %d, header ABI %d\n", (int)z1_abi_version(), Z1_ABI_VERSION);
        return 5;
    }
    const int64_t numel[NT] = {1000, 7, 4099, 1, 3000};
    int64_t start[NT], len[NT], off[NT], arena = 0;
    int64_t ostart[NT], olen[NT];
    CHECK_Z1(z1_shard_plan(NT, numel, D, RANK, start, len, off, &arena));
    if (z1o_shard_plan(NT, numel, D, RANK, ostart, olen) != 0)
        return 4;
    int64_t L = 0;
    for (int i = 0; i < NT; ++i) {
        if (start[i] != ostart[i] || len[i] != olen[i]) {
            fprintf(stderr, "plan differs at tensor %d\n", i);
            return 5;
        }
        L += len[i];
    }

    /* inputs: full bf16 tensors (weights zero, K gradients), fp32 master slices */
    void *w[NT], *g[K * NT];
    uint16_t *hg = malloc(sizeof(uint16_t) * K * L); /* packed, for the oracle */
    float *hp_ = malloc(sizeof(float) * L), *hm = calloc(L, 4), *hv = calloc(L, 4);
    float *hacc = malloc(sizeof(float) * L);
    uint16_t *hw = malloc(sizeof(uint16_t) * L);
    float *arena_host = calloc(arena, 4);
    int64_t pos = 0;
    for (int i = 0; i < NT; ++i) {
        CHECK_HIP(hipMalloc(&w[i], numel[i] * 2 + 16));
        CHECK_HIP(hipMemset(w[i], 0, numel[i] * 2 + 16));
        for (int64_t e = 0; e < len[i]; ++e) {
            float m = normal(0.02);
            hp_[pos + e] = m;
            arena_host[off[i] + e] = m;
        }
        pos += len[i];
    }
    for (int k = 0; k < K; ++k) {
        pos = 0;
        for (int i = 0; i < NT; ++i) {
            uint16_t *full = malloc(numel[i] * 2 + 2);
            for (int64_t e = 0; e < numel[i]; ++e)
                full[e] = bf16_trunc(normal(1e-2));
            memcpy(hg + (int64_t)k * L + pos, full + start[i], len[i] * 2);
            pos += len[i];
            CHECK_HIP(hipMalloc(&g[k * NT + i], numel[i] * 2 + 16));
            CHECK_HIP(hipMemcpy(g[k * NT + i], full, numel[i] * 2, hipMemcpyHostToDevice));
            free(full);
        }
    }
    float *d_master, *d_m, *d_v, *d_acc;
    double *d_S;
    CHECK_HIP(hipMalloc((void **)&d_master, arena * 4 + 16));
    CHECK_HIP(hipMalloc((void **)&d_m, arena * 4 + 16));
    CHECK_HIP(hipMalloc((void **)&d_v, arena * 4 + 16));
    CHECK_HIP(hipMalloc((void **)&d_acc, arena * 4 + 16));
    CHECK_HIP(hipMalloc((void **)&d_S, 8));
    CHECK_HIP(hipMemcpy(d_master, arena_host, arena * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(d_m, 0, arena * 4));
    CHECK_HIP(hipMemset(d_v, 0, arena * 4));

    z1_bind b;
    memset(&b, 0, sizeof b);
    b.n_tensors = NT;
    b.dp_size = D;
    b.rank = RANK;
    b.n_micro = K;
    b.numel = numel;
    b.weights = w;
    b.grads = (const void *const *)g;
    b.master = d_master;
    b.exp_avg = d_m;
    b.exp_avg_sq = d_v;
    b.acc = d_acc;
    b.arena_elems = arena;
    z1_plan *plan = NULL;
    CHECK_Z1(z1_plan_create(&plan, &b, NULL));
    /* the same gradients as packed bf16 shards in arena order, and a packed
     * weight shard whose padding holds a canary, bound to a second plan over
     * the same fp32 arenas (Z1_LAYOUT_PACKED) */
    void *gp[K], *wp = NULL;
    uint16_t *packed_host = malloc(arena * 2 + 16);
    for (int k = 0; k < K; ++k) {
        memset(packed_host, 0, arena * 2);
        pos = 0;
        for (int i = 0; i < NT; ++i) {
            memcpy(packed_host + off[i], hg + (int64_t)k * L + pos, len[i] * 2);
            pos += len[i];
        }
        CHECK_HIP(hipMalloc(&gp[k], arena * 2 + 16));
        CHECK_HIP(hipMemcpy(gp[k], packed_host, arena * 2, hipMemcpyHostToDevice));
    }
    CHECK_HIP(hipMalloc(&wp, arena * 2 + 16));
    CHECK_HIP(hipMemset(wp, 0x5A, arena * 2 + 16));
    z1_bind bp = b;
    bp.weights = (void *const *)&wp;
    bp.grads = (const void *const *)gp;
    bp.layout = Z1_LAYOUT_PACKED;
    z1_plan *plan_packed = NULL;
    CHECK_Z1(z1_plan_create(&plan_packed, &bp, NULL));

    /* step 4 runs through a one-row schedule (device constants for t = 4) */
    z1_schedule *sched = NULL;
    {
        z1_adamw_hp h4 = {1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, 4};
        CHECK_Z1(z1_schedule_create(&sched, &h4, NULL, 1, NULL));
    }

    /* step 1: one accumulation call per micro-batch; step 2: all K resident
     * slots in one z1_accum_grads_range call; step 3: the packed layout;
     * step 4: the scheduled AdamW.  Each must match the oracle. */
    int bad = 0;
    double S = 0.0, S_gpu = 0.0, c = 0.0;
    float *back = malloc(arena * 4);
    for (int t = 1; t <= 4; ++t) {
        z1_adamw_hp hp = {1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, t};
        z1_plan *pl = t == 3 ? plan_packed : plan;
        if (t == 1) {
            for (int k = 0; k < K; ++k)
                CHECK_Z1(z1_accum_grads(pl, k, NULL));
        } else {
            CHECK_Z1(z1_accum_grads_range(pl, 0, K, NULL));
        }
        CHECK_Z1(z1_grad_norm_sq(pl, d_S, NULL));
        if (t == 2) {
            /* the norm as an unrounded pair, combined over one rank: the same S */
            double *d_pair = NULL, *d_S1 = NULL, S_a = 0.0, S_b = 1.0;
            CHECK_HIP(hipMalloc((void **)&d_pair, 16));
            CHECK_HIP(hipMalloc((void **)&d_S1, 8));
            CHECK_Z1(z1_grad_norm_sq_pair(pl, d_pair, NULL));
            CHECK_Z1(z1_norm_combine(d_pair, 1, d_S1, NULL));
            CHECK_HIP(hipMemcpy(&S_a, d_S, 8, hipMemcpyDeviceToHost));
            CHECK_HIP(hipMemcpy(&S_b, d_S1, 8, hipMemcpyDeviceToHost));
            bad += memcmp(&S_a, &S_b, 8) != 0;
            CHECK_HIP(hipFree(d_pair));
            CHECK_HIP(hipFree(d_S1));
        }
        if (t == 4)
            CHECK_Z1(z1_adamw_step_scheduled(pl, sched, d_S, NULL));
        else
            CHECK_Z1(z1_adamw_step(pl, &hp, d_S, NULL));
        CHECK_HIP(hipDeviceSynchronize());

        z1o_hp ohp = {1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, t};
        S = z1o_step(L, K, hg, hacc, hp_, hm, hv, hw, &ohp, &c);
        CHECK_HIP(hipMemcpy(&S_gpu, d_S, 8, hipMemcpyDeviceToHost));
        bad += S_gpu != S;
        const float *refs[4] = {hp_, hm, hv, hacc};
        float *devs[4] = {d_master, d_m, d_v, d_acc};
        for (int a = 0; a < 4; ++a) {
            CHECK_HIP(hipMemcpy(back, devs[a], arena * 4, hipMemcpyDeviceToHost));
            pos = 0;
            for (int i = 0; i < NT; ++i) {
                bad += memcmp(back + off[i], refs[a] + pos, len[i] * 4) != 0;
                pos += len[i];
            }
        }
        pos = 0;
        if (t == 3) {
            CHECK_HIP(hipMemcpy(packed_host, wp, arena * 2, hipMemcpyDeviceToHost));
            int64_t used = 0;
            for (int i = 0; i < NT; ++i) {
                bad += memcmp(packed_host + off[i], hw + pos, len[i] * 2) != 0;
                pos += len[i];
                used += len[i];
            }
            int64_t canaries = 0;
            for (int64_t e = 0; e < arena; ++e)
                canaries += packed_host[e] == 0x5A5A;
            bad += canaries != arena - used; /* padding: untouched */
        }
        for (int i = 0; i < NT && t != 3; ++i) {
            uint16_t *full = malloc(numel[i] * 2 + 2);
            CHECK_HIP(hipMemcpy(full, w[i], numel[i] * 2, hipMemcpyDeviceToHost));
            bad += memcmp(full + start[i], hw + pos, len[i] * 2) != 0;
            for (int64_t e = 0; e < numel[i]; ++e)
                if ((e < start[i] || e >= start[i] + len[i]) && full[e] != 0)
                    ++bad; /* outside the slice: untouched */
            pos += len[i];
            free(full);
        }
        printf("C ABI step %d (%s): L=%lld S=%.17g (oracle %.17g) c=%.6g bad=%d\n", t,
               t == 1   ? "z1_accum_grads per micro-batch"
               : t == 2 ? "z1_accum_grads_range"
               : t == 3 ? "packed layout, range"
                        : "scheduled AdamW",
               (long long)L, S_gpu, S, c, bad);
    }
    free(back);
    int64_t next_step = 0, overrun = -1;
    CHECK_Z1(z1_schedule_query(sched, &next_step, &overrun));
    bad += next_step != 5 || overrun != 0;
    printf("C ABI schedule: next step %lld, overrun %lld\n", (long long)next_step,
           (long long)overrun);
    CHECK_Z1(z1_schedule_destroy(sched));
    CHECK_Z1(z1_plan_destroy(plan));
    CHECK_Z1(z1_plan_destroy(plan_packed));
    printf("C ABI: %s\n", bad ? "MISMATCH" : "bit-exact");
    return bad ? 1 : 0;
}
