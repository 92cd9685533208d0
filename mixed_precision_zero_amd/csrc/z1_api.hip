// z1_api.hip -- host side of the C ABI declared in include/z1.h: argument
// validation, the shard plan, the chunk table, call-order state and the
// kernel launches.  Everything device-side is in z1_kernels.hip.
#define _USE_MATH_DEFINES
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <memory>
#include <mutex>
#include <new>
#include <vector>

#include "z1.h"
#include "z1_internal.h"

using z1::AdamConsts;
using z1::Chunk;
using z1::DD;

struct z1_plan {
    int device = -1;  // the GPU current at creation; every call must run there
    int32_t n = 0, K = 0, dp = 0, rank = 0;
    int64_t L = 0, arena_elems = 0, chunk_elems = 0, n_chunks = 0;
    int grid = 0;
    int32_t sub = 1;        // one-wave workgroups per piece (AdamW, wide slot passes)
    int64_t n_partials = 0; // norm partials the last accumulation or norm pass left
    int64_t adam_grid = 0;  // AdamW's chunk-walk grid
    uint32_t adam_lds = 0;  // LDS reserved per AdamW workgroup
    std::vector<int64_t> start, len, arena_off;
    std::vector<const uint16_t *> gbase;  // packed plans: the K gradient shards, arena-indexed
    // device memory owned by the plan
    Chunk *d_chunks = nullptr;
    const uint16_t **d_grads = nullptr;  // [K][n]
    uint16_t **d_weights = nullptr;      // [n]
    DD *d_partials = nullptr;            // [n_chunks]
    DD *d_stage = nullptr;               // [kFinStages] second-level norm partials
    unsigned int *d_counter = nullptr;   // norm reduction arrival counter (zero between launches)
    z1::Scale *d_scales = nullptr;       // [n] per-tensor lr / weight-decay multipliers
    // AdamW's arena walk (n_tiles == 0 when AdamW walks the chunk table)
    int32_t *d_tags = nullptr;           // [n_tiles]
    Chunk *d_segs = nullptr;             // [n_segs]
    int64_t *d_wdelta = nullptr;         // [n] full-size bf16 layout: ArenaWalk::wdelta
    int64_t n_tiles = 0, n_full = 0, n_segs = 0, n_boundary = 0;
    uint16_t *wbase = nullptr;
    // caller's arenas
    float *master = nullptr, *exp_avg = nullptr, *exp_avg_sq = nullptr, *acc = nullptr;
    // call order: next micro-batch index expected; norm enqueued since the last pass
    int32_t next_k = 0;
    bool acc_complete = false;
    bool norm_done = false;
};

struct z1_schedule {
    int device = -1;
    int64_t t_first = 1, n_steps = 0;
    bool clipping = false;
    AdamConsts *d_table = nullptr;  // [n_steps] constants of steps t_first ...
    int64_t *d_state = nullptr;     // [0] next row, [1] scheduled steps asked for past the end
};

struct z1_pack {
    int device = -1;
    int32_t n = 0, K = 0, dp = 0;
    int64_t seg = 0, n_chunks = 0;
    int32_t sub = 1;  // one-wave workgroups per piece of a wide slot pass
    bool divide = false;
    float *send = nullptr;
    Chunk *d_chunks = nullptr;
    const uint16_t **d_grads = nullptr;  // [K][n]
    int32_t next_k = 0;
};

// --------------------------------------------------------------------------
// Scratch of the entry point that allocates nothing (z1_grad_norm_sq_flat_noalloc):
// the per-tile norm partials, the finalise's second-level stage and its
// arrival counter, in one file-scope device array.  Each GPU the library runs
// on holds its own copy until the process ends; every call on a GPU shares it.
constexpr int64_t kFlatMaxTiles = Z1_NORM_FLAT_MAX_ELEMS / z1::kTileElems;
constexpr size_t kScratchPartials = (size_t)kFlatMaxTiles * sizeof(DD);  // 4 MiB
constexpr size_t kScratchStage = (size_t)z1::kFinStages * sizeof(DD);     // 4 KiB
constexpr size_t kScratchBytes = kScratchPartials + kScratchStage + 256;  // + counter
static_assert(Z1_NORM_FLAT_MAX_ELEMS % z1::kTileElems == 0, "whole tiles");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on each GPU, resolved once per GPU (with that
// GPU current) by hipGetSymbolAddress: in host code the array's name stands
// for a host-side placeholder, never for device memory.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

void *scratch_on(int dev)
{
    if (dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The GPU current on the calling thread, -1 if HIP reports none.
int current_device()
{
    int d = -1;
    if (hipGetDevice(&d) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return d;
}

// True when `stream` is a stream of GPU `dev`.  NULL and the legacy /
// per-thread default handles always name a stream of the current GPU.
bool stream_on(int dev, z1_stream stream)
{
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!s || s == hipStreamLegacy || s == hipStreamPerThread)
        return current_device() == dev;
    hipDevice_t d = -1;
    if (hipStreamGetDevice(s, &d) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return d == dev;
}

// True when p is device memory of GPU `dev` (or managed memory), as the HIP
// runtime records it; host memory, unknown pointers and another GPU's memory
// are not.
bool device_memory_on(int dev, const void *ptr)
{
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, ptr) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) && a.device == dev;
}

// A call on an object created on GPU `owner` may enqueue work only with that
// GPU current and on one of its streams; otherwise its kernels would run on
// another GPU with this one's pointers.
bool on_owner(int owner, z1_stream stream)
{
    return current_device() == owner && stream_on(owner, stream);
}

// Makes GPU `dev` current for the scope and restores the previous one
// (destroy and query calls, which any thread may make).
class DeviceScope {
  public:
    explicit DeviceScope(int dev) : prev_(current_device())
    {
        if (dev >= 0 && prev_ >= 0 && dev != prev_ && hipSetDevice(dev) != hipSuccess) {
            (void)hipGetLastError();
            prev_ = -1;
        }
        switched_ = dev >= 0 && prev_ >= 0 && dev != prev_;
    }
    ~DeviceScope()
    {
        if (switched_)
            (void)hipSetDevice(prev_);
    }

  private:
    int prev_;
    bool switched_ = false;
};

void free_plan_memory(z1_plan *p)
{
    if (p->d_chunks)
        (void)hipFree(p->d_chunks);
    if (p->d_grads)
        (void)hipFree(p->d_grads);
    if (p->d_weights)
        (void)hipFree(p->d_weights);
    if (p->d_partials)
        (void)hipFree(p->d_partials);
    if (p->d_stage)
        (void)hipFree(p->d_stage);
    if (p->d_counter)
        (void)hipFree(p->d_counter);
    if (p->d_scales)
        (void)hipFree(p->d_scales);
    if (p->d_tags)
        (void)hipFree(p->d_tags);
    if (p->d_segs)
        (void)hipFree(p->d_segs);
    if (p->d_wdelta)
        (void)hipFree(p->d_wdelta);
    p->d_wdelta = nullptr;
    p->d_scales = nullptr;
    p->d_tags = nullptr;
    p->d_segs = nullptr;
    p->d_stage = nullptr;
    p->d_counter = nullptr;
    p->d_chunks = nullptr;
    p->d_grads = nullptr;
    p->d_weights = nullptr;
    p->d_partials = nullptr;
}

// Owners of a plan or pack under construction: on any early return (or an
// exception) the device memory allocated so far is released.
struct PlanDeleter {
    void operator()(z1_plan *p) const
    {
        if (p->d_chunks || p->d_grads || p->d_weights || p->d_partials || p->d_stage ||
            p->d_counter || p->d_scales || p->d_tags || p->d_segs || p->d_wdelta)
            (void)hipDeviceSynchronize();  // an upload may still be in flight
        free_plan_memory(p);
        delete p;
    }
};

struct PackDeleter {
    void operator()(z1_pack *p) const
    {
        if (p->d_chunks || p->d_grads)
            (void)hipDeviceSynchronize();
        if (p->d_chunks)
            (void)hipFree(p->d_chunks);
        if (p->d_grads)
            (void)hipFree(p->d_grads);
        delete p;
    }
};

// Runs the body of an entry point that builds host tables.  The only
// operations in those bodies that can throw are host allocations
// (std::vector growth), so any exception means the host ran out of memory;
// it becomes Z1_ENOMEM and never crosses the C interface.
template <typename F>
z1_status no_throw(F &&body)
{
    try {
        return body();
    } catch (...) {
        return Z1_ENOMEM;
    }
}

template <typename T>
z1_status device_alloc(T **out, size_t count)
{
    *out = nullptr;
    if (count == 0)
        count = 1;  // keep a valid pointer for empty tables
    void *p = nullptr;
    if (hipMalloc(&p, count * sizeof(T)) != hipSuccess) {
        (void)hipGetLastError();
        return Z1_ENOMEM;
    }
    *out = static_cast<T *>(p);
    return Z1_OK;
}

z1::LaunchGeom geom(const z1_plan *p)
{
    z1::LaunchGeom g{p->d_chunks, p->n_chunks, p->grid};
    g.sub = p->sub;
    g.adam_grid = p->adam_grid;
    g.adam_lds = p->adam_lds;
    if (p->n_tiles > 0) {
        g.arena.tags = p->d_tags;
        g.arena.segs = p->d_segs;
        g.arena.n_tiles = p->n_tiles;
        g.arena.n_full = p->n_full;
        g.arena.n_segs = p->n_segs;
        g.arena.wbase = p->wbase;
        g.arena.wdelta = p->d_wdelta;
    }
    return g;
}

// The arena walk of a plan (AdamW's, and in packed plans the single and wide
// accumulation passes'): tile j covers arena elements [j * T, (j + 1) * T)
// with T = kAdamBlockElems (one one-wave workgroup's block).  tags[j] is the
// tensor whose slice holds the whole tile, -1 for a tile that crosses a slice
// boundary or the arena's end (and for a tile no slice touches); the parts
// of slices in such tiles become segments in the chunk table's format (src, dst, tensor,
// count), in arena order.  Padding between slices is in no segment.
void arena_walk(int32_t n, const int64_t *start, const int64_t *len, const int64_t *arena_off,
                int64_t arena_elems, std::vector<int32_t> &tags, std::vector<Chunk> &segs,
                int64_t &n_full, int64_t &n_boundary)
{
    const int64_t T = z1::kAdamBlockElems;
    const int64_t n_tiles = (arena_elems + T - 1) / T;
    n_full = arena_elems / T;
    tags.assign((size_t)n_tiles, -1);
    segs.clear();
    for (int32_t i = 0; i < n; ++i) {
        if (len[i] == 0)
            continue;
        const int64_t a = arena_off[i], e = a + len[i];
        for (int64_t j = a / T; j * T < e; ++j) {
            const int64_t lo = a > j * T ? a : j * T;
            const int64_t hi = e < (j + 1) * T ? e : (j + 1) * T;
            if (lo == j * T && hi == (j + 1) * T && j < n_full) {
                tags[(size_t)j] = i;
                continue;
            }
            Chunk c;
            c.src = start[i] + (lo - a);
            c.dst = lo;
            c.tensor = i;
            c.count = (int32_t)(hi - lo);
            c.pad = 0;
            segs.push_back(c);
        }
    }
    n_boundary = 0;
    for (int32_t t : tags)
        n_boundary += t < 0;
}

// Appends the pieces of slices [start[i], start[i]+len[i]) of tensors 0..n-1,
// cut at multiples of `chunk` inside each tensor; element e of slice i lands
// at dst_base + arena_off[i] + e.  The table stays in this (tensor) order;
// each kernel picks its own issue order over it on the device.
void append_chunks(std::vector<Chunk> &chunks, int32_t n, const int64_t *start, const int64_t *len,
                   const int64_t *arena_off, int64_t dst_base, int64_t chunk)
{
    for (int32_t i = 0; i < n; ++i) {
        const int64_t s0 = start[i], s1 = start[i] + len[i];
        int64_t s = s0;
        while (s < s1) {
            const int64_t cut = (s / chunk + 1) * chunk;
            const int64_t e = cut < s1 ? cut : s1;
            Chunk c;
            c.src = s;
            c.dst = dst_base + arena_off[i] + (s - s0);
            c.tensor = i;
            c.count = (int32_t)(e - s);
            c.pad = 0;
            chunks.push_back(c);
            s = e;
        }
    }
}

int64_t chunk_or_default(int64_t c) { return c ? c : z1::kDefaultChunk; }

bool hp_ok(const z1_adamw_hp *hp)
{
    return isfinite(hp->lr) && hp->beta1 >= 0.0 && hp->beta1 < 1.0 && hp->beta2 >= 0.0 &&
           hp->beta2 < 1.0 && hp->eps > 0.0 && isfinite(hp->eps) && hp->weight_decay >= 0.0 &&
           isfinite(hp->weight_decay) && !isnan(hp->clip) && hp->step >= 1;
}

// The binary64 constants of one step, derived on the host (bias corrections
// from libm pow, as the oracle derives them, and their reciprocals, which the
// kernels divide by exactly).
AdamConsts consts_of(const z1_adamw_hp *hp)
{
    AdamConsts k;
    const double t = (double)hp->step;
    k.lr = hp->lr;
    k.beta1 = hp->beta1;
    k.beta2 = hp->beta2;
    k.omb1 = 1.0 - hp->beta1;
    k.omb2 = 1.0 - hp->beta2;
    k.eps = hp->eps;
    k.weight_decay = hp->weight_decay;
    k.bc1 = 1.0 - pow(hp->beta1, t);
    k.bc2 = 1.0 - pow(hp->beta2, t);
    k.rbc1 = 1.0 / k.bc1;
    k.rbc2 = 1.0 / k.bc2;
    k.clip = hp->clip > 0.0 ? hp->clip : 0.0;
    return k;
}
bool chunk_ok(int64_t c) { return c >= 1024 && c <= z1::kMaxChunk && c % 1024 == 0; }

}  // namespace

extern "C" {

int32_t z1_abi_version(void) { return Z1_ABI_VERSION; }

const char *z1_strerror(z1_status s)
{
    switch (s) {
    case Z1_OK: return "success";
    case Z1_EINVAL: return "invalid argument";
    case Z1_EALIGN: return "device pointer not aligned";
    case Z1_ENOMEM: return "out of memory";
    case Z1_EHIP: return "HIP runtime error";
    case Z1_ESTATE: return "call out of order";
    }
    return "unknown status";
}

z1_status z1_shard_plan_kind(int32_t kind, int32_t n_tensors, const int64_t *numel,
                             const int64_t *rows, int32_t dp_size, int32_t rank,
                             int64_t *start, int64_t *len, int64_t *arena_off,
                             int64_t *arena_elems)
{
    if (n_tensors < 0 || dp_size < 1 || rank < 0 || rank >= dp_size || !arena_elems)
        return Z1_EINVAL;
    if (kind != Z1_PLAN_PER_TENSOR && kind != Z1_PLAN_FLAT && kind != Z1_PLAN_DIM0)
        return Z1_EINVAL;
    if (n_tensors > 0 && (!numel || !start || !len || !arena_off))
        return Z1_EINVAL;
    if (n_tensors > 0 && kind == Z1_PLAN_DIM0 && !rows)
        return Z1_EINVAL;
    int64_t total = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (numel[i] < 0 || total > INT64_MAX - numel[i])
            return Z1_EINVAL;
        total += numel[i];
        if (kind == Z1_PLAN_DIM0 &&
            (rows[i] < 0 || (rows[i] == 0 && numel[i] != 0) ||
             (rows[i] > 0 && numel[i] % rows[i] != 0)))
            return Z1_EINVAL;
    }
    // the rank's range of the concatenation (flat kind)
    const int64_t fq = total / dp_size, frho = total % dp_size;
    const int64_t flo = (int64_t)rank * fq + (rank < frho ? rank : frho);
    const int64_t fhi = flo + fq + (rank < frho ? 1 : 0);
    int64_t base = 0;  // tensor i's first element in the concatenation
    int64_t next = 0;  // first free arena element
    for (int32_t i = 0; i < n_tensors; ++i) {
        int64_t s0 = 0, ln = 0;
        if (kind == Z1_PLAN_PER_TENSOR) {
            const int64_t q = numel[i] / dp_size, rho = numel[i] % dp_size;
            const int64_t extra = rank < rho ? 1 : 0;
            s0 = (int64_t)rank * q + (extra ? rank : rho);
            ln = q + extra;
        } else if (kind == Z1_PLAN_FLAT) {
            const int64_t a = flo > base ? flo : base;
            const int64_t e = fhi < base + numel[i] ? fhi : base + numel[i];
            if (a < e) {
                s0 = a - base;
                ln = e - a;
            }
        } else {
            const int64_t row_len = rows[i] ? numel[i] / rows[i] : 0;
            const int64_t per = (rows[i] + dp_size - 1) / dp_size;
            int64_t r0 = (int64_t)rank * per, r1 = r0 + per;
            if (r0 > rows[i])
                r0 = rows[i];
            if (r1 > rows[i])
                r1 = rows[i];
            ln = (r1 - r0) * row_len;
            s0 = ln ? r0 * row_len : 0;
        }
        base += numel[i];
        start[i] = s0;
        len[i] = ln;
        // smallest offset >= next with the slice start's residue mod 64: the
        // pieces cut at multiples of chunk_elems inside the tensor then start
        // on a 128-byte line of every fp32 arena and packed bf16 shard, so no
        // line is split between two workgroups.  (Measured on a ragged list:
        // matching only mod 8 made AdamW 7-8% slower; mod 32, which leaves
        // packed bf16 pieces 64 bytes into a line, made the packed
        // accumulation 5% slower.)
        const int64_t R = z1::kArenaResidue;
        const int64_t off = next + (((s0 - next) % R) + R) % R;
        arena_off[i] = off;
        next = off + ln;
    }
    *arena_elems = next;
    return Z1_OK;
}

z1_status z1_shard_plan(int32_t n_tensors, const int64_t *numel, int32_t dp_size, int32_t rank,
                        int64_t *start, int64_t *len, int64_t *arena_off, int64_t *arena_elems)
{
    return z1_shard_plan_kind(Z1_PLAN_PER_TENSOR, n_tensors, numel, nullptr, dp_size, rank,
                              start, len, arena_off, arena_elems);
}

z1_status z1_lr_at(const z1_lr_schedule *sc, int64_t t, double *lr)
{
    if (!sc || !lr || t < 0 || sc->warmup_steps < 0 || sc->decay_steps < 0 ||
        sc->reserved != 0 ||
        (sc->decay_style != Z1_DECAY_NONE && sc->decay_style != Z1_DECAY_LINEAR &&
         sc->decay_style != Z1_DECAY_COSINE))
        return Z1_EINVAL;
    const int64_t W = sc->warmup_steps;
    if (W > 0 && t <= W) {
        *lr = sc->lr_max * (double)t / (double)W;
        return Z1_OK;
    }
    if (sc->decay_style == Z1_DECAY_NONE) {
        *lr = sc->lr_max;
        return Z1_OK;
    }
    const int64_t d = t - W;
    if (d >= sc->decay_steps) {
        *lr = sc->lr_min;
        return Z1_OK;
    }
    const double tau = (double)d / (double)sc->decay_steps;
    if (sc->decay_style == Z1_DECAY_LINEAR)
        *lr = sc->lr_max + (sc->lr_min - sc->lr_max) * tau;
    else
        *lr = sc->lr_min + (sc->lr_max - sc->lr_min) * 0.5 * (1.0 + cos(M_PI * tau));
    return Z1_OK;
}

static z1_status plan_create_body(z1_plan **out, const z1_bind *b, z1_stream stream)
{
    if (!out)
        return Z1_EINVAL;
    *out = nullptr;
    if (!b || b->n_tensors < 0 || b->n_micro < 1 || b->dp_size < 1 || b->rank < 0 ||
        b->rank >= b->dp_size || b->max_blocks < 0 ||
        (b->layout != Z1_LAYOUT_FULL && b->layout != Z1_LAYOUT_PACKED))
        return Z1_EINVAL;
    if (b->walk != Z1_WALK_AUTO && b->walk != Z1_WALK_CHUNKS && b->walk != Z1_WALK_ARENA_TILES)
        return Z1_EINVAL;
    if (b->walk == Z1_WALK_ARENA_TILES && b->max_blocks > 0)
        return Z1_EINVAL;
    const int32_t n = b->n_tensors, K = b->n_micro;
    if (n > 0 && (!b->numel || !b->weights || !b->grads))
        return Z1_EINVAL;
    if (!b->master || !b->exp_avg || !b->exp_avg_sq || !b->acc)
        return Z1_EINVAL;
    const int64_t chunk = chunk_or_default(b->chunk_elems);
    if (!chunk_ok(chunk))
        return Z1_EINVAL;

    std::unique_ptr<z1_plan, PlanDeleter> owner(new (std::nothrow) z1_plan());
    z1_plan *p = owner.get();
    if (!p)
        return Z1_ENOMEM;
    p->n = n;
    p->K = K;
    p->dp = b->dp_size;
    p->rank = b->rank;
    p->chunk_elems = chunk;
    p->start.resize(n);
    p->len.resize(n);
    p->arena_off.resize(n);
    z1_status st = z1_shard_plan_kind(b->plan_kind, n, b->numel, b->rows, b->dp_size, b->rank,
                                      p->start.data(), p->len.data(), p->arena_off.data(),
                                      &p->arena_elems);
    if (st != Z1_OK)
        return st;
    if (b->arena_elems < p->arena_elems)
        return Z1_EINVAL;

    // per-tensor lr / weight-decay multipliers
    std::vector<z1::Scale> scales(n > 0 ? n : 1, z1::Scale{1.0, 1.0});
    for (int32_t i = 0; i < n; ++i) {
        const double ls = b->lr_scale ? b->lr_scale[i] : 1.0;
        const double ws = b->wd_scale ? b->wd_scale[i] : 1.0;
        if (!isfinite(ls) || !isfinite(ws) || ws < 0.0)
            return Z1_EINVAL;
        scales[i] = z1::Scale{ls, ws};
    }

    // pointers: non-null for tensors this rank touches, 16-byte aligned
    std::vector<uint16_t *> wptr(n);
    std::vector<const uint16_t *> gptr((size_t)K * n);
    const bool packed = b->layout == Z1_LAYOUT_PACKED;
    int64_t shard_elems = 0;
    for (int32_t i = 0; i < n; ++i)
        shard_elems += p->len[i];
    if (packed && shard_elems > 0) {
        // one shard buffer per role; tensor i's pointer is placed so that
        // element start[i] + e lands on arena element arena_off[i] + e
        // (arena_off[i] - start[i] is a multiple of 64: 128-byte aligned)
        const void *wbase = b->weights[0];
        if (!wbase)
            return Z1_EINVAL;
        if (!aligned(wbase, 16))
            return Z1_EALIGN;
        p->wbase = static_cast<uint16_t *>(const_cast<void *>(wbase));
        for (int32_t k = 0; k < K; ++k) {
            if (!b->grads[k])
                return Z1_EINVAL;
            if (!aligned(b->grads[k], 16))
                return Z1_EALIGN;
            p->gbase.push_back(static_cast<const uint16_t *>(b->grads[k]));
        }
        auto at = [&](const void *base, int32_t i) {
            return reinterpret_cast<uintptr_t>(base) +
                   (uintptr_t)(2 * (p->arena_off[i] - p->start[i]));
        };
        for (int32_t i = 0; i < n; ++i) {
            wptr[i] = reinterpret_cast<uint16_t *>(at(wbase, i));
            for (int32_t k = 0; k < K; ++k)
                gptr[(size_t)k * n + i] = reinterpret_cast<const uint16_t *>(at(b->grads[k], i));
        }
    }
    for (int32_t i = 0; i < n && !packed; ++i) {
        wptr[i] = static_cast<uint16_t *>(b->weights[i]);
        for (int32_t k = 0; k < K; ++k)
            gptr[(size_t)k * n + i] = static_cast<const uint16_t *>(b->grads[(size_t)k * n + i]);
        if (p->len[i] == 0)
            continue;
        if (!wptr[i])
            return Z1_EINVAL;
        if (!aligned(wptr[i], 16))
            return Z1_EALIGN;
        for (int32_t k = 0; k < K; ++k) {
            const void *g = gptr[(size_t)k * n + i];
            if (!g)
                return Z1_EINVAL;
            if (!aligned(g, 16))
                return Z1_EALIGN;
        }
    }
    if (!aligned(b->master, 16) || !aligned(b->exp_avg, 16) || !aligned(b->exp_avg_sq, 16) ||
        !aligned(b->acc, 16)) {
        return Z1_EALIGN;
    }
    p->master = b->master;
    p->exp_avg = b->exp_avg;
    p->exp_avg_sq = b->exp_avg_sq;
    p->acc = b->acc;

    // chunk table: pieces cut at multiples of `chunk` inside each tensor
    std::vector<Chunk> chunks;
    for (int32_t i = 0; i < n; ++i)
        p->L += p->len[i];
    append_chunks(chunks, n, p->start.data(), p->len.data(), p->arena_off.data(), 0, chunk);
    p->n_chunks = (int64_t)chunks.size();
    if (p->n_chunks > INT32_MAX)
        return Z1_EINVAL;
    int64_t grid = p->n_chunks;
    if (b->max_blocks > 0 && grid > b->max_blocks)
        grid = b->max_blocks;
    p->grid = (int)(grid > 0 ? grid : 1);
    // AdamW: chunk / kAdamBlockElems one-wave workgroups per piece; a capped
    // grid keeps the lanes of max_blocks 256-lane workgroups
    p->sub = (int32_t)(chunk / z1::kAdamBlockElems);
    int64_t adam_grid = p->n_chunks * p->sub;
    if (b->max_blocks > 0 && adam_grid > (int64_t)b->max_blocks * (z1::kBlock / z1::kWave))
        adam_grid = (int64_t)b->max_blocks * (z1::kBlock / z1::kWave);
    if (adam_grid > INT32_MAX)
        adam_grid = INT32_MAX;
    p->adam_grid = adam_grid > 0 ? adam_grid : 1;

    // AdamW's arena walk: forced, or chosen for a plan whose tiles cross
    // slice boundaries rarely (at most 1 in 100; the loads such a tile issues
    // before reading its tag are wasted).  With full-size bf16 tensors a
    // tile's bf16 store address comes from its tensor's entry of a
    // per-tensor table, read with the tag (7B shard: 1.2-2.2% faster than
    // the chunk walk over the same buffers, three processes).
    std::vector<int32_t> tags;
    std::vector<Chunk> segs;
    std::vector<int64_t> wdelta;
    if (b->max_blocks == 0 && b->walk != Z1_WALK_CHUNKS && p->arena_elems > 0) {
        int64_t n_full = 0, n_boundary = 0;
        arena_walk(n, p->start.data(), p->len.data(), p->arena_off.data(), p->arena_elems, tags,
                   segs, n_full, n_boundary);
        const int64_t n_tiles = (int64_t)tags.size();
        const bool fits = n_tiles + (int64_t)segs.size() <= INT32_MAX;
        if (b->walk == Z1_WALK_ARENA_TILES && !fits)
            return Z1_EINVAL;
        if (fits && (b->walk == Z1_WALK_ARENA_TILES || n_boundary * 100 <= n_tiles)) {
            p->n_tiles = n_tiles;
            p->n_full = n_full;
            p->n_segs = (int64_t)segs.size();
            p->n_boundary = n_boundary;
        }
    }
    if (p->n_tiles == 0) {
        tags.clear();
        segs.clear();
    } else if (!packed) {
        // byte address of arena element 0 as slice i maps it: element e of
        // the slice (arena position arena_off_i + e) is tensor element
        // start_i + e, so its address is wdelta[i] + 2 (arena_off_i + e)
        wdelta.resize((size_t)n, 0);
        for (int32_t i = 0; i < n; ++i)
            wdelta[(size_t)i] = (int64_t)reinterpret_cast<uintptr_t>(wptr[(size_t)i]) +
                                2 * (p->start[(size_t)i] - p->arena_off[(size_t)i]);
    }

    if ((p->device = current_device()) < 0)
        return Z1_EHIP;
    if (!stream_on(p->device, stream))
        return Z1_EINVAL;
    int lds_per_cu = 0;
    if (hipDeviceGetAttribute(&lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              p->device) != hipSuccess || lds_per_cu < 0)
        return Z1_EHIP;
    p->adam_lds = (uint32_t)(lds_per_cu / (p->n_tiles > 0 ? z1::kAdamPerCUTiles
                                                           : z1::kAdamPerCUChunks));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if ((st = device_alloc(&p->d_chunks, chunks.size())) != Z1_OK ||
        (st = device_alloc(&p->d_grads, gptr.size())) != Z1_OK ||
        (st = device_alloc(&p->d_weights, wptr.size())) != Z1_OK ||
        (st = device_alloc(&p->d_partials, (size_t)std::max(p->n_chunks * p->sub,
                                                            p->n_tiles + p->n_segs))) != Z1_OK ||
        (st = device_alloc(&p->d_stage, (size_t)z1::kFinStages)) != Z1_OK ||
        (st = device_alloc(&p->d_scales, scales.size())) != Z1_OK ||
        (st = device_alloc(&p->d_counter, 1)) != Z1_OK ||
        (p->n_tiles > 0 && ((st = device_alloc(&p->d_tags, tags.size())) != Z1_OK ||
                            (st = device_alloc(&p->d_segs, segs.size())) != Z1_OK)) ||
        (!wdelta.empty() && (st = device_alloc(&p->d_wdelta, wdelta.size())) != Z1_OK)) {
        return st;
    }
    hipError_t e = hipSuccess;
    if (!chunks.empty())
        e = hipMemcpyAsync(p->d_chunks, chunks.data(), chunks.size() * sizeof(Chunk),
                           hipMemcpyHostToDevice, s);
    if (e == hipSuccess && !gptr.empty())
        e = hipMemcpyAsync(p->d_grads, gptr.data(), gptr.size() * sizeof(void *),
                           hipMemcpyHostToDevice, s);
    if (e == hipSuccess && !wptr.empty())
        e = hipMemcpyAsync(p->d_weights, wptr.data(), wptr.size() * sizeof(void *),
                           hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(p->d_scales, scales.data(), scales.size() * sizeof(z1::Scale),
                           hipMemcpyHostToDevice, s);
    if (e == hipSuccess && !tags.empty())
        e = hipMemcpyAsync(p->d_tags, tags.data(), tags.size() * sizeof(int32_t),
                           hipMemcpyHostToDevice, s);
    if (e == hipSuccess && !segs.empty())
        e = hipMemcpyAsync(p->d_segs, segs.data(), segs.size() * sizeof(Chunk),
                           hipMemcpyHostToDevice, s);
    if (e == hipSuccess && !wdelta.empty())
        e = hipMemcpyAsync(p->d_wdelta, wdelta.data(), wdelta.size() * sizeof(int64_t),
                           hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipMemsetAsync(p->d_counter, 0, sizeof(unsigned int), s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);  // host staging vectors die with this call
    if (e != hipSuccess) {
        (void)hipStreamSynchronize(s);  // no upload may still read them
        (void)hipGetLastError();
        return Z1_EHIP;
    }
    *out = owner.release();
    return Z1_OK;
}

z1_status z1_plan_destroy(z1_plan *p)
{
    if (!p)
        return Z1_OK;
    DeviceScope on(p->device);
    (void)hipDeviceSynchronize();
    free_plan_memory(p);
    delete p;
    return Z1_OK;
}

z1_status z1_plan_query(const z1_plan *p, z1_plan_info *info)
{
    if (!p || !info)
        return Z1_EINVAL;
    info->n_tensors = p->n;
    info->n_micro = p->K;
    info->shard_elems = p->L;
    info->arena_elems = p->arena_elems;
    info->chunk_elems = p->chunk_elems;
    info->n_chunks = p->n_chunks;
    info->adamw_tiles = p->n_tiles;
    info->boundary_tiles = p->n_boundary;
    return Z1_OK;
}

z1_status z1_plan_layout(const z1_plan *p, int64_t *start, int64_t *len, int64_t *arena_off)
{
    if (!p)
        return Z1_EINVAL;
    const size_t bytes = (size_t)p->n * sizeof(int64_t);
    if (start && bytes)
        memcpy(start, p->start.data(), bytes);
    if (len && bytes)
        memcpy(len, p->len.data(), bytes);
    if (arena_off && bytes)
        memcpy(arena_off, p->arena_off.data(), bytes);
    return Z1_OK;
}

namespace {

// One accumulation pass over slots k .. k + g - 1: on the arena walk when the
// plan has one and the pass is a single or a wide one (slot addresses from
// the packed shards' bases), else over the chunk table.  A last pass records
// how many norm partials it leaves.
hipError_t accum_pass(z1_plan *p, int32_t k, int32_t g, bool first, bool last, hipStream_t s)
{
    const z1::LaunchGeom geo = geom(p);
    const bool on_arena = z1::slots_arena(geo, g) && p->gbase.size() == (size_t)p->K;
    hipError_t e;
    if (on_arena) {
        z1::SlotBases sb{};
        for (int32_t j = 0; j < g; ++j)
            sb.g[j] = p->gbase[(size_t)(k + j)];
        e = z1::launch_accum_arena(geo, sb, g, p->acc, p->d_partials, first, last, s);
    } else {
        const uint16_t *const *tab = p->d_grads + (size_t)k * p->n;
        e = g == 1 ? z1::launch_accum(geo, tab, p->acc, p->d_partials, first, last, s)
                   : z1::launch_accum_slots(geo, tab, p->n, g, p->acc, p->d_partials, first,
                                            last, false, 1.0f, s);
    }
    if (e == hipSuccess && last)
        p->n_partials = z1::pass_partials(geo, g, on_arena);
    return e;
}

}  // namespace

z1_status z1_accum_grads(z1_plan *p, int32_t k, z1_stream stream)
{
    if (!p || k < 0 || k >= p->K)
        return Z1_EINVAL;
    if (!on_owner(p->device, stream))
        return Z1_EINVAL;
    if (k != 0 && k != p->next_k)
        return Z1_ESTATE;
    const bool first = k == 0, last = k == p->K - 1;
    const hipError_t e = accum_pass(p, k, 1, first, last, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        p->next_k = 0;
        p->acc_complete = false;
        p->norm_done = false;
        return Z1_EHIP;
    }
    p->next_k = k + 1;
    p->acc_complete = last;
    p->norm_done = false;
    return Z1_OK;
}

z1_status z1_accum_grads_range(z1_plan *p, int32_t k_begin, int32_t k_end, z1_stream stream)
{
    if (!p || k_begin < 0 || k_end > p->K || k_begin >= k_end)
        return Z1_EINVAL;
    if (!on_owner(p->device, stream))
        return Z1_EINVAL;
    if (k_begin != 0 && k_begin != p->next_k)
        return Z1_ESTATE;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int32_t k = k_begin; k < k_end;) {
        // passes of at most kMaxSlots slots, as even as possible
        const int32_t left = k_end - k;
        const int32_t passes = (left + z1::kMaxSlots - 1) / z1::kMaxSlots;
        const int32_t g = (left + passes - 1) / passes;
        const bool first = k == 0, last = k + g == p->K;
        const hipError_t e = accum_pass(p, k, g, first, last, s);
        if (e != hipSuccess) {
            p->next_k = 0;
            p->acc_complete = false;
            p->norm_done = false;
            return Z1_EHIP;
        }
        k += g;
    }
    p->next_k = k_end;
    p->acc_complete = k_end == p->K;
    p->norm_done = false;
    return Z1_OK;
}

z1_status z1_grad_norm_sq(z1_plan *p, double *d_S, z1_stream stream)
{
    if (!p || !d_S)
        return Z1_EINVAL;
    if (!on_owner(p->device, stream))
        return Z1_EINVAL;
    if (!aligned(d_S, 8))
        return Z1_EALIGN;
    if (!p->acc_complete)
        return Z1_ESTATE;
    if (z1::launch_norm_fin(p->d_partials, p->n_partials, p->d_stage, p->d_counter, d_S,
                            reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return Z1_EHIP;
    p->norm_done = true;
    return Z1_OK;
}

z1_status z1_grad_norm_sq_pair(z1_plan *p, double *d_pair, z1_stream stream)
{
    if (!p || !d_pair)
        return Z1_EINVAL;
    if (!on_owner(p->device, stream))
        return Z1_EINVAL;
    if (!aligned(d_pair, 16))
        return Z1_EALIGN;
    if (!p->acc_complete)
        return Z1_ESTATE;
    if (z1::launch_norm_fin(p->d_partials, p->n_partials, p->d_stage, p->d_counter, nullptr,
                            reinterpret_cast<hipStream_t>(stream),
                            reinterpret_cast<DD *>(d_pair)) != hipSuccess)
        return Z1_EHIP;
    p->norm_done = true;
    return Z1_OK;
}

z1_status z1_norm_combine(const double *d_pairs, int32_t n, double *d_S, z1_stream stream)
{
    if (!d_pairs || !d_S || n < 1)
        return Z1_EINVAL;
    if (!aligned(d_pairs, 16) || !aligned(d_S, 8))
        return Z1_EALIGN;
    // no plan owns this call: the current GPU must own the stream and both
    // buffers, as a plan's GPU must for the calls on a plan
    const int dev = current_device();
    if (dev < 0)
        return Z1_EHIP;
    if (!stream_on(dev, stream) || !device_memory_on(dev, d_pairs) ||
        !device_memory_on(dev, d_S))
        return Z1_EINVAL;
    return z1::launch_norm_combine(reinterpret_cast<const DD *>(d_pairs), n, d_S,
                                   reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? Z1_OK
               : Z1_EHIP;
}

z1_status z1_adamw_step(z1_plan *p, const z1_adamw_hp *hp, const double *d_S_global,
                        z1_stream stream)
{
    if (!p || !hp || !hp_ok(hp))
        return Z1_EINVAL;
    const bool clipping = hp->clip > 0.0;
    if (clipping && !d_S_global)
        return Z1_EINVAL;
    if (!on_owner(p->device, stream))
        return Z1_EINVAL;
    if (d_S_global && !aligned(d_S_global, 8))
        return Z1_EALIGN;
    if (!p->acc_complete || (clipping && !p->norm_done))
        return Z1_ESTATE;

    const AdamConsts k = consts_of(hp);
    hipError_t e = z1::launch_adamw(geom(p), p->d_weights, p->d_scales, p->acc, p->master,
                                    p->exp_avg, p->exp_avg_sq, k, d_S_global,
                                    reinterpret_cast<hipStream_t>(stream));
    p->next_k = 0;
    p->acc_complete = false;
    p->norm_done = false;
    return e == hipSuccess ? Z1_OK : Z1_EHIP;
}

z1_status z1_grad_norm_sq_acc(z1_plan *p, double *d_S, z1_stream stream)
{
    if (!p || !d_S)
        return Z1_EINVAL;
    if (!on_owner(p->device, stream))
        return Z1_EINVAL;
    if (!aligned(d_S, 8))
        return Z1_EALIGN;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (z1::launch_norm_acc(geom(p), p->acc, p->d_partials, s) != hipSuccess ||
        z1::launch_norm_fin(p->d_partials, p->n_chunks, p->d_stage, p->d_counter, d_S, s) !=
            hipSuccess) {
        p->next_k = 0;
        p->acc_complete = false;
        p->norm_done = false;
        return Z1_EHIP;
    }
    p->n_partials = p->n_chunks;
    p->next_k = 0;
    p->acc_complete = true;
    p->norm_done = true;
    return Z1_OK;
}

static z1_status pack_layout_body(int32_t kind, int32_t n, const int64_t *numel,
                                  const int64_t *rows, int32_t dp_size, int64_t *seg_elems)
{
    if (!seg_elems || n < 0 || dp_size < 1)
        return Z1_EINVAL;
    std::vector<int64_t> st(n > 0 ? n : 1), ln(n > 0 ? n : 1), off(n > 0 ? n : 1);
    int64_t seg = 0;
    for (int32_t r = 0; r < dp_size; ++r) {
        int64_t ae = 0;
        const z1_status e =
            z1_shard_plan_kind(kind, n, numel, rows, dp_size, r, st.data(), ln.data(), off.data(), &ae);
        if (e != Z1_OK)
            return e;
        if (ae > seg)
            seg = ae;
    }
    *seg_elems = (seg + z1::kArenaResidue - 1) / z1::kArenaResidue * z1::kArenaResidue;
    return Z1_OK;
}

static z1_status pack_create_body(z1_pack **out, const z1_pack_bind *b, z1_stream stream)
{
    if (!out)
        return Z1_EINVAL;
    *out = nullptr;
    if (!b || b->n_tensors < 0 || b->dp_size < 1 || b->n_micro < 1 || b->reserved != 0 ||
        !b->send)
        return Z1_EINVAL;
    const int32_t n = b->n_tensors, K = b->n_micro, D = b->dp_size;
    if (n > 0 && (!b->numel || !b->grads))
        return Z1_EINVAL;
    const int64_t chunk = chunk_or_default(b->chunk_elems);
    if (!chunk_ok(chunk))
        return Z1_EINVAL;
    int64_t seg = 0;
    z1_status st = pack_layout_body(b->plan_kind, n, b->numel, b->rows, D, &seg);
    if (st != Z1_OK)
        return st;
    if (seg > 0 && b->send_elems / seg < D)
        return Z1_EINVAL;
    if (!aligned(b->send, 16))
        return Z1_EALIGN;
    std::vector<const uint16_t *> gptr((size_t)K * n);
    for (size_t j = 0; j < gptr.size(); ++j) {
        gptr[j] = static_cast<const uint16_t *>(b->grads[j]);
        if (b->numel[j % n] == 0)
            continue;
        if (!gptr[j])
            return Z1_EINVAL;
        if (!aligned(gptr[j], 16))
            return Z1_EALIGN;
    }
    std::unique_ptr<z1_pack, PackDeleter> owner(new (std::nothrow) z1_pack());
    z1_pack *p = owner.get();
    if (!p)
        return Z1_ENOMEM;
    p->n = n;
    p->K = K;
    p->dp = D;
    p->seg = seg;
    p->sub = (int32_t)(chunk / z1::kAdamBlockElems);
    p->divide = b->divide != 0;
    p->send = b->send;
    std::vector<Chunk> chunks;
    std::vector<int64_t> sv(n > 0 ? n : 1), lv(n > 0 ? n : 1), ov(n > 0 ? n : 1);
    for (int32_t r = 0; r < D; ++r) {
        int64_t ae = 0;
        z1_shard_plan_kind(b->plan_kind, n, b->numel, b->rows, D, r, sv.data(), lv.data(),
                           ov.data(), &ae);
        append_chunks(chunks, n, sv.data(), lv.data(), ov.data(), (int64_t)r * seg, chunk);
    }
    p->n_chunks = (int64_t)chunks.size();
    if (p->n_chunks > INT32_MAX)
        return Z1_EINVAL;
    if ((p->device = current_device()) < 0)
        return Z1_EHIP;
    if (!stream_on(p->device, stream))
        return Z1_EINVAL;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    void *dc = nullptr, *dg = nullptr;
    if (hipMalloc(&dc, (chunks.empty() ? 1 : chunks.size()) * sizeof(Chunk)) != hipSuccess ||
        hipMalloc(&dg, (gptr.empty() ? 1 : gptr.size()) * sizeof(void *)) != hipSuccess) {
        (void)hipGetLastError();
        if (dc)
            (void)hipFree(dc);
        return Z1_ENOMEM;
    }
    p->d_chunks = static_cast<Chunk *>(dc);
    p->d_grads = static_cast<const uint16_t **>(dg);
    hipError_t e = hipSuccess;
    if (!chunks.empty())
        e = hipMemcpyAsync(p->d_chunks, chunks.data(), chunks.size() * sizeof(Chunk),
                           hipMemcpyHostToDevice, s);
    if (e == hipSuccess && !gptr.empty())
        e = hipMemcpyAsync(p->d_grads, gptr.data(), gptr.size() * sizeof(void *),
                           hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);  // host staging vectors die with this call
    if (e != hipSuccess) {
        (void)hipStreamSynchronize(s);  // no upload may still read them
        (void)hipGetLastError();
        return Z1_EHIP;
    }
    *out = owner.release();
    return Z1_OK;
}

z1_status z1_pack_destroy(z1_pack *p)
{
    if (!p)
        return Z1_OK;
    DeviceScope on(p->device);
    (void)hipDeviceSynchronize();
    if (p->d_chunks)
        (void)hipFree(p->d_chunks);
    if (p->d_grads)
        (void)hipFree(p->d_grads);
    delete p;
    return Z1_OK;
}

z1_status z1_pack_accum(z1_pack *p, int32_t k, z1_stream stream)
{
    if (!p || k < 0 || k >= p->K)
        return Z1_EINVAL;
    if (!on_owner(p->device, stream))
        return Z1_EINVAL;
    if (k != 0 && k != p->next_k)
        return Z1_ESTATE;
    const bool last = k == p->K - 1;
    z1::LaunchGeom g{p->d_chunks, p->n_chunks, (int)(p->n_chunks > 0 ? p->n_chunks : 1)};
    g.sub = p->sub;
    if (z1::launch_pack(g, p->d_grads + (size_t)k * p->n, p->send, k == 0, last && p->divide,
                        (float)p->dp, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) {
        p->next_k = 0;
        return Z1_EHIP;
    }
    p->next_k = last ? 0 : k + 1;
    return Z1_OK;
}

z1_status z1_pack_accum_range(z1_pack *p, int32_t k_begin, int32_t k_end, z1_stream stream)
{
    if (!p || k_begin < 0 || k_end > p->K || k_begin >= k_end)
        return Z1_EINVAL;
    if (!on_owner(p->device, stream))
        return Z1_EINVAL;
    if (k_begin != 0 && k_begin != p->next_k)
        return Z1_ESTATE;
    z1::LaunchGeom geo{p->d_chunks, p->n_chunks, (int)(p->n_chunks > 0 ? p->n_chunks : 1)};
    geo.sub = p->sub;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int32_t k = k_begin; k < k_end;) {
        const int32_t left = k_end - k;
        const int32_t passes = (left + z1::kMaxSlots - 1) / z1::kMaxSlots;
        const int32_t g = (left + passes - 1) / passes;
        const bool first = k == 0, divide = p->divide && k + g == p->K;
        const uint16_t *const *tab = p->d_grads + (size_t)k * p->n;
        const hipError_t e =
            g == 1 ? z1::launch_pack(geo, tab, p->send, first, divide, (float)p->dp, s)
                   : z1::launch_accum_slots(geo, tab, p->n, g, p->send, nullptr, first, false,
                                            divide, (float)p->dp, s);
        if (e != hipSuccess) {
            p->next_k = 0;
            return Z1_EHIP;
        }
        k += g;
    }
    p->next_k = k_end == p->K ? 0 : k_end;
    return Z1_OK;
}

static z1_status schedule_create_body(z1_schedule **out, const z1_adamw_hp *hp,
                                      const z1_lr_schedule *lr, int64_t n_steps,
                                      z1_stream stream)
{
    if (!out)
        return Z1_EINVAL;
    *out = nullptr;
    if (!hp || !hp_ok(hp) || n_steps < 1 || n_steps > Z1_SCHEDULE_MAX_STEPS ||
        hp->step > INT64_MAX - n_steps)
        return Z1_EINVAL;
    std::vector<AdamConsts> table((size_t)n_steps);
    for (int64_t j = 0; j < n_steps; ++j) {
        z1_adamw_hp h = *hp;
        h.step = hp->step + j;
        if (lr) {
            const z1_status st = z1_lr_at(lr, h.step, &h.lr);
            if (st != Z1_OK)
                return st;
            if (!isfinite(h.lr))
                return Z1_EINVAL;
        }
        table[(size_t)j] = consts_of(&h);
    }
    z1_schedule *sc = new (std::nothrow) z1_schedule();
    if (!sc)
        return Z1_ENOMEM;
    sc->t_first = hp->step;
    sc->n_steps = n_steps;
    sc->clipping = hp->clip > 0.0;
    if ((sc->device = current_device()) < 0) {
        delete sc;
        return Z1_EHIP;
    }
    if (!stream_on(sc->device, stream)) {
        delete sc;
        return Z1_EINVAL;
    }
    auto fail = [&](z1_status st) {
        if (sc->d_table)
            (void)hipFree(sc->d_table);
        if (sc->d_state)
            (void)hipFree(sc->d_state);
        delete sc;
        return st;
    };
    z1_status st;
    if ((st = device_alloc(&sc->d_table, table.size())) != Z1_OK ||
        (st = device_alloc(&sc->d_state, 2)) != Z1_OK)
        return fail(st);
    const int64_t zero[2] = {0, 0};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(sc->d_table, table.data(), table.size() * sizeof(AdamConsts),
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(sc->d_state, zero, sizeof zero, hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);  // the host table dies with this call
    if (e != hipSuccess) {
        (void)hipStreamSynchronize(s);  // no upload may still read it
        (void)hipGetLastError();
        return fail(Z1_EHIP);
    }
    *out = sc;
    return Z1_OK;
}

z1_status z1_schedule_destroy(z1_schedule *sc)
{
    if (!sc)
        return Z1_OK;
    DeviceScope on(sc->device);
    (void)hipDeviceSynchronize();
    (void)hipFree(sc->d_table);
    (void)hipFree(sc->d_state);
    delete sc;
    return Z1_OK;
}

z1_status z1_schedule_query(const z1_schedule *sc, int64_t *next_step, int64_t *overrun)
{
    if (!sc)
        return Z1_EINVAL;
    DeviceScope on(sc->device);
    int64_t st[2] = {0, 0};
    if (hipMemcpy(st, sc->d_state, sizeof st, hipMemcpyDeviceToHost) != hipSuccess) {
        (void)hipGetLastError();
        return Z1_EHIP;
    }
    if (next_step)
        *next_step = sc->t_first + st[0];
    if (overrun)
        *overrun = st[1];
    return Z1_OK;
}

z1_status z1_adamw_step_scheduled(z1_plan *p, z1_schedule *sc, const double *d_S_global,
                                  z1_stream stream)
{
    if (!p || !sc)
        return Z1_EINVAL;
    if (sc->clipping && !d_S_global)
        return Z1_EINVAL;
    if (sc->device != p->device)
        return Z1_EINVAL;
    if (!on_owner(p->device, stream))
        return Z1_EINVAL;
    if (d_S_global && !aligned(d_S_global, 8))
        return Z1_EALIGN;
    if (!p->acc_complete || (sc->clipping && !p->norm_done))
        return Z1_ESTATE;
    const hipError_t e = z1::launch_adamw_scheduled(
        geom(p), p->d_weights, p->d_scales, p->acc, p->master, p->exp_avg, p->exp_avg_sq,
        sc->d_table, sc->n_steps, sc->d_state, d_S_global, reinterpret_cast<hipStream_t>(stream));
    p->next_k = 0;
    p->acc_complete = false;
    p->norm_done = false;
    return e == hipSuccess ? Z1_OK : Z1_EHIP;
}

z1_status z1_probe_plan(z1_plan *p, int32_t kind, z1_stream stream)
{
    if (!p || kind != Z1_PROBE_PLAN_ADAMW)
        return Z1_EINVAL;
    if (!on_owner(p->device, stream))
        return Z1_EINVAL;
    if (z1::launch_adamw_traffic(geom(p), p->d_weights, p->acc, p->master, p->exp_avg,
                                 p->exp_avg_sq, reinterpret_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return Z1_EHIP;
    return Z1_OK;
}

z1_status z1_grad_norm_sq_flat_noalloc(const float *acc, int64_t n, double *d_S,
                                       z1_stream stream)
{
    if (!d_S || n < 0 || n > Z1_NORM_FLAT_MAX_ELEMS || (n > 0 && !acc))
        return Z1_EINVAL;
    if ((n > 0 && !aligned(acc, 16)) || !aligned(d_S, 8))
        return Z1_EALIGN;
    const int dev = current_device();
    if (dev < 0)
        return Z1_EHIP;
    if (!stream_on(dev, stream) || !device_memory_on(dev, d_S) ||
        (n > 0 && !device_memory_on(dev, acc)))
        return Z1_EINVAL;
    char *base = static_cast<char *>(scratch_on(dev));
    if (!base)
        return Z1_EHIP;
    DD *partials = reinterpret_cast<DD *>(base);
    DD *stage = reinterpret_cast<DD *>(base + kScratchPartials);
    unsigned int *counter = reinterpret_cast<unsigned int *>(base + kScratchPartials + kScratchStage);
    return z1::launch_norm_flat(acc, n, partials, stage, counter, d_S,
                                reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? Z1_OK
               : Z1_EHIP;
}

z1_status z1_probe_copy(const void *src, void *dst, int64_t n_bytes, z1_stream stream)
{
    if (!src || !dst || n_bytes < 0 || n_bytes % 16 != 0)
        return Z1_EINVAL;
    if (!aligned(src, 16) || !aligned(dst, 16))
        return Z1_EALIGN;
    return z1::launch_copy(src, dst, n_bytes, reinterpret_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? Z1_OK
               : Z1_EHIP;
}

// The entry points that build host tables, behind the exception guard.
z1_status z1_plan_create(z1_plan **out, const z1_bind *b, z1_stream stream)
{
    return no_throw([&] { return plan_create_body(out, b, stream); });
}

z1_status z1_pack_layout(int32_t kind, int32_t n, const int64_t *numel, const int64_t *rows,
                         int32_t dp_size, int64_t *seg_elems)
{
    return no_throw([&] { return pack_layout_body(kind, n, numel, rows, dp_size, seg_elems); });
}

z1_status z1_pack_create(z1_pack **out, const z1_pack_bind *b, z1_stream stream)
{
    return no_throw([&] { return pack_create_body(out, b, stream); });
}

z1_status z1_schedule_create(z1_schedule **out, const z1_adamw_hp *hp,
                             const z1_lr_schedule *lr, int64_t n_steps, z1_stream stream)
{
    return no_throw([&] { return schedule_create_body(out, hp, lr, n_steps, stream); });
}

}  // extern "C"
