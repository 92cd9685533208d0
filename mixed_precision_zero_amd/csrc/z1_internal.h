// z1_internal.h -- types shared by the host API (z1_api.hip) and the kernels
// (z1_kernels.hip) of the ZeRO-1 shard optimizer step.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace z1 {

// Workgroup of four wave64s (the chunk-table kernels of narrow passes and
// the norm; AdamW and single or wide passes run one-wave workgroups); every
// lane moves 4 elements per vector (16-byte fp32 accesses, 8-byte bf16
// accesses), so one such workgroup touches 1024 consecutive elements per
// vector step.
constexpr int kBlock = 256;
constexpr int kWave = 64;       // lanes of one wavefront
constexpr int kVec = 4;
constexpr int64_t kDefaultChunk = 4096;
constexpr int64_t kMaxChunk = 1 << 20;
// The chunk table is stored in tensor order.  The accumulation and norm
// kernels issue it in kInterleave interleaved regions (consecutive workgroups
// land on different XCDs, each XCD walking one contiguous region); AdamW
// issues it in table order.
constexpr int kInterleave = 8;
// A whole tile: 4 vectors of 4 elements per lane of a kBlock workgroup (the
// default piece, the flat norm's unit).
constexpr int64_t kTileElems = 4 * kBlock * kVec;
// AdamW runs one-wave workgroups of one vector per lane: a block of
// kWave * kVec elements (also the arena walk's tile).  Each workgroup
// reserves 1/N of a compute unit's LDS, so at most N are resident per compute
// unit: N = kAdamPerCUTiles on the arena walk, whose loads wait for nothing,
// and kAdamPerCUChunks on the chunk walk, whose loads wait for the piece's
// descriptor (measured on the 7B shard, 10-24: 14 for both; the chunk walk
// wanted 20 until the bias corrections were divided with their reciprocals).
constexpr int kAdamBlockElems = kWave * kVec;
#ifndef Z1_ADAM_CAP_TILES
#define Z1_ADAM_CAP_TILES 14
#endif
#ifndef Z1_ADAM_CAP_CHUNKS
#define Z1_ADAM_CAP_CHUNKS 14
#endif
constexpr int kAdamPerCUTiles = Z1_ADAM_CAP_TILES;
constexpr int kAdamPerCUChunks = Z1_ADAM_CAP_CHUNKS;
constexpr int kMaxSlots = 16;    // micro-batch slots one multi-slot pass reads
constexpr int kFinBlock = 256;
// first-level workgroups of the norm reduction (1024 were slower: 40 against
// 20 us for the 3.3M partials of a one-wave last pass on the 7B shard)
constexpr int kFinStages = 256;
constexpr int kFinUnroll = 8;    // partials each finalise thread loads at once
// Arena offsets share the slice start's residue mod kArenaResidue elements:
// 64 elements are one 128-byte cache line of bf16 (two of fp32), so a piece
// that starts at a multiple of chunk_elems inside its tensor starts on a line
// in the fp32 arenas and in a packed bf16 shard alike.
constexpr int64_t kArenaResidue = 64;

// One unit of work: a piece of one tensor's slice of at most chunk_elems
// elements.  Pieces are cut at multiples of chunk_elems inside the tensor,
// so every piece except a slice's first one starts on a 128-byte line of the
// fp32 arenas and of the bf16 buffers.
struct alignas(32) Chunk {
    int64_t src;     // first element of the piece inside the full tensor
    int64_t dst;     // same element's index inside the fp32 arenas
    int32_t tensor;  // parameter index (selects the bf16 pointers)
    int32_t count;   // elements in the piece, 1..chunk_elems
    int64_t pad;
};
static_assert(sizeof(Chunk) == 32, "chunk descriptor is 32 bytes");

// Unevaluated sum hi + lo with |lo| <= ulp(hi)/2 (a double-double).
struct alignas(16) DD {
    double hi, lo;
};

// Per-step AdamW constants, all binary64, derived on the host.
struct AdamConsts {
    double lr;
    double beta1, beta2;
    double omb1, omb2;     // 1 - beta1, 1 - beta2
    double eps;
    double weight_decay;
    double bc1, bc2;       // 1 - beta1^t, 1 - beta2^t
    double rbc1, rbc2;     // 1 / bc1, 1 / bc2, each rounded once
    double clip;           // <= 0: no clipping
};

// Per-tensor multipliers of lr and weight decay.
struct alignas(16) Scale {
    double lr, wd;
};

// The arena walk of a packed plan: tile j covers arena elements
// [j * kAdamBlockElems, (j + 1) * kAdamBlockElems).  tags[j] >= 0 is the
// tensor whose slice holds the whole tile; -1 marks a tile that crosses a
// slice boundary or the arena's end, whose slice segments (pieces in the
// chunk table's format) are listed in segs, each run by a workgroup of its
// own.
struct ArenaWalk {
    const int32_t *tags = nullptr;   // device [n_tiles]
    const Chunk *segs = nullptr;     // device [n_segs]
    int64_t n_tiles = 0;             // 0: the plan walks the chunk table
    int64_t n_full = 0;              // tiles that end inside the arena
    int64_t n_segs = 0;
    uint16_t *wbase = nullptr;       // the packed bf16 weight shard
    // full-size bf16 tensors: device [n_tensors], the byte address of arena
    // element 0 as tensor i's slice maps it (weights[i] + 2 (start_i -
    // arena_off_i)); nullptr for packed plans
    const int64_t *wdelta = nullptr;
};

struct LaunchGeom {
    const Chunk *chunks;  // device
    int64_t n_chunks;
    int grid;             // workgroups for the chunk kernels
    ArenaWalk arena{};    // AdamW's arena walk, when n_tiles > 0
    int32_t sub = 1;         // one-wave workgroups per piece (chunk_elems / kAdamBlockElems)
    int64_t adam_grid = 0;   // AdamW's chunk-walk grid (< n_chunks * sub: it loops)
    uint32_t adam_lds = 0;   // LDS bytes each AdamW workgroup reserves (the residency cap)
};

// Accumulation passes of one slot or of at least kSlotsOneWave slots run
// one-wave workgroups of one vector per lane: on the arena walk when the
// plan has one (packed plans; every slot's element at its arena position,
// one workgroup per tile, one norm partial per tile and per boundary
// segment), else on the chunk table with sub workgroups per piece (one norm
// partial per workgroup; uncapped grids only).  Passes of 2 to
// kSlotsOneWave - 1 slots, and capped grids, keep 256-lane workgroups (one
// partial per piece).  Measured on packed slots against 256-lane
// workgroups, alternating: one slot (per call) 5-11% faster on the arena
// walk and 1-7% on the chunk table; 8 and 16 slots 10% and 8% on the chunk
// table and 2-6% more on the arena walk; 4 slots 7% slower on the one-wave
// chunk walk (too few loads per lane to cover each workgroup's lookups) and
// no faster on the arena walk (below).
constexpr int kSlotsOneWave = 8;

inline bool slots_wide_or_single(int n_slots)
{
    return n_slots == 1 || n_slots >= kSlotsOneWave;
}

// The arena walk (packed plans that have one) takes single and wide passes.
// Passes of 2 to kSlotsOneWave - 1 slots keep the 256-lane chunk kernel:
// on the arena walk the 7B shard's 4-slot pass (no boundary tile) ran
// 0.3-2.8% faster, but its finalise then sums one partial per tile (3.3M
// instead of 206K, 21 against 12 us), which left pass and finalise together
// even (three processes with the model's full-size gradients allocated, as
// in the benchmark); SmolLM-135M's (211 boundary tiles) ran 1.4-8.5% slower.
inline bool slots_arena(const LaunchGeom &geo, int n_slots)
{
    return geo.arena.n_tiles > 0 && slots_wide_or_single(n_slots);
}

inline bool slots_one_wave(const LaunchGeom &geo, int n_slots)
{
    return slots_wide_or_single(n_slots) && geo.grid >= geo.n_chunks &&
           geo.n_chunks * geo.sub <= INT32_MAX;
}

// norm partials a last accumulation pass of n_slots slots leaves (the arena
// walk when on_arena, else the chunk table)
inline int64_t pass_partials(const LaunchGeom &geo, int n_slots, bool on_arena)
{
    if (on_arena)
        return geo.arena.n_tiles + geo.arena.n_segs;
    return slots_one_wave(geo, n_slots) ? geo.n_chunks * geo.sub : geo.n_chunks;
}

// The bases of a pass's slots in a packed plan: slot j's element at arena
// position x is slots[j][x].
struct SlotBases {
    const uint16_t *g[kMaxSlots];
};

hipError_t launch_accum(const LaunchGeom &geo, const uint16_t *const *grad_tab, float *acc,
                        DD *partials, bool first, bool last, hipStream_t s);
// accumulation into the send buffer: no norm; the last pass may divide by dp
hipError_t launch_pack(const LaunchGeom &geo, const uint16_t *const *grad_tab, float *send,
                       bool first, bool divide, float dp, hipStream_t s);
// slots 0..n_slots-1 of grad_tab (slot j's pointers at grad_tab + j * slot_stride)
// in one pass, 2 <= n_slots <= kMaxSlots; first overwrites, last writes the
// norm partials (pass_partials of them), divide divides the final sum by dp
hipError_t launch_accum_slots(const LaunchGeom &geo, const uint16_t *const *grad_tab,
                              int32_t slot_stride, int n_slots, float *acc, DD *partials,
                              bool first, bool last, bool divide, float dp, hipStream_t s);
// the same on the arena walk of a packed plan (slots_arena): slot j of the
// pass at sb.g[j]
hipError_t launch_accum_arena(const LaunchGeom &geo, const SlotBases &sb, int n_slots,
                              float *acc, DD *partials, bool first, bool last, hipStream_t s);
// norm partials of an acc arena filled by the caller
hipError_t launch_norm_acc(const LaunchGeom &geo, const float *acc, DD *partials, hipStream_t s);
// S (when S != nullptr) and/or the unrounded pair (when pair != nullptr)
hipError_t launch_norm_fin(const DD *partials, int64_t n_chunks, DD *stage,
                           unsigned int *counter, double *S, hipStream_t s,
                           DD *pair = nullptr);
// S of a contiguous acc buffer of n elements: per-tile partials (one per
// kTileElems elements) into `partials`, then the finalise into *S; the first
// kernel clears *counter
hipError_t launch_norm_flat(const float *acc, int64_t n, DD *partials, DD *stage,
                           unsigned int *counter, double *S, hipStream_t s);
// S from n pairs added in index order
hipError_t launch_norm_combine(const DD *pairs, int32_t n, double *S, hipStream_t s);
hipError_t launch_adamw(const LaunchGeom &geo, uint16_t *const *weight_tab, const Scale *scales,
                        const float *acc, float *master, float *m, float *v,
                        const AdamConsts &k, const double *S, hipStream_t s);
// k_adamw with the constants of row state[0] of a per-step table (skipped when
// the table is exhausted), then one thread advances state (row or overrun)
hipError_t launch_adamw_scheduled(const LaunchGeom &geo, uint16_t *const *weight_tab,
                                  const Scale *scales, const float *acc, float *master, float *m,
                                  float *v, const AdamConsts *table, int64_t n_rows,
                                  int64_t *state, const double *S, hipStream_t s);
// k_adamw's loads and stores over the same plan with no arithmetic (measurement)
hipError_t launch_adamw_traffic(const LaunchGeom &geo, uint16_t *const *weight_tab,
                                const float *acc, float *master, float *m, float *v,
                                hipStream_t s);
hipError_t launch_copy(const void *src, void *dst, int64_t n_bytes, hipStream_t s);

}  // namespace z1
