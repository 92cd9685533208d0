// z1_kernels.hip -- gfx950 kernels of the ZeRO-1 shard optimizer step.
//
// The step is a streaming, HBM-bound pass over one rank's shard (about 0.5
// flop per byte), so nothing here uses MFMA.  Each kernel walks a
// device-resident chunk table (a workgroup takes one piece of one tensor's
// slice, or a 256-element block of it) or the arena itself in 256-element
// tiles (AdamW, and in packed plans single and wide accumulation passes);
// its lanes move 4 consecutive elements each with one 16-byte fp32 access
// per arena and one 8-byte bf16 access, consecutive lanes on consecutive
// addresses.  The fp32 arenas are laid out so that an arena
// element and its bf16 element share their position within a vector (the
// arena offset matches the slice start mod 64 elements), so the pieces cut
// at multiples of the chunk size inside a tensor start on whole 128-byte
// lines of every buffer; only the first and last vector of a slice can be
// partial and take a per-element path.
//
// Arithmetic follows the definition exactly (this file is built with
// -ffp-contract=off and without fast-math):
//   * accumulation is one binary32 add per micro-batch, in order, whether
//     one pass reads one micro-batch slot or several;
//   * the squared norm is an exact-square, double-double sum (+Inf or NaN
//     when a square is);
//   * the clip coefficient is clip / (sqrt(S) + 1e-6) clamped at 1, a NaN
//     norm giving a NaN coefficient;
//   * AdamW is evaluated in binary64 with the same operation sequence as the
//     definition (separate multiply and add, correctly rounded division and
//     square root; the divisions by the bias corrections use their
//     reciprocals with exact remainders), then rounded once to binary32 and,
//     for the weight, to bf16 (nearest even).
#include "z1_internal.h"

namespace z1 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Every byte of the shard is touched once per kernel, so loads and stores
// are marked non-temporal.  Measured on the 7B shard (842M elements), NT
// loads + NT stores take the accumulation pass from 1.60 to 1.44 ms and
// AdamW from 4.9 to 4.5 ms; either alone gains little.  U vectors per lane
// are in flight per iteration (U = 4: one 4096-element chunk per workgroup
// in a single unrolled iteration).
#ifndef Z1_NT_LOAD
#define Z1_NT_LOAD 1
#endif
#ifndef Z1_NT_STORE
#define Z1_NT_STORE 1
#endif
#ifndef Z1_UNROLL_ACC
#define Z1_UNROLL_ACC 4
#endif
// Multi-slot passes keep G x U gradient vectors per lane in flight; above 6
// slots U = 2 (7B shard, 8 slots: 5.1 -> 5.95 TB/s; at 6 slots U = 4 and 2
// are within 1%; at 16 slots U = 2 was 1-2% faster than U = 1, with 128
// VGPRs and 4 waves per SIMD).
#ifndef Z1_UNROLL_SLOTS_WIDE
#define Z1_UNROLL_SLOTS_WIDE 2
#endif

template <typename P>
__device__ __forceinline__ auto ld_stream(P p)
{
#if Z1_NT_LOAD
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

template <typename P, typename T>
__device__ __forceinline__ void st_stream(P p, T x)
{
#if Z1_NT_STORE
    __builtin_nontemporal_store(x, p);
#else
    *p = x;
#endif
}

// A pointer read from one of the plan's pointer tables (bf16 weights,
// gradient slots) is generic to the compiler, which then emits flat
// accesses: those count against both the vector-memory and the LDS wait
// counters and may complete out of order with global accesses, so every use
// of a load then waits for all outstanding memory operations.  Every such
// pointer is device memory; in the global address space the accesses are
// global ones and each use waits only for its own loads.
template <typename T>
using gmem = __attribute__((address_space(1))) T;
template <typename T>
__device__ __forceinline__ gmem<T> *to_global(T *p)
{
    return (gmem<T> *)p;
}

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// Round-to-nearest-even of binary32 to bfloat16: adding 0x7FFF plus the
// lowest kept bit carries into the kept half exactly when the dropped half is
// above one half, or exactly one half with an odd kept half.  A carry out of
// the largest finite value lands on infinity; NaN is kept quiet with its sign.
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------- double-double ----
// Knuth's two-sum: s + e == a + b exactly, s = fl(a + b).
__device__ __forceinline__ void two_sum(double a, double b, double &s, double &e)
{
    s = a + b;
    const double bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

// A non-finite plain sum (an Inf or NaN square somewhere) makes the error
// terms meaningless (Inf - Inf); the sum is then the plain one, +Inf or NaN,
// and the low part is dropped so it cannot turn an Inf into NaN.  Finite
// sums take the double-double path unchanged.
__device__ __forceinline__ void dd_add(double &hi, double &lo, double bhi, double blo)
{
    double s, e;
    two_sum(hi, bhi, s, e);
    if (!__builtin_isfinite(s)) {
        hi = s;
        lo = 0.0;
        return;
    }
    e = e + (lo + blo);
    two_sum(s, e, hi, lo);
}

// acc^2 of a binary32 value is exact in binary64.
__device__ __forceinline__ void dd_add_sq(double &hi, double &lo, float a)
{
    const double x = (double)a * (double)a;
    double s, e;
    two_sum(hi, x, s, e);
    hi = s;
    lo = lo + e;
}

// Cross-lane moves of a binary64 value, as two 32-bit halves.  pair32 and
// pair16 give, in every lane, the values of the two lanes l and l ^ 32 (or
// l ^ 16) in lane order (v_permlane32_swap / v_permlane16_swap with the
// value as both operands); dpp_d<CTRL> reads the lane that the DPP control
// names (row_ror:N rotates within a row of 16 lanes, quad_perm permutes
// within a quad).  All of them run on the vector ALU; none goes through the
// LDS crossbar as a generic lane shuffle does.
__device__ __forceinline__ void pair32(double x, double &a, double &b)
{
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const auto l = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32),
                                                    false, false);
    a = __longlong_as_double((long long)(((uint64_t)h[0] << 32) | l[0]));
    b = __longlong_as_double((long long)(((uint64_t)h[1] << 32) | l[1]));
}

__device__ __forceinline__ void pair16(double x, double &a, double &b)
{
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const auto l = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32),
                                                    false, false);
    a = __longlong_as_double((long long)(((uint64_t)h[0] << 32) | l[0]));
    b = __longlong_as_double((long long)(((uint64_t)h[1] << 32) | l[1]));
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double x)
{
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF,
                                                              0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL,
                                                              0xF, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

constexpr int kDppRowRor8 = 0x128;  // lane p of a row reads lane (p - 8) mod 16
constexpr int kDppRowRor4 = 0x124;  // ... (p - 4) mod 16
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]

// Fixed-order sum of a double-double over the 64 lanes of a wave (all lanes
// active), left in every lane: a butterfly over lane distances 32, 16, 8, 4,
// 2 and 1, each step adding the value of lane l ^ d.  Every combine is
// symmetric in its operands, so after each step all lanes of a group hold
// the same value; that is why the row rotations meet the right partners
// (after distances 32 and 16 a lane's value depends only on its position p
// in the row, and p - 8 mod 16 is p ^ 8; after 8 it depends on p mod 8, and
// p - 4 is p ^ 4 mod 8).  The result depends only on the inputs' placement.
__device__ __forceinline__ void wave_reduce_dd(double &hi, double &lo)
{
    double ah, bh, al, bl;
    pair32(hi, ah, bh);
    pair32(lo, al, bl);
    hi = ah;
    lo = al;
    dd_add(hi, lo, bh, bl);
    pair16(hi, ah, bh);
    pair16(lo, al, bl);
    hi = ah;
    lo = al;
    dd_add(hi, lo, bh, bl);
    dd_add(hi, lo, dpp_d<kDppRowRor8>(hi), dpp_d<kDppRowRor8>(lo));
    dd_add(hi, lo, dpp_d<kDppRowRor4>(hi), dpp_d<kDppRowRor4>(lo));
    dd_add(hi, lo, dpp_d<kDppQuadXor2>(hi), dpp_d<kDppQuadXor2>(lo));
    dd_add(hi, lo, dpp_d<kDppQuadXor1>(hi), dpp_d<kDppQuadXor1>(lo));
}

// The same butterfly with generic lane shuffles (ds_bpermute through the LDS
// crossbar): the bits of wave_reduce_dd.  The multi-wave kernels keep it:
// their waves have more vector work to overlap, and on the resident 4-slot
// pass the vector-ALU form ran 0.1-0.3% slower (7B shard, four alternations),
// while on the one-wave passes it took 35-40 us off the 7B last pass.
__device__ __forceinline__ void wave_reduce_dd_lds(double &hi, double &lo)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double ohi = __shfl_xor(hi, off, 64);
        const double olo = __shfl_xor(lo, off, 64);
        dd_add(hi, lo, ohi, olo);
    }
}

// Fixed-order reduction of a double-double across the workgroup: each wave's
// sum, then the waves' sums in wave order.
template <int NT>
__device__ __forceinline__ void block_reduce_dd(double &hi, double &lo, DD *lds)
{
    wave_reduce_dd_lds(hi, lo);
    constexpr int kWaves = NT / 64;
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        lds[wave] = DD{hi, lo};
    __syncthreads();
    if (threadIdx.x == 0) {
        hi = lds[0].hi;
        lo = lds[0].lo;
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            dd_add(hi, lo, lds[w].hi, lds[w].lo);
    }
    __syncthreads();  // lds is reused by the next chunk
}

// ------------------------------------------------------- accumulation ----
// A piece covers elements [src, src+count) of one tensor.  Vector q of the
// piece covers piece-relative elements [4q - lead, 4q + 4 - lead) with
// lead = src mod 4; it is full when it lies inside the piece.  Full vectors
// run in an unrolled loop with no per-lane bounds tests (all loads of U
// vectors are issued before any result is used); the at most two partial
// vectors (the slice's first and last) take a per-element path.
struct Span {
    int lead;  // src mod 4
    int end;   // lead + count
    int qb;    // first full vector
    int qe;    // one past the last full vector
};

__device__ __forceinline__ Span span_of(const Chunk &ch)
{
    Span s;
    s.lead = (int)(ch.src & (kVec - 1));
    s.end = s.lead + ch.count;
    s.qb = (s.lead + kVec - 1) / kVec;
    s.qe = s.end / kVec;
    return s;
}

// Issue order of the accumulation and norm kernels: the c-th workgroup (or
// grid-stride iteration) takes table entry issue_order(c).  The table is cut
// into kInterleave regions of as equal size as possible (the first n mod
// kInterleave one entry longer) and consecutive workgroups alternate between
// them, entry i of region j going to workgroup i * kInterleave + j; the
// entries left over after the last full round go to the longer regions.  The
// hardware hands workgroups to the 8 XCDs round-robin, so each XCD walks one
// contiguous region through its own L2.  A bijection on [0, n): results do
// not depend on it (elements are independent, norm partials are indexed by
// table entry and reduced in table order).
__device__ __forceinline__ int64_t issue_order(int64_t c, int64_t n)
{
    constexpr int64_t P = kInterleave;
    const int64_t q = n / P, r = n % P;
    int64_t i, j;
    if (c < P * q) {
        i = c / P;
        j = c % P;
    } else {
        i = q;
        j = c - P * q;
    }
    return j * q + (j < r ? j : r) + i;
}

// Calls f(e) for every element of the partial vectors (piece-relative
// element index e + lead, i.e. the index into the lead-adjusted pointers).
template <typename F>
__device__ __forceinline__ void for_partial_elems(const Span &sp, F f)
{
    // head vector 0 when lead > 0, tail vector qe when end is not a multiple
    // of 4; a piece shorter than one vector may have both in the same vector
    const int t = (int)threadIdx.x;
    if (t < kVec) {
        if (sp.lead > 0) {
            const int e = t;  // vector 0
            if (e >= sp.lead && e < sp.end)
                f(e);
        }
        if (sp.end % kVec != 0 && !(sp.lead > 0 && sp.qe == 0)) {
            const int e = sp.qe * kVec + t;  // tail vector
            if (e >= sp.lead && e < sp.end)
                f(e);
        }
    }
}

template <bool FIRST, bool LAST>
__device__ __forceinline__ f32x4 accum_vec(u32x2 gr, f32x4 ar)
{
    f32x4 s;
    s.x = bf16_lo(gr.x);
    s.y = bf16_hi(gr.x);
    s.z = bf16_lo(gr.y);
    s.w = bf16_hi(gr.y);
    if (!FIRST) {
        s.x = ar.x + s.x;
        s.y = ar.y + s.y;
        s.z = ar.z + s.z;
        s.w = ar.w + s.w;
    }
    return s;
}

template <bool DIV>
__device__ __forceinline__ f32x4 divide_vec(f32x4 s, float dp)
{
    if (DIV) {
        s.x = s.x / dp;
        s.y = s.y / dp;
        s.z = s.z / dp;
        s.w = s.w / dp;
    }
    return s;
}

// acc = (FIRST ? 0 : acc) + float(g); LAST also sums acc^2 per chunk; DIV
// divides the sum by dp (binary32, correctly rounded) before it is stored.
template <bool FIRST, bool LAST, bool DIV, int U>
__global__ __launch_bounds__(kBlock) void k_accum(const Chunk *__restrict__ chunks,
                                                  int64_t n_chunks,
                                                  const uint16_t *const *__restrict__ gtab,
                                                  float *__restrict__ acc,
                                                  DD *__restrict__ partials, float dp)
{
    __shared__ DD lds[kBlock / 64];
    const int t = (int)threadIdx.x;
    for (int64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
        const int64_t ci = issue_order(c, n_chunks);
        const Chunk ch = chunks[ci];
        const Span sp = span_of(ch);
        const gmem<const uint16_t> *g = to_global(gtab[ch.tensor]) + (ch.src - sp.lead);
        float *a = acc + (ch.dst - sp.lead);
        const gmem<const u32x2> *gv = reinterpret_cast<const gmem<const u32x2> *>(g);
        f32x4 *av = reinterpret_cast<f32x4 *>(a);
        double hi = 0.0, lo = 0.0;

        int q0 = sp.qb;
        for (; q0 + U * kBlock <= sp.qe; q0 += U * kBlock) {
            u32x2 gr[U];
            f32x4 ar[U] = {};
#pragma unroll
            for (int u = 0; u < U; ++u) {
                gr[u] = ld_stream(gv + q0 + u * kBlock + t);
                if (!FIRST)
                    ar[u] = ld_stream(av + q0 + u * kBlock + t);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const f32x4 s = divide_vec<DIV>(accum_vec<FIRST, LAST>(gr[u], ar[u]), dp);
                st_stream(av + q0 + u * kBlock + t, s);
                if (LAST) {
                    dd_add_sq(hi, lo, s.x);
                    dd_add_sq(hi, lo, s.y);
                    dd_add_sq(hi, lo, s.z);
                    dd_add_sq(hi, lo, s.w);
                }
            }
        }
        for (int q = q0 + t; q < sp.qe; q += kBlock) {
            f32x4 ar = {};
            const u32x2 gr = ld_stream(gv + q);
            if (!FIRST)
                ar = ld_stream(av + q);
            const f32x4 s = divide_vec<DIV>(accum_vec<FIRST, LAST>(gr, ar), dp);
            st_stream(av + q, s);
            if (LAST) {
                dd_add_sq(hi, lo, s.x);
                dd_add_sq(hi, lo, s.y);
                dd_add_sq(hi, lo, s.z);
                dd_add_sq(hi, lo, s.w);
            }
        }
        for_partial_elems(sp, [&](int e) {
            float s = __uint_as_float((uint32_t)g[e] << 16);
            if (!FIRST)
                s = a[e] + s;
            if (DIV)
                s = s / dp;
            a[e] = s;
            if (LAST)
                dd_add_sq(hi, lo, s);
        });
        if (LAST) {
            block_reduce_dd<kBlock>(hi, lo, lds);
            if (t == 0)
                partials[ci] = DD{hi, lo};
        }
    }
}

// ------------------------------------------------- norm of a given acc ----
// Same per-chunk double-double partials as the last accumulation pass, from
// an acc arena the caller filled (for example by a reduce-scatter).
// G micro-batch slots in one pass: acc = (FIRST ? 0 : acc) + g_0 + ... +
// g_{G-1}, every addition rounded to binary32 in slot order, which is the
// value G single-slot passes store (each of them rounds the same sum to
// binary32).  The acc arena is read and written once per pass instead of once
// per slot.  LAST and DIV as in k_accum.
template <bool FIRST, bool LAST, bool DIV, int G, int U>
__global__ __launch_bounds__(kBlock) void k_accum_slots(const Chunk *__restrict__ chunks,
                                                        int64_t n_chunks,
                                                        const uint16_t *const *__restrict__ gtab,
                                                        int32_t slot_stride,
                                                        float *__restrict__ acc,
                                                        DD *__restrict__ partials, float dp)
{
    __shared__ DD lds[kBlock / 64];
    const int t = (int)threadIdx.x;
    for (int64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
        const int64_t ci = issue_order(c, n_chunks);
        const Chunk ch = chunks[ci];
        const Span sp = span_of(ch);
        const gmem<const uint16_t> *g[G];
#pragma unroll
        for (int j = 0; j < G; ++j)
            g[j] = to_global(gtab[(int64_t)j * slot_stride + ch.tensor]) + (ch.src - sp.lead);
        float *a = acc + (ch.dst - sp.lead);
        f32x4 *av = reinterpret_cast<f32x4 *>(a);
        double hi = 0.0, lo = 0.0;

        int q0 = sp.qb;
        for (; q0 + U * kBlock <= sp.qe; q0 += U * kBlock) {
            u32x2 gr[G][U];
            f32x4 ar[U] = {};
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int q = q0 + u * kBlock + t;
#pragma unroll
                for (int j = 0; j < G; ++j)
                    gr[j][u] = ld_stream(reinterpret_cast<const gmem<const u32x2> *>(g[j]) + q);
                if (!FIRST)
                    ar[u] = ld_stream(av + q);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                f32x4 s = accum_vec<FIRST, false>(gr[0][u], ar[u]);
#pragma unroll
                for (int j = 1; j < G; ++j)
                    s = accum_vec<false, false>(gr[j][u], s);
                s = divide_vec<DIV>(s, dp);
                st_stream(av + q0 + u * kBlock + t, s);
                if (LAST) {
                    dd_add_sq(hi, lo, s.x);
                    dd_add_sq(hi, lo, s.y);
                    dd_add_sq(hi, lo, s.z);
                    dd_add_sq(hi, lo, s.w);
                }
            }
        }
        for (int q = q0 + t; q < sp.qe; q += kBlock) {
            u32x2 gr[G];
            f32x4 ar = {};
#pragma unroll
            for (int j = 0; j < G; ++j)
                gr[j] = ld_stream(reinterpret_cast<const gmem<const u32x2> *>(g[j]) + q);
            if (!FIRST)
                ar = ld_stream(av + q);
            f32x4 s = accum_vec<FIRST, false>(gr[0], ar);
#pragma unroll
            for (int j = 1; j < G; ++j)
                s = accum_vec<false, false>(gr[j], s);
            s = divide_vec<DIV>(s, dp);
            st_stream(av + q, s);
            if (LAST) {
                dd_add_sq(hi, lo, s.x);
                dd_add_sq(hi, lo, s.y);
                dd_add_sq(hi, lo, s.z);
                dd_add_sq(hi, lo, s.w);
            }
        }
        for_partial_elems(sp, [&](int e) {
            float s = __uint_as_float((uint32_t)g[0][e] << 16);
            if (!FIRST)
                s = a[e] + s;
#pragma unroll
            for (int j = 1; j < G; ++j)
                s = s + __uint_as_float((uint32_t)g[j][e] << 16);
            if (DIV)
                s = s / dp;
            a[e] = s;
            if (LAST)
                dd_add_sq(hi, lo, s);
        });
        if (LAST) {
            block_reduce_dd<kBlock>(hi, lo, lds);
            if (t == 0)
                partials[ci] = DD{hi, lo};
        }
    }
}

// The same pass on one-wave workgroups of one vector per lane, for single
// and wide passes (slots_one_wave): workgroup w takes block b = issue_order(w, n_chunks
// * nsub) -- piece b / nsub, its vectors (b mod nsub) * kWave + t, + nsub *
// kWave, ... -- so each XCD walks one contiguous region of blocks.  A lane
// whose vector is partial (a slice's head or tail) adds its elements one by
// one.  LAST writes the block's double-double partial to partials[b] (zero for
// a block with no elements), so the finalise sums them in table order.
template <bool FIRST, bool LAST, bool DIV, int G>
__global__ __launch_bounds__(kWave) void k_accum_slots_wave(
    const Chunk *__restrict__ chunks, int64_t n_chunks, int32_t nsub,
    const uint16_t *const *__restrict__ gtab, int32_t slot_stride, float *__restrict__ acc,
    DD *__restrict__ partials, float dp)
{
    const int t = (int)threadIdx.x;
    const int64_t b = issue_order(blockIdx.x, n_chunks * nsub);
    const int64_t ci = b / nsub;
    const int sub = (int)(b - ci * nsub);
    const Chunk ch = chunks[ci];
    const Span sp = span_of(ch);
    const int nvec = (sp.end + kVec - 1) / kVec;
    const gmem<const uint16_t> *g[G];
#pragma unroll
    for (int j = 0; j < G; ++j)
        g[j] = to_global(gtab[(int64_t)j * slot_stride + ch.tensor]) + (ch.src - sp.lead);
    float *a = acc + (ch.dst - sp.lead);
    f32x4 *av = reinterpret_cast<f32x4 *>(a);
    double hi = 0.0, lo = 0.0;
    for (int q0 = sub * kWave; q0 < nvec; q0 += nsub * kWave) {
        const int q = q0 + t;
        if (q >= sp.qb && q < sp.qe) {
            u32x2 gr[G];
            f32x4 ar = {};
#pragma unroll
            for (int j = 0; j < G; ++j)
                gr[j] = ld_stream(reinterpret_cast<const gmem<const u32x2> *>(g[j]) + q);
            if (!FIRST)
                ar = ld_stream(av + q);
            f32x4 sv = accum_vec<FIRST, false>(gr[0], ar);
#pragma unroll
            for (int j = 1; j < G; ++j)
                sv = accum_vec<false, false>(gr[j], sv);
            sv = divide_vec<DIV>(sv, dp);
            st_stream(av + q, sv);
            if (LAST) {
                dd_add_sq(hi, lo, sv.x);
                dd_add_sq(hi, lo, sv.y);
                dd_add_sq(hi, lo, sv.z);
                dd_add_sq(hi, lo, sv.w);
            }
            continue;
        }
        const int e0 = q * kVec > sp.lead ? q * kVec : sp.lead;
        const int e1 = q * kVec + kVec < sp.end ? q * kVec + kVec : sp.end;
        for (int e = e0; e < e1; ++e) {
            float sv = __uint_as_float((uint32_t)g[0][e] << 16);
            if (!FIRST)
                sv = a[e] + sv;
#pragma unroll
            for (int j = 1; j < G; ++j)
                sv = sv + __uint_as_float((uint32_t)g[j][e] << 16);
            if (DIV)
                sv = sv / dp;
            a[e] = sv;
            if (LAST)
                dd_add_sq(hi, lo, sv);
        }
    }
    if (LAST) {
        wave_reduce_dd(hi, lo);
        if (t == 0)
            partials[b] = DD{hi, lo};
    }
}

// The same pass on the arena walk of a packed plan (slots_arena): workgroup
// b < n_tiles takes 256-element tile b, its lanes one vector each of every
// slot (and of acc after the first pass) at the tile's arena position, all
// issued before the tile's tag is read; a tile inside one slice sums and
// stores, a boundary tile (tag -1) leaves through a branch that consumes the
// loaded registers.  Workgroup n_tiles + i adds the i-th boundary segment
// element by element.  Every addition is the same binary32 addition in slot
// order as in the chunk-table kernels.  LAST writes the workgroup's
// double-double partial to partials[b] (zero for a boundary tile), the
// tiles' partials then the segments', in arena order.
template <bool FIRST, bool LAST, int G>
__global__ __launch_bounds__(kWave) void k_accum_arena(SlotBases sb,
                                                       const int32_t *__restrict__ tags,
                                                       const Chunk *__restrict__ segs,
                                                       int64_t n_tiles, int64_t n_full,
                                                       float *__restrict__ acc,
                                                       DD *__restrict__ partials)
{
    const int t = (int)threadIdx.x;
    const int64_t b = blockIdx.x;
    // A single pass's slot base and the tag table pointer are kernel
    // arguments; used here, their loads join the first batch with n_tiles
    // and n_full instead of waiting behind the branch, so one scalar round
    // trip precedes the first vector load instead of two.  (Wide passes keep
    // the compiler's placement: one such use per slot pointer makes it wait
    // after every few of their loads.)
    if constexpr (G == 1)
        __asm__ volatile("" ::"s"(sb.g[0]), "s"(tags), "s"(acc));
    double hi = 0.0, lo = 0.0;
    if (b >= n_tiles) {
        const Chunk ch = segs[b - n_tiles];
        for (int e = t; e < ch.count; e += kWave) {
            const int64_t x = ch.dst + e;
            float sv = __uint_as_float((uint32_t)to_global(sb.g[0])[x] << 16);
            if (!FIRST)
                sv = acc[x] + sv;
#pragma unroll
            for (int j = 1; j < G; ++j)
                sv = sv + __uint_as_float((uint32_t)to_global(sb.g[j])[x] << 16);
            acc[x] = sv;
            if (LAST)
                dd_add_sq(hi, lo, sv);
        }
    } else if (b < n_full) {
        const int64_t q = b * kWave + t;
        f32x4 *av = reinterpret_cast<f32x4 *>(acc) + q;
        u32x2 gr[G];
        f32x4 ar = {};
#pragma unroll
        for (int j = 0; j < G; ++j)
            gr[j] = ld_stream(reinterpret_cast<const gmem<const u32x2> *>(to_global(sb.g[j])) + q);
        if (!FIRST)
            ar = ld_stream(av);
        __builtin_amdgcn_sched_barrier(0);
        if (tags[b] >= 0) {
            f32x4 sv = accum_vec<FIRST, false>(gr[0], ar);
#pragma unroll
            for (int j = 1; j < G; ++j)
                sv = accum_vec<false, false>(gr[j], sv);
            st_stream(av, sv);
            if (LAST) {
                dd_add_sq(hi, lo, sv.x);
                dd_add_sq(hi, lo, sv.y);
                dd_add_sq(hi, lo, sv.z);
                dd_add_sq(hi, lo, sv.w);
            }
        } else {
#pragma unroll
            for (int j = 0; j < G; ++j)
                __asm__ volatile("" ::"v"(gr[j]));
            __asm__ volatile("" ::"v"(ar));
        }
    }
    if (LAST) {
        wave_reduce_dd(hi, lo);
        if (t == 0)
            partials[b] = DD{hi, lo};
    }
}

template <int U>
__global__ __launch_bounds__(kBlock) void k_norm_acc(const Chunk *__restrict__ chunks,
                                                     int64_t n_chunks,
                                                     const float *__restrict__ acc,
                                                     DD *__restrict__ partials)
{
    __shared__ DD lds[kBlock / 64];
    const int t = (int)threadIdx.x;
    for (int64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
        const int64_t ci = issue_order(c, n_chunks);
        const Chunk ch = chunks[ci];
        const Span sp = span_of(ch);
        const float *a = acc + (ch.dst - sp.lead);
        const f32x4 *av = reinterpret_cast<const f32x4 *>(a);
        double hi = 0.0, lo = 0.0;
        int q0 = sp.qb;
        for (; q0 + U * kBlock <= sp.qe; q0 += U * kBlock) {
            f32x4 ar[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                ar[u] = ld_stream(av + q0 + u * kBlock + t);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                dd_add_sq(hi, lo, ar[u].x);
                dd_add_sq(hi, lo, ar[u].y);
                dd_add_sq(hi, lo, ar[u].z);
                dd_add_sq(hi, lo, ar[u].w);
            }
        }
        for (int q = q0 + t; q < sp.qe; q += kBlock) {
            const f32x4 x = ld_stream(av + q);
            dd_add_sq(hi, lo, x.x);
            dd_add_sq(hi, lo, x.y);
            dd_add_sq(hi, lo, x.z);
            dd_add_sq(hi, lo, x.w);
        }
        for_partial_elems(sp, [&](int e) { dd_add_sq(hi, lo, a[e]); });
        block_reduce_dd<kBlock>(hi, lo, lds);
        if (t == 0)
            partials[ci] = DD{hi, lo};
    }
}

// ------------------------------------------------- norm of a flat acc ----
// Per-tile double-double partials of sum(acc^2) over a contiguous buffer of n
// elements: tile b covers elements [b * kTileElems, min(n, (b + 1) *
// kTileElems)), one workgroup per tile, the same exact squares and pair
// arithmetic as the plan's passes.  Workgroup 0 also clears the finalise's
// arrival counter (the buffer holding it keeps whatever the last call left).
__global__ __launch_bounds__(kBlock) void k_norm_flat(const float *__restrict__ acc, int64_t n,
                                                      DD *__restrict__ partials,
                                                      unsigned int *__restrict__ counter)
{
    __shared__ DD lds[kBlock / 64];
    const int t = (int)threadIdx.x;
    if (blockIdx.x == 0 && t == 0)
        counter[0] = 0u;
    const int64_t b = blockIdx.x;
    const int64_t e0 = b * kTileElems;
    if (e0 >= n)
        return;
    const float *a = acc + e0;
    const f32x4 *av = reinterpret_cast<const f32x4 *>(a);
    double hi = 0.0, lo = 0.0;
    if (e0 + kTileElems <= n) {
        f32x4 ar[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            ar[u] = ld_stream(av + u * kBlock + t);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            dd_add_sq(hi, lo, ar[u].x);
            dd_add_sq(hi, lo, ar[u].y);
            dd_add_sq(hi, lo, ar[u].z);
            dd_add_sq(hi, lo, ar[u].w);
        }
    } else {
        const int m = (int)(n - e0);  // 1 .. kTileElems - 1
        for (int q = t; q < m / kVec; q += kBlock) {
            const f32x4 x = ld_stream(av + q);
            dd_add_sq(hi, lo, x.x);
            dd_add_sq(hi, lo, x.y);
            dd_add_sq(hi, lo, x.z);
            dd_add_sq(hi, lo, x.w);
        }
        const int e = (m / kVec) * kVec + t;
        if (t < kVec && e < m)
            dd_add_sq(hi, lo, a[e]);
    }
    block_reduce_dd<kBlock>(hi, lo, lds);
    if (t == 0)
        partials[b] = DD{hi, lo};
}

// ------------------------------------------------------ norm finalise ----
// Two levels in one launch: workgroup b sums the per-chunk partials of a
// fixed contiguous range, writes its double-double to stage[b], and the
// workgroup that finishes last (a device-scope counter) sums stage[0..G) in
// index order and writes S.  Every range and every order is fixed by n alone,
// so S does not depend on timing; nothing waits on another workgroup.
__global__ __launch_bounds__(kFinBlock) void k_norm_fin(const DD *__restrict__ partials,
                                                        int64_t n, DD *__restrict__ stage,
                                                        unsigned int *__restrict__ counter,
                                                        double *__restrict__ S,
                                                        DD *__restrict__ pair)
{
    __shared__ DD lds[kFinBlock / 64];
    __shared__ bool is_last;
    const int64_t G = gridDim.x;
    const int64_t per = (n + G - 1) / G;
    const int64_t lo_i = (int64_t)blockIdx.x * per;
    const int64_t hi_i = lo_i + per < n ? lo_i + per : n;
    double hi = 0.0, lo = 0.0;
    // thread t adds partials t, t + kFinBlock, t + 2 kFinBlock, ... of its
    // range in that order; kFinUnroll of them are loaded before the first is
    // added, so a thread waits for one round trip per kFinUnroll partials
    // instead of one per partial (the 3.3M partials of a one-wave last pass
    // on the 7B shard: 31 -> 20 us; the sum's order, and so S, unchanged)
    for (int64_t i0 = lo_i + threadIdx.x; i0 < hi_i; i0 += kFinUnroll * kFinBlock) {
        DD p[kFinUnroll];
#pragma unroll
        for (int u = 0; u < kFinUnroll; ++u) {
            const int64_t i = i0 + (int64_t)u * kFinBlock;
            p[u] = i < hi_i ? partials[i] : DD{0.0, 0.0};
        }
#pragma unroll
        for (int u = 0; u < kFinUnroll; ++u)
            if (i0 + (int64_t)u * kFinBlock < hi_i)
                dd_add(hi, lo, p[u].hi, p[u].lo);
    }
    block_reduce_dd<kFinBlock>(hi, lo, lds);
    if (threadIdx.x == 0) {
        stage[blockIdx.x] = DD{hi, lo};
        __threadfence();
        const unsigned int done = atomicAdd(counter, 1u);
        is_last = done == (unsigned int)(G - 1);
    }
    __syncthreads();
    if (!is_last)
        return;
    __threadfence();
    hi = 0.0;
    lo = 0.0;
    for (int64_t i = threadIdx.x; i < G; i += kFinBlock) {
        const DD p = stage[i];
        dd_add(hi, lo, p.hi, p.lo);
    }
    block_reduce_dd<kFinBlock>(hi, lo, lds);
    if (threadIdx.x == 0) {
        if (S)
            S[0] = hi + lo;
        if (pair)
            pair[0] = DD{hi, lo};  // the unrounded pair, for an exchange between ranks
        counter[0] = 0u;           // ready for the next launch on this plan
    }
}

// S from n double-double pairs (one per rank), added in index order with the
// same pair arithmetic, rounded once.
__global__ __launch_bounds__(64) void k_norm_combine(const DD *__restrict__ pairs, int32_t n,
                                                     double *__restrict__ S)
{
    if (threadIdx.x == 0) {
        double hi = 0.0, lo = 0.0;
        for (int32_t i = 0; i < n; ++i)
            dd_add(hi, lo, pairs[i].hi, pairs[i].lo);
        S[0] = hi + lo;
    }
}

// -------------------------------------------------------------- AdamW ----
struct Elem {
    float p, m, v;
};

// This tensor's learning rate and decay factor (uniform per chunk).
struct TensorRate {
    double lr;     // lr * lr_scale
    double decay;  // 1 - lr_i * (weight_decay * wd_scale)
};

__device__ __forceinline__ TensorRate tensor_rate(const AdamConsts &k, Scale sc)
{
    const double lr = k.lr * sc.lr;
    const double wd = k.weight_decay * sc.wd;
    return TensorRate{lr, 1.0 - lr * wd};
}

// a / b correctly rounded, for a step constant b > 0 that comes with rb, its
// reciprocal rounded once.  q = a * rb is within about an ulp of a / b, and
// q + (a - q * b) * rb, rounded once (the remainder is exact by FMA), is the
// correctly rounded quotient as soon as q is within an ulp (Markstein's
// correction theorem, IBM J. Res. Develop. 34(1), 1990); two corrections
// make sure of that.  The remainders cannot underflow while |a| lies in
// [2^-960, 2^960]; zero, tiny, huge and non-finite a take the IEEE division.
// A multiply and four multiply-adds (after two compares) in place of the
// division sequence and its reciprocal approximation: on the 7B shard AdamW
// took 3.87-3.88 ms against 3.96-3.97 on the arena walk and 3.89 against
// 4.04-4.05 on the chunk walk, bits identical.
__device__ __forceinline__ double div_by_step_const(double a, double b, double rb)
{
    const double aa = __builtin_fabs(a);
    if (aa >= 0x1p-960 && aa <= 0x1p960) {
        const double q0 = a * rb;
        const double q1 = __builtin_fma(-__builtin_fma(q0, b, -a), rb, q0);
        return __builtin_fma(-__builtin_fma(q1, b, -a), rb, q1);
    }
    return a / b;
}

// One element of the step in binary64 (see the header comment of z1.h for
// the formula); the operation order matches the definition term by term, and
// every operation is correctly rounded.
__device__ __forceinline__ Elem adamw_elem(float acc, float p32, float m32, float v32,
                                           const AdamConsts &k, const TensorRate &tr, double c)
{
    const double g = c * (double)acc;
    double p = (double)p32;
    double m = (double)m32;
    double v = (double)v32;
    p = p * tr.decay;
    m = k.beta1 * m + k.omb1 * g;
    v = k.beta2 * v + k.omb2 * g * g;
    const double mhat = div_by_step_const(m, k.bc1, k.rbc1);
    const double vhat = div_by_step_const(v, k.bc2, k.rbc2);
    p = p - tr.lr * mhat / (sqrt(vhat) + k.eps);
    return Elem{(float)p, (float)m, (float)v};
}

__device__ __forceinline__ void adamw_vec(f32x4 a, f32x4 &p, f32x4 &m, f32x4 &v, u32x2 &w,
                                          const AdamConsts &k, const TensorRate &tr, double c)
{
    Elem r;
    r = adamw_elem(a.x, p.x, m.x, v.x, k, tr, c);
    p.x = r.p; m.x = r.m; v.x = r.v;
    r = adamw_elem(a.y, p.y, m.y, v.y, k, tr, c);
    p.y = r.p; m.y = r.m; v.y = r.v;
    r = adamw_elem(a.z, p.z, m.z, v.z, k, tr, c);
    p.z = r.p; m.z = r.m; v.z = r.v;
    r = adamw_elem(a.w, p.w, m.w, v.w, k, tr, c);
    p.w = r.p; m.w = r.m; v.w = r.v;
    w.x = bf16_rne(p.x) | (bf16_rne(p.y) << 16);
    w.y = bf16_rne(p.z) | (bf16_rne(p.w) << 16);
}

// Element-wise traffic stand-in for adamw_vec (measurement only): the same
// inputs and outputs, an add instead of the update, a truncating cast.
__device__ __forceinline__ void traffic_vec(f32x4 a, f32x4 &p, f32x4 &m, f32x4 &v, u32x2 &w)
{
    p = p + a;
    m = m + a;
    v = v + a;
    w.x = (__float_as_uint(p.x) >> 16) | (__float_as_uint(p.y) & 0xFFFF0000u);
    w.y = (__float_as_uint(p.z) >> 16) | (__float_as_uint(p.w) & 0xFFFF0000u);
}

// The clip coefficient from the device S: clip / (sqrt(S) + 1e-6) clamped at
// 1 (a NaN norm gives a NaN coefficient); 1 when clipping is off (S is then
// not read, and may be NULL).
__device__ __forceinline__ double clip_coef(const AdamConsts &k, const double *__restrict__ S)
{
    if (!(k.clip > 0.0))
        return 1.0;
    const double cc = k.clip / (sqrt(S[0]) + 1e-6);
    return cc >= 1.0 ? 1.0 : cc;
}

// The step's constants: the kernel argument, or row `row` of a per-step
// table (false when the table is exhausted: nothing may then be stored).  The
// kernel reads the row index as it starts, and the row itself is read here,
// after a piece's loads are issued, so neither lookup delays them.
template <bool TABLE>
__device__ __forceinline__ bool step_consts(const AdamConsts &k_arg,
                                            const AdamConsts *__restrict__ table, int64_t row,
                                            int64_t n_rows, AdamConsts &k)
{
    k = k_arg;
    if constexpr (TABLE) {
        if (row >= n_rows)
            return false;
        k = table[row];
    }
    return true;
}

// AdamW runs on one-wave workgroups with one vector (4 elements) per lane: a
// block is kWave consecutive vectors; a 4096-element piece is 16 blocks on as
// many workgroups, and an arena tile is one block.  Each launch reserves
// dynamic LDS (which no lane touches) so that only a few of its workgroups
// share a compute unit (kAdamPerCUTiles on the arena walk, kAdamPerCUChunks
// on the chunk walk).  This mix is half writes: with the chip full of loads
// the memory controller's write credits run short, and a lower, steady number
// of waves in flight streams it faster.  Measured on the 7B shard's buffers
// with the update in place: 256-lane workgroups with 4 vectors per lane
// 5.5-6.1 TB/s, one-wave workgroups with 1 vector per lane 6.1-6.6 TB/s at
// 14-16 per compute unit (6 per CU: 4.3; no cap: 6.1-6.4).

// Lane t's vector of the four fp32 streams of a block, at byte offset o from
// the block's bases, loads issued back to back.
struct LaneVec {
    f32x4 a, p, m, v;
};

__device__ __forceinline__ LaneVec load_lane(const char *ab, const char *pb, const char *mb,
                                             const char *vb, uint32_t o)
{
    LaneVec x;
    x.a = ld_stream(reinterpret_cast<const f32x4 *>(ab + o));
    x.p = ld_stream(reinterpret_cast<const f32x4 *>(pb + o));
    x.m = ld_stream(reinterpret_cast<const f32x4 *>(mb + o));
    x.v = ld_stream(reinterpret_cast<const f32x4 *>(vb + o));
    return x;
}

// An exit that stores nothing still consumes the loaded registers, so the
// compiler keeps the loads ahead of the test that leads to it.
__device__ __forceinline__ void discard_lane(const LaneVec &x)
{
    __asm__ volatile("" ::"v"(x.a), "v"(x.p), "v"(x.m), "v"(x.v));
}

// The update of lane t's vector and its four stores (the bf16 stream at half
// the fp32 offset).  MATH = false is the measurement twin (traffic_vec).
template <bool MATH>
__device__ __forceinline__ void update_store_lane(LaneVec x, char *pb, char *mb, char *vb,
                                                  gmem<char> *wb, uint32_t o,
                                                  const AdamConsts &k, const TensorRate &tr,
                                                  double c)
{
    u32x2 w;
    if constexpr (MATH)
        adamw_vec(x.a, x.p, x.m, x.v, w, k, tr, c);
    else
        traffic_vec(x.a, x.p, x.m, x.v, w);
    st_stream(reinterpret_cast<f32x4 *>(pb + o), x.p);
    st_stream(reinterpret_cast<f32x4 *>(mb + o), x.m);
    st_stream(reinterpret_cast<f32x4 *>(vb + o), x.v);
    st_stream(reinterpret_cast<gmem<u32x2> *>(wb + o / 2), w);
}

// The blocks sub, sub + nsub, ... of the piece ch (vector q of the piece
// covers piece-relative elements [4q - lead, 4q + 4 - lead), as in Span).
// A block of full vectors runs straight-line: its loads first, then the
// step's constants, the clip coefficient, the tensor's rate and its bf16
// pointer (lookups whose latency hides behind the loads), then the update
// and the stores.  A block holding a slice's partial head or tail vector,
// or the piece's end, runs lane by lane, each lane its own vector: full ones
// whole, partial ones element by element.  False (nothing more stored) when
// the per-step table is exhausted.
template <bool MATH, bool TABLE>
__device__ __forceinline__ bool adamw_piece(const Chunk &ch, int sub, int nsub,
                                            uint16_t *const *__restrict__ wtab,
                                            const Scale *__restrict__ scales,
                                            const float *__restrict__ acc,
                                            float *__restrict__ master,
                                            float *__restrict__ exp_avg,
                                            float *__restrict__ exp_avg_sq,
                                            const AdamConsts &k_arg,
                                            const double *__restrict__ S,
                                            const AdamConsts *__restrict__ table, int64_t row,
                                            int64_t n_rows)
{
    const int t = (int)threadIdx.x;
    const Span sp = span_of(ch);
    const int nvec = (sp.end + kVec - 1) / kVec;
    // lead-adjusted bases: vector 0 of the piece, on a 16-byte boundary of
    // every fp32 arena (the arena offset shares the source's residue)
    const int64_t off = ch.dst - sp.lead;
    const char *ab = reinterpret_cast<const char *>(acc + off);
    char *pb = reinterpret_cast<char *>(master + off);
    char *mb = reinterpret_cast<char *>(exp_avg + off);
    char *vb = reinterpret_cast<char *>(exp_avg_sq + off);
    for (int q0 = sub * kWave; q0 < nvec; q0 += nsub * kWave) {
        const uint32_t o = (uint32_t)(q0 + t) * 16u;
        AdamConsts k;
        if (q0 >= sp.qb && q0 + kWave <= sp.qe) {
            const LaneVec x = load_lane(ab, pb, mb, vb, o);
            __builtin_amdgcn_sched_barrier(0);
            if (!step_consts<TABLE>(k_arg, table, row, n_rows, k)) {
                discard_lane(x);
                return false;
            }
            const double c = MATH ? clip_coef(k, S) : 1.0;
            const TensorRate tr = MATH ? tensor_rate(k, scales[ch.tensor]) : TensorRate{};
            gmem<char> *wb = reinterpret_cast<gmem<char> *>(to_global(wtab[ch.tensor]) +
                                                            (ch.src - sp.lead));
            update_store_lane<MATH>(x, pb, mb, vb, wb, o, k, tr, c);
            continue;
        }
        if (!step_consts<TABLE>(k_arg, table, row, n_rows, k))
            return false;
        const double c = MATH ? clip_coef(k, S) : 1.0;
        const TensorRate tr = MATH ? tensor_rate(k, scales[ch.tensor]) : TensorRate{};
        gmem<uint16_t> *w = to_global(wtab[ch.tensor]) + (ch.src - sp.lead);
        const int q = q0 + t;
        if (q >= sp.qb && q < sp.qe) {
            update_store_lane<MATH>(load_lane(ab, pb, mb, vb, o), pb, mb, vb,
                                    reinterpret_cast<gmem<char> *>(w), o, k, tr, c);
            continue;
        }
        // a partial vector: its elements inside [lead, end), one by one
        const float *a = acc + off;
        float *p = master + off;
        float *m = exp_avg + off;
        float *v = exp_avg_sq + off;
        const int e0 = q * kVec > sp.lead ? q * kVec : sp.lead;
        const int e1 = q * kVec + kVec < sp.end ? q * kVec + kVec : sp.end;
        for (int e = e0; e < e1; ++e) {
            if constexpr (MATH) {
                const Elem r = adamw_elem(a[e], p[e], m[e], v[e], k, tr, c);
                p[e] = r.p;
                m[e] = r.m;
                v[e] = r.v;
                w[e] = (uint16_t)bf16_rne(r.p);
            } else {
                const float x = p[e] + a[e];
                p[e] = x;
                m[e] = m[e] + a[e];
                v[e] = v[e] + a[e];
                w[e] = (uint16_t)(__float_as_uint(x) >> 16);
            }
        }
    }
    return true;
}

// AdamW over the chunk table: workgroup b takes blocks of piece b / nsub
// (nsub = chunk_elems / 256 per piece), pieces in table (tensor) order.  The
// only lookup before the first vector load is the piece's descriptor.
// ONE: one workgroup per (piece, sub) and no loop, so no store of an earlier
// block is in flight when the loads are consumed (loads and stores share one
// counter); otherwise the grid strides over the n_pieces * nsub indices.
// MATH = false is a measurement twin: the same walk, loads and stores over
// the same buffers, with the arithmetic replaced by traffic_vec, so the cost
// of the update itself can be read off on the step's own buffers.
// TABLE = true takes the step's constants from row state[0] of the per-step
// table.  The row index is read as the kernel starts, and the row itself
// after the block's loads are issued; when the table is exhausted every
// workgroup returns before its first store.
template <bool MATH, bool TABLE, bool ONE>
__global__ __launch_bounds__(kWave) void k_adamw(
    const Chunk *__restrict__ chunks, int64_t n_work, int32_t nsub,
    uint16_t *const *__restrict__ wtab, const Scale *__restrict__ scales,
    const float *__restrict__ acc, float *__restrict__ master, float *__restrict__ exp_avg,
    float *__restrict__ exp_avg_sq, const AdamConsts k_arg, const double *__restrict__ S,
    const AdamConsts *__restrict__ table, int64_t n_rows, const int64_t *__restrict__ state)
{
    const int64_t row = TABLE ? state[0] : 0;
    for (int64_t b = blockIdx.x; b < n_work; b += gridDim.x) {
        const int64_t ci = b / nsub;
        if (!adamw_piece<MATH, TABLE>(chunks[ci], (int)(b - ci * nsub), nsub, wtab, scales, acc,
                                      master, exp_avg, exp_avg_sq, k_arg, S, table, row,
                                      n_rows))
            return;
        if constexpr (ONE)
            break;
    }
}

// AdamW over the arena of a plan (ArenaWalk): workgroup b takes tile b (one
// block); past the tiles, workgroup n_tiles + i takes the i-th boundary
// segment.  Every fp32 stream is addressed by arena position, so a tile that
// ends inside the arena is loaded first, at addresses that depend on nothing
// fetched; its tag, read after the loads are issued, names the tensor whose
// slice holds it (and, FULL, with full-size bf16 tensors, the entry of the
// per-tensor table that places its bf16 store; a packed shard is addressed
// by arena position too).  A tile that crosses a slice boundary (or the
// arena's end) stores nothing, and neither does any tile when the per-step
// table is exhausted; those leave through discard_lane, so the update and
// stores of a live tile stay one unconditional sequence whose waits count its
// own stores.  Same arithmetic, constants, table handling and twin
// (MATH = false) as k_adamw.
template <bool MATH, bool TABLE, bool FULL>
__global__ __launch_bounds__(kWave) void k_adamw_tiles(
    const int32_t *__restrict__ tags, const Chunk *__restrict__ segs, int64_t n_tiles,
    int64_t n_full, uint16_t *__restrict__ wbase, const int64_t *__restrict__ wdelta,
    uint16_t *const *__restrict__ wtab,
    const Scale *__restrict__ scales, const float *__restrict__ acc, float *__restrict__ master,
    float *__restrict__ exp_avg, float *__restrict__ exp_avg_sq, const AdamConsts k_arg,
    const double *__restrict__ S, const AdamConsts *__restrict__ table, int64_t n_rows,
    const int64_t *__restrict__ state)
{
    const int64_t row = TABLE ? state[0] : 0;
    const int64_t b = blockIdx.x;
    if (b >= n_tiles) {
        adamw_piece<MATH, TABLE>(segs[b - n_tiles], 0, 1, wtab, scales, acc, master, exp_avg,
                                 exp_avg_sq, k_arg, S, table, row, n_rows);
        return;
    }
    if (b >= n_full)
        return;
    const uint32_t o = (uint32_t)threadIdx.x * 16u;
    const int64_t q0 = b * kWave;
    const char *ab = reinterpret_cast<const char *>(reinterpret_cast<const f32x4 *>(acc) + q0);
    char *pb = reinterpret_cast<char *>(reinterpret_cast<f32x4 *>(master) + q0);
    char *mb = reinterpret_cast<char *>(reinterpret_cast<f32x4 *>(exp_avg) + q0);
    char *vb = reinterpret_cast<char *>(reinterpret_cast<f32x4 *>(exp_avg_sq) + q0);
    const LaneVec x = load_lane(ab, pb, mb, vb, o);
    __builtin_amdgcn_sched_barrier(0);
    const int32_t tag = tags[b];
    AdamConsts k;
    if (!step_consts<TABLE>(k_arg, table, row, n_rows, k) || tag < 0) {
        discard_lane(x);
        return;
    }
    const double c = MATH ? clip_coef(k, S) : 1.0;
    const TensorRate tr = MATH ? tensor_rate(k, scales[tag]) : TensorRate{};
    // the bf16 weight of arena element e: the packed shard's element e, or
    // (full-size tensors) byte wdelta[tag] + 2e, the tensor's element
    // start + (e - arena offset)
    gmem<char> *wb;
    if constexpr (FULL)
        wb = reinterpret_cast<gmem<char> *>(wdelta[tag]) + q0 * 8;
    else
        wb = reinterpret_cast<gmem<char> *>(to_global(wbase)) + q0 * 8;
    update_store_lane<MATH>(x, pb, mb, vb, wb, o, k, tr, c);
}

// Runs after the scheduled AdamW launch on the same stream: the next replay
// takes the next row; a step asked for past the last row is counted.
__global__ __launch_bounds__(64) void k_schedule_advance(int64_t *__restrict__ state,
                                                         int64_t n_rows)
{
    if (threadIdx.x == 0) {
        const int64_t row = state[0];
        if (row < n_rows)
            state[0] = row + 1;
        else
            state[1] = state[1] + 1;
    }
}

// -------------------------------------------------------- probe copy ----
// Streaming copy, one 16-byte vector per lane and one workgroup per
// 256-vector tile (the loop runs more than once only when the tiles outnumber
// the largest grid).  Of the shapes measured on 4 GB buffers this one copied
// fastest: 6.5 TB/s, against 6.0-6.1 with 4 vectors per lane and 5.4 with a
// fixed grid of 8192 workgroups looping over the tiles.
__global__ __launch_bounds__(kBlock) void k_copy(const f32x4 *__restrict__ src,
                                                 f32x4 *__restrict__ dst, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock)
        st_stream(dst + i, ld_stream(src + i));
}


}  // namespace

hipError_t launch_accum(const LaunchGeom &geo, const uint16_t *const *grad_tab, float *acc,
                        DD *partials, bool first, bool last, hipStream_t s)
{
    if (geo.n_chunks == 0)
        return hipSuccess;
    if (slots_one_wave(geo, 1)) {
        const dim3 g1((unsigned)(geo.n_chunks * geo.sub)), b1(kWave);
        const int32_t ns = geo.sub;
        if (first && last)
            k_accum_slots_wave<true, true, false, 1><<<g1, b1, 0, s>>>(
                geo.chunks, geo.n_chunks, ns, grad_tab, 0, acc, partials, 1.0f);
        else if (first)
            k_accum_slots_wave<true, false, false, 1><<<g1, b1, 0, s>>>(
                geo.chunks, geo.n_chunks, ns, grad_tab, 0, acc, partials, 1.0f);
        else if (last)
            k_accum_slots_wave<false, true, false, 1><<<g1, b1, 0, s>>>(
                geo.chunks, geo.n_chunks, ns, grad_tab, 0, acc, partials, 1.0f);
        else
            k_accum_slots_wave<false, false, false, 1><<<g1, b1, 0, s>>>(
                geo.chunks, geo.n_chunks, ns, grad_tab, 0, acc, partials, 1.0f);
        return hipGetLastError();
    }
    const dim3 grid(geo.grid), block(kBlock);
    constexpr int U = Z1_UNROLL_ACC;
    if (first && last)
        k_accum<true, true, false, U><<<grid, block, 0, s>>>(geo.chunks, geo.n_chunks, grad_tab,
                                                             acc, partials, 1.0f);
    else if (first)
        k_accum<true, false, false, U><<<grid, block, 0, s>>>(geo.chunks, geo.n_chunks, grad_tab,
                                                              acc, partials, 1.0f);
    else if (last)
        k_accum<false, true, false, U><<<grid, block, 0, s>>>(geo.chunks, geo.n_chunks, grad_tab,
                                                              acc, partials, 1.0f);
    else
        k_accum<false, false, false, U><<<grid, block, 0, s>>>(geo.chunks, geo.n_chunks,
                                                               grad_tab, acc, partials, 1.0f);
    return hipGetLastError();
}

template <int G>
void launch_slots_g(const LaunchGeom &geo, const uint16_t *const *grad_tab, int32_t stride,
                    float *acc, DD *partials, bool first, bool last, bool divide, float dp,
                    hipStream_t s)
{
    if constexpr (G >= kSlotsOneWave) {
        if (slots_one_wave(geo, G)) {
            const dim3 g1((unsigned)(geo.n_chunks * geo.sub)), b1(kWave);
            const int32_t ns = geo.sub;
            if (first && last)
                k_accum_slots_wave<true, true, false, G><<<g1, b1, 0, s>>>(
                    geo.chunks, geo.n_chunks, ns, grad_tab, stride, acc, partials, dp);
            else if (last)
                k_accum_slots_wave<false, true, false, G><<<g1, b1, 0, s>>>(
                    geo.chunks, geo.n_chunks, ns, grad_tab, stride, acc, partials, dp);
            else if (first && divide)
                k_accum_slots_wave<true, false, true, G><<<g1, b1, 0, s>>>(
                    geo.chunks, geo.n_chunks, ns, grad_tab, stride, acc, partials, dp);
            else if (divide)
                k_accum_slots_wave<false, false, true, G><<<g1, b1, 0, s>>>(
                    geo.chunks, geo.n_chunks, ns, grad_tab, stride, acc, partials, dp);
            else if (first)
                k_accum_slots_wave<true, false, false, G><<<g1, b1, 0, s>>>(
                    geo.chunks, geo.n_chunks, ns, grad_tab, stride, acc, partials, dp);
            else
                k_accum_slots_wave<false, false, false, G><<<g1, b1, 0, s>>>(
                    geo.chunks, geo.n_chunks, ns, grad_tab, stride, acc, partials, dp);
            return;
        }
    }
    const dim3 grid(geo.grid), block(kBlock);
    constexpr int U = G <= 6 ? Z1_UNROLL_ACC : Z1_UNROLL_SLOTS_WIDE;
    // the norm (last) and the division (divide) are never asked for together
    if (first && last)
        k_accum_slots<true, true, false, G, U><<<grid, block, 0, s>>>(
            geo.chunks, geo.n_chunks, grad_tab, stride, acc, partials, dp);
    else if (last)
        k_accum_slots<false, true, false, G, U><<<grid, block, 0, s>>>(
            geo.chunks, geo.n_chunks, grad_tab, stride, acc, partials, dp);
    else if (first && divide)
        k_accum_slots<true, false, true, G, U><<<grid, block, 0, s>>>(
            geo.chunks, geo.n_chunks, grad_tab, stride, acc, partials, dp);
    else if (divide)
        k_accum_slots<false, false, true, G, U><<<grid, block, 0, s>>>(
            geo.chunks, geo.n_chunks, grad_tab, stride, acc, partials, dp);
    else if (first)
        k_accum_slots<true, false, false, G, U><<<grid, block, 0, s>>>(
            geo.chunks, geo.n_chunks, grad_tab, stride, acc, partials, dp);
    else
        k_accum_slots<false, false, false, G, U><<<grid, block, 0, s>>>(
            geo.chunks, geo.n_chunks, grad_tab, stride, acc, partials, dp);
}

hipError_t launch_pack(const LaunchGeom &geo, const uint16_t *const *grad_tab, float *send,
                       bool first, bool divide, float dp, hipStream_t s)
{
    if (geo.n_chunks == 0)
        return hipSuccess;
    if (slots_one_wave(geo, 1)) {
        const dim3 g1((unsigned)(geo.n_chunks * geo.sub)), b1(kWave);
        const int32_t ns = geo.sub;
        if (first && divide)
            k_accum_slots_wave<true, false, true, 1><<<g1, b1, 0, s>>>(
                geo.chunks, geo.n_chunks, ns, grad_tab, 0, send, nullptr, dp);
        else if (first)
            k_accum_slots_wave<true, false, false, 1><<<g1, b1, 0, s>>>(
                geo.chunks, geo.n_chunks, ns, grad_tab, 0, send, nullptr, dp);
        else if (divide)
            k_accum_slots_wave<false, false, true, 1><<<g1, b1, 0, s>>>(
                geo.chunks, geo.n_chunks, ns, grad_tab, 0, send, nullptr, dp);
        else
            k_accum_slots_wave<false, false, false, 1><<<g1, b1, 0, s>>>(
                geo.chunks, geo.n_chunks, ns, grad_tab, 0, send, nullptr, dp);
        return hipGetLastError();
    }
    const dim3 grid(geo.grid), block(kBlock);
    constexpr int U = Z1_UNROLL_ACC;
    if (first && divide)
        k_accum<true, false, true, U><<<grid, block, 0, s>>>(geo.chunks, geo.n_chunks, grad_tab,
                                                             send, nullptr, dp);
    else if (first)
        k_accum<true, false, false, U><<<grid, block, 0, s>>>(geo.chunks, geo.n_chunks, grad_tab,
                                                              send, nullptr, dp);
    else if (divide)
        k_accum<false, false, true, U><<<grid, block, 0, s>>>(geo.chunks, geo.n_chunks, grad_tab,
                                                              send, nullptr, dp);
    else
        k_accum<false, false, false, U><<<grid, block, 0, s>>>(geo.chunks, geo.n_chunks,
                                                               grad_tab, send, nullptr, dp);
    return hipGetLastError();
}

hipError_t launch_accum_slots(const LaunchGeom &geo, const uint16_t *const *grad_tab,
                              int32_t slot_stride, int n_slots, float *acc, DD *partials,
                              bool first, bool last, bool divide, float dp, hipStream_t s)
{
    if (geo.n_chunks == 0)
        return hipSuccess;
    if (last && divide)
        return hipErrorInvalidValue;
    static_assert(kMaxSlots == 16, "one case per slot count 2..kMaxSlots");
    switch (n_slots) {
    case 2: launch_slots_g<2>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 3: launch_slots_g<3>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 4: launch_slots_g<4>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 5: launch_slots_g<5>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 6: launch_slots_g<6>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 7: launch_slots_g<7>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 8: launch_slots_g<8>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 9: launch_slots_g<9>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 10: launch_slots_g<10>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 11: launch_slots_g<11>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 12: launch_slots_g<12>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 13: launch_slots_g<13>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 14: launch_slots_g<14>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 15: launch_slots_g<15>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    case 16: launch_slots_g<16>(geo, grad_tab, slot_stride, acc, partials, first, last, divide, dp, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int G>
void launch_arena_g(const LaunchGeom &geo, const SlotBases &sb, float *acc, DD *partials,
                    bool first, bool last, hipStream_t s)
{
    const ArenaWalk &aw = geo.arena;
    const dim3 grid((unsigned)(aw.n_tiles + aw.n_segs)), block(kWave);
    if (first && last)
        k_accum_arena<true, true, G><<<grid, block, 0, s>>>(sb, aw.tags, aw.segs, aw.n_tiles,
                                                             aw.n_full, acc, partials);
    else if (first)
        k_accum_arena<true, false, G><<<grid, block, 0, s>>>(sb, aw.tags, aw.segs, aw.n_tiles,
                                                              aw.n_full, acc, partials);
    else if (last)
        k_accum_arena<false, true, G><<<grid, block, 0, s>>>(sb, aw.tags, aw.segs, aw.n_tiles,
                                                              aw.n_full, acc, partials);
    else
        k_accum_arena<false, false, G><<<grid, block, 0, s>>>(sb, aw.tags, aw.segs, aw.n_tiles,
                                                               aw.n_full, acc, partials);
}

hipError_t launch_accum_arena(const LaunchGeom &geo, const SlotBases &sb, int n_slots,
                              float *acc, DD *partials, bool first, bool last, hipStream_t s)
{
    if (!slots_arena(geo, n_slots))
        return hipErrorInvalidValue;
    static_assert(kMaxSlots == 16 && kSlotsOneWave == 8, "one case per slot count 1, 8..16");
    switch (n_slots) {
    case 1: launch_arena_g<1>(geo, sb, acc, partials, first, last, s); break;
    case 8: launch_arena_g<8>(geo, sb, acc, partials, first, last, s); break;
    case 9: launch_arena_g<9>(geo, sb, acc, partials, first, last, s); break;
    case 10: launch_arena_g<10>(geo, sb, acc, partials, first, last, s); break;
    case 11: launch_arena_g<11>(geo, sb, acc, partials, first, last, s); break;
    case 12: launch_arena_g<12>(geo, sb, acc, partials, first, last, s); break;
    case 13: launch_arena_g<13>(geo, sb, acc, partials, first, last, s); break;
    case 14: launch_arena_g<14>(geo, sb, acc, partials, first, last, s); break;
    case 15: launch_arena_g<15>(geo, sb, acc, partials, first, last, s); break;
    case 16: launch_arena_g<16>(geo, sb, acc, partials, first, last, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_norm_acc(const LaunchGeom &geo, const float *acc, DD *partials, hipStream_t s)
{
    if (geo.n_chunks == 0)
        return hipSuccess;
    k_norm_acc<Z1_UNROLL_ACC><<<dim3(geo.grid), dim3(kBlock), 0, s>>>(geo.chunks, geo.n_chunks,
                                                                      acc, partials);
    return hipGetLastError();
}

hipError_t launch_norm_fin(const DD *partials, int64_t n_chunks, DD *stage,
                           unsigned int *counter, double *S, hipStream_t s, DD *pair)
{
    // about 8 partials per thread per stage-1 workgroup, at most kFinStages
    int64_t g = (n_chunks + 8 * kFinBlock - 1) / (8 * kFinBlock);
    if (g < 1)
        g = 1;
    if (g > kFinStages)
        g = kFinStages;
    k_norm_fin<<<dim3((unsigned)g), dim3(kFinBlock), 0, s>>>(partials, n_chunks, stage, counter,
                                                             S, pair);
    return hipGetLastError();
}

hipError_t launch_norm_flat(const float *acc, int64_t n, DD *partials, DD *stage,
                           unsigned int *counter, double *S, hipStream_t s)
{
    const int64_t tiles = (n + kTileElems - 1) / kTileElems;
    k_norm_flat<<<dim3((unsigned)(tiles > 0 ? tiles : 1)), dim3(kBlock), 0, s>>>(acc, n, partials,
                                                                              counter);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_norm_fin(partials, tiles, stage, counter, S, s);
}

hipError_t launch_norm_combine(const DD *pairs, int32_t n, double *S, hipStream_t s)
{
    k_norm_combine<<<dim3(1), dim3(64), 0, s>>>(pairs, n, S);
    return hipGetLastError();
}

// AdamW over a plan: the arena walk, or the chunk table with one workgroup
// per (piece, sub) (the loop-free variant) or a capped grid looping over
// them; every launch reserves geo.adam_lds bytes of LDS per workgroup.
template <bool MATH, bool TABLE>
void launch_adamw_kernel(const LaunchGeom &geo, uint16_t *const *weight_tab, const Scale *scales,
                         const float *acc, float *master, float *m, float *v,
                         const AdamConsts &k, const double *S, const AdamConsts *table,
                         int64_t n_rows, const int64_t *state, hipStream_t s)
{
    const dim3 block(kWave);
    const size_t lds = geo.adam_lds;
    if (geo.arena.n_tiles > 0) {
        const ArenaWalk &aw = geo.arena;
        const dim3 grid((unsigned)(aw.n_tiles + aw.n_segs));
        if (aw.wdelta)
            k_adamw_tiles<MATH, TABLE, true><<<grid, block, lds, s>>>(
                aw.tags, aw.segs, aw.n_tiles, aw.n_full, nullptr, aw.wdelta, weight_tab, scales,
                acc, master, m, v, k, S, table, n_rows, state);
        else
            k_adamw_tiles<MATH, TABLE, false><<<grid, block, lds, s>>>(
                aw.tags, aw.segs, aw.n_tiles, aw.n_full, aw.wbase, nullptr, weight_tab, scales,
                acc, master, m, v, k, S, table, n_rows, state);
        return;
    }
    const int64_t n_work = geo.n_chunks * geo.sub;
    if (geo.adam_grid < n_work)
        k_adamw<MATH, TABLE, false><<<dim3((unsigned)geo.adam_grid), block, lds, s>>>(
            geo.chunks, n_work, geo.sub, weight_tab, scales, acc, master, m, v, k, S, table,
            n_rows, state);
    else
        k_adamw<MATH, TABLE, true><<<dim3((unsigned)n_work), block, lds, s>>>(
            geo.chunks, n_work, geo.sub, weight_tab, scales, acc, master, m, v, k, S, table,
            n_rows, state);
}

hipError_t launch_adamw(const LaunchGeom &geo, uint16_t *const *weight_tab, const Scale *scales,
                        const float *acc, float *master, float *m, float *v,
                        const AdamConsts &k, const double *S, hipStream_t s)
{
    if (geo.n_chunks == 0)
        return hipSuccess;
    launch_adamw_kernel<true, false>(geo, weight_tab, scales, acc, master, m, v, k, S, nullptr,
                                     0, nullptr, s);
    return hipGetLastError();
}

hipError_t launch_adamw_scheduled(const LaunchGeom &geo, uint16_t *const *weight_tab,
                                  const Scale *scales, const float *acc, float *master, float *m,
                                  float *v, const AdamConsts *table, int64_t n_rows,
                                  int64_t *state, const double *S, hipStream_t s)
{
    if (geo.n_chunks > 0)
        launch_adamw_kernel<true, true>(geo, weight_tab, scales, acc, master, m, v, AdamConsts{},
                                        S, table, n_rows, state, s);
    k_schedule_advance<<<dim3(1), dim3(64), 0, s>>>(state, n_rows);
    return hipGetLastError();
}

hipError_t launch_adamw_traffic(const LaunchGeom &geo, uint16_t *const *weight_tab,
                                const float *acc, float *master, float *m, float *v,
                                hipStream_t s)
{
    if (geo.n_chunks == 0)
        return hipSuccess;
    launch_adamw_kernel<false, false>(geo, weight_tab, nullptr, acc, master, m, v, AdamConsts{},
                                      nullptr, nullptr, 0, nullptr, s);
    return hipGetLastError();
}

hipError_t launch_copy(const void *src, void *dst, int64_t n_bytes, hipStream_t s)
{
    const int64_t n = n_bytes / 16;
    if (n == 0)
        return hipSuccess;
    int64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > INT32_MAX)
        blocks = INT32_MAX;
    k_copy<<<dim3((unsigned)blocks), dim3(kBlock), 0, s>>>(
        static_cast<const f32x4 *>(src), static_cast<f32x4 *>(dst), n);
    return hipGetLastError();
}

}  // namespace z1
