// z1_kernels.hip -- gfx950 kernels of the ZeRO-1 shard optimizer step.
//
// The step is a streaming, HBM-bound pass over one rank's shard (about 0.5
// flop per byte), so nothing here uses MFMA.  Each kernel walks a
// device-resident chunk table: a workgroup takes one piece of one tensor's
// slice, its lanes move 4 consecutive elements each with one 16-byte fp32
// access per arena and one 8-byte bf16 access, consecutive lanes on
// consecutive addresses.  The fp32 arenas are laid out so that an arena
// element and its bf16 element share their position within a vector; only
// the first and last vector of a slice can be partial and take a per-element
// path.
//
// Arithmetic follows the definition exactly (this file is built with
// -ffp-contract=off and without fast-math):
//   * accumulation is one binary32 add per micro-batch, in order;
//   * the squared norm is an exact-square, double-double sum;
//   * AdamW is evaluated in binary64 with the same operation sequence as the
//     definition (separate multiply and add, IEEE division and square root),
//     then rounded once to binary32 and, for the weight, to bf16 (nearest
//     even).
#include "z1_internal.h"

namespace z1 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ void dd_add(double &hi, double &lo, double bhi, double blo)
{
    double s, e;
    two_sum(hi, bhi, s, e);
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

__device__ __forceinline__ double shfl_xor_d(double x, int mask)
{
    return __shfl_xor(x, mask, 64);
}

// Fixed-order reduction of a double-double across the workgroup; every
// combine is symmetric in its operands, so the butterfly leaves the same
// value in every lane and the result depends only on the inputs' placement.
template <int NT>
__device__ __forceinline__ void block_reduce_dd(double &hi, double &lo, DD *lds)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double ohi = shfl_xor_d(hi, off);
        const double olo = shfl_xor_d(lo, off);
        dd_add(hi, lo, ohi, olo);
    }
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
// acc = (FIRST ? 0 : acc) + float(g); LAST also sums acc^2 per chunk.
template <bool FIRST, bool LAST, int U>
__global__ __launch_bounds__(kBlock) void k_accum(const Chunk *__restrict__ chunks,
                                                  int64_t n_chunks,
                                                  const uint16_t *const *__restrict__ gtab,
                                                  float *__restrict__ acc,
                                                  DD *__restrict__ partials)
{
    __shared__ DD lds[kBlock / 64];
    for (int64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
        const Chunk ch = chunks[c];
        const int lead = (int)(ch.src & (kVec - 1));
        const int end = lead + ch.count;
        const int nv = (end + kVec - 1) / kVec;
        const uint16_t *g = gtab[ch.tensor] + (ch.src - lead);
        float *a = acc + (ch.dst - lead);
        double hi = 0.0, lo = 0.0;

        for (int base = 0; base < nv; base += kBlock * U) {
            u32x2 gr[U];
            f32x4 ar[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e0 = (base + u * kBlock + (int)threadIdx.x) * kVec;
                if (e0 >= lead && e0 + kVec <= end) {
                    gr[u] = *reinterpret_cast<const u32x2 *>(g + e0);
                    if (!FIRST)
                        ar[u] = *reinterpret_cast<const f32x4 *>(a + e0);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e0 = (base + u * kBlock + (int)threadIdx.x) * kVec;
                if (e0 >= end)
                    continue;
                if (e0 >= lead && e0 + kVec <= end) {
                    f32x4 s;
                    s.x = bf16_lo(gr[u].x);
                    s.y = bf16_hi(gr[u].x);
                    s.z = bf16_lo(gr[u].y);
                    s.w = bf16_hi(gr[u].y);
                    if (!FIRST) {
                        s.x = ar[u].x + s.x;
                        s.y = ar[u].y + s.y;
                        s.z = ar[u].z + s.z;
                        s.w = ar[u].w + s.w;
                    }
                    *reinterpret_cast<f32x4 *>(a + e0) = s;
                    if (LAST) {
                        dd_add_sq(hi, lo, s.x);
                        dd_add_sq(hi, lo, s.y);
                        dd_add_sq(hi, lo, s.z);
                        dd_add_sq(hi, lo, s.w);
                    }
                } else {
                    for (int j = 0; j < kVec; ++j) {
                        const int e = e0 + j;
                        if (e < lead || e >= end)
                            continue;
                        float s = __uint_as_float((uint32_t)g[e] << 16);
                        if (!FIRST)
                            s = a[e] + s;
                        a[e] = s;
                        if (LAST)
                            dd_add_sq(hi, lo, s);
                    }
                }
            }
        }
        if (LAST) {
            block_reduce_dd<kBlock>(hi, lo, lds);
            if (threadIdx.x == 0)
                partials[c] = DD{hi, lo};
        }
    }
}

// ------------------------------------------------------ norm finalise ----
__global__ __launch_bounds__(kFinBlock) void k_norm_fin(const DD *__restrict__ partials,
                                                        int64_t n, double *__restrict__ S)
{
    __shared__ DD lds[kFinBlock / 64];
    double hi = 0.0, lo = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += kFinBlock) {
        const DD p = partials[i];
        dd_add(hi, lo, p.hi, p.lo);
    }
    block_reduce_dd<kFinBlock>(hi, lo, lds);
    if (threadIdx.x == 0)
        S[0] = hi + lo;
}

// -------------------------------------------------------------- AdamW ----
struct Elem {
    float p, m, v;
};

// One element of the step in binary64 (see the header comment of z1.h for
// the formula); the operation order matches the definition term by term.
__device__ __forceinline__ Elem adamw_elem(float acc, float p32, float m32, float v32,
                                           const AdamConsts &k, double c)
{
    const double g = c * (double)acc;
    double p = (double)p32;
    double m = (double)m32;
    double v = (double)v32;
    p = p * k.decay;
    m = k.beta1 * m + k.omb1 * g;
    v = k.beta2 * v + k.omb2 * g * g;
    const double mhat = m / k.bc1;
    const double vhat = v / k.bc2;
    p = p - k.lr * mhat / (sqrt(vhat) + k.eps);
    return Elem{(float)p, (float)m, (float)v};
}

template <int U>
__global__ __launch_bounds__(kBlock) void k_adamw(const Chunk *__restrict__ chunks,
                                                  int64_t n_chunks,
                                                  uint16_t *const *__restrict__ wtab,
                                                  const float *__restrict__ acc,
                                                  float *__restrict__ master,
                                                  float *__restrict__ exp_avg,
                                                  float *__restrict__ exp_avg_sq,
                                                  const AdamConsts k,
                                                  const double *__restrict__ S)
{
    double c = 1.0;
    if (k.clip > 0.0) {
        const double cc = k.clip / (sqrt(S[0]) + 1e-6);
        c = cc < 1.0 ? cc : 1.0;
    }
    for (int64_t ci = blockIdx.x; ci < n_chunks; ci += gridDim.x) {
        const Chunk ch = chunks[ci];
        const int lead = (int)(ch.src & (kVec - 1));
        const int end = lead + ch.count;
        const int nv = (end + kVec - 1) / kVec;
        uint16_t *w = wtab[ch.tensor] + (ch.src - lead);
        const int64_t off = ch.dst - lead;
        const float *a = acc + off;
        float *p = master + off;
        float *m = exp_avg + off;
        float *v = exp_avg_sq + off;

        for (int base = 0; base < nv; base += kBlock * U) {
            f32x4 ar[U], pr[U], mr[U], vr[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e0 = (base + u * kBlock + (int)threadIdx.x) * kVec;
                if (e0 >= lead && e0 + kVec <= end) {
                    ar[u] = *reinterpret_cast<const f32x4 *>(a + e0);
                    pr[u] = *reinterpret_cast<const f32x4 *>(p + e0);
                    mr[u] = *reinterpret_cast<const f32x4 *>(m + e0);
                    vr[u] = *reinterpret_cast<const f32x4 *>(v + e0);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e0 = (base + u * kBlock + (int)threadIdx.x) * kVec;
                if (e0 >= end)
                    continue;
                if (e0 >= lead && e0 + kVec <= end) {
                    f32x4 po, mo, vo;
                    Elem r;
                    r = adamw_elem(ar[u].x, pr[u].x, mr[u].x, vr[u].x, k, c);
                    po.x = r.p; mo.x = r.m; vo.x = r.v;
                    r = adamw_elem(ar[u].y, pr[u].y, mr[u].y, vr[u].y, k, c);
                    po.y = r.p; mo.y = r.m; vo.y = r.v;
                    r = adamw_elem(ar[u].z, pr[u].z, mr[u].z, vr[u].z, k, c);
                    po.z = r.p; mo.z = r.m; vo.z = r.v;
                    r = adamw_elem(ar[u].w, pr[u].w, mr[u].w, vr[u].w, k, c);
                    po.w = r.p; mo.w = r.m; vo.w = r.v;
                    *reinterpret_cast<f32x4 *>(p + e0) = po;
                    *reinterpret_cast<f32x4 *>(m + e0) = mo;
                    *reinterpret_cast<f32x4 *>(v + e0) = vo;
                    u32x2 wb;
                    wb.x = bf16_rne(po.x) | (bf16_rne(po.y) << 16);
                    wb.y = bf16_rne(po.z) | (bf16_rne(po.w) << 16);
                    *reinterpret_cast<u32x2 *>(w + e0) = wb;
                } else {
                    for (int j = 0; j < kVec; ++j) {
                        const int e = e0 + j;
                        if (e < lead || e >= end)
                            continue;
                        const Elem r = adamw_elem(a[e], p[e], m[e], v[e], k, c);
                        p[e] = r.p;
                        m[e] = r.m;
                        v[e] = r.v;
                        w[e] = (uint16_t)bf16_rne(r.p);
                    }
                }
            }
        }
    }
}

// -------------------------------------------------------- probe copy ----
__global__ __launch_bounds__(kBlock) void k_copy(const f32x4 *__restrict__ src,
                                                 f32x4 *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

constexpr int kUnroll = 2;

}  // namespace

hipError_t launch_accum(const LaunchGeom &geo, const uint16_t *const *grad_tab, float *acc,
                        DD *partials, bool first, bool last, hipStream_t s)
{
    if (geo.n_chunks == 0)
        return hipSuccess;
    const dim3 grid(geo.grid), block(kBlock);
    if (first && last)
        k_accum<true, true, kUnroll><<<grid, block, 0, s>>>(geo.chunks, geo.n_chunks, grad_tab,
                                                            acc, partials);
    else if (first)
        k_accum<true, false, kUnroll><<<grid, block, 0, s>>>(geo.chunks, geo.n_chunks, grad_tab,
                                                             acc, partials);
    else if (last)
        k_accum<false, true, kUnroll><<<grid, block, 0, s>>>(geo.chunks, geo.n_chunks, grad_tab,
                                                             acc, partials);
    else
        k_accum<false, false, kUnroll><<<grid, block, 0, s>>>(geo.chunks, geo.n_chunks,
                                                              grad_tab, acc, partials);
    return hipGetLastError();
}

hipError_t launch_norm_fin(const DD *partials, int64_t n_chunks, double *S, hipStream_t s)
{
    k_norm_fin<<<dim3(1), dim3(kFinBlock), 0, s>>>(partials, n_chunks, S);
    return hipGetLastError();
}

hipError_t launch_adamw(const LaunchGeom &geo, uint16_t *const *weight_tab, const float *acc,
                        float *master, float *m, float *v, const AdamConsts &k,
                        const double *S, hipStream_t s)
{
    if (geo.n_chunks == 0)
        return hipSuccess;
    k_adamw<kUnroll><<<dim3(geo.grid), dim3(kBlock), 0, s>>>(geo.chunks, geo.n_chunks,
                                                             weight_tab, acc, master, m, v, k, S);
    return hipGetLastError();
}

hipError_t launch_copy(const void *src, void *dst, int64_t n_bytes, hipStream_t s)
{
    const int64_t n = n_bytes / 16;
    if (n == 0)
        return hipSuccess;
    int64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 256 * 32)
        blocks = 256 * 32;
    k_copy<<<dim3((unsigned)blocks), dim3(kBlock), 0, s>>>(
        static_cast<const f32x4 *>(src), static_cast<f32x4 *>(dst), n);
    return hipGetLastError();
}

}  // namespace z1
