// z1_probe.hip -- measurement aids (not part of the step): streaming kernels
// with the traffic of the step's kernels and no arithmetic, so a benchmark can
// report the HBM bandwidth this machine reaches for each traffic mix next to
// what the step's kernels reach.  The default shape is the step kernels' own:
// 256-thread workgroups, 4 x 16-byte vectors per lane, non-temporal loads and
// stores, one 1024-vector tile per workgroup.  Two mixes also come in the
// shape at which they stream fastest without arithmetic (measured on the 7B
// shard's buffers): the AdamW mix in one-wave workgroups (3.5-4% above the
// default shape) and the resident-slot mix with one vector per lane.
#include "z1.h"
#include "z1_internal.h"

namespace z1 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kTileVec = 4 * kBlock;

template <typename T>
__device__ __forceinline__ T ld(const T *p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void st(T *p, T x) { __builtin_nontemporal_store(x, p); }

// Reads every vector; the sum feeds a store that only happens for an
// impossible value, so the loads stay live.
__global__ __launch_bounds__(kBlock) void k_probe_read(const f32x4 *__restrict__ src, int64_t n,
                                                       float *__restrict__ sink)
{
    const int64_t base = (int64_t)blockIdx.x * kTileVec + threadIdx.x;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i = base + u * kBlock;
        if (i < n) {
            const f32x4 x = ld(src + i);
            acc += x.x + x.y + x.z + x.w;
        }
    }
    if (acc == -1234.5f)
        sink[0] = acc;
}

__global__ __launch_bounds__(kBlock) void k_probe_write(f32x4 *__restrict__ dst, int64_t n)
{
    const int64_t base = (int64_t)blockIdx.x * kTileVec + threadIdx.x;
    const f32x4 z = {1.f, 2.f, 3.f, 4.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i = base + u * kBlock;
        if (i < n)
            st(dst + i, z);
    }
}

// k_adamw's traffic: read a, p, m, v; write p, m, v and a half-width w.
// NT lanes per workgroup, 4 vectors per lane (a 4 * NT-vector tile).
template <int NT>
__global__ __launch_bounds__(NT) void k_probe_adamw(const f32x4 *__restrict__ a,
                                                    f32x4 *__restrict__ p,
                                                    f32x4 *__restrict__ m,
                                                    f32x4 *__restrict__ v,
                                                    u32x2 *__restrict__ w, int64_t n)
{
    const int64_t base = (int64_t)blockIdx.x * (4 * NT) + threadIdx.x;
    f32x4 ar[4], pr[4], mr[4], vr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i = base + u * NT;
        if (i < n) {
            ar[u] = ld(a + i);
            pr[u] = ld(p + i);
            mr[u] = ld(m + i);
            vr[u] = ld(v + i);
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i = base + u * NT;
        if (i < n) {
            st(p + i, pr[u] + ar[u]);
            st(m + i, mr[u] + ar[u]);
            st(v + i, vr[u] + ar[u]);
            u32x2 wb;
            wb.x = __float_as_uint(pr[u].x);
            wb.y = __float_as_uint(pr[u].y);
            st(w + i, wb);
        }
    }
}

// The same traffic in one-wave workgroups with one vector per lane, the
// launch reserving LDS so that at most kProbeAdamPerCU workgroups share a
// compute unit: the shape and residency at which this mix streams fastest
// without arithmetic (measured on the 7B shard's buffers: 10-12 per compute
// unit best, 6.3-6.6 TB/s, against 5.8-6.2 with no cap).
constexpr int kProbeAdamPerCU = 12;

__global__ __launch_bounds__(kWave) void k_probe_adamw_one(const f32x4 *__restrict__ a,
                                                           f32x4 *__restrict__ p,
                                                           f32x4 *__restrict__ m,
                                                           f32x4 *__restrict__ v,
                                                           u32x2 *__restrict__ w, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * kWave + threadIdx.x;
    if (i < n) {
        const f32x4 ar = ld(a + i), pr = ld(p + i), mr = ld(m + i), vr = ld(v + i);
        st(p + i, pr + ar);
        st(m + i, mr + ar);
        st(v + i, vr + ar);
        u32x2 wb;
        wb.x = __float_as_uint(pr.x);
        wb.y = __float_as_uint(pr.y);
        st(w + i, wb);
    }
}

// k_accum's traffic (k >= 1): read a half-width g and acc, write acc.
__global__ __launch_bounds__(kBlock) void k_probe_accum(const u32x2 *__restrict__ g,
                                                        f32x4 *__restrict__ acc, int64_t n)
{
    const int64_t base = (int64_t)blockIdx.x * kTileVec + threadIdx.x;
    u32x2 gr[4];
    f32x4 ar[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i = base + u * kBlock;
        if (i < n) {
            gr[u] = ld(g + i);
            ar[u] = ld(acc + i);
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i = base + u * kBlock;
        if (i < n) {
            f32x4 s = ar[u];
            s.x += __uint_as_float(gr[u].x << 16);
            s.y += __uint_as_float(gr[u].y << 16);
            st(acc + i, s);
        }
    }
}

// The first resident-slot pass's traffic: read G half-width streams, write
// one fp32 stream (2G + 4 bytes per element); the G pointers come by value.
// R rounds of U vectors per lane over an R * U * NT-vector tile per
// workgroup of NT lanes: as in the 256-lane accumulation kernel (U = 4 up to
// 6 slots, 2 above, over a 1024-vector tile), or one-wave workgroups of one
// vector per lane and one round (the shape of the wide passes).
struct SlotPtrs {
    const u32x2 *p[kMaxSlots];
};

template <int G, int U, int R, int NT>
__global__ __launch_bounds__(NT) void k_probe_slots(SlotPtrs sp, f32x4 *__restrict__ acc,
                                                    int64_t n)
{
    const int64_t tile = (int64_t)blockIdx.x * (R * U * NT) + threadIdx.x;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t base = tile + (int64_t)r * U * NT;
        u32x2 gr[G][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * NT;
            if (i < n) {
#pragma unroll
                for (int j = 0; j < G; ++j)
                    gr[j][u] = ld(sp.p[j] + i);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * NT;
            if (i < n) {
                f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    s.x += __uint_as_float(gr[j][u].x << 16);
                    s.y += __uint_as_float(gr[j][u].y << 16);
                }
                st(acc + i, s);
            }
        }
    }
}

template <int G>
void launch_slots_probe(void *const *bufs, int64_t n_vec, bool one, hipStream_t s)
{
    SlotPtrs sp{};
    for (int j = 0; j < G; ++j)
        sp.p[j] = static_cast<const u32x2 *>(bufs[j]);
    f32x4 *acc = static_cast<f32x4 *>(bufs[G]);
    if (one) {
        k_probe_slots<G, 1, 1, kWave><<<dim3((unsigned)((n_vec + kWave - 1) / kWave)),
                                        dim3(kWave), 0, s>>>(sp, acc, n_vec);
    } else {
        constexpr int U = G <= 6 ? 4 : 2;
        k_probe_slots<G, U, 4 / U, kBlock><<<dim3((unsigned)((n_vec + kTileVec - 1) / kTileVec)),
                                             dim3(kBlock), 0, s>>>(sp, acc, n_vec);
    }
}

}  // namespace
}  // namespace z1

extern "C" z1_status z1_probe(int32_t kind, void *const *bufs, int32_t n_bufs, int64_t n_vec,
                              z1_stream stream)
{
    using namespace z1;
    static const int32_t need[] = {2, 1, 5, 2, 3, 5, 3};
    if (kind < Z1_PROBE_READ || kind > Z1_PROBE_SLOTS_TRAFFIC_ONE || !bufs || n_vec < 0 ||
        n_bufs < need[kind])
        return Z1_EINVAL;
    const bool slots = kind == Z1_PROBE_SLOTS_TRAFFIC || kind == Z1_PROBE_SLOTS_TRAFFIC_ONE;
    if (slots && n_bufs > kMaxSlots + 1)
        return Z1_EINVAL;
    const int32_t used = slots ? n_bufs : need[kind];
    for (int32_t i = 0; i < used; ++i) {
        if (!bufs[i])
            return Z1_EINVAL;
        if (reinterpret_cast<uintptr_t>(bufs[i]) % 16 != 0)
            return Z1_EALIGN;
    }
    if (n_vec == 0)
        return Z1_OK;
    // workgroups of the finest shape (64 vectors each) must fit the grid
    const int64_t blocks = (n_vec + kTileVec - 1) / kTileVec;
    if ((n_vec + kWave - 1) / kWave > INT32_MAX)
        return Z1_EINVAL;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)blocks), block(kBlock);
    switch (kind) {
    case Z1_PROBE_READ:
        k_probe_read<<<grid, block, 0, s>>>(static_cast<const f32x4 *>(bufs[0]), n_vec,
                                            static_cast<float *>(bufs[1]));
        break;
    case Z1_PROBE_WRITE:
        k_probe_write<<<grid, block, 0, s>>>(static_cast<f32x4 *>(bufs[0]), n_vec);
        break;
    case Z1_PROBE_ADAMW_TRAFFIC:
        k_probe_adamw<kBlock><<<grid, block, 0, s>>>(
            static_cast<const f32x4 *>(bufs[0]), static_cast<f32x4 *>(bufs[1]),
            static_cast<f32x4 *>(bufs[2]), static_cast<f32x4 *>(bufs[3]),
            static_cast<u32x2 *>(bufs[4]), n_vec);
        break;
    case Z1_PROBE_ADAMW_TRAFFIC_WAVE: {
        int dev = 0, lds_per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                  dev) != hipSuccess || lds_per_cu < 0)
            return Z1_EHIP;
        k_probe_adamw_one<<<dim3((unsigned)((n_vec + kWave - 1) / kWave)), dim3(kWave),
                            (size_t)(lds_per_cu / kProbeAdamPerCU), s>>>(
            static_cast<const f32x4 *>(bufs[0]), static_cast<f32x4 *>(bufs[1]),
            static_cast<f32x4 *>(bufs[2]), static_cast<f32x4 *>(bufs[3]),
            static_cast<u32x2 *>(bufs[4]), n_vec);
        break;
    }
    case Z1_PROBE_ACCUM_TRAFFIC:
        k_probe_accum<<<grid, block, 0, s>>>(static_cast<const u32x2 *>(bufs[0]),
                                             static_cast<f32x4 *>(bufs[1]), n_vec);
        break;
    default: {
        const bool one = kind == Z1_PROBE_SLOTS_TRAFFIC_ONE;
        static_assert(kMaxSlots == 16, "one case per slot count 2..kMaxSlots");
        switch (n_bufs - 1) {
        case 2: launch_slots_probe<2>(bufs, n_vec, one, s); break;
        case 3: launch_slots_probe<3>(bufs, n_vec, one, s); break;
        case 4: launch_slots_probe<4>(bufs, n_vec, one, s); break;
        case 5: launch_slots_probe<5>(bufs, n_vec, one, s); break;
        case 6: launch_slots_probe<6>(bufs, n_vec, one, s); break;
        case 7: launch_slots_probe<7>(bufs, n_vec, one, s); break;
        case 8: launch_slots_probe<8>(bufs, n_vec, one, s); break;
        case 9: launch_slots_probe<9>(bufs, n_vec, one, s); break;
        case 10: launch_slots_probe<10>(bufs, n_vec, one, s); break;
        case 11: launch_slots_probe<11>(bufs, n_vec, one, s); break;
        case 12: launch_slots_probe<12>(bufs, n_vec, one, s); break;
        case 13: launch_slots_probe<13>(bufs, n_vec, one, s); break;
        case 14: launch_slots_probe<14>(bufs, n_vec, one, s); break;
        case 15: launch_slots_probe<15>(bufs, n_vec, one, s); break;
        default: launch_slots_probe<16>(bufs, n_vec, one, s); break;
        }
        break;
    }
    }
    return hipGetLastError() == hipSuccess ? Z1_OK : Z1_EHIP;
}
