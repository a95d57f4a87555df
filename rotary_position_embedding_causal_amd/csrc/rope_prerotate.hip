// rope_prerotate.hip -- the pre-rotation pass: q_rot = RoPE(q), k_rot = RoPE(k).
//
// "AttnFuse Makes RoPE a First-Class Attention Compilation Operation",
// paragraph 3, models pre-rotation as a memory-bandwidth cost: every query and
// key element is read once and written once. This kernel is a pure HBM stream
// sized for that: each lane moves 16-byte chunks, and the cos/sin table entries
// a lane needs depend only on (position, chunk), so a lane loads them once and
// reuses them across a group of heads, keeping the table's share of the
// traffic small next to Q and K.
//
// Q, K, Q' and K' are touched once, so their loads and stores are
// non-temporal (streaming) accesses: with a cold cache (the pages' protocol
// clears it before each timed call) that took the pass from 3.7-4.2 TB/s to
// 5.1-5.7 TB/s on MI355X at 160-320 MiB per call, above a plain device copy
// of the same bytes (3.6-4.0 TB/s); warm-cache times barely moved.
//
// Work split: a (token position, 16-byte chunk) pair per lane, blockIdx.y
// selecting a group of PR_HEADS heads ("slabs") from the concatenation of the
// B*Hq query slabs and the B*Hkv key slabs, each slab being one [N, D] matrix.
// PR_HEADS is 2 (1 for a single slab); with no query slabs the same kernel
// rotates K alone.
#include "rac_device.h"
#include "rac_internal.h"

namespace rac {

constexpr int PR_THREADS = 256;

// The inverse turn R(-p) = R(p)^T of rope_rotate8 on 8 elements (4 pairs),
// same table entries: x0 = y0*c + y1*s, x1 = y1*c - y0*s, in fp32 with one
// fused multiply-add each, then one rounding to the storage format.
template <int DT>
__device__ __forceinline__ u32x4 rope_unrotate8(u32x4 y, f32x4 cs_lo, f32x4 cs_hi) {
    typedef Fmt<DT> F;
    u32x4 x;
    const float c[4] = {cs_lo[0], cs_lo[2], cs_hi[0], cs_hi[2]};
    const float s[4] = {cs_lo[1], cs_lo[3], cs_hi[1], cs_hi[3]};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float y0 = F::lo(y[t]), y1 = F::hi(y[t]);
        x[t] = F::pack2(__builtin_fmaf(y0, c[t], y1 * s[t]), __builtin_fmaf(y1, c[t], -(y0 * s[t])));
    }
    return x;
}

// PR_HEADS slabs per lane: that many independent 16-byte loads in flight.
// INV: turn by -p instead of +p (the gradient of the pass).
// q_rot and k_rot may be q and k themselves (exact in-place use): those
// pointers carry no __restrict__, and each lane stores only the chunks it has
// already loaded.
template <int DT, int D, int PR_HEADS, bool INV>
__global__ __launch_bounds__(PR_THREADS) void rope_prerotate_kernel(
    const uint16_t* q, const uint16_t* k, uint16_t* q_rot, uint16_t* k_rot,
    const float* __restrict__ table, int N, int64_t q_slabs, int64_t total_slabs) {
    constexpr int CHUNKS = D / 8;  // 16-byte chunks per row
    const int64_t idx = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
    const int64_t row = idx / CHUNKS;
    const int chunk = (int)(idx % CHUNKS);
    if (row >= N) return;
    const f32x4* tab = reinterpret_cast<const f32x4*>(table + row * D + chunk * 8);
    const f32x4 cs_lo = tab[0];
    const f32x4 cs_hi = tab[1];
    const int64_t slab0 = (int64_t)blockIdx.y * PR_HEADS;
    const int64_t within = row * D + chunk * 8;  // element offset inside a slab
    const int64_t slab_elems = (int64_t)N * D;

    u32x4 x[PR_HEADS];
#pragma unroll
    for (int s = 0; s < PR_HEADS; ++s) {
        const int64_t slab = slab0 + s;
        if (slab < total_slabs) {
            const uint16_t* src = slab < q_slabs ? q + slab * slab_elems
                                                 : k + (slab - q_slabs) * slab_elems;
            x[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + within));
        }
    }
#pragma unroll
    for (int s = 0; s < PR_HEADS; ++s) {
        const int64_t slab = slab0 + s;
        if (slab < total_slabs) {
            uint16_t* dst = slab < q_slabs ? q_rot + slab * slab_elems
                                           : k_rot + (slab - q_slabs) * slab_elems;
            __builtin_nontemporal_store(INV ? rope_unrotate8<DT>(x[s], cs_lo, cs_hi)
                                            : rope_rotate8<DT>(x[s], cs_lo, cs_hi),
                                        reinterpret_cast<u32x4*>(dst + within));
        }
    }
}

// The inverse turn of rope_rotate_half8: each pair (a', b') = (lo[j], hi[j])
// goes back by R(-p), a = a' c + b' s and b = b' c - a' s, in fp32 with one
// fused multiply-add each, then one rounding to the storage format.
template <int DT>
__device__ __forceinline__ void rope_unrotate_half8(u32x4 lo, u32x4 hi, const f32x4 (&cs)[4],
                                                    u32x4& lo_out, u32x4& hi_out) {
    typedef Fmt<DT> F;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float x[2], y[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int j = 2 * t + e;  // frequency d0 + j
            const float c = cs[j >> 1][2 * (j & 1)], sn = cs[j >> 1][2 * (j & 1) + 1];
            const float a = e ? F::hi(lo[t]) : F::lo(lo[t]);
            const float b = e ? F::hi(hi[t]) : F::lo(hi[t]);
            x[e] = __builtin_fmaf(a, c, b * sn);
            y[e] = __builtin_fmaf(b, c, -(a * sn));
        }
        lo_out[t] = F::pack2(x[0], x[1]);
        hi_out[t] = F::pack2(y[0], y[1]);
    }
}

// The half-split pairing: a lane owns chunk c < D/16 of a row and its
// partner chunk c + D/16 (elements d and d + D/2 pair), with the 16 table
// floats of frequencies 8c .. 8c+7, for PR_HEADS slabs. INV: turn by -p
// (the gradient of the pass).
// (in-place use as for rope_prerotate_kernel)
template <int DT, int D, int PR_HEADS, bool INV>
__global__ __launch_bounds__(PR_THREADS) void rope_prerotate_half_kernel(
    const uint16_t* q, const uint16_t* k, uint16_t* q_rot, uint16_t* k_rot,
    const float* __restrict__ table, int N, int64_t q_slabs, int64_t total_slabs) {
    constexpr int HALF_CHUNKS = D / 16;  // chunk pairs per row
    const int64_t idx = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
    const int64_t row = idx / HALF_CHUNKS;
    const int chunk = (int)(idx % HALF_CHUNKS);
    if (row >= N) return;
    const f32x4* tab = reinterpret_cast<const f32x4*>(table + row * D + chunk * 16);
    const f32x4 cs[4] = {tab[0], tab[1], tab[2], tab[3]};
    const int64_t slab0 = (int64_t)blockIdx.y * PR_HEADS;
    const int64_t lo_off = row * D + chunk * 8;  // element offsets inside a slab
    const int64_t hi_off = lo_off + D / 2;
    const int64_t slab_elems = (int64_t)N * D;

    u32x4 lo[PR_HEADS], hi[PR_HEADS];
#pragma unroll
    for (int s = 0; s < PR_HEADS; ++s) {
        const int64_t slab = slab0 + s;
        if (slab < total_slabs) {
            const uint16_t* src = slab < q_slabs ? q + slab * slab_elems
                                                 : k + (slab - q_slabs) * slab_elems;
            lo[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + lo_off));
            hi[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + hi_off));
        }
    }
#pragma unroll
    for (int s = 0; s < PR_HEADS; ++s) {
        const int64_t slab = slab0 + s;
        if (slab < total_slabs) {
            uint16_t* dst = slab < q_slabs ? q_rot + slab * slab_elems
                                           : k_rot + (slab - q_slabs) * slab_elems;
            u32x4 a, b;
            if (INV)
                rope_unrotate_half8<DT>(lo[s], hi[s], cs, a, b);
            else
                rope_rotate_half8<DT>(lo[s], hi[s], cs, a, b);
            __builtin_nontemporal_store(a, reinterpret_cast<u32x4*>(dst + lo_off));
            __builtin_nontemporal_store(b, reinterpret_cast<u32x4*>(dst + hi_off));
        }
    }
}

template <int DT, int D, int H, bool INV>
static hipError_t launch_heads(const void* q, const void* k, void* q_rot, void* k_rot,
                               const float* table, int N, int64_t q_slabs, int64_t total,
                               unsigned gx, hipStream_t stream) {
    dim3 grid(gx, (unsigned)((total + H - 1) / H));
    return launch_kernel(rope_prerotate_kernel<DT, D, H, INV>, grid, dim3(PR_THREADS), stream,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<uint16_t*>(q_rot), static_cast<uint16_t*>(k_rot), table, N,
                         q_slabs, total);
}

// Slabs per lane. Measured kernel times on the Llama-3-8B and D = 64 shapes
// (8 to 320 MiB per call): two slabs per lane was the fastest or within 10 %
// of it everywhere, while eight (the most table reuse per lane) was up to
// 15 % slower at the large sizes and 60 % slower with few slabs: the grid's
// parallelism matters more than the table loads, which stay in cache. From
// 40 to 64 MiB per call four slabs per lane were 2-9 % faster cold and up to
// 15 % warm (twice the loads in flight per lane; the grid, still at least
// 1280 workgroups, fits on the chip at once), at 32 MiB with 1024 workgroups
// 2 % slower, from 128 MiB up 0-2 % slower; a grid-stride loop over (slab,
// row, chunk) items was 5-20 % slower than either. `bytes` = the call's
// reads and writes (0: not counted, two slabs).
// More slabs per lane only where the grid's y extent (<= 65535) needs it;
// the entry points cap the slab count at 8 * 65535.
inline int prerotate_heads(int64_t total, int64_t bytes = 0, int64_t gx = 0) {
    if (total < 2) return 1;
    int h = 2;
    if (bytes > 0 && bytes <= (int64_t(64) << 20) && gx * ((total + 3) / 4) >= 1280) h = 4;
    while (h < 8 && (total + h - 1) / h > 65535) h *= 2;
    return h;
}

template <int DT, int D, bool INV>
static hipError_t launch_typed(const void* q, const void* k, void* q_rot, void* k_rot,
                               const float* table, int B, int Hq, int Hkv, int N,
                               hipStream_t stream) {
    const int64_t lanes = (int64_t)N * (D / 8);
    const int64_t q_slabs = (int64_t)B * Hq;
    const int64_t total = q_slabs + (int64_t)B * Hkv;
    const unsigned gx = (unsigned)((lanes + PR_THREADS - 1) / PR_THREADS);
    const int64_t bytes = total * N * D * 4;  // 2-byte elements, read and written
    switch (prerotate_heads(total, bytes, gx)) {
        case 8: return launch_heads<DT, D, 8, INV>(q, k, q_rot, k_rot, table, N, q_slabs, total, gx, stream);
        case 4: return launch_heads<DT, D, 4, INV>(q, k, q_rot, k_rot, table, N, q_slabs, total, gx, stream);
        case 2: return launch_heads<DT, D, 2, INV>(q, k, q_rot, k_rot, table, N, q_slabs, total, gx, stream);
        default: return launch_heads<DT, D, 1, INV>(q, k, q_rot, k_rot, table, N, q_slabs, total, gx, stream);
    }
}

template <bool INV>
static hipError_t launch_any(const void* q, const void* k, void* q_rot, void* k_rot,
                             const float* table, int B, int Hq, int Hkv, int N, int D, int dtype,
                             hipStream_t stream) {
    if (dtype == DT_BF16)
        return D == 64 ? launch_typed<DT_BF16, 64, INV>(q, k, q_rot, k_rot, table, B, Hq, Hkv, N, stream)
                       : launch_typed<DT_BF16, 128, INV>(q, k, q_rot, k_rot, table, B, Hq, Hkv, N, stream);
    return D == 64 ? launch_typed<DT_FP16, 64, INV>(q, k, q_rot, k_rot, table, B, Hq, Hkv, N, stream)
                   : launch_typed<DT_FP16, 128, INV>(q, k, q_rot, k_rot, table, B, Hq, Hkv, N, stream);
}

// A plain device copy with the pass's access pattern: 16-byte non-temporal
// loads and stores, 256-lane workgroups, COPY_CHUNKS chunks per lane in
// flight (a workgroup moves COPY_CHUNKS * 4 KiB; chunk j of lane t sits at
// (j * 256 + t) * 16 bytes into the workgroup's span, so each load and store
// instruction of a wave covers 1 KiB of consecutive bytes). It computes
// nothing: it is the bandwidth ceiling the pass is measured against.
constexpr int COPY_CHUNKS = 4;

__global__ __launch_bounds__(PR_THREADS) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                                 u32x4* __restrict__ dst,
                                                                 int64_t chunks) {
    const int64_t first = (int64_t)blockIdx.x * (COPY_CHUNKS * PR_THREADS) + threadIdx.x;
    u32x4 x[COPY_CHUNKS];
#pragma unroll
    for (int j = 0; j < COPY_CHUNKS; ++j) {
        const int64_t c = first + (int64_t)j * PR_THREADS;
        if (c < chunks) x[j] = __builtin_nontemporal_load(src + c);
    }
#pragma unroll
    for (int j = 0; j < COPY_CHUNKS; ++j) {
        const int64_t c = first + (int64_t)j * PR_THREADS;
        if (c < chunks) __builtin_nontemporal_store(x[j], dst + c);
    }
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    const int64_t chunks = bytes / 16;
    const int64_t per_block = (int64_t)COPY_CHUNKS * PR_THREADS;
    const unsigned grid = (unsigned)((chunks + per_block - 1) / per_block);
    return launch_kernel(stream_copy_kernel, dim3(grid), dim3(PR_THREADS), stream,
                         static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), chunks);
}

hipError_t launch_rope_prerotate(const void* q, const void* k, void* q_rot, void* k_rot,
                                 const float* table, int B, int Hq, int Hkv, int N, int D,
                                 int dtype, hipStream_t stream) {
    return launch_any<false>(q, k, q_rot, k_rot, table, B, Hq, Hkv, N, D, dtype, stream);
}

hipError_t launch_rope_unrotate(const void* dq_rot, const void* dk_rot, void* dq, void* dk,
                                const float* table, int B, int Hq, int Hkv, int N, int D,
                                int dtype, hipStream_t stream) {
    return launch_any<true>(dq_rot, dk_rot, dq, dk, table, B, Hq, Hkv, N, D, dtype, stream);
}

template <int DT, int D, int H, bool INV>
static hipError_t launch_half_heads(const void* q, const void* k, void* q_rot, void* k_rot,
                                    const float* table, int N, int64_t q_slabs, int64_t total,
                                    unsigned gx, hipStream_t stream) {
    dim3 grid(gx, (unsigned)((total + H - 1) / H));
    return launch_kernel(rope_prerotate_half_kernel<DT, D, H, INV>, grid, dim3(PR_THREADS), stream,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<uint16_t*>(q_rot), static_cast<uint16_t*>(k_rot), table, N,
                         q_slabs, total);
}

// Same grid policy as the adjacent pairing, with one lane per chunk pair.
template <int DT, int D, bool INV>
static hipError_t launch_half(const void* q, const void* k, void* q_rot, void* k_rot,
                              const float* table, int B, int Hq, int Hkv, int N,
                              hipStream_t stream) {
    const int64_t lanes = (int64_t)N * (D / 16);
    const int64_t q_slabs = (int64_t)B * Hq;
    const int64_t total = q_slabs + (int64_t)B * Hkv;
    const unsigned gx = (unsigned)((lanes + PR_THREADS - 1) / PR_THREADS);
    switch (prerotate_heads(total)) {
        case 8: return launch_half_heads<DT, D, 8, INV>(q, k, q_rot, k_rot, table, N, q_slabs, total, gx, stream);
        case 4: return launch_half_heads<DT, D, 4, INV>(q, k, q_rot, k_rot, table, N, q_slabs, total, gx, stream);
        case 2: return launch_half_heads<DT, D, 2, INV>(q, k, q_rot, k_rot, table, N, q_slabs, total, gx, stream);
        default: return launch_half_heads<DT, D, 1, INV>(q, k, q_rot, k_rot, table, N, q_slabs, total, gx, stream);
    }
}

template <bool INV>
static hipError_t launch_half_any(const void* q, const void* k, void* q_rot, void* k_rot,
                                  const float* table, int B, int Hq, int Hkv, int N, int D,
                                  int dtype, hipStream_t stream) {
    if (dtype == DT_BF16)
        return D == 64 ? launch_half<DT_BF16, 64, INV>(q, k, q_rot, k_rot, table, B, Hq, Hkv, N, stream)
                       : launch_half<DT_BF16, 128, INV>(q, k, q_rot, k_rot, table, B, Hq, Hkv, N, stream);
    return D == 64 ? launch_half<DT_FP16, 64, INV>(q, k, q_rot, k_rot, table, B, Hq, Hkv, N, stream)
                   : launch_half<DT_FP16, 128, INV>(q, k, q_rot, k_rot, table, B, Hq, Hkv, N, stream);
}

hipError_t launch_rope_prerotate_half(const void* q, const void* k, void* q_rot, void* k_rot,
                                      const float* table, int B, int Hq, int Hkv, int N, int D,
                                      int dtype, hipStream_t stream) {
    return launch_half_any<false>(q, k, q_rot, k_rot, table, B, Hq, Hkv, N, D, dtype, stream);
}

hipError_t launch_rope_unrotate_half(const void* dq_rot, const void* dk_rot, void* dq, void* dk,
                                     const float* table, int B, int Hq, int Hkv, int N, int D,
                                     int dtype, hipStream_t stream) {
    return launch_half_any<true>(dq_rot, dk_rot, dq, dk, table, B, Hq, Hkv, N, D, dtype, stream);
}

}  // namespace rac
