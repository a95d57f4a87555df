// attn_fwd.hip -- causal MHA/GQA attention forward for gfx950, with RoPE fused
// into the tile loads (ROPE = true) or not (ROPE = false).
//
// Method: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (rainbus digest), background "FlashAttention and online softmax"
// and the forward Algorithm 1: one workgroup per query tile walks the key
// tiles, keeps the running row maximum m and denominator l on chip, and writes
// o = u / l and the log-sum-exp L. The digest's precision design is kept:
// fp32 statistics and accumulators, base-2 exponent. The fused variant is the
// single kernel of "AttnFuse Makes RoPE a First-Class Attention Compilation
// Operation", paragraph 3 ("in-kernel rotation"): the query tile is rotated
// once when loaded, and every key tile is rotated each time a workgroup loads
// it -- the compute-and-tiling cost that paragraph contrasts with pre-rotation.
//
// gfx950 mapping (64-lane waves, v_mfma_f32_32x32x16 bf16/fp16):
//   * workgroup = 4 waves = BM = 128 query rows of one (b, query head);
//     wave w owns rows q0 + 32w .. +31, lane (n, hh) = (lane % 32, lane / 32).
//   * Scores are computed transposed, S^T = K Q^T: A = K tile from LDS
//     (row = key), B = the wave's Q rows kept in registers for the whole loop.
//     The fp32 result puts one query per lane column, so row statistics need
//     only in-lane reductions plus one exchange between the two lane halves.
//   * O^T = V^T P^T: the P^T accumulator registers are reused directly as the
//     B operand (the key order inside each 16-key step is permuted, and V^T is
//     stored in LDS in that same permuted order), A = V^T from LDS.
//   * Key tiles of BN = 64 rows; tiles past the wave's last query are skipped
//     and only tiles straddling the diagonal are masked.
//   * Workgroups with the most key tiles (the last query tiles) launch first.
#include <math.h>

#include "rac_device.h"
#include "rac_internal.h"

namespace rac {

constexpr int BM = 128;
constexpr int BN = 64;
constexpr int NWAVES = 4;
constexpr int THREADS = NWAVES * 64;
constexpr int VT_PAD = 8;  // elements of padding per V^T row

// Slot of key r (0..BN-1) inside the V^T row: bits 2 and 3 of the key index
// are swapped. With that order the 8 keys a lane half feeds to one PV MFMA step
// sit contiguously, matching where the score MFMA left their probabilities.
__device__ __forceinline__ int vt_slot(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <int DT, int D, bool ROPE>
__global__ __launch_bounds__(THREADS) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, float* __restrict__ lse,
    const float* __restrict__ table, int Hq, int Hkv, int N, float scale_log2) {
    typedef Fmt<DT> F;
    typedef typename F::vec8 vec8;
    constexpr int KS_STRIDE = D + 8;    // elements per K row in LDS (padding vs bank conflicts)
    constexpr int VT_STRIDE = BN + VT_PAD;
    constexpr int QCH = D / 16;         // 16-deep MFMA steps over the head dim
    constexpr int DBLK = D / 32;        // 32-row blocks of O^T
    constexpr int CHUNKS = D / 8;       // 16-byte chunks per row
    constexpr int LOAD_ITERS = BN * CHUNKS / THREADS;

    __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VT_STRIDE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 31;
    const int hh = lane >> 5;

    const int qtile = gridDim.x - 1 - blockIdx.x;  // heaviest tiles first
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int g = h / (Hq / Hkv);
    const int q0 = qtile * BM;
    const int qw0 = q0 + wave * 32;       // first query row of this wave
    const int my_q = qw0 + n;

    const int64_t q_head = ((int64_t)b * Hq + h) * N;
    const int64_t kv_head = ((int64_t)b * Hkv + g) * N;

    // ---- this wave's Q rows as MFMA B operands (rotated once if ROPE) ----
    vec8 qf[QCH];
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (my_q < N) {
            const int d0 = 16 * c + 8 * hh;
            w = *reinterpret_cast<const u32x4*>(q + (q_head + my_q) * D + d0);
            if (ROPE) {
                const f32x4* t = reinterpret_cast<const f32x4*>(table + (int64_t)my_q * D + d0);
                w = rope_rotate8<DT>(w, t[0], t[1]);
            }
        }
        qf[c] = as_vec8<DT>(w);
    }

    f32x16 acc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
    float m_run = -INFINITY;  // running max of the base-2 scaled scores
    float l_run = 0.f;        // this lane half's share of the denominator

    const int last_row = min(q0 + BM, N) - 1;
    const int n_tiles = last_row / BN + 1;
    const int wave_last = min(qw0 + 31, N - 1);
    const int wave_tiles = qw0 < N ? wave_last / BN + 1 : 0;

    for (int t = 0; t < n_tiles; ++t) {
        const int k0 = t * BN;
        __syncthreads();  // previous tile fully consumed
        // ---- K tile -> LDS (rotated if ROPE), V tile -> LDS transposed ----
#pragma unroll
        for (int it = 0; it < LOAD_ITERS; ++it) {
            const int idx = tid + it * THREADS;
            const int r = idx / CHUNKS;
            const int cc = idx % CHUNKS;
            const int key = k0 + r;
            u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
            if (key < N) {
                kw = *reinterpret_cast<const u32x4*>(k + (kv_head + key) * D + cc * 8);
                vw = *reinterpret_cast<const u32x4*>(v + (kv_head + key) * D + cc * 8);
                if (ROPE) {
                    const f32x4* tb =
                        reinterpret_cast<const f32x4*>(table + (int64_t)key * D + cc * 8);
                    kw = rope_rotate8<DT>(kw, tb[0], tb[1]);
                }
            }
            *reinterpret_cast<u32x4*>(&Ks[r * KS_STRIDE + cc * 8]) = kw;
            const int slot = vt_slot(r);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Vt[(cc * 8 + 2 * e) * VT_STRIDE + slot] = (uint16_t)(vw[e] & 0xffffu);
                Vt[(cc * 8 + 2 * e + 1) * VT_STRIDE + slot] = (uint16_t)(vw[e] >> 16);
            }
        }
        __syncthreads();
        if (t >= wave_tiles) continue;  // wave-uniform: every key here is above the diagonal

        // ---- S^T = K Q^T for two 32-key blocks ----
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
#pragma unroll
            for (int c = 0; c < QCH; ++c) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(
                    &Ks[(32 * kb + n) * KS_STRIDE + 16 * c + 8 * hh]);
                s[kb] = F::mfma(as_vec8<DT>(a), qf[c], s[kb]);
            }
        }

        // ---- online softmax (base 2); lane holds query my_q, 32 keys ----
        const bool diag = k0 + BN - 1 > qw0;  // wave-uniform
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float x = s[kb][j] * scale_log2;
                if (diag) {
                    const int key = k0 + 32 * kb + 8 * (j >> 2) + 4 * hh + (j & 3);
                    if (key > my_q) x = -INFINITY;
                }
                s[kb][j] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        float psum = 0.f;
        u32x4 pw[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int t2 = 0; t2 < 4; ++t2) {
                    const float p0 = exp2f(s[kb][8 * e + 2 * t2] - m_new);
                    const float p1 = exp2f(s[kb][8 * e + 2 * t2 + 1] - m_new);
                    psum += p0 + p1;
                    pw[kb][e][t2] = F::pack2(p0, p1);
                }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int i = 0; i < DBLK; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[i][j] *= alpha;

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int i = 0; i < DBLK; ++i)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(
                        &Vt[(32 * i + n) * VT_STRIDE + 32 * kb + 16 * e + 8 * hh]);
                    acc[i] = F::mfma(as_vec8<DT>(a), as_vec8<DT>(pw[kb][e]), acc[i]);
                }
    }

    // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l) ----
    if (wave_tiles == 0 || my_q >= N) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    uint16_t* orow = out + (q_head + my_q) * D;
#pragma unroll
    for (int i = 0; i < DBLK; ++i)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            const int d0 = 32 * i + 8 * grp + 4 * hh;
            u32x2 w;
            w[0] = F::pack2(acc[i][4 * grp] * inv, acc[i][4 * grp + 1] * inv);
            w[1] = F::pack2(acc[i][4 * grp + 2] * inv, acc[i][4 * grp + 3] * inv);
            *reinterpret_cast<u32x2*>(orow + d0) = w;
        }
    if (lse != nullptr && hh == 0)
        lse[q_head + my_q] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
}

template <int DT, int D, bool ROPE>
static hipError_t launch_typed(const AttnArgs& a, hipStream_t stream) {
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    dim3 grid((unsigned)((a.N + BM - 1) / BM), (unsigned)a.Hq, (unsigned)a.B);
    attn_fwd_kernel<DT, D, ROPE><<<grid, THREADS, 0, stream>>>(
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
        static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.out), a.lse, a.table,
        a.Hq, a.Hkv, a.N, scale_log2);
    return hipGetLastError();
}

template <int DT, bool ROPE>
static hipError_t launch_dt(const AttnArgs& a, hipStream_t stream) {
    return a.D == 64 ? launch_typed<DT, 64, ROPE>(a, stream) : launch_typed<DT, 128, ROPE>(a, stream);
}

hipError_t launch_attn_fwd(const AttnArgs& a, bool rope, hipStream_t stream) {
    if (a.dtype == DT_BF16)
        return rope ? launch_dt<DT_BF16, true>(a, stream) : launch_dt<DT_BF16, false>(a, stream);
    return rope ? launch_dt<DT_FP16, true>(a, stream) : launch_dt<DT_FP16, false>(a, stream);
}

}  // namespace rac
