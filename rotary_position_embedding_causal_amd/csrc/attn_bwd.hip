// attn_bwd.hip -- causal MHA/GQA attention backward for gfx950, with RoPE
// fused into the operand loads (RM = ROT_QK) or not (RM = ROT_NONE).
//
// Method: the chain rule through the forward's definition ("Fast and Exact
// Relative-Position Attention via Structure-Aware Kernels", rainbus digest,
// background "FlashAttention and online softmax"): with P_ij = exp(s_ij - L_i)
// rebuilt from the forward's log-sum-exp L,
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - Delta),   Delta_i = dO_i . O_i,
//     dQ = tau dS K,   dK = tau dS^T Q,
// dK and dV of a key/value head summed over the query heads that read it.
// The schedule is the digest's method section, backward (Algorithm 2): a
// query-parallel pass rebuilds S, P, dS and accumulates dQ; a key-parallel
// pass rebuilds them again and accumulates dK, dV. Every gradient element has
// one writer -- no atomics, deterministic results.
//
// RoPE: the forward rotates q and k by their positions (the turn R(p)); its
// gradient is the inverse turn R(-p) = R(p)^T. Fused, both passes rotate the
// Q and K operands in the kernel exactly as the forward does (the same
// rope_rotate8, so the same bf16/fp16 operands) and apply R(-p) to dQ and dK
// in fp32 before the one rounding to the storage format. "AttnFuse Makes RoPE
// a First-Class Attention Compilation Operation", paragraph 3, reports a
// Llama-3-8B training step with RoPE fused; this is that step's attention
// backward.
//
// gfx950 mapping (64-lane waves, v_mfma_f32_32x32x16 bf16/fp16), the same two
// MFMA patterns as the forward:
//   * "score" pattern, C[32 x 32] = A B: A = 32 rows of an LDS tile (16-byte
//     chunk reads), B = the wave's 32 stationary rows held in registers
//     (lane (n, hh) holds row n, chunks 16c + 8hh). The fp32 result has one
//     stationary row per lane column.
//   * "PV" pattern, C^T[D x 32] += X^T Y: A = X^T from an LDS tile through the
//     transpose read (ds_read_b64_tr_b16), B = score-pattern results packed to
//     the storage format, rows permuted inside each 16-row step the same way
//     on both sides.
//   dQ pass: stationary = 32 query rows (Q, dO); streamed = 64-key tiles of K
//     and V. S^T = K Q^T and dP^T = V dO^T (score), dQ^T += K^T dS^T (PV).
//   dK/dV pass: stationary = 32 key rows (K, V); streamed = 64-query tiles of
//     Q and dO (with their L and Delta) of every query head of the group.
//     S = Q K^T and dP = dO V^T (score), dV^T += dO^T P and dK^T += Q^T dS (PV).
//   Tiles are double-buffered in LDS and move straight from global memory
//   into LDS (buffer_load_dwordx4 ... lds); with RoPE the rotated tile (K in
//   the dQ pass, Q in the dK/dV pass) is turned in place by the threads that
//   loaded it before the workgroup's barrier.
#include <math.h>

#include <type_traits>

#include "rac_device.h"
#include "rac_internal.h"

namespace rac {
namespace bwd {

constexpr int BR = 128;  // stationary query rows per dQ-pass workgroup (4 waves x 32)
constexpr int BT = 64;   // rows of a streamed tile
constexpr int NUM_CUS = 256;
constexpr int NXCD = 8;
constexpr float LOG2E = 1.4426950408889634f;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Transposed LDS read: in each 16-lane group, lane i receives element i%4 of
// the 8-byte chunks addressed by lanes 4e + i/4, e = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Position of logical 16-byte chunk c of tile row `row`: c ^ swz(row). Every
// streamed tile is read in both patterns, so the swizzle serves both:
//   * score pattern: 16 lanes read one chunk column of 16 consecutive rows,
//     so swz must take distinct values over any 16 consecutive rows (with
//     D = 64 two rows share a 256-byte bank period: over the 8 rows of each
//     parity);
//   * transpose (PV) pattern: a 16-lane group reads chunks 4i + {lc, lc + 1}
//     of 4 consecutive rows 4k .. 4k+3, so the 4 rows must land on disjoint
//     chunk positions (D = 128: swz's bits 2-3 take the row's low two bits;
//     D = 64: rows 4k and 4k + 2, of one parity, differ in swz's bit 1).
// (A swizzle for the score pattern alone, row & 15, left the transpose
// reads two-way bank-conflicted.)
template <int D>
__device__ __forceinline__ int swz(int row) {
    return D == 128 ? 4 * (row & 3) + ((row >> 2) & 3)
                    : 2 * ((row >> 1) & 1) + 4 * ((row >> 2) & 1) + ((row >> 3) & 1);
}

constexpr int BUF_RSRC_FLAGS = 0x00020000;  // raw (unformatted) 32-bit data

// Buffer descriptor of rows t*BT .. N-1 of a [N][row_elems] tensor; rows past
// N read as zeros (a tile at or past the end: a record count of zero).
template <typename E>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const E* base, int row_elems, int t,
                                                            int N) {
    const int64_t r0 = (int64_t)t * BT;
    const int64_t bytes = (N > r0 ? N - r0 : 0) * row_elems * (int64_t)sizeof(E);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + r0 * row_elems), 0,
                                             (int)min(bytes, (int64_t)0x7fffffff),
                                             BUF_RSRC_FLAGS);
}

// Loads of two streamed [BT][D] tiles (A, rotated in place when ROPE, and B)
// by the workgroup's NW waves, global -> LDS; block b of a tile holds chunks
// 64b .. 64b+63. Optionally also 64 per-row floats x 2 (the tile rows' scaled
// L and Delta) through registers into LDS.
template <int DT, int D, bool ROPE, int NW>
struct Streamer {
    static constexpr int CH = D / 8;
    static constexpr int INSTR = BT * CH / (64 * NW);
    f32x4 cs[ROPE ? INSTR : 1][2];
    f32x4 rowv;  // this lane's 4 row floats (L or Delta), lanes 0..31 of wave 0

    __device__ __forceinline__ void issue(uint16_t* abuf, uint16_t* bbuf,
                                          __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          __amdgpu_buffer_rsrc_t rt, int wave, int lane) {
#pragma unroll
        for (int j = 0; j < INSTR; ++j) {
            const int blk = wave * INSTR + j;
            const int g = blk * 64 + lane;
            const int row = g / CH;
            const int el = row * D + 8 * ((g % CH) ^ swz<D>(row));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(abuf + blk * 512), 16, el * 2,
                                                     0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(bbuf + blk * 512), 16, el * 2,
                                                     0, 0, 0);
            if (ROPE) {
                cs[j][0] = __builtin_bit_cast(f32x4,
                                              __builtin_amdgcn_raw_buffer_load_b128(rt, el * 4, 0, 0));
                cs[j][1] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rt, el * 4 + 16, 0, 0));
            }
        }
    }

    // Row floats of the tile: lanes 0..15 of wave 0 load 4 of L's, lanes
    // 16..31 4 of Delta's (rows past N read as zeros).
    __device__ __forceinline__ void issue_rows(__amdgpu_buffer_rsrc_t rl,
                                               __amdgpu_buffer_rsrc_t rd, int wave, int lane) {
        if (wave != 0) return;
        if (lane < 16)
            rowv = __builtin_bit_cast(f32x4,
                                      __builtin_amdgcn_raw_buffer_load_b128(rl, lane * 16, 0, 0));
        else if (lane < 32)
            rowv = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rd, (lane - 16) * 16, 0, 0));
    }

    // After this thread's loads landed, before the barrier: rotate its chunks
    // of tile A (ROPE) and store its row floats (L scaled to base 2).
    __device__ __forceinline__ void finish(uint16_t* abuf, float* rows, bool with_rows, int wave,
                                           int lane) {
        if (ROPE) {
#pragma unroll
            for (int j = 0; j < INSTR; ++j) {
                u32x4* p = reinterpret_cast<u32x4*>(abuf + (wave * INSTR + j) * 512 + lane * 8);
                *p = rope_rotate8<DT>(*p, cs[j][0], cs[j][1]);
            }
        }
        if (with_rows && wave == 0 && lane < 32) {
            f32x4 x = rowv;
            if (lane < 16) x = x * LOG2E;
            *reinterpret_cast<f32x4*>(rows + lane * 4) = x;
        }
    }
};

__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0); }

// Per-wave pieces shared by both passes.
template <int DT, int D>
struct Wave {
    typedef Fmt<DT> F;
    typedef typename F::vec8 vec8;
    static constexpr int QCH = D / 16;   // 16-deep MFMA steps over the head dim
    static constexpr int DBLK = D / 32;  // 32-row blocks of a C^T accumulator

    // 32 rows (r0 + n) of a [N][D] tensor as score-pattern B operands,
    // rotated by their positions when `table` is given.
    __device__ __forceinline__ static void load_rows(vec8 (&f)[QCH], const uint16_t* base,
                                                     const float* table, int r0, int N, int n,
                                                     int hh) {
        const int row = r0 + n;
#pragma unroll
        for (int c = 0; c < QCH; ++c) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (row < N) {
                const int d0 = 16 * c + 8 * hh;
                w = *reinterpret_cast<const u32x4*>(base + (int64_t)row * D + d0);
                if (table) {
                    const f32x4* t = reinterpret_cast<const f32x4*>(table + (int64_t)row * D + d0);
                    w = rope_rotate8<DT>(w, t[0], t[1]);
                }
            }
            f[c] = as_vec8<DT>(w);
        }
    }

    // Score pattern: C = X[r0 .. r0+31] (LDS tile rows) times the stationary
    // rows f, over the head dimension.
    __device__ __forceinline__ static f32x16 score(const uint16_t* X, int r0, const vec8 (&f)[QCH],
                                                   int n, int hh) {
        f32x16 acc = {};
        const int row = r0 + n;
        const int sw = swz<D>(row);
#pragma unroll
        for (int c = 0; c < QCH; ++c) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(X + row * D + 8 * ((2 * c + hh) ^ sw));
            acc = F::mfma(as_vec8<DT>(a), f[c], acc);
        }
        return acc;
    }

    // PV pattern: acc^T (DBLK blocks of 32 d-rows x 32 lanes) += X^T Y for the
    // 32 tile rows r0 .. r0+31 of LDS tile X, with Y given as the packed
    // score-pattern values y[e] (e = 16-row step). The transpose-read lane
    // geometry takes rows r0 + 16e + lrow (and + 8), chunk 4i + lc, elements
    // le .. le+3, in the same permuted order as the packed registers.
    __device__ __forceinline__ static void pv(f32x16 (&acc)[DBLK], const uint16_t* X, int r0,
                                              const u32x4 (&y)[2], int lane) {
        const int g4 = lane >> 4, j16 = lane & 15;
        const int lrow = 4 * (g4 >> 1) + (j16 >> 2);
        const int lc = 2 * (g4 & 1) + ((j16 & 3) >> 1);
        const int le = 4 * (j16 & 1);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int rlo = r0 + 16 * e + lrow, rhi = rlo + 8;
            const int slo = swz<D>(rlo), shi = swz<D>(rhi);
            const vec8 b = as_vec8<DT>(y[e]);
#pragma unroll
            for (int i = 0; i < DBLK; ++i) {
                const u32x2 lo = __builtin_bit_cast(
                    u32x2, lds_read_tr16(X + rlo * D + 8 * ((4 * i + lc) ^ slo) + le));
                const u32x2 hi = __builtin_bit_cast(
                    u32x2, lds_read_tr16(X + rhi * D + 8 * ((4 * i + lc) ^ shi) + le));
                const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                acc[i] = F::mfma(as_vec8<DT>(a), b, acc[i]);
            }
        }
    }

    // Packs a score-pattern result into the two 16-row PV operands.
    __device__ __forceinline__ static void pack(const f32x16& x, u32x4 (&y)[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2) y[e][t2] = F::pack2(x[8 * e + 2 * t2], x[8 * e + 2 * t2 + 1]);
    }

    // Writes C^T (scaled by `scale`) as row `row` of a [N][D] tensor: this
    // lane's elements d = 32i + 8gq + 4hh + (0..3). With `table`, the pairs
    // are first turned back by the row's position, R(-p):
    //   x0 = y0 c + y1 s,  x1 = y1 c - y0 s.
    // The table entries are all loaded before the first store: the output and
    // the table never overlap, but the compiler cannot know it and would wait
    // for each load after the previous store.
    __device__ __forceinline__ static void write(const f32x16 (&acc)[DBLK], float scale,
                                                 uint16_t* orow, const float* trow, int hh) {
        f32x4 tab[DBLK][4];
        if (trow) {
#pragma unroll
            for (int i = 0; i < DBLK; ++i)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    tab[i][gq] = *reinterpret_cast<const f32x4*>(trow + 32 * i + 8 * gq + 4 * hh);
        }
#pragma unroll
        for (int i = 0; i < DBLK; ++i)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d0 = 32 * i + 8 * gq + 4 * hh;
                float y[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) y[t] = acc[i][4 * gq + t] * scale;
                if (trow) {
                    const f32x4 cs = tab[i][gq];
#pragma unroll
                    for (int pr = 0; pr < 2; ++pr) {
                        const float c = cs[2 * pr], s = cs[2 * pr + 1];
                        const float y0 = y[2 * pr], y1 = y[2 * pr + 1];
                        y[2 * pr] = __builtin_fmaf(y0, c, y1 * s);
                        y[2 * pr + 1] = __builtin_fmaf(y1, c, -(y0 * s));
                    }
                }
                u32x2 w;
                w[0] = F::pack2(y[0], y[1]);
                w[1] = F::pack2(y[2], y[3]);
                *reinterpret_cast<u32x2*>(orow + d0) = w;
            }
    }

    // Writes C^T unscaled in fp32 as row `row` of a [N][D] fp32 tensor (the
    // same elements per lane as write()).
    __device__ __forceinline__ static void write_f32(const f32x16 (&acc)[DBLK], float* orow,
                                                     int hh) {
#pragma unroll
        for (int i = 0; i < DBLK; ++i)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d0 = 32 * i + 8 * gq + 4 * hh;
                const f32x4 y = {acc[i][4 * gq], acc[i][4 * gq + 1], acc[i][4 * gq + 2],
                                 acc[i][4 * gq + 3]};
                *reinterpret_cast<f32x4*>(orow + d0) = y;
            }
    }
};

// dS^T = P * (dP - Delta) for one 32 x 32 score block of the dQ pass (lane
// column = query row `row`, element j = key key0 + 8(j/4) + 4hh + j%4), with
// P = 2^(s * scale_log2 - l2) rebuilt from the forward's log-sum-exp. MASK:
// keys after the row get P = 0 (only blocks on the diagonal need it; keys
// past the sequence end are after every row). ALIBI: the exponent also
// carries the penalty, sl2 (key - row) in base-2 units (sl2 = the head's
// slope times log2 e).
template <bool MASK, bool ALIBI>
__device__ __forceinline__ f32x16 ds_block(const f32x16& s, const f32x16& dp, float scale_log2,
                                           float l2, float dl, int key0, int hh, int row,
                                           float sl2) {
    f32x16 ds;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int key = key0 + 8 * (j >> 2) + 4 * hh + (j & 3);
        const float off = ALIBI ? __builtin_fmaf(sl2, (float)(key - row), -l2) : -l2;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], scale_log2, off));
        if (MASK && key > row) p = 0.f;
        ds[j] = p * (dp[j] - dl);
    }
    return ds;
}

// P, or (DK) dS = P * (dP - Delta), in place for one 32 x 32 score block of
// the dK/dV pass (lane column = key `key`, element j = query row
// r0 + 8(j/4) + 4hh + j%4 of the tile, whose base-2 L and Delta sit in
// rl[row] and rl[BT + row]); P = 2^(s * scale_log2 - L). MASK: query rows
// before the key, or past the sequence end (q_first + row >= N), get P = 0.
// q_first: the block's first query row. ALIBI: the exponent also carries the
// penalty sl2 (key - query row), as in ds_block.
template <bool MASK, bool DK, bool ALIBI>
__device__ __forceinline__ void kv_p_block(f32x16& x, const f32x16& dp, const float* rl,
                                           int q_first, int r0, int hh, int key, int N,
                                           float scale_log2, float sl2) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
        const int r = r0 + 8 * gq + 4 * hh;  // the lane's 4 query rows in the tile
        const f32x4 lq = *reinterpret_cast<const f32x4*>(rl + r);
        f32x4 dq4;
        if (DK) dq4 = *reinterpret_cast<const f32x4*>(rl + BT + r);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int j = 4 * gq + jj;
            const int qrow = q_first + 8 * gq + 4 * hh + jj;
            const float off = ALIBI ? __builtin_fmaf(sl2, (float)(key - qrow), -lq[jj]) : -lq[jj];
            float pj = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], scale_log2, off));
            if (MASK) {
                if (qrow < key || qrow >= N) pj = 0.f;
            }
            x[j] = DK ? pj * (dp[j] - dq4[jj]) : pj;  // dS or P
        }
    }
}

// dS = P * (dP - Delta) in place for one 32 x 32 score block of the dK/dV
// pass, from the block's P as kv_p_block<MASK, false, ALIBI> left it (zero
// where masked): the same product, so the same bits, as kv_p_block with DK.
__device__ __forceinline__ void kv_ds_from_p(f32x16& x, const f32x16& dp, const float* rl, int r0,
                                             int hh) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
        const f32x4 dq4 = *reinterpret_cast<const f32x4*>(rl + BT + r0 + 8 * gq + 4 * hh);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) x[4 * gq + jj] = x[4 * gq + jj] * (dp[4 * gq + jj] - dq4[jj]);
    }
}

// 1-D work-unit index, XCD-aware order (the hardware deals workgroup ids
// round-robin over 8 XCDs; consecutive units on one XCD share a head), then
// (outer, tile) with the heaviest tile first.
__device__ __forceinline__ void decode(int per_outer, int& outer, int& idx) {
    const int units = gridDim.x;
    int u = blockIdx.x;
    if (units % NXCD == 0) u = (u % NXCD) * (units / NXCD) + u / NXCD;
    idx = u % per_outer;
    outer = u / per_outer;
}

// ---------------------------------------------------------------------------
// dQ pass: one workgroup per (b, query head, 128-row query tile), heaviest
// first. Also writes Delta = rowsum(dO * O) for the dK/dV pass.
// ---------------------------------------------------------------------------
template <int DT, int D, int RM>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ out,
    const float* __restrict__ lse, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dq,
    float* __restrict__ delta, const float* __restrict__ table,
    const float* __restrict__ slopes, int Hq, int Hkv, int N, int n_qtiles, float scale_log2,
    float scale) {
    constexpr bool ALIBI = (RM & MOD_ALIBI) != 0;           // distance penalty on the scores
    constexpr int ROT = RM & ~MOD_ALIBI;
    constexpr bool ROPE = ROT == ROT_QK;                     // rotate the loaded q, k
    constexpr bool ROPE_OUT = ROPE || ROT == ROT_QK_OUT;    // turn dq, dk back
    typedef Wave<DT, D> W;
    typedef Streamer<DT, D, ROPE, 4> S;
    constexpr int TILE = BT * D;
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE];  // K0 V0 K1 V1

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, n = lane & 31, hh = lane >> 5;
    int bh, slot;
    decode(n_qtiles, bh, slot);
    const int qt = n_qtiles - 1 - slot;
    const int b = bh / Hq, h = bh % Hq;
    const int g = h / (Hq / Hkv);
    const int qw0 = qt * BR + 32 * wave;
    const int row = qw0 + n;
    const float sl2 = ALIBI ? slopes[h] * LOG2E : 0.f;
    const int64_t qhead = ((int64_t)b * Hq + h) * N;
    const int64_t kvhead = ((int64_t)b * Hkv + g) * N;
    const uint16_t* kbase = k + kvhead * D;
    const uint16_t* vbase = v + kvhead * D;
    const int n_tiles = (min(qt * BR + BR, N) - 1) / BT + 1;
    const int wave_tiles = qw0 < N ? min(qw0 + 31, N - 1) / BT + 1 : 0;

    typename W::vec8 qf[W::QCH], dof[W::QCH];
    W::load_rows(qf, q + qhead * D, ROPE ? table : nullptr, qw0, N, n, hh);
    W::load_rows(dof, dout + qhead * D, nullptr, qw0, N, n, hh);
    // Delta_i = dO_i . O_i (this lane's half of the head dim, then the other's)
    float dl = 0.f, l2 = 0.f;
    if (row < N) {
        const uint16_t* orow = out + (qhead + row) * D;
#pragma unroll
        for (int c = 0; c < W::QCH; ++c) {
            const u32x4 o = *reinterpret_cast<const u32x4*>(orow + 16 * c + 8 * hh);
            const u32x4 d = __builtin_bit_cast(u32x4, dof[c]);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                dl += W::F::lo(o[t]) * W::F::lo(d[t]) + W::F::hi(o[t]) * W::F::hi(d[t]);
        }
        l2 = lse[qhead + row] * LOG2E;
    }
    dl += __shfl_xor(dl, 32);
    if (row < N && hh == 0) delta[qhead + row] = dl;

    f32x16 acc[W::DBLK];
#pragma unroll
    for (int i = 0; i < W::DBLK; ++i) acc[i] = f32x16{};

    S st;
    auto rt = [&](int t) { return rows_rsrc(table, ROPE ? D : 0, t, N); };
    st.issue(smem, smem + TILE, rows_rsrc(kbase, D, 0, N), rows_rsrc(vbase, D, 0, N), rt(0), wave,
             lane);
    for (int t = 0; t < n_tiles; ++t) {
        uint16_t* Ks = smem + (t & 1) * 2 * TILE;
        const uint16_t* Vs = Ks + TILE;
        wait_all_loads();
        st.finish(Ks, nullptr, false, wave, lane);
        __syncthreads();  // tile t complete; the other buffers are no longer read
        if (t + 1 < n_tiles) {
            uint16_t* nk = smem + ((t + 1) & 1) * 2 * TILE;
            st.issue(nk, nk + TILE, rows_rsrc(kbase, D, t + 1, N), rows_rsrc(vbase, D, t + 1, N),
                     rt(t + 1), wave, lane);
        }
        if (t >= wave_tiles) continue;
        const int k0 = t * BT;
        const bool diag = k0 + BT - 1 > qw0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            // S^T and dP^T for keys k0 + 32kb .. +31 (lane column = query row)
            f32x16 s = W::score(Ks, 32 * kb, qf, n, hh);
            const f32x16 dp = W::score(Vs, 32 * kb, dof, n, hh);
            // only tiles on the diagonal mask (a wave-uniform branch)
            const f32x16 ds =
                diag ? ds_block<true, ALIBI>(s, dp, scale_log2, l2, dl, k0 + 32 * kb, hh, row, sl2)
                     : ds_block<false, ALIBI>(s, dp, scale_log2, l2, dl, k0 + 32 * kb, hh, row,
                                              sl2);
            u32x4 y[2];
            W::pack(ds, y);
            W::pv(acc, Ks, 32 * kb, y, lane);
        }
    }
    if (row < N)
        W::write(acc, scale, dq + (qhead + row) * D, ROPE_OUT ? table + (int64_t)row * D : nullptr,
                 hh);
}

// ---------------------------------------------------------------------------
// dQ pass, balanced: one 8-wave workgroup per (b, query head, pair p of
// 128-row query tiles), used where one workgroup per tile would be resident
// on the chip all at once, so that its heaviest tile would set the time. The
// heavy tile T-1-p needs nh key tiles and the light tile p needs nl (an odd
// T's middle tile has no partner: nl = 0). Half A (waves 0-3) takes the
// heavy rows over key tiles [0, X), X = ceil((nh + nl) / 2); half B (waves
// 4-7) the light rows over [0, nl), then the heavy rows over [X, nh), so
// neither half takes more than X steps. Each half streams its own key tiles
// through its own LDS buffers. At the end half B hands its fp32 sums of the
// heavy rows to half A through LDS; A adds them to its own (A + B, a fixed
// order: deterministic) and writes those rows, B writes the light rows.
// ---------------------------------------------------------------------------
template <int DT, int D, int RM>
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_pair_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ out,
    const float* __restrict__ lse, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dq,
    float* __restrict__ delta, const float* __restrict__ table,
    const float* __restrict__ slopes, int Hq, int Hkv, int N, int n_qtiles, float scale_log2,
    float scale) {
    constexpr bool ALIBI = (RM & MOD_ALIBI) != 0;           // distance penalty on the scores
    constexpr int ROT = RM & ~MOD_ALIBI;
    constexpr bool ROPE = ROT == ROT_QK;                     // rotate the loaded q, k
    constexpr bool ROPE_OUT = ROPE || ROT == ROT_QK_OUT;    // turn dq, dk back
    typedef Wave<DT, D> W;
    typedef Streamer<DT, D, ROPE, 4> S;
    constexpr int TILE = BT * D;
    __shared__ __attribute__((aligned(16))) uint16_t smem[8 * TILE];  // per half: K0 V0 K1 V1

    const int tid = threadIdx.x;
    const int wave_wg = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave_wg >> 2;  // 0: A, 1: B
    const int wave = wave_wg & 3;   // wave inside its half
    const int lane = tid & 63, n = lane & 31, hh = lane >> 5;
    int bh, slot;
    decode((n_qtiles + 1) / 2, bh, slot);
    const int hv = n_qtiles - 1 - slot;     // the heavy tile
    const int lt = slot < hv ? slot : -1;   // the light tile, if any
    const int b = bh / Hq, h = bh % Hq;
    const int g = h / (Hq / Hkv);
    const float sl2 = ALIBI ? slopes[h] * LOG2E : 0.f;
    const int64_t qhead = ((int64_t)b * Hq + h) * N;
    const int64_t kvhead = ((int64_t)b * Hkv + g) * N;
    const uint16_t* kbase = k + kvhead * D;
    const uint16_t* vbase = v + kvhead * D;
    const int nh = (min(hv * BR + BR, N) - 1) / BT + 1;
    const int nl = lt >= 0 ? (min(lt * BR + BR, N) - 1) / BT + 1 : 0;
    const int X = (nh + nl + 1) / 2;
    const bool b_heavy = nh > X;  // half B also takes heavy key tiles
    uint16_t* hbuf = smem + half * 4 * TILE;

    // the key tile this half reads at step s, or -1 for none
    auto tile_at = [&](int s) -> int {
        if (half == 0 || s < nl) return s;
        const int t = X + (s - nl);
        return t < nh ? t : -1;
    };

    // the wave's stationary rows, their Delta and L, and its dQ sums
    typename W::vec8 qf[W::QCH], dof[W::QCH];
    float dl = 0.f, l2 = 0.f;
    int qw0 = 0, row = 0, wave_tiles = 0;
    f32x16 acc[W::DBLK];
    auto setup = [&](int qt, bool write_delta) {
        qw0 = qt * BR + 32 * wave;
        row = qw0 + n;
        wave_tiles = qw0 < N ? min(qw0 + 31, N - 1) / BT + 1 : 0;
        W::load_rows(qf, q + qhead * D, ROPE ? table : nullptr, qw0, N, n, hh);
        W::load_rows(dof, dout + qhead * D, nullptr, qw0, N, n, hh);
        dl = 0.f;
        l2 = 0.f;
        if (row < N) {
            const uint16_t* orow = out + (qhead + row) * D;
#pragma unroll
            for (int c = 0; c < W::QCH; ++c) {
                const u32x4 o = *reinterpret_cast<const u32x4*>(orow + 16 * c + 8 * hh);
                const u32x4 d = __builtin_bit_cast(u32x4, dof[c]);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    dl += W::F::lo(o[t]) * W::F::lo(d[t]) + W::F::hi(o[t]) * W::F::hi(d[t]);
            }
            l2 = lse[qhead + row] * LOG2E;
        }
        dl += __shfl_xor(dl, 32);
        if (write_delta && row < N && hh == 0) delta[qhead + row] = dl;
#pragma unroll
        for (int i = 0; i < W::DBLK; ++i) acc[i] = f32x16{};
    };
    // B starts on the light rows, or with no light tile on the heavy rows
    // (whose Delta A writes)
    setup(half == 1 && nl > 0 ? lt : hv, half == 0 || nl > 0);

    S st;
    auto rt = [&](int t) { return rows_rsrc(table, ROPE ? D : 0, t, N); };
    {
        const int t0 = tile_at(0);
        if (t0 >= 0)
            st.issue(hbuf, hbuf + TILE, rows_rsrc(kbase, D, t0, N), rows_rsrc(vbase, D, t0, N),
                     rt(t0), wave, lane);
    }
    for (int s = 0; s < X; ++s) {
        const int t = tile_at(s);
        uint16_t* Ks = hbuf + (s & 1) * 2 * TILE;
        const uint16_t* Vs = Ks + TILE;
        wait_all_loads();
        if (t >= 0) st.finish(Ks, nullptr, false, wave, lane);
        __syncthreads();  // step s's tiles complete; the other buffers are no longer read
        const int tn = s + 1 < X ? tile_at(s + 1) : -1;
        if (tn >= 0) {
            uint16_t* nk = hbuf + ((s + 1) & 1) * 2 * TILE;
            st.issue(nk, nk + TILE, rows_rsrc(kbase, D, tn, N), rows_rsrc(vbase, D, tn, N),
                     rt(tn), wave, lane);
        }
        if (half == 1 && s == nl && nl > 0 && b_heavy) {
            // the light rows are complete: write them, then take the heavy rows
            if (row < N)
                W::write(acc, scale, dq + (qhead + row) * D,
                         ROPE_OUT ? table + (int64_t)row * D : nullptr, hh);
            setup(hv, false);
        }
        if (t < 0 || t >= wave_tiles) continue;
        const int k0 = t * BT;
        const bool diag = k0 + BT - 1 > qw0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            // S^T and dP^T for keys k0 + 32kb .. +31 (lane column = query row)
            const f32x16 sc = W::score(Ks, 32 * kb, qf, n, hh);
            const f32x16 dp = W::score(Vs, 32 * kb, dof, n, hh);
            // only tiles on the diagonal mask (a wave-uniform branch)
            const f32x16 ds = diag
                ? ds_block<true, ALIBI>(sc, dp, scale_log2, l2, dl, k0 + 32 * kb, hh, row, sl2)
                : ds_block<false, ALIBI>(sc, dp, scale_log2, l2, dl, k0 + 32 * kb, hh, row, sl2);
            u32x4 y[2];
            W::pack(ds, y);
            W::pv(acc, Ks, 32 * kb, y, lane);
        }
    }
    __syncthreads();  // every wave is done with the stream buffers
    constexpr int SLOTS = 16 * W::DBLK;
    float* red = reinterpret_cast<float*>(smem) + (wave * SLOTS) * 64 + lane;
    if (b_heavy && half == 1) {
#pragma unroll
        for (int i = 0; i < W::DBLK; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) red[(16 * i + j) * 64] = acc[i][j];
    }
    __syncthreads();
    if (half == 0) {
        if (b_heavy) {
#pragma unroll
            for (int i = 0; i < W::DBLK; ++i)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[i][j] += red[(16 * i + j) * 64];
        }
        if (row < N)
            W::write(acc, scale, dq + (qhead + row) * D,
                     ROPE_OUT ? table + (int64_t)row * D : nullptr, hh);
    } else if (!b_heavy && nl > 0 && row < N) {
        // half B stayed on the light rows
        W::write(acc, scale, dq + (qhead + row) * D, ROPE_OUT ? table + (int64_t)row * D : nullptr,
                 hh);
    }
}

// ---------------------------------------------------------------------------
// dK/dV pass: one workgroup per (b, key/value head, 32*RW-key tile),
// heaviest first; it walks the 64-row query tiles at or after its keys for
// every query head of the group. Its 2*RW waves take two roles on the same
// keys and the same streamed tiles: waves 0 .. RW-1 accumulate dV (S, P),
// waves RW .. 2RW-1 accumulate dK (dP, and dS from the P that the dV wave on
// the same keys hands over through LDS). Split this way each wave holds one
// D-wide accumulator and one stationary operand, so two waves fit on a SIMD
// (wave w and w + 4 share one), where a wave holding both accumulators would
// run alone; and S is computed once.
// With QS > 1 the workgroup holds QS such groups of 2*RW waves on the same
// keys: group c takes the query tiles c, c + QS, c + 2QS, ... of the walk,
// each with its own stream buffers, and at the end the groups' partial dK
// and dV are added in a fixed order through LDS (still one writer per
// element and deterministic). The heaviest key tiles then finish QS times
// sooner when there are too few workgroups to keep every CU busy.
// With HS = 2 (GQA, an even group) two workgroups share each key tile, one
// per half of the group's query heads, so the heaviest tiles carry half the
// steps and the heaviest-first order balances the CUs; each writes its
// unscaled fp32 sums to `part` ([half][dK, dV][B*Hkv*N][D]) and
// kv_reduce_kernel adds the two halves (a + b: the same value whichever
// finished first) and finishes dK and dV as the single-writer epilogue does.
// ---------------------------------------------------------------------------
template <int DT, int D, int RM, int RW, int QS, int HS>
__global__ __launch_bounds__(128 * RW * QS, RW * QS == 2 ? 2 : 1) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ lse,
    const uint16_t* __restrict__ dout, const float* __restrict__ delta, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, float* __restrict__ part, const float* __restrict__ table,
    const float* __restrict__ slopes, int Hq, int Hkv, int N, int n_ktiles, float scale_log2,
    float scale) {
    constexpr bool ALIBI = (RM & MOD_ALIBI) != 0;           // distance penalty on the scores
    constexpr int ROT = RM & ~MOD_ALIBI;
    constexpr bool ROPE = ROT == ROT_QK;                     // rotate the loaded q, k
    constexpr bool ROPE_OUT = ROPE || ROT == ROT_QK_OUT;    // turn dq, dk back
    constexpr int KW = 32 * RW;  // keys per workgroup
    typedef Wave<DT, D> W;
    typedef Streamer<DT, D, ROPE, 2 * RW> S;
    constexpr int TILE = BT * D;
    // per query group: Q0 dO0 Q1 dO1, and per buffer 64 scaled L and 64 Delta values
    __shared__ __attribute__((aligned(16))) uint16_t smem[QS * 4 * TILE];
    __shared__ __attribute__((aligned(16))) float rows_lds[QS][2][2 * BT];
    // P of one 32-query block, handed from each dV wave to the dK wave on the
    // same keys: [block parity][query group][key block][4][64 lanes][4], fp32;
    // one buffer per block of a tile where LDS allows (then no barrier is
    // needed before the second block's P is written), else one shared
    constexpr int STREAM_BYTES = QS * 4 * TILE * 2 + QS * 2 * 2 * BT * 4;
    constexpr int P_BYTES = QS * RW * 4 * 64 * 16;
    constexpr int WG_PER_CU = RW * QS == 2 ? 2 : 1;
    constexpr int PB = WG_PER_CU * (STREAM_BYTES + 2 * P_BYTES) <= 160 * 1024 ? 2 : 1;
    __shared__ __attribute__((aligned(16))) f32x4 p_lds[PB][QS][RW][4][64];

    const int tid = threadIdx.x;
    const int wave_wg = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qg = wave_wg / (2 * RW);   // query group
    // wave inside its group (its role and keys). Waves w and w + 4 of the
    // workgroup share a SIMD, so with two 4-wave groups the second group's
    // roles are swapped: every SIMD then runs one dV and one dK wave, instead
    // of two dK waves (S, dP, dS and dK: 1.5x the matrix work) on two SIMDs.
    const int wave = (QS == 2 && RW == 2 && (qg & 1)) ? (wave_wg + RW) % (2 * RW)
                                                      : wave_wg % (2 * RW);
    const bool dk_role = wave >= RW;
    const int lane = tid & 63, n = lane & 31, hh = lane >> 5;
    int bg, slot;
    decode(n_ktiles * HS, bg, slot);
    const int kt = slot / HS;  // heaviest first: key tile 0 sees every query
    const int hs = slot % HS;  // which half of the group's query heads (HS = 2)
    const int b = bg / Hkv, g = bg % Hkv;
    const int group = Hq / Hkv / HS;  // query heads this workgroup walks
    const int kw0 = kt * KW + 32 * (wave % RW);
    const int key = kw0 + n;
    const int64_t kvhead = ((int64_t)b * Hkv + g) * N;

    // the query tiles of one head that see the workgroup's keys, all heads
    const int t0 = (kt * KW) / BT;
    const int per_head = (N - 1) / BT + 1 - t0;
    const int steps = per_head * group;
    const int rounds = (steps + QS - 1) / QS;  // group qg takes step s * QS + qg of round s
    auto job = [&](int i, int& qh, int& tq) {
        qh = (g * HS + hs) * group + i / per_head;
        tq = t0 + i % per_head;
    };
    uint16_t* gbuf = smem + qg * 4 * TILE;

    S st;
    auto start = [&](int s) {
        const int i = s * QS + qg;
        if (i >= steps) return;
        int qh, tq;
        job(i, qh, tq);
        const int64_t qhead = ((int64_t)b * Hq + qh) * N;
        uint16_t* a = gbuf + (s & 1) * 2 * TILE;
        st.issue(a, a + TILE, rows_rsrc(q + qhead * D, D, tq, N),
                 rows_rsrc(dout + qhead * D, D, tq, N),
                 rows_rsrc(table, ROPE ? D : 0, tq, N), wave, lane);
        st.issue_rows(rows_rsrc(lse + qhead, 1, tq, N), rows_rsrc(delta + qhead, 1, tq, N), wave,
                      lane);
    };

    // The whole loop of one role (the same barriers in the same order for
    // both, so the workgroup stays in step), compiled separately per role.
    // Per 32-query block the dV wave computes S and P and hands P to the dK
    // wave on its keys through LDS; the dK wave computes dP meanwhile and
    // then dS from that P (so S is computed once per block, by the dV wave).
    // Every wave passes the same barriers, with or without work.
    auto run = [&](auto dk_tag) {
        constexpr bool DK = decltype(dk_tag)::value;
        typename W::vec8 kf[W::QCH], vf[W::QCH];  // stationary K (dV waves) or V (dK waves)
        if constexpr (!DK) W::load_rows(kf, k + kvhead * D, ROPE ? table : nullptr, kw0, N, n, hh);
        if constexpr (DK) W::load_rows(vf, v + kvhead * D, nullptr, kw0, N, n, hh);
        f32x16 acc[W::DBLK];  // dK^T (DK) or dV^T
#pragma unroll
        for (int i = 0; i < W::DBLK; ++i) acc[i] = f32x16{};
        start(0);
        for (int s = 0; s < rounds; ++s) {
            const int i = s * QS + qg;
            const bool live = i < steps;  // the last round may leave a group idle
            int qh = 0, tq = 0;
            if (live) job(i, qh, tq);
            uint16_t* Qs = gbuf + (s & 1) * 2 * TILE;
            const uint16_t* dOs = Qs + TILE;
            float* rl = rows_lds[qg][s & 1];
            wait_all_loads();
            if (live) st.finish(Qs, rl, true, wave, lane);
            __syncthreads();  // round s complete; the other buffers are no longer read
            if (s + 1 < rounds) start(s + 1);
            const int q0 = tq * BT;
            const float sl2 = ALIBI && live ? slopes[qh] * LOG2E : 0.f;  // the tile's query head
            // work unless the group is idle, the wave has no keys or every
            // query of the tile precedes them (uniform over the wave pair)
            const bool work = live && kw0 < N && q0 + BT - 1 >= kw0;
            // masking only where the tile crosses the wave's keys or the
            // sequence end (a wave-uniform branch)
            const bool mask = q0 < kw0 + 31 || q0 + BT > N;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                // queries q0 + 32qb .. +31 (lane column = key)
                f32x4* pex = &p_lds[qb % PB][qg][wave % RW][0][lane];  // this pair's P, this lane's
                f32x16 x, dp{};  // dp: dK waves only
                u32x4 y[2];
                if (work) {
                    if constexpr (!DK) {
                        x = W::score(Qs, 32 * qb, kf, n, hh);
                        if (mask)
                            kv_p_block<true, false, ALIBI>(x, dp, rl, q0 + 32 * qb, 32 * qb, hh, key,
                                                           N, scale_log2, sl2);
                        else
                            kv_p_block<false, false, ALIBI>(x, dp, rl, q0 + 32 * qb, 32 * qb, hh,
                                                            key, N, scale_log2, sl2);
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4)
                            pex[64 * g4] = f32x4{x[4 * g4], x[4 * g4 + 1], x[4 * g4 + 2], x[4 * g4 + 3]};
                        W::pack(x, y);
                    } else {
                        dp = W::score(dOs, 32 * qb, vf, n, hh);
                    }
                }
                __syncthreads();  // P of this block is in LDS
                if (work) {
                    if constexpr (DK) {
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const f32x4 t = pex[64 * g4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) x[4 * g4 + e] = t[e];
                        }
                        kv_ds_from_p(x, dp, rl, 32 * qb, hh);
                        W::pack(x, y);
                    }
                    W::pv(acc, DK ? Qs : dOs, 32 * qb, y, lane);  // dK^T += Q^T dS, dV^T += dO^T P
                }
                // with one buffer, the dK wave has read this P before the next
                // block's is written (after the last block, and with two
                // buffers, the next round's barrier does it)
                if (PB == 1 && qb == 0) __syncthreads();
            }
        }
        if constexpr (QS > 1) {
            // groups 1.. hand their partial sums to group 0 through LDS, in order
            static_assert(QS == 2, "one partner group");
            constexpr int SLOTS = 16 * W::DBLK;
            float* red = reinterpret_cast<float*>(smem) + (wave * SLOTS) * 64 + lane;
            __syncthreads();  // every group is done with its stream buffers
            if (qg == 1) {
#pragma unroll
                for (int i = 0; i < W::DBLK; ++i)
#pragma unroll
                    for (int j = 0; j < 16; ++j) red[(16 * i + j) * 64] = acc[i][j];
            }
            __syncthreads();
            if (qg != 0) return;
#pragma unroll
            for (int i = 0; i < W::DBLK; ++i)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[i][j] += red[(16 * i + j) * 64];
        }
        if (key < N) {
            if constexpr (HS > 1) {
                const int64_t kv_rows = (int64_t)gridDim.x / (n_ktiles * HS) * N;
                W::write_f32(acc, part + ((2 * hs + (DK ? 0 : 1)) * kv_rows + kvhead + key) * D,
                             hh);
            } else if (DK) {
                W::write(acc, scale, dk + (kvhead + key) * D,
                         ROPE_OUT ? table + (int64_t)key * D : nullptr, hh);
            } else {
                W::write(acc, 1.f, dv + (kvhead + key) * D, nullptr, hh);
            }
        }
    };
    if (dk_role)
        run(std::integral_constant<bool, true>());
    else
        run(std::integral_constant<bool, false>());
}

// The two halves' sums of a head-split dK/dV pass: dV = a + b, and dK the
// same sum scaled by tau and (RoPE) turned back by R(-p), exactly as
// Wave::write finishes a single workgroup's sums. One thread per 4 elements
// (two pairs) of a row of dK and of dV.
template <int DT, bool ROPE>
__global__ __launch_bounds__(256) void kv_reduce_kernel(const float* __restrict__ part,
                                                        uint16_t* __restrict__ dk,
                                                        uint16_t* __restrict__ dv,
                                                        const float* __restrict__ table,
                                                        int64_t kv_rows, int N, int D,
                                                        float scale) {
    typedef Fmt<DT> F;
    const int64_t quads = kv_rows * D / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= quads) return;
    const int64_t e = 4 * i;  // element offset in [kv_rows][D]
    const int64_t span = kv_rows * D;
    const f32x4 k0 = *reinterpret_cast<const f32x4*>(part + e);
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(part + span + e);
    const f32x4 k1 = *reinterpret_cast<const f32x4*>(part + 2 * span + e);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(part + 3 * span + e);
    float y[4], x[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        y[t] = (k0[t] + k1[t]) * scale;
        x[t] = (v0[t] + v1[t]) * 1.f;
    }
    if (ROPE) {
        const int64_t row = e / D;
        const int d0 = (int)(e % D);
        const f32x4 cs = *reinterpret_cast<const f32x4*>(table + (row % N) * D + d0);
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            const float c = cs[2 * pr], s = cs[2 * pr + 1];
            const float y0 = y[2 * pr], y1 = y[2 * pr + 1];
            y[2 * pr] = __builtin_fmaf(y0, c, y1 * s);
            y[2 * pr + 1] = __builtin_fmaf(y1, c, -(y0 * s));
        }
    }
    u32x2 wk, wv;
    wk[0] = F::pack2(y[0], y[1]);
    wk[1] = F::pack2(y[2], y[3]);
    wv[0] = F::pack2(x[0], x[1]);
    wv[1] = F::pack2(x[2], x[3]);
    *reinterpret_cast<u32x2*>(dk + e) = wk;
    *reinterpret_cast<u32x2*>(dv + e) = wv;
}

template <int DT, int D, int RM>
static hipError_t launch_typed(const BwdArgs& a, hipStream_t stream) {
    const float scale = (float)(1.0 / sqrt((double)D));
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const int n_qtiles = (a.N + BR - 1) / BR;
    // dK/dV pass: 128 keys per workgroup (8 waves), or 64 (4 waves) when that
    // leaves fewer workgroups than CUs; and with at most two 64-key
    // workgroups per CU, two query groups per workgroup (8 waves)
    const int64_t k_units_128 = (int64_t)((a.N + 127) / 128) * a.Hkv * a.B;
    int rw = k_units_128 >= 256 ? 4 : 2;
    if (a.shape == BWD_SHAPE_K128) rw = 4;
    if (a.shape == BWD_SHAPE_K64 || a.shape == BWD_SHAPE_K64X2 || a.shape == BWD_SHAPE_K64X2H)
        rw = 2;
    const int n_ktiles = (a.N + 32 * rw - 1) / (32 * rw);
    const int64_t q_units = (int64_t)n_qtiles * a.Hq * a.B;
    const int64_t k_units = (int64_t)n_ktiles * a.Hkv * a.B;
    if (q_units > 0x7fffffff || k_units > 0x7fffffff) return hipErrorInvalidConfiguration;
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
    const uint16_t* k = static_cast<const uint16_t*>(a.k);
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    const uint16_t* out = static_cast<const uint16_t*>(a.out);
    const uint16_t* dout = static_cast<const uint16_t*>(a.dout);
    // the dQ pass writes Delta, which the dK/dV pass reads: same stream, in order.
    // Where one workgroup per query tile (two per CU) would all be resident at
    // once, the heaviest tile would set the time: pair heavy and light tiles.
    if (n_qtiles >= 2 && a.dq_shape != BWD_DQ_TILE &&
        (a.dq_shape == BWD_DQ_PAIR || q_units <= 2 * NUM_CUS))
        attn_bwd_dq_pair_kernel<DT, D, RM>
            <<<dim3((unsigned)((n_qtiles + 1) / 2 * (int64_t)a.Hq * a.B)), 512, 0, stream>>>(
                q, k, v, out, a.lse, dout, static_cast<uint16_t*>(a.dq), a.delta, a.table, a.slopes, a.Hq,
                a.Hkv, a.N, n_qtiles, scale_log2, scale);
    else
        attn_bwd_dq_kernel<DT, D, RM><<<dim3((unsigned)q_units), 256, 0, stream>>>(
            q, k, v, out, a.lse, dout, static_cast<uint16_t*>(a.dq), a.delta, a.table, a.slopes, a.Hq,
            a.Hkv, a.N, n_qtiles, scale_log2, scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    uint16_t* dk = static_cast<uint16_t*>(a.dk);
    uint16_t* dv = static_cast<uint16_t*>(a.dv);
    const int group = a.Hq / a.Hkv;
    // two workgroups per 64-key tile, one per half of the query heads, where
    // one workgroup per tile would leave the CUs unbalanced (at most two
    // rounds of them, so the heaviest tile sets the time)
    const bool split = rw == 2 && group % 2 == 0 &&
                       (a.shape == BWD_SHAPE_K64X2H ||
                        (a.shape == BWD_SHAPE_AUTO && k_units <= 2 * NUM_CUS));
    if (split) {
        const int64_t kv_rows = (int64_t)a.B * a.Hkv * a.N;
        const int64_t quads = kv_rows * a.D / 4;
        if (2 * k_units > 0x7fffffff || (quads + 255) / 256 > 0x7fffffff)
            return hipErrorInvalidConfiguration;
        float* part = nullptr;
        e = hipMallocAsync(reinterpret_cast<void**>(&part), 4 * kv_rows * a.D * sizeof(float),
                           stream);
        if (e != hipSuccess) return e;
        attn_bwd_dkdv_kernel<DT, D, RM, 2, 2, 2><<<dim3((unsigned)(2 * k_units)), 512, 0, stream>>>(
            q, k, v, a.lse, dout, a.delta, dk, dv, part, a.table, a.slopes, a.Hq, a.Hkv, a.N, n_ktiles,
            scale_log2, scale);
        e = hipGetLastError();
        if (e == hipSuccess) {
            constexpr int ROT = RM & ~MOD_ALIBI;
            kv_reduce_kernel<DT, ROT == ROT_QK || ROT == ROT_QK_OUT><<<dim3((unsigned)((quads + 255) / 256)), 256, 0,
                                                 stream>>>(part, dk, dv, a.table, kv_rows, a.N,
                                                           a.D, scale);
            e = hipGetLastError();
        }
        const hipError_t f = hipFreeAsync(part, stream);
        return e != hipSuccess ? e : f;
    }
    if (rw == 4)
        attn_bwd_dkdv_kernel<DT, D, RM, 4, 1, 1><<<dim3((unsigned)k_units), 512, 0, stream>>>(
            q, k, v, a.lse, dout, a.delta, dk, dv, nullptr, a.table, a.slopes, a.Hq, a.Hkv, a.N, n_ktiles,
            scale_log2, scale);
    else if (a.shape == BWD_SHAPE_K64X2 || a.shape == BWD_SHAPE_K64X2H ||
             (a.shape != BWD_SHAPE_K64 && k_units <= 2 * NUM_CUS))
        attn_bwd_dkdv_kernel<DT, D, RM, 2, 2, 1><<<dim3((unsigned)k_units), 512, 0, stream>>>(
            q, k, v, a.lse, dout, a.delta, dk, dv, nullptr, a.table, a.slopes, a.Hq, a.Hkv, a.N, n_ktiles,
            scale_log2, scale);
    else
        attn_bwd_dkdv_kernel<DT, D, RM, 2, 1, 1><<<dim3((unsigned)k_units), 256, 0, stream>>>(
            q, k, v, a.lse, dout, a.delta, dk, dv, nullptr, a.table, a.slopes, a.Hq, a.Hkv, a.N, n_ktiles,
            scale_log2, scale);
    return hipGetLastError();
}

template <int DT, int RM>
static hipError_t launch_dt(const BwdArgs& a, hipStream_t stream) {
    return a.D == 64 ? launch_typed<DT, 64, RM>(a, stream) : launch_typed<DT, 128, RM>(a, stream);
}

}  // namespace bwd

template <int DT>
static hipError_t launch_rot(const BwdArgs& a, int rot, hipStream_t stream) {
    if (a.slopes != nullptr) {  // ALiBi: on operands rotated beforehand, or none
        if (rot == ROT_QK_OUT) return bwd::launch_dt<DT, ROT_QK_OUT | MOD_ALIBI>(a, stream);
        if (rot == ROT_NONE) return bwd::launch_dt<DT, ROT_NONE | MOD_ALIBI>(a, stream);
        return hipErrorInvalidValue;
    }
    return rot == ROT_QK       ? bwd::launch_dt<DT, ROT_QK>(a, stream)
           : rot == ROT_QK_OUT ? bwd::launch_dt<DT, ROT_QK_OUT>(a, stream)
                               : bwd::launch_dt<DT, ROT_NONE>(a, stream);
}

hipError_t launch_attn_bwd(const BwdArgs& a, int rot, hipStream_t stream) {
    return a.dtype == DT_BF16 ? launch_rot<DT_BF16>(a, rot, stream)
                              : launch_rot<DT_FP16>(a, rot, stream);
}

}  // namespace rac
