// attn_fwd.hip -- causal MHA/GQA attention forward for gfx950, with RoPE fused
// into the loads of both Q and K (RM = ROT_QK, or ROT_QK_HALF for the
// half-split pairing), of Q only (RM = ROT_Q: the GQA split path, K rotated
// beforehand) or of neither (RM = ROT_NONE); MOD_ALIBI added to the mode
// puts the ALiBi distance penalty on the scores (it starts the score
// accumulators, so the softmax is unchanged).
//
// Method: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (rainbus digest), background "FlashAttention and online softmax"
// and the forward Algorithm 1: a block of query rows walks the key tiles,
// keeps the running row maximum m and denominator l on chip, and writes
// o = u / l and the log-sum-exp L. The digest's precision design is kept:
// fp32 statistics and accumulators, base-2 exponent. The fused variant is the
// single kernel of "AttnFuse Makes RoPE a First-Class Attention Compilation
// Operation", paragraph 3 ("in-kernel rotation"): query rows are rotated once
// when loaded, and every key tile is rotated each time a workgroup loads it --
// the compute-and-tiling cost that paragraph contrasts with pre-rotation.
//
// gfx950 mapping (64-lane waves, v_mfma_f32_32x32x16 bf16/fp16):
//   * A "row block" is 4 waves = BM = 128 query rows of one (b, query head);
//     wave w owns rows q0 + 32w .. +31, lane (n, hh) = (lane % 32, lane / 32).
//   * Scores are computed transposed, S^T = K Q^T: A = K tile from LDS
//     (row = key), B = the wave's Q rows, kept in registers for the whole loop.
//     The fp32 result holds one query per lane column, so row statistics need
//     only in-lane reductions plus one exchange between the two lane halves.
//   * O^T = V^T P^T: the P^T accumulator registers are reused directly as the
//     B operand (the key order inside each 16-key step is permuted); the V^T
//     operand comes from the row-major V tile through the LDS transpose read
//     (ds_read_b64_tr_b16), gathering keys in that same permuted order.
//   * Key tiles of BN = 64 rows, double-buffered in LDS (V triple-buffered
//     where a wave runs the lagged schedule) with one barrier per tile. The
//     next tile's K and V go straight from global memory into LDS
//     (buffer_load_dwordx4 ... lds) while the current tile is computed; with RoPE
//     each thread also prefetches the cos/sin rows of the K chunks it loads
//     and rotates them in place before the barrier. Tiles past a wave's last
//     query are skipped and only tiles straddling the diagonal are masked.
//   * Running-max updates are lazy: a row keeps its maximum until a tile
//     raises it by more than 2^8, so most tiles skip the accumulator rescale;
//     probabilities stay <= 2^8 and the final o = u / l and L are unchanged.
//   * MFMA operands are read from LDS two MFMAs ahead of their use, and in
//     the two-head tile launch the waves that share a SIMD run half a step
//     apart (step() / step_lag()), so one's matrix work overlaps the other's
//     softmax.
//
// Two launch shapes share that per-wave core:
//   * attn_pair_kernel (the default): causal rows see a prefix of the keys, so
//     query tile t costs ~t+1 key-tile steps. A workgroup of 8 waves takes the
//     light tile p and its mirror T-1-p; half A (waves 0-3) runs the heavy
//     tile over the first X key tiles, half B (waves 4-7) runs the light tile
//     and then the heavy tile's remaining key tiles, X chosen so both halves
//     take the same number of steps. The two partial softmax states of the
//     heavy rows are merged through LDS at the end (each half merging and
//     writing half of the head dimension). Every workgroup then does
//     the same work, so a grid of one workgroup per CU finishes together.
//     While half B is on the light rows, both halves work on the same key
//     tile each step; half A alone loads (and rotates) it.
//   * attn_fwd_kernel: one workgroup per query tile (4 waves, or 8 for the
//     same tile of two query heads of a GQA group), heaviest first; used when
//     the grid has enough workgroups (>= 4 per CU) for that order to balance.
//   * attn_pair_heads_kernel: an 8-wave workgroup takes the 64-row query
//     tiles T-1-p and p of two query heads of one GQA group (heavy rows on
//     waves 0-3, light rows on waves 4-7); all four row blocks share every key
//     tile. Chosen only when forced (RAC_ATTN_SHAPE=pairheads).
//   All use a 1-D grid whose consecutive workgroups on one XCD (the hardware
//   deals workgroup ids round-robin over 8 XCDs) share a key/value head, so
//   each XCD's L2 serves one K/V head to all its readers.
#include <math.h>

#include "rac_device.h"
#include "rac_internal.h"

namespace rac {

constexpr int BM = 128;
constexpr int BN = 64;
constexpr int NXCD = 8;
constexpr int NUM_CUS = 256;
constexpr float LAZY_RESCALE_LOG2 = 8.0f;
constexpr float LN2 = 0.69314718055994530942f;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposed LDS read: in each 16-lane group, lane i receives element i%4 of
// the 8-byte chunks addressed by lanes 4e + i/4, e = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

template <int D>
struct Tile {
    // K and V tiles are stored unpadded, row = key, as 16-byte chunks whose
    // position inside the row is XOR-swizzled so that the MFMA operand reads
    // hit distinct LDS banks (see kswz / vswz).
    static constexpr int CH = D / 8;                     // 16-byte chunks per row
    static constexpr int K_ELEMS = BN * D;
    static constexpr int V_ELEMS = BN * D;
    static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
};

// Chunk swizzles. K: the score MFMA reads one chunk column from 16 consecutive
// rows at once, so rows spread over all chunk positions. V: the transpose read
// takes 4 adjacent chunks from each of 4 consecutive rows, so rows take
// disjoint aligned groups of 4 chunks.
template <int D>
__device__ __forceinline__ int kswz(int row) {
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int row) {
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// Number of key tiles query tile `qt` needs (keys 0 .. its last row).
__device__ __forceinline__ int kv_tiles_of(int qt, int N) {
    return (min(qt * BM + BM, N) - 1) / BN + 1;
}

typedef __attribute__((address_space(3))) void lds_void;

// Buffer descriptors of one key tile: K, V and (RoPE) cos/sin rows starting
// at the tile's first key. The descriptor's record count ends at the sequence
// end, so rows past it read as zeros (their scores are masked by causality and
// their probabilities are zero) without any per-lane clamping. A tile that
// starts at or past the end (the second 64-row half of a query tile of fewer
// than 65 rows, staged like a key tile) gets a record count of zero: every
// row reads as zero and nothing past the tensor is touched.
constexpr int BUF_RSRC_FLAGS = 0x00020000;  // raw (unformatted) 32-bit data
struct TileRsrc {
    __amdgpu_buffer_rsrc_t k, v, t;
};
template <int D>
__device__ __forceinline__ TileRsrc tile_rsrc(const uint16_t* kbase, const uint16_t* vbase,
                                              const float* table, int t, int N) {
    const int k0 = t * BN;
    const int64_t rows = N > k0 ? N - k0 : 0;
    const int kv_bytes = (int)min(rows * D * 2, (int64_t)0x7fffffff);
    const int tab_bytes = (int)min(rows * D * 4, (int64_t)0x7fffffff);
    TileRsrc r;
    r.k = __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (int64_t)k0 * D), 0, kv_bytes,
                                            BUF_RSRC_FLAGS);
    r.v = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (int64_t)k0 * D), 0, kv_bytes,
                                            BUF_RSRC_FLAGS);
    r.t = __builtin_amdgcn_make_buffer_rsrc((void*)(table ? table + (int64_t)k0 * D : nullptr), 0,
                                            table ? tab_bytes : 0, BUF_RSRC_FLAGS);
    return r;
}

// Loads of one K/V tile by a block of NW waves, straight from global memory
// into LDS (buffer_load ... lds: lane i of an instruction fills bytes
// 16i..16i+15 of a 1 KiB block). Block b of a tile holds chunks 64b..64b+63;
// a lane fetches the global chunk that the swizzle places there.
// With ROPE the K chunks land unrotated; each thread prefetches the cos/sin
// entries of the chunks it loaded and, once its loads have landed, rotates
// those chunks in place before the block's barrier.
// ROPE: 0 = K not rotated, 1 = adjacent pairs (2i, 2i+1), 2 = half-split
// pairs (d, d + D/2). With the half-split pairing a chunk's partner (same row,
// logical chunk XOR D/16) lands in the same 1 KiB block, loaded by lane
// XOR D/16 of the same instruction. The two lanes split the chunk pair's 8
// element pairs: the lane of the first-half chunk turns pairs 0-3, its partner
// lane pairs 4-7, each prefetching exactly the 8 table floats of its 4
// frequencies and reading and writing only its own 8-byte halves of the two
// chunks, so the lanes share no data.
template <int DT, int D, int ROPE, int NW>
struct TileStage {
    typedef Tile<D> T;
    static constexpr int INSTR = BN * T::CH / (64 * NW);  // 1 KiB blocks per wave and tensor
    f32x4 cs[ROPE ? INSTR : 1][2];

    // Loads block j (0 <= j < INSTR) of this wave's share: one 1 KiB block of
    // K into kbuf, one of V into vbuf, and (ROPE) the cos/sin entries of the K
    // block. `wave` must be wave-uniform.
    __device__ __forceinline__ void issue_part(int j, uint16_t* kbuf, uint16_t* vbuf,
                                               const TileRsrc& rs, int wave, int lane,
                                               bool with_v = true) {
        const int blk = wave * INSTR + j;
        const int g = blk * 64 + lane;          // chunk index inside the tile
        const int row = g / T::CH;
        const int pc = g % T::CH;               // physical chunk position
        const int lc = pc ^ kswz<D>(row);       // logical chunk
        const int kel = row * D + 8 * lc;       // element offsets in the tile
        const int vel = row * D + 8 * (pc ^ vswz<D>(row));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.k, (lds_void*)(kbuf + blk * 512), 16, kel * 2,
                                                 0, 0, 0);
        if (with_v)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.v, (lds_void*)(vbuf + blk * 512), 16,
                                                     vel * 2, 0, 0, 0);
        if (ROPE) {
            // adjacent: the 8 floats of this chunk's 4 pairs; half-split: this
            // lane's half (8 floats) of the 16 of frequencies 8 (lc mod CH/2) ..
            const int tel = ROPE == 1 ? kel
                                      : row * D + 16 * (lc % (T::CH / 2)) + 8 * (lc / (T::CH / 2));
            cs[j][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rs.t, tel * 4, 0, 0));
            cs[j][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rs.t, tel * 4 + 16, 0, 0));
        }
    }

    __device__ __forceinline__ void issue(uint16_t* kbuf, uint16_t* vbuf, const TileRsrc& rs,
                                          int wave, int lane) {
#pragma unroll
        for (int j = 0; j < INSTR; ++j) issue_part(j, kbuf, vbuf, rs, wave, lane);
    }
    // The "K" rows alone (staging query rows the same way).
    __device__ __forceinline__ void issue_k(uint16_t* kbuf, const TileRsrc& rs, int wave,
                                            int lane) {
#pragma unroll
        for (int j = 0; j < INSTR; ++j) issue_part(j, kbuf, nullptr, rs, wave, lane, false);
    }

    // ROPE only: rotate the K chunks this thread loaded. Call after its loads
    // have completed (s_waitcnt) and before the block's barrier. All reads
    // are issued before the first write, so their latencies overlap.
    __device__ __forceinline__ void rotate(uint16_t* buf, int wave, int lane) {
        if (ROPE == 0) return;
        if (ROPE == 1) {
            u32x4 x[INSTR];
#pragma unroll
            for (int j = 0; j < INSTR; ++j)
                x[j] = *reinterpret_cast<const u32x4*>(buf + (wave * INSTR + j) * 512 + lane * 8);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < INSTR; ++j)
                *reinterpret_cast<u32x4*>(buf + (wave * INSTR + j) * 512 + lane * 8) =
                    rope_rotate8<DT>(x[j], cs[j][0], cs[j][1]);
        } else {
            constexpr int X = T::CH / 2;  // partner lane / chunk offset
            u32x2* pa[INSTR];
            u32x2* pb[INSTR];
            u32x2 a[INSTR], b[INSTR];
#pragma unroll
            for (int j = 0; j < INSTR; ++j) {
                const int blk = wave * INSTR + j;
                const int g = blk * 64 + lane;
                const bool lo = ((g % T::CH) ^ kswz<D>(g / T::CH)) < X;
                // first-half chunk's lane: pairs 0-3; partner lane: pairs 4-7
                uint16_t* blk0 = buf + blk * 512;
                pa[j] = reinterpret_cast<u32x2*>(blk0 + (lane ^ (lo ? 0 : X)) * 8 + (lo ? 0 : 4));
                pb[j] = reinterpret_cast<u32x2*>(blk0 + (lane ^ (lo ? X : 0)) * 8 + (lo ? 0 : 4));
                a[j] = *pa[j];
                b[j] = *pb[j];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < INSTR; ++j) {
                rope_rotate_half4<DT>(a[j], b[j], cs[j][0], cs[j][1]);
                *pa[j] = a[j];
                *pb[j] = b[j];
            }
        }
    }
};

// The next tile's loads, handed to the score MFMA loop so that their issue
// (which stalls while the memory pipeline drains earlier requests) overlaps
// matrix work instead of stalling the wave between tiles.
struct NextLoads {
    bool active;  // false: nothing to load
    uint16_t* kbuf;
    uint16_t* vbuf;
    TileRsrc rs;
    int wave, lane;
};

// Waits for this wave's outstanding memory operations, including its loads
// into LDS.
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0); }

// Per-wave flash-attention state for QB blocks of 32 query rows (rows
// q_first + 32b + n, b < QB) and its per-tile work. Every block's scores use
// the same K operands and its PV the same V operands; with QB = 2 the second
// block's score MFMAs overlap the first block's softmax, and the first block's
// PV MFMAs overlap the second block's softmax, inside one wave.
template <int DT, int D, int RM, int QB, int NW = 4 / QB>
struct WaveAttn {
    static constexpr int ROT = RM & 3;                // rotation part of the mode
    static constexpr bool ALIBI = (RM & MOD_ALIBI) != 0;  // linear distance penalty
    static constexpr bool ROPE_Q = ROT != ROT_NONE;   // rotate Q rows when loading them
    static constexpr bool HALF = ROT == ROT_QK_HALF;  // half-split pairs (d, d + D/2)
    // rotate every K tile in LDS: 0 no, 1 adjacent pairs, 2 half-split pairs
    static constexpr int ROPE_K = ROT == ROT_QK ? 1 : (ROT == ROT_QK_HALF ? 2 : 0);
    // softmax() fast path, where it measured faster: D = 64, whose softmax
    // outweighs its matrix work (plain +5 %, fused +16 % at N = 8192 on
    // MI355X); at D = 128 it was within +-2 %. Not with ALiBi (scores keep
    // rising towards the diagonal, so most tiles raise the maximum and the
    // fast path's exponentials are wasted) nor the half-split K rotation.
    static constexpr bool FAST_SOFTMAX = D == 64 && !ALIBI && ROPE_K != 2;
    typedef Fmt<DT> F;
    typedef typename F::vec8 vec8;
    typedef Tile<D> T;
    typedef TileStage<DT, D, ROPE_K, NW> Stage;  // NW waves share each key tile
    static constexpr int QCH = D / 16;   // 16-deep MFMA steps over the head dim
    static constexpr int DBLK = D / 32;  // 32-row blocks of O^T

    vec8 qf[QB][QCH];
    f32x16 acc[QB][DBLK];
    f32x16 s[QB][2];    // the current tile's raw scores
    float m_run[QB];    // running max of the base-2 scaled scores (lazy)
    float l_run[QB];    // this lane half's share of the denominator
    float alpha[QB];    // rescale factor of acc still to apply (1 = none)
    u32x4 pw[QB][2][2];  // the tile's probabilities, packed as PV B operands
    float slope_raw;     // ALIBI: the head's slope in raw-score units, m * sqrt(D)

    // ALIBI: the slope of query head `head` (slopes[head] is m in the
    // penalty -m (i - j) on the scaled scores; raw scores are sqrt(D) larger).
    __device__ __forceinline__ void set_slope(const float* __restrict__ slopes, int64_t head) {
        if (ALIBI) slope_raw = slopes[head] * __builtin_sqrtf((float)D);
    }

    // Staged Q rows (block 0): this wave's 32 rows arrive in LDS through the
    // key-tile path (coalesced loads, chunk swizzle, rotation of the chunks
    // each lane loaded, with coalesced cos/sin reads), as rows 32 pw .. +31
    // of a 64-row tile at qbuf shared with the partner wave pw ^ 1; then each
    // lane reads its MFMA operands. Same rotation routines, same bits as
    // load_q(); the direct reads of load_q touch 32 table rows per load
    // instruction, which made the fused kernels' start 4-5 us slower.
    static constexpr int ROPE_QS = ROPE_Q ? (HALF ? 2 : 1) : 0;
    typedef TileStage<DT, D, ROPE_QS, 2> QStage;
    __device__ __forceinline__ void stage_q_issue(QStage& qs, uint16_t* qbuf, const TileRsrc& rs,
                                                  int pw, int lane) {
        qs.issue_k(qbuf, rs, pw, lane);
    }
    // After this wave's staging loads have completed (s_waitcnt).
    __device__ __forceinline__ void stage_q_finish(QStage& qs, uint16_t* qbuf, int pw, int lane,
                                                   int n, int hh) {
        qs.rotate(qbuf, pw, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        const int r = 32 * pw + n;
#pragma unroll
        for (int c = 0; c < QCH; ++c) {
            const int pc = (2 * c + hh) ^ kswz<D>(r);
            qf[0][c] = as_vec8<DT>(*reinterpret_cast<const u32x4*>(qbuf + r * D + 8 * pc));
        }
    }

    // Block 0's Q operands to / from LDS (lane-major per 16-deep step, so a
    // wave's 64 lanes touch 1 KiB of consecutive bytes per step).
    __device__ __forceinline__ void save_q(u32x4* dst, int lane) const {
#pragma unroll
        for (int c = 0; c < QCH; ++c) dst[c * 64 + lane] = __builtin_bit_cast(u32x4, qf[0][c]);
    }
    __device__ __forceinline__ void restore_q(const u32x4* src, int lane) {
#pragma unroll
        for (int c = 0; c < QCH; ++c) qf[0][c] = as_vec8<DT>(src[c * 64 + lane]);
    }

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
#pragma unroll
            for (int i = 0; i < DBLK; ++i)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[b][i][j] = 0.f;
            m_run[b] = -INFINITY;
            l_run[b] = 0.f;
            alpha[b] = 1.f;
        }
    }

    // Q rows q_first + 32b + n as MFMA B operands (rotated once if ROPE_Q).
    __device__ __forceinline__ void load_q(const uint16_t* qrow0, const float* __restrict__ table,
                                           int q_first, int N, int n, int hh) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            const int row = q_first + 32 * b + n;
            u32x4 w[QCH];
#pragma unroll
            for (int c = 0; c < QCH; ++c) {
                w[c] = u32x4{0u, 0u, 0u, 0u};
                if (row < N) {
                    const int d0 = 16 * c + 8 * hh;
                    w[c] = *reinterpret_cast<const u32x4*>(qrow0 + (int64_t)row * D + d0);
                    if (ROPE_Q && !HALF) {
                        const f32x4* t =
                            reinterpret_cast<const f32x4*>(table + (int64_t)row * D + d0);
                        w[c] = rope_rotate8<DT>(w[c], t[0], t[1]);
                    }
                }
            }
            if (HALF && row < N) {
                // chunk d0 of the first half pairs with chunk d0 + D/2 = step c + QCH/2
#pragma unroll
                for (int c = 0; c < QCH / 2; ++c) {
                    const int d0 = 16 * c + 8 * hh;
                    const f32x4* t =
                        reinterpret_cast<const f32x4*>(table + (int64_t)row * D + 2 * d0);
                    const f32x4 tab[4] = {t[0], t[1], t[2], t[3]};
                    u32x4 lo, hi;
                    rope_rotate_half8<DT>(w[c], w[c + QCH / 2], tab, lo, hi);
                    w[c] = lo;
                    w[c + QCH / 2] = hi;
                }
            }
#pragma unroll
            for (int c = 0; c < QCH; ++c) qf[b][c] = as_vec8<DT>(w[c]);
        }
    }

    // S^T = K Q^T for block b and both 32-key halves of the tile (raw scores).
    // Each half's MFMAs run back to back on one accumulator (a dependent
    // chain issues at full rate through accumulator forwarding). With LOADS,
    // one block of the next tile's loads follows every second MFMA of the
    // second half, so their issue overlaps matrix work.
    // The K operands are read from LDS two MFMA steps ahead of their use, and
    // the two 32-key halves form two independent accumulator chains, so a
    // single wave keeps the matrix pipe busy on its own.
    // With ALIBI the accumulators start at the penalty in raw-score units,
    // m sqrt(D) (key - row) for this lane's row and keys (key k0 + 32 kb +
    // 8 (j >> 2) + 4 hh + (j & 3) for element j), so the scores leave the
    // matrix cores with the penalty added and the softmax is unchanged.
    template <bool LOADS>
    __device__ __forceinline__ void score(int b, const uint16_t* Ks, int n, int hh, int k0,
                                          int row, Stage& stage, const NextLoads& next) {
        float base = 0.f;
        if (ALIBI) base = slope_raw * (float)(k0 + 4 * hh - row);
        __builtin_amdgcn_s_setprio(1);  // matrix phase first when waves share a SIMD
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                s[b][kb][j] = ALIBI ? __builtin_fmaf(slope_raw,
                                                     (float)(32 * kb + 8 * (j >> 2) + (j & 3)), base)
                                    : 0.f;
        constexpr int PD = 2;  // MFMA steps the operand reads run ahead
        u32x4 fk[QCH][2];
        auto read_k = [&](int c) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                fk[c][kb] = *reinterpret_cast<const u32x4*>(
                    Ks + (32 * kb + n) * D + 8 * ((2 * c + hh) ^ kswz<D>(n)));
        };
#pragma unroll
        for (int c = 0; c < PD; ++c) read_k(c);
#pragma unroll
        for (int c = 0; c < QCH; ++c) {
            if (c + PD < QCH) read_k(c + PD);
            __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                s[b][kb] = F::mfma(as_vec8<DT>(fk[c][kb]), qf[b][c], s[b][kb]);
            if (LOADS && next.active) {
                // Stage::INSTR / QCH blocks per MFMA step
                constexpr int PER = (Stage::INSTR + QCH - 1) / QCH;
#pragma unroll
                for (int j = 0; j < PER; ++j)
                    if (c * PER + j < Stage::INSTR)
                        stage.issue_part(c * PER + j, next.kbuf, next.vbuf, next.rs, next.wave,
                                         next.lane);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    }

    // Online softmax (base 2) of block b's scores: masks keys above the row
    // (MASK), raises the running maximum lazily (only when a tile exceeds it
    // by more than 2^8), records the acc rescale factor for rescale(), adds
    // the probabilities to l and packs them for pv(). The row maximum is
    // taken on raw scores (the scale is positive); the scale is folded into
    // the exponent's fused multiply-add.
    //
    // Fast path (FAST_SOFTMAX): the probabilities are first taken against the
    // current maximum. If every lane's tile sum is at most 2^7, no
    // probability exceeds 2^7, so no score is within 2^8 of raising the
    // maximum: the maximum stays, these probabilities are exactly those the
    // full path would compute, and the max tree is skipped. Otherwise (the
    // row's first tile, whose maximum is -inf, or a tile that may raise it,
    // including one whose exponentials overflow) the full path runs and
    // overwrites them. Both paths give the same bits.
    template <bool MASK>
    __device__ __forceinline__ void softmax(int b, int k0, int row, int hh, float scale_log2) {
        if (MASK) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = k0 + 32 * kb + 8 * (j >> 2) + 4 * hh + (j & 3);
                    if (key > row) s[b][kb][j] = -INFINITY;
                }
        }
        if (FAST_SOFTMAX) {
            // a row's first tile (maximum -inf) always takes the full path; the
            // stand-in 0 keeps the discarded probabilities free of NaN (this
            // file is compiled on the assumption that no NaN arises)
            const bool first = m_run[b] == -INFINITY;
            const float neg_m0 = first ? 0.f : -m_run[b];
            float qs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int t2 = 0; t2 < 4; ++t2) {
                        const float p0 = __builtin_amdgcn_exp2f(
                            __builtin_fmaf(s[b][kb][8 * e + 2 * t2], scale_log2, neg_m0));
                        const float p1 = __builtin_amdgcn_exp2f(
                            __builtin_fmaf(s[b][kb][8 * e + 2 * t2 + 1], scale_log2, neg_m0));
                        qs[t2] += p0 + p1;
                        pw[b][kb][e][t2] = F::pack2(p0, p1);
                    }
            const float tsum = (qs[0] + qs[1]) + (qs[2] + qs[3]);
            if (!__any(first || tsum > 128.f)) {
                alpha[b] = 1.f;
                l_run[b] = l_run[b] * 1.f + tsum;  // as the full path with alpha = 1
                return;
            }
        }
        // row maximum over the lane's 32 scores in 16 three-input maxima (four
        // chains of seven scores, then the chains and the last four scores),
        // then the other lane half's value (v_permlane32_swap leaves
        // {x[l], x[l^32]} in its two results)
        auto sc = [&](int i) { return s[b][i >> 4][i & 15]; };
        float m4[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float c = fmaxf(fmaxf(sc(7 * g), sc(7 * g + 1)), sc(7 * g + 2));
            c = fmaxf(fmaxf(c, sc(7 * g + 3)), sc(7 * g + 4));
            m4[g] = fmaxf(fmaxf(c, sc(7 * g + 5)), sc(7 * g + 6));
        }
        const float ma = fmaxf(fmaxf(m4[0], m4[1]), sc(28));
        const float mb = fmaxf(fmaxf(m4[2], m4[3]), sc(29));
        float mx = fmaxf(fmaxf(fmaxf(ma, mb), sc(30)), sc(31));
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                             false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
        }
        const float m_old = m_run[b];
        const float m_new = mx > m_old + LAZY_RESCALE_LOG2 ? mx : m_old;
        const float al = __builtin_amdgcn_exp2f(m_old - m_new);  // 1 when unchanged
        alpha[b] = al;
        m_run[b] = m_new;
        const float neg_m = -m_new;
        float ps[4] = {0.f, 0.f, 0.f, 0.f};  // independent partial sums (short add chains)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int t2 = 0; t2 < 4; ++t2) {
                    const float p0 = __builtin_amdgcn_exp2f(
                        __builtin_fmaf(s[b][kb][8 * e + 2 * t2], scale_log2, neg_m));
                    const float p1 = __builtin_amdgcn_exp2f(
                        __builtin_fmaf(s[b][kb][8 * e + 2 * t2 + 1], scale_log2, neg_m));
                    ps[t2] += p0 + p1;
                    pw[b][kb][e][t2] = F::pack2(p0, p1);
                }
        l_run[b] = l_run[b] * al + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
    }

    // Applies block b's pending acc rescale; skipped (wave-uniform branch)
    // when no row of the wave moved its maximum, which is most tiles.
    __device__ __forceinline__ void rescale(int b) {
        if (__any(alpha[b] != 1.f)) {
#pragma unroll
            for (int i = 0; i < DBLK; ++i)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[b][i][j] *= alpha[b];
        }
    }

    // O^T += V^T P^T for block b (V tile at Vs). The V^T operands are read two
    // MFMAs ahead of their use; the D/32 output blocks are independent chains.
    __device__ __forceinline__ void pv(int b, const uint16_t* Vs, int lane) {
        // transpose-read lane geometry (see lds_read_tr16): each 16-lane group
        // reads 4 rows x 4 elements; rows repeat every 8, so the swizzle is fixed
        const int grp = lane >> 4, j16 = lane & 15;
        const int v_lane_row = 4 * (grp >> 1) + (j16 >> 2);
        const int v_lane_c = 2 * (grp & 1) + ((j16 & 3) >> 1);
        const int v_lane_e = 4 * (j16 & 1);
        const int v_lane_sw = vswz<D>(v_lane_row);
        constexpr int NM = 4 * DBLK;  // MFMAs: key step (kb, e) major, output block i minor
        constexpr int PD = 2;         // MFMAs the operand reads run ahead
        u32x4 fv[NM];
        auto read_v = [&](int m) {
            const int kb = m / (2 * DBLK), e = (m / DBLK) & 1, i = m % DBLK;
            const uint16_t* vp = Vs + (32 * kb + 16 * e) * D;
            const int off = v_lane_row * D + 8 * ((4 * i + v_lane_c) ^ v_lane_sw) + v_lane_e;
            const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(vp + off));
            const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16(vp + 8 * D + off));
            fv[m] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int m = 0; m < PD; ++m) read_v(m);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m + PD < NM) read_v(m + PD);
            __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
            const int kb = m / (2 * DBLK), e = (m / DBLK) & 1, i = m % DBLK;
            acc[b][i] = F::mfma(as_vec8<DT>(fv[m]), as_vec8<DT>(pw[b][kb][e]), acc[b][i]);
        }
        __builtin_amdgcn_s_setprio(0);
    }

    // One key tile for all blocks: keys k0 .. k0+63, K at Ks, V at Vs;
    // q_first = the wave's first row. MASK: the tile reaches past q_first.
    template <bool MASK>
    __device__ __forceinline__ void step(const uint16_t* Ks, const uint16_t* Vs, int k0,
                                         int q_first, int n, int hh, int lane, float scale_log2,
                                         Stage& stage, const NextLoads& next) {
        if (QB == 1) {
            score<true>(0, Ks, n, hh, k0, q_first + n, stage, next);
            softmax<MASK>(0, k0, q_first + n, hh, scale_log2);
            rescale(0);
            pv(0, Vs, lane);
        } else {
            score<false>(0, Ks, n, hh, k0, q_first + n, stage, next);
            score<true>(1, Ks, n, hh, k0, q_first + 32 + n, stage, next);
            softmax<MASK>(0, k0, q_first + n, hh, scale_log2);
            rescale(0);
            pv(0, Vs, lane);
            softmax<MASK>(1, k0, q_first + 32 + n, hh, scale_log2);
            rescale(1);
            pv(1, Vs, lane);
        }
    }

    // The same tile half a step later (one 32-row block): first PV of the
    // previous tile's probabilities (V at Vprev, if `prev`), then this tile's
    // scores and softmax; its PV is left for the next call (or a final pv()).
    // A wave that runs this schedule while the other wave on its SIMD runs
    // step() does its matrix work while that wave computes its softmax, and
    // the other way round.
    template <bool MASK>
    __device__ __forceinline__ void step_lag(const uint16_t* Ks, const uint16_t* Vprev, bool prev,
                                             int k0, int q_first, int n, int hh, int lane,
                                             float scale_log2, Stage& stage,
                                             const NextLoads& next) {
        static_assert(QB == 1, "the lagged schedule takes one row block per wave");
        if (prev) pv(0, Vprev, lane);
        score<true>(0, Ks, n, hh, k0, q_first + n, stage, next);
        softmax<MASK>(0, k0, q_first + n, hh, scale_log2);
        rescale(0);
    }

    // O = acc / l and LSE = ln2 * (m + log2 l) for block b's row of this
    // lane; l_tot is the full denominator (both lane halves).
    // Output blocks i0 .. i1 - 1 only (32 head-dim columns each) with write_part.
    __device__ __forceinline__ void write(int b, uint16_t* orow, float* lse_row, float l_tot,
                                          int hh) {
        write_part(b, orow, lse_row, l_tot, hh, 0, DBLK);
    }
    __device__ __forceinline__ void write_part(int b, uint16_t* orow, float* lse_row, float l_tot,
                                               int hh, int i0, int i1) {
        const float inv = 1.f / l_tot;
#pragma unroll
        for (int i = 0; i < DBLK; ++i)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                if (i < i0 || i >= i1) continue;
                const int d0 = 32 * i + 8 * gq + 4 * hh;
                u32x2 w;
                w[0] = F::pack2(acc[b][i][4 * gq] * inv, acc[b][i][4 * gq + 1] * inv);
                w[1] = F::pack2(acc[b][i][4 * gq + 2] * inv, acc[b][i][4 * gq + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + d0) = w;
            }
        if (lse_row != nullptr && hh == 0) *lse_row = (m_run[b] + __log2f(l_tot)) * LN2;
    }
};

// Decodes a 1-D work-unit index: XCD-aware order, (b, kv head) major, then
// the per-head index, then the query head inside its GQA group.
struct Unit {
    int b, g, h, idx;  // idx = query tile slot (unpaired) or pair index
};
// hpu = query heads per unit (consecutive heads of one GQA group); h is the
// first of them.
__device__ __forceinline__ Unit decode_unit(int Hq, int Hkv, int per_head, int hpu = 1) {
    const int group = Hq / Hkv;
    const int packs = group / hpu;
    const int units = gridDim.x;
    int u = blockIdx.x;
    if (units % NXCD == 0) u = (u % NXCD) * (units / NXCD) + u / NXCD;
    Unit r;
    const int hp = u % packs;
    const int rest = u / packs;
    r.idx = rest % per_head;
    const int bg = rest / per_head;
    r.g = bg % Hkv;
    r.b = bg / Hkv;
    r.h = r.g * group + hp * hpu;
    return r;
}

// ---------------------------------------------------------------------------
// One workgroup per query tile (BM = 128 rows), heaviest first. The
// workgroup serves HG query heads of one GQA group (4 / QB waves per head),
// which all read the same key/value tiles: each tile is loaded (and, with
// RoPE, rotated) once for HG x 128 query rows.
// ---------------------------------------------------------------------------
template <int DT, int D, int RM, int QB, int HG>
__global__ __launch_bounds__(256 * HG / QB, HG == 1 ? 2 : 1) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, float* __restrict__ lse,
    const float* __restrict__ table, const float* __restrict__ slopes, int Hq, int Hkv, int N,
    int n_qtiles, float scale_log2) {
    typedef Tile<D> T;
    constexpr int WPH = 4 / QB;  // waves per head
    typedef WaveAttn<DT, D, RM, QB, WPH * HG> W;
    // With two heads, the second head's waves (which share SIMDs with the
    // first head's) run the lagged schedule; they still read the previous
    // tile's V while the next tile loads, hence three V buffers.
    constexpr bool LAG = HG == 2 && QB == 1;
    constexpr int NVB = LAG ? 3 : 2;
    // Q rows are staged through 64-row regions (one per pair of waves): the
    // second K buffer and the V buffers the first tile does not use, plus one
    // more region with two heads
    constexpr int QREG = 2 * HG;                          // staging regions needed
    constexpr int QEXTRA = QREG - 1 - (NVB - 1);          // beyond K1 and the spare V buffers
    __shared__ __attribute__((aligned(16)))
    uint16_t smem[2 * T::K_ELEMS + NVB * T::V_ELEMS + (QEXTRA > 0 ? QEXTRA : 0) * T::K_ELEMS];
    auto kbuf = [&](int t) { return smem + (t & 1) * T::K_ELEMS; };
    auto vbuf = [&](int t) { return smem + 2 * T::K_ELEMS + (t % NVB) * T::V_ELEMS; };
    auto vprev = [&](int t) { return vbuf(t + NVB - 1); };  // tile t - 1's V buffer

    const int tid = threadIdx.x;
    const int wave = tid >> 6;         // 0 .. WPH * HG - 1: every wave loads a share of each tile
    const int rwave = wave % WPH;      // row block of the wave inside its head
    const int lane = tid & 63;
    const int n = lane & 31;
    const int hh = lane >> 5;

    const Unit un = decode_unit(Hq, Hkv, n_qtiles, HG);
    const int qtile = n_qtiles - 1 - un.idx;
    const int qw0 = qtile * BM + rwave * 32 * QB;  // the wave's first row
    const int64_t q_head = ((int64_t)un.b * Hq + un.h + wave / WPH) * N;
    const int64_t kv_head = ((int64_t)un.b * Hkv + un.g) * N;
    const uint16_t* kbase = k + kv_head * D;
    const uint16_t* vbase = v + kv_head * D;

    W st;
    typename W::Stage stage;
    const int uwave = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform for the LDS bases
    if constexpr (QB == 1) {
        // region r: K1 (r = 0), then V1 .. V(NVB-1), then the extra ones
        const int r = uwave / 2;
        uint16_t* qbuf = r == 0 ? smem + T::K_ELEMS : smem + 2 * T::K_ELEMS + r * T::V_ELEMS;
        typename W::QStage qs;
        st.stage_q_issue(qs, qbuf,
                         tile_rsrc<D>(q + q_head * D, q + q_head * D, table,
                                      (qtile * BM) / BN + rwave / 2, N),
                         uwave & 1, lane);
        stage.issue(kbuf(0), vbuf(0), tile_rsrc<D>(kbase, vbase, table, 0, N), uwave, lane);
        wait_all_loads();
        st.stage_q_finish(qs, qbuf, uwave & 1, lane, n, hh);
    } else {
        st.load_q(q + q_head * D, table, qw0, N, n, hh);
        stage.issue(kbuf(0), vbuf(0), tile_rsrc<D>(kbase, vbase, table, 0, N), uwave, lane);
    }
    st.reset();
    st.set_slope(slopes, un.h + wave / WPH);

    const int n_tiles = kv_tiles_of(qtile, N);
    const int wave_tiles = qw0 < N ? (min(qw0 + 32 * QB - 1, N - 1)) / BN + 1 : 0;

    // (from the thread index, not the wave-uniform copy: as a divergent-looking
    // branch both schedules share one register allocation, which fits in 256
    // VGPRs; as a scalar branch the compiler allocates them apart and spills)
    const bool lag = LAG && wave >= WPH;
    for (int t = 0; t < n_tiles; ++t) {
        uint16_t* Ks = kbuf(t);
        wait_all_loads();              // this wave's part of tile t has landed
        stage.rotate(Ks, uwave, lane);  // RoPE on the K chunks this thread loaded
        __syncthreads();               // tile t complete; the buffers tile t+1 takes are free
        const NextLoads next{t + 1 < n_tiles, kbuf(t + 1), vbuf(t + 1),
                             tile_rsrc<D>(kbase, vbase, table, t + 1, N), uwave, lane};
        const bool mask = t * BN + BN - 1 > qw0;  // tile reaches past the wave's first row
        if (t < wave_tiles) {
            if (lag) {
                if (mask)
                    st.template step_lag<true>(Ks, vprev(t), t > 0, t * BN, qw0, n, hh, lane,
                                               scale_log2, stage, next);
                else
                    st.template step_lag<false>(Ks, vprev(t), t > 0, t * BN, qw0, n, hh, lane,
                                                scale_log2, stage, next);
            } else if (mask) {
                st.template step<true>(Ks, vbuf(t), t * BN, qw0, n, hh, lane, scale_log2, stage,
                                       next);
            } else {
                st.template step<false>(Ks, vbuf(t), t * BN, qw0, n, hh, lane, scale_log2, stage,
                                        next);
            }
        } else {
            if (lag && t == wave_tiles && t > 0) st.pv(0, vprev(t), lane);  // pending PV
            if (next.active) stage.issue(next.kbuf, next.vbuf, next.rs, uwave, lane);
        }
    }
    if (lag && wave_tiles == n_tiles && n_tiles > 0) st.pv(0, vbuf(n_tiles - 1), lane);
    if (wave_tiles == 0) return;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const int row = qw0 + 32 * b + n;
        const float l_tot = st.l_run[b] + __shfl_xor(st.l_run[b], 32);
        if (row < N)
            st.write(b, out + (q_head + row) * D, lse ? lse + q_head + row : nullptr, l_tot, hh);
    }
}

// ---------------------------------------------------------------------------
// Paired query tiles of two GQA heads: one 8-wave workgroup takes the 64-row
// query tiles T-1-p (heavy) and p (light) of two query heads of one GQA
// group. Waves 0-3 hold the heavy tile's rows (2 waves per head), waves 4-7
// the light tile's, so each SIMD (waves w and w + 4) runs one heavy and one
// light wave and every workgroup does the same work. All four row blocks read
// the same key/value tiles: each tile is loaded (and, with RoPE, rotated)
// once for 256 query rows while the light rows are still active, and the
// causal imbalance needs no merge of partial results.
// ---------------------------------------------------------------------------
template <int DT, int D, int RM>
__global__ __launch_bounds__(512, 1) void attn_pair_heads_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, float* __restrict__ lse,
    const float* __restrict__ table, const float* __restrict__ slopes, int Hq, int Hkv, int N,
    int n_tiles64, int n_pairs, float scale_log2) {
    typedef Tile<D> T;
    typedef WaveAttn<DT, D, RM, 1, 8> W;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::BUF_ELEMS];
    auto kbuf = [&](int t) { return smem + (t & 1) * T::BUF_ELEMS; };
    auto vbuf = [&](int t) { return smem + (t & 1) * T::BUF_ELEMS + T::K_ELEMS; };

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 31;
    const int hh = lane >> 5;

    const Unit un = decode_unit(Hq, Hkv, n_pairs, 2);
    const int t_heavy = n_tiles64 - 1 - un.idx;
    const int t_light = un.idx < t_heavy ? un.idx : -1;  // none for the middle tile of an odd count
    const int tile = wave < 4 ? t_heavy : t_light;
    const int qw0 = tile * 64 + 32 * (wave & 1);  // the wave's first row
    const int64_t q_head = ((int64_t)un.b * Hq + un.h + ((wave >> 1) & 1)) * N;
    const int64_t kv_head = ((int64_t)un.b * Hkv + un.g) * N;
    const uint16_t* kbase = k + kv_head * D;
    const uint16_t* vbase = v + kv_head * D;

    W st;
    const bool has_rows = tile >= 0 && qw0 < N;
    if (has_rows) st.load_q(q + q_head * D, table, qw0, N, n, hh);
    st.reset();
    st.set_slope(slopes, un.h + ((wave >> 1) & 1));

    const int n_tiles = (min(t_heavy * 64 + 64, N) - 1) / BN + 1;
    const int wave_tiles = has_rows ? (min(qw0 + 31, N - 1)) / BN + 1 : 0;

    typename W::Stage stage;
    const int uwave = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform for the LDS bases
    stage.issue(kbuf(0), vbuf(0), tile_rsrc<D>(kbase, vbase, table, 0, N), uwave, lane);
    for (int t = 0; t < n_tiles; ++t) {
        uint16_t* Ks = kbuf(t);
        wait_all_loads();              // this wave's part of tile t has landed
        stage.rotate(Ks, uwave, lane);  // RoPE on the K chunks this thread loaded
        __syncthreads();               // tile t complete; the other buffer is no longer read
        const NextLoads next{t + 1 < n_tiles, kbuf(t + 1), vbuf(t + 1),
                             tile_rsrc<D>(kbase, vbase, table, t + 1, N), uwave, lane};
        if (t < wave_tiles) {
            if (t * BN + BN - 1 > qw0)  // tile reaches past the wave's first row
                st.template step<true>(Ks, vbuf(t), t * BN, qw0, n, hh, lane, scale_log2, stage,
                                       next);
            else
                st.template step<false>(Ks, vbuf(t), t * BN, qw0, n, hh, lane, scale_log2, stage,
                                        next);
        } else if (next.active) {
            stage.issue(next.kbuf, next.vbuf, next.rs, uwave, lane);
        }
    }
    if (wave_tiles == 0) return;
    const int row = qw0 + n;
    const float l_tot = st.l_run[0] + __shfl_xor(st.l_run[0], 32);
    if (row < N) st.write(0, out + (q_head + row) * D, lse ? lse + q_head + row : nullptr, l_tot, hh);
}

// ---------------------------------------------------------------------------
// Paired, split, load-balanced launch: two halves of 4 / QB waves each.
// ---------------------------------------------------------------------------
template <int DT, int D, int RM, int QB>
__global__ __launch_bounds__(512 / QB, 1) void attn_pair_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, float* __restrict__ lse,
    const float* __restrict__ table, const float* __restrict__ slopes, int Hq, int Hkv, int N,
    int n_qtiles, int n_pairs, float scale_log2) {
    typedef Tile<D> T;
    typedef WaveAttn<DT, D, RM, QB> W;
    constexpr int HT = 256 / QB;  // threads per half
    // per half: K0 K1 V0 V1; after the loop the same memory holds the merge
    // data. (Running half B on the lagged schedule of the tile launch was
    // measured 2.5 % slower here, so both halves run step().)
    // At step i < len_l both halves need key tile i (half A for the heavy
    // rows, half B for the light rows): half A alone loads (and with RoPE
    // rotates) it and half B reads half A's copy, so those steps cost one tile
    // load and rotation instead of two.
    constexpr int H_ELEMS = 2 * T::K_ELEMS + 2 * T::V_ELEMS;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * H_ELEMS];
    // With RoPE on Q: half A's rotated Q operands of the heavy rows, which
    // half B takes over when it moves to those rows instead of loading and
    // rotating them again (3-4 % faster fused at N = 2048 on MI355X; for
    // unrotated Q the copy cost more in the prologue than the reload it saved)
    constexpr bool QCOPY = W::ROPE_Q;
    static_assert(QB == 1, "the Q copy holds one row block per wave");
    __shared__ __attribute__((aligned(16))) u32x4 qcopy[QCOPY ? 4 * W::QCH * 64 : 1];

    const int tid = threadIdx.x;
    // wave-uniform by construction; readfirstlane lets the compiler see it,
    // so the tile descriptors stay scalar
    const int half = __builtin_amdgcn_readfirstlane(tid / HT);  // 0 = A, 1 = B
    const int htid = tid % HT;       // thread index inside the half
    const int wave = htid >> 6;      // wave inside the half
    const int lane = tid & 63;
    const int n = lane & 31;
    const int hh = lane >> 5;
    const Unit un = decode_unit(Hq, Hkv, n_pairs);
    const int p = un.idx;
    const int t_heavy = n_qtiles - 1 - p;
    const int t_light = p;                     // == t_heavy for the middle tile of an odd count
    const int len_h = kv_tiles_of(t_heavy, N);
    const int len_l = t_light < t_heavy ? kv_tiles_of(t_light, N) : 0;
    const int split = (len_l + len_h + 1) / 2;  // heavy key tiles [0, split) go to half A
    const int steps = split;                     // half B needs len_l + len_h - split <= split

    const int64_t q_head = ((int64_t)un.b * Hq + un.h) * N;
    const int64_t kv_head = ((int64_t)un.b * Hkv + un.g) * N;
    const uint16_t* qhead = q + q_head * D;
    const uint16_t* kbase = k + kv_head * D;
    const uint16_t* vbase = v + kv_head * D;

    // job of this half at step i: the key tile (or -1 for none) and its query tile
    auto job_tile = [&](int i, int& qt) -> int {
        if (half == 0) {
            qt = t_heavy;
            return i < split ? i : -1;
        }
        if (i < len_l) {
            qt = t_light;
            return i;
        }
        qt = t_heavy;
        const int j = split + (i - len_l);
        return j < len_h ? j : -1;
    };

    W st;
    st.reset();
    st.set_slope(slopes, un.h);
    int cur_qt = -1;   // query tile whose rows this wave holds
    int qw0 = 0, wave_tiles = 0;

    uint16_t* hbuf = smem + half * H_ELEMS;
    auto kbuf = [&](int i) { return hbuf + (i & 1) * T::K_ELEMS; };
    auto vbuf = [&](int i) { return hbuf + 2 * T::K_ELEMS + (i & 1) * T::V_ELEMS; };
    typename W::Stage stage;
    const int uwave = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform for the LDS bases
    {
        // the first rows' Q loads go out together with the first tile's
        int qt;
        const int kt = job_tile(0, qt);
        if (kt >= 0) {
            cur_qt = qt;
            qw0 = qt * BM + wave * 32 * QB;
            wave_tiles = qw0 < N ? (min(qw0 + 32 * QB - 1, N - 1)) / BN + 1 : 0;
            // Q rows staged in the half's second K (waves 0, 1) or V (2, 3)
            // buffer, free until the first step issues the next tile
            uint16_t* qbuf = uwave < 2 ? hbuf + T::K_ELEMS
                                       : hbuf + 2 * T::K_ELEMS + T::V_ELEMS;
            typename W::QStage qs;
            st.stage_q_issue(qs, qbuf, tile_rsrc<D>(qhead, qhead, table, (qt * BM) / BN + uwave / 2, N),
                             uwave & 1, lane);
            if (!(half == 1 && len_l > 0))  // a shared first tile comes from half A
                stage.issue(kbuf(0), vbuf(0), tile_rsrc<D>(kbase, vbase, table, kt, N), uwave,
                            lane);
            wait_all_loads();
            st.stage_q_finish(qs, qbuf, uwave & 1, lane, n, hh);
            if (QCOPY && half == 0) st.save_q(qcopy + uwave * W::QCH * 64, lane);
        }
    }
    for (int i = 0; i < steps; ++i) {
        int qt;
        const int kt = job_tile(i, qt);
        const bool shared = half == 1 && i < len_l;  // key tile i from half A's buffers
        uint16_t* Ks = shared ? smem + (i & 1) * T::K_ELEMS : kbuf(i);
        uint16_t* Vs = shared ? smem + 2 * T::K_ELEMS + (i & 1) * T::V_ELEMS : vbuf(i);
        wait_all_loads();  // this wave's part of the half's tile i has landed
        if (kt >= 0 && !shared) stage.rotate(Ks, uwave, lane);
        if (kt >= 0 && qt != cur_qt) {
            // new rows: only half B changes rows, from the light rows (its first
            // job) to the heavy rows, whose rotated Q operands half A left in
            // LDS before the first barrier; unrotated ones are loaded again, the
            // loads going out before the old rows' write
            const int qw_new = qt * BM + wave * 32 * QB;
            if (QCOPY)
                st.restore_q(qcopy + uwave * W::QCH * 64, lane);
            else
                st.load_q(qhead, table, qw_new, N, n, hh);
            if (cur_qt >= 0 && wave_tiles > 0) {
#pragma unroll
                for (int b = 0; b < QB; ++b) {
                    const int row = qw0 + 32 * b + n;
                    const float l_tot = st.l_run[b] + __shfl_xor(st.l_run[b], 32);
                    if (row < N)
                        st.write(b, out + (q_head + row) * D, lse ? lse + q_head + row : nullptr,
                                 l_tot, hh);
                }
            }
            cur_qt = qt;
            qw0 = qw_new;
            wave_tiles = qw0 < N ? (min(qw0 + 32 * QB - 1, N - 1)) / BN + 1 : 0;
            st.reset();
        }
        __syncthreads();  // tile i complete in both halves; the buffers of tile i+1 are free
        int qt1;
        const int kt1 = job_tile(i + 1, qt1);
        const bool next_shared = half == 1 && i + 1 < len_l;  // half A loads it
        const NextLoads next{i + 1 < steps && kt1 >= 0 && !next_shared, kbuf(i + 1), vbuf(i + 1),
                             tile_rsrc<D>(kbase, vbase, table, kt1 < 0 ? 0 : kt1, N), uwave, lane};
        if (kt >= 0 && kt < wave_tiles) {
            if (kt * BN + BN - 1 > qw0)  // tile reaches past the wave's first row
                st.template step<true>(Ks, Vs, kt * BN, qw0, n, hh, lane, scale_log2, stage,
                                       next);
            else
                st.template step<false>(Ks, Vs, kt * BN, qw0, n, hh, lane, scale_log2, stage,
                                        next);
        } else if (next.active) {
            stage.issue(next.kbuf, next.vbuf, next.rs, uwave, lane);
        }
    }

    // half B: if its last rows were the light ones, they are complete now
    if (half == 1 && cur_qt == t_light && t_light != t_heavy) {
        if (wave_tiles > 0) {
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                const int row = qw0 + 32 * b + n;
                const float l_tot = st.l_run[b] + __shfl_xor(st.l_run[b], 32);
                if (row < N)
                    st.write(b, out + (q_head + row) * D, lse ? lse + q_head + row : nullptr, l_tot,
                             hh);
            }
        }
        st.reset();  // no share of the heavy rows
    }

    // ---- merge the two halves' partial states of the heavy rows ----
    // Each half merges and writes half of the output columns: half A blocks
    // 0 .. DBLK/2 - 1, half B the rest. Each exports to LDS the blocks the
    // other merges, with its running max and denominator; both evaluate the
    // same expression, A's state * a_a + B's state * a_b.
    __syncthreads();  // every wave is done with the tile buffers
    constexpr int HB = W::DBLK / 2;     // output blocks per half
    constexpr int SLOTS = 16 * HB + 2;  // [half][wave][slot][lane]
    float* xch = reinterpret_cast<float*>(smem);
    float* mine = xch + ((half * 4 + wave) * SLOTS) * 64 + lane;
    const float* other = xch + (((1 - half) * 4 + wave) * SLOTS) * 64 + lane;
    const int own0 = half == 0 ? 0 : HB;  // first block this half merges
    const float l_half = st.l_run[0] + __shfl_xor(st.l_run[0], 32);
#pragma unroll
    for (int i = 0; i < W::DBLK; ++i) {
        if (i >= own0 && i < own0 + HB) continue;  // kept: exported are the other's blocks
#pragma unroll
        for (int j = 0; j < 16; ++j) mine[(16 * (i % HB) + j) * 64] = st.acc[0][i][j];
    }
    mine[(16 * HB) * 64] = st.m_run[0];
    mine[(16 * HB + 1) * 64] = l_half;
    __syncthreads();
    const int hq = t_heavy * BM + wave * 32 + n;  // this lane's heavy row
    if (hq >= N) return;
    const float m_o = other[(16 * HB) * 64];
    const float l_o = other[(16 * HB + 1) * 64];
    const float m_a = half == 0 ? st.m_run[0] : m_o, l_a = half == 0 ? l_half : l_o;
    const float m_b = half == 0 ? m_o : st.m_run[0], l_b = half == 0 ? l_o : l_half;
    const float m = fmaxf(m_a, m_b);
    const float a_a = __builtin_amdgcn_exp2f(m_a - m);
    const float a_b = l_b > 0.f ? __builtin_amdgcn_exp2f(m_b - m) : 0.f;
#pragma unroll
    for (int i = 0; i < W::DBLK; ++i) {
        if (i < own0 || i >= own0 + HB) continue;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float x = other[(16 * (i % HB) + j) * 64];
            st.acc[0][i][j] = half == 0 ? st.acc[0][i][j] * a_a + x * a_b
                                        : x * a_a + st.acc[0][i][j] * a_b;
        }
    }
    st.m_run[0] = m;
    const float l_tot = l_a * a_a + l_b * a_b;
    st.write_part(0, out + (q_head + hq) * D, half == 0 && lse ? lse + q_head + hq : nullptr,
                  l_tot, hh, own0, own0 + HB);
}

// Rows per wave: 32 x QB. One 64-row wave per SIMD (QB = 2) uses the full
// register file and overlaps one block's softmax with the other's MFMAs.
template <int D>
constexpr int qb_for() { return 1; }

template <int DT, int D, int RM>
static hipError_t launch_typed(const AttnArgs& a, hipStream_t stream) {
    constexpr int QB = qb_for<D>();
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const int n_qtiles = (a.N + BM - 1) / BM;
    const int n_pairs = (n_qtiles + 1) / 2;
    const int64_t pair_units = (int64_t)n_pairs * a.Hq * a.B;
    const int64_t tile_units = (int64_t)n_qtiles * a.Hq * a.B;
    if (tile_units > 0x7fffffff) return hipErrorInvalidConfiguration;
    // The pair launch balances the causal work inside each workgroup but runs
    // one 8-wave workgroup per CU, so it pays while its workgroups fill at
    // most one round of the CUs; beyond, the heaviest-first tile launch
    // balances as well (and, with two heads per workgroup, shares each key
    // tile among 256 query rows). Without the two-head tile launch (MHA, odd
    // GQA groups) the pair launch also wins at exactly two full rounds.
    // Measured on MI355X: D = 64 MHA at N = 8192 (two rounds) pair 3-9 %
    // faster; at N = 6144 (1.5 rounds) the tile launch 12-14 % faster; from
    // N = 16384, and for GQA from B * N = 4096, the tile launch faster.
    // Below half a round the pair launch still wins once a head has enough
    // query tiles for its shorter critical path (n_qtiles + 1 steps against
    // the heaviest tile's 2 n_qtiles) to outweigh its merge: from 4 tiles
    // against the two-head tile launch, from 12 against one head per 4-wave
    // workgroup (MHA). With one head per tile workgroup the pair launch
    // also wins at 1.5-2 rounds at D = 128. Measured on MI355X (fused,
    // plain and Q-rotating kernels alike): GQA 8/2 D = 128 N = 1024-2048
    // pair 17-28 % faster, GQA 32/8 N = 512-768 3-15 %, MHA 16/16 D = 64
    // N = 1536-1792 1-10 % but N = 768-1024 0-12 % slower, MHA 32/32
    // D = 128 N = 3072-3840 2-17 % faster, while at D = 64 N = 5120-7168
    // (1.25-1.75 rounds) the tile launch stays 3-22 % faster.
    const bool heads_ok = (a.Hq / a.Hkv) % 2 == 0;
    const int min_tiles = heads_ok ? 4 : 12;
    bool pair = n_qtiles >= 2 && pair_units <= NUM_CUS &&
                (pair_units >= NUM_CUS / 2 || n_qtiles >= min_tiles);
    if (!heads_ok && n_qtiles >= 2 &&
        (pair_units == 2 * NUM_CUS ||
         (D == 128 && pair_units >= 3 * NUM_CUS / 2 && pair_units <= 2 * NUM_CUS)))
        pair = true;
    // pair_heads (two GQA heads sharing every key tile) only when forced: on
    // the Llama-3-8B GQA shape (Hq = 32, Hkv = 8, D = 128, bf16) it measured
    // 4-17 % slower than the pair launch at N = 1024-3072 and B = 1-2 for
    // every rotation mode (fused 60.8 vs 56.0 us at N = 2048), and level at
    // B = 4, N = 1024. Keeping one automatic choice for all rotation modes
    // also makes every path run the same attention arithmetic on the same
    // rotated operands, so the paths agree bit for bit.
    bool pair_heads = false;
    if (a.shape == ATTN_SHAPE_PAIR) pair = true;
    if (a.shape == ATTN_SHAPE_TILE) pair = false, pair_heads = false;
    if (a.shape == ATTN_SHAPE_PAIR_HEADS && heads_ok) pair = false, pair_heads = true;
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
    const uint16_t* k = static_cast<const uint16_t*>(a.k);
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    uint16_t* out = static_cast<uint16_t*>(a.out);
    if (pair_heads) {
        const int n_t64 = (a.N + 63) / 64;
        const int n_pairs64 = (n_t64 + 1) / 2;
        const int64_t units = (int64_t)n_pairs64 * (a.Hq / 2) * a.B;
        return launch_kernel(attn_pair_heads_kernel<DT, D, RM>, dim3((unsigned)units), dim3(512),
                             stream, q, k, v, out, a.lse, a.table, a.slopes, a.Hq, a.Hkv, a.N,
                             n_t64, n_pairs64, scale_log2);
    }
    if (pair)
        return launch_kernel(attn_pair_kernel<DT, D, RM, QB>, dim3((unsigned)pair_units),
                             dim3(512 / QB), stream, q, k, v, out, a.lse, a.table, a.slopes, a.Hq,
                             a.Hkv, a.N, n_qtiles, n_pairs, scale_log2);
    if ((a.Hq / a.Hkv) % 2 == 0)  // GQA: two query heads of a group share every key tile
        return launch_kernel(attn_fwd_kernel<DT, D, RM, QB, 2>, dim3((unsigned)(tile_units / 2)),
                             dim3(512 / QB), stream, q, k, v, out, a.lse, a.table, a.slopes, a.Hq,
                             a.Hkv, a.N, n_qtiles, scale_log2);
    return launch_kernel(attn_fwd_kernel<DT, D, RM, QB, 1>, dim3((unsigned)tile_units),
                         dim3(256 / QB), stream, q, k, v, out, a.lse, a.table, a.slopes, a.Hq,
                         a.Hkv, a.N, n_qtiles, scale_log2);
}

// One (dtype, head dim, mode) per object file: the build compiles this file
// once per combination with RAC_FWD_DT / RAC_FWD_D / RAC_FWD_MODE defined
// (the kernels are large; the parts compile in parallel), and once without
// them for the dispatcher below, which only declares the parts.
template <int DT, int D, int RM>
hipError_t launch_part(const AttnArgs& a, hipStream_t stream);

#ifdef RAC_FWD_MODE
template <int DT, int D, int RM>
hipError_t launch_part(const AttnArgs& a, hipStream_t stream) {
    return launch_typed<DT, D, RM>(a, stream);
}
template hipError_t launch_part<RAC_FWD_DT, RAC_FWD_D, RAC_FWD_MODE>(const AttnArgs&, hipStream_t);
#else
template <int DT, int RM>
static hipError_t launch_dt(const AttnArgs& a, hipStream_t stream) {
    return a.D == 64 ? launch_part<DT, 64, RM>(a, stream) : launch_part<DT, 128, RM>(a, stream);
}

template <int DT>
static hipError_t launch_rot(const AttnArgs& a, int rot, hipStream_t stream) {
    if (a.slopes != nullptr) {  // ALiBi: with RoPE on Q and K (either pairing) or none
        if (rot == ROT_QK)
            return a.half_pairs ? launch_dt<DT, ROT_QK_HALF | MOD_ALIBI>(a, stream)
                                : launch_dt<DT, ROT_QK | MOD_ALIBI>(a, stream);
        if (rot == ROT_NONE) return launch_dt<DT, ROT_NONE | MOD_ALIBI>(a, stream);
        return hipErrorInvalidValue;
    }
    if (rot == ROT_QK) return a.half_pairs ? launch_dt<DT, ROT_QK_HALF>(a, stream)
                                           : launch_dt<DT, ROT_QK>(a, stream);
    if (rot == ROT_Q) return launch_dt<DT, ROT_Q>(a, stream);
    return launch_dt<DT, ROT_NONE>(a, stream);
}

hipError_t launch_attn_fwd(const AttnArgs& a, int rot, hipStream_t stream) {
    return a.dtype == DT_BF16 ? launch_rot<DT_BF16>(a, rot, stream)
                              : launch_rot<DT_FP16>(a, rot, stream);
}
#endif

}  // namespace rac
