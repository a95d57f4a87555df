/*
 * rac.h -- RoPE + causal attention forward on AMD MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels: the forward operations of the
 * fused, pre-rotation and GQA split paths, a dispatcher, the backward of the
 * fused and pre-rotation paths, a second RoPE pairing and the ALiBi score
 * modification:
 *
 *   attn_rope_causal_fwd  one kernel: rotary position embedding applied to the
 *                         query and key tiles inside a causal attention
 *                         forward ("in-kernel rotation").
 *   rope_prerotate        a separate streaming pass writing rotated copies of
 *                         Q and K ("pre-rotation").
 *   attn_causal_fwd       causal attention forward on already-rotated inputs;
 *                         with rope_prerotate it forms the pre-rotation path.
 *   rope_prerotate_k      the pre-rotation pass on K alone, and
 *   attn_rope_q_causal_fwd  causal attention that rotates Q in the kernel (once
 *                         per query row) and takes K already rotated: together
 *                         the "GQA split" path, which moves only the Hkv key
 *                         heads through the streaming pass instead of all
 *                         Hq + Hkv heads and rotates no key tile in the kernel.
 *   attn_rope_causal_bwd, attn_causal_bwd, rope_prerotate_bwd
 *                         the gradients of the fused and pre-rotation paths.
 *   attn_rope_causal_auto the same result as attn_rope_causal_fwd through
 *                         whichever of the three paths is fastest for the
 *                         shape on MI355X (the report's paragraph 5: the
 *                         choice is measured per architecture and shape).
 *   rope_prerotate_ex, attn_rope_causal_fwd_ex, attn_rope_causal_bwd_ex,
 *   rope_prerotate_bwd_ex the pass, the fused kernel and their gradients with
 *                         the half-split RoPE pairing (i, i + D/2) as an
 *                         alternative.
 *   attn_alibi_causal_fwd, attn_alibi_causal_bwd
 *                         causal attention with the ALiBi distance penalty
 *                         after the QK product, alone or with fused RoPE, and
 *                         its gradients.
 *
 * The two paths and the choice between them are the subject of "AttnFuse Makes
 * RoPE a First-Class Attention Compilation Operation" (tdteach paper-news,
 * 2026-09-13), paragraphs 3 and 4, and of the AttnFuse abstract (arxivdaily
 * 2609.13612): pre-rotation costs memory bandwidth, in-kernel rotation costs
 * compute and tiling, and which wins depends on the GPU and the shape.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are contiguous row-major [B, H, N, D]: batch, head, token, head dim.
 *   q, out          [B, Hq,  N, D]
 *   k, v            [B, Hkv, N, D]
 *   lse             [B, Hq,  N]     fp32
 * Every tensor pointer is a DEVICE pointer on the current HIP device, owned by
 * the caller, who keeps it alive until the enqueued work completes. Element
 * type is `dtype` (RAC_BF16 or RAC_FP16) for q, k, v, out, q_rot and k_rot.
 * Pointers must be 16-byte aligned.
 *
 * RoPE (rotary position embedding; "Fast and Exact Relative-Position Attention
 * via Structure-Aware Kernels", rainbus digest, background "RoPE and
 * parameter-free position encodings": each query and key is rotated by an
 * angle set by its absolute position). Readings where the pages are silent:
 * token n of every (b, h) sits at position n; coordinates (2i, 2i+1) form a
 * pair turned counter-clockwise by n * theta_i, theta_i = rope_base^(-2i/D);
 * values are not rotated. Angles and their cos/sin are formed in fp64 on the
 * host, stored as fp32, and the rotation runs in fp32 on the device, rounded
 * once to `dtype` (round to nearest even). Both paths feed the same rotated
 * operands to the matrix cores.
 *
 * Causal attention (same digest, "FlashAttention and online softmax" and its
 * forward Algorithm 1; MHA/GQA per the AttnFuse report, paragraph 4): query
 * head h reads key/value head h / (Hq / Hkv); query n attends to keys j <= n;
 * scores are scaled by 1/sqrt(D); softmax statistics are kept in fp32 with a
 * base-2 exponent; out = softmax(scores) V rounded to `dtype`;
 * lse[n] = natural log of sum_j exp(score_nj), fp32.
 *
 * Supported: D in {64, 128}; Hq % Hkv == 0; 1 <= Hq, Hkv <= 65535;
 * 0 <= B <= 65535; 0 <= N <= RAC_MAX_N. B == 0 or N == 0 is a no-op that
 * returns RAC_OK without touching any pointer.
 *
 * Errors: arguments are validated before anything is enqueued; a non-zero
 * return means nothing was launched, and rac_last_error() gives the reason
 * (per calling thread). Calls enqueue on `stream` (NULL = the null stream)
 * and return without synchronising; a fault inside a kernel surfaces at the
 * caller's next synchronisation. No C++ exception crosses this boundary.
 *
 * Launch shape: the attention kernels pick between a load-balanced launch
 * that pairs light and heavy causal query tiles in one workgroup and one
 * workgroup per query tile, by problem size. The environment variable
 * RAC_ATTN_SHAPE=pair|tile|pairheads forces one of them (results are
 * identical up to floating-point summation order); any other value, or none,
 * means automatic. Likewise RAC_BWD_SHAPE=k128|k64|k64x2 forces the backward
 * key-parallel pass's workgroup shape (128 keys, 64 keys, or 64 keys with two
 * query groups).
 *
 * Library-owned memory: the cos/sin table for each (device, D, rope_base),
 * fp32 [capacity, D], grown on demand. The first call that needs a new or
 * larger table allocates it and uploads it synchronously (so warm up before
 * timing). rac_release_tables() frees every table.
 */
#ifndef RAC_H
#define RAC_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { RAC_BF16 = 0, RAC_FP16 = 1 };

enum {
    RAC_OK = 0,
    RAC_ERR_ARG = -1,          /* bad size, null pointer, overlap, bad rope_base or dtype */
    RAC_ERR_ALIGN = -2,        /* a pointer is not 16-byte aligned */
    RAC_ERR_UNSUPPORTED = -3,  /* valid but not implemented: D not in {64, 128} */
    RAC_ERR_HIP = -4           /* a HIP runtime call failed (no device, out of memory, launch) */
};

#define RAC_MAX_N (1 << 22)

/*
 * Fused path: one kernel applies RoPE to each query tile once and to every key
 * tile it visits, then runs causal attention on the rotated operands.
 * q, k, v: inputs as above (not rotated). out: [B,Hq,N,D], must not overlap
 * q, k or v. lse: [B,Hq,N] fp32, or NULL to skip it. rope_base > 0, finite.
 */
int attn_rope_causal_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                         int B, int Hq, int Hkv, int N, int D, double rope_base,
                         int dtype, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * attn_rope_causal_fwd with its cos/sin table, the one buffer that call's
 * kernel reads beyond its inputs and outputs, in a library-owned static
 * device array of RAC_NOALLOC_MAX_N * 128 fp32 values (16 MiB, held on every
 * GPU the library runs on until the process ends) instead of the table cache,
 * which allocates. Each call rebuilds the N rows it needs on `stream` (one
 * small kernel; the angles in fp64 as for the cache) and then runs the fused
 * kernel: it calls no hipMalloc, hipFree or other allocating routine and no
 * synchronous copy. Same arguments, results (to rounding of the table's fp64
 * sines and cosines) and rules as attn_rope_causal_fwd, and additionally
 * N * D <= RAC_NOALLOC_MAX_N * 128 (N <= 32768 at D = 128, 65536 at D = 64),
 * else RAC_ERR_ARG. Every call on a GPU uses that GPU's one array: calls that
 * overlap on one GPU (different streams, or threads) race and must not be
 * issued; calls on one stream are ordered.
 */
#define RAC_NOALLOC_MAX_N 32768
int attn_rope_causal_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                                 float* lse, int B, int Hq, int Hkv, int N, int D,
                                 double rope_base, int dtype, void* stream);

/*
 * Pre-rotation pass: q_rot = RoPE(q), k_rot = RoPE(k), each element rounded
 * once to `dtype`. Memory-bound streaming kernel. q_rot may equal q and k_rot
 * may equal k (in place); any other overlap between the four buffers is an
 * error.
 */
int rope_prerotate(const void* q, const void* k, void* q_rot, void* k_rot,
                   int B, int Hq, int Hkv, int N, int D, double rope_base,
                   int dtype, void* stream);

/*
 * Causal attention forward on inputs that already carry their rotation (for
 * example the output of rope_prerotate). Same layouts and rules as
 * attn_rope_causal_fwd, without rope_base.
 */
int attn_causal_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                    int B, int Hq, int Hkv, int N, int D,
                    int dtype, void* stream);

/*
 * GQA split path, first half: k_rot = RoPE(k), each element rounded once to
 * `dtype` -- exactly the k_rot that rope_prerotate writes. k, k_rot:
 * [B,Hkv,N,D]; k_rot may equal k (in place), any other overlap is an error.
 * B*Hkv <= 524280. Not a method step of its own on the pages: it splits the
 * cost model of the AttnFuse report (paragraph 3) between its two terms, the
 * bandwidth cost paid for K only and the in-kernel cost for Q only.
 */
int rope_prerotate_k(const void* k, void* k_rot, int B, int Hkv, int N, int D,
                     double rope_base, int dtype, void* stream);

/*
 * GQA split path, second half: causal attention with RoPE applied to each
 * query row inside the kernel (as attn_rope_causal_fwd does) and keys taken
 * already rotated (k_rot, e.g. from rope_prerotate_k). With k_rot =
 * rope_prerotate_k(k) the result is bit-identical to attn_rope_causal_fwd.
 * Same layouts and rules as attn_rope_causal_fwd.
 */
int attn_rope_q_causal_fwd(const void* q, const void* k_rot, const void* v, void* out,
                           float* lse, int B, int Hq, int Hkv, int N, int D,
                           double rope_base, int dtype, void* stream);

enum { RAC_PAIR_ADJACENT = 0, RAC_PAIR_HALF = 1, RAC_ROPE_NONE = 2 };

/*
 * RoPE with a choice of which coordinates turn together (`pairing`):
 *   RAC_PAIR_ADJACENT  (2i, 2i+1), the pairing of every other entry point;
 *   RAC_PAIR_HALF      (i, i + D/2), the "rotate half" layout;
 * both with pair i turned by n * theta_i, theta_i = rope_base^(-2i/D),
 * 0 <= i < D/2, and the same fp32 arithmetic and rounding. The background on
 * RoPE in "Fast and Exact Relative-Position Attention via Structure-Aware
 * Kernels" (rainbus digest) fixes the rotation by absolute position but not
 * the pairing; the two give different results for the same inputs, so both
 * are offered.
 *
 * rope_prerotate_ex and attn_rope_causal_fwd_ex are rope_prerotate and
 * attn_rope_causal_fwd with that argument; with RAC_PAIR_ADJACENT they give
 * exactly those functions' results. For either pairing,
 * attn_causal_fwd(rope_prerotate_ex(q, k)) equals attn_rope_causal_fwd_ex
 * bit for bit. Any other value of `pairing` (RAC_ROPE_NONE included) is
 * RAC_ERR_ARG. Same layouts, limits and rules as the functions they extend.
 */
int rope_prerotate_ex(const void* q, const void* k, void* q_rot, void* k_rot,
                      int B, int Hq, int Hkv, int N, int D, double rope_base,
                      int pairing, int dtype, void* stream);
int attn_rope_causal_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                            int B, int Hq, int Hkv, int N, int D, double rope_base,
                            int pairing, int dtype, void* stream);

/*
 * Causal attention with the ALiBi distance penalty, a score modification
 * applied after the QK product: the score of key j for query i of query head
 * h is
 *     q_i . k_j / sqrt(D) - slopes[h] * (i - j)
 * ("Fast and Exact Relative-Position Attention via Structure-Aware Kernels",
 * rainbus digest, background "RoPE and parameter-free position encodings":
 * ALiBi penalises attention linearly with distance), then the same causal
 * softmax, out and lse as attn_causal_fwd. The penalty enters the score
 * accumulators before the product, in fp32.
 *
 * slopes: DEVICE pointer to Hq fp32 values, one per query head, finite (the
 *   ALiBi method's own choice is the geometric sequence 2^(-8(h+1)/Hq));
 *   4-byte aligned; must not overlap out or lse.
 * pairing: RAC_ROPE_NONE for no rotation (rope_base is then ignored), or
 *   RAC_PAIR_ADJACENT / RAC_PAIR_HALF to rotate q and k in the kernel as
 *   attn_rope_causal_fwd_ex does, composing RoPE (before the product) with
 *   ALiBi (after it).
 * With every slope zero the results equal attn_causal_fwd (RAC_ROPE_NONE) or
 * attn_rope_causal_fwd_ex (a RoPE pairing) bit for bit. Same layouts, limits
 * and rules as attn_rope_causal_fwd.
 */
int attn_alibi_causal_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int Hq, int Hkv, int N, int D, const float* slopes,
                          double rope_base, int pairing, int dtype, void* stream);

enum { RAC_PATH_FUSED = 0, RAC_PATH_PREROTATE = 1, RAC_PATH_SPLIT = 2 };

/*
 * Dispatcher: out/lse of attn_rope_causal_fwd (bit-identical: every path hands
 * the same rotated operands to the same attention arithmetic), computed by the
 * path with the least modelled time on MI355X for this shape. The model costs
 * the streaming pass by its bytes (4 B H N D for H rotated heads) at a fitted
 * fraction of 8 TB/s plus a fixed cost and a second launch, and each
 * attention kernel (plain, rotating Q and K, rotating Q only) by a fitted
 * time per workgroup step over one 64-key tile times the makespan of its
 * launch: every workgroup's key tiles plus a fitted fixed part, scheduled on
 * the CUs of each XCD in launch order; the constants are fitted per head dim
 * (64, 128) and MHA/GQA to kernel times measured over D = 64 and 128, bf16
 * and fp16, MHA, GQA 4:1 and 8:1, N = 1024 .. 32768. It weighs the whole
 * problem: more batch or heads at the
 * same N moves the choice as the work moves it. The choice of pre-rotation
 * versus in-kernel rotation is the one the AttnFuse report, paragraphs 3 and
 * 5, says depends on the GPU and the shape.
 *
 * workspace: caller-owned device memory for the rotated copies (Q' and K',
 * or K' alone), 16-byte aligned; its whole workspace_bytes must not overlap
 * any tensor argument (checked whichever path is taken); the library
 * allocates nothing (the fused path needs none). If it is NULL or
 * smaller than the preferred path needs, the next path it holds is taken
 * (split, then fused); so is a path whose streaming pass would exceed its
 * grid (more than 8 * 65535 slabs). rac_auto_plan tells the path and the
 * bytes the preferred path needs. Calls that share a workspace must not run
 * concurrently.
 */
int attn_rope_causal_auto(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int Hq, int Hkv, int N, int D, double rope_base,
                          int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The path (RAC_PATH_*) attn_rope_causal_auto takes for this shape and
 * workspace size, and the workspace bytes its preferred path needs. Either
 * output pointer may be NULL. Host only: no GPU work, no allocation.
 */
int rac_auto_plan(int B, int Hq, int Hkv, int N, int D, int dtype, size_t workspace_bytes,
                  int* path, size_t* preferred_bytes);

/*
 * Backward of attn_rope_causal_fwd: the gradients of the loss with respect to
 * the UNROTATED q and k and to v, given dout = dLoss/dout. The chain rule
 * through the forward's definition; the schedule is the two-pass backward of
 * "Fast and Exact Relative-Position Attention via Structure-Aware Kernels"
 * (rainbus digest), method section, Algorithm 2: a query-parallel pass
 * computes dq, a key-parallel pass dk and dv, each element with one writer
 * (no atomics; deterministic). RoPE's gradient, the inverse turn R(-p), is
 * applied to dq and dk in fp32 inside the kernels' epilogues. Both passes
 * read every query and key tile many times, so q and k are rotated once by
 * the streaming pass into 2 * B * (Hq + Hkv) * N * D bytes of stream-ordered
 * scratch (hipMallocAsync / hipFreeAsync on `stream`) rather than at each
 * tile visit; the results are bit for bit those of rotating in the kernels. The training step of
 * "AttnFuse Makes RoPE a First-Class Attention Compilation Operation",
 * paragraph 3, needs this backward.
 *
 *   q, dout, out, dq: [B,Hq,N,D]; k, v, dk, dv: [B,Hkv,N,D]; all `dtype`.
 *   out, lse: the forward's outputs for these inputs (lse fp32 [B,Hq,N],
 *             natural log) -- the backward rebuilds the probabilities from
 *             them rather than recomputing the row statistics.
 *   delta:    fp32 [B,Hq,N], written: rowsum(dout * out), which the
 *             key-parallel pass reads (caller-allocated, like the outputs).
 *   dk, dv:   summed over the Hq/Hkv query heads of each group.
 * Every pointer is a caller-owned device pointer, 16-byte aligned; lse is
 * required. Outputs must not overlap inputs or each other. Two kernels are
 * enqueued on `stream` (the dq pass first: it writes delta). For GQA shapes
 * whose key/value pass would leave the CUs unbalanced (at most two rounds
 * of its workgroups) two workgroups share each key tile: their fp32 sums
 * go to 16 * B * Hkv * N * D bytes of scratch taken with hipMallocAsync on
 * `stream` and released there with hipFreeAsync after a third kernel adds
 * them (RAC_ERR_HIP if that allocation fails).
 */
int attn_rope_causal_bwd(const void* q, const void* k, const void* v, const void* out,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         float* delta, int B, int Hq, int Hkv, int N, int D, double rope_base,
                         int dtype, void* stream);

/*
 * Backward of attn_causal_fwd (q and k already rotated): the gradients with
 * respect to the rotated q and k (and v). Same arguments and rules as
 * attn_rope_causal_bwd without rope_base. With rope_prerotate_bwd it is the
 * backward of the pre-rotation path.
 */
int attn_causal_bwd(const void* q, const void* k, const void* v, const void* out,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    float* delta, int B, int Hq, int Hkv, int N, int D, int dtype, void* stream);

/*
 * Backward of rope_prerotate: dq = R(-p) dq_rot, dk = R(-p) dk_rot, each pair
 * turned back by its position (x0 = y0 cos + y1 sin, x1 = y1 cos - y0 sin in
 * fp32, one rounding to `dtype`). Same shapes and aliasing rules as
 * rope_prerotate (exact in-place use allowed).
 */
int rope_prerotate_bwd(const void* dq_rot, const void* dk_rot, void* dq, void* dk, int B, int Hq,
                       int Hkv, int N, int D, double rope_base, int dtype, void* stream);

/*
 * The backward with a choice of RoPE pairing (RAC_PAIR_ADJACENT or
 * RAC_PAIR_HALF), for the forward of attn_rope_causal_fwd_ex and of
 * rope_prerotate_ex: "rotate half" checkpoints (the Llama layout) train
 * through it. The gradient of the turn is the inverse turn of the same pairs
 * (for the half-split pairing, element d with d + D/2: x_d = y_d cos +
 * y_{d+D/2} sin, x_{d+D/2} = y_{d+D/2} cos - y_d sin, in fp32, one rounding).
 *
 * attn_rope_causal_bwd_ex: as attn_rope_causal_bwd. With RAC_PAIR_HALF the
 *   two passes run on q and k rotated once by the half-split streaming pass
 *   (the same 2 * B * (Hq + Hkv) * N * D bytes of stream-ordered scratch),
 *   write dq and dk in the rotated frame, and a third streaming pass turns
 *   them back in place; B * (Hq + Hkv) <= 524280 (RAC_ERR_ARG beyond: the
 *   pass's grid), and RAC_BWD_ROT has no effect. Its results are those of
 *   rope_prerotate_ex, attn_causal_bwd and rope_prerotate_bwd_ex in turn,
 *   bit for bit. RAC_PAIR_ADJACENT is attn_rope_causal_bwd.
 * rope_prerotate_bwd_ex: as rope_prerotate_bwd, with the pairing.
 * Any other pairing value: RAC_ERR_ARG.
 */
int attn_rope_causal_bwd_ex(const void* q, const void* k, const void* v, const void* out,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            float* delta, int B, int Hq, int Hkv, int N, int D, double rope_base,
                            int pairing, int dtype, void* stream);
int rope_prerotate_bwd_ex(const void* dq_rot, const void* dk_rot, void* dq, void* dk, int B,
                          int Hq, int Hkv, int N, int D, double rope_base, int pairing, int dtype,
                          void* stream);

/*
 * Backward of attn_alibi_causal_fwd: the gradients with respect to q, k (the
 * unrotated ones when a RoPE pairing is given) and v. The penalty depends on
 * no input, so the gradients keep the form of attn_rope_causal_bwd's and only
 * the rebuilt probabilities carry it: P = exp(q_i . k_j / sqrt(D) -
 * slopes[h] (i - j) - lse_i), the penalty entering the base-2 exponent as
 * slopes[h] log2(e) (j - i) in fp32. Arguments, layouts, scratch and rules
 * as attn_rope_causal_bwd_ex, plus slopes and pairing as in
 * attn_alibi_causal_fwd (slopes must not overlap dq, dk, dv or delta); with
 * RoPE, B * (Hq + Hkv) <= 524280 (the streaming pass forms the rotated
 * operands; RAC_BWD_ROT has no effect).
 */
int attn_alibi_causal_bwd(const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          float* delta, int B, int Hq, int Hkv, int N, int D, const float* slopes,
                          double rope_base, int pairing, int dtype, void* stream);

/* Text for the last non-zero return on the calling thread ("" if none). */
const char* rac_last_error(void);

/* Synchronises every device holding a table, then frees all cos/sin tables
 * (the next call that needs one builds it again). It must not run
 * concurrently with any other call of this library: another thread may have
 * taken a table pointer and not yet enqueued the kernel that reads it.
 * Returns RAC_OK or RAC_ERR_HIP. */
int rac_release_tables(void);

/* Bandwidth ceiling (instrumentation; defines no part of the method). A
 * plain device-to-device copy of `bytes` bytes from `src` to `dst` (device
 * pointers, 16-byte aligned, not overlapping; `bytes` a multiple of 16) with
 * the pre-rotation pass's memory access pattern (16-byte non-temporal loads
 * and stores, 256-lane workgroups): the rate the pass could reach if rotating
 * cost nothing. Enqueued on `stream`; the kernel timer times it like a pass.
 * bytes == 0 is a no-op. Returns RAC_OK, RAC_ERR_ARG or RAC_ERR_ALIGN. */
int rac_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Kernel timing (instrumentation; defines no part of the method). Arms a
 * pair of HIP events (hipEvent_t handles, created by the caller with timing
 * enabled, owned by the caller) for the next forward attention or
 * pre-rotation kernel this library launches from the calling thread: that
 * kernel is launched with hipExtLaunchKernel, which records `start_event`
 * and `stop_event` at the kernel's own start and end on its stream, so
 * hipEventElapsedTime gives its execution time without the queue's dispatch
 * latency. The events are disarmed once used, and when the next forward or
 * pass entry point returns without launching (an argument error, an empty
 * problem); an entry point that makes several launches (the dispatcher's
 * two-kernel paths) times the first. Backward kernels ignore the timer.
 * Both NULL disarms.
 * Returns RAC_OK, or RAC_ERR_ARG if exactly one event is NULL. */
int rac_time_next_kernel(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* RAC_H */
