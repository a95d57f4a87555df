// rac_internal.h -- host-side launch interface between the C ABI layer and the
// kernel translation units. Arguments are already validated by the caller.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rac {

// Kernel timing: a pair of caller-created HIP events that the next kernel
// launched through launch_kernel() on this thread records at its own start
// and end (then the pair is cleared). Null: no timing.
void take_kernel_timer(hipEvent_t* start, hipEvent_t* stop);

// Launches `kernel` on `stream` (no dynamic LDS), through hipExtLaunchKernel
// so that an armed kernel timer stamps the kernel's own start and end.
template <typename... Params, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block,
                                hipStream_t stream, Args... args) {
    hipEvent_t start = nullptr, stop = nullptr;
    take_kernel_timer(&start, &stop);
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0,
                          static_cast<Params>(args)...);
    return hipGetLastError();
}

// Launch shape of the attention kernels: chosen from the problem size, or
// forced (tests cover both shapes on small problems; tuning).
enum { ATTN_SHAPE_AUTO = 0, ATTN_SHAPE_PAIR = 1, ATTN_SHAPE_TILE = 2, ATTN_SHAPE_PAIR_HEADS = 3 };

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;          // may be null
    const float* table;  // cos/sin table [>= N][D] (fp32, cos/sin interleaved); null for ROT_NONE
    int B, Hq, Hkv, N, D;
    int dtype;
    int shape;           // ATTN_SHAPE_*
    int half_pairs;      // 1: RoPE pairs (d, d + D/2) instead of (2i, 2i+1)
    const float* slopes = nullptr;  // ALiBi slope per query head [Hq], or null for none
};

// Rotation applied inside the attention kernel: none (inputs already
// rotated), Q and K (the fused path), or Q only (K rotated beforehand).
enum { ROT_NONE = 0, ROT_QK = 1, ROT_Q = 2, ROT_QK_HALF = 3 };
// Backward only: q and k arrive already rotated; dq and dk are turned back
// by R(-p) in the epilogues (the gradients with respect to the unrotated q, k).
enum { ROT_QK_OUT = 8 };
// Added to a rotation mode: the ALiBi distance penalty on the scores.
enum { MOD_ALIBI = 4 };

// Causal attention forward; `rot` is a ROT_* mode.
hipError_t launch_attn_fwd(const AttnArgs& a, int rot, hipStream_t stream);

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* out;     // the forward's output
    const float* lse;    // the forward's log-sum-exp (natural log), [B, Hq, N]
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* delta;        // written: rowsum(dout * out), [B, Hq, N]
    const float* table;  // cos/sin table (ROT_QK only)
    int B, Hq, Hkv, N, D;
    int dtype;
    int shape = 0;       // BWD_SHAPE_* (the dK/dV pass)
    int dq_shape = 0;    // BWD_DQ_* (the dQ pass)
    const float* slopes = nullptr;  // ALiBi: one slope per query head, or none
};

// dK/dV pass workgroup shapes: automatic, 128 keys (8 waves), 64 keys (4
// waves), or 64 keys with two query groups (8 waves).
enum { BWD_SHAPE_AUTO = 0, BWD_SHAPE_K128 = 1, BWD_SHAPE_K64 = 2, BWD_SHAPE_K64X2 = 3,
       BWD_SHAPE_K64X2H = 4 };
enum { BWD_DQ_AUTO = 0, BWD_DQ_TILE = 1, BWD_DQ_PAIR = 2 };

// Causal attention backward (ROT_QK: RoPE fused, gradients with respect to
// the unrotated q and k; ROT_QK_OUT: q and k already rotated, gradients with
// respect to the unrotated ones; ROT_NONE: inputs already rotated, gradients
// with respect to them). With a.slopes the scores carry the ALiBi penalty
// (ROT_NONE and ROT_QK_OUT only).
hipError_t launch_attn_bwd(const BwdArgs& a, int rot, hipStream_t stream);

// q_rot = RoPE(q), k_rot = RoPE(k).
// A plain streaming device copy of `bytes` (a multiple of 16) bytes.
hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

hipError_t launch_rope_prerotate(const void* q, const void* k, void* q_rot, void* k_rot,
                                 const float* table, int B, int Hq, int Hkv, int N, int D,
                                 int dtype, hipStream_t stream);

// The same pass with the half-split pairing (elements d, d + D/2).
hipError_t launch_rope_prerotate_half(const void* q, const void* k, void* q_rot, void* k_rot,
                                      const float* table, int B, int Hq, int Hkv, int N, int D,
                                      int dtype, hipStream_t stream);

// The inverse turn R(-p) of the same pass: dq = R(-p) dq_rot, dk = R(-p)
// dk_rot (the gradient of the pre-rotation).
hipError_t launch_rope_unrotate(const void* dq_rot, const void* dk_rot, void* dq, void* dk,
                                const float* table, int B, int Hq, int Hkv, int N, int D,
                                int dtype, hipStream_t stream);

// The inverse turn with the half-split pairing.
hipError_t launch_rope_unrotate_half(const void* dq_rot, const void* dk_rot, void* dq, void* dk,
                                     const float* table, int B, int Hq, int Hkv, int N, int D,
                                     int dtype, hipStream_t stream);

}  // namespace rac
