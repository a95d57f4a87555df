// rac_internal.h -- host-side launch interface between the C ABI layer and the
// kernel translation units. Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rac {

// Launch shape of the attention kernels: chosen from the problem size, or
// forced (tests cover both shapes on small problems; tuning).
enum { ATTN_SHAPE_AUTO = 0, ATTN_SHAPE_PAIR = 1, ATTN_SHAPE_TILE = 2 };

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;          // may be null
    const float* table;  // cos/sin table [>= N][D] (fp32, cos/sin interleaved); null when no RoPE
    int B, Hq, Hkv, N, D;
    int dtype;
    int shape;           // ATTN_SHAPE_*
};

// Causal attention forward; rotates Q/K tiles in the kernel when `rope`.
hipError_t launch_attn_fwd(const AttnArgs& a, bool rope, hipStream_t stream);

// q_rot = RoPE(q), k_rot = RoPE(k).
hipError_t launch_rope_prerotate(const void* q, const void* k, void* q_rot, void* k_rot,
                                 const float* table, int B, int Hq, int Hkv, int N, int D,
                                 int dtype, hipStream_t stream);

}  // namespace rac
