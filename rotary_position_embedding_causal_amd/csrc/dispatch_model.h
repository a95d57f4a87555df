// dispatch_model.h -- fitted constants of the path-cost model that
// attn_rope_causal_auto evaluates to pick the fused, pre-rotation or GQA
// split path. Written by `python -m rotary_position_embedding_causal_amd.
// dispatch_fit <bench json line>` from the crossover rows of one bench run;
// the run's summary sits beside the other measurements as
// profiles/crossover_fit.json.
//
// The model reads "AttnFuse Makes RoPE a First-Class Attention Compilation
// Operation" (tdteach paper-news, 2026-09-13), paragraph 3: pre-rotation is a
// memory-bandwidth cost, in-kernel rotation a compute-and-tiling cost; per
// paragraph 5 the choice is measured per architecture and shape. In
// microseconds, with F = 2 B Hq N^2 D, P = 2516.6 TFLOP/s, BW = 8 TB/s:
//   T_k     = max(F / (ETA_k P), TPRO_US_k + TILE_US_k N / 128)  for the plain
//             attention kernel (k = ATTN), the one rotating Q and K tiles
//             (FUSED) and the one rotating Q rows (Q); the second term is an
//             under-filled chip: one workgroup's prologue and N / 128 key tiles
//   fused   = T_FUSED
//   prerot  = T0_US + 4 B (Hq + Hkv) N D / (ETA_BW BW) + T_ATTN + T_GAP_US
//   split   = T0_US + 4 B Hkv N D / (ETA_BW BW) + T_Q + T_GAP_US
// Per class of shape (head dim 64 or 128; MHA, or GQA when Hq / Hkv >= 2) the
// nine kernel constants, and the three pass/launch constants shared by all,
// are least-squares fits to kernel times measured on MI355X back to back
// (steady clocks) over the crossover families:
//   MHA D=64 fp16, B=1 H=16, N = 1024, 2048, 4096, 6144, 8192, 16384, 32768
//   MHA D=128 bf16, B=1 H=32, N = 1024, 2048, 4096, 8192, 16384
//   GQA 4:1 D=64 bf16, B=1 Hq=32 Hkv=8, N = 1024, 2048, 4096, 8192, 16384
//   GQA 4:1 D=128 bf16 (Llama-3-8B layer), B=1 Hq=32 Hkv=8, N = 1024, 2048, 4096, 8192, 16384
//   GQA 4:1 D=128 fp16, B=1 Hq=32 Hkv=8, N = 1024, 2048, 4096, 8192
//   GQA 8:1 D=128 bf16, B=1 Hq=64 Hkv=8, N = 1024, 2048, 4096, 8192
#pragma once

namespace rac_model {

constexpr double MFMA_PEAK = 2516.6e12;  // FLOP/s, dense bf16/fp16
constexpr double HBM_BW = 8.0e12;        // B/s

constexpr double D64_MHA_ETA_ATTN = 0.327305;
constexpr double D64_MHA_TPRO_US_ATTN = 8.75;
constexpr double D64_MHA_TILE_US_ATTN = 1.21982;
constexpr double D64_MHA_ETA_FUSED = 0.261231;
constexpr double D64_MHA_TPRO_US_FUSED = 7.65;
constexpr double D64_MHA_TILE_US_FUSED = 1.61918;
constexpr double D64_MHA_ETA_Q = 0.321517;
constexpr double D64_MHA_TPRO_US_Q = 8.4;
constexpr double D64_MHA_TILE_US_Q = 1.28665;

constexpr double D128_MHA_ETA_ATTN = 0.366479;
constexpr double D128_MHA_TPRO_US_ATTN = 7.25;
constexpr double D128_MHA_TILE_US_ATTN = 2.23296;
constexpr double D128_MHA_ETA_FUSED = 0.273001;
constexpr double D128_MHA_TPRO_US_FUSED = 5.5;
constexpr double D128_MHA_TILE_US_FUSED = 3.15368;
constexpr double D128_MHA_ETA_Q = 0.356813;
constexpr double D128_MHA_TPRO_US_Q = 9.6;
constexpr double D128_MHA_TILE_US_Q = 2.09965;

constexpr double D64_GQA_ETA_ATTN = 0.340929;
constexpr double D64_GQA_TPRO_US_ATTN = 8.3;
constexpr double D64_GQA_TILE_US_ATTN = 1.2929;
constexpr double D64_GQA_ETA_FUSED = 0.29406;
constexpr double D64_GQA_TPRO_US_FUSED = 8.25;
constexpr double D64_GQA_TILE_US_FUSED = 1.61937;
constexpr double D64_GQA_ETA_Q = 0.335883;
constexpr double D64_GQA_TPRO_US_Q = 8.85;
constexpr double D64_GQA_TILE_US_Q = 1.27393;

constexpr double D128_GQA_ETA_ATTN = 0.430263;
constexpr double D128_GQA_TPRO_US_ATTN = 9.55;
constexpr double D128_GQA_TILE_US_ATTN = 2.07093;
constexpr double D128_GQA_ETA_FUSED = 0.349817;
constexpr double D128_GQA_TPRO_US_FUSED = 8.5;
constexpr double D128_GQA_TILE_US_FUSED = 2.85299;
constexpr double D128_GQA_ETA_Q = 0.424949;
constexpr double D128_GQA_TPRO_US_Q = 9.7;
constexpr double D128_GQA_TILE_US_Q = 2.08077;

constexpr double ETA_BW = 0.839877;
constexpr double T0_US = 3.32335;
constexpr double T_GAP_US = 0;

struct Kernel {
    double eta, tpro_us, tile_us;
};
struct Class {
    Kernel attn, fused, q;
};

#define RAC_MODEL_CLASS(P)                                                          \
    Class {                                                                         \
        {P##_ETA_ATTN, P##_TPRO_US_ATTN, P##_TILE_US_ATTN},                         \
            {P##_ETA_FUSED, P##_TPRO_US_FUSED, P##_TILE_US_FUSED},                  \
            {P##_ETA_Q, P##_TPRO_US_Q, P##_TILE_US_Q}                               \
    }

inline Class shape_class(int D, int Hq, int Hkv) {
    const bool gqa = Hq / Hkv >= 2;
    if (D == 64) return gqa ? RAC_MODEL_CLASS(D64_GQA) : RAC_MODEL_CLASS(D64_MHA);
    return gqa ? RAC_MODEL_CLASS(D128_GQA) : RAC_MODEL_CLASS(D128_MHA);
}

#undef RAC_MODEL_CLASS

inline double kernel_us(const Kernel& k, double flops, double n) {
    const double thr = flops / (k.eta * MFMA_PEAK) * 1e6;
    const double lat = k.tpro_us + k.tile_us * n / 128.0;
    return thr > lat ? thr : lat;
}

// Modelled times in microseconds of the fused, pre-rotation and split paths.
inline void path_times(int B, int Hq, int Hkv, int N, int D, double* fused, double* prerot,
                       double* split) {
    const Class c = shape_class(D, Hq, Hkv);
    const double n = (double)N;
    const double f = 2.0 * B * (double)Hq * n * n * D;
    const double qk_bytes = 2.0 * B * ((double)Hq + Hkv) * n * D * 2.0;
    const double k_bytes = 2.0 * B * (double)Hkv * n * D * 2.0;
    const double bw = ETA_BW * HBM_BW;
    *fused = kernel_us(c.fused, f, n);
    *prerot = T0_US + qk_bytes / bw * 1e6 + kernel_us(c.attn, f, n) + T_GAP_US;
    *split = T0_US + k_bytes / bw * 1e6 + kernel_us(c.q, f, n) + T_GAP_US;
}

}  // namespace rac_model
