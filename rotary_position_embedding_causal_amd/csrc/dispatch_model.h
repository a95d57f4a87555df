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
// microseconds, with BW = 8 TB/s:
//   T_k     = LAUNCH_US_k + (PAIR_US_k or TILE_US_k) * M   for the plain
//             attention kernel (k = ATTN), the one rotating Q and K tiles
//             (FUSED) and the one rotating Q rows (Q), where M is the
//             attention launch's makespan in 64-key steps (makespan() below:
//             each workgroup's key tiles plus WG_STEPS, list-scheduled per
//             XCD) and PAIR or TILE the launch shape attn_fwd.hip takes
//   fused   = T_FUSED
//   prerot  = T0_US + 4 B (Hq + Hkv) N D / (ETA_BW BW) + T_ATTN + T_GAP_US
//   split   = T0_US + 4 B Hkv N D / (ETA_BW BW) + T_Q + T_GAP_US
// Per class of shape (head dim 64 or 128; MHA, or GQA when Hq / Hkv >= 2) the
// ten kernel constants, and the three pass/launch constants shared by all,
// are least-squares fits to kernel times measured on MI355X back to back
// (steady clocks) over the crossover families:
//   MHA D=64 fp16, B=1 H=16, N = 1024, 1536, 2048, 3072, 4096, 6144, 8192, 16384, 32768
//   MHA D=128 bf16, B=1 H=32, N = 1024, 1536, 2048, 3072, 4096, 8192, 16384
//   GQA 4:1 D=64 bf16, B=1 Hq=32 Hkv=8, N = 1024, 1536, 2048, 3072, 4096, 8192, 16384
//   GQA 4:1 D=128 bf16 (Llama-3-8B layer), B=1 Hq=32 Hkv=8, N = 1024, 1536, 2048, 3072, 4096, 8192, 16384
//   GQA 4:1 D=128 fp16, B=1 Hq=32 Hkv=8, N = 1024, 1536, 2048, 3072, 4096, 8192
//   GQA 8:1 D=128 bf16, B=1 Hq=64 Hkv=8, N = 1024, 1536, 2048, 3072, 4096, 8192
#pragma once

#include <stdint.h>

namespace rac_model {

constexpr double HBM_BW = 8.0e12;  // B/s

constexpr double D64_MHA_WG_STEPS = 1;
constexpr double D64_MHA_LAUNCH_US_ATTN = 1.33028103;
constexpr double D64_MHA_PAIR_US_ATTN = 1.44042737;
constexpr double D64_MHA_TILE_US_ATTN = 1.12064664;
constexpr double D64_MHA_LAUNCH_US_FUSED = 0;
constexpr double D64_MHA_PAIR_US_FUSED = 1.77276363;
constexpr double D64_MHA_TILE_US_FUSED = 1.38400788;
constexpr double D64_MHA_LAUNCH_US_Q = 1.40886934;
constexpr double D64_MHA_PAIR_US_Q = 1.46980464;
constexpr double D64_MHA_TILE_US_Q = 1.14752419;

constexpr double D128_MHA_WG_STEPS = 1.75;
constexpr double D128_MHA_LAUNCH_US_ATTN = 4.96495382;
constexpr double D128_MHA_PAIR_US_ATTN = 1.95978548;
constexpr double D128_MHA_TILE_US_ATTN = 1.93141411;
constexpr double D128_MHA_LAUNCH_US_FUSED = 4.12203553;
constexpr double D128_MHA_PAIR_US_FUSED = 2.6025811;
constexpr double D128_MHA_TILE_US_FUSED = 2.58639366;
constexpr double D128_MHA_LAUNCH_US_Q = 5.28914155;
constexpr double D128_MHA_PAIR_US_Q = 2.00084926;
constexpr double D128_MHA_TILE_US_Q = 1.96642368;

constexpr double D64_GQA_WG_STEPS = 5.25;
constexpr double D64_GQA_LAUNCH_US_ATTN = 0;
constexpr double D64_GQA_PAIR_US_ATTN = 1.33728808;
constexpr double D64_GQA_TILE_US_ATTN = 1.12933704;
constexpr double D64_GQA_LAUNCH_US_FUSED = 0;
constexpr double D64_GQA_PAIR_US_FUSED = 1.51494905;
constexpr double D64_GQA_TILE_US_FUSED = 1.29885201;
constexpr double D64_GQA_LAUNCH_US_Q = 0.946686296;
constexpr double D64_GQA_PAIR_US_Q = 1.30998915;
constexpr double D64_GQA_TILE_US_Q = 1.13206002;

constexpr double D128_GQA_WG_STEPS = 3.25;
constexpr double D128_GQA_LAUNCH_US_ATTN = 0;
constexpr double D128_GQA_PAIR_US_ATTN = 2.10000806;
constexpr double D128_GQA_TILE_US_ATTN = 1.79329759;
constexpr double D128_GQA_LAUNCH_US_FUSED = 0;
constexpr double D128_GQA_PAIR_US_FUSED = 2.57983097;
constexpr double D128_GQA_TILE_US_FUSED = 2.17299282;
constexpr double D128_GQA_LAUNCH_US_Q = 0;
constexpr double D128_GQA_PAIR_US_Q = 2.14474025;
constexpr double D128_GQA_TILE_US_Q = 1.82515334;

constexpr double ETA_BW = 0.83386083;
constexpr double T0_US = 3.28226962;
constexpr double T_GAP_US = 0;

// The attention launch (as attn_fwd.hip takes it automatically): 128-row
// query tiles over 64-key tiles, 256 CUs in 8 XCDs.
constexpr int NUM_CUS = 256, NXCD = 8, BM = 128, BN = 64;
constexpr int64_t JOB_CAP = 4096;  // jobs per XCD scheduled one by one

struct Kernel {
    double launch_us, pair_us, tile_us;
};
struct Class {
    double wg_steps;
    Kernel attn, fused, q;
};

#define RAC_MODEL_KERNEL(P, K) Kernel{P##_LAUNCH_US_##K, P##_PAIR_US_##K, P##_TILE_US_##K}
#define RAC_MODEL_CLASS(P)                                                             \
    Class {                                                                            \
        P##_WG_STEPS, RAC_MODEL_KERNEL(P, ATTN), RAC_MODEL_KERNEL(P, FUSED),            \
            RAC_MODEL_KERNEL(P, Q)                                                     \
    }

inline Class shape_class(int D, int Hq, int Hkv) {
    const bool gqa = Hq / Hkv >= 2;
    if (D == 64) return gqa ? RAC_MODEL_CLASS(D64_GQA) : RAC_MODEL_CLASS(D64_MHA);
    return gqa ? RAC_MODEL_CLASS(D128_GQA) : RAC_MODEL_CLASS(D128_MHA);
}

#undef RAC_MODEL_CLASS
#undef RAC_MODEL_KERNEL

inline int64_t kv_tiles_of(int64_t qt, int64_t N) {
    const int64_t last = qt * BM + BM < N ? qt * BM + BM : N;
    return (last - 1) / BN + 1;
}

// The attention launch's makespan in 64-key steps (pair: whether it is the
// paired launch). Workgroup u walks base[(u / packs) % per_head] key tiles
// plus r steps of fixed work; XCD x runs units x U/8 .. (x+1) U/8 - 1 in
// order when 8 divides U (the launch's XCD-aware order), else units x,
// x + 8, ..., each on its least-loaded slot (one per CU, or two for the
// one-head tile launch's 4-wave workgroups). Past JOB_CAP jobs per XCD the
// XCD is taken as balanced: its mean load plus half the heaviest workgroup.
inline double makespan(int B, int Hq, int Hkv, int N, int D, double r, bool* pair) {
    const int64_t nq = ((int64_t)N + BM - 1) / BM;
    const int64_t n_pairs = (nq + 1) / 2;
    const int64_t pair_units = n_pairs * Hq * B;
    const int group = Hq / Hkv;
    const bool heads_ok = group % 2 == 0;
    *pair = nq >= 2 && pair_units <= NUM_CUS &&
            (pair_units >= NUM_CUS / 2 || nq >= (heads_ok ? 4 : 12));
    if (!heads_ok && nq >= 2 &&
        (pair_units == 2 * NUM_CUS ||
         (D == 128 && pair_units >= 3 * NUM_CUS / 2 && pair_units <= 2 * NUM_CUS)))
        *pair = true;
    int64_t units, per_head, packs, slots;
    if (*pair) {
        units = pair_units, per_head = n_pairs, packs = group, slots = NUM_CUS / NXCD;
    } else {
        const int hg = heads_ok ? 2 : 1;
        units = nq * Hq * B / hg, per_head = nq, packs = group / hg;
        slots = (NUM_CUS / NXCD) * (hg == 2 ? 1 : 2);
    }
    if (units <= 0) return 0.0;
    auto base = [&](int64_t i) -> int64_t {
        if (!*pair) return kv_tiles_of(nq - 1 - i, N);
        const int64_t th = nq - 1 - i;
        const int64_t len_l = i < th ? kv_tiles_of(i, N) : 0;
        return (len_l + kv_tiles_of(th, N) + 1) / 2;
    };
    // sum of base over units 0 .. x-1 (prefix over one head, then periods)
    int64_t total = 0, wmax_steps = 0;
    for (int64_t i = 0; i < per_head; ++i) {
        total += base(i);
        if (base(i) > wmax_steps) wmax_steps = base(i);
    }
    auto prefix = [&](int64_t m) {
        int64_t s = 0;
        for (int64_t i = 0; i < m; ++i) s += base(i);
        return s;
    };
    auto weight_sum = [&](int64_t x) -> double {
        const int64_t v = x / packs, rem = x % packs;
        const int64_t full = v / per_head, part = v % per_head;
        return (double)packs * ((double)full * total + prefix(part)) +
               (double)rem * (part < per_head ? base(part) : 0);
    };
    const double wmax = (double)wmax_steps + r;
    const bool div = units % NXCD == 0;
    double best = 0.0;
    double heap[64];
    for (int x = 0; x < NXCD; ++x) {
        const int64_t lo = div ? x * (units / NXCD) : x;
        const int64_t hi = div ? (x + 1) * (units / NXCD) : units;
        const int64_t step = div ? 1 : NXCD;
        const int64_t n = hi > lo ? (hi - lo + step - 1) / step : 0;
        if (n == 0) continue;
        double m;
        if (n > JOB_CAP) {
            const double steps = div ? weight_sum(hi) - weight_sum(lo) : weight_sum(units) / NXCD;
            m = (steps + r * (double)n) / (double)slots + 0.5 * wmax;
        } else {
            // list scheduling: a binary min-heap of the slots' loads
            const int k = (int)(n < slots ? n : slots);
            for (int i = 0; i < k; ++i) heap[i] = 0.0;
            for (int64_t u = lo; u < hi; u += step) {
                const double w = (double)base((u / packs) % per_head) + r;
                double v = heap[0] + w;  // the least-loaded slot takes it
                int i = 0;
                for (;;) {
                    int c = 2 * i + 1;
                    if (c >= k) break;
                    if (c + 1 < k && heap[c + 1] < heap[c]) ++c;
                    if (heap[c] >= v) break;
                    heap[i] = heap[c];
                    i = c;
                }
                heap[i] = v;
            }
            m = 0.0;
            for (int i = 0; i < k; ++i) m = heap[i] > m ? heap[i] : m;
        }
        if (m > best) best = m;
    }
    return best;
}

inline double kernel_us(const Kernel& k, bool pair, double m) {
    return k.launch_us + (pair ? k.pair_us : k.tile_us) * m;
}

// Modelled times in microseconds of the fused, pre-rotation and split paths.
inline void path_times(int B, int Hq, int Hkv, int N, int D, double* fused, double* prerot,
                       double* split) {
    const Class c = shape_class(D, Hq, Hkv);
    bool pair = false;
    const double m = makespan(B, Hq, Hkv, N, D, c.wg_steps, &pair);
    const double n = (double)N;
    const double qk_bytes = 2.0 * B * ((double)Hq + Hkv) * n * D * 2.0;
    const double k_bytes = 2.0 * B * (double)Hkv * n * D * 2.0;
    const double bw = ETA_BW * HBM_BW;
    *fused = kernel_us(c.fused, pair, m);
    *prerot = T0_US + qk_bytes / bw * 1e6 + kernel_us(c.attn, pair, m) + T_GAP_US;
    *split = T0_US + k_bytes / bw * 1e6 + kernel_us(c.q, pair, m) + T_GAP_US;
}

}  // namespace rac_model
