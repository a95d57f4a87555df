// rac_api.hip -- the C ABI declared in include/rac.h: argument validation,
// the per-device cos/sin table cache, and kernel dispatch. Host code only.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/rac.h"
#include "dispatch_model.h"
#include "rac_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return RAC_OK;
}

// armed by rac_time_next_kernel(), taken by the next launch_kernel() call
thread_local hipEvent_t g_timer_start = nullptr;
thread_local hipEvent_t g_timer_stop = nullptr;

}  // namespace

namespace rac {
void take_kernel_timer(hipEvent_t* start, hipEvent_t* stop) {
    *start = g_timer_start;
    *stop = g_timer_stop;
    g_timer_start = g_timer_stop = nullptr;
}
}  // namespace rac

namespace {

// Disarms the kernel timer when a forward or pass entry point returns, so a
// call that launches nothing (an argument error, an empty problem) does not
// leave it armed for an unrelated later launch, whose caller may have
// destroyed the events by then. (A launch has already taken it.)
struct TimerScope {
    ~TimerScope() { g_timer_start = g_timer_stop = nullptr; }
};

}  // namespace

namespace {

// ---- cos/sin tables --------------------------------------------------------
//
// Entry [p][2i] = cos(p * theta_i), [p][2i+1] = sin(p * theta_i), with
// theta_i = base^(-2i/D) and the angle formed in fp64 (p up to millions times
// theta would lose the low bits of the angle in fp32), rounded once to fp32.

struct Table {
    float* dev = nullptr;
    int64_t capacity = 0;  // positions held
};

std::mutex g_mutex;
std::map<std::tuple<int, int, uint64_t>, Table> g_tables;  // (device, D, base bits)
std::vector<std::pair<int, float*>> g_retired;             // outgrown tables, freed on release

uint64_t bits_of(double x) {
    uint64_t u;
    memcpy(&u, &x, sizeof u);
    return u;
}

// theta_i = base^(-2i/D), i < D/2, in fp64 (the same expression for every table)
void table_thetas(int D, double base, double* theta) {
    for (int i = 0; i < D / 2; ++i) theta[i] = pow(base, -(2.0 * i) / (double)D);
}

int get_table(int D, double base, int N, const float** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(RAC_ERR_HIP, "hipGetDevice failed (no HIP device?)");
    std::lock_guard<std::mutex> lock(g_mutex);
    Table& t = g_tables[std::make_tuple(dev, D, bits_of(base))];
    if (t.capacity >= N) {
        *out = t.dev;
        return RAC_OK;
    }
    int64_t cap = 4096;
    while (cap < N) cap *= 2;
    std::vector<float> host((size_t)cap * D);
    std::vector<double> theta(D / 2);
    table_thetas(D, base, theta.data());
    for (int64_t p = 0; p < cap; ++p)
        for (int i = 0; i < D / 2; ++i) {
            const double ang = (double)p * theta[i];
            host[(size_t)p * D + 2 * i] = (float)cos(ang);
            host[(size_t)p * D + 2 * i + 1] = (float)sin(ang);
        }
    float* d = nullptr;
    if (hipMalloc(reinterpret_cast<void**>(&d), host.size() * sizeof(float)) != hipSuccess)
        return fail(RAC_ERR_HIP, "hipMalloc of a %lld-position RoPE table failed", (long long)cap);
    if (hipMemcpy(d, host.data(), host.size() * sizeof(float), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(d);
        return fail(RAC_ERR_HIP, "upload of the RoPE table failed");
    }
    // in-flight kernels may still read the old table: keep it until release
    if (t.dev) g_retired.emplace_back(dev, t.dev);
    t.dev = d;
    t.capacity = cap;
    *out = d;
    return RAC_OK;
}

// ---- the allocation-free entry point's table -------------------------------
//
// attn_rope_causal_fwd_noalloc keeps its cos/sin table in this fixed array
// instead of the cache above: each GPU the library runs on holds one copy
// (16 MiB) until the process ends. In host code `scratch` only stands in for
// the device symbol; its address on each device comes from
// hipGetSymbolAddress (kept per device in g_scratch_ptr) and only that
// address is handed to kernels.
constexpr int64_t SCRATCH_FLOATS = (int64_t)RAC_NOALLOC_MAX_N * 128;
static __device__ __align__(256) float scratch[SCRATCH_FLOATS];
constexpr int MAX_DEVICES = 64;
float* g_scratch_ptr[MAX_DEVICES] = {};  // under g_mutex

// The frequencies of one table, by value (a kernel argument).
struct Thetas {
    double t[64];
};

// Rows 0 .. N-1 of the table: [p][2i] = cos(p theta_i), [p][2i+1] = sin(p theta_i),
// the angle formed in fp64 and each value rounded once to fp32, as in get_table.
__global__ void build_table_kernel(float* tab, Thetas th, int D, int N) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int half = D / 2;
    const int64_t p = idx / half;
    const int i = (int)(idx % half);
    if (p >= N) return;
    const double ang = (double)p * th.t[i];
    tab[p * D + 2 * i] = (float)cos(ang);
    tab[p * D + 2 * i + 1] = (float)sin(ang);
}

// This device's address of `scratch` (looked up once per device, with it current).
int scratch_table(float** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(RAC_ERR_HIP, "hipGetDevice failed (no HIP device?)");
    if (dev < 0 || dev >= MAX_DEVICES) return fail(RAC_ERR_HIP, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(RAC_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<float*>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return RAC_OK;
}

// ---- validation --------------------------------------------------------------

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// Checks shared by every entry point. Returns RAC_OK, or an error code with
// the message set. Sets *empty when there is nothing to compute.
int check_shape(int B, int Hq, int Hkv, int N, int D, int dtype, bool* empty) {
    if (dtype != RAC_BF16 && dtype != RAC_FP16)
        return fail(RAC_ERR_ARG, "dtype must be RAC_BF16 (0) or RAC_FP16 (1), got %d", dtype);
    if (B < 0 || N < 0) return fail(RAC_ERR_ARG, "B and N must be >= 0 (B=%d, N=%d)", B, N);
    if (Hq < 1 || Hkv < 1) return fail(RAC_ERR_ARG, "Hq and Hkv must be >= 1 (Hq=%d, Hkv=%d)", Hq, Hkv);
    if (Hq % Hkv != 0)
        return fail(RAC_ERR_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (Hq > 65535 || B > 65535)
        return fail(RAC_ERR_ARG, "Hq and B must be <= 65535 (Hq=%d, B=%d)", Hq, B);
    if (N > RAC_MAX_N) return fail(RAC_ERR_ARG, "N=%d exceeds RAC_MAX_N=%d", N, RAC_MAX_N);
    if (D != 64 && D != 128)
        return fail(RAC_ERR_UNSUPPORTED, "head dim D=%d is not supported (64 or 128)", D);
    *empty = (B == 0 || N == 0);
    return RAC_OK;
}

int check_base(double base) {
    if (!(base > 0.0) || !isfinite(base))
        return fail(RAC_ERR_ARG, "rope_base must be finite and > 0");
    return RAC_OK;
}

int check_pairing(int pairing) {
    if (pairing != RAC_PAIR_ADJACENT && pairing != RAC_PAIR_HALF)
        return fail(RAC_ERR_ARG, "pairing must be RAC_PAIR_ADJACENT or RAC_PAIR_HALF");
    return RAC_OK;
}

int check_attn_ptrs(const void* q, const void* k, const void* v, const void* out, const float* lse,
                    int B, int Hq, int Hkv, int N, int D) {
    if (!q || !k || !v || !out) return fail(RAC_ERR_ARG, "q, k, v and out must be non-null");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (lse && !aligned16(lse)))
        return fail(RAC_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    const int64_t qbytes = (int64_t)B * Hq * N * D * 2;
    const int64_t kvbytes = (int64_t)B * Hkv * N * D * 2;
    if (overlap(out, qbytes, q, qbytes) || overlap(out, qbytes, k, kvbytes) ||
        overlap(out, qbytes, v, kvbytes))
        return fail(RAC_ERR_ARG, "out must not overlap q, k or v");
    if (lse) {
        const int64_t lbytes = (int64_t)B * Hq * N * 4;
        if (overlap(lse, lbytes, q, qbytes) || overlap(lse, lbytes, k, kvbytes) ||
            overlap(lse, lbytes, v, kvbytes) || overlap(lse, lbytes, out, qbytes))
            return fail(RAC_ERR_ARG, "lse must not overlap q, k, v or out");
    }
    return RAC_OK;
}

// The pre-rotation pass and its inverse: x (q or dq_rot), y (k or dk_rot) in,
// x_out, y_out written. Exact in-place use is allowed; any other overlap is not.
int check_pass_ptrs(const void* x, const void* y, const void* x_out, const void* y_out, int B,
                    int Hq, int Hkv, int N, int D) {
    if (!x || !y || !x_out || !y_out)
        return fail(RAC_ERR_ARG, "input and output tensors must be non-null");
    if (!aligned16(x) || !aligned16(y) || !aligned16(x_out) || !aligned16(y_out))
        return fail(RAC_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    const int64_t xb = (int64_t)B * Hq * N * D * 2;
    const int64_t yb = (int64_t)B * Hkv * N * D * 2;
    if ((x_out != x && overlap(x_out, xb, x, xb)) || overlap(x_out, xb, y, yb) ||
        (y_out != y && overlap(y_out, yb, y, yb)) || overlap(y_out, yb, x, xb) ||
        overlap(x_out, xb, y_out, yb))
        return fail(RAC_ERR_ARG,
                    "outputs may alias their inputs exactly, and must not overlap otherwise");
    return RAC_OK;
}

// RAC_ATTN_SHAPE=pair|tile|pairheads forces the attention launch shape (default: by size).
int attn_shape_from_env() {
    const char* e = getenv("RAC_ATTN_SHAPE");
    if (!e) return rac::ATTN_SHAPE_AUTO;
    if (!strcmp(e, "pair")) return rac::ATTN_SHAPE_PAIR;
    if (!strcmp(e, "tile")) return rac::ATTN_SHAPE_TILE;
    if (!strcmp(e, "pairheads")) return rac::ATTN_SHAPE_PAIR_HEADS;
    return rac::ATTN_SHAPE_AUTO;
}

int bwd_shape_from_env() {
    const char* e = getenv("RAC_BWD_SHAPE");
    if (!e) return rac::BWD_SHAPE_AUTO;
    if (!strcmp(e, "k128")) return rac::BWD_SHAPE_K128;
    if (!strcmp(e, "k64")) return rac::BWD_SHAPE_K64;
    if (!strcmp(e, "k64x2")) return rac::BWD_SHAPE_K64X2;
    if (!strcmp(e, "k64x2h")) return rac::BWD_SHAPE_K64X2H;
    return rac::BWD_SHAPE_AUTO;
}

// RAC_BWD_ROT=kernel makes the fused backward rotate q and k inside its
// kernels instead of once through the streaming pass (tests, timing).
bool bwd_rotation_in_kernel() {
    const char* e = getenv("RAC_BWD_ROT");
    return e && !strcmp(e, "kernel");
}

// RAC_BWD_DQ=tile|pair forces the dQ pass's launch shape (default: by size).
int bwd_dq_from_env() {
    const char* e = getenv("RAC_BWD_DQ");
    if (!e) return rac::BWD_DQ_AUTO;
    if (!strcmp(e, "tile")) return rac::BWD_DQ_TILE;
    if (!strcmp(e, "pair")) return rac::BWD_DQ_PAIR;
    return rac::BWD_DQ_AUTO;
}

// ---- the path dispatcher ------------------------------------------------------
//
// All three paths give bit-identical results (they hand the same rotated
// operands to the same attention arithmetic), so the choice is about time
// only: the path with the least modelled time (dispatch_model.h: a cost model
// of the attention kernels and the streaming pass, fitted per head dim and
// MHA/GQA class to kernel times measured on MI355X). The model weighs the
// whole problem (B, heads, N, D), not N alone: the pass costs bytes, each
// attention kernel a time per workgroup step times its launch's makespan
// (rounds of workgroups over the CUs), so an under-filled grid (few heads,
// short N) keeps the attention time from shrinking with the work.
size_t path_workspace(int path, int B, int Hq, int Hkv, int N, int D) {
    const size_t q = (size_t)B * Hq * N * D * 2, k = (size_t)B * Hkv * N * D * 2;
    const size_t q16 = (q + 255) & ~(size_t)255;  // K' starts 256-byte aligned
    if (path == RAC_PATH_PREROTATE) return q16 + k;
    if (path == RAC_PATH_SPLIT) return k;
    return 0;
}

int preferred_path(int B, int Hq, int Hkv, int N, int D) {
    double fused = 0, prerot = 0, split = 0;
    rac_model::path_times(B, Hq, Hkv, N, D, &fused, &prerot, &split);
    int best = RAC_PATH_FUSED;
    double t = fused;
    if (prerot < t) best = RAC_PATH_PREROTATE, t = prerot;
    if (split < t) best = RAC_PATH_SPLIT;
    return best;
}

// Whether a path's streaming pass fits its grid (at most 8 * 65535 slabs:
// B * (Hq + Hkv) for pre-rotation, B * Hkv for the K-only pass).
bool pass_fits(int path, int B, int Hq, int Hkv) {
    const int64_t slabs = path == RAC_PATH_PREROTATE ? (int64_t)B * (Hq + (int64_t)Hkv)
                          : path == RAC_PATH_SPLIT   ? (int64_t)B * Hkv
                                                     : 0;
    return slabs <= 8LL * 65535;
}

// The preferred path if the workspace holds it (and its pass fits its grid),
// else the next one that does: pre-rotation, then split, then fused.
int plan_path(int B, int Hq, int Hkv, int N, int D, size_t workspace_bytes) {
    const int pref = preferred_path(B, Hq, Hkv, N, D);
    auto usable = [&](int path) {
        return pass_fits(path, B, Hq, Hkv) &&
               workspace_bytes >= path_workspace(path, B, Hq, Hkv, N, D);
    };
    if (usable(pref)) return pref;
    if (pref == RAC_PATH_PREROTATE && usable(RAC_PATH_SPLIT)) return RAC_PATH_SPLIT;
    return RAC_PATH_FUSED;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(RAC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}


// Backward arguments: inputs q, k, v, out, lse, dout; outputs dq, dk, dv, delta.
int check_bwd_ptrs(const rac::BwdArgs& a) {
    if (!a.q || !a.k || !a.v || !a.out || !a.lse || !a.dout || !a.dq || !a.dk || !a.dv || !a.delta)
        return fail(RAC_ERR_ARG, "q, k, v, out, lse, dout, dq, dk, dv and delta must be non-null");
    const void* all[] = {a.q, a.k, a.v, a.out, a.lse, a.dout, a.dq, a.dk, a.dv, a.delta};
    for (const void* p : all)
        if (!aligned16(p)) return fail(RAC_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    const int64_t qb = (int64_t)a.B * a.Hq * a.N * a.D * 2;
    const int64_t kb = (int64_t)a.B * a.Hkv * a.N * a.D * 2;
    const int64_t rb = (int64_t)a.B * a.Hq * a.N * 4;
    const void* in[] = {a.q, a.k, a.v, a.out, a.lse, a.dout};
    const int64_t in_bytes[] = {qb, kb, kb, qb, rb, qb};
    const void* outs[] = {a.dq, a.dk, a.dv, a.delta};
    const int64_t out_bytes[] = {qb, kb, kb, rb};
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 6; ++i)
            if (overlap(outs[o], out_bytes[o], in[i], in_bytes[i]))
                return fail(RAC_ERR_ARG, "dq, dk, dv and delta must not overlap any input");
        for (int o2 = o + 1; o2 < 4; ++o2)
            if (overlap(outs[o], out_bytes[o], outs[o2], out_bytes[o2]))
                return fail(RAC_ERR_ARG, "dq, dk, dv and delta must not overlap each other");
    }
    return RAC_OK;
}

// Launches a streaming pass (pre-rotation or its inverse) from inside a
// backward call, which leaves the kernel timer armed for the next forward or
// pass call.
template <typename Launch>
hipError_t untimed(Launch launch) {
    const hipEvent_t timer_start = g_timer_start, timer_stop = g_timer_stop;
    g_timer_start = g_timer_stop = nullptr;
    const hipError_t e = launch();
    g_timer_start = timer_start;
    g_timer_stop = timer_stop;
    return e;
}

// The backward entry points: rot ROT_QK (RoPE fused; half: the half-split
// pairing) or ROT_NONE; alibi: slopes carry the ALiBi penalty (validated
// here: non-null, aligned, clear of the outputs).
int attn_bwd_common(const void* q, const void* k, const void* v, const void* out,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv, float* delta,
                    int B, int Hq, int Hkv, int N, int D, double rope_base, int dtype, int rot,
                    void* stream, const char* what, bool half = false, bool alibi = false,
                    const float* slopes = nullptr) {
    bool empty = false;
    int rc = check_shape(B, Hq, Hkv, N, D, dtype, &empty);
    if (rc != RAC_OK) return rc;
    if (rot == rac::ROT_QK && (rc = check_base(rope_base)) != RAC_OK) return rc;
    const bool pass_fits = (int64_t)B * (Hq + (int64_t)Hkv) <= 8LL * 65535;
    if (half && !pass_fits)
        return fail(RAC_ERR_ARG, "B*(Hq+Hkv) must be <= 524280 for the half-split pairing");
    if (alibi && rot == rac::ROT_QK && !pass_fits)
        return fail(RAC_ERR_ARG, "B*(Hq+Hkv) must be <= 524280 for RoPE with ALiBi");
    if (empty) return ok();
    rac::BwdArgs a{q, k, v, out, lse, dout, dq, dk, dv, delta, nullptr, B, Hq, Hkv, N, D, dtype,
                   bwd_shape_from_env(), bwd_dq_from_env()};
    if ((rc = check_bwd_ptrs(a)) != RAC_OK) return rc;
    if (alibi) {
        if (!slopes) return fail(RAC_ERR_ARG, "slopes must be non-null");
        if (reinterpret_cast<uintptr_t>(slopes) % 4 != 0)
            return fail(RAC_ERR_ALIGN, "slopes must be 4-byte aligned");
        const int64_t sb = (int64_t)Hq * 4;
        const int64_t qb = (int64_t)B * Hq * N * D * 2, kb = (int64_t)B * Hkv * N * D * 2;
        if (overlap(slopes, sb, dq, qb) || overlap(slopes, sb, dk, kb) ||
            overlap(slopes, sb, dv, kb) || overlap(slopes, sb, delta, (int64_t)B * Hq * N * 4))
            return fail(RAC_ERR_ARG, "slopes must not overlap dq, dk, dv or delta");
        a.slopes = slopes;
    }
    if (rot == rac::ROT_QK && (rc = get_table(D, rope_base, N, &a.table)) != RAC_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (rot != rac::ROT_QK || (!half && !alibi && bwd_rotation_in_kernel()))
        return hip_status(rac::launch_attn_bwd(a, rot, st), what);
    // Both passes read every query and key tile many times (each key tile once
    // per query tile that sees it, and the reverse), so the rotated operands
    // are formed once by the streaming pass into stream-ordered scratch; the
    // kernels then read them as they are and turn dq and dk back by R(-p) in
    // their epilogues, exactly as when rotating in the kernel (the same
    // operands, the same arithmetic).
    // With the half-split pairing the kernels run plain on the rotated
    // operands and write the gradients in the rotated frame, which a second
    // streaming pass turns back by R(-p) in place (the epilogues' in-register
    // turn handles adjacent pairs only).
    const size_t qbytes = (size_t)B * Hq * N * D * 2, kbytes = (size_t)B * Hkv * N * D * 2;
    const size_t q16 = (qbytes + 255) & ~(size_t)255;
    char* scratch = nullptr;
    if (!pass_fits)  // the pass's grid: rotate in the kernel
        return hip_status(rac::launch_attn_bwd(a, rot, st), what);
    hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&scratch), q16 + kbytes, st);
    if (e != hipSuccess) return hip_status(e, "attn_rope_causal_bwd scratch allocation");
    e = untimed([&] {
        return half ? rac::launch_rope_prerotate_half(q, k, scratch, scratch + q16, a.table, B,
                                                      Hq, Hkv, N, D, dtype, st)
                    : rac::launch_rope_prerotate(q, k, scratch, scratch + q16, a.table, B, Hq,
                                                 Hkv, N, D, dtype, st);
    });
    if (e == hipSuccess) {
        a.q = scratch;
        a.k = scratch + q16;
        e = rac::launch_attn_bwd(a, half ? rac::ROT_NONE : rac::ROT_QK_OUT, st);
    }
    if (e == hipSuccess && half)
        e = untimed([&] {
            return rac::launch_rope_unrotate_half(dq, dk, dq, dk, a.table, B, Hq, Hkv, N, D,
                                                  dtype, st);
        });
    const hipError_t f = hipFreeAsync(scratch, st);
    return hip_status(e != hipSuccess ? e : f, what);
}

}  // namespace

extern "C" {

int attn_rope_causal_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                            int B, int Hq, int Hkv, int N, int D, double rope_base, int pairing,
                            int dtype, void* stream) {
    const TimerScope timer_scope;
    bool empty = false;
    int rc = check_shape(B, Hq, Hkv, N, D, dtype, &empty);
    if (rc != RAC_OK) return rc;
    if ((rc = check_base(rope_base)) != RAC_OK) return rc;
    if ((rc = check_pairing(pairing)) != RAC_OK) return rc;
    if (empty) return ok();
    if ((rc = check_attn_ptrs(q, k, v, out, lse, B, Hq, Hkv, N, D)) != RAC_OK) return rc;
    const float* table = nullptr;
    if ((rc = get_table(D, rope_base, N, &table)) != RAC_OK) return rc;
    rac::AttnArgs a{q, k, v, out, lse, table, B, Hq, Hkv, N, D, dtype, attn_shape_from_env(),
                    pairing == RAC_PAIR_HALF};
    return hip_status(rac::launch_attn_fwd(a, rac::ROT_QK, static_cast<hipStream_t>(stream)),
                      "attn_rope_causal_fwd launch");
}

int attn_rope_causal_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                                 float* lse, int B, int Hq, int Hkv, int N, int D,
                                 double rope_base, int dtype, void* stream) {
    const TimerScope timer_scope;
    bool empty = false;
    int rc = check_shape(B, Hq, Hkv, N, D, dtype, &empty);
    if (rc != RAC_OK) return rc;
    if ((rc = check_base(rope_base)) != RAC_OK) return rc;
    if ((int64_t)N * D > SCRATCH_FLOATS)
        return fail(RAC_ERR_ARG, "N*D=%lld exceeds the static table (%lld floats: N <= %lld at D=%d)",
                    (long long)N * D, (long long)SCRATCH_FLOATS, (long long)(SCRATCH_FLOATS / D), D);
    if (empty) return ok();
    if ((rc = check_attn_ptrs(q, k, v, out, lse, B, Hq, Hkv, N, D)) != RAC_OK) return rc;
    float* table = nullptr;
    if ((rc = scratch_table(&table)) != RAC_OK) return rc;
    // the rows this call needs, rebuilt on its stream (so a call, or a
    // captured graph of it, never depends on another call's table)
    Thetas th;
    table_thetas(D, rope_base, th.t);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t items = (int64_t)N * (D / 2);
    build_table_kernel<<<dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st>>>(table, th, D, N);
    if ((rc = hip_status(hipGetLastError(), "table build launch")) != RAC_OK) return rc;
    rac::AttnArgs a{q, k, v, out, lse, table, B, Hq, Hkv, N, D, dtype, attn_shape_from_env()};
    return hip_status(rac::launch_attn_fwd(a, rac::ROT_QK, st), "attn_rope_causal_fwd_noalloc launch");
}

int attn_alibi_causal_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int Hq, int Hkv, int N, int D, const float* slopes,
                          double rope_base, int pairing, int dtype, void* stream) {
    const TimerScope timer_scope;
    bool empty = false;
    int rc = check_shape(B, Hq, Hkv, N, D, dtype, &empty);
    if (rc != RAC_OK) return rc;
    const bool rope = pairing != RAC_ROPE_NONE;
    if (rope && (rc = check_pairing(pairing)) != RAC_OK) return rc;
    if (rope && (rc = check_base(rope_base)) != RAC_OK) return rc;
    if (empty) return ok();
    if ((rc = check_attn_ptrs(q, k, v, out, lse, B, Hq, Hkv, N, D)) != RAC_OK) return rc;
    if (!slopes) return fail(RAC_ERR_ARG, "slopes must be non-null");
    if (reinterpret_cast<uintptr_t>(slopes) % 4 != 0)
        return fail(RAC_ERR_ALIGN, "slopes must be 4-byte aligned");
    const int64_t slope_bytes = (int64_t)Hq * 4;
    const int64_t out_bytes = (int64_t)B * Hq * N * D * 2;
    if (overlap(slopes, slope_bytes, out, out_bytes) ||
        (lse && overlap(slopes, slope_bytes, lse, (int64_t)B * Hq * N * 4)))
        return fail(RAC_ERR_ARG, "slopes must not overlap out or lse");
    const float* table = nullptr;
    if (rope && (rc = get_table(D, rope_base, N, &table)) != RAC_OK) return rc;
    rac::AttnArgs a{q, k, v, out, lse, table, B, Hq, Hkv, N, D, dtype, attn_shape_from_env(),
                    pairing == RAC_PAIR_HALF, slopes};
    return hip_status(rac::launch_attn_fwd(a, rope ? rac::ROT_QK : rac::ROT_NONE,
                                           static_cast<hipStream_t>(stream)),
                      "attn_alibi_causal_fwd launch");
}

int attn_rope_causal_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                         int B, int Hq, int Hkv, int N, int D, double rope_base, int dtype,
                         void* stream) {
    return attn_rope_causal_fwd_ex(q, k, v, out, lse, B, Hq, Hkv, N, D, rope_base,
                                   RAC_PAIR_ADJACENT, dtype, stream);
}

int attn_rope_q_causal_fwd(const void* q, const void* k_rot, const void* v, void* out,
                           float* lse, int B, int Hq, int Hkv, int N, int D, double rope_base,
                           int dtype, void* stream) {
    const TimerScope timer_scope;
    bool empty = false;
    int rc = check_shape(B, Hq, Hkv, N, D, dtype, &empty);
    if (rc != RAC_OK) return rc;
    if ((rc = check_base(rope_base)) != RAC_OK) return rc;
    if (empty) return ok();
    if ((rc = check_attn_ptrs(q, k_rot, v, out, lse, B, Hq, Hkv, N, D)) != RAC_OK) return rc;
    const float* table = nullptr;
    if ((rc = get_table(D, rope_base, N, &table)) != RAC_OK) return rc;
    rac::AttnArgs a{q, k_rot, v, out, lse, table, B, Hq, Hkv, N, D, dtype, attn_shape_from_env()};
    return hip_status(rac::launch_attn_fwd(a, rac::ROT_Q, static_cast<hipStream_t>(stream)),
                      "attn_rope_q_causal_fwd launch");
}

int attn_causal_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                    int Hq, int Hkv, int N, int D, int dtype, void* stream) {
    const TimerScope timer_scope;
    bool empty = false;
    int rc = check_shape(B, Hq, Hkv, N, D, dtype, &empty);
    if (rc != RAC_OK) return rc;
    if (empty) return ok();
    if ((rc = check_attn_ptrs(q, k, v, out, lse, B, Hq, Hkv, N, D)) != RAC_OK) return rc;
    rac::AttnArgs a{q, k, v, out, lse, nullptr, B, Hq, Hkv, N, D, dtype, attn_shape_from_env()};
    return hip_status(rac::launch_attn_fwd(a, rac::ROT_NONE, static_cast<hipStream_t>(stream)),
                      "attn_causal_fwd launch");
}

int rope_prerotate_ex(const void* q, const void* k, void* q_rot, void* k_rot, int B, int Hq,
                      int Hkv, int N, int D, double rope_base, int pairing, int dtype,
                      void* stream) {
    const TimerScope timer_scope;
    bool empty = false;
    int rc = check_shape(B, Hq, Hkv, N, D, dtype, &empty);
    if (rc != RAC_OK) return rc;
    if ((rc = check_base(rope_base)) != RAC_OK) return rc;
    if ((rc = check_pairing(pairing)) != RAC_OK) return rc;
    if ((int64_t)B * (Hq + (int64_t)Hkv) > 8LL * 65535)
        return fail(RAC_ERR_ARG, "B*(Hq+Hkv) must be <= 524280");
    if (empty) return ok();
    if ((rc = check_pass_ptrs(q, k, q_rot, k_rot, B, Hq, Hkv, N, D)) != RAC_OK) return rc;
    const float* table = nullptr;
    if ((rc = get_table(D, rope_base, N, &table)) != RAC_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(
        pairing == RAC_PAIR_HALF
            ? rac::launch_rope_prerotate_half(q, k, q_rot, k_rot, table, B, Hq, Hkv, N, D, dtype, st)
            : rac::launch_rope_prerotate(q, k, q_rot, k_rot, table, B, Hq, Hkv, N, D, dtype, st),
        "rope_prerotate launch");
}

int rope_prerotate(const void* q, const void* k, void* q_rot, void* k_rot, int B, int Hq,
                   int Hkv, int N, int D, double rope_base, int dtype, void* stream) {
    return rope_prerotate_ex(q, k, q_rot, k_rot, B, Hq, Hkv, N, D, rope_base, RAC_PAIR_ADJACENT,
                             dtype, stream);
}

int rope_prerotate_bwd_ex(const void* dq_rot, const void* dk_rot, void* dq, void* dk, int B,
                          int Hq, int Hkv, int N, int D, double rope_base, int pairing, int dtype,
                          void* stream) {
    const TimerScope timer_scope;
    bool empty = false;
    int rc = check_shape(B, Hq, Hkv, N, D, dtype, &empty);
    if (rc != RAC_OK) return rc;
    if ((rc = check_base(rope_base)) != RAC_OK) return rc;
    if ((rc = check_pairing(pairing)) != RAC_OK) return rc;
    if ((int64_t)B * (Hq + (int64_t)Hkv) > 8LL * 65535)
        return fail(RAC_ERR_ARG, "B*(Hq+Hkv) must be <= 524280");
    if (empty) return ok();
    if ((rc = check_pass_ptrs(dq_rot, dk_rot, dq, dk, B, Hq, Hkv, N, D)) != RAC_OK) return rc;
    const float* table = nullptr;
    if ((rc = get_table(D, rope_base, N, &table)) != RAC_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(
        pairing == RAC_PAIR_HALF
            ? rac::launch_rope_unrotate_half(dq_rot, dk_rot, dq, dk, table, B, Hq, Hkv, N, D,
                                             dtype, st)
            : rac::launch_rope_unrotate(dq_rot, dk_rot, dq, dk, table, B, Hq, Hkv, N, D, dtype,
                                        st),
        "rope_prerotate_bwd launch");
}

int rope_prerotate_bwd(const void* dq_rot, const void* dk_rot, void* dq, void* dk, int B, int Hq,
                       int Hkv, int N, int D, double rope_base, int dtype, void* stream) {
    return rope_prerotate_bwd_ex(dq_rot, dk_rot, dq, dk, B, Hq, Hkv, N, D, rope_base,
                                 RAC_PAIR_ADJACENT, dtype, stream);
}


int attn_rope_causal_bwd_ex(const void* q, const void* k, const void* v, const void* out,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            float* delta, int B, int Hq, int Hkv, int N, int D, double rope_base,
                            int pairing, int dtype, void* stream) {
    const int rc = check_pairing(pairing);
    if (rc != RAC_OK) return rc;
    return attn_bwd_common(q, k, v, out, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, N, D,
                           rope_base, dtype, rac::ROT_QK, stream, "attn_rope_causal_bwd launch",
                           pairing == RAC_PAIR_HALF);
}

int attn_rope_causal_bwd(const void* q, const void* k, const void* v, const void* out,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         float* delta, int B, int Hq, int Hkv, int N, int D, double rope_base,
                         int dtype, void* stream) {
    return attn_rope_causal_bwd_ex(q, k, v, out, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, N, D,
                                   rope_base, RAC_PAIR_ADJACENT, dtype, stream);
}

int attn_causal_bwd(const void* q, const void* k, const void* v, const void* out,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    float* delta, int B, int Hq, int Hkv, int N, int D, int dtype, void* stream) {
    return attn_bwd_common(q, k, v, out, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, N, D, 1.0,
                           dtype, rac::ROT_NONE, stream, "attn_causal_bwd launch");
}

int attn_alibi_causal_bwd(const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          float* delta, int B, int Hq, int Hkv, int N, int D, const float* slopes,
                          double rope_base, int pairing, int dtype, void* stream) {
    const bool rope = pairing != RAC_ROPE_NONE;
    int rc = RAC_OK;
    if (rope && (rc = check_pairing(pairing)) != RAC_OK) return rc;
    return attn_bwd_common(q, k, v, out, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, N, D,
                           rope ? rope_base : 1.0, dtype, rope ? rac::ROT_QK : rac::ROT_NONE,
                           stream, "attn_alibi_causal_bwd launch", pairing == RAC_PAIR_HALF, true,
                           slopes);
}

int rope_prerotate_k(const void* k, void* k_rot, int B, int Hkv, int N, int D, double rope_base,
                     int dtype, void* stream) {
    const TimerScope timer_scope;
    bool empty = false;
    int rc = check_shape(B, Hkv, Hkv, N, D, dtype, &empty);
    if (rc != RAC_OK) return rc;
    if ((rc = check_base(rope_base)) != RAC_OK) return rc;
    if ((int64_t)B * Hkv > 8LL * 65535) return fail(RAC_ERR_ARG, "B*Hkv must be <= 524280");
    if (empty) return ok();
    if (!k || !k_rot) return fail(RAC_ERR_ARG, "k and k_rot must be non-null");
    if (!aligned16(k) || !aligned16(k_rot))
        return fail(RAC_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    const int64_t kbytes = (int64_t)B * Hkv * N * D * 2;
    if (k_rot != k && overlap(k_rot, kbytes, k, kbytes))
        return fail(RAC_ERR_ARG, "k_rot may alias k exactly, and must not overlap it otherwise");
    const float* table = nullptr;
    if ((rc = get_table(D, rope_base, N, &table)) != RAC_OK) return rc;
    // the pre-rotation pass with no query slabs
    return hip_status(rac::launch_rope_prerotate(nullptr, k, nullptr, k_rot, table, B, 0, Hkv, N,
                                                 D, dtype, static_cast<hipStream_t>(stream)),
                      "rope_prerotate_k launch");
}

int rac_auto_plan(int B, int Hq, int Hkv, int N, int D, int dtype, size_t workspace_bytes,
                  int* path, size_t* preferred_bytes) {
    bool empty = false;
    const int rc = check_shape(B, Hq, Hkv, N, D, dtype, &empty);
    if (rc != RAC_OK) return rc;
    const int pref = preferred_path(B, Hq, Hkv, N, D);
    if (path) *path = empty ? RAC_PATH_FUSED : plan_path(B, Hq, Hkv, N, D, workspace_bytes);
    if (preferred_bytes) *preferred_bytes = empty ? 0 : path_workspace(pref, B, Hq, Hkv, N, D);
    return ok();
}

int attn_rope_causal_auto(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int Hq, int Hkv, int N, int D, double rope_base, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
    const TimerScope timer_scope;
    bool empty = false;
    int rc = check_shape(B, Hq, Hkv, N, D, dtype, &empty);
    if (rc != RAC_OK) return rc;
    if ((rc = check_base(rope_base)) != RAC_OK) return rc;
    if (empty) return ok();
    if ((rc = check_attn_ptrs(q, k, v, out, lse, B, Hq, Hkv, N, D)) != RAC_OK) return rc;
    if (!workspace) workspace_bytes = 0;
    const int64_t qbytes = (int64_t)B * Hq * N * D * 2;
    const int64_t kvbytes = (int64_t)B * Hkv * N * D * 2;
    if (workspace_bytes > 0) {
        // the whole workspace given, whichever path is taken
        if (!aligned16(workspace)) return fail(RAC_ERR_ALIGN, "workspace must be 16-byte aligned");
        const int64_t wbytes = workspace_bytes > ((size_t)1 << 62) ? (int64_t)1 << 62
                                                                   : (int64_t)workspace_bytes;
        if (overlap(workspace, wbytes, q, qbytes) || overlap(workspace, wbytes, k, kvbytes) ||
            overlap(workspace, wbytes, v, kvbytes) || overlap(workspace, wbytes, out, qbytes) ||
            (lse && overlap(workspace, wbytes, lse, (int64_t)B * Hq * N * 4)))
            return fail(RAC_ERR_ARG, "workspace must not overlap q, k, v, out or lse");
    }
    const int path = plan_path(B, Hq, Hkv, N, D, workspace_bytes);
    if (path == RAC_PATH_FUSED)
        return attn_rope_causal_fwd(q, k, v, out, lse, B, Hq, Hkv, N, D, rope_base, dtype, stream);
    char* ws = static_cast<char*>(workspace);
    if (path == RAC_PATH_SPLIT) {
        if ((rc = rope_prerotate_k(k, ws, B, Hkv, N, D, rope_base, dtype, stream)) != RAC_OK)
            return rc;
        return attn_rope_q_causal_fwd(q, ws, v, out, lse, B, Hq, Hkv, N, D, rope_base, dtype,
                                      stream);
    }
    char* kr = ws + (((size_t)qbytes + 255) & ~(size_t)255);
    if ((rc = rope_prerotate(q, k, ws, kr, B, Hq, Hkv, N, D, rope_base, dtype, stream)) != RAC_OK)
        return rc;
    return attn_causal_fwd(ws, kr, v, out, lse, B, Hq, Hkv, N, D, dtype, stream);
}

const char* rac_last_error(void) { return g_last_error.c_str(); }

int rac_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
    const TimerScope timer_scope;
    if (bytes == 0) return ok();
    if (!src || !dst) return fail(RAC_ERR_ARG, "src and dst must be non-null");
    if (bytes % 16 != 0) return fail(RAC_ERR_ARG, "bytes must be a multiple of 16");
    if (bytes > (size_t)1 << 46) return fail(RAC_ERR_ARG, "bytes must be <= 2^46");
    if (!aligned16(src) || !aligned16(dst))
        return fail(RAC_ERR_ALIGN, "src and dst must be 16-byte aligned");
    if (overlap(dst, (int64_t)bytes, src, (int64_t)bytes))
        return fail(RAC_ERR_ARG, "src and dst must not overlap");
    return hip_status(rac::launch_stream_copy(src, dst, (int64_t)bytes,
                                              static_cast<hipStream_t>(stream)),
                      "rac_stream_copy launch");
}

int rac_time_next_kernel(void* start_event, void* stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr))
        return fail(RAC_ERR_ARG, "rac_time_next_kernel: pass both events or neither");
    g_timer_start = static_cast<hipEvent_t>(start_event);
    g_timer_stop = static_cast<hipEvent_t>(stop_event);
    return ok();
}

int rac_release_tables(void) {
    std::lock_guard<std::mutex> lock(g_mutex);
    int prev = 0;
    bool have_prev = hipGetDevice(&prev) == hipSuccess;
    bool failed = false;
    std::map<int, bool> synced;
    auto sync_dev = [&](int dev) {
        if (synced.count(dev)) return;
        synced[dev] = true;
        if (hipSetDevice(dev) != hipSuccess || hipDeviceSynchronize() != hipSuccess) failed = true;
    };
    for (auto& kv : g_tables) {
        const int dev = std::get<0>(kv.first);
        if (!kv.second.dev) continue;
        sync_dev(dev);
        if (hipFree(kv.second.dev) != hipSuccess) failed = true;
    }
    for (auto& r : g_retired) {
        sync_dev(r.first);
        if (hipFree(r.second) != hipSuccess) failed = true;
    }
    g_tables.clear();
    g_retired.clear();
    if (have_prev) (void)hipSetDevice(prev);
    if (failed) return fail(RAC_ERR_HIP, "freeing the RoPE tables failed");
    return ok();
}

}  // extern "C"
