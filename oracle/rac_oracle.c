/*
 * rac_oracle.c -- the fp64 CPU oracle for rotary position embedding (RoPE)
 * followed by causal softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * bench's CPU-baseline leg load this library. The product path (the HIP
 * library and its Python binding) never links, loads or calls it, and this
 * file shares no code, header, table or constant with that path.
 *
 * What it computes, and where the definition comes from:
 *
 *   RoPE. "Fast and Exact Relative-Position Attention via Structure-Aware
 *   Kernels" (rainbus digest), background section "RoPE and parameter-free
 *   position encodings": RoPE rotates each token's query and key by an angle
 *   that depends on the token's absolute position. The pages fix neither the
 *   pairing nor the frequencies; the readings taken are: adjacent pairs
 *   (2i, 2i+1), frequency theta_i = base^(-2i/D) for i < D/2, position p =
 *   the token's index in its sequence, and the pair (x, y) is turned counter-
 *   clockwise by p*theta_i:
 *       x' = x cos(p theta_i) - y sin(p theta_i)
 *       y' = x sin(p theta_i) + y cos(p theta_i)
 *   Values are not rotated. A second pairing, the half-split (x_i, x_{i+D/2})
 *   used by many checkpoints ("rotate_half"), is provided as its own routine.
 *
 *   Causal attention. Same digest, background section "FlashAttention and
 *   online softmax" and its method section (forward, Algorithm 1): scores
 *   s_ij = tau * q_i . k_j with tau = 1/sqrt(D), a causal mask that keeps key
 *   j for query i iff j <= i, softmax over j, o_i = sum_j P_ij v_j, and the
 *   per-row log-sum-exp L_i. Which key head a query head reads (MHA or GQA,
 *   "AttnFuse Makes RoPE a First-Class Attention Compilation Operation",
 *   paragraph 4): query head h reads key/value head floor(h / (Hq/Hkv)).
 *   The oracle takes the plain two-pass definition: the row maximum M_i,
 *   then l_i = sum_j exp(s_ij - M_i), o_i = sum_j exp(s_ij - M_i) v_j / l_i,
 *   L_i = M_i + ln l_i (natural log). No tiling, no online rescaling.
 *
 *   ALiBi. Same digest, same background section: a linear penalty on the
 *   attention score that grows with the distance between query and key. The
 *   reading taken: s_ij = tau * q_i . k_j - m_h * (i - j) with one slope m_h
 *   per query head, then the same causal softmax (its own routine,
 *   oracle_attn_alibi_rows).
 *
 *   Storage formats. bf16 and fp16 inputs are decoded exactly to fp64, and
 *   fp64 values are rounded to bf16/fp16 once, round-to-nearest-even, by this
 *   file's own code (the "rounded rotation" variant of the oracle).
 *
 *   Backward. The gradients of that attention with respect to q, k and v,
 *   given the gradient dO of the output, by the chain rule through the same
 *   definition: P_ij = exp(s_ij - L_i), dv_j = sum_i P_ij dO_i,
 *   dP_ij = dO_i . v_j, dS_ij = P_ij (dP_ij - Delta_i) with
 *   Delta_i = sum_j P_ij dP_ij (the softmax Jacobian), dq_i = tau sum_j dS_ij
 *   k_j and dk_j = tau sum_i dS_ij q_i; dk and dv of a key/value head sum
 *   over the query heads that read it. With ALiBi (oracle_attn_alibi_bwd)
 *   s_ij carries the penalty, which depends on no input, so only P changes.
 *   RoPE's gradient is the inverse
 *   rotation (turn by -p theta_i), i.e. oracle_rope at negated positions. The
 *   digest's method section describes its own backward as a two-pass
 *   recomputation from the stored L_i; this oracle recomputes everything from
 *   the definition and stores nothing between rows.
 *
 * Every routine is plain fp64 C; OpenMP only splits independent rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_FP16 = 1 };

/* ---- storage formats ---------------------------------------------------- */

static double decode_bf16(uint16_t b) {
    /* bf16 is the top half of an IEEE binary32. */
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double decode_fp16(uint16_t h) {
    /* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* zero / subnormal */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + (double)m, e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Round |a| > 0 to a grid with `frac_bits` fraction bits and smallest normal
 * exponent `emin`, round-to-nearest-even. Returns the rounded magnitude. */
static double rne_magnitude(double a, int frac_bits, int emin) {
    int e;
    frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) -> a in [2^(e-1), 2^e) */
    int ulp_exp = (e - 1 < emin ? emin : e - 1) - frac_bits;
    double r = ldexp(a, -ulp_exp);        /* exact: a power-of-two scaling */
    double n = nearbyint(r);              /* default mode: nearest, ties to even */
    return ldexp(n, ulp_exp);
}

static uint16_t encode_bf16(double x) {
    if (isnan(x)) return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    double r = rne_magnitude(a, 7, -126);
    /* largest finite bf16 is (2 - 2^-7) * 2^127; anything rounded past it is inf */
    if (r > ldexp(2.0 - ldexp(1.0, -7), 127)) return sign | 0x7f80;
    float f = (float)r;                   /* exact: r lies on the bf16 grid */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

static uint16_t encode_fp16(double x) {
    if (isnan(x)) return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    double r = rne_magnitude(a, 10, -14);
    if (r > 65504.0) return sign | 0x7c00;
    if (r < ldexp(1.0, -14))                          /* subnormal: r = m * 2^-24 */
        return sign | (uint16_t)ldexp(r, 24);
    int e;
    double f = frexp(r, &e);                          /* r = f * 2^e, f in [0.5,1) */
    int m = (int)(ldexp(f, 11) - 1024.0);             /* r = (1 + m/1024) * 2^(e-1) */
    return sign | (uint16_t)(((e - 1 + 15) << 10) | m);
}

void oracle_decode(const uint16_t* bits, int64_t n, int dtype, double* out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype == ORACLE_BF16 ? decode_bf16(bits[i]) : decode_fp16(bits[i]);
}

void oracle_encode(const double* x, int64_t n, int dtype, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype == ORACLE_BF16 ? encode_bf16(x[i]) : encode_fp16(x[i]);
}

/* ---- RoPE ---------------------------------------------------------------- */

/* x: `rows` rows of D values; pos[r] is the absolute position of row r.
 * out may equal x. */
void oracle_rope(const double* x, const int64_t* pos, int64_t rows, int D,
                 double base, double* out) {
    const double log_base = log(base);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double* xr = x + r * D;
        double* yr = out + r * D;
        for (int i = 0; i < D / 2; ++i) {
            double theta = exp(-((2.0 * i) / D) * log_base);
            double angle = (double)pos[r] * theta;
            double c = cos(angle), s = sin(angle);
            double x0 = xr[2 * i], x1 = xr[2 * i + 1];
            yr[2 * i] = x0 * c - x1 * s;
            yr[2 * i + 1] = x0 * s + x1 * c;
        }
    }
}

/* The half-split pairing (the "rotate_half" convention): pair i is
 * (x_i, x_{i+D/2}) instead of (x_2i, x_2i+1), same frequency theta_i and the
 * same counter-clockwise turn by p*theta_i. out may equal x. */
void oracle_rope_half(const double* x, const int64_t* pos, int64_t rows, int D,
                      double base, double* out) {
    const double log_base = log(base);
    const int half = D / 2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double* xr = x + r * D;
        double* yr = out + r * D;
        for (int i = 0; i < half; ++i) {
            const double freq = exp(-(2.0 * i / D) * log_base);
            const double turn = (double)pos[r] * freq;
            const double cs = cos(turn), sn = sin(turn);
            double a = xr[i], b = xr[i + half];
            yr[i] = a * cs - b * sn;
            yr[i + half] = a * sn + b * cs;
        }
    }
}

/* ---- causal attention ---------------------------------------------------- */

/* q [B,Hq,N,D], k and v [B,Hkv,N,D], all fp64 and contiguous.
 * rows: flattened query-row indices (b*Hq + h)*N + i to compute, or NULL for
 * every row. o receives D values per computed row (in the order of `rows`),
 * lse one value per row. Returns 0, or -1 on bad arguments. */
int oracle_attn_rows(const double* q, const double* k, const double* v,
                     int B, int Hq, int Hkv, int N, int D,
                     const int64_t* rows, int64_t nrows,
                     double* o, double* lse) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1 || Hq % Hkv != 0) return -1;
    const int64_t total = (int64_t)B * Hq * N;
    if (!rows) nrows = total;
    const int group = Hq / Hkv;
    const double tau = 1.0 / sqrt((double)D);
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t row = rows ? rows[r] : r;
            if (!s || row < 0 || row >= total) { bad = 1; continue; }
            int64_t i = row % N;
            int64_t bh = row / N;
            int64_t h = bh % Hq, b = bh / Hq;
            int64_t g = h / group;
            const double* qi = q + row * D;
            const double* kb = k + (b * Hkv + g) * (int64_t)N * D;
            const double* vb = v + (b * Hkv + g) * (int64_t)N * D;
            /* pass 1: scores of the visible keys j <= i and their maximum */
            double M = -INFINITY;
            for (int64_t j = 0; j <= i; ++j) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += qi[d] * kb[j * D + d];
                s[j] = tau * dot;
                if (s[j] > M) M = s[j];
            }
            /* pass 2: normaliser and the weighted sum of values */
            double l = 0.0;
            double* orow = o + r * D;
            for (int d = 0; d < D; ++d) orow[d] = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                double p = exp(s[j] - M);
                l += p;
                for (int d = 0; d < D; ++d) orow[d] += p * vb[j * D + d];
            }
            for (int d = 0; d < D; ++d) orow[d] /= l;
            lse[r] = M + log(l);
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/* ---- causal attention with a linear distance penalty (ALiBi) ------------ */

/* The attention of oracle_attn_rows with one post-product term: the score of
 * key j for query i of query head h is lowered in proportion to how far back
 * the key lies, slopes[h] * (i - j) ("Fast and Exact Relative-Position
 * Attention via Structure-Aware Kernels", rainbus digest, background "RoPE and
 * parameter-free position encodings": ALiBi adds a linear penalty by
 * distance). The penalty is added to the scaled product:
 *     s_ij = q_i . k_j / sqrt(D) - slopes[h] * (i - j),
 * one slope per QUERY head (slopes has Hq entries), then the same causal
 * softmax, output and natural-log LSE as oracle_attn_rows. */
int oracle_attn_alibi_rows(const double* q, const double* k, const double* v,
                           int B, int Hq, int Hkv, int N, int D, const double* slopes,
                           const int64_t* rows, int64_t nrows, double* o, double* lse) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1 || Hq % Hkv != 0 || !slopes) return -1;
    const int64_t all_rows = (int64_t)B * Hq * N;
    if (!rows) nrows = all_rows;
    const int heads_per_kv = Hq / Hkv;
    const double inv_sqrt_d = sqrt(1.0 / (double)D);
    int bad = 0;
#pragma omp parallel
    {
        double* score = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t flat = rows ? rows[r] : r;
            if (!score || flat < 0 || flat >= all_rows) { bad = 1; continue; }
            const int64_t qpos = flat % N;
            const int64_t qhead = (flat / N) % Hq, batch = flat / N / Hq;
            const int64_t kvh = batch * Hkv + qhead / heads_per_kv;
            const double slope = slopes[qhead];
            const double* qv = q + flat * D;
            const double* keys = k + kvh * (int64_t)N * D;
            const double* vals = v + kvh * (int64_t)N * D;
            double top = -INFINITY;
            for (int64_t kpos = 0; kpos <= qpos; ++kpos) {
                double qk = 0.0;
                for (int d = 0; d < D; ++d) qk += qv[d] * keys[kpos * D + d];
                const double distance = (double)(qpos - kpos);
                score[kpos] = inv_sqrt_d * qk - slope * distance;
                top = score[kpos] > top ? score[kpos] : top;
            }
            double denom = 0.0;
            double* out = o + r * D;
            for (int d = 0; d < D; ++d) out[d] = 0.0;
            for (int64_t kpos = 0; kpos <= qpos; ++kpos) {
                const double w = exp(score[kpos] - top);
                denom += w;
                for (int d = 0; d < D; ++d) out[d] += w * vals[kpos * D + d];
            }
            for (int d = 0; d < D; ++d) out[d] = out[d] / denom;
            lse[r] = top + log(denom);
        }
        free(score);
    }
    return bad ? -1 : 0;
}

/* ---- causal attention, backward ------------------------------------------ */

/* The ALiBi penalty of query head h for query i and key j (0 without
 * slopes): the term oracle_attn_alibi_rows subtracts from the scaled score. */
static double alibi_penalty(const double* slopes, int64_t h, int64_t i, int64_t j) {
    return slopes ? slopes[h] * (double)(i - j) : 0.0;
}

/* The scores of query row `row` (flattened (b*Hq + h)*N + i) against the
 * visible keys j = 0..i of its key head, s[j] = tau q_i . k_j minus the
 * ALiBi penalty when slopes are given; returns i. */
static int64_t row_scores(const double* q, const double* k, int Hq, int Hkv, int N, int D,
                          int64_t row, double tau, const double* slopes, double* s) {
    const int group = Hq / Hkv;
    int64_t i = row % N;
    int64_t bh = row / N;
    int64_t h = bh % Hq, b = bh / Hq;
    const int64_t kv_head = b * Hkv + h / group;
    const double* qi = q + row * D;
    const double* kb = k + kv_head * (int64_t)N * D;
    for (int64_t j = 0; j <= i; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qi[d] * kb[j * D + d];
        s[j] = tau * dot - alibi_penalty(slopes, h, i, j);
    }
    return i;
}

/* q [B,Hq,N,D], k, v [B,Hkv,N,D], dout [B,Hq,N,D], all fp64 and contiguous.
 * Writes dq [B,Hq,N,D], dk and dv [B,Hkv,N,D], and per query row its
 * log-sum-exp lse and Delta [B,Hq,N]. Three passes, each recomputing the
 * scores: (1) per query row, L_i and Delta_i; (2) per query row, dq_i;
 * (3) per key row j of each key head, dk_j and dv_j over the query rows
 * i >= j of every query head of its group. With slopes (one per query
 * head) the scores carry the ALiBi penalty of oracle_attn_alibi_rows; the
 * penalty does not depend on q, k or v, so the gradients keep their form
 * and only P changes. Returns 0, or -1 on bad arguments. */
static int attn_bwd(const double* q, const double* k, const double* v, const double* dout,
                    int B, int Hq, int Hkv, int N, int D, const double* slopes,
                    double* dq, double* dk, double* dv, double* lse, double* delta) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1 || Hq % Hkv != 0) return -1;
    const int64_t qrows = (int64_t)B * Hq * N;
    const int64_t krows = (int64_t)B * Hkv * N;
    const int group = Hq / Hkv;
    const double tau = pow((double)D, -0.5);
    int bad = 0;
    /* pass 1: L_i and Delta_i */
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 16)
        for (int64_t row = 0; row < qrows; ++row) {
            if (!s) { bad = 1; continue; }
            int64_t i = row_scores(q, k, Hq, Hkv, N, D, row, tau, slopes, s);
            int64_t bh = row / N;
            int64_t g = (bh % Hq) / group, b = bh / Hq;
            const double* vb = v + (b * Hkv + g) * (int64_t)N * D;
            const double* doi = dout + row * D;
            double M = -INFINITY;
            for (int64_t j = 0; j <= i; ++j)
                if (s[j] > M) M = s[j];
            double l = 0.0;
            for (int64_t j = 0; j <= i; ++j) l += exp(s[j] - M);
            double L = M + log(l);
            double dl = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                double dp = 0.0;
                for (int d = 0; d < D; ++d) dp += doi[d] * vb[j * D + d];
                dl += exp(s[j] - L) * dp;
            }
            lse[row] = L;
            delta[row] = dl;
        }
        free(s);
    }
    if (bad) return -1;
    /* pass 2: dq_i = tau sum_j P_ij (dP_ij - Delta_i) k_j */
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 16)
        for (int64_t row = 0; row < qrows; ++row) {
            if (!s) { bad = 1; continue; }
            int64_t i = row_scores(q, k, Hq, Hkv, N, D, row, tau, slopes, s);
            int64_t bh = row / N;
            int64_t g = (bh % Hq) / group, b = bh / Hq;
            const double* kb = k + (b * Hkv + g) * (int64_t)N * D;
            const double* vb = v + (b * Hkv + g) * (int64_t)N * D;
            const double* doi = dout + row * D;
            double* dqi = dq + row * D;
            for (int d = 0; d < D; ++d) dqi[d] = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                double dp = 0.0;
                for (int d = 0; d < D; ++d) dp += doi[d] * vb[j * D + d];
                double ds = exp(s[j] - lse[row]) * (dp - delta[row]);
                for (int d = 0; d < D; ++d) dqi[d] += tau * ds * kb[j * D + d];
            }
        }
        free(s);
    }
    if (bad) return -1;
    /* pass 3: dk_j = tau sum_{h, i >= j} dS_ij q_i, dv_j = sum_{h, i >= j} P_ij dO_i */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t krow = 0; krow < krows; ++krow) {
        int64_t j = krow % N;
        int64_t bg = krow / N;
        int64_t g = bg % Hkv, b = bg / Hkv;
        const double* kj = k + krow * D;
        const double* vj = v + krow * D;
        double* dkj = dk + krow * D;
        double* dvj = dv + krow * D;
        for (int d = 0; d < D; ++d) dkj[d] = dvj[d] = 0.0;
        for (int64_t h = g * group; h < (g + 1) * group; ++h) {
            for (int64_t i = j; i < N; ++i) {
                int64_t row = (b * Hq + h) * (int64_t)N + i;
                const double* qi = q + row * D;
                const double* doi = dout + row * D;
                double dot = 0.0, dp = 0.0;
                for (int d = 0; d < D; ++d) {
                    dot += qi[d] * kj[d];
                    dp += doi[d] * vj[d];
                }
                double p = exp(tau * dot - alibi_penalty(slopes, h, i, j) - lse[row]);
                double ds = p * (dp - delta[row]);
                for (int d = 0; d < D; ++d) {
                    dkj[d] += tau * ds * qi[d];
                    dvj[d] += p * doi[d];
                }
            }
        }
    }
    return 0;
}

int oracle_attn_bwd(const double* q, const double* k, const double* v, const double* dout,
                    int B, int Hq, int Hkv, int N, int D,
                    double* dq, double* dk, double* dv, double* lse, double* delta) {
    return attn_bwd(q, k, v, dout, B, Hq, Hkv, N, D, NULL, dq, dk, dv, lse, delta);
}

/* The backward of oracle_attn_alibi_rows (slopes: Hq values, required). */
int oracle_attn_alibi_bwd(const double* q, const double* k, const double* v, const double* dout,
                          int B, int Hq, int Hkv, int N, int D, const double* slopes,
                          double* dq, double* dk, double* dv, double* lse, double* delta) {
    if (!slopes) return -1;
    return attn_bwd(q, k, v, dout, B, Hq, Hkv, N, D, slopes, dq, dk, dv, lse, delta);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
