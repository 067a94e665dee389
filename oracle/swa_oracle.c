/*
 * swa_oracle.c -- plain fp64 CPU oracle for sliding-window attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent reference that the
 * GPU library is checked against.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * table or helper with the HIP library, and the HIP library never calls it.
 *
 * What it computes (all arithmetic in IEEE double):
 *
 *   For query row i of batch b and query head h, with kv head
 *   kh = h / (Hq / Hkv), the attended set S(i) is
 *     - Band(i) = { i + t*dil : -wl <= t <= wr } clipped to [0, N)
 *       (the window around each query, truncated at the sequence edges:
 *        bmjup.com "Sliding window attention", section "core principle /
 *        mathematical form"; the dilated index sets i +- t*d:
 *        mhpn.cn "Dilated sliding window", section 2 "structure comparison"),
 *     - united with every global position g (g <= i when causal), and
 *     - if i itself is global, every key j (j <= i when causal)
 *       (global tokens attend to all positions and all positions attend to
 *        them: aiqz.cc "Sliding window attention: Mistral", section
 *        "global attention tokens"; mhpn.cn section 3 "attention sink").
 *   The call is causal exactly when wr == 0 (a left-only window: bmjup.com,
 *   section "bidirectional vs unidirectional sliding window").
 *   S(i) is a set: a key that is both in the band and global counts once.
 *
 *     s_j   = scale * sum_c q[b,i,h,c] * k[b,j,kh,c]
 *     M     = max_{j in S(i)} s_j
 *     L     = sum_{j in S(i)} exp(s_j - M)
 *     out   = sum_{j in S(i)} exp(s_j - M) * v[b,j,kh,:] / L
 *     lse   = M + log(L)
 *   which is y_i = sum_j softmax(q_i.k_j / sqrt(d)) v_j over the window
 *   (bmjup.com, "mathematical form"), with the max subtracted before the
 *   exponential as in the numpy decode demo (aiqz.cc, "Python demo").
 *   Excluding a key is the same as giving it a score of -infinity before the
 *   softmax (bmjup.com, section 2 "mask implementation").
 *
 * Decode over a ring-buffer KV cache (intelliparadigm.com, section 3.1
 * "cache mechanism", the RingBuffer class: write at idx % size, then idx += 1;
 * aiqz.cc, "inference optimisation": the cache keeps only the last W entries):
 *   append writes slot ring_head, then ring_head = (ring_head + 1) % W and
 *   cache_len = min(cache_len + 1, W).  A decode step attends the new query
 *   over the valid slots { (ring_head - 1 - a) mod W : 0 <= a < cache_len },
 *   i.e. the last cache_len appended entries, the newest included (aiqz.cc
 *   demo: keys are the last window_size entries, current token included).
 *
 * Layouts (row-major): q,out [B,N,Hq,D]; k,v [B,N,Hkv,D]; lse [B,Hq,N];
 * decode q,out [B,Hq,D]; kcache,vcache [B,Hkv,W,D]; decode lse [B,Hq].
 * Element types of the inputs: 0 = float32, 1 = bfloat16 (raw 16-bit
 * patterns).  Values are widened to double exactly.
 *
 * Parity pins: see tests/test_oracle_pins.py (dense-mask brute force, the
 * dilated index sets printed on the dilated-window page, closed forms and
 * invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- element access: exact widening to double ------------------------ */

static double load_elem(const void* base, int dtype, int64_t idx) {
    if (dtype == 0) return (double)((const float*)base)[idx];
    /* bfloat16: the upper half of an IEEE float32 */
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static void copy_elem(void* dst, const void* src, int dtype, int64_t di, int64_t si) {
    if (dtype == 0) ((float*)dst)[di] = ((const float*)src)[si];
    else ((uint16_t*)dst)[di] = ((const uint16_t*)src)[si];
}

/* ---- the attended set S(i) ------------------------------------------- */

static int cmp_int64(const void* a, const void* b) {
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

/* Sorted, duplicate-free copy of the global positions.  Returns the count. */
static int64_t normalise_globals(const int32_t* g, int64_t ng, int64_t* out) {
    for (int64_t t = 0; t < ng; t++) out[t] = g[t];
    qsort(out, (size_t)ng, sizeof(int64_t), cmp_int64);
    int64_t m = 0;
    for (int64_t t = 0; t < ng; t++)
        if (m == 0 || out[t] != out[m - 1]) out[m++] = out[t];
    return m;
}

static int is_member(const int64_t* sorted, int64_t n, int64_t x) {
    for (int64_t t = 0; t < n; t++)
        if (sorted[t] == x) return 1;
    return 0;
}

/* Fills idx (capacity N) with S(i) in increasing order; returns |S(i)|. */
static int64_t attended_set(int64_t i, int64_t N, int64_t wl, int64_t wr, int64_t dil,
                            const int64_t* G, int64_t nG, int64_t* idx) {
    const int causal = (wr == 0);
    int64_t n = 0;
    if (is_member(G, nG, i)) {
        for (int64_t j = 0; j < N; j++)
            if (!causal || j <= i) idx[n++] = j;
        return n;
    }
    for (int64_t t = -wl; t <= wr; t++) {
        int64_t j = i + t * dil;
        if (j >= 0 && j < N) idx[n++] = j;
    }
    for (int64_t t = 0; t < nG; t++)
        if (!causal || G[t] <= i) idx[n++] = G[t];
    qsort(idx, (size_t)n, sizeof(int64_t), cmp_int64);
    int64_t m = 0;
    for (int64_t t = 0; t < n; t++)
        if (m == 0 || idx[t] != idx[m - 1]) idx[m++] = idx[t];
    return m;
}

/* Public: S(i) as int64 positions.  Returns |S(i)|, or -1 on bad input. */
int64_t oracle_attended_set(int64_t i, int64_t N, int64_t wl, int64_t wr, int64_t dil,
                            const int32_t* gidx, int64_t ng, int64_t* out_idx) {
    if (N <= 0 || i < 0 || i >= N || wl < 0 || wr < 0 || dil < 1 || ng < 0) return -1;
    int64_t* G = (int64_t*)malloc(sizeof(int64_t) * (size_t)(ng > 0 ? ng : 1));
    int64_t nG = normalise_globals(gidx, ng, G);
    int64_t n = attended_set(i, N, wl, wr, dil, G, nG, out_idx);
    free(G);
    return n;
}

/* ---- one softmax-attention row over an explicit key list ------------- */

/* qrow: pointer-free access through (base, dtype, offset, stride 1).
 * Keys/values: element (j, c) at kbase + j*kstride + c. */
static void attend_row(const void* q, int64_t qoff, const void* k, const void* v,
                       int64_t kvoff, int64_t kvstride, int dtype, int64_t D,
                       const int64_t* keys, int64_t nkeys, double scale,
                       double* s /* scratch, nkeys */, double* out, double* lse) {
    double M = -INFINITY;
    for (int64_t t = 0; t < nkeys; t++) {
        double dot = 0.0;
        int64_t ko = kvoff + keys[t] * kvstride;
        for (int64_t c = 0; c < D; c++)
            dot += load_elem(q, dtype, qoff + c) * load_elem(k, dtype, ko + c);
        s[t] = scale * dot;
        if (s[t] > M) M = s[t];
    }
    double L = 0.0;
    for (int64_t c = 0; c < D; c++) out[c] = 0.0;
    for (int64_t t = 0; t < nkeys; t++) {
        double p = exp(s[t] - M);
        L += p;
        int64_t vo = kvoff + keys[t] * kvstride;
        for (int64_t c = 0; c < D; c++) out[c] += p * load_elem(v, dtype, vo + c);
    }
    for (int64_t c = 0; c < D; c++) out[c] /= L;
    *lse = M + log(L);
}

/* ---- forward --------------------------------------------------------- */

static int fwd_args_ok(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
                       int64_t wl, int64_t wr, int64_t dil, int dtype) {
    return B > 0 && Hq > 0 && Hkv > 0 && N > 0 && D > 0 && Hq % Hkv == 0 &&
           wl >= 0 && wr >= 0 && dil >= 1 && (dtype == 0 || dtype == 1);
}

/* Computes rows (b, h, i) listed in rows[3*r .. 3*r+2] into
 * out_rows[r*D .. r*D+D-1] and lse_rows[r].  Returns 0, or -1 on bad input. */
int oracle_fwd_rows(const void* q, const void* k, const void* v, int dtype,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
                    int64_t wl, int64_t wr, int64_t dil,
                    const int32_t* gidx, int64_t ng, double scale,
                    const int64_t* rows, int64_t n_rows,
                    double* out_rows, double* lse_rows) {
    if (!fwd_args_ok(B, Hq, Hkv, N, D, wl, wr, dil, dtype)) return -1;
    for (int64_t t = 0; t < ng; t++)
        if (gidx[t] < 0 || gidx[t] >= N) return -1;
    for (int64_t r = 0; r < n_rows; r++)
        if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 ||
            rows[3 * r + 1] >= Hq || rows[3 * r + 2] < 0 || rows[3 * r + 2] >= N)
            return -1;
    int64_t* G = (int64_t*)malloc(sizeof(int64_t) * (size_t)(ng > 0 ? ng : 1));
    int64_t nG = normalise_globals(gidx, ng, G);
    const int64_t group = Hq / Hkv;

#pragma omp parallel
    {
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N + wl + wr + nG + 1));
        double* s = (double*)malloc(sizeof(double) * (size_t)(N + wl + wr + nG + 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; r++) {
            int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            int64_t kh = h / group;
            int64_t nk = attended_set(i, N, wl, wr, dil, G, nG, keys);
            int64_t qoff = ((b * N + i) * Hq + h) * D;
            int64_t kvoff = (b * N * Hkv + kh) * D; /* key j at kvoff + j*Hkv*D */
            attend_row(q, qoff, k, v, kvoff, Hkv * D, dtype, D, keys, nk, scale, s,
                       out_rows + r * D, lse_rows + r);
        }
        free(keys);
        free(s);
    }
    free(G);
    return 0;
}

/* All rows: out [B,N,Hq,D] and lse [B,Hq,N] in double. */
int oracle_fwd(const void* q, const void* k, const void* v, int dtype,
               int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
               int64_t wl, int64_t wr, int64_t dil,
               const int32_t* gidx, int64_t ng, double scale,
               double* out, double* lse) {
    if (!fwd_args_ok(B, Hq, Hkv, N, D, wl, wr, dil, dtype)) return -1;
    int64_t n_rows = B * N * Hq;
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * 3 * (size_t)n_rows);
    double* lse_rows = (double*)malloc(sizeof(double) * (size_t)n_rows);
    /* row order (b, i, h) matches the out layout [B,N,Hq,D] */
    int64_t r = 0;
    for (int64_t b = 0; b < B; b++)
        for (int64_t i = 0; i < N; i++)
            for (int64_t h = 0; h < Hq; h++) {
                rows[3 * r] = b; rows[3 * r + 1] = h; rows[3 * r + 2] = i; r++;
            }
    int rc = oracle_fwd_rows(q, k, v, dtype, B, Hq, Hkv, N, D, wl, wr, dil, gidx, ng,
                             scale, rows, n_rows, out, lse_rows);
    if (rc == 0)
        for (r = 0; r < n_rows; r++) {
            int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            lse[(b * Hq + h) * N + i] = lse_rows[r];
        }
    free(rows);
    free(lse_rows);
    return rc;
}

/* ---- backward ---------------------------------------------------------- */

/* Gradients of the forward above for an upstream gradient dout [B,N,Hq,D]
 * (the training use of the window attention: bmjup.com Q&A "training vs
 * inference"; intelliparadigm.com section 5.1, blocked computation and
 * mixed-precision training with a backward pass).  With
 * P_ij = exp(s_ij - M_i) / L_i over j in S(i) and dP_ij = dout_i . v_j:
 *   dv_j += P_ij dout_i
 *   dS_ij = P_ij (dP_ij - sum_{j' in S(i)} P_ij' dP_ij')
 *   dq_i  = scale sum_j dS_ij k_j,   dk_j += scale dS_ij q_i
 * (the chain rule through s = scale q.k, softmax and the weighted sum; a kv
 * head collects the terms of every query head that reads it).  dq [B,N,Hq,D],
 * dk, dv [B,N,Hkv,D] in double. */
int oracle_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
               int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
               int64_t wl, int64_t wr, int64_t dil, const int32_t* gidx, int64_t ng,
               double scale, double* dq, double* dk, double* dv) {
    if (!fwd_args_ok(B, Hq, Hkv, N, D, wl, wr, dil, dtype)) return -1;
    for (int64_t t = 0; t < ng; t++)
        if (gidx[t] < 0 || gidx[t] >= N) return -1;
    int64_t* G = (int64_t*)malloc(sizeof(int64_t) * (size_t)(ng > 0 ? ng : 1));
    int64_t nG = normalise_globals(gidx, ng, G);
    const int64_t group = Hq / Hkv;
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N + wl + wr + nG + 1));
    double* p = (double*)malloc(sizeof(double) * (size_t)(N + wl + wr + nG + 1));
    double* dp = (double*)malloc(sizeof(double) * (size_t)(N + wl + wr + nG + 1));
    for (int64_t x = 0; x < B * N * Hkv * D; x++) dk[x] = dv[x] = 0.0;
    /* serial over rows: dk and dv are sums over many rows */
    for (int64_t b = 0; b < B; b++)
        for (int64_t h = 0; h < Hq; h++)
            for (int64_t i = 0; i < N; i++) {
                const int64_t kh = h / group;
                const int64_t nk = attended_set(i, N, wl, wr, dil, G, nG, keys);
                const int64_t qo = ((b * N + i) * Hq + h) * D;
                double M = -INFINITY;
                for (int64_t t = 0; t < nk; t++) {
                    const int64_t ko = ((b * N + keys[t]) * Hkv + kh) * D;
                    double dot = 0.0;
                    for (int64_t c = 0; c < D; c++)
                        dot += load_elem(q, dtype, qo + c) * load_elem(k, dtype, ko + c);
                    p[t] = scale * dot;
                    if (p[t] > M) M = p[t];
                }
                double L = 0.0;
                for (int64_t t = 0; t < nk; t++) {
                    p[t] = exp(p[t] - M);
                    L += p[t];
                }
                double rowdot = 0.0; /* sum_j P_ij dP_ij */
                for (int64_t t = 0; t < nk; t++) {
                    p[t] /= L;
                    const int64_t vo = ((b * N + keys[t]) * Hkv + kh) * D;
                    double d = 0.0;
                    for (int64_t c = 0; c < D; c++)
                        d += load_elem(dout, dtype, qo + c) * load_elem(v, dtype, vo + c);
                    dp[t] = d;
                    rowdot += p[t] * d;
                }
                for (int64_t c = 0; c < D; c++) dq[qo + c] = 0.0;
                for (int64_t t = 0; t < nk; t++) {
                    const int64_t ko = ((b * N + keys[t]) * Hkv + kh) * D;
                    const double ds = p[t] * (dp[t] - rowdot);
                    for (int64_t c = 0; c < D; c++) {
                        dq[qo + c] += scale * ds * load_elem(k, dtype, ko + c);
                        dk[ko + c] += scale * ds * load_elem(q, dtype, qo + c);
                        dv[ko + c] += p[t] * load_elem(dout, dtype, qo + c);
                    }
                }
            }
    free(keys);
    free(p);
    free(dp);
    free(G);
    return 0;
}

/* Softmax weights and dP of one query row over its attended set: fills
 * keys[0..n), p (normalised weights) and dp; returns n and the row term
 * sum_j p_j dp_j in *rowdot.  Helper of the sampled backward below. */
static int64_t bwd_row(const void* q, const void* k, const void* v, const void* dout, int dtype,
                       int64_t b, int64_t h, int64_t i, int64_t N, int64_t Hq, int64_t Hkv,
                       int64_t D, int64_t wl, int64_t wr, int64_t dil, const int64_t* G,
                       int64_t nG, double scale, int64_t* keys, double* p, double* dp,
                       double* rowdot) {
    const int64_t kh = h / (Hq / Hkv);
    const int64_t nk = attended_set(i, N, wl, wr, dil, G, nG, keys);
    const int64_t qo = ((b * N + i) * Hq + h) * D;
    double M = -INFINITY;
    for (int64_t t = 0; t < nk; t++) {
        const int64_t ko = ((b * N + keys[t]) * Hkv + kh) * D;
        double dot = 0.0, g = 0.0;
        for (int64_t c = 0; c < D; c++) {
            dot += load_elem(q, dtype, qo + c) * load_elem(k, dtype, ko + c);
            g += load_elem(dout, dtype, qo + c) * load_elem(v, dtype, ko + c);
        }
        p[t] = scale * dot;
        dp[t] = g;
        if (p[t] > M) M = p[t];
    }
    double L = 0.0;
    for (int64_t t = 0; t < nk; t++) {
        p[t] = exp(p[t] - M);
        L += p[t];
    }
    double rd = 0.0;
    for (int64_t t = 0; t < nk; t++) {
        p[t] /= L;
        rd += p[t] * dp[t];
    }
    *rowdot = rd;
    return nk;
}

/* dq of the listed query rows (b, h, i) only: out_rows[r*D .. r*D+D-1]. */
int oracle_bwd_dq_rows(const void* q, const void* k, const void* v, const void* dout, int dtype,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int64_t wl,
                       int64_t wr, int64_t dil, const int32_t* gidx, int64_t ng, double scale,
                       const int64_t* rows, int64_t n_rows, double* out_rows) {
    if (!fwd_args_ok(B, Hq, Hkv, N, D, wl, wr, dil, dtype)) return -1;
    for (int64_t t = 0; t < ng; t++)
        if (gidx[t] < 0 || gidx[t] >= N) return -1;
    for (int64_t r = 0; r < n_rows; r++)
        if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 ||
            rows[3 * r + 1] >= Hq || rows[3 * r + 2] < 0 || rows[3 * r + 2] >= N)
            return -1;
    int64_t* G = (int64_t*)malloc(sizeof(int64_t) * (size_t)(ng > 0 ? ng : 1));
    int64_t nG = normalise_globals(gidx, ng, G);
#pragma omp parallel
    {
        const size_t cap = (size_t)(N + wl + wr + nG + 1);
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * cap);
        double* p = (double*)malloc(sizeof(double) * cap);
        double* dp = (double*)malloc(sizeof(double) * cap);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; r++) {
            const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            double rowdot;
            const int64_t nk = bwd_row(q, k, v, dout, dtype, b, h, i, N, Hq, Hkv, D, wl, wr, dil,
                                       G, nG, scale, keys, p, dp, &rowdot);
            double* o = out_rows + r * D;
            for (int64_t c = 0; c < D; c++) o[c] = 0.0;
            const int64_t kh = h / (Hq / Hkv);
            for (int64_t t = 0; t < nk; t++) {
                const int64_t ko = ((b * N + keys[t]) * Hkv + kh) * D;
                const double dsq = p[t] * (dp[t] - rowdot);
                for (int64_t c = 0; c < D; c++) o[c] += scale * dsq * load_elem(k, dtype, ko + c);
            }
        }
        free(keys);
        free(p);
        free(dp);
    }
    free(G);
    return 0;
}

/* dk and dv of the listed keys (b, kv head, j) only: every query row i of the
 * kv head's query heads whose attended set holds j contributes; rows are
 * scanned over [0, N) (the set test decides).  dk_rows, dv_rows [r*D ..]. */
int oracle_bwd_dkv_keys(const void* q, const void* k, const void* v, const void* dout, int dtype,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int64_t wl,
                        int64_t wr, int64_t dil, const int32_t* gidx, int64_t ng, double scale,
                        const int64_t* sel, int64_t n_sel, double* dk_rows, double* dv_rows) {
    if (!fwd_args_ok(B, Hq, Hkv, N, D, wl, wr, dil, dtype)) return -1;
    for (int64_t t = 0; t < ng; t++)
        if (gidx[t] < 0 || gidx[t] >= N) return -1;
    for (int64_t r = 0; r < n_sel; r++)
        if (sel[3 * r] < 0 || sel[3 * r] >= B || sel[3 * r + 1] < 0 || sel[3 * r + 1] >= Hkv ||
            sel[3 * r + 2] < 0 || sel[3 * r + 2] >= N)
            return -1;
    int64_t* G = (int64_t*)malloc(sizeof(int64_t) * (size_t)(ng > 0 ? ng : 1));
    int64_t nG = normalise_globals(gidx, ng, G);
    const int64_t group = Hq / Hkv;
    for (int64_t r = 0; r < n_sel; r++) {
        double* dkr = dk_rows + r * D;
        double* dvr = dv_rows + r * D;
        for (int64_t c = 0; c < D; c++) dkr[c] = dvr[c] = 0.0;
    }
    for (int64_t r = 0; r < n_sel; r++) {
        const int64_t b = sel[3 * r], kh = sel[3 * r + 1], j = sel[3 * r + 2];
        double* dkr = dk_rows + r * D;
        double* dvr = dv_rows + r * D;
#pragma omp parallel
        {
            const size_t cap = (size_t)(N + wl + wr + nG + 1);
            int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * cap);
            double* p = (double*)malloc(sizeof(double) * cap);
            double* dp = (double*)malloc(sizeof(double) * cap);
            double* dk_l = (double*)calloc((size_t)D, sizeof(double));
            double* dv_l = (double*)calloc((size_t)D, sizeof(double));
#pragma omp for schedule(dynamic, 16)
            for (int64_t x = 0; x < group * N; x++) {
                const int64_t h = kh * group + x / N, i = x % N;
                /* cheap pre-test: is j in S(i)?  (globals make any row possible) */
                int64_t ks_tmp_n;
                int in = 0;
                {
                    const int64_t dj = j - i;
                    if (dj % dil == 0 && dj / dil >= -wl && dj / dil <= wr) in = 1;
                }
                if (!in && nG == 0) continue;
                double rowdot;
                ks_tmp_n = bwd_row(q, k, v, dout, dtype, b, h, i, N, Hq, Hkv, D, wl, wr, dil, G,
                                   nG, scale, keys, p, dp, &rowdot);
                for (int64_t t = 0; t < ks_tmp_n; t++) {
                    if (keys[t] != j) continue;
                    const int64_t qo = ((b * N + i) * Hq + h) * D;
                    const double dsk = p[t] * (dp[t] - rowdot);
                    for (int64_t c = 0; c < D; c++) {
                        dk_l[c] += scale * dsk * load_elem(q, dtype, qo + c);
                        dv_l[c] += p[t] * load_elem(dout, dtype, qo + c);
                    }
                }
            }
#pragma omp critical
            for (int64_t c = 0; c < D; c++) {
                dkr[c] += dk_l[c];
                dvr[c] += dv_l[c];
            }
            free(keys);
            free(p);
            free(dp);
            free(dk_l);
            free(dv_l);
        }
    }
    free(G);
    return 0;
}

/* ---- ring-buffer KV cache -------------------------------------------- */

/* Appends k_new, v_new [B,Hkv,D] into kcache, vcache [B,Hkv,W,D] (element type
 * dtype) at slot ring_head[b], then advances ring_head and cache_len. */
int oracle_kv_append(void* kcache, void* vcache, const void* k_new, const void* v_new,
                     int64_t* ring_head, int64_t* cache_len,
                     int64_t B, int64_t Hkv, int64_t W, int64_t D, int dtype) {
    if (B <= 0 || Hkv <= 0 || W <= 0 || D <= 0 || (dtype != 0 && dtype != 1)) return -1;
    for (int64_t b = 0; b < B; b++) {
        if (ring_head[b] < 0 || ring_head[b] >= W || cache_len[b] < 0 || cache_len[b] > W)
            return -1;
        int64_t slot = ring_head[b];
        for (int64_t h = 0; h < Hkv; h++)
            for (int64_t c = 0; c < D; c++) {
                int64_t di = ((b * Hkv + h) * W + slot) * D + c;
                int64_t si = (b * Hkv + h) * D + c;
                copy_elem(kcache, k_new, dtype, di, si);
                copy_elem(vcache, v_new, dtype, di, si);
            }
        ring_head[b] = (slot + 1) % W;
        cache_len[b] = cache_len[b] + 1 < W ? cache_len[b] + 1 : W;
    }
    return 0;
}

/* One decode step for every (b, h): q [B,Hq,D] over the valid ring slots.
 * out [B,Hq,D] and lse [B,Hq] in double.  Rows with cache_len == 0 have no
 * keys; they are reported as an error (-1). */
int oracle_decode(const void* q, const void* kcache, const void* vcache, int dtype,
                  const int64_t* ring_head, const int64_t* cache_len,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t W, int64_t D, double scale,
                  double* out, double* lse) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || W <= 0 || D <= 0 ||
        (dtype != 0 && dtype != 1))
        return -1;
    for (int64_t b = 0; b < B; b++)
        if (ring_head[b] < 0 || ring_head[b] >= W || cache_len[b] < 1 || cache_len[b] > W)
            return -1;
    const int64_t group = Hq / Hkv;
#pragma omp parallel
    {
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)W);
        double* s = (double*)malloc(sizeof(double) * (size_t)W);
#pragma omp for schedule(static)
        for (int64_t bh = 0; bh < B * Hq; bh++) {
            int64_t b = bh / Hq, h = bh % Hq, kh = h / group;
            int64_t n = cache_len[b];
            for (int64_t a = 0; a < n; a++) keys[a] = ((ring_head[b] - 1 - a) % W + W) % W;
            int64_t qoff = (b * Hq + h) * D;
            int64_t kvoff = (b * Hkv + kh) * W * D; /* slot j at kvoff + j*D */
            attend_row(q, qoff, kcache, vcache, kvoff, D, dtype, D, keys, n, scale, s,
                       out + bh * D, lse + bh);
        }
        free(keys);
        free(s);
    }
    return 0;
}

/* ---- chunked prefill over the ring ----------------------------------- */

/* Appends a chunk of n tokens, k, v [B,n,Hkv,D], to the ring: the same state
 * as n single appends in token order (intelliparadigm.com, section 3.1, the
 * RingBuffer class).  Token t lands in slot (ring_head + t) mod W; when n > W
 * only the last W tokens survive, the older ones being overwritten within the
 * chunk (aiqz.cc, "inference optimisation": the cache rolls, keeping only the
 * last W entries).  Then ring_head advances by n (mod W) and cache_len grows
 * by n, capped at W.  n == 0 changes nothing. */
int oracle_kv_append_chunk(void* kcache, void* vcache, const void* k, const void* v,
                           int64_t* ring_head, int64_t* cache_len,
                           int64_t B, int64_t Hkv, int64_t W, int64_t n, int64_t D, int dtype) {
    if (B <= 0 || Hkv <= 0 || W <= 0 || D <= 0 || n < 0 || (dtype != 0 && dtype != 1))
        return -1;
    for (int64_t b = 0; b < B; b++)
        if (ring_head[b] < 0 || ring_head[b] >= W || cache_len[b] < 0 || cache_len[b] > W)
            return -1;
    const int64_t first = n > W ? n - W : 0; /* older tokens would be overwritten */
    for (int64_t b = 0; b < B; b++) {
        for (int64_t t = first; t < n; t++) {
            int64_t slot = (ring_head[b] + t) % W;
            for (int64_t h = 0; h < Hkv; h++)
                for (int64_t c = 0; c < D; c++) {
                    int64_t di = ((b * Hkv + h) * W + slot) * D + c;
                    int64_t si = ((b * n + t) * Hkv + h) * D + c;
                    copy_elem(kcache, k, dtype, di, si);
                    copy_elem(vcache, v, dtype, di, si);
                }
        }
        ring_head[b] = (ring_head[b] + n) % W;
        cache_len[b] = cache_len[b] + n < W ? cache_len[b] + n : W;
    }
    return 0;
}

/* Causal sliding-window attention of a prompt chunk that follows the tokens
 * held in the ring (streaming inference: aiqz.cc, "inference optimisation",
 * third strategy; bmjup.com, Q&A "training vs inference": at inference only
 * the window's keys and values are kept).
 *
 * The chunk holds n tokens: q [B,n,Hq,D], k, v [B,n,Hkv,D].  Let P be the
 * position of chunk token 0; the ring of sequence b holds the cache_len[b]
 * tokens before it, the one of age a (a = 0 newest) at position P - 1 - a in
 * slot (ring_head[b] - 1 - a) mod W.  Query t of the chunk (position P + t)
 * attends to every available key at positions P + t - wl .. P + t:
 *   ring tokens of age a < cache_len[b] with a <= wl - 1 - t, and
 *   chunk tokens j with max(0, t - wl) <= j <= t.
 * out [B,n,Hq,D] and lse [B,Hq,n] in double.  Requires wl <= W, so that no
 * key the window asks for could have been evicted while a ring slot was
 * still free. */
int oracle_fwd_cached(const void* q, const void* k, const void* v, const void* kcache,
                      const void* vcache, int dtype, const int64_t* ring_head,
                      const int64_t* cache_len, int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                      int64_t W, int64_t D, int64_t wl, double scale, double* out,
                      double* lse) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || n <= 0 || W <= 0 || D <= 0 ||
        wl < 0 || wl > W || (dtype != 0 && dtype != 1))
        return -1;
    for (int64_t b = 0; b < B; b++)
        if (ring_head[b] < 0 || ring_head[b] >= W || cache_len[b] < 0 || cache_len[b] > W)
            return -1;
    const int64_t group = Hq / Hkv;
    const int64_t cap = W + wl + 1; /* room for every ring slot and window key */
    const size_t esz = dtype == 0 ? 4 : 2;
#pragma omp parallel
    {
        /* the query's keys and values gathered in attention order (exact
         * copies of the stored elements), then one softmax row over them */
        void* kt = malloc(esz * (size_t)(cap * D));
        void* vt = malloc(esz * (size_t)(cap * D));
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
        double* s = (double*)malloc(sizeof(double) * (size_t)cap);
        for (int64_t t = 0; t < cap; t++) keys[t] = t;
#pragma omp for schedule(dynamic, 8)
        for (int64_t row = 0; row < B * n * Hq; row++) {
            int64_t nk = 0;
            int64_t h = row % Hq, t = (row / Hq) % n, b = row / (Hq * n), kh = h / group;
            /* ring part, oldest first: ages a = a_max .. 0 */
            int64_t a_max = wl - 1 - t;
            if (a_max > cache_len[b] - 1) a_max = cache_len[b] - 1;
            for (int64_t a = a_max; a >= 0; a--) {
                int64_t slot = ((ring_head[b] - 1 - a) % W + W) % W;
                int64_t base = ((b * Hkv + kh) * W + slot) * D;
                for (int64_t c = 0; c < D; c++) {
                    copy_elem(kt, kcache, dtype, nk * D + c, base + c);
                    copy_elem(vt, vcache, dtype, nk * D + c, base + c);
                }
                nk++;
            }
            /* chunk part */
            for (int64_t j = t - wl > 0 ? t - wl : 0; j <= t; j++) {
                int64_t base = ((b * n + j) * Hkv + kh) * D;
                for (int64_t c = 0; c < D; c++) {
                    copy_elem(kt, k, dtype, nk * D + c, base + c);
                    copy_elem(vt, v, dtype, nk * D + c, base + c);
                }
                nk++;
            }
            attend_row(q, ((b * n + t) * Hq + h) * D, kt, vt, 0, D, dtype, D, keys, nk, scale,
                       s, out + ((b * n + t) * Hq + h) * D, lse + (b * Hq + h) * n + t);
        }
        free(kt);
        free(vt);
        free(keys);
        free(s);
    }
    return 0;
}

/* ---- decode with attention-sink slots ------------------------------------ */

/* One decode step over the ring plus n_sink pinned entries (mhpn.cn "Dilated
 * sliding window", section 3: keep the first tokens as attention-sink anchors;
 * aiqz.cc "global attention tokens": some tokens stay visible to every later
 * token).  ksink, vsink [B,Hkv,n_sink,D] hold the first n_sink tokens of each
 * sequence, which never enter the ring (it holds the tokens after them) and
 * are never evicted.  Query (b, h) attends the cache_len[b] valid ring slots
 * and all n_sink sink entries.  out [B,Hq,D], lse [B,Hq] in double.  A row with
 * no key at all (cache_len == 0 and n_sink == 0) is an error (-1). */
int oracle_decode_sinks(const void* q, const void* kcache, const void* vcache,
                        const void* ksink, const void* vsink, int64_t n_sink, int dtype,
                        const int64_t* ring_head, const int64_t* cache_len, int64_t B,
                        int64_t Hq, int64_t Hkv, int64_t W, int64_t D, double scale,
                        double* out, double* lse) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || W <= 0 || D <= 0 || n_sink < 0 ||
        (dtype != 0 && dtype != 1))
        return -1;
    for (int64_t b = 0; b < B; b++)
        if (ring_head[b] < 0 || ring_head[b] >= W || cache_len[b] < 0 || cache_len[b] > W ||
            cache_len[b] + n_sink < 1)
            return -1;
    const int64_t group = Hq / Hkv;
    const int64_t cap = W + n_sink;
    const size_t esz = dtype == 0 ? 4 : 2;
#pragma omp parallel
    {
        void* kt = malloc(esz * (size_t)(cap * D));
        void* vt = malloc(esz * (size_t)(cap * D));
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
        double* s = (double*)malloc(sizeof(double) * (size_t)cap);
        for (int64_t t = 0; t < cap; t++) keys[t] = t;
#pragma omp for schedule(static)
        for (int64_t bh = 0; bh < B * Hq; bh++) {
            int64_t nk = 0;
            const int64_t b = bh / Hq, kh = (bh % Hq) / group;
            for (int64_t t = 0; t < n_sink; t++) { /* the pinned entries */
                const int64_t base = ((b * Hkv + kh) * n_sink + t) * D;
                for (int64_t c = 0; c < D; c++) {
                    copy_elem(kt, ksink, dtype, nk * D + c, base + c);
                    copy_elem(vt, vsink, dtype, nk * D + c, base + c);
                }
                nk++;
            }
            for (int64_t a = 0; a < cache_len[b]; a++) { /* the valid ring slots */
                const int64_t slot = ((ring_head[b] - 1 - a) % W + W) % W;
                const int64_t base = ((b * Hkv + kh) * W + slot) * D;
                for (int64_t c = 0; c < D; c++) {
                    copy_elem(kt, kcache, dtype, nk * D + c, base + c);
                    copy_elem(vt, vcache, dtype, nk * D + c, base + c);
                }
                nk++;
            }
            attend_row(q, bh * D, kt, vt, 0, D, dtype, D, keys, nk, scale, s, out + bh * D,
                       lse + bh);
        }
        free(kt);
        free(vt);
        free(keys);
        free(s);
    }
    return 0;
}

/* ---- paged window cache ------------------------------------------------- */

/* A shared pool of pages kpool, vpool [n_pages, Hkv, P, D]; a page holds P
 * consecutive positions of one sequence for every kv head.  Sequence b keeps a
 * circular block table of nb entries: position t lives in page
 * block_table[b*nb + (t / P) % nb], slot t % P.  With nb*P >= W + P - 1 the
 * blocks that intersect the last W positions have distinct table entries, so
 * a table entry can be re-pointed (its old page released to the pool) once
 * its block has left the window (mhpn.cn "Dilated sliding window", section 4,
 * KV-cache management: out-of-window entries freed page by page;
 * intelliparadigm.com, section 6: pre-allocated memory pool, cache updates
 * without copies).  seq_len[b] counts the tokens appended so far. */

/* Appends n tokens, k, v [B,n,Hkv,D], at positions seq_len[b] .. seq_len[b]+n-1.
 * Only the last min(n, W) of them are written (older ones are out of every
 * later window); the table entries of their blocks must already point to the
 * pages the caller assigned.  Then seq_len[b] += n. */
int oracle_kv_append_paged(void* kpool, void* vpool, const void* k, const void* v,
                           const int32_t* block_table, int64_t nb, int64_t P, int64_t n_pages,
                           int64_t* seq_len, int64_t B, int64_t Hkv, int64_t W, int64_t n,
                           int64_t D, int dtype) {
    if (B <= 0 || Hkv <= 0 || W <= 0 || P <= 0 || nb <= 0 || nb * P < W + P - 1 || n < 0 ||
        D <= 0 || (dtype != 0 && dtype != 1))
        return -1;
    for (int64_t b = 0; b < B; b++) {
        if (seq_len[b] < 0) return -1;
        const int64_t first = n > W ? n - W : 0;
        for (int64_t t = first; t < n; t++) {
            const int64_t pos = seq_len[b] + t;
            const int64_t page = block_table[b * nb + (pos / P) % nb];
            if (page < 0 || page >= n_pages) return -1;
            for (int64_t h = 0; h < Hkv; h++)
                for (int64_t c = 0; c < D; c++) {
                    int64_t di = ((page * Hkv + h) * P + pos % P) * D + c;
                    int64_t si = ((b * n + t) * Hkv + h) * D + c;
                    copy_elem(kpool, k, dtype, di, si);
                    copy_elem(vpool, v, dtype, di, si);
                }
        }
        seq_len[b] += n;
    }
    return 0;
}

/* One decode step: query (b, h) attends positions max(0, L - W) .. L - 1 of
 * sequence b (L = seq_len[b], the newest token included), fetched through
 * the block table.  out [B,Hq,D], lse [B,Hq] in double; L == 0 is an error. */
int oracle_decode_paged(const void* q, const void* kpool, const void* vpool, int dtype,
                        const int32_t* block_table, int64_t nb, int64_t P, int64_t n_pages,
                        const int64_t* seq_len, int64_t B, int64_t Hq, int64_t Hkv, int64_t W,
                        int64_t D, double scale, double* out, double* lse) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || W <= 0 || P <= 0 || nb <= 0 ||
        nb * P < W + P - 1 || D <= 0 || (dtype != 0 && dtype != 1))
        return -1;
    for (int64_t b = 0; b < B; b++) {
        if (seq_len[b] < 1) return -1;
        for (int64_t pos = seq_len[b] > W ? seq_len[b] - W : 0; pos < seq_len[b]; pos++) {
            const int64_t page = block_table[b * nb + (pos / P) % nb];
            if (page < 0 || page >= n_pages) return -1;
        }
    }
    const int64_t group = Hq / Hkv;
    const size_t esz = dtype == 0 ? 4 : 2;
#pragma omp parallel
    {
        void* kt = malloc(esz * (size_t)(W * D));
        void* vt = malloc(esz * (size_t)(W * D));
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)W);
        double* s = (double*)malloc(sizeof(double) * (size_t)W);
        for (int64_t t = 0; t < W; t++) keys[t] = t;
#pragma omp for schedule(static)
        for (int64_t bh = 0; bh < B * Hq; bh++) {
            const int64_t bb = bh / Hq, kvh = (bh % Hq) / group;
            int64_t nk = 0;
            for (int64_t pos = seq_len[bb] > W ? seq_len[bb] - W : 0; pos < seq_len[bb]; pos++) {
                const int64_t page = block_table[bb * nb + (pos / P) % nb];
                const int64_t base = ((page * Hkv + kvh) * P + pos % P) * D;
                for (int64_t c = 0; c < D; c++) {
                    copy_elem(kt, kpool, dtype, nk * D + c, base + c);
                    copy_elem(vt, vpool, dtype, nk * D + c, base + c);
                }
                nk++;
            }
            attend_row(q, bh * D, kt, vt, 0, D, dtype, D, keys, nk, scale, s, out + bh * D,
                       lse + bh);
        }
        free(kt);
        free(vt);
        free(keys);
        free(s);
    }
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
