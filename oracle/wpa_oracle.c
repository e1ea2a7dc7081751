/*
 * wpa_oracle.c -- plain, slow, fp64 CPU oracle for per-RoPE-wavelength windowed
 * causal attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the package smoke check and the bench's CPU-baseline
 * leg do.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (ATFlash abstract, "Per-RoPE-Wavelength Attention Windows",
 * and WavePrune, "One period is often enough for RoPE", original abstract):
 *   - the RoPE attention score is an exact sum over 2-D rotation frequency
 *     pairs (ATFlash abstract, first sentence);
 *   - pair i has wavelength lambda_i = 2*pi*base^(2i/d), one full rotation
 *     period (WavePrune abstract: each channel kept for its first rotation
 *     period); its query-key term is kept only while the query-key distance
 *     is at most alpha*lambda_i (ATFlash abstract: terms farther than a
 *     distance proportional to the wavelength are dropped);
 *   - a pruned term contributes zero but the key stays in the softmax
 *     (ATFlash abstract: no key becomes unreachable, unlike a sliding window);
 *   - the softmax over the windowed logits is ordinary (ATFlash abstract: the
 *     online-softmax recurrences are not modified).
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   - pair i is made of head dims i and i + d/2 ("half-split" layout);
 *   - the window edge is inclusive: |dt| <= alpha*lambda_i keeps the term;
 *   - alpha*lambda_i is evaluated in IEEE double as
 *       alpha * ((2.0*M_PI) * pow(base, (2.0*i)/d));
 *   - logits are scaled by `scale` (1/sqrt(d) by default) after the windowed sum;
 *   - causality is by token index: key c is visible to query r iff c <= r;
 *   - q head h reads kv head h / (Hq/Hkv);
 *   - rotation: x'_i = x_i cos(t th_i) - x_{i+P} sin(t th_i),
 *               x'_{i+P} = x_{i+P} cos(t th_i) + x_i sin(t th_i),
 *     th_i = base^(-2i/d), angle formed in double, libm cos/sin;
 *   - decode: the one query sits at token index kv_len-1 (its own key included).
 *
 * RoPE variants (the `_ex` entry points): a caller-given frequency table th_i
 * (frequency-scaled RoPE, e.g. Llama-3 style, carries its own per-pair
 * frequencies), with wavelength lambda_i = 2*pi/th_i evaluated in IEEE double as
 * alpha * ((2.0*M_PI) / th_i); and the interleaved pair layout, pair i = dims
 * (2i, 2i+1), rotated by the same formulas.
 *
 * Per-head frequencies (AdaRoPE, on the cards page: rotation frequencies chosen per
 * head): with n_tables = Hkv the table is [Hkv][d/2] and kv head g, with the q heads that
 * read it (h / (Hq/Hkv) = g), rotates and windows by its own row, lambda_{g,i} =
 * 2*pi/th_{g,i}.  n_tables = 0 or 1 is the shared table (or base) above.
 *
 * Inputs are the exact values the GPU consumes (bf16 bit patterns as uint16, or
 * fp32); step 1 upcasts them to double.  All arithmetic is double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BF16 0
#define ORC_FP32 1

/* Step 1: exact upcast of one input element. */
static double orc_load(const void* base_ptr, int dtype, int64_t idx) {
    if (dtype == ORC_FP32) return (double)((const float*)base_ptr)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t*)base_ptr)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* The two head dims of pair i: (i, i + d/2) half-split, (2i, 2i + 1) interleaved. */
static int orc_dim_x(int i, int d, int interleaved) { return interleaved ? 2 * i : i; }
static int orc_dim_y(int i, int d, int interleaved) { return interleaved ? 2 * i + 1 : i + d / 2; }

/* Step 2: per-pair window thresholds alpha*lambda_i (may be +inf); lambda_i from
 * base, or 2*pi/th_i for a given frequency table. */
void orc_thresholds_ex(int d, double base, const double* inv_freq, double alpha, double* thr) {
    for (int i = 0; i < d / 2; ++i) {
        double lam = inv_freq ? (2.0 * M_PI) / inv_freq[i]
                              : (2.0 * M_PI) * pow(base, (2.0 * i) / (double)d);
        thr[i] = alpha * lam;
    }
}

void orc_thresholds(int d, double base, double alpha, double* thr) {
    orc_thresholds_ex(d, base, NULL, alpha, thr);
}

/* Rotation frequencies: th_i = base^(-2i/d), or the given table. */
static void orc_freqs(int d, double base, const double* inv_freq, double* th) {
    for (int i = 0; i < d / 2; ++i) th[i] = inv_freq ? inv_freq[i] : pow(base, -(2.0 * i) / (double)d);
}

/* Step 3: rotate n_tok tokens x[n_tok][H][d] at positions pos[n_tok]. */
void orc_rope_ex(const void* x, int dtype, int64_t n_tok, int H, int d, const int64_t* pos,
                 double base, const double* inv_freq, int interleaved, double* out) {
    int P = d / 2;
    double* th = (double*)malloc(sizeof(double) * P);
    orc_freqs(d, base, inv_freq, th);
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tok; ++t) {
        for (int h = 0; h < H; ++h) {
            int64_t row = (t * H + h) * (int64_t)d;
            for (int i = 0; i < P; ++i) {
                int ix = orc_dim_x(i, d, interleaved), iy = orc_dim_y(i, d, interleaved);
                double a = (double)pos[t] * th[i];
                double c = cos(a), s = sin(a);
                double x0 = orc_load(x, dtype, row + ix);
                double x1 = orc_load(x, dtype, row + iy);
                out[row + ix] = x0 * c - x1 * s;
                out[row + iy] = x1 * c + x0 * s;
            }
        }
    }
    free(th);
}

void orc_rope(const void* x, int dtype, int64_t n_tok, int H, int d,
              const int64_t* pos, double base, double* out) {
    orc_rope_ex(x, dtype, n_tok, H, d, pos, base, NULL, 0, out);
}

/* Step 3 with one frequency table per group of heads: head h of x[n_tok][H][d] rotates by
 * row h / heads_per_table of tables[][d/2]. */
static void orc_rope_heads(const void* x, int dtype, int64_t n_tok, int H, int d,
                           const int64_t* pos, const double* tables, int heads_per_table,
                           int interleaved, double* out) {
    int P = d / 2;
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tok; ++t) {
        for (int h = 0; h < H; ++h) {
            const double* th = tables + (int64_t)(h / heads_per_table) * P;
            int64_t row = (t * H + h) * (int64_t)d;
            for (int i = 0; i < P; ++i) {
                int ix = orc_dim_x(i, d, interleaved), iy = orc_dim_y(i, d, interleaved);
                double a = (double)pos[t] * th[i];
                double c = cos(a), s = sin(a);
                double x0 = orc_load(x, dtype, row + ix);
                double x1 = orc_load(x, dtype, row + iy);
                out[row + ix] = x0 * c - x1 * s;
                out[row + iy] = x1 * c + x0 * s;
            }
        }
    }
}

/* Rotation of n_tok tokens of H heads, by the shared table (n_tables <= 1: inv_freq or
 * base) or by one row of inv_freq[n_tables][d/2] per group of H / n_tables heads. */
static void orc_rotate(const void* x, int dtype, int64_t n_tok, int H, int d, const int64_t* pos,
                       double base, const double* inv_freq, int n_tables, int interleaved,
                       double* out) {
    if (n_tables > 1) orc_rope_heads(x, dtype, n_tok, H, d, pos, inv_freq, H / n_tables, interleaved, out);
    else orc_rope_ex(x, dtype, n_tok, H, d, pos, base, inv_freq, interleaved, out);
}

/* Window thresholds of every kv head: thr[Hkv][d/2] (a copy of the shared row when
 * n_tables <= 1). */
static double* orc_head_thresholds(int d, double base, const double* inv_freq, int n_tables,
                                   int Hkv, double alpha) {
    int P = d / 2;
    double* thr = (double*)malloc(sizeof(double) * P * Hkv);
    for (int g = 0; g < Hkv; ++g)
        orc_thresholds_ex(d, base, n_tables > 1 ? inv_freq + (int64_t)g * P : inv_freq, alpha,
                          thr + (int64_t)g * P);
    return thr;
}

/* Steps 4-5 for one query row: windowed logits over visible keys 0..last,
 * ordinary softmax, out = sum p v, lse = log sum exp(logit).
 *   qr  : rotated query [d]          kr : rotated keys [n_k][Hkv][d]
 *   v   : raw values (dtype)         g  : kv head
 *   logit: scratch of length last+1
 * Returns the number of kept (key, pair) terms for this row. */
static int64_t orc_row(const double* qr, int64_t qpos, const double* kr, const int64_t* kpos,
                       const void* v, int dtype, int64_t last, int Hkv, int g, int d,
                       int interleaved, const double* thr, double scale, double* logit,
                       double* out, double* lse, const unsigned char* vis) {
    /* vis (nullable): vis[c] == 0 removes key c from this row's softmax altogether */
    int P = d / 2;
    int64_t kept = 0;
    double m = -INFINITY;
    for (int64_t c = 0; c <= last; ++c) {
        if (vis && !vis[c]) { logit[c] = -INFINITY; continue; }
        const double* k = kr + (c * Hkv + g) * (int64_t)d;
        double dist = fabs((double)(qpos - kpos[c]));
        double s = 0.0;
        for (int i = 0; i < P; ++i) {
            if (dist <= thr[i]) {
                int ix = orc_dim_x(i, d, interleaved), iy = orc_dim_y(i, d, interleaved);
                s += qr[ix] * k[ix] + qr[iy] * k[iy];
                ++kept;
            }
        }
        logit[c] = scale * s;
        if (logit[c] > m) m = logit[c];
    }
    double den = 0.0;
    for (int e = 0; e < d; ++e) out[e] = 0.0;
    for (int64_t c = 0; c <= last; ++c) {
        if (vis && !vis[c]) continue;
        double p = exp(logit[c] - m);
        den += p;
        int64_t vrow = (c * Hkv + g) * (int64_t)d;
        for (int e = 0; e < d; ++e) out[e] += p * orc_load(v, dtype, vrow + e);
    }
    for (int e = 0; e < d; ++e) out[e] /= den;
    *lse = m + log(den);
    return kept;
}

/*
 * Causal prefill.
 *   q [B][N][Hq][d], k, v [B][N][Hkv][d] (pre-RoPE, dtype), pos [B][N] (NULL -> 0..N-1)
 *   rows[n_rows]: query token indices to evaluate (NULL -> all N rows, n_rows = N)
 *   out [B][n_rows][Hq][d], lse [B][Hq][n_rows]  (double)
 *   kept_out (nullable): total kept (query, key, pair) terms over all evaluated rows/heads.
 * Returns 0, or -1 on bad arguments.
 */
int orc_prefill_ex(const void* q, const void* k, const void* v, int dtype, const int32_t* pos,
                   int B, int64_t N, int Hq, int Hkv, int d, double base,
                   const double* inv_freq, int n_tables, int interleaved, double alpha,
                   double scale, const int64_t* rows, int64_t n_rows,
                   double* out, double* lse, int64_t* kept_out, int nthreads) {
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || d < 2 || d % 2 != 0)
        return -1;
    if (n_tables > 1 && (n_tables != Hkv || !inv_freq)) return -1;
    if (!rows) n_rows = N;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    int G = Hq / Hkv;
    int P = d / 2;
    double* thr = orc_head_thresholds(d, base, inv_freq, n_tables, Hkv, alpha);
    int64_t* p64 = (int64_t*)malloc(sizeof(int64_t) * N);
    double* kr = (double*)malloc(sizeof(double) * N * Hkv * d);
    double* qr = (double*)malloc(sizeof(double) * n_rows * Hq * d);
    int64_t* qp = (int64_t*)malloc(sizeof(int64_t) * n_rows);
    int64_t kept_total = 0;
    for (int b = 0; b < B; ++b) {
        for (int64_t t = 0; t < N; ++t) p64[t] = pos ? (int64_t)pos[(int64_t)b * N + t] : t;
        orc_rotate((const char*)k + (dtype == ORC_FP32 ? 4 : 2) * (int64_t)b * N * Hkv * d, dtype,
                   N, Hkv, d, p64, base, inv_freq, n_tables, interleaved, kr);
        /* gather the evaluated query rows, then rotate them at their own positions */
        const char* qb = (const char*)q + (dtype == ORC_FP32 ? 4 : 2) * (int64_t)b * N * Hq * d;
        int esz = dtype == ORC_FP32 ? 4 : 2;
        char* qsel = (char*)malloc((size_t)esz * n_rows * Hq * d);
        for (int64_t j = 0; j < n_rows; ++j) {
            int64_t r = rows ? rows[j] : j;
            memcpy(qsel + (size_t)esz * j * Hq * d, qb + (size_t)esz * r * Hq * d, (size_t)esz * Hq * d);
            qp[j] = p64[r];
        }
        orc_rotate(qsel, dtype, n_rows, Hq, d, qp, base, inv_freq, n_tables, interleaved, qr);
        free(qsel);
        const char* vb = (const char*)v + (size_t)esz * b * N * Hkv * d;
        int64_t kept_b = 0;
        #pragma omp parallel reduction(+:kept_b)
        {
            double* logit = (double*)malloc(sizeof(double) * N);
            #pragma omp for schedule(dynamic, 1) collapse(2)
            for (int64_t j = 0; j < n_rows; ++j) {
                for (int h = 0; h < Hq; ++h) {
                    int64_t r = rows ? rows[j] : j;
                    double* o = out + (((int64_t)b * n_rows + j) * Hq + h) * d;
                    double* l = lse + ((int64_t)b * Hq + h) * n_rows + j;
                    kept_b += orc_row(qr + (j * Hq + h) * (int64_t)d, qp[j], kr, p64, vb, dtype,
                                      r, Hkv, h / G, d, interleaved, thr + (int64_t)(h / G) * P,
                                      scale, logit, o, l, NULL);
                }
            }
            free(logit);
        }
        kept_total += kept_b;
    }
    if (kept_out) *kept_out = kept_total;
    free(thr); free(p64); free(kr); free(qr); free(qp);
    return 0;
}

int orc_prefill(const void* q, const void* k, const void* v, int dtype, const int32_t* pos,
                int B, int64_t N, int Hq, int Hkv, int d, double base, double alpha,
                double scale, const int64_t* rows, int64_t n_rows,
                double* out, double* lse, int64_t* kept_out, int nthreads) {
    return orc_prefill_ex(q, k, v, dtype, pos, B, N, Hq, Hkv, d, base, NULL, 0, 0, alpha, scale,
                          rows, n_rows, out, lse, kept_out, nthreads);
}

/*
 * Causal prefill composed with token-level block sparsity (ATFlash abstract: the window
 * can be applied on top of other sparse attention methods).  Tokens form blocks of
 * `blk` consecutive indices; the row of query r (block R = r / blk) of head h attends key c
 * iff c <= r and c's block is R itself or one of the first count[b][h][R] entries of
 * idx[b][h][R][0 .. max_blocks).  Keys outside the listed blocks leave the softmax
 * altogether; the listed ones get the windowed logits of orc_prefill_ex.
 *   count int32 [B][Hq][nblk], idx int32 [B][Hq][nblk][max_blocks], nblk = ceil(N / blk).
 * Blocks are formed by token index; the rotation and the window take the positions pos
 * ([B][N], NULL = token indices), as in orc_prefill_ex.  Other arguments (inv_freq with
 * n_tables: one shared table, or one row per kv head) and outputs as for orc_prefill_ex.
 */
int orc_prefill_sparse(const void* q, const void* k, const void* v, int dtype, const int32_t* pos,
                       int B, int64_t N,
                       int Hq, int Hkv, int d, double base, const double* inv_freq, int n_tables,
                       int interleaved, double alpha, double scale, const int32_t* count,
                       const int32_t* idx, int max_blocks, int blk, const int64_t* rows,
                       int64_t n_rows, double* out, double* lse, int64_t* kept_out,
                       int nthreads) {
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || d < 2 || d % 2 != 0 || blk < 1 ||
        max_blocks < 0 || !count || (max_blocks > 0 && !idx))
        return -1;
    if (n_tables > 1 && (n_tables != Hkv || !inv_freq)) return -1;
    if (!rows) n_rows = N;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    int G = Hq / Hkv, P = d / 2;
    int esz = dtype == ORC_FP32 ? 4 : 2;
    int64_t nblk = (N + blk - 1) / blk;
    double* thr = orc_head_thresholds(d, base, inv_freq, n_tables, Hkv, alpha);
    int64_t* p64 = (int64_t*)malloc(sizeof(int64_t) * N);
    double* kr = (double*)malloc(sizeof(double) * N * Hkv * d);
    double* qr = (double*)malloc(sizeof(double) * n_rows * Hq * d);
    int64_t* qp = (int64_t*)malloc(sizeof(int64_t) * n_rows);
    int64_t kept_total = 0;
    for (int b = 0; b < B; ++b) {
        for (int64_t t = 0; t < N; ++t) p64[t] = pos ? (int64_t)pos[(int64_t)b * N + t] : t;
        orc_rotate((const char*)k + (size_t)esz * b * N * Hkv * d, dtype, N, Hkv, d, p64, base,
                   inv_freq, n_tables, interleaved, kr);
        const char* qb = (const char*)q + (size_t)esz * b * N * Hq * d;
        char* qsel = (char*)malloc((size_t)esz * n_rows * Hq * d);
        for (int64_t j = 0; j < n_rows; ++j) {
            int64_t r = rows ? rows[j] : j;
            memcpy(qsel + (size_t)esz * j * Hq * d, qb + (size_t)esz * r * Hq * d, (size_t)esz * Hq * d);
            qp[j] = p64[r];
        }
        orc_rotate(qsel, dtype, n_rows, Hq, d, qp, base, inv_freq, n_tables, interleaved, qr);
        free(qsel);
        const char* vb = (const char*)v + (size_t)esz * b * N * Hkv * d;
        int64_t kept_b = 0;
        #pragma omp parallel reduction(+:kept_b)
        {
            double* logit = (double*)malloc(sizeof(double) * N);
            unsigned char* vis = (unsigned char*)malloc((size_t)N);
            #pragma omp for schedule(dynamic, 1) collapse(2)
            for (int64_t j = 0; j < n_rows; ++j) {
                for (int h = 0; h < Hq; ++h) {
                    int64_t r = rows ? rows[j] : j;
                    int64_t R = r / blk;
                    int64_t li = ((int64_t)b * Hq + h) * nblk + R;
                    memset(vis, 0, (size_t)N);
                    for (int64_t c = R * blk; c <= r; ++c) vis[c] = 1;
                    int n = count[li] < max_blocks ? count[li] : max_blocks;
                    for (int e = 0; e < n; ++e) {
                        int64_t kb = idx[li * max_blocks + e];
                        if (kb < 0 || kb > R) continue;
                        for (int64_t c = kb * blk; c < (kb + 1) * blk && c <= r; ++c) vis[c] = 1;
                    }
                    double* o = out + (((int64_t)b * n_rows + j) * Hq + h) * d;
                    double* l = lse + ((int64_t)b * Hq + h) * n_rows + j;
                    kept_b += orc_row(qr + (j * Hq + h) * (int64_t)d, qp[j], kr, p64, vb, dtype,
                                      r, Hkv, h / G, d, interleaved, thr + (int64_t)(h / G) * P,
                                      scale, logit, o, l, vis);
                }
            }
            free(logit);
            free(vis);
        }
        kept_total += kept_b;
    }
    if (kept_out) *kept_out = kept_total;
    free(thr); free(p64); free(kr); free(qr); free(qp);
    return 0;
}

/*
 * One decode step per sequence.
 *   q [B][Hq][d] pre-RoPE; k, v [B][Lmax][Hkv][d] pre-RoPE cache contents, key c at position c;
 *   kv_len[B] (1..Lmax); q_pos[B] (NULL -> kv_len-1); the query sees keys 0..kv_len-1.
 *   out [B][Hq][d], lse [B][Hq] (double).
 */
int orc_decode_ex(const void* q, const void* k, const void* v, int dtype, const int32_t* kv_len,
                  const int32_t* q_pos, int B, int64_t Lmax, int Hq, int Hkv, int d, double base,
                  const double* inv_freq, int n_tables, int interleaved, double alpha, double scale,
                  double* out, double* lse, int64_t* kept_out, int nthreads) {
    if (B < 1 || Lmax < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || d < 2 || d % 2 != 0)
        return -1;
    if (n_tables > 1 && (n_tables != Hkv || !inv_freq)) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    int G = Hq / Hkv, P = d / 2;
    int esz = dtype == ORC_FP32 ? 4 : 2;
    double* thr = orc_head_thresholds(d, base, inv_freq, n_tables, Hkv, alpha);
    int64_t kept_total = 0;
    for (int b = 0; b < B; ++b) {
        int64_t L = kv_len[b];
        if (L < 1 || L > Lmax) { free(thr); return -1; }
        int64_t qp = q_pos ? (int64_t)q_pos[b] : L - 1;
        int64_t* kp = (int64_t*)malloc(sizeof(int64_t) * L);
        for (int64_t c = 0; c < L; ++c) kp[c] = c;
        double* kr = (double*)malloc(sizeof(double) * L * Hkv * d);
        orc_rotate((const char*)k + (size_t)esz * b * Lmax * Hkv * d, dtype, L, Hkv, d, kp, base,
                   inv_freq, n_tables, interleaved, kr);
        double* qr = (double*)malloc(sizeof(double) * Hq * d);
        orc_rotate((const char*)q + (size_t)esz * b * Hq * d, dtype, 1, Hq, d, &qp, base,
                   inv_freq, n_tables, interleaved, qr);
        const char* vb = (const char*)v + (size_t)esz * b * Lmax * Hkv * d;
        int64_t kept_b = 0;
        #pragma omp parallel reduction(+:kept_b)
        {
            double* logit = (double*)malloc(sizeof(double) * L);
            #pragma omp for schedule(dynamic, 1)
            for (int h = 0; h < Hq; ++h)
                kept_b += orc_row(qr + (int64_t)h * d, qp, kr, kp, vb, dtype, L - 1, Hkv, h / G, d,
                                  interleaved, thr + (int64_t)(h / G) * P, scale, logit,
                                  out + ((int64_t)b * Hq + h) * d, lse + (int64_t)b * Hq + h, NULL);
            free(logit);
        }
        kept_total += kept_b;
        free(kp); free(kr); free(qr);
    }
    if (kept_out) *kept_out = kept_total;
    free(thr);
    return 0;
}

int orc_decode(const void* q, const void* k, const void* v, int dtype, const int32_t* kv_len,
               const int32_t* q_pos, int B, int64_t Lmax, int Hq, int Hkv, int d, double base,
               double alpha, double scale, double* out, double* lse, int64_t* kept_out, int nthreads) {
    return orc_decode_ex(q, k, v, dtype, kv_len, q_pos, B, Lmax, Hq, Hkv, d, base, NULL, 0, 0, alpha,
                         scale, out, lse, kept_out, nthreads);
}

/*
 * Backward of the windowed causal prefill (WavePrune, What the paper found: models trained
 * with the window from scratch; training needs these gradients).  Given dout = dL/dout for a
 * scalar loss L, the chain rule through the forward above, step by step:
 *   P_rc    = softmax over visible c of the windowed logits l_rc (recomputed, fp64)
 *   dv_c   += P_rc dout_r                                  (every q head of kv head g)
 *   dP_rc   = dout_r . v_c
 *   D_r     = sum_c P_rc dP_rc                             (= dout_r . out_r)
 *   dl_rc   = P_rc (dP_rc - D_r)
 *   dq'_r  += scale * dl_rc * [pair of x kept at r-c] * k'_c[x]     (rotated coordinates)
 *   dk'_c  += scale * dl_rc * [pair of x kept at r-c] * q'_r[x]
 *   dq_r    = R(t_r)^T dq'_r,  dk_c = R(t_c)^T dk'_c      (rotation by minus the angle)
 * Only the gradients asked for are formed: dq at query rows rows[n_rows], dk and dv at key
 * rows keys[n_keys] (NULL: all N).  Inputs as for orc_prefill_ex; dout [B][N][Hq][d] in the
 * same dtype.  Outputs (double): dq [B][n_rows][Hq][d], dk and dv [B][n_keys][Hkv][d].
 */
int orc_prefill_backward_ex(const void* q, const void* k, const void* v, const void* dout,
                            int dtype, const int32_t* pos, int B, int64_t N, int Hq, int Hkv,
                            int d, double base, const double* inv_freq, int n_tables,
                            int interleaved, double alpha, double scale, const int64_t* rows,
                            int64_t n_rows, const int64_t* keys, int64_t n_keys, double* dq,
                            double* dk, double* dv, int nthreads) {
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || d < 2 || d % 2 != 0 || d > 256)
        return -1;
    if (n_tables > 1 && (n_tables != Hkv || !inv_freq)) return -1;
    if (!rows) n_rows = N;
    if (!keys) n_keys = N;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    int G = Hq / Hkv, P = d / 2;
    int esz = dtype == ORC_FP32 ? 4 : 2;
    double* thr = orc_head_thresholds(d, base, inv_freq, n_tables, Hkv, alpha);
    int64_t* p64 = (int64_t*)malloc(sizeof(int64_t) * N);
    double* kr = (double*)malloc(sizeof(double) * N * Hkv * d);
    double* qr = (double*)malloc(sizeof(double) * N * Hq * d);
    double* lse = (double*)malloc(sizeof(double) * N * Hq);
    double* Dr = (double*)malloc(sizeof(double) * N * Hq);
    unsigned char* need = (unsigned char*)malloc((size_t)N);
    for (int b = 0; b < B; ++b) {
        for (int64_t t = 0; t < N; ++t) p64[t] = pos ? (int64_t)pos[(int64_t)b * N + t] : t;
        const char* qb = (const char*)q + (size_t)esz * b * N * Hq * d;
        const char* kb = (const char*)k + (size_t)esz * b * N * Hkv * d;
        const char* vb = (const char*)v + (size_t)esz * b * N * Hkv * d;
        const char* ob = (const char*)dout + (size_t)esz * b * N * Hq * d;
        orc_rotate(kb, dtype, N, Hkv, d, p64, base, inv_freq, n_tables, interleaved, kr);
        orc_rotate(qb, dtype, N, Hq, d, p64, base, inv_freq, n_tables, interleaved, qr);
        /* rows whose softmax statistics are needed: the dq rows, and every row at or after
         * the first dk/dv key (those rows see it) */
        int64_t kmin = N;
        for (int64_t j = 0; j < n_keys; ++j) {
            int64_t c = keys ? keys[j] : j;
            if (c < kmin) kmin = c;
        }
        for (int64_t r = 0; r < N; ++r) need[r] = r >= kmin;
        for (int64_t j = 0; j < n_rows; ++j) need[rows ? rows[j] : j] = 1;
        /* forward statistics of the needed rows: lse_r and D_r = dout_r . out_r */
        #pragma omp parallel
        {
            double* logit = (double*)malloc(sizeof(double) * N);
            double* o = (double*)malloc(sizeof(double) * d);
            #pragma omp for schedule(dynamic, 1) collapse(2)
            for (int64_t r = 0; r < N; ++r) {
                for (int h = 0; h < Hq; ++h) {
                    if (!need[r]) continue;
                    double l;
                    orc_row(qr + (r * Hq + h) * (int64_t)d, p64[r], kr, p64, vb, dtype, r, Hkv,
                            h / G, d, interleaved, thr + (int64_t)(h / G) * P, scale, logit, o, &l,
                            NULL);
                    double dd = 0.0;
                    for (int e = 0; e < d; ++e) dd += orc_load(ob, dtype, (r * Hq + h) * (int64_t)d + e) * o[e];
                    lse[r * Hq + h] = l;
                    Dr[r * Hq + h] = dd;
                }
            }
            free(logit);
            free(o);
        }
        /* dq at the requested rows */
        #pragma omp parallel for schedule(dynamic, 1) collapse(2)
        for (int64_t j = 0; j < n_rows; ++j) {
            for (int h = 0; h < Hq; ++h) {
                int64_t r = rows ? rows[j] : j;
                int g = h / G;
                const double* th = thr + (int64_t)g * P;
                const double* qv = qr + (r * Hq + h) * (int64_t)d;
                double acc[256];
                for (int e = 0; e < d; ++e) acc[e] = 0.0;
                for (int64_t c = 0; c <= r; ++c) {
                    const double* kv = kr + (c * Hkv + g) * (int64_t)d;
                    double dist = fabs((double)(p64[r] - p64[c]));
                    double s = 0.0, dp = 0.0;
                    for (int i = 0; i < P; ++i) {
                        if (dist <= th[i]) {
                            int ix = orc_dim_x(i, d, interleaved), iy = orc_dim_y(i, d, interleaved);
                            s += qv[ix] * kv[ix] + qv[iy] * kv[iy];
                        }
                    }
                    double pr = exp(scale * s - lse[r * Hq + h]);
                    for (int e = 0; e < d; ++e)
                        dp += orc_load(ob, dtype, (r * Hq + h) * (int64_t)d + e) *
                              orc_load(vb, dtype, (c * Hkv + g) * (int64_t)d + e);
                    double dl = pr * (dp - Dr[r * Hq + h]);
                    for (int i = 0; i < P; ++i) {
                        if (dist <= th[i]) {
                            int ix = orc_dim_x(i, d, interleaved), iy = orc_dim_y(i, d, interleaved);
                            acc[ix] += scale * dl * kv[ix];
                            acc[iy] += scale * dl * kv[iy];
                        }
                    }
                }
                /* back to pre-RoPE coordinates: R(t_r)^T */
                double* out = dq + (((int64_t)b * n_rows + j) * Hq + h) * d;
                for (int i = 0; i < P; ++i) {
                    double th_i = n_tables > 1 ? inv_freq[(int64_t)g * P + i]
                                               : (inv_freq ? inv_freq[i] : pow(base, -(2.0 * i) / (double)d));
                    double a = (double)p64[r] * th_i, cs = cos(a), sn = sin(a);
                    int ix = orc_dim_x(i, d, interleaved), iy = orc_dim_y(i, d, interleaved);
                    out[ix] = acc[ix] * cs + acc[iy] * sn;
                    out[iy] = -acc[ix] * sn + acc[iy] * cs;
                }
            }
        }
        /* dk, dv at the requested keys: every row r >= c of every q head of kv head g */
        #pragma omp parallel for schedule(dynamic, 1) collapse(2)
        for (int64_t j = 0; j < n_keys; ++j) {
            for (int g = 0; g < Hkv; ++g) {
                int64_t c = keys ? keys[j] : j;
                const double* th = thr + (int64_t)g * P;
                const double* kv = kr + (c * Hkv + g) * (int64_t)d;
                double acck[256], accv[256];
                for (int e = 0; e < d; ++e) acck[e] = accv[e] = 0.0;
                for (int h = g * G; h < (g + 1) * G; ++h) {
                    for (int64_t r = c; r < N; ++r) {
                        const double* qv = qr + (r * Hq + h) * (int64_t)d;
                        double dist = fabs((double)(p64[r] - p64[c]));
                        double s = 0.0, dp = 0.0;
                        for (int i = 0; i < P; ++i) {
                            if (dist <= th[i]) {
                                int ix = orc_dim_x(i, d, interleaved), iy = orc_dim_y(i, d, interleaved);
                                s += qv[ix] * kv[ix] + qv[iy] * kv[iy];
                            }
                        }
                        double pr = exp(scale * s - lse[r * Hq + h]);
                        for (int e = 0; e < d; ++e) {
                            double go = orc_load(ob, dtype, (r * Hq + h) * (int64_t)d + e);
                            accv[e] += pr * go;
                            dp += go * orc_load(vb, dtype, (c * Hkv + g) * (int64_t)d + e);
                        }
                        double dl = pr * (dp - Dr[r * Hq + h]);
                        for (int i = 0; i < P; ++i) {
                            if (dist <= th[i]) {
                                int ix = orc_dim_x(i, d, interleaved), iy = orc_dim_y(i, d, interleaved);
                                acck[ix] += scale * dl * qv[ix];
                                acck[iy] += scale * dl * qv[iy];
                            }
                        }
                    }
                }
                double* ok = dk + (((int64_t)b * n_keys + j) * Hkv + g) * d;
                double* ov = dv + (((int64_t)b * n_keys + j) * Hkv + g) * d;
                for (int e = 0; e < d; ++e) ov[e] = accv[e];
                for (int i = 0; i < P; ++i) {
                    double th_i = n_tables > 1 ? inv_freq[(int64_t)g * P + i]
                                               : (inv_freq ? inv_freq[i] : pow(base, -(2.0 * i) / (double)d));
                    double a = (double)p64[c] * th_i, cs = cos(a), sn = sin(a);
                    int ix = orc_dim_x(i, d, interleaved), iy = orc_dim_y(i, d, interleaved);
                    ok[ix] = acck[ix] * cs + acck[iy] * sn;
                    ok[iy] = -acck[ix] * sn + acck[iy] * cs;
                }
            }
        }
    }
    free(thr); free(p64); free(kr); free(qr); free(lse); free(Dr); free(need);
    return 0;
}

/*
 * Kept-term count by enumeration (no closed form): queries at token indices
 * q_idx0 .. q_idx0+n_q-1 with positions equal to their indices, keys 0..n_k-1,
 * key c visible to query r iff c <= r; counts (r, c, i) with |r-c| <= alpha*lambda_i.
 * total = (d/2) * #visible (r, c).  O(n_q * n_k * d/2).
 */
void orc_count_enumerate_ex(int d, double base, const double* inv_freq, double alpha,
                            int64_t n_q, int64_t q_idx0, int64_t n_k, int64_t* kept, int64_t* total) {
    int P = d / 2;
    double* thr = (double*)malloc(sizeof(double) * P);
    orc_thresholds_ex(d, base, inv_freq, alpha, thr);
    int64_t kk = 0, tt = 0;
    #pragma omp parallel for reduction(+:kk, tt) schedule(dynamic, 16)
    for (int64_t j = 0; j < n_q; ++j) {
        int64_t r = q_idx0 + j;
        for (int64_t c = 0; c < n_k && c <= r; ++c) {
            double dist = (double)(r - c);
            tt += P;
            for (int i = 0; i < P; ++i) kk += (dist <= thr[i]);
        }
    }
    *kept = kk;
    *total = tt;
    free(thr);
}

void orc_count_enumerate(int d, double base, double alpha, int64_t n_q, int64_t q_idx0,
                         int64_t n_k, int64_t* kept, int64_t* total) {
    orc_count_enumerate_ex(d, base, NULL, alpha, n_q, q_idx0, n_k, kept, total);
}
