/*
 * mla_oracle.c -- plain fp64 CPU oracle for absorbed MLA decode over a paged latent cache.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load this library. It shares no code, header, table or helper with the GPU library,
 * and includes nothing from it.
 *
 * Sources (web pages; sections as numbered on each page):
 *   [FMLA]    bhfrc.com/news/60867  -- notes on FlashMLA / TensorRT-LLM MLA operators.
 *             S1 cache format (512-d latent c_KV + 64-d shared RoPE key k_R per token),
 *             S3 dimension constants and 64-token pages, S4 naive-vs-absorbed score check.
 *   [MHA2MLA] lpnh.cn/news/2494972 -- enabling DeepSeek MLA on a Transformer.
 *             S2.1 the MLA equations (k_nope = c_kv W_uk, v = c_kv W_uv, output = softmax of
 *             RoPE term plus NoPE term, times v) and the absorption of W_uk into the query.
 *
 * Every floating-point step is fp64. Inputs are bf16 bit patterns (uint16), widened exactly.
 *
 * Conventions (readings of the pages, one per line):
 *   - W_UK is [H][d_n][d_c]: k_nope[t,h,d] = sum_c W_UK[h,d,c] * c_t[c]  ([FMLA] S4 einsum).
 *   - W_UV is [H][d_c][d_v]: v[t,h,e]      = sum_c c_t[c] * W_UV[h,c,e]  ([MHA2MLA] S2.1, c_kv W_uv).
 *   - a cache token is [c_KV (d_c) | k_R (d_R)], pages are page_size consecutive tokens,
 *     token t of sequence b lives at page page_table[b][t / page_size], slot t % page_size.
 *   - k_R is one vector shared by all heads; q_rope and k_R arrive already rotated.
 *   - score scale: a positive value is used as given; <= 0 selects 1/sqrt(d_n + d_R), the
 *     pages' choice ([FMLA] S4).
 *   - only tokens t < seq_lens[b] exist; seq_lens[b] < 1 is an error (returns -2).
 *
 * ORACLE_MUTANT (compile-time, default 0) plants one known mistake so that the tests can
 * show each pin catches it. Product builds never define it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

typedef struct {
    int B, H, d_n, d_c, d_R, d_v; /* batch, heads, NoPE dim, latent dim, RoPE dim, value dim */
    int page_size;                /* tokens per page */
    int max_pages;                /* row stride of page_table */
} odims;

/* bf16 -> double, exact: a bf16 is the top 16 bits of an IEEE fp32. */
static double bf(uint16_t x) {
    uint32_t u = (uint32_t)x << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Address of logical token t of sequence b in the paged pool ([FMLA] S1, S3). */
static const uint16_t *token(const odims *D, const uint16_t *kv, const int32_t *page_table,
                             int b, int t) {
    int page = page_table[(size_t)b * D->max_pages + t / D->page_size];
#if ORACLE_MUTANT == 4 /* page table ignored: logical page index used as physical */
    page = t / D->page_size;
#endif
    int slot = t % D->page_size;
    return kv + ((size_t)page * D->page_size + slot) * (size_t)(D->d_c + D->d_R);
}

/* Absorbed query: qt[c] = sum_d q_nope[b,h,d] * W_UK[h,d,c]  ([MHA2MLA] S2.1; [FMLA] S4 path B). */
static void absorb(const odims *D, const uint16_t *q_nope, const uint16_t *W_UK, int b, int h,
                   double *qt) {
    const uint16_t *q = q_nope + ((size_t)b * D->H + h) * D->d_n;
    const uint16_t *W = W_UK + (size_t)h * D->d_n * D->d_c;
    for (int c = 0; c < D->d_c; ++c) {
        double s = 0.0;
        for (int d = 0; d < D->d_n; ++d) {
#if ORACLE_MUTANT == 2 /* W_UK read as [h][d_c][d_n] */
            s += bf(q[d]) * bf(W[(size_t)c * D->d_n + d]);
#else
            s += bf(q[d]) * bf(W[(size_t)d * D->d_c + c]);
#endif
        }
        qt[c] = s;
    }
}

/* Logit of one token: scale * (qt . c_t + q_rope . k_R_t)  ([MHA2MLA] S2.1; [FMLA] S4). */
static double logit(const odims *D, const double *qt, const uint16_t *q_rope_bh,
                    const uint16_t *tok, double scale) {
    double nope = 0.0, rope = 0.0;
    for (int c = 0; c < D->d_c; ++c) nope += qt[c] * bf(tok[c]);
    for (int j = 0; j < D->d_R; ++j) rope += bf(q_rope_bh[j]) * bf(tok[D->d_c + j]);
#if ORACLE_MUTANT == 1 /* RoPE term dropped */
    rope = 0.0;
#endif
    return scale * (nope + rope);
}

static int seq_len(const odims *D, const int32_t *seq_lens, int b) {
    int S = seq_lens[b];
#if ORACLE_MUTANT == 5 /* last token dropped */
    if (S > 1) S -= 1;
#endif
    (void)D;
    return S;
}

/*
 * Attention of one (b,h) over tokens [t0, t1) in latent space:
 *   s_t = logit, m = max s_t, Z = sum exp(s_t - m), p_t = exp(s_t - m) / Z,
 *   obar[c] = sum_t p_t * c_t[c]  (value stays in latent space: v = c_kv W_uv, [MHA2MLA] S2.1),
 *   returns lse = m + log Z.  If p is not NULL the probabilities are stored there.
 */
static double attend_range(const odims *D, const double *qt, const uint16_t *q_rope,
                           const uint16_t *kv, const int32_t *page_table, int b, int h, int t0,
                           int t1, double scale, double *obar, double *p) {
    const uint16_t *qr = q_rope + ((size_t)b * D->H + h) * D->d_R;
#if ORACLE_MUTANT == 8 /* RoPE query taken from head 0 */
    qr = q_rope + (size_t)b * D->H * D->d_R;
#endif
    int n = t1 - t0;
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int i = 0; i < n; ++i) {
        s[i] = logit(D, qt, qr, token(D, kv, page_table, b, t0 + i), scale);
        if (s[i] > m) m = s[i];
    }
    double Z = 0.0;
    for (int i = 0; i < n; ++i) Z += exp(s[i] - m);
    for (int c = 0; c < D->d_c; ++c) obar[c] = 0.0;
    for (int i = 0; i < n; ++i) {
        double pt = exp(s[i] - m) / Z;
        if (p) p[i] = pt;
        const uint16_t *tok = token(D, kv, page_table, b, t0 + i);
        for (int c = 0; c < D->d_c; ++c) obar[c] += pt * bf(tok[c]);
    }
    free(s);
#if ORACLE_MUTANT == 7 /* log missing from the log-sum-exp */
    return m + Z;
#else
    return m + log(Z);
#endif
}

/* Up-projection: out[e] = sum_c obar[c] * W_UV[h,c,e]  ([MHA2MLA] S2.1, v = c_kv W_uv). */
static void up_project(const odims *D, const uint16_t *W_UV, int h, const double *obar,
                       double *out) {
#if ORACLE_MUTANT == 6 /* every head uses head 0's W_UV */
    h = 0;
#endif
    const uint16_t *W = W_UV + (size_t)h * D->d_c * D->d_v;
    for (int e = 0; e < D->d_v; ++e) {
        double s = 0.0;
        for (int c = 0; c < D->d_c; ++c) s += obar[c] * bf(W[(size_t)c * D->d_v + e]);
        out[e] = s;
    }
}

/* Score scale: a value <= 0 selects 1/sqrt(d_n + d_R), the pages' choice ([FMLA] S4). */
static double pick_scale(const odims *D, double scale) {
    if (scale > 0.0) return scale;
#if ORACLE_MUTANT == 3 /* scale from the NoPE width only */
    return 1.0 / sqrt((double)D->d_n);
#else
    return 1.0 / sqrt((double)(D->d_n + D->d_R));
#endif
}

static int check_lens(const odims *D, const int32_t *seq_lens) {
    for (int b = 0; b < D->B; ++b)
        if (seq_lens[b] < 1 || seq_lens[b] > D->max_pages * D->page_size) return -2;
    return 0;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/*
 * Absorbed decode for a list of (b,h) pairs (pairs = NULL means all B*H pairs, in order).
 * out: [npairs][d_v] (or [B][H][d_v] when pairs is NULL), lse: [npairs] (nullable).
 * n_split <= 1: one pass over [0, S_b). n_split > 1: the tokens are cut into n_split
 * contiguous ranges of ceil(S_b / n_split) tokens, each range is attended on its own and the
 * partial results are merged by their log-sum-exp weights:
 *   lse = log sum_i exp(lse_i),  obar = sum_i exp(lse_i - lse) * obar_i.
 */
int oracle_decode_absorbed(int B, int H, int d_n, int d_c, int d_R, int d_v, int page_size,
                           int max_pages, const uint16_t *q_nope, const uint16_t *q_rope,
                           const uint16_t *W_UK, const uint16_t *W_UV, const uint16_t *kv,
                           const int32_t *page_table, const int32_t *seq_lens, double scale,
                           const int32_t *pairs, int npairs, int n_split, double *out,
                           double *lse, int nthreads) {
    odims D = {B, H, d_n, d_c, d_R, d_v, page_size, max_pages};
    if (check_lens(&D, seq_lens)) return -2;
    scale = pick_scale(&D, scale);
    if (!pairs) npairs = B * H;
    for (int i = 0; i < npairs; ++i)
        if (pairs && (pairs[2 * i] < 0 || pairs[2 * i] >= B || pairs[2 * i + 1] < 0 ||
                      pairs[2 * i + 1] >= H))
            return -3;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < npairs; ++i) {
        int b = pairs ? pairs[2 * i] : i / H;
        int h = pairs ? pairs[2 * i + 1] : i % H;
        int S = seq_len(&D, seq_lens, b);
        double *qt = (double *)malloc(sizeof(double) * (size_t)d_c);
        double *obar = (double *)malloc(sizeof(double) * (size_t)d_c);
        absorb(&D, q_nope, W_UK, b, h, qt);
        double L;
        if (n_split <= 1) {
            L = attend_range(&D, qt, q_rope, kv, page_table, b, h, 0, S, scale, obar, NULL);
        } else {
            int len = (S + n_split - 1) / n_split;
            int nr = (S + len - 1) / len; /* non-empty ranges */
            double *ob = (double *)malloc(sizeof(double) * (size_t)nr * d_c);
            double *ls = (double *)malloc(sizeof(double) * (size_t)nr);
            double mx = -INFINITY;
            for (int r = 0; r < nr; ++r) {
                int t0 = r * len, t1 = t0 + len < S ? t0 + len : S;
                ls[r] = attend_range(&D, qt, q_rope, kv, page_table, b, h, t0, t1, scale,
                                     ob + (size_t)r * d_c, NULL);
                if (ls[r] > mx) mx = ls[r];
            }
            double z = 0.0;
            for (int r = 0; r < nr; ++r) z += exp(ls[r] - mx);
            L = mx + log(z);
            for (int c = 0; c < d_c; ++c) obar[c] = 0.0;
            for (int r = 0; r < nr; ++r) {
                double w = exp(ls[r] - L);
                for (int c = 0; c < d_c; ++c) obar[c] += w * ob[(size_t)r * d_c + c];
            }
            free(ob);
            free(ls);
        }
        up_project(&D, W_UV, h, obar, out + (size_t)i * d_v);
        if (lse) lse[i] = L;
        free(qt);
        free(obar);
    }
    return 0;
}

/*
 * Naive (decompressed) decode, the brute-force form ([FMLA] S4 path A; [MHA2MLA] S2.1):
 * per token and head K[t,h,d] = sum_c W_UK[h,d,c] c_t[c] and V[t,h,e] = sum_c c_t[c] W_UV[h,c,e]
 * are materialised, then standard attention with logits scale * (q_nope.K + q_rope.k_R).
 * Shares only token addressing and bf16 widening with the absorbed form.
 */
int oracle_decode_naive(int B, int H, int d_n, int d_c, int d_R, int d_v, int page_size,
                        int max_pages, const uint16_t *q_nope, const uint16_t *q_rope,
                        const uint16_t *W_UK, const uint16_t *W_UV, const uint16_t *kv,
                        const int32_t *page_table, const int32_t *seq_lens, double scale,
                        double *out, double *lse, int nthreads) {
    odims D = {B, H, d_n, d_c, d_R, d_v, page_size, max_pages};
    if (check_lens(&D, seq_lens)) return -2;
    scale = pick_scale(&D, scale);
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < B * H; ++i) {
        int b = i / H, h = i % H;
        int S = seq_len(&D, seq_lens, b);
        const uint16_t *qn = q_nope + ((size_t)b * H + h) * d_n;
        const uint16_t *qr = q_rope + ((size_t)b * H + h) * d_R;
        const uint16_t *Wk = W_UK + (size_t)h * d_n * d_c;
        const uint16_t *Wv = W_UV + (size_t)h * d_c * d_v;
        double *s = (double *)malloc(sizeof(double) * (size_t)S);
        double *V = (double *)malloc(sizeof(double) * (size_t)S * d_v);
        double m = -INFINITY;
        for (int t = 0; t < S; ++t) {
            const uint16_t *tok = token(&D, kv, page_table, b, t);
            double qk = 0.0;
            for (int d = 0; d < d_n; ++d) {
                double k = 0.0;
                for (int c = 0; c < d_c; ++c) k += bf(Wk[(size_t)d * d_c + c]) * bf(tok[c]);
                qk += bf(qn[d]) * k;
            }
            double qr_kr = 0.0;
            for (int j = 0; j < d_R; ++j) qr_kr += bf(qr[j]) * bf(tok[d_c + j]);
            s[t] = scale * (qk + qr_kr);
            if (s[t] > m) m = s[t];
            for (int e = 0; e < d_v; ++e) {
                double v = 0.0;
                for (int c = 0; c < d_c; ++c) v += bf(tok[c]) * bf(Wv[(size_t)c * d_v + e]);
                V[(size_t)t * d_v + e] = v;
            }
        }
        double Z = 0.0;
        for (int t = 0; t < S; ++t) Z += exp(s[t] - m);
        for (int e = 0; e < d_v; ++e) {
            double o = 0.0;
            for (int t = 0; t < S; ++t) o += exp(s[t] - m) / Z * V[(size_t)t * d_v + e];
            out[(size_t)i * d_v + e] = o;
        }
        if (lse) lse[i] = m + log(Z);
        free(s);
        free(V);
    }
    return 0;
}

/* Softmax weights p_t (t < S_b) of one (b,h), through the same steps as the absorbed decode. */
int oracle_probs(int B, int H, int d_n, int d_c, int d_R, int d_v, int page_size, int max_pages,
                 const uint16_t *q_nope, const uint16_t *q_rope, const uint16_t *W_UK,
                 const uint16_t *kv, const int32_t *page_table, const int32_t *seq_lens,
                 double scale, int b, int h, double *p) {
    odims D = {B, H, d_n, d_c, d_R, d_v, page_size, max_pages};
    if (check_lens(&D, seq_lens)) return -2;
    if (b < 0 || b >= B || h < 0 || h >= H) return -3;
    scale = pick_scale(&D, scale);
    double *qt = (double *)malloc(sizeof(double) * (size_t)d_c);
    double *obar = (double *)malloc(sizeof(double) * (size_t)d_c);
    absorb(&D, q_nope, W_UK, b, h, qt);
    attend_range(&D, qt, q_rope, kv, page_table, b, h, 0, seq_len(&D, seq_lens, b), scale, obar,
                 p);
    free(qt);
    free(obar);
    return 0;
}

/*
 * Page gather: dst[b][t][:] = token t of sequence b for t < S_b, zero for S_b <= t < S_max.
 * Pure copy of bf16 bit patterns; the definition of reading a paged cache ([FMLA] S3).
 */
int oracle_gather_pages(int B, int d_c, int d_R, int page_size, int max_pages,
                        const uint16_t *kv, const int32_t *page_table, const int32_t *seq_lens,
                        int S_max, uint16_t *dst) {
    odims D = {B, 0, 0, d_c, d_R, 0, page_size, max_pages};
    int w = d_c + d_R;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] < 0 || seq_lens[b] > S_max) return -2;
        for (int t = 0; t < S_max; ++t) {
            uint16_t *d = dst + ((size_t)b * S_max + t) * w;
            int live = t < seq_lens[b];
#if ORACLE_MUTANT == 9 /* zero fill starts one row late */
            live = t < seq_lens[b] + 1 && t < S_max;
#endif
            int copy = w;
#if ORACLE_MUTANT == 10 /* the RoPE part of each row is not copied */
            copy = d_c;
            memset(d, 0, sizeof(uint16_t) * (size_t)w);
#endif
            if (live)
                memcpy(d, token(&D, kv, page_table, b, t), sizeof(uint16_t) * (size_t)copy);
            else
                memset(d, 0, sizeof(uint16_t) * (size_t)w);
        }
    }
    return 0;
}

int oracle_mutant(void) { return ORACLE_MUTANT; }
