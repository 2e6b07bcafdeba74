/*
 * HHR decode-path ORACLE -- test infrastructure only.
 *
 * This file is a plain, slow, obviously-correct CPU statement of what the
 * HHR decode path computes.  It exists to check the GPU library; nothing in
 * the product may link, load or call it.  Only the test suite, the smoke
 * entry point and the CPU-baseline leg of the benchmark use it.  It shares no
 * source, header, table or helper with the GPU library.
 *
 * Sources (cited by page title and section; no formula survives on the
 * pages, so every formula below is the plainest reading of the prose):
 *   [ABS]  "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation"
 *          (arXiv 2610.01230), Abstract and the Chinese summary on the
 *          modelscope paper card.
 *   [FIG]  thelatestinai.com page on arXiv 2610.01230, "Figures & tables":
 *          captions of Figure 2, Figure 3 and Figure 4; Appendix Table 4.
 *   [BLOG] rit.work blog post on HHR (hhr-hash-retrieval-long-context),
 *          sections "Почему расстояние Хэмминга пропускает важные ключи" and
 *          "Два уровня маршрутизации решают разные ошибки".
 *
 * Precision rules (the pages fix none):
 *   - Projections whose sign becomes a hash bit, and the rotated vectors that
 *     feed the page metadata, use the "canonical chain": fp32 fused
 *     multiply-add in ascending dimension order starting from +0.0f.  The
 *     GPU takes the same integer decisions in the same precision.
 *   - Page bounds are summed in fp64 in ascending dimension order; every
 *     product of two fp32 numbers is exact in fp64.
 *   - Attention is computed in fp64.
 *
 * Compile with -O2 -ffp-contract=off and without fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t batch;      /* B                                   */
    int32_t n_q_heads;  /* Hq                                  */
    int32_t n_kv_heads; /* Hkv; Hq must be a multiple of Hkv    */
    int32_t head_dim;   /* D                                   */
    int32_t page_size;  /* P                                   */
    int32_t hash_bits;  /* b, a multiple of 64                 */
    int32_t max_ctx;    /* Tmax: row capacity of K, V, codes   */
    int32_t kv_bf16;    /* 1: Q, K, V hold bf16 bit patterns (uint16); 0: fp32 */
    int32_t meta_bf16;  /* 1: page max/min are stored rounded outward to bf16 values */
    int32_t sink_tokens;  /* decode: the first sink_tokens keys are always attended    */
    int32_t local_window; /* decode: the last local_window keys are always attended    */
    int32_t page_group;    /* decode: 0 = page score max over the group's heads, 1 = min    */
    int32_t hamming_group; /* decode: 0 = H summed over the group's query codes,
                              1 = H against the code of the group's mean query            */
} oracle_dims;

enum { ORACLE_OK = 0, ORACLE_BAD_DIMS = 1, ORACLE_NOMEM = 2 };

static int dims_ok(const oracle_dims* d) {
    if (d->batch < 1 || d->n_kv_heads < 1 || d->n_q_heads < d->n_kv_heads) return 0;
    if (d->n_q_heads % d->n_kv_heads) return 0;
    if (d->head_dim < 1 || d->page_size < 1 || d->max_ctx < 0) return 0;
    if (d->hash_bits < 64 || d->hash_bits % 64) return 0;
    if (d->sink_tokens < 0 || d->local_window < 0) return 0;
    if ((d->page_group != 0 && d->page_group != 1) || (d->hamming_group != 0 && d->hamming_group != 1)) return 0;
    return 1;
}

static int64_t n_pages_of(int64_t len, int64_t page) { return (len + page - 1) / page; }

/* One element of a Q/K/V array, widened to fp32.  A bf16 value is the top
 * half of an fp32 bit pattern, so widening it is exact. */
static float elem(const void* base, int64_t i, int bf16) {
    if (bf16) {
        uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return f;
    }
    return ((const float*)base)[i];
}

/* Canonical chain: acc = +0; acc = fma(a[d], x[d], acc) for d ascending. */
static float dot_canon(const float* a, const float* x, int n) {
    float acc = 0.0f;
    for (int d = 0; d < n; ++d) acc = fmaf(a[d], x[d], acc);
    return acc;
}

/*
 * Project one vector x (length D) of KV head h:
 *   xrot[r] = (R_h x)_r            -- GKR's head-wise orthogonal transform [ABS]
 *   bit j   = [ (W_h x)_j > 0 ]    -- LHP's head-wise projection, binarised [ABS]
 * Bit j lives in word j/64 at bit position j%64 (least significant first).
 * R is D x D row-major (xrot_r = sum_c R[r][c] x_c); W is b x D row-major.
 */
static void project(int D, int nbits, const float* R, const float* W, const float* x,
                    float* xrot, uint64_t* code) {
    if (xrot)
        for (int r = 0; r < D; ++r) xrot[r] = dot_canon(R + (int64_t)r * D, x, D);
    if (code) {
        for (int w = 0; w < nbits / 64; ++w) code[w] = 0;
        for (int j = 0; j < nbits; ++j) {
            float y = dot_canon(W + (int64_t)j * D, x, D);
            if (y > 0.0f) code[j / 64] |= (uint64_t)1 << (j % 64);
        }
    }
}

/* Public helper for the pins: project n vectors with one head's R and W. */
int oracle_project(int32_t D, int32_t nbits, const float* R, const float* W, const float* X,
                   int64_t n, float* Xrot, uint64_t* codes) {
    if (D < 1 || nbits < 64 || nbits % 64) return ORACLE_BAD_DIMS;
    for (int64_t i = 0; i < n; ++i)
        project(D, nbits, R, W, X + i * D, Xrot ? Xrot + i * D : NULL,
                codes ? codes + i * (nbits / 64) : NULL);
    return ORACLE_OK;
}

/* bf16 neighbours of a finite fp32 x: bf16_trunc drops the low 16 bits
 * (rounds toward zero); bf16_away is the next bf16 one step further from
 * zero than the truncation. */
static float bf16_trunc(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    u &= 0xffff0000u;
    float y;
    memcpy(&y, &u, 4);
    return y;
}
static float bf16_away(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    u = (u & 0xffff0000u) + 0x10000u;
    float y;
    memcpy(&y, &u, 4);
    return y;
}
/* Outward rounding of a page statistic to bf16, so that the stored interval
 * [kmin, kmax] still contains every key of the page ("store page bounds":
 * the bound must stay an upper bound): the smallest bf16 >= x for a max, the
 * largest bf16 <= x for a min.  x and its truncation enclose nothing but
 * each other, and the truncation and bf16_away enclose x. */
static float bf16_ceil(float x) {
    const float t = bf16_trunc(x);
    return t >= x ? t : bf16_away(x);
}
static float bf16_floor(float x) {
    const float t = bf16_trunc(x);
    return t <= x ? t : bf16_away(x);
}

/*
 * Encode keys [start[b], start[b]+count[b]) of every sequence b.
 *
 * - codes[b][h][t][w] for t in that range: the LHP code of key t [ABS].
 * - meta[b][h][p][r][0|1] = max|min over the keys t of page p (pages group P
 *   adjacent keys [BLOG, "Два уровня..."]) of the rotated key (R_h k_t)_r,
 *   for every page p the range touches, over that page's keys below
 *   start+count.  These are the stored page bounds [BLOG, "Когда HHR...";
 *   ABS].  A rotated value of -0 is taken as +0 so that max/min are unique.
 *   With meta_bf16 the max is then rounded up and the min down to bf16
 *   values (bf16_ceil / bf16_floor), kept here as fp32.
 * Layouts: K [B][Hkv][Tmax][D]; R [Hkv][D][D]; W [Hkv][b][D];
 *          meta [B][Hkv][ceil(Tmax/P)][D][2] fp32; codes [B][Hkv][Tmax][b/64].
 */
int oracle_encode(const oracle_dims* dm, const void* K, const float* R, const float* W,
                  const int32_t* start, const int32_t* count, float* meta, uint64_t* codes) {
    if (!dims_ok(dm)) return ORACLE_BAD_DIMS;
    const int B = dm->batch, Hkv = dm->n_kv_heads, D = dm->head_dim, P = dm->page_size;
    const int nb = dm->hash_bits, NW = nb / 64;
    const int64_t T = dm->max_ctx, NPmax = n_pages_of(T, P);
    for (int b = 0; b < B; ++b)
        if (start[b] < 0 || count[b] < 0 || (int64_t)start[b] + count[b] > T) return ORACLE_BAD_DIMS;
    int status = ORACLE_OK;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            const int64_t s = start[b], e = (int64_t)start[b] + count[b];
            if (e <= s) continue;
            const float* Rh = R + (int64_t)h * D * D;
            const float* Wh = W + (int64_t)h * nb * D;
            float* x = malloc(sizeof(float) * D);
            float* xr = malloc(sizeof(float) * D);
            if (!x || !xr) {
                free(x); free(xr);
#pragma omp atomic write
                status = ORACLE_NOMEM;
                continue;
            }
            const int64_t kbase = ((int64_t)b * Hkv + h) * T;
            for (int64_t p = s / P; p <= (e - 1) / P; ++p) {
                float* m = meta + (((int64_t)b * Hkv + h) * NPmax + p) * D * 2;
                const int64_t lo = p * P, hi = (p + 1) * P < e ? (p + 1) * P : e;
                for (int64_t t = lo; t < hi; ++t) {
                    for (int d = 0; d < D; ++d) x[d] = elem(K, (kbase + t) * D + d, dm->kv_bf16);
                    project(D, nb, Rh, Wh, x, xr, t >= s ? codes + (kbase + t) * NW : NULL);
                    for (int r = 0; r < D; ++r) {
                        float v = xr[r] == 0.0f ? 0.0f : xr[r];
                        if (t == lo || v > m[2 * r]) m[2 * r] = v;
                        if (t == lo || v < m[2 * r + 1]) m[2 * r + 1] = v;
                    }
                }
                if (dm->meta_bf16)
                    for (int r = 0; r < D; ++r) {
                        m[2 * r] = bf16_ceil(m[2 * r]);
                        m[2 * r + 1] = bf16_floor(m[2 * r + 1]);
                    }
            }
            free(x);
            free(xr);
        }
    }
    return status;
}

typedef struct { double s; int32_t p; } page_key;   /* order: s descending, then p ascending */
typedef struct { int32_t h; int32_t t; } key_key;   /* order: h ascending, then t ascending  */

static int cmp_page(const void* a, const void* b) {
    const page_key* x = a; const page_key* y = b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->p > y->p) - (x->p < y->p);
}
static int cmp_key(const void* a, const void* b) {
    const key_key* x = a; const key_key* y = b;
    if (x->h != y->h) return (x->h > y->h) - (x->h < y->h);
    return (x->t > y->t) - (x->t < y->t);
}
static int cmp_int(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* Page select of one (b, h) [ABS; BLOG, "Два уровня маршрутизации решают
 * разные ошибки": pages with a low bound are dropped whole]: sort the NP
 * (S, p) pairs by S descending, then p ascending (S compared as values, so
 * -0 and +0 tie), take the first `keep`, list them ascending.  `pk` is
 * reordered.  Returns keep after the clamp to [1, min(NP, max_keep)]. */
static int64_t select_pages_one(page_key* pk, int64_t NP, int64_t keep, int32_t max_keep, int32_t* plist) {
    if (keep < 1) keep = 1;
    if (keep > NP) keep = NP;
    if (keep > max_keep) keep = max_keep;
    qsort(pk, NP, sizeof(page_key), cmp_page);
    for (int64_t j = 0; j < keep; ++j) plist[j] = pk[j].p;
    qsort(plist, keep, sizeof(int32_t), cmp_int);
    return keep;
}

/* Softmax scale: the caller's when positive, else 1/sqrt(D). */
static double softmax_scale(float scale_in, int D) {
    return scale_in > 0.0f ? (double)scale_in : 1.0 / sqrt((double)D);
}

/* Attention of the G query heads q [G][D] (fp32 values) over the keff keys
 * sel[] of one (b, h), whose rows start at row0 of K and V: out_i =
 * sum_j softmax_j(scale * q_i . k_j) v_j, all in fp64 (the logit summed with
 * d ascending, the softmax shifted by its maximum) [ABS: attention over the
 * retrieved keys].  out [G][D]; zero when keff = 0.  sc holds >= keff doubles. */
static void attend_selected(const float* q, int G, int D, const void* K, const void* V, int64_t row0, int bf,
                            const int32_t* sel, int64_t keff, double scale, double* sc, double* out) {
    for (int i = 0; i < G; ++i) {
        double* o = out + (int64_t)i * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (keff == 0) continue;
        double mx = 0.0;
        for (int64_t j = 0; j < keff; ++j) {
            const int64_t row = (row0 + sel[j]) * D;
            double s = 0.0;
            for (int d = 0; d < D; ++d) s += (double)q[i * D + d] * (double)elem(K, row + d, bf);
            sc[j] = s * scale;
            if (j == 0 || sc[j] > mx) mx = sc[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < keff; ++j) {
            const double wgt = exp(sc[j] - mx);
            const int64_t row = (row0 + sel[j]) * D;
            l += wgt;
            for (int d = 0; d < D; ++d) o[d] += wgt * (double)elem(V, row + d, bf);
        }
        for (int d = 0; d < D; ++d) o[d] /= l;
    }
}

/*
 * One decode step for one layer: every sequence b, every KV head h, with the
 * G = Hq/Hkv query heads i = h*G .. h*G+G-1 that share KV head h.
 *
 * Steps, in the order the pages give them (coarse stage, then fine stage
 * inside the surviving pages, then exact attention on the chosen keys)
 * [ABS; BLOG, "Два уровня маршрутизации решают разные ошибки"]:
 *  1. query prep: qrot_i = R_h q_i, code_q,i = LHP code of q_i.
 *  2. page bound (GKR): U_i(p) = sum_r max(qrot_i,r * kmax[p][r],
 *     qrot_i,r * kmin[p][r]) in fp64, r ascending.  It bounds qrot_i . krot_t
 *     from above for every key t of page p; since R_h is orthogonal that is
 *     q_i . k_t up to rounding [ABS; FIG, Figure 3].  The group shares one
 *     selection, scored S(p) = max_i U_i(p).
 *  3. page select: keep the `keep` pages with the largest S; equal S goes to
 *     the lower page index.  keep = clamp(keep_pages[b], 1, min(NP, max_keep)).
 *  4. candidates: keys t < L of the kept pages, ascending.
 *  5. Hamming (LHP): H(t) = sum_i popcount(code_q,i XOR code_t), summed over
 *     the group and over the code words [ABS; BLOG, "Почему расстояние..."].
 *  6. key select (top-k): the k_eff = min(top_k, |C|) candidates with the
 *     smallest (H, t); listed ascending, padded with -1 [FIG, Table 4 "Top-k"].
 *  7. attention: out_i = softmax(scale * q_i . k_t) weighted sum of v_t over
 *     the selected t, fp64; scale = 1/sqrt(D) when scale <= 0.
 * An empty sequence (L = 0) yields out = 0, no pages, no keys.
 *
 * Sink tokens and a local window (a variant; the HHR pages use none, the
 * baselines they compare against do [FIG, Appendix Table 4: 4 sink tokens
 * and a local window of 64 keys]): with sink_tokens = s and local_window =
 * w, the forced keys F = {t < min(s, L)} and {max(min(s, L), L - w) <= t < L}
 * are always attended; steps 4-6 run on the candidates outside F, and the
 * selection lists the sinks, then the step-6 keys, then the window keys
 * (ascending, since the step-6 keys lie between them).  k_eff = |F| + the
 * step-6 count; the list holds top_k + s + w entries.
 *
 * Group aggregation variants (the pages leave the GQA grouping open; see
 * [FIG, Figure 4]: recall is measured per KV head): page_group = 1 scores a
 * page by the min over the group of U_i(p) instead of the max;
 * hamming_group = 1 replaces step 5's sum by H(t) = popcount(code(qm) XOR
 * code_t), where qm is the group's mean query, qm_d = (sum_i q_i,d) / G in
 * fp32 (i ascending, then one division), coded by the same canonical chain.
 *
 * Outputs (any pointer may be NULL to skip it):
 *   qrot  [B][Hq][D] fp32        code_q [B][Hq][b/64]
 *   score [B][Hkv][NPmax] fp64   (+0.0 for p >= NP)
 *   pages [B][Hkv][max_keep] int32 ascending, -1 padded; n_pages [B][Hkv]
 *   ham   [B][Hkv][max_keep*P] uint16: H of candidate slot j*P + r = key
 *         pages[j]*P + r; 0xFFFF where that key is >= L, forced, or the slot is unused
 *   sel   [B][Hkv][top_k + s + w] int32 ascending, -1 padded; k_eff [B][Hkv]
 *   out   [B][Hq][D] fp64
 */
int oracle_decode(const oracle_dims* dm, const void* Q, const void* K, const void* V,
                  const float* R, const float* W, const float* meta, const uint64_t* codes,
                  const int32_t* seq_len, const int32_t* keep_pages, int32_t max_keep,
                  int32_t top_k, float scale_in,
                  float* qrot_out, uint64_t* codeq_out, double* score_out,
                  int32_t* pages_out, int32_t* npages_out, uint16_t* ham_out,
                  int32_t* sel_out, int32_t* keff_out, double* out) {
    if (!dims_ok(dm) || max_keep < 1 || top_k < 1) return ORACLE_BAD_DIMS;
    const int B = dm->batch, Hq = dm->n_q_heads, Hkv = dm->n_kv_heads, G = Hq / Hkv;
    const int D = dm->head_dim, P = dm->page_size, nb = dm->hash_bits, NW = nb / 64;
    const int64_t T = dm->max_ctx, NPmax = n_pages_of(T, P);
    const int bf = dm->kv_bf16;
    const double scale = softmax_scale(scale_in, D);
    const int64_t cap = (int64_t)top_k + dm->sink_tokens + dm->local_window;  /* sel row length */
    int status = ORACLE_OK;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int64_t L = seq_len[b];
            if (L < 0) L = 0;
            if (L > T) L = T;
            const int64_t NP = n_pages_of(L, P);
            /* forced keys: [0, s_end) and [w_start, L) */
            const int64_t s_end = dm->sink_tokens < L ? dm->sink_tokens : L;
            const int64_t w_start = L - dm->local_window > s_end ? L - dm->local_window : s_end;
            const int64_t bh = (int64_t)b * Hkv + h;
            const float* Rh = R + (int64_t)h * D * D;
            const float* Wh = W + (int64_t)h * nb * D;

            float* q = malloc(sizeof(float) * G * D);
            float* qr = malloc(sizeof(float) * G * D);
            uint64_t* cq = malloc(sizeof(uint64_t) * (G + 1) * NW);  /* the group's codes, then the mean query's */
            page_key* pk = malloc(sizeof(page_key) * (NP > 0 ? NP : 1));
            int32_t* plist = malloc(sizeof(int32_t) * max_keep);
            key_key* cand = malloc(sizeof(key_key) * (int64_t)max_keep * P);
            int32_t* sel = malloc(sizeof(int32_t) * cap);
            double* sc = malloc(sizeof(double) * cap);
            if (!q || !qr || !cq || !pk || !plist || !cand || !sel || !sc) {
                free(q); free(qr); free(cq); free(pk); free(plist); free(cand); free(sel); free(sc);
#pragma omp atomic write
                status = ORACLE_NOMEM;
                continue;
            }

            /* 1. query prep */
            for (int i = 0; i < G; ++i) {
                const int64_t qi = (int64_t)b * Hq + h * G + i;
                for (int d = 0; d < D; ++d) q[i * D + d] = elem(Q, qi * D + d, bf);
                project(D, nb, Rh, Wh, q + i * D, qr + i * D, cq + i * NW);
                if (qrot_out) memcpy(qrot_out + qi * D, qr + i * D, sizeof(float) * D);
                if (codeq_out) memcpy(codeq_out + qi * NW, cq + i * NW, sizeof(uint64_t) * NW);
            }
            if (dm->hamming_group) {  /* the group's mean query and its code */
                float* qm = malloc(sizeof(float) * D * 2);
                if (qm) {
                    for (int d = 0; d < D; ++d) {
                        float acc = 0.0f;
                        for (int i = 0; i < G; ++i) acc += q[i * D + d];
                        qm[d] = acc / (float)G;
                    }
                    project(D, nb, Rh, Wh, qm, qm + D, cq + G * NW);
                    free(qm);
                } else {
#pragma omp atomic write
                    status = ORACLE_NOMEM;
                }
            }

            /* 2. page bounds */
            for (int64_t p = 0; p < NP; ++p) {
                const float* m = meta + (bh * NPmax + p) * D * 2;
                double S = 0.0;
                for (int i = 0; i < G; ++i) {
                    double U = 0.0;
                    for (int r = 0; r < D; ++r) {
                        double a = (double)qr[i * D + r] * (double)m[2 * r];
                        double c = (double)qr[i * D + r] * (double)m[2 * r + 1];
                        U += a > c ? a : c;
                    }
                    if (i == 0 || (dm->page_group ? U < S : U > S)) S = U;
                }
                if (S == 0.0) S = 0.0; /* -0 and +0 are the same score */
                pk[p].s = S;
                pk[p].p = (int32_t)p;
            }
            if (score_out) {
                for (int64_t p = 0; p < NPmax; ++p) score_out[bh * NPmax + p] = p < NP ? pk[p].s : 0.0;
            }

            /* 3. page select */
            const int64_t keep = select_pages_one(pk, NP, keep_pages[b], max_keep, plist);
            if (pages_out)
                for (int64_t j = 0; j < max_keep; ++j) pages_out[bh * max_keep + j] = j < keep ? plist[j] : -1;
            if (npages_out) npages_out[bh] = (int32_t)keep;

            /* 4.-5. candidates and their Hamming distances */
            int64_t nc = 0;
            for (int64_t j = 0; j < (int64_t)max_keep * P && ham_out; ++j)
                ham_out[bh * (int64_t)max_keep * P + j] = 0xFFFF;
            for (int64_t j = 0; j < keep; ++j) {
                for (int r = 0; r < P; ++r) {
                    const int64_t t = (int64_t)plist[j] * P + r;
                    if (t >= L || t < s_end || t >= w_start) continue;
                    int32_t H = 0;
                    if (dm->hamming_group) {
                        for (int w = 0; w < NW; ++w)
                            H += __builtin_popcountll(cq[G * NW + w] ^ codes[(bh * T + t) * NW + w]);
                    } else {
                        for (int i = 0; i < G; ++i)
                            for (int w = 0; w < NW; ++w)
                                H += __builtin_popcountll(cq[i * NW + w] ^ codes[(bh * T + t) * NW + w]);
                    }
                    if (ham_out) ham_out[bh * (int64_t)max_keep * P + j * P + r] = (uint16_t)H;
                    cand[nc].h = H;
                    cand[nc].t = (int32_t)t;
                    ++nc;
                }
            }

            /* 6. key select, then the forced keys around it */
            const int64_t kh = nc < top_k ? nc : top_k;
            qsort(cand, nc, sizeof(key_key), cmp_key);
            for (int64_t j = 0; j < kh; ++j) sel[s_end + j] = cand[j].t;
            qsort(sel + s_end, kh, sizeof(int32_t), cmp_int);
            for (int64_t t = 0; t < s_end; ++t) sel[t] = (int32_t)t;
            for (int64_t t = w_start; t < L; ++t) sel[s_end + kh + (t - w_start)] = (int32_t)t;
            const int64_t keff = s_end + kh + (L - w_start);
            if (sel_out)
                for (int64_t j = 0; j < cap; ++j) sel_out[bh * cap + j] = j < keff ? sel[j] : -1;
            if (keff_out) keff_out[bh] = (int32_t)keff;

            /* 7. attention over the selected keys */
            if (out) attend_selected(q, G, D, K, V, bh * T, bf, sel, keff, scale, sc, out + ((int64_t)b * Hq + h * G) * D);
            free(q); free(qr); free(cq); free(pk); free(plist); free(cand); free(sel); free(sc);
        }
    }
    return status;
}

/* Threads an OpenMP region of this library will use. */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Step 3 of oracle_decode alone, on given page scores score [B][Hkv][NPmax]
 * (entries p >= NP_b are ignored): pages [B][Hkv][max_keep] ascending, -1
 * padded, and n_pages [B][Hkv].  Same rule and clamp as oracle_decode.
 */
int oracle_select_pages(const oracle_dims* dm, const double* score, const int32_t* seq_len,
                        const int32_t* keep_pages, int32_t max_keep, int32_t* pages_out, int32_t* npages_out) {
    if (!dims_ok(dm) || max_keep < 1) return ORACLE_BAD_DIMS;
    const int B = dm->batch, Hkv = dm->n_kv_heads, P = dm->page_size;
    const int64_t T = dm->max_ctx, NPmax = n_pages_of(T, P);
    int status = ORACLE_OK;
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int64_t L = seq_len[b];
            if (L < 0) L = 0;
            if (L > T) L = T;
            const int64_t NP = n_pages_of(L, P), bh = (int64_t)b * Hkv + h;
            page_key* pk = malloc(sizeof(page_key) * (NP > 0 ? NP : 1));
            int32_t* plist = malloc(sizeof(int32_t) * max_keep);
            if (!pk || !plist) {
                free(pk); free(plist);
                status = ORACLE_NOMEM;
                continue;
            }
            for (int64_t p = 0; p < NP; ++p) {
                pk[p].s = score[bh * NPmax + p];
                pk[p].p = (int32_t)p;
            }
            const int64_t keep = select_pages_one(pk, NP, keep_pages[b], max_keep, plist);
            for (int64_t j = 0; j < max_keep; ++j) pages_out[bh * max_keep + j] = j < keep ? plist[j] : -1;
            npages_out[bh] = (int32_t)keep;
            free(pk); free(plist);
        }
    }
    return status;
}

/*
 * TopK (Oracle): the comparison row of the pages that keeps the keys with the
 * largest exact attention logit, with no bounds and no codes [FIG, the
 * "TopK (Oracle)" rows of Table 1 and Table 2, and "TopK-1.5%" in Appendix
 * Table 4; BLOG, "Когда HHR меняет планы запуска модели": selection by exact
 * scores].  For every sequence b and KV head h, the G query heads of h
 * sharing one selection as in oracle_decode:
 *  1. z(t) = max_i sum_d q_i,d * k_t,d for t < L, in fp64, d ascending from
 *     +0: a product of two fp32 numbers is exact in fp64, so only the
 *     additions round.  -0 is read as +0.  The group max mirrors the page
 *     score S(p) = max_i U_i(p) of the HHR path.
 *  2. key select: the k_eff = min(top_k, L) keys with the largest z, equal z
 *     going to the lower t; listed ascending, padded with -1.
 *  3. attention over them, as step 7 of oracle_decode.
 * Outputs (NULL skips): score [B][Hkv][Tmax] fp64 (z; +0 for t >= L),
 * sel [B][Hkv][top_k], k_eff [B][Hkv], out [B][Hq][D] fp64.
 */
int oracle_topk(const oracle_dims* dm, const void* Q, const void* K, const void* V, const int32_t* seq_len,
                int32_t top_k, float scale_in, double* score_out, int32_t* sel_out, int32_t* keff_out,
                double* out) {
    if (!dims_ok(dm) || top_k < 1) return ORACLE_BAD_DIMS;
    const int B = dm->batch, Hq = dm->n_q_heads, Hkv = dm->n_kv_heads, G = Hq / Hkv, D = dm->head_dim;
    const int64_t T = dm->max_ctx;
    const int bf = dm->kv_bf16;
    const double scale = softmax_scale(scale_in, D);
    int status = ORACLE_OK;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int64_t L = seq_len[b];
            if (L < 0) L = 0;
            if (L > T) L = T;
            const int64_t bh = (int64_t)b * Hkv + h;
            float* q = malloc(sizeof(float) * G * D);
            page_key* zk = malloc(sizeof(page_key) * (L > 0 ? L : 1));
            int32_t* sel = malloc(sizeof(int32_t) * top_k);
            double* sc = malloc(sizeof(double) * top_k);
            if (!q || !zk || !sel || !sc) {
                free(q); free(zk); free(sel); free(sc);
#pragma omp atomic write
                status = ORACLE_NOMEM;
                continue;
            }
            for (int i = 0; i < G; ++i)
                for (int d = 0; d < D; ++d) q[i * D + d] = elem(Q, ((int64_t)b * Hq + h * G + i) * D + d, bf);

            /* 1. exact logits, max over the group */
            for (int64_t t = 0; t < L; ++t) {
                const int64_t row = (bh * T + t) * D;
                double z = 0.0;
                for (int i = 0; i < G; ++i) {
                    double s = 0.0;
                    for (int d = 0; d < D; ++d) s += (double)q[i * D + d] * (double)elem(K, row + d, bf);
                    if (i == 0 || s > z) z = s;
                }
                if (z == 0.0) z = 0.0;
                zk[t].s = z;
                zk[t].p = (int32_t)t;
            }
            if (score_out)
                for (int64_t t = 0; t < T; ++t) score_out[bh * T + t] = t < L ? zk[t].s : 0.0;

            /* 2. key select: the same order as the page select, over keys */
            const int64_t keff = select_pages_one(zk, L, top_k, top_k, sel);
            if (sel_out)
                for (int64_t j = 0; j < top_k; ++j) sel_out[bh * top_k + j] = j < keff ? sel[j] : -1;
            if (keff_out) keff_out[bh] = (int32_t)keff;

            /* 3. attention over the selected keys */
            if (out) attend_selected(q, G, D, K, V, bh * T, bf, sel, keff, scale, sc, out + ((int64_t)b * Hq + h * G) * D);
            free(q); free(zk); free(sel); free(sc);
        }
    }
    return status;
}
