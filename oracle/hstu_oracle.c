/*
 * HSTU attention forward: CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file; only the tests, the smoke check and the benchmark's
 * cpu_baseline leg do.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (CK example README "18_hstu_attention", section "Forward
 * computation", and the same operator description on the older README):
 *   s[b,h,i,j] = alpha * q[b,i,h,:] . k[b,j,h,:]
 *   masked positions of s are zeroed by the functional mask ("Masking" table)
 *   SiLU variant:    o[b,i,h,:] = attn_scale * sum_j vis(i,j) * SiLU(s) * v[b,j,h,:]
 *   softmax variant: o[b,i,h,:] = attn_scale * sum_{j vis} softmax_j(s) * v[b,j,h,:],
 *                    masked entries take -inf before the softmax (the HSTU
 *                    explainer page, section 1.2: -inf entries are exactly zero
 *                    after softmax), LSE_i = ln sum_{j vis} exp(s_ij); an empty
 *                    row gives o = 0 and LSE = -inf.
 * Everything is evaluated in double precision from the fp32 values of the
 * rounded inputs, one (sequence, head, row) at a time, with the dense mask of
 * each sequence materialised first from the rule below.  Built with
 * -DORACLE_FP32 the same steps run in single precision (scores, SiLU, softmax
 * sums and the output accumulation in float, expf/logf): the fp32 oracle, whose
 * own rounding error the double build bounds.
 *
 * The mask rule (CK README "Masking" table; readings of the points the pages
 * leave open are listed with each step).  Per sequence, with C = context_len,
 * L = local_len, M = minfull_len, T = num_targets[b]:
 *   physical query order  [context C | UIH U_q | targets T]
 *   physical key order    [context C | UIH U_kv | targets T (self-attention only)]
 *   (1) a target key is never attended ("excluded from attending").
 *   (2) a context key is visible to every query ("always visible to all queries").
 *   (3) otherwise the key is a UIH key at UIH position v, and the query is placed
 *       on the key-UIH axis at x: a UIH query at UIH position u sits at
 *       x = u + (U_kv - U_q) (its own key in self-attention; the tail of the
 *       key history in cross-attention); a target query sits after the whole
 *       history, x = U_kv; a context query precedes every UIH key, x = -1.
 *   (4) causal: the key must not lie after the query, x - v >= 0.
 *   (5) full rows: L == 0 disables the local window; with M > 0 the last M UIH
 *       queries and every target query attend the whole (causal) history.
 *   (6) otherwise local window: |x - v| <= L (the diagonal plus the L keys
 *       before it).
 * Lengths that do not fit (S < C + T) are clamped: C' = min(C, S),
 * T' = min(T, S - C'), U = S - C' - T'.
 *
 * Relative attention bias (HSTU explainer, "The layer, line by line" (b) and
 * "The relative attention bias"; self-attention only), added to the score
 * before the mask and the non-linearity:
 *   s[b,h,i,j] = alpha * q_i . k_j + rab_pos[h][min(|i - j|, P - 1)]
 *                                  + rab_time[h][bucket(|ts_i - ts_j|)]
 * with i, j the physical positions in the sequence, ts the per-token integer
 * timestamps (seconds) and bucket(d) the number of the explainer's bucket edges
 * 1, 5, 30, 60, 300, 1800, 3600, 86400, 604800, 2.6e6 that are <= d (11
 * buckets, 0 for d < 1, 10 for d >= 2.6e6).  Either term may be absent.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* arithmetic type of one row's evaluation (see the header) */
#ifdef ORACLE_FP32
typedef float real_t;
#define R_EXP expf
#define R_LOG logf
#else
typedef double real_t;
#define R_EXP exp
#define R_LOG log
#endif

/* per-sequence class boundaries of the query and key axes */
typedef struct {
    int64_t q0, kv0;      /* first token of the sequence in q/o and in k/v */
    int S_q, S_kv;        /* physical lengths */
    int Cq, Uq, Tq;       /* query-side context / UIH / target counts */
    int Ck, Ukv, Tk;      /* key-side counts */
    int L, M, causal;
    double a;             /* attn_scale of the sequence's group */
} seq_t;

static int imin(int a, int b) { return a < b ? a : b; }
static int imax(int a, int b) { return a > b ? a : b; }

static void describe(seq_t *s, int64_t q0, int64_t q1, int64_t kv0, int64_t kv1, int C, int T,
                     int cross, int L, int M, int causal)
{
    s->q0 = q0;
    s->kv0 = kv0;
    s->S_q = (int)(q1 - q0);
    s->S_kv = (int)(kv1 - kv0);
    s->Cq = imin(C, s->S_q);
    s->Tq = imin(imax(T, 0), s->S_q - s->Cq);
    s->Uq = s->S_q - s->Cq - s->Tq;
    s->Ck = imin(C, s->S_kv);
    s->Tk = cross ? 0 : imin(imax(T, 0), s->S_kv - s->Ck);
    s->Ukv = s->S_kv - s->Ck - s->Tk;
    s->L = L;
    s->M = M;
    s->causal = causal;
}

/* the mask rule, steps (1)-(6) of the header */
static int visible(const seq_t *s, int i, int j)
{
    if (j >= s->Ck + s->Ukv) return 0;   /* (1) target key */
    if (j < s->Ck) return 1;             /* (2) context key */
    int v = j - s->Ck;                   /* UIH key position */
    int x, full;
    if (i < s->Cq) {                     /* context query */
        if (s->causal) return 0;         /* precedes every UIH key */
        x = -1;
        full = (s->L == 0);
    } else if (i < s->Cq + s->Uq) {      /* UIH query */
        int u = i - s->Cq;
        x = u + (s->Ukv - s->Uq);
        full = (s->L == 0) || (s->M > 0 && u >= s->Uq - s->M);
    } else {                             /* target query */
        x = s->Ukv;
        full = (s->L == 0) || (s->M > 0);
    }
    int d = x - v;
    if (s->causal && d < 0) return 0;    /* (4) */
    if (full) return 1;                  /* (5) */
    return d <= s->L && d >= -s->L;      /* (6) */
}

/* relative attention bias tables (NULL members: term absent) */
typedef struct {
    const int32_t *ts;        /* [tokens] timestamps of the sequence tokens */
    const double *time_tab;   /* [H][11] */
    const double *pos_tab;    /* [H][P] */
    int P;
} rab_t;

#define RAB_BUCKETS 11
/* the explainer's time-gap bucket edges (seconds): 1 s, 5 s, 30 s, 1 min, 5 min,
 * 30 min, 1 h, 1 d, 1 w, ~1 mo */
static const int64_t kRabEdges[RAB_BUCKETS - 1] = {1, 5, 30, 60, 300, 1800, 3600, 86400, 604800, 2600000};

int oracle_rab_bucket(int64_t d)
{
    if (d < 0) d = -d;
    int b = 0;
    for (int e = 0; e < RAB_BUCKETS - 1; ++e)
        if (kRabEdges[e] <= d) b = e + 1;
    return b;
}

static double rab_bias(const rab_t *r, const seq_t *s, int h, int i, int j)
{
    double bias = 0.0;
    if (!r) return bias;
    if (r->pos_tab) {
        int d = i > j ? i - j : j - i;
        bias += r->pos_tab[(int64_t)h * r->P + imin(d, r->P - 1)];
    }
    if (r->ts) {
        int64_t d = (int64_t)r->ts[s->q0 + i] - (int64_t)r->ts[s->kv0 + j];
        bias += r->time_tab[(int64_t)h * RAB_BUCKETS + oracle_rab_bucket(d)];
    }
    return bias;
}

/* one output row: o_row[Dv] (and *lse) from the row's dense mask; sbuf holds
 * S_kv + Dv values (the row's scores, then its output accumulator) */
static void row_forward(const seq_t *s, int h, int i, const unsigned char *mask_row,
                        int H, int Dqk, int Dv, int softmax, double alpha,
                        const float *q, const float *k, const float *v, const rab_t *rab,
                        double *o_row, double *lse_out, real_t *sbuf)
{
    const float *qi = q + ((s->q0 + i) * H + h) * (int64_t)Dqk;
    real_t *acc = sbuf + s->S_kv;
    const real_t al = (real_t)alpha, a = (real_t)s->a;
    for (int e = 0; e < Dv; ++e) acc[e] = 0;
    /* scores of the visible keys */
    real_t smax = -INFINITY;
    int nvis = 0;
    for (int j = 0; j < s->S_kv; ++j) {
        if (!mask_row[j]) continue;
        const float *kj = k + ((s->kv0 + j) * H + h) * (int64_t)Dqk;
        real_t dot = 0;
        for (int e = 0; e < Dqk; ++e) dot += (real_t)qi[e] * (real_t)kj[e];
        sbuf[j] = al * dot + (real_t)rab_bias(rab, s, h, i, j);
        if (sbuf[j] > smax) smax = sbuf[j];
        ++nvis;
    }
    if (!softmax) {
        for (int j = 0; j < s->S_kv; ++j) {
            if (!mask_row[j]) continue;
            real_t x = sbuf[j];
            real_t p = x / (1 + R_EXP(-x));           /* SiLU(x) = x * sigmoid(x) */
            const float *vj = v + ((s->kv0 + j) * H + h) * (int64_t)Dv;
            for (int e = 0; e < Dv; ++e) acc[e] += p * (real_t)vj[e];
        }
        for (int e = 0; e < Dv; ++e) o_row[e] = (double)(acc[e] * a);
        if (lse_out) *lse_out = 0.0;
        return;
    }
    if (nvis == 0) {                                  /* empty row: o = 0, LSE = -inf */
        for (int e = 0; e < Dv; ++e) o_row[e] = 0.0;
        if (lse_out) *lse_out = -INFINITY;
        return;
    }
    real_t denom = 0;
    for (int j = 0; j < s->S_kv; ++j)
        if (mask_row[j]) denom += R_EXP(sbuf[j] - smax);
    real_t lse = smax + R_LOG(denom);
    for (int j = 0; j < s->S_kv; ++j) {
        if (!mask_row[j]) continue;
        real_t p = R_EXP(sbuf[j] - lse);
        const float *vj = v + ((s->kv0 + j) * H + h) * (int64_t)Dv;
        for (int e = 0; e < Dv; ++e) acc[e] += p * (real_t)vj[e];
    }
    for (int e = 0; e < Dv; ++e) o_row[e] = (double)(acc[e] * a);
    if (lse_out) *lse_out = (double)lse;
}

/* shared argument bundle of the exported functions */
typedef struct {
    int B, H, Dqk, Dv;
    const int64_t *q_off, *kv_off;   /* [B+1] token offsets */
    const int32_t *num_targets;      /* [B] or NULL */
    int cross, causal, softmax;
    double alpha;                    /* 0 -> 1/sqrt(Dqk) */
    int G;
    const int32_t *g_L, *g_C, *g_M;  /* [G] */
    const double *g_a;               /* [G]; 0 -> 1 / max UIH length of Q in the group */
} problem_t;

/* group of sequence b: groups are contiguous runs of B/G sequences */
static int group_of(const problem_t *p, int b) { return b / (p->B / p->G); }

static void setup(const problem_t *p, seq_t *seqs)
{
    for (int b = 0; b < p->B; ++b) {
        int g = group_of(p, b);
        int T = p->num_targets ? p->num_targets[b] : 0;
        describe(&seqs[b], p->q_off[b], p->q_off[b + 1], p->kv_off[b], p->kv_off[b + 1],
                 p->g_C[g], T, p->cross, p->g_L[g], p->g_M[g], p->causal);
    }
    for (int g = 0; g < p->G; ++g) {
        double a = p->g_a[g];
        if (a == 0.0) {
            int mx = 0;
            for (int b = 0; b < p->B; ++b)
                if (group_of(p, b) == g && seqs[b].Uq > mx) mx = seqs[b].Uq;
            a = 1.0 / (double)(mx > 0 ? mx : 1);
        }
        for (int b = 0; b < p->B; ++b)
            if (group_of(p, b) == g) seqs[b].a = a;
    }
}

static int check(const problem_t *p)
{
    if (p->B < 0 || p->H <= 0 || p->Dqk <= 0 || p->Dv <= 0 || p->G <= 0) return 1;
    if (p->B % p->G != 0) return 1;
    return 0;
}

static double alpha_of(const problem_t *p)
{
    return p->alpha != 0.0 ? p->alpha : 1.0 / sqrt((double)p->Dqk);
}

/* ---------------------------------------------------------------- exports */

/* Dense mask of one sequence, row-major [S_q][S_kv], 1 = attended. */
int oracle_mask(int S_q, int S_kv, int C, int T, int cross, int L, int M, int causal,
                unsigned char *mask)
{
    seq_t s;
    describe(&s, 0, S_q, 0, S_kv, C, T, cross, L, M, causal);
    for (int i = 0; i < S_q; ++i)
        for (int j = 0; j < S_kv; ++j) mask[(int64_t)i * S_kv + j] = (unsigned char)visible(&s, i, j);
    return 0;
}

#define PROBLEM_ARGS                                                                          \
    int B, int H, int Dqk, int Dv, const int64_t *q_off, const int64_t *kv_off,              \
        const int32_t *num_targets, int cross, int causal, int softmax, double alpha, int G, \
        const int32_t *g_L, const int32_t *g_C, const int32_t *g_M, const double *g_a

#define PROBLEM_INIT                                                                     \
    problem_t p = {B, H, Dqk, Dv, q_off, kv_off, num_targets, cross, causal, softmax, alpha, \
                   G, g_L, g_C, g_M, g_a}

/* Full forward.  q,k: [tokens][H][Dqk] fp32, v: [tokens][H][Dv] fp32.
 * o: [total_q][H][Dv] double; lse (softmax, may be NULL): [total_q][H] double;
 * *pairs (may be NULL): number of visible (b, h, i, j).  nthreads <= 0: default. */
static int hstu_fwd_impl(const problem_t *pp, const rab_t *rab, const float *q, const float *k,
                         const float *v, double *o, double *lse, int64_t *pairs, int nthreads);

int oracle_hstu_fwd(PROBLEM_ARGS, const float *q, const float *k, const float *v,
                    double *o, double *lse, int64_t *pairs, int nthreads)
{
    PROBLEM_INIT;
    return hstu_fwd_impl(&p, NULL, q, k, v, o, lse, pairs, nthreads);
}

/* The same with the relative attention bias (self-attention only): ts [tokens]
 * or NULL, time_tab [H][11] (with ts), pos_tab [H][P] or NULL. */
int oracle_hstu_fwd_rab(PROBLEM_ARGS, const int32_t *ts, const double *time_tab, const double *pos_tab,
                        int P, const float *q, const float *k, const float *v, double *o, double *lse,
                        int64_t *pairs, int nthreads)
{
    PROBLEM_INIT;
    if (cross || (pos_tab && P < 1) || (ts && !time_tab)) return 1;
    rab_t r = {ts, time_tab, pos_tab, P};
    return hstu_fwd_impl(&p, &r, q, k, v, o, lse, pairs, nthreads);
}

static int hstu_fwd_impl(const problem_t *pp, const rab_t *rab, const float *q, const float *k,
                         const float *v, double *o, double *lse, int64_t *pairs, int nthreads)
{
    const problem_t p = *pp;
    const int B = p.B, H = p.H, Dqk = p.Dqk, Dv = p.Dv, softmax = p.softmax, cross = p.cross,
              causal = p.causal;
    const int32_t *num_targets = p.num_targets;
    if (check(&p)) return 1;
    double al = alpha_of(&p);
    seq_t *seqs = (seq_t *)calloc((size_t)(B > 0 ? B : 1), sizeof(seq_t));
    setup(&p, seqs);
    int64_t total = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    for (int b = 0; b < B; ++b) {
        const seq_t *s = &seqs[b];
        unsigned char *mask = (unsigned char *)malloc((size_t)s->S_q * s->S_kv + 1);
        oracle_mask(s->S_q, s->S_kv, p.g_C[group_of(&p, b)],
                    num_targets ? num_targets[b] : 0, cross, s->L, s->M, causal, mask);
        int64_t cnt = 0;
        for (int64_t e = 0; e < (int64_t)s->S_q * s->S_kv; ++e) cnt += mask[e];
        total += cnt * H;
        int rows = s->S_q * H;
#pragma omp parallel
        {
            real_t *sbuf = (real_t *)malloc(sizeof(real_t) * (size_t)(s->S_kv + Dv + 1));
#pragma omp for schedule(dynamic, 4)
            for (int r = 0; r < rows; ++r) {
                int h = r % H, i = r / H;
                int64_t tok = s->q0 + i;
                row_forward(s, h, i, mask + (int64_t)i * s->S_kv, H, Dqk, Dv, softmax, al, q, k, v, rab,
                            o + (tok * H + h) * Dv, lse ? lse + tok * H + h : NULL, sbuf);
            }
            free(sbuf);
        }
        free(mask);
    }
    if (pairs) *pairs = total;
    free(seqs);
    return 0;
}

static int hstu_rows_impl(const problem_t *pp, const rab_t *rab, const float *q, const float *k,
                          const float *v, int n, const int32_t *rows_b, const int32_t *rows_h,
                          const int32_t *rows_i, double *o_rows, double *lse_rows, int nthreads);

/* Selected rows only: row r is (rows_b[r], rows_h[r], rows_i[r]) with i the row inside
 * its sequence.  o_rows: [n][Dv] double; lse_rows (may be NULL): [n] double. */
int oracle_hstu_rows(PROBLEM_ARGS, const float *q, const float *k, const float *v, int n,
                     const int32_t *rows_b, const int32_t *rows_h, const int32_t *rows_i,
                     double *o_rows, double *lse_rows, int nthreads)
{
    PROBLEM_INIT;
    return hstu_rows_impl(&p, NULL, q, k, v, n, rows_b, rows_h, rows_i, o_rows, lse_rows, nthreads);
}

/* Selected rows with the relative attention bias (arguments as oracle_hstu_fwd_rab). */
int oracle_hstu_rows_rab(PROBLEM_ARGS, const int32_t *ts, const double *time_tab, const double *pos_tab,
                         int P, const float *q, const float *k, const float *v, int n,
                         const int32_t *rows_b, const int32_t *rows_h, const int32_t *rows_i,
                         double *o_rows, double *lse_rows, int nthreads)
{
    PROBLEM_INIT;
    if (cross || (pos_tab && P < 1) || (ts && !time_tab)) return 1;
    rab_t r = {ts, time_tab, pos_tab, P};
    return hstu_rows_impl(&p, &r, q, k, v, n, rows_b, rows_h, rows_i, o_rows, lse_rows, nthreads);
}

static int hstu_rows_impl(const problem_t *pp, const rab_t *rab, const float *q, const float *k,
                          const float *v, int n, const int32_t *rows_b, const int32_t *rows_h,
                          const int32_t *rows_i, double *o_rows, double *lse_rows, int nthreads)
{
    const problem_t p = *pp;
    const int B = p.B, H = p.H, Dqk = p.Dqk, Dv = p.Dv, softmax = p.softmax;
    if (check(&p)) return 1;
    double al = alpha_of(&p);
    seq_t *seqs = (seq_t *)calloc((size_t)(B > 0 ? B : 1), sizeof(seq_t));
    setup(&p, seqs);
    for (int r = 0; r < n; ++r) {
        if (rows_b[r] < 0 || rows_b[r] >= B) { free(seqs); return 1; }
        const seq_t *s = &seqs[rows_b[r]];
        if (rows_i[r] < 0 || rows_i[r] >= s->S_q || rows_h[r] < 0 || rows_h[r] >= H) {
            free(seqs);
            return 1;
        }
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        int maxkv = 1;
        for (int b = 0; b < B; ++b) maxkv = imax(maxkv, seqs[b].S_kv);
        real_t *sbuf = (real_t *)malloc(sizeof(real_t) * (size_t)(maxkv + Dv));
        unsigned char *mrow = (unsigned char *)malloc((size_t)maxkv);
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < n; ++r) {
            const seq_t *s = &seqs[rows_b[r]];
            for (int j = 0; j < s->S_kv; ++j) mrow[j] = (unsigned char)visible(s, rows_i[r], j);
            row_forward(s, rows_h[r], rows_i[r], mrow, H, Dqk, Dv, softmax, al, q, k, v, rab,
                        o_rows + (int64_t)r * Dv, lse_rows ? lse_rows + r : NULL, sbuf);
        }
        free(sbuf);
        free(mrow);
    }
    free(seqs);
    return 0;
}

/* Number of visible (i, j) pairs of each sequence (per head), counted from the rule. */
int oracle_count_pairs(PROBLEM_ARGS, int64_t *per_seq)
{
    PROBLEM_INIT;
    (void)softmax;
    (void)alpha;
    if (check(&p)) return 1;
    seq_t *seqs = (seq_t *)calloc((size_t)(B > 0 ? B : 1), sizeof(seq_t));
    setup(&p, seqs);
    for (int b = 0; b < B; ++b) {
        int64_t c = 0;
        for (int i = 0; i < seqs[b].S_q; ++i)
            for (int j = 0; j < seqs[b].S_kv; ++j) c += visible(&seqs[b], i, j);
        per_seq[b] = c;
    }
    free(seqs);
    return 0;
}

/* Threads an OpenMP region of the oracle uses by default. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* The resolved per-sequence scalars, for inspection by the tests. */
int oracle_seq_info(PROBLEM_ARGS, int32_t *info /* [B][6]: Cq Uq Tq Ck Ukv Tk */,
                    double *scale /* [B] */)
{
    PROBLEM_INIT;
    (void)softmax;
    (void)alpha;
    if (check(&p)) return 1;
    seq_t *seqs = (seq_t *)calloc((size_t)(B > 0 ? B : 1), sizeof(seq_t));
    setup(&p, seqs);
    for (int b = 0; b < B; ++b) {
        int32_t *o = info + 6 * b;
        o[0] = seqs[b].Cq; o[1] = seqs[b].Uq; o[2] = seqs[b].Tq;
        o[3] = seqs[b].Ck; o[4] = seqs[b].Ukv; o[5] = seqs[b].Tk;
        scale[b] = seqs[b].a;
    }
    free(seqs);
    return 0;
}
