/*
 * WKV-7 oracle: plain fp64 token-order CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and
 * the benchmark's CPU-baseline leg load this file's library. It shares no code,
 * header, table or helper with the GPU library and includes nothing from it.
 *
 * What it computes (the RWKV-7 "Goose" WKV-7 recurrence; the model card on the
 * Hugging Face catalog page calls this token-order form the "eager" reference,
 * section "Transformers quickstart"). Per independent unit -- one (sequence,
 * head) pair -- with head size N and state S in R^{N x N} indexed
 * [value i, key j], for each token t of the unit in order:
 *
 *     sa[i]   = sum_j S[i,j] * a_t[j]                  (reads S_{t-1})
 *     S[i,j]  = S[i,j]*w_t[j] + sa[i]*b_t[j] + v_t[i]*k_t[j]
 *     y_t[i]  = sum_j S[i,j] * r_t[j]                  (reads the updated S_t)
 *
 * The a-term reads the undecayed S_{t-1}. This is the reading under which the
 * rwkv-lab page's mapping of a gated DeltaNet step onto this kernel (section
 * "Highlight result - GDN in RWKV-7") reproduces the gated delta rule: there
 * the b vector carries the step's decay factor itself, which is right only if
 * the (S a) b^T term starts from the undecayed state. Training forwards also store the state entering every 16th token
 * of the unit (rwkv-metal page, section "The Metal WKV-7 kernel": a state
 * checkpoint every 16 tokens), chunk c holding the state entering token 16c,
 * so chunk 0 holds the initial state.
 *
 * The backward is reverse-mode differentiation of the same loop, for the loss
 * L = sum <dy, y> + <ds_out, S_T>, with the forward states kept in fp64. It
 * does not use the checkpoints: it is the definition, not an optimisation.
 * An initial state given as h_in is differentiable (rwkv-metal page, section
 * "The Metal WKV-7 kernel", wkv7_train_with_state), hence ds0.
 *
 * Packed and ragged inputs (rwkv-lab page, post-training trainer paragraph:
 * state reset at every packing boundary; model card: packed sequences run
 * with a state reset at each boundary; rwkv-metal page: exact right-padding
 * for ragged batches): every sequence is its own unit with its own initial
 * state, so nothing flows across a boundary in either direction. Tokens that
 * belong to no sequence are never read and their outputs are left untouched.
 *
 * Layouts: token streams [B, T, H, N] (N contiguous); flat token index
 * b*T + t; states [S, H, N, N]; checkpoints [slots, H, N, N] with sequence s's
 * chunk c at slot seq_ckpt[s] + c (dense mode: slot b*ceil(T/16) + c).
 */
#include <stdlib.h>
#include <string.h>
#include <stdint.h>
#include <omp.h>

#define ORACLE_CHUNK 16

typedef struct {
    long start;    /* flat token index of the sequence's first token */
    long len;
    long ckpt;     /* first checkpoint slot */
} seg_t;

/* Strided view of one unit: token t, element j of stream p at p[t*ts + j]. */
typedef struct {
    int T, N;
    long ts;
    const double *r, *w, *k, *v, *a, *b;
} unit_in_t;

static void unit_forward(const unit_in_t *u, const double *s0, double *y,
                         double *sT, double *ckpt, long ckpt_stride)
{
    const int N = u->N;
    double *S = (double *)calloc((size_t)N * N, sizeof(double));
    double *sa = (double *)malloc((size_t)N * sizeof(double));
    if (s0) memcpy(S, s0, (size_t)N * N * sizeof(double));
    for (int t = 0; t < u->T; ++t) {
        const double *rt = u->r + t * u->ts, *wt = u->w + t * u->ts;
        const double *kt = u->k + t * u->ts, *vt = u->v + t * u->ts;
        const double *at = u->a + t * u->ts, *bt = u->b + t * u->ts;
        if (ckpt && t % ORACLE_CHUNK == 0)
            memcpy(ckpt + (t / ORACLE_CHUNK) * ckpt_stride, S, (size_t)N * N * sizeof(double));
        for (int i = 0; i < N; ++i) {
            double acc = 0.0;
            for (int j = 0; j < N; ++j) acc += S[i * N + j] * at[j];
            sa[i] = acc;
        }
        for (int i = 0; i < N; ++i)
            for (int j = 0; j < N; ++j)
                S[i * N + j] = S[i * N + j] * wt[j] + sa[i] * bt[j] + vt[i] * kt[j];
        if (y) {
            double *yt = y + t * u->ts;
            for (int i = 0; i < N; ++i) {
                double acc = 0.0;
                for (int j = 0; j < N; ++j) acc += S[i * N + j] * rt[j];
                yt[i] = acc;
            }
        }
    }
    if (sT) memcpy(sT, S, (size_t)N * N * sizeof(double));
    free(S);
    free(sa);
}

/* Returns 0 on success, -1 when the state history does not fit in memory. */
static int unit_backward(const unit_in_t *u, const double *s0, const double *dy,
                         const double *ds_out, double *dr, double *dw, double *dk,
                         double *dv, double *da, double *db, double *ds0)
{
    const int N = u->N, T = u->T;
    const size_t NN = (size_t)N * N;
    /* hist[t] = state before token t (S_{t-1} in 1-based notation); hist[T] = S_T. */
    double *hist = (double *)malloc((size_t)(T + 1) * NN * sizeof(double));
    double *sa_all = (double *)malloc((size_t)(T > 0 ? T : 1) * N * sizeof(double));
    double *dS = (double *)malloc(NN * sizeof(double));
    double *dsa = (double *)malloc((size_t)N * sizeof(double));
    if (!hist || !sa_all || !dS || !dsa) {
        free(hist); free(sa_all); free(dS); free(dsa);
        return -1;
    }
    if (s0) memcpy(hist, s0, NN * sizeof(double));
    else memset(hist, 0, NN * sizeof(double));
    for (int t = 0; t < T; ++t) {
        const double *wt = u->w + t * u->ts, *kt = u->k + t * u->ts;
        const double *vt = u->v + t * u->ts, *at = u->a + t * u->ts, *bt = u->b + t * u->ts;
        const double *Sp = hist + (size_t)t * NN;
        double *Sn = hist + (size_t)(t + 1) * NN;
        double *sa = sa_all + (size_t)t * N;
        for (int i = 0; i < N; ++i) {
            double acc = 0.0;
            for (int j = 0; j < N; ++j) acc += Sp[i * N + j] * at[j];
            sa[i] = acc;
        }
        for (int i = 0; i < N; ++i)
            for (int j = 0; j < N; ++j)
                Sn[i * N + j] = Sp[i * N + j] * wt[j] + sa[i] * bt[j] + vt[i] * kt[j];
    }
    if (ds_out) memcpy(dS, ds_out, NN * sizeof(double));
    else memset(dS, 0, NN * sizeof(double));
    for (int t = T - 1; t >= 0; --t) {
        const long o = t * u->ts;
        const double *rt = u->r + o, *wt = u->w + o, *kt = u->k + o;
        const double *vt = u->v + o, *at = u->a + o, *bt = u->b + o;
        const double *Sp = hist + (size_t)t * NN;        /* S_{t-1} */
        const double *Sn = hist + (size_t)(t + 1) * NN;  /* S_t */
        const double *sa = sa_all + (size_t)t * N;
        /* y_t = S_t r_t */
        for (int j = 0; j < N; ++j) {
            double acc = 0.0;
            if (dy)
                for (int i = 0; i < N; ++i) acc += Sn[i * N + j] * dy[o + i];
            dr[o + j] = acc;
        }
        if (dy)
            for (int i = 0; i < N; ++i)
                for (int j = 0; j < N; ++j) dS[i * N + j] += dy[o + i] * rt[j];
        /* S_t = S_{t-1} diag(w) + sa b^T + v k^T, sa = S_{t-1} a */
        for (int i = 0; i < N; ++i) {
            double acc_v = 0.0, acc_sa = 0.0;
            for (int j = 0; j < N; ++j) {
                acc_v += dS[i * N + j] * kt[j];
                acc_sa += dS[i * N + j] * bt[j];
            }
            dv[o + i] = acc_v;
            dsa[i] = acc_sa;
        }
        for (int j = 0; j < N; ++j) {
            double acc_k = 0.0, acc_b = 0.0, acc_w = 0.0, acc_a = 0.0;
            for (int i = 0; i < N; ++i) {
                acc_k += dS[i * N + j] * vt[i];
                acc_b += dS[i * N + j] * sa[i];
                acc_w += dS[i * N + j] * Sp[i * N + j];
                acc_a += dsa[i] * Sp[i * N + j];
            }
            dk[o + j] = acc_k;
            db[o + j] = acc_b;
            dw[o + j] = acc_w;
            da[o + j] = acc_a;
        }
        for (int i = 0; i < N; ++i)
            for (int j = 0; j < N; ++j)
                dS[i * N + j] = dS[i * N + j] * wt[j] + dsa[i] * at[j];
    }
    if (ds0) memcpy(ds0, dS, NN * sizeof(double));
    free(hist); free(sa_all); free(dS); free(dsa);
    return 0;
}

/* Build the sequence list. Dense mode (nseq == 0): row b is one sequence. */
static seg_t *make_segments(int B, int T, int nseq, const int32_t *seq_start,
                            const int32_t *seq_len, const int32_t *seq_ckpt, int *count)
{
    const int n = nseq > 0 ? nseq : B;
    seg_t *s = (seg_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(seg_t));
    const long nc = (T + ORACLE_CHUNK - 1) / ORACLE_CHUNK;
    for (int q = 0; q < n; ++q) {
        if (nseq > 0) {
            s[q].start = seq_start[q];
            s[q].len = seq_len[q];
            s[q].ckpt = seq_ckpt ? seq_ckpt[q] : 0;
        } else {
            s[q].start = (long)q * T;
            s[q].len = T;
            s[q].ckpt = (long)q * nc;
        }
    }
    *count = n;
    return s;
}

static unit_in_t unit_view(const seg_t *sg, int h, int H, int N, const double *r,
                           const double *w, const double *k, const double *v,
                           const double *a, const double *b, long *off)
{
    unit_in_t u;
    u.T = (int)sg->len;
    u.N = N;
    u.ts = (long)H * N;
    *off = (sg->start * H + h) * (long)N;
    u.r = r + *off; u.w = w + *off; u.k = k + *off;
    u.v = v + *off; u.a = a + *off; u.b = b + *off;
    return u;
}

/*
 * Forward over a batch. units: nunits (sequence, head) pairs, or NULL for all.
 * s0 / s_out: [S, H, N, N] (S = B dense, nseq in segment mode), either may be NULL.
 * ckpt: [slots, H, N, N] or NULL. Returns 0.
 */
int wkv7o_forward(int B, int T, int H, int N,
                  const double *r, const double *w, const double *k,
                  const double *v, const double *a, const double *b,
                  int nseq, const int32_t *seq_start, const int32_t *seq_len,
                  const int32_t *seq_ckpt,
                  const double *s0, double *y, double *s_out, double *ckpt,
                  int nunits, const int32_t *units, int nthreads)
{
    int S;
    seg_t *segs = make_segments(B, T, nseq, seq_start, seq_len, seq_ckpt, &S);
    const long total = units ? nunits : (long)S * H;
    const size_t NN = (size_t)N * N;
    if (nthreads > 0) omp_set_num_threads(nthreads);
    #pragma omp parallel for schedule(dynamic, 1)
    for (long q = 0; q < total; ++q) {
        const int s = units ? units[2 * q] : (int)(q / H);
        const int h = units ? units[2 * q + 1] : (int)(q % H);
        long off;
        unit_in_t u = unit_view(&segs[s], h, H, N, r, w, k, v, a, b, &off);
        const size_t sidx = ((size_t)s * H + h) * NN;
        unit_forward(&u, s0 ? s0 + sidx : NULL, y ? y + off : NULL,
                     s_out ? s_out + sidx : NULL,
                     ckpt ? ckpt + ((size_t)segs[s].ckpt * H + h) * NN : NULL,
                     (long)H * (long)NN);
    }
    free(segs);
    return 0;
}

/*
 * Backward over a batch for L = sum <dy, y> + <ds_out, S_T>.
 * dy [B,T,H,N] or NULL (= 0); ds_out [S,H,N,N] or NULL (= 0);
 * gradients are written only at tokens of the computed units.
 * Returns 0, or -1 if a unit's state history could not be allocated.
 */
int wkv7o_backward(int B, int T, int H, int N,
                   const double *r, const double *w, const double *k,
                   const double *v, const double *a, const double *b,
                   int nseq, const int32_t *seq_start, const int32_t *seq_len,
                   const double *s0, const double *dy, const double *ds_out,
                   double *dr, double *dw, double *dk, double *dv, double *da,
                   double *db, double *ds0, int nunits, const int32_t *units,
                   int nthreads)
{
    int S;
    seg_t *segs = make_segments(B, T, nseq, seq_start, seq_len, NULL, &S);
    const long total = units ? nunits : (long)S * H;
    const size_t NN = (size_t)N * N;
    int failed = 0;
    if (nthreads > 0) omp_set_num_threads(nthreads);
    #pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long q = 0; q < total; ++q) {
        const int s = units ? units[2 * q] : (int)(q / H);
        const int h = units ? units[2 * q + 1] : (int)(q % H);
        long off;
        unit_in_t u = unit_view(&segs[s], h, H, N, r, w, k, v, a, b, &off);
        const size_t sidx = ((size_t)s * H + h) * NN;
        if (unit_backward(&u, s0 ? s0 + sidx : NULL, dy ? dy + off : NULL,
                          ds_out ? ds_out + sidx : NULL,
                          dr + off, dw + off, dk + off, dv + off, da + off, db + off,
                          ds0 ? ds0 + sidx : NULL) != 0)
            failed |= 1;
    }
    free(segs);
    return failed ? -1 : 0;
}

int wkv7o_max_threads(void) { return omp_get_max_threads(); }
