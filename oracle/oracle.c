/*
 * CPU oracle for the exact attention forward pass. TEST INFRASTRUCTURE ONLY:
 * the tests, the smoke check and the benchmark's CPU-baseline leg call it; the
 * HIP library never does, and the two share no code.
 *
 * What it computes is the plain definition of scaled dot-product attention,
 * Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V (aiinarabic.com
 * "flash-attention" page, equation (1); inskillml course module 9, "Where n^2
 * comes from"), written out in float64 with every softmax row materialised,
 * i.e. the standard (unfused) attention the pages contrast the fused kernel
 * with (aiinarabic.com page, Figure 3: S is formed, then softmax, then the
 * product with V). The fused method reaches this same result up to rounding
 * (inskillml module 9, "FlashAttention: compute without writing the
 * weights": it is not an approximation).
 *
 * Per query row i of head (b, h):
 *   i' = i + (Nk - Nq)                       (bottom-right causal alignment)
 *   J  = { j < Nk : (!causal || j <= i') && (window == 0 || j > i' - window) }
 *   s_j = scale * sum_d Q[i,d] K[j,d]        for j in J only
 *   m = max_j s_j;  e_j = exp(s_j - m);  l = sum_j e_j
 *   P_j = e_j / l                             (the materialised softmax row)
 *   O[i,d] = sum_j P_j V[j,d];  LSE[i] = m + ln(l)
 * An empty J gives O[i,:] = 0 and LSE[i] = -inf.
 * The causal mask follows the SDPA call with is_causal=True in the inskillml
 * module; the window keeps the w keys i-w < j <= i (a causal sliding window;
 * the same module's "Sparse patterns" section names sliding windows).
 *
 * oracle_attn_fwd_window takes the mask as two extents instead:
 *   J  = { j < Nk : (wl < 0 || j >= i' - wl) && (wr < 0 || j <= i' + wr) }
 * This is the sliding window of that "Sparse patterns" section, where each
 * token sees the w tokens on either side of it (its example mask keeps columns
 * max(0, i-w) .. min(n, i+w+1)-1 of row i), with the two sides allowed to
 * differ and a negative extent leaving a side open.
 *
 * oracle_attn_fwd_mod adds a score modifier, applied to each visible s_j
 * before the softmax (FLASHLIGHT's score_mod variants in the gist.science
 * summary, Results: ALiBi and Softcap):
 *   softcap: s_j <- cap * tanh(s_j / cap)
 *   ALiBi:   s_j <- s_j + slope[h] * (j - i')      (h the head of the row)
 *
 * Inputs are float64 arrays the caller decoded exactly from the storage
 * dtype. Layout: Q [B,H,Nq,D], K and V [B,H,Nk,D], contiguous.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v;
    double *o, *lse;
    long B, H, Nq, Nk, D, window;
    double scale;
    int causal;
    int extents;        /* 1: the mask is (wl, wr) below, not (causal, window) */
    long wl, wr;
    int mod;            /* 0 none, 1 softcap, 2 ALiBi */
    double cap;
    const double *slopes;   /* [H] for ALiBi */
    const long *rows;   /* flattened (b*H + h)*Nq + i, or NULL for every row */
    long nrows;
    long next;          /* work counter, shared */
    pthread_mutex_t lock;
    int bad;            /* set if a softmax row failed to sum to one */
} job_t;

/* One query row, following the definition above step by step. */
static int one_row(const job_t *jb, long flat, double *s, double *o_row, double *lse_out)
{
    const long D = jb->D, Nq = jb->Nq, Nk = jb->Nk;
    const long bh = flat / Nq, i = flat % Nq;
    const double *qi = jb->q + flat * D;
    const double *K = jb->k + bh * Nk * D;
    const double *V = jb->v + bh * Nk * D;
    const long ip = i + (Nk - Nq);

    /* Visible keys J_i: j in [lo, hi). */
    long lo = 0, hi = Nk;
    if (jb->extents) {
        if (jb->wl >= 0) lo = ip - jb->wl > 0 ? ip - jb->wl : 0;
        if (jb->wr >= 0) hi = ip + jb->wr + 1 < Nk ? ip + jb->wr + 1 : Nk;
    } else {
        if (jb->causal) hi = ip + 1 < Nk ? ip + 1 : Nk;
        if (jb->window > 0) lo = ip - jb->window + 1 > 0 ? ip - jb->window + 1 : 0;
    }
    if (hi < 0) hi = 0;
    if (lo > hi) lo = hi;

    for (long d = 0; d < D; ++d) o_row[d] = 0.0;
    if (hi == lo) {
        *lse_out = -INFINITY;
        return 0;
    }

    /* Scores s_j = scale * q_i . k_j */
    for (long j = lo; j < hi; ++j) {
        const double *kj = K + j * D;
        double dot = 0.0;
        for (long d = 0; d < D; ++d) dot += qi[d] * kj[d];
        s[j - lo] = jb->scale * dot;
    }
    /* Score modifier. */
    if (jb->mod == 1) {
        for (long j = lo; j < hi; ++j) s[j - lo] = jb->cap * tanh(s[j - lo] / jb->cap);
    } else if (jb->mod == 2) {
        const double slope = jb->slopes[bh % jb->H];
        for (long j = lo; j < hi; ++j) s[j - lo] += slope * (double)(j - ip);
    }
    /* Softmax of the row: max, exponentials, sum, normalise. */
    double m = s[0];
    for (long j = 1; j < hi - lo; ++j) if (s[j] > m) m = s[j];
    double l = 0.0;
    for (long j = 0; j < hi - lo; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    double psum = 0.0;
    for (long j = 0; j < hi - lo; ++j) {
        s[j] = s[j] / l;
        psum += s[j];
    }
    /* P times V */
    for (long j = lo; j < hi; ++j) {
        const double p = s[j - lo];
        const double *vj = V + j * D;
        for (long d = 0; d < D; ++d) o_row[d] += p * vj[d];
    }
    *lse_out = m + log(l);
    return fabs(psum - 1.0) <= 1e-12 ? 0 : 1;
}

static void *worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)(jb->Nk > 0 ? jb->Nk : 1));
    int bad = 0;
    const long total = jb->rows ? jb->nrows : jb->B * jb->H * jb->Nq;
    const long grab = 16;
    for (;;) {
        pthread_mutex_lock(&jb->lock);
        long r0 = jb->next;
        jb->next += grab;
        pthread_mutex_unlock(&jb->lock);
        if (r0 >= total) break;
        long r1 = r0 + grab < total ? r0 + grab : total;
        for (long r = r0; r < r1; ++r) {
            long flat = jb->rows ? jb->rows[r] : r;
            bad |= one_row(jb, flat, s, jb->o + r * jb->D, jb->lse + r);
        }
    }
    free(s);
    if (bad) {
        pthread_mutex_lock(&jb->lock);
        jb->bad = 1;
        pthread_mutex_unlock(&jb->lock);
    }
    return NULL;
}

/*
 * Computes O and LSE for the requested rows.
 *   rows == NULL: every row; o is [B,H,Nq,D] and lse [B,H,Nq].
 *   rows != NULL: nrows flattened row ids; o is [nrows,D] and lse [nrows].
 * Returns 0 on success, 1 if some softmax row failed the sum-to-one check,
 * -1 on bad arguments.
 */
static int run_job(job_t *jbp, int nthreads);

int oracle_attn_fwd(const double *q, const double *k, const double *v, double *o, double *lse,
                    long B, long H, long Nq, long Nk, long D, double scale, int causal,
                    long window, const long *rows, long nrows, int nthreads)
{
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || D <= 0 || window < 0 || nthreads <= 0) return -1;
    job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.q = q; jb.k = k; jb.v = v; jb.o = o; jb.lse = lse;
    jb.B = B; jb.H = H; jb.Nq = Nq; jb.Nk = Nk; jb.D = D;
    jb.window = window; jb.scale = scale; jb.causal = causal;
    jb.rows = rows; jb.nrows = nrows;
    return run_job(&jb, nthreads);
}

/* The same with the mask as the extents (wl, wr); a negative extent is open. */
int oracle_attn_fwd_window(const double *q, const double *k, const double *v, double *o, double *lse,
                           long B, long H, long Nq, long Nk, long D, double scale, long wl, long wr,
                           const long *rows, long nrows, int nthreads)
{
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || D <= 0 || nthreads <= 0) return -1;
    job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.q = q; jb.k = k; jb.v = v; jb.o = o; jb.lse = lse;
    jb.B = B; jb.H = H; jb.Nq = Nq; jb.Nk = Nk; jb.D = D;
    jb.scale = scale; jb.extents = 1; jb.wl = wl; jb.wr = wr;
    jb.rows = rows; jb.nrows = nrows;
    return run_job(&jb, nthreads);
}

/* The extents mask with a score modifier: mod 1 softcap (cap > 0), mod 2
   ALiBi (slopes[H]). */
int oracle_attn_fwd_mod(const double *q, const double *k, const double *v, double *o, double *lse,
                        long B, long H, long Nq, long Nk, long D, double scale, long wl, long wr,
                        int mod, double cap, const double *slopes,
                        const long *rows, long nrows, int nthreads)
{
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || D <= 0 || nthreads <= 0) return -1;
    if (mod < 0 || mod > 2 || (mod == 1 && !(cap > 0.0)) || (mod == 2 && !slopes)) return -1;
    job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.q = q; jb.k = k; jb.v = v; jb.o = o; jb.lse = lse;
    jb.B = B; jb.H = H; jb.Nq = Nq; jb.Nk = Nk; jb.D = D;
    jb.scale = scale; jb.extents = 1; jb.wl = wl; jb.wr = wr;
    jb.mod = mod; jb.cap = cap; jb.slopes = slopes;
    jb.rows = rows; jb.nrows = nrows;
    return run_job(&jb, nthreads);
}

static int run_job(job_t *jbp, int nthreads)
{
    job_t jb = *jbp;
    pthread_mutex_init(&jb.lock, NULL);
    if (nthreads > 256) nthreads = 256;
    pthread_t tid[256];
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&tid[started], NULL, worker, &jb) == 0) ++started;
    worker(&jb);
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
    pthread_mutex_destroy(&jb.lock);
    return jb.bad ? 1 : 0;
}

/*
 * Backward pass (the gradients of O with respect to Q, K, V, contracted with
 * an upstream gradient dO). The pages' method recomputes the softmax weights
 * in the backward pass from Q, K and the stored normaliser instead of keeping
 * them (aiinarabic.com flash-attention page, the recomputation paragraph);
 * what it computes is the plain derivative of O = softmax(scale Q K^T) V:
 *   P_j   = exp(s_j - LSE)                 the softmax row, s_j = scale q_i.k_j
 *   dV_j += P_j dO_i
 *   dP_j  = dO_i . V_j
 *   Dv    = sum_j P_j dP_j                  (= dO_i . O_i)
 *   dS_j  = P_j (dP_j - Dv)                 (the softmax Jacobian applied)
 *   dQ_i  = scale sum_j dS_j K_j
 *   dK_j += scale dS_j Q_i
 * over the visible keys J_i of the extents mask (wl, wr; negative = open).
 * With a score modifier s_j <- f(s_j) (softcap or ALiBi, as in the forward),
 * P_j is the softmax of the modified scores and the chain rule multiplies the
 * softmax gradient by f'(s_j):
 *   softcap: f(x) = cap tanh(x / cap),  f'(x) = 1 - tanh(x / cap)^2
 *   ALiBi:   f(x) = x + slope[h] (j - i'),  f'(x) = 1
 * Rows are taken in order within a head; heads run in parallel threads.
 */
typedef struct {
    const double *q, *k, *v, *dout;
    double *dq, *dk, *dv;
    long B, H, Nq, Nk, D, wl, wr;
    double scale;
    int mod;                /* 0 none, 1 softcap, 2 ALiBi */
    double cap;
    const double *slopes;   /* [H] for ALiBi */
    long next;
    pthread_mutex_t lock;
} bjob_t;

static void bwd_head(const bjob_t *jb, long bh, double *s, double *dp, double *g)
{
    const long D = jb->D, Nq = jb->Nq, Nk = jb->Nk;
    const double *Q = jb->q + bh * Nq * D, *K = jb->k + bh * Nk * D, *V = jb->v + bh * Nk * D;
    const double *dO = jb->dout + bh * Nq * D;
    double *dQ = jb->dq + bh * Nq * D, *dK = jb->dk + bh * Nk * D, *dV = jb->dv + bh * Nk * D;
    for (long x = 0; x < Nq * D; ++x) dQ[x] = 0.0;
    for (long x = 0; x < Nk * D; ++x) { dK[x] = 0.0; dV[x] = 0.0; }
    for (long i = 0; i < Nq; ++i) {
        const long ip = i + Nk - Nq;
        long lo = 0, hi = Nk;
        if (jb->wl >= 0 && ip - jb->wl > 0) lo = ip - jb->wl;
        if (jb->wr >= 0 && ip + jb->wr + 1 < Nk) hi = ip + jb->wr + 1;
        if (hi <= lo) continue;
        const double *qi = Q + i * D, *doi = dO + i * D;
        /* the softmax row of the modified scores, materialised, and f' */
        double m = -INFINITY;
        for (long j = lo; j < hi; ++j) {
            double dot = 0.0;
            for (long d = 0; d < D; ++d) dot += qi[d] * K[j * D + d];
            s[j - lo] = dot * jb->scale;
            g[j - lo] = 1.0;
            if (jb->mod == 1) {
                const double t = tanh(s[j - lo] / jb->cap);
                s[j - lo] = jb->cap * t;
                g[j - lo] = 1.0 - t * t;
            } else if (jb->mod == 2) {
                s[j - lo] += jb->slopes[bh % jb->H] * (double)(j - ip);
            }
            if (s[j - lo] > m) m = s[j - lo];
        }
        double l = 0.0;
        for (long j = lo; j < hi; ++j) l += exp(s[j - lo] - m);
        const double lse = m + log(l);
        double dv_row = 0.0;
        for (long j = lo; j < hi; ++j) {
            const double p = exp(s[j - lo] - lse);
            s[j - lo] = p;
            double x = 0.0;
            for (long d = 0; d < D; ++d) x += doi[d] * V[j * D + d];
            dp[j - lo] = x;
            dv_row += p * x;
            for (long d = 0; d < D; ++d) dV[j * D + d] += p * doi[d];
        }
        for (long j = lo; j < hi; ++j) {
            const double dsm = s[j - lo] * (dp[j - lo] - dv_row);   /* w.r.t. the modified score */
            const double ds = dsm * g[j - lo];                       /* w.r.t. scale q.k */
            for (long d = 0; d < D; ++d) {
                dQ[i * D + d] += jb->scale * ds * K[j * D + d];
                dK[j * D + d] += jb->scale * ds * qi[d];
            }
        }
    }
}

static void *bwd_worker(void *arg)
{
    bjob_t *jb = (bjob_t *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)(jb->Nk > 0 ? jb->Nk : 1));
    double *dp = (double *)malloc(sizeof(double) * (size_t)(jb->Nk > 0 ? jb->Nk : 1));
    double *g = (double *)malloc(sizeof(double) * (size_t)(jb->Nk > 0 ? jb->Nk : 1));
    for (;;) {
        pthread_mutex_lock(&jb->lock);
        const long bh = jb->next++;
        pthread_mutex_unlock(&jb->lock);
        if (bh >= jb->B * jb->H) break;
        bwd_head(jb, bh, s, dp, g);
    }
    free(s);
    free(dp);
    free(g);
    return NULL;
}

/* dQ [B,H,Nq,D], dK and dV [B,H,Nk,D] of the extents-masked attention with
   a score modifier: mod 0 none, 1 softcap (cap > 0), 2 ALiBi (slopes[H]). */
int oracle_attn_bwd_mod(const double *q, const double *k, const double *v, const double *dout,
                        double *dq, double *dk, double *dv, long B, long H, long Nq, long Nk, long D,
                        double scale, long wl, long wr, int mod, double cap, const double *slopes,
                        int nthreads)
{
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || D <= 0 || nthreads <= 0) return -1;
    if (mod < 0 || mod > 2 || (mod == 1 && !(cap > 0.0)) || (mod == 2 && !slopes)) return -1;
    bjob_t jb;
    memset(&jb, 0, sizeof jb);
    jb.q = q; jb.k = k; jb.v = v; jb.dout = dout; jb.dq = dq; jb.dk = dk; jb.dv = dv;
    jb.B = B; jb.H = H; jb.Nq = Nq; jb.Nk = Nk; jb.D = D; jb.wl = wl; jb.wr = wr; jb.scale = scale;
    jb.mod = mod; jb.cap = cap; jb.slopes = slopes;
    pthread_mutex_init(&jb.lock, NULL);
    if (nthreads > 256) nthreads = 256;
    pthread_t tid[256];
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&tid[started], NULL, bwd_worker, &jb) == 0) ++started;
    bwd_worker(&jb);
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
    pthread_mutex_destroy(&jb.lock);
    return 0;
}

/* The same without a score modifier. */
int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dout,
                    double *dq, double *dk, double *dv, long B, long H, long Nq, long Nk, long D,
                    double scale, long wl, long wr, int nthreads)
{
    return oracle_attn_bwd_mod(q, k, v, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, wl, wr, 0, 0.0, NULL,
                               nthreads);
}
