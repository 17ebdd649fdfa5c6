/*
 * Sequential FP64 oracle for the gated delta rule forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test-suite, the smoke check and the benchmark's CPU-baseline leg load
 * it.  It shares no code, header or constant with the HIP library.
 *
 * What it computes, per head (one "chain" = one (batch, head) pair, or one
 * (sequence, head) pair of a packed batch):
 *
 *   S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *   o_t = S_t q_t,            alpha_t = exp(g_t).
 *
 * This is the online-learning delta rule "change = rate x (target -
 * prediction) x input" (HyMo "Model Architecture Walkthrough", section
 * 5.2.2) with rate beta_t, target v_t, input k_t and prediction
 * alpha_t S_{t-1} k_t, applied after the per-head scalar decay exp(g_t) of
 * section 5.2.1 / 5.3.1 of the same page.  The read o_t uses the state after
 * the step's write (section 5.2.1 reads from H_t, not H_{t-1}), and there is
 * no 1/sqrt(dk) output scale (neither the pages nor the rule has one).
 *
 * The state is kept as M = S^T (dk x dv), which is the layout of h0/hT
 * (B,H,dk,dv): the pages' hidden state H_t is S x D = (key dim) x (value dim)
 * ("Model Architecture Walkthrough", section 5.2.1).  Expanding the rule in
 * this orientation:
 *
 *   p   = M^T k_t                        (= S_{t-1} k_t, length dv)
 *   M  <- alpha M + beta k_t (v_t - alpha p)^T
 *   o_t = M^T q_t
 *
 * Strictly sequential in t; independent chains run on separate threads.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *h0;
    const int32_t *cu_seqlens;
    double *out, *hT;
    int B, T, H, dk, dv;
    const int32_t *chains;  /* chain ids (b*H + h) to compute, or NULL = all */
    int nchains;
    int next;               /* work counter, guarded by lock */
    pthread_mutex_t lock;
} job_t;

/* One chain: tokens [t0, t1) of sequence/batch row `b`, head `h`.  Token
 * `t` of the chain lives at flat row index (rowbase + t) of the (rows,H,d)
 * tensors. */
static void run_chain(const job_t *J, int b, int h, double *M, double *p) {
    const int H = J->H, dk = J->dk, dv = J->dv;
    long rowbase, len;
    if (J->cu_seqlens) {
        rowbase = J->cu_seqlens[b];
        len = (long)J->cu_seqlens[b + 1] - J->cu_seqlens[b];
    } else {
        rowbase = (long)b * J->T;
        len = J->T;
    }
    const long sidx = ((long)b * H + h) * (long)dk * dv;
    if (J->h0)
        memcpy(M, J->h0 + sidx, sizeof(double) * (size_t)dk * dv);
    else
        memset(M, 0, sizeof(double) * (size_t)dk * dv);

    for (long t = 0; t < len; ++t) {
        const long row = (rowbase + t) * H + h;
        const double *qt = J->q + row * dk;
        const double *kt = J->k + row * dk;
        const double *vt = J->v + row * dv;
        const double alpha = exp(J->g[row]);
        const double beta = J->beta[row];
        double *ot = J->out + row * dv;

        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double ki = kt[i];
            const double *Mi = M + (long)i * dv;
            for (int j = 0; j < dv; ++j) p[j] += Mi[j] * ki;
        }
        /* p <- beta (v - alpha p): the error-correcting write direction */
        for (int j = 0; j < dv; ++j) p[j] = beta * (vt[j] - alpha * p[j]);
        for (int i = 0; i < dk; ++i) {
            const double ki = kt[i];
            double *Mi = M + (long)i * dv;
            for (int j = 0; j < dv; ++j) Mi[j] = alpha * Mi[j] + ki * p[j];
        }
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double qi = qt[i];
            const double *Mi = M + (long)i * dv;
            for (int j = 0; j < dv; ++j) ot[j] += Mi[j] * qi;
        }
    }
    memcpy(J->hT + sidx, M, sizeof(double) * (size_t)dk * dv);
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    double *M = (double *)malloc(sizeof(double) * (size_t)J->dk * J->dv);
    double *p = (double *)malloc(sizeof(double) * (size_t)J->dv);
    const int total = J->chains ? J->nchains : J->B * J->H;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int w = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (w >= total) break;
        const int c = J->chains ? J->chains[w] : w;
        run_chain(J, c / J->H, c % J->H, M, p);
    }
    free(M);
    free(p);
    return NULL;
}

/*
 * Layouts (row-major, float64):
 *   dense  (cu_seqlens == NULL): q,k (B,T,H,dk); v,out (B,T,H,dv); g,beta (B,T,H)
 *   packed (cu_seqlens != NULL): the same without B, T = packed total;
 *                                cu_seqlens has B+1 non-decreasing offsets.
 *   h0 (B,H,dk,dv) or NULL (zero state); hT (B,H,dk,dv).
 * `chains` selects a subset of chain ids b*H+h (NULL = all); outputs of other
 * chains are left untouched.  Returns 0, or -1 on a bad argument.
 */
int gdn_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *h0,
                   const int32_t *cu_seqlens, double *out, double *hT,
                   int B, int T, int H, int dk, int dv,
                   const int32_t *chains, int nchains, int nthreads) {
    if (!q || !k || !v || !g || !beta || !out || !hT) return -1;
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (chains && nchains < 0) return -1;
    if (chains)
        for (int i = 0; i < nchains; ++i)
            if (chains[i] < 0 || chains[i] >= B * H) return -1;
    if (cu_seqlens) {
        if (cu_seqlens[0] != 0 || cu_seqlens[B] != T) return -1;
        for (int b = 0; b < B; ++b)
            if (cu_seqlens[b + 1] < cu_seqlens[b]) return -1;
    }
    job_t J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0;
    J.cu_seqlens = cu_seqlens; J.out = out; J.hT = hT;
    J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv;
    J.chains = chains; J.nchains = nchains; J.next = 0;
    pthread_mutex_init(&J.lock, NULL);
    const int total = chains ? nchains : B * H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > total) nthreads = total > 0 ? total : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return 0;
}
