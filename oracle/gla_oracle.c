/*
 * gla_oracle.c -- plain, slow, fp64 CPU oracle for the key-only gated linear
 * attention (GLA) token mixer of "GTR: Gated Token Recurrence for Efficient
 * Dense Prediction".
 *
 * TEST INFRASTRUCTURE ONLY. This is the reference the HIP path is checked
 * against. It shares no code, header, table or helper with that path, and the
 * product path never loads it: only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark do.
 *
 * What is computed (GTR summary page "GTR:门控Token循环实现高效稠密预测",
 * section 前置知识 › 门控线性注意力(GLA), and section 核心方法): for every
 * batch entry b and head h, along one scan order over the patch grid,
 *
 *     S_t = Diag(gamma_t) S_{t-1} + k_t^T v_t          (S_t is d_k x d_v)
 *     o_t = d_k^{-1/2} q_t S_t
 *
 * gamma_t = exp(log_gamma_t) is a per-key-dimension gate; the value side is
 * not decayed (key-only variant, section 核心方法 of the same page, and
 * section 3.1 of the 0539edu.com page). The state starts at zero (the
 * operator is specialised to a zero initial state, section 方法步骤详情).
 *
 * Layouts (this library's reading; the pages fix none):
 *   q, k, log_gamma : [B, L, H, d_k] row-major, float64
 *   v, o            : [B, L, H, d_v]
 *   final_state     : [B, H, d_k, d_v]  (state after the last scan step, no scale)
 *   L = grid_h * grid_w spatial tokens, p = row * grid_w + col.
 *
 * Scan orders (the pages only name them: section 核心方法 of the summary page
 * and section 3.1 of the 0539edu.com page list left->right, right->left,
 * top->bottom, bottom->top). Reading used here: dir 0 = raster order,
 * dir 1 = the whole raster reversed, dir 2 = column-major raster,
 * dir 3 = column-major raster reversed. Outputs are stored at the spatial
 * position of their token, not in scan order.
 *
 * Entry points, each independent of the others:
 *   gla_oracle_recurrent  - the recurrence above, token by token (the oracle);
 *   gla_oracle_recurrent_init - the same recurrence from a given state S_0
 *                           instead of zero (the state a preceding span of
 *                           the scan leaves; the pages' operator fixes S_0 = 0,
 *                           summary page section 方法步骤详情 step 5, so this
 *                           is the general form of that recurrence);
 *   gla_oracle_lowrank_gate - the data-dependent gate of the summary page,
 *                           section 核心方法: gamma_t = sigma(x_t W1 W2 + b)^{1/tau}
 *                           with a rank-16 factorisation W1 W2 and tau = 16, so
 *                           log_gamma = (1/tau) logsigmoid(x W1 W2 + b), per
 *                           token, over the H * d_k key dims of all heads;
 *   gla_oracle_rmsnorm_gate - the output epilogue that the end-to-end operator
 *                           fuses (0539edu.com page, appendix E.3.1): per
 *                           (batch, token, head) row of d_v outputs,
 *                           y = o / sqrt(mean(o^2) + eps) * w * SiLU(z),
 *                           SiLU(z) = z / (1 + e^{-z});
 *   gla_oracle_bruteforce - the same outputs as an explicit double sum
 *                           o_t = d_k^{-1/2} sum_{s<=t} (q_t * prod_{r=s+1..t} gamma_r) . k_s  v_s
 *                           (used only to pin the recurrence on small inputs);
 *   gla_oracle_chunked    - the three-phase chunkwise evaluation of the
 *                           summary page, section 前置知识 › Chunkwise(分块)并行
 *                           (chunk summaries U_c and decays d_c, then the
 *                           boundary scan S_[c+1] = Diag(d_c) S_[c] + U_c, then
 *                           per-chunk outputs), in fp64.
 *
 * Return value of every entry point: 0 on success, -1 on invalid arguments,
 * -2 when memory cannot be allocated.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Step t of the scan visits spatial token gla_oracle_scan_position(t). */
long gla_oracle_scan_position(long t, int grid_h, int grid_w, int dir)
{
    long L = (long)grid_h * (long)grid_w;
    if (t < 0 || t >= L) return -1;
    switch (dir) {
    case 0: /* left -> right */
        return t;
    case 1: /* right -> left */
        return L - 1 - t;
    case 2: /* top -> bottom: walk down each column, columns left to right */
        return (t % grid_h) * grid_w + t / grid_h;
    case 3: { /* bottom -> top: the top -> bottom walk, reversed */
        long u = L - 1 - t;
        return (u % grid_h) * grid_w + u / grid_h;
    }
    default:
        return -1;
    }
}

typedef struct {
    const double *q, *k, *v, *lg;
    const double *init;          /* [B, H, d_k, d_v] state before the first step, or NULL (zero) */
    int B, H, grid_h, grid_w, d_k, d_v, dir, chunk;
    double *out, *final_state;
    int nthreads, tid;
    int status;
} job_t;

static int check_args(const job_t *a)
{
    if (!a->q || !a->k || !a->v || !a->lg || !a->out) return -1;
    if (a->B < 1 || a->H < 1 || a->grid_h < 1 || a->grid_w < 1) return -1;
    if (a->d_k < 1 || a->d_v < 1 || a->dir < 0 || a->dir > 3) return -1;
    return 0;
}

/* index of element (b, p, h, e) in a [B, L, H, d] array */
static inline size_t at(const job_t *a, int b, long p, int h, int d)
{
    long L = (long)a->grid_h * a->grid_w;
    return (((size_t)b * L + (size_t)p) * a->H + h) * (size_t)d;
}

/* ---- the recurrence, one (b, h) sequence --------------------------------- */
static int recurrent_one(const job_t *a, int b, int h)
{
    const int dk = a->d_k, dv = a->d_v;
    const long L = (long)a->grid_h * a->grid_w;
    const double scale = 1.0 / sqrt((double)dk);
    double *S = calloc((size_t)dk * dv, sizeof(double));
    if (!S) return -2;
    if (a->init)
        memcpy(S, a->init + ((size_t)b * a->H + h) * dk * dv, (size_t)dk * dv * sizeof(double));
    for (long t = 0; t < L; ++t) {
        long p = gla_oracle_scan_position(t, a->grid_h, a->grid_w, a->dir);
        const double *qt = a->q + at(a, b, p, h, dk);
        const double *kt = a->k + at(a, b, p, h, dk);
        const double *gt = a->lg + at(a, b, p, h, dk);
        const double *vt = a->v + at(a, b, p, h, dv);
        double *ot = a->out + at(a, b, p, h, dv);
        /* S <- Diag(gamma_t) S + k_t^T v_t */
        for (int i = 0; i < dk; ++i) {
            double g = exp(gt[i]);
            for (int j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] = g * S[(size_t)i * dv + j] + kt[i] * vt[j];
        }
        /* o_t <- d_k^{-1/2} q_t S */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += qt[i] * S[(size_t)i * dv + j];
            ot[j] = scale * acc;
        }
    }
    if (a->final_state)
        memcpy(a->final_state + ((size_t)b * a->H + h) * dk * dv, S,
               (size_t)dk * dv * sizeof(double));
    free(S);
    return 0;
}

/* ---- the explicit double sum, one (b, h) sequence ------------------------- */
static int bruteforce_one(const job_t *a, int b, int h)
{
    const int dk = a->d_k, dv = a->d_v;
    const long L = (long)a->grid_h * a->grid_w;
    const double scale = 1.0 / sqrt((double)dk);
    double *decay = malloc((size_t)dk * sizeof(double));
    double *acc = malloc((size_t)dv * sizeof(double));
    if (!decay || !acc) { free(decay); free(acc); return -2; }
    for (long t = 0; t < L; ++t) {
        long pt = gla_oracle_scan_position(t, a->grid_h, a->grid_w, a->dir);
        const double *qt = a->q + at(a, b, pt, h, dk);
        for (int i = 0; i < dk; ++i) decay[i] = 1.0;   /* prod_{r=s+1..t} gamma_r, empty at s = t */
        for (int j = 0; j < dv; ++j) acc[j] = 0.0;
        for (long s = t; s >= 0; --s) {
            long ps = gla_oracle_scan_position(s, a->grid_h, a->grid_w, a->dir);
            const double *ks = a->k + at(a, b, ps, h, dk);
            const double *vs = a->v + at(a, b, ps, h, dv);
            const double *gs = a->lg + at(a, b, ps, h, dk);
            double score = 0.0;  /* (q_t * decay) . k_s */
            for (int i = 0; i < dk; ++i) score += qt[i] * decay[i] * ks[i];
            for (int j = 0; j < dv; ++j) acc[j] += score * vs[j];
            for (int i = 0; i < dk; ++i) decay[i] *= exp(gs[i]);  /* now covers r = s..t */
        }
        double *ot = a->out + at(a, b, pt, h, dv);
        for (int j = 0; j < dv; ++j) ot[j] = scale * acc[j];
    }
    if (a->final_state) {
        /* S_L = sum_s Diag(prod_{r=s+1..L-1} gamma_r) k_s^T v_s */
        double *F = a->final_state + ((size_t)b * a->H + h) * dk * dv;
        for (size_t e = 0; e < (size_t)dk * dv; ++e) F[e] = 0.0;
        for (int i = 0; i < dk; ++i) decay[i] = 1.0;
        for (long s = L - 1; s >= 0; --s) {
            long ps = gla_oracle_scan_position(s, a->grid_h, a->grid_w, a->dir);
            const double *ks = a->k + at(a, b, ps, h, dk);
            const double *vs = a->v + at(a, b, ps, h, dv);
            const double *gs = a->lg + at(a, b, ps, h, dk);
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    F[(size_t)i * dv + j] += decay[i] * ks[i] * vs[j];
            for (int i = 0; i < dk; ++i) decay[i] *= exp(gs[i]);
        }
    }
    free(decay);
    free(acc);
    return 0;
}

/* ---- the three-phase chunkwise form, one (b, h) sequence ------------------ */
static int chunked_one(const job_t *a, int b, int h)
{
    const int dk = a->d_k, dv = a->d_v, C = a->chunk;
    const long L = (long)a->grid_h * a->grid_w;
    const long nc = (L + C - 1) / C;
    const double scale = 1.0 / sqrt((double)dk);
    const size_t sz = (size_t)dk * dv;
    double *U = malloc((size_t)nc * sz * sizeof(double));      /* U_c          */
    double *D = malloc((size_t)nc * dk * sizeof(double));      /* d_c          */
    double *Sb = malloc((size_t)(nc + 1) * sz * sizeof(double)); /* S_[c], c=0..nc */
    double *bp = malloc((size_t)C * dk * sizeof(double));      /* local prefix */
    long *pos = malloc((size_t)C * sizeof(long));
    if (!U || !D || !Sb || !bp || !pos) {
        free(U); free(D); free(Sb); free(bp); free(pos);
        return -2;
    }

    /* phase 1: every chunk's summary, independently */
    for (long c = 0; c < nc; ++c) {
        long t0 = c * C, n = (L - t0 < C) ? (L - t0) : C;
        for (long u = 0; u < n; ++u) {
            pos[u] = gla_oracle_scan_position(t0 + u, a->grid_h, a->grid_w, a->dir);
            const double *g = a->lg + at(a, b, pos[u], h, dk);
            for (int i = 0; i < dk; ++i)
                bp[u * dk + i] = g[i] + (u ? bp[(u - 1) * dk + i] : 0.0);
        }
        double *Uc = U + c * sz;
        for (int i = 0; i < dk; ++i) D[c * dk + i] = exp(bp[(n - 1) * dk + i]);
        for (size_t e = 0; e < sz; ++e) Uc[e] = 0.0;
        for (long s = 0; s < n; ++s) {
            const double *ks = a->k + at(a, b, pos[s], h, dk);
            const double *vs = a->v + at(a, b, pos[s], h, dv);
            for (int i = 0; i < dk; ++i) {
                double w = exp(bp[(n - 1) * dk + i] - bp[s * dk + i]) * ks[i];
                for (int j = 0; j < dv; ++j) Uc[(size_t)i * dv + j] += w * vs[j];
            }
        }
    }

    /* phase 2: boundary scan S_[0] = 0, S_[c+1] = Diag(d_c) S_[c] + U_c */
    for (size_t e = 0; e < sz; ++e) Sb[e] = 0.0;
    for (long c = 0; c < nc; ++c)
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) {
                size_t e = (size_t)i * dv + j;
                Sb[(c + 1) * sz + e] = D[c * dk + i] * Sb[c * sz + e] + U[c * sz + e];
            }

    /* phase 3: every chunk's outputs, independently, from S_[c] */
    for (long c = 0; c < nc; ++c) {
        long t0 = c * C, n = (L - t0 < C) ? (L - t0) : C;
        for (long u = 0; u < n; ++u) {
            pos[u] = gla_oracle_scan_position(t0 + u, a->grid_h, a->grid_w, a->dir);
            const double *g = a->lg + at(a, b, pos[u], h, dk);
            for (int i = 0; i < dk; ++i)
                bp[u * dk + i] = g[i] + (u ? bp[(u - 1) * dk + i] : 0.0);
        }
        const double *Sc = Sb + c * sz;
        for (long t = 0; t < n; ++t) {
            const double *qt = a->q + at(a, b, pos[t], h, dk);
            double *ot = a->out + at(a, b, pos[t], h, dv);
            for (int j = 0; j < dv; ++j) ot[j] = 0.0;
            /* inter-chunk: (q_t * exp(b_t)) S_[c] */
            for (int i = 0; i < dk; ++i) {
                double w = qt[i] * exp(bp[t * dk + i]);
                for (int j = 0; j < dv; ++j) ot[j] += w * Sc[(size_t)i * dv + j];
            }
            /* intra-chunk: sum_{s<=t} ((q_t * exp(b_t - b_s)) . k_s) v_s */
            for (long s = 0; s <= t; ++s) {
                const double *ks = a->k + at(a, b, pos[s], h, dk);
                const double *vs = a->v + at(a, b, pos[s], h, dv);
                double score = 0.0;
                for (int i = 0; i < dk; ++i)
                    score += qt[i] * exp(bp[t * dk + i] - bp[s * dk + i]) * ks[i];
                for (int j = 0; j < dv; ++j) ot[j] += score * vs[j];
            }
            for (int j = 0; j < dv; ++j) ot[j] *= scale;
        }
    }
    if (a->final_state)
        memcpy(a->final_state + ((size_t)b * a->H + h) * sz, Sb + nc * sz, sz * sizeof(double));
    free(U); free(D); free(Sb); free(bp); free(pos);
    return 0;
}

/* ---- threading over the independent (b, h) sequences ---------------------- */
typedef int (*one_fn)(const job_t *, int, int);
typedef struct { job_t job; one_fn fn; } task_t;

static void *worker(void *arg)
{
    task_t *tk = (task_t *)arg;
    job_t *a = &tk->job;
    int nseq = a->B * a->H;
    for (int s = a->tid; s < nseq; s += a->nthreads) {
        int r = tk->fn(a, s / a->H, s % a->H);
        if (r) { a->status = r; break; }
    }
    return NULL;
}

static int run(job_t base, one_fn fn)
{
    if (check_args(&base)) return -1;
    int nseq = base.B * base.H;
    int nt = base.nthreads;
    if (nt < 1) nt = 1;
    if (nt > nseq) nt = nseq;
    task_t *tasks = calloc((size_t)nt, sizeof(task_t));
    pthread_t *th = calloc((size_t)nt, sizeof(pthread_t));
    if (!tasks || !th) { free(tasks); free(th); return -2; }
    for (int i = 0; i < nt; ++i) {
        tasks[i].job = base;
        tasks[i].job.nthreads = nt;
        tasks[i].job.tid = i;
        tasks[i].job.status = 0;
        tasks[i].fn = fn;
    }
    int started = 0;
    for (int i = 1; i < nt; ++i) {
        if (pthread_create(&th[i], NULL, worker, &tasks[i]) != 0) break;
        started = i;
    }
    /* threads that could not be started: thread 0 runs their share too */
    for (int i = started + 1; i < nt; ++i) {
        tasks[i].job.tid = i;
        worker(&tasks[i]);
    }
    worker(&tasks[0]);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    int status = 0;
    for (int i = 0; i < nt; ++i)
        if (tasks[i].job.status) status = tasks[i].job.status;
    free(tasks);
    free(th);
    return status;
}

static job_t make_job(const double *q, const double *k, const double *v, const double *lg,
                      int B, int H, int gh, int gw, int dk, int dv, int dir, int chunk,
                      double *out, double *fs, int nthreads)
{
    job_t a;
    memset(&a, 0, sizeof a);
    a.q = q; a.k = k; a.v = v; a.lg = lg;
    a.B = B; a.H = H; a.grid_h = gh; a.grid_w = gw; a.d_k = dk; a.d_v = dv;
    a.dir = dir; a.chunk = chunk; a.out = out; a.final_state = fs; a.nthreads = nthreads;
    return a;
}

int gla_oracle_recurrent(const double *q, const double *k, const double *v, const double *lg,
                         int B, int H, int grid_h, int grid_w, int d_k, int d_v, int dir,
                         double *out, double *final_state, int nthreads)
{
    return run(make_job(q, k, v, lg, B, H, grid_h, grid_w, d_k, d_v, dir, 0, out,
                        final_state, nthreads), recurrent_one);
}

int gla_oracle_recurrent_init(const double *q, const double *k, const double *v, const double *lg,
                              const double *init, int B, int H, int grid_h, int grid_w, int d_k,
                              int d_v, int dir, double *out, double *final_state, int nthreads)
{
    job_t a = make_job(q, k, v, lg, B, H, grid_h, grid_w, d_k, d_v, dir, 0, out, final_state,
                       nthreads);
    a.init = init;
    return run(a, recurrent_one);
}

/* Low-rank gate: x [rows, C], W1 [C, R], W2 [R, K], b [K] -> lg [rows, K],
 * lg = inv_tau * logsigmoid(x W1 W2 + b), logsigmoid(y) = -log(1 + e^{-y}). */
int gla_oracle_lowrank_gate(const double *x, const double *w1, const double *w2, const double *b,
                            double inv_tau, long rows, int C, int R, int K, double *lg)
{
    if (!x || !w1 || !w2 || !b || !lg || rows < 0 || C < 1 || R < 1 || K < 1) return -1;
    double *z = malloc((size_t)R * sizeof(double));
    if (!z) return -2;
    for (long n = 0; n < rows; ++n) {
        const double *xn = x + (size_t)n * C;
        for (int r = 0; r < R; ++r) {
            double acc = 0.0;
            for (int c = 0; c < C; ++c) acc += xn[c] * w1[(size_t)c * R + r];
            z[r] = acc;
        }
        for (int kk = 0; kk < K; ++kk) {
            double y = b[kk];
            for (int r = 0; r < R; ++r) y += z[r] * w2[(size_t)r * K + kk];
            /* log sigma(y) without overflow on either side */
            const double ls = y < 0.0 ? y - log1p(exp(y)) : -log1p(exp(-y));
            lg[(size_t)n * K + kk] = inv_tau * ls;
        }
    }
    free(z);
    return 0;
}

/* Output epilogue, row by row: rows of d values, o and z [rows, d], w [d]. */
int gla_oracle_rmsnorm_gate(const double *o, const double *z, const double *w, double eps,
                            long rows, int d, double *y)
{
    if (!o || !z || !w || !y || rows < 0 || d < 1 || !(eps >= 0.0)) return -1;
    for (long n = 0; n < rows; ++n) {
        const double *on = o + (size_t)n * d, *zn = z + (size_t)n * d;
        double *yn = y + (size_t)n * d;
        double ms = 0.0;
        for (int j = 0; j < d; ++j) ms += on[j] * on[j];
        ms /= d;
        const double inv = 1.0 / sqrt(ms + eps);
        for (int j = 0; j < d; ++j) {
            const double silu = zn[j] / (1.0 + exp(-zn[j]));
            yn[j] = on[j] * inv * w[j] * silu;
        }
    }
    return 0;
}

int gla_oracle_bruteforce(const double *q, const double *k, const double *v, const double *lg,
                          int B, int H, int grid_h, int grid_w, int d_k, int d_v, int dir,
                          double *out, double *final_state, int nthreads)
{
    return run(make_job(q, k, v, lg, B, H, grid_h, grid_w, d_k, d_v, dir, 0, out,
                        final_state, nthreads), bruteforce_one);
}

int gla_oracle_chunked(const double *q, const double *k, const double *v, const double *lg,
                       int B, int H, int grid_h, int grid_w, int d_k, int d_v, int dir,
                       int chunk, double *out, double *final_state, int nthreads)
{
    if (chunk < 1) return -1;
    return run(make_job(q, k, v, lg, B, H, grid_h, grid_w, d_k, d_v, dir, chunk, out,
                        final_state, nthreads), chunked_one);
}
