/* Host sanitizer driver for the fp64 oracle (built with -fsanitize=address,undefined
 * by tests/test_host_sanitizers.py): every oracle function on small shapes, all four
 * scan orders, one and several threads, ragged chunks, plus its argument checks.
 * The recurrence, the quadratic form and the chunked form must agree; any memory
 * or undefined-behaviour error aborts the run. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int gla_oracle_recurrent(const double *, const double *, const double *, const double *, int,
                         int, int, int, int, int, int, double *, double *, int);
int gla_oracle_recurrent_init(const double *, const double *, const double *, const double *,
                              const double *, int, int, int, int, int, int, int, double *,
                              double *, int);
int gla_oracle_bruteforce(const double *, const double *, const double *, const double *, int,
                          int, int, int, int, int, int, double *, double *, int);
int gla_oracle_chunked(const double *, const double *, const double *, const double *, int, int,
                       int, int, int, int, int, int, double *, double *, int);
int gla_oracle_lowrank_gate(const double *, const double *, const double *, const double *,
                            double, long, int, int, int, double *);
int gla_oracle_rmsnorm_gate(const double *, const double *, const double *, double, long, int,
                            double *);
long gla_oracle_scan_position(long, int, int, int);

static unsigned long long rng = 88172645463325252ull;
static double uniform(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double *fill(size_t n, int negative)
{
    double *p = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = negative ? -0.3 * fabs(uniform()) : uniform();
    return p;
}
static double maxdiff(const double *a, const double *b, size_t n)
{
    double m = 0.0, s = 0.0;
    for (size_t i = 0; i < n; ++i) {
        m = fmax(m, fabs(a[i] - b[i]));
        s = fmax(s, fabs(b[i]));
    }
    return s > 0 ? m / s : m;
}

int main(void)
{
    const int shapes[][6] = {{1, 1, 3, 5, 4, 3}, {2, 2, 7, 9, 8, 16}, {1, 3, 1, 13, 5, 7},
                             {1, 1, 1, 1, 2, 2}, {1, 1, 11, 1, 3, 1}};
    const int chunks[] = {1, 3, 16, 64, 1000};
    int fails = 0;
    for (size_t si = 0; si < sizeof shapes / sizeof shapes[0]; ++si) {
        const int B = shapes[si][0], H = shapes[si][1], gh = shapes[si][2], gw = shapes[si][3];
        const int dk = shapes[si][4], dv = shapes[si][5];
        const size_t L = (size_t)gh * gw, nk = B * L * H * dk, nv = B * L * H * dv;
        const size_t ns = (size_t)B * H * dk * dv;
        double *q = fill(nk, 0), *k = fill(nk, 0), *v = fill(nv, 0), *lg = fill(nk, 1);
        double *s0 = fill(ns, 0);
        double *o1 = malloc(nv * sizeof(double)), *o2 = malloc(nv * sizeof(double));
        double *f1 = malloc(ns * sizeof(double)), *f2 = malloc(ns * sizeof(double));
        for (int dir = 0; dir < 4; ++dir) {
            for (long t = 0; t < (long)L; ++t) {
                const long p = gla_oracle_scan_position(t, gh, gw, dir);
                if (p < 0 || p >= (long)L) ++fails;
            }
            for (int th = 1; th <= 3; th += 2) {
                if (gla_oracle_recurrent(q, k, v, lg, B, H, gh, gw, dk, dv, dir, o1, f1, th)) ++fails;
                if (gla_oracle_bruteforce(q, k, v, lg, B, H, gh, gw, dk, dv, dir, o2, f2, th)) ++fails;
                if (maxdiff(o2, o1, nv) > 1e-10 || maxdiff(f2, f1, ns) > 1e-10) ++fails;
                for (size_t ci = 0; ci < sizeof chunks / sizeof chunks[0]; ++ci) {
                    if (gla_oracle_chunked(q, k, v, lg, B, H, gh, gw, dk, dv, dir, chunks[ci], o2,
                                           f2, th))
                        ++fails;
                    if (maxdiff(o2, o1, nv) > 1e-10 || maxdiff(f2, f1, ns) > 1e-10) ++fails;
                }
                if (gla_oracle_recurrent_init(q, k, v, lg, s0, B, H, gh, gw, dk, dv, dir, o2, f2, th))
                    ++fails;
            }
        }
        /* argument checks: no crash, an error code */
        if (gla_oracle_recurrent(NULL, k, v, lg, B, H, gh, gw, dk, dv, 0, o1, f1, 1) == 0) ++fails;
        if (gla_oracle_recurrent(q, k, v, lg, 0, H, gh, gw, dk, dv, 0, o1, f1, 1) == 0) ++fails;
        if (gla_oracle_recurrent(q, k, v, lg, B, H, gh, gw, dk, dv, 4, o1, f1, 1) == 0) ++fails;
        if (gla_oracle_chunked(q, k, v, lg, B, H, gh, gw, dk, dv, 0, 0, o1, f1, 1) == 0) ++fails;
        free(q), free(k), free(v), free(lg), free(s0), free(o1), free(o2), free(f1), free(f2);
    }
    {   /* gate and epilogue */
        const long rows = 37;
        const int C = 19, R = 16, K = 24, d = 24;
        double *x = fill(rows * C, 0), *w1 = fill(C * R, 0), *w2 = fill(R * K, 0), *b = fill(K, 0);
        double *lg = malloc(rows * K * sizeof(double)), *y = malloc(rows * d * sizeof(double));
        double *w = fill(d, 0);
        if (gla_oracle_lowrank_gate(x, w1, w2, b, 1.0 / 16, rows, C, R, K, lg)) ++fails;
        for (long i = 0; i < rows * K; ++i)
            if (!(lg[i] <= 0.0)) ++fails;
        if (gla_oracle_rmsnorm_gate(lg, lg, w, 1e-5, rows, d, y)) ++fails;
        if (gla_oracle_lowrank_gate(x, w1, w2, b, 1.0 / 16, rows, 0, R, K, lg) == 0) ++fails;
        if (gla_oracle_rmsnorm_gate(lg, lg, w, -1.0, rows, d, y) == 0) ++fails;
        free(x), free(w1), free(w2), free(b), free(lg), free(y), free(w);
    }
    printf("oracle sanitizer driver: %d failures\n", fails);
    return fails ? 1 : 0;
}
