/*
 * Runs every entry point of the oracle (oracle/ssm_oracle.c) on exact-size
 * heap buffers under AddressSanitizer and UndefinedBehaviorSanitizer (built
 * and run by tests/test_sanitize.py): an out-of-bounds access, a use of
 * freed memory or undefined arithmetic in the oracle's indexing aborts the
 * run.  Shapes cover L = 1, ragged lengths, every state size, conv widths
 * shorter and longer than the sequence, and the optional arguments present
 * or absent, on one and on several threads.  Values are arbitrary; only the
 * memory behaviour is checked here (the pins check the values).
 */
#include <stdio.h>
#include <stdlib.h>

int ssm_oracle_scan_f64(int, int, int, int, int, const double *, const double *, const double *,
                        const double *, const double *, const double *, const double *,
                        const double *, const double *, double *, double *, int);
int ssm_oracle_state_update_f64(int, int, int, int, double *, const double *, const double *,
                                const double *, const double *, const double *, const double *,
                                const double *, const double *, double *, int);
int ssm_oracle_conv1d_f64(int, int, int, int, int, const double *, const double *,
                          const double *, const double *, double *, double *, int);
int ssm_oracle_conv1d_update_f64(int, int, int, int, double *, const double *, const double *,
                                 const double *, double *, int);
int ssm_oracle_scan_bwd_f64(int, int, int, int, int, const double *, const double *,
                            const double *, const double *, const double *, const double *,
                            const double *, const double *, const double *, const double *,
                            const double *, double *, double *, double *, double *, double *,
                            double *, double *, double *, double *, int);

static unsigned long long rng = 88172645463325252ull;

static double *buf(size_t n)
{
    double *p = malloc((n ? n : 1) * sizeof(double));
    if (!p) exit(3);
    for (size_t i = 0; i < n; ++i) {
        rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
        p[i] = (double)(rng % 2001) / 1000.0 - 1.0;
    }
    return p;
}

#define CHECK(call)                                                        \
    do {                                                                   \
        int rc_ = (call);                                                  \
        if (rc_ != 0) {                                                    \
            fprintf(stderr, "%s returned %d at line %d\n", #call, rc_, __LINE__); \
            return 1;                                                      \
        }                                                                  \
    } while (0)

static int scan_case(int B, int D, int L, int N, int zoh, int opt, int nt)
{
    size_t s = (size_t)B * D * L, bc = (size_t)B * N * L, st = (size_t)B * D * N;
    double *x = buf(s), *dt = buf(s), *z = buf(s), *bias = buf(D), *A = buf((size_t)D * N);
    double *Bm = buf(bc), *Cm = buf(bc), *Dk = buf(D), *h0 = buf(st), *y = buf(s), *hL = buf(st);
    for (size_t i = 0; i < (size_t)D * N; ++i) A[i] = -1.0 - (double)(i % N);
    CHECK(ssm_oracle_scan_f64(B, D, L, N, zoh, x, dt, opt ? bias : NULL, A, Bm, Cm,
                              opt ? Dk : NULL, opt ? z : NULL, opt ? h0 : NULL, y,
                              opt ? hL : NULL, nt));
    double *dy = buf(s), *dhL = buf(st), *dx = buf(s), *ddt = buf(s), *dbias = buf(D);
    double *dA = buf((size_t)D * N), *dB = buf(bc), *dC = buf(bc), *dD = buf(D), *dz = buf(s);
    double *dh0 = buf(st);
    CHECK(ssm_oracle_scan_bwd_f64(B, D, L, N, zoh, x, dt, opt ? bias : NULL, A, Bm, Cm,
                                  opt ? Dk : NULL, opt ? z : NULL, opt ? h0 : NULL, dy,
                                  opt ? dhL : NULL, dx, ddt, dbias, dA, dB, dC, dD,
                                  opt ? dz : NULL, opt ? dh0 : NULL, nt));
    /* the decode step on the [B][D][N] state with [B][D] / [B][N] inputs */
    CHECK(ssm_oracle_state_update_f64(B, D, N, zoh, h0, x, dt, opt ? bias : NULL, A, Bm, Cm,
                                      opt ? Dk : NULL, opt ? z : NULL, y, nt));
    double *ps[] = {x, dt, z, bias, A, Bm, Cm, Dk, h0, y, hL, dy, dhL, dx, ddt, dbias, dA, dB,
                    dC, dD, dz, dh0};
    for (size_t i = 0; i < sizeof ps / sizeof ps[0]; ++i) free(ps[i]);
    return 0;
}

static int conv_case(int B, int D, int L, int W, int opt, int nt)
{
    size_t s = (size_t)B * D * L, st = (size_t)B * D * (W - 1);
    double *x = buf(s), *w = buf((size_t)D * W), *b = buf(D), *s0 = buf(st), *y = buf(s);
    double *sL = buf(st), *x1 = buf((size_t)B * D), *y1 = buf((size_t)B * D);
    CHECK(ssm_oracle_conv1d_f64(B, D, L, W, opt, x, w, opt ? b : NULL, opt ? s0 : NULL, y,
                                opt ? sL : NULL, nt));
    CHECK(ssm_oracle_conv1d_f64(B, D, L, W, 1, x, w, b, s0, y, s0, nt));  /* stateL == state0 */
    CHECK(ssm_oracle_conv1d_update_f64(B, D, W, opt, s0, x1, w, opt ? b : NULL, y1, nt));
    double *ps[] = {x, w, b, s0, y, sL, x1, y1};
    for (size_t i = 0; i < sizeof ps / sizeof ps[0]; ++i) free(ps[i]);
    return 0;
}

int main(void)
{
    const int shapes[][4] = {{1, 1, 1, 1}, {1, 3, 7, 2}, {2, 5, 64, 4}, {3, 17, 129, 8},
                             {2, 4, 300, 16}, {1, 2, 1000, 16}};
    for (size_t k = 0; k < sizeof shapes / sizeof shapes[0]; ++k)
        for (int zoh = 0; zoh < 2; ++zoh)
            for (int opt = 0; opt < 2; ++opt)
                for (int nt = 1; nt <= 3; nt += 2)
                    if (scan_case(shapes[k][0], shapes[k][1], shapes[k][2], shapes[k][3], zoh, opt,
                                  nt))
                        return 1;
    const int cshapes[][4] = {{1, 1, 1, 2}, {2, 3, 2, 4}, {1, 5, 3, 3}, {3, 7, 100, 4},
                              {2, 9, 40, 2}};
    for (size_t k = 0; k < sizeof cshapes / sizeof cshapes[0]; ++k)
        for (int opt = 0; opt < 2; ++opt)
            for (int nt = 1; nt <= 3; nt += 2)
                if (conv_case(cshapes[k][0], cshapes[k][1], cshapes[k][2], cshapes[k][3], opt, nt))
                    return 1;
    printf("oracle sanitizer run: ok\n");
    return 0;
}
