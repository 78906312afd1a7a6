/*
 * Runs every oracle entry point once on small seeded inputs (float32 and bfloat16, ragged
 * lengths, groups, separate reverse parameters, per-channel skip weights, the convolution)
 * so that a build with AddressSanitizer and UndefinedBehaviorSanitizer sees every array
 * access and integer operation of the oracle. Exits non-zero if a call rejects valid
 * arguments or returns a non-finite value; the sanitizers report any memory or undefined-
 * behaviour error themselves (and abort).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t batch, nheads, headdim, d_state, ngroups, in_dtype;
} dims_t;
typedef struct {
    const void *x, *dt, *B, *C;
} seq_t;

int oracle_scan(const dims_t *, int64_t, int64_t, const seq_t *, const float *, const float *, const double *,
                double *, double *, double *, const int8_t *, int);
int oracle_block_step_ex(const dims_t *, int64_t, const double *, const seq_t *, const seq_t *, const float *,
                         const float *, const float *, const float *, double *, double *, double *, const int8_t *,
                         int);
int oracle_block_step_dch(const dims_t *, int64_t, const double *, const seq_t *, const seq_t *, const float *,
                          const float *, const float *, const float *, double *, const int8_t *, int);
int oracle_commit(const dims_t *, int64_t, const seq_t *, const float *, const float *, double *, double *,
                  const int8_t *, int);
int oracle_full_window(const dims_t *, int64_t, const seq_t *, const seq_t *, const float *, const float *,
                       const float *, const float *, double *, const int8_t *, int);
int oracle_conv(const dims_t *, int64_t, int32_t, int32_t, int32_t, const float *, const float *, const void *,
                const seq_t *, const seq_t *, void *, int);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void)  /* splitmix64 -> [0, 1) */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}

static void *fill(int dtype, int64_t n, double lo, double hi)
{
    void *p = malloc((size_t)n * (dtype ? 2 : 4));
    for (int64_t i = 0; i < n; ++i) {
        const float f = (float)(lo + (hi - lo) * uniform());
        if (dtype) {
            uint32_t b;
            memcpy(&b, &f, 4);
            ((uint16_t *)p)[i] = (uint16_t)(b >> 16);
        } else {
            ((float *)p)[i] = f;
        }
    }
    return p;
}

static seq_t make_seq(const dims_t *d, int64_t len)
{
    const int64_t tok = (int64_t)d->batch * len;
    seq_t s;
    s.x = fill(d->in_dtype, tok * d->nheads * d->headdim, -2, 2);
    s.dt = fill(d->in_dtype, tok * d->nheads, 1e-3, 0.1);
    s.B = fill(d->in_dtype, tok * d->ngroups * d->d_state, -0.5, 0.5);
    s.C = fill(d->in_dtype, tok * d->ngroups * d->d_state, -0.5, 0.5);
    return s;
}

static void free_seq(seq_t *s)
{
    free((void *)s->x);
    free((void *)s->dt);
    free((void *)s->B);
    free((void *)s->C);
}

static int finite_all(const double *v, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(v[i]))
            return 0;
    return 1;
}

#define CHECK(cond, what)                                      \
    do {                                                       \
        if (!(cond)) {                                         \
            fprintf(stderr, "oracle check failed: %s\n", what); \
            return 1;                                          \
        }                                                      \
    } while (0)

static int run(int dtype, int b, int H, int P, int N, int G, int64_t L, int64_t Q, int64_t T)
{
    dims_t d = {b, H, P, N, G, dtype};
    const int64_t NP = (int64_t)N * P, nch = (L + Q - 1) / Q;
    float *A = fill(0, H, -4, -0.5), *D = fill(0, H, -1, 1), *Ar = fill(0, H, -4, -0.5), *Dr = fill(0, H, -1, 1);
    float *Dc = fill(0, (int64_t)H * P, -1, 1);
    seq_t pre = make_seq(&d, L), fwd = make_seq(&d, T), rev = make_seq(&d, T), win_r = make_seq(&d, L);
    double *h0 = calloc((size_t)(b * H * NP), sizeof(double));
    double *y = calloc((size_t)(b * L * H * P), sizeof(double));
    double *cs = calloc((size_t)(b * nch * H * NP), sizeof(double));
    double *h = calloc((size_t)(b * H * NP), sizeof(double));
    double *yb = calloc((size_t)(b * T * H * P), sizeof(double));
    double *yf = calloc((size_t)(b * T * H * P), sizeof(double));
    double *yr = calloc((size_t)(b * T * H * P), sizeof(double));
    double *yw = calloc((size_t)(b * L * H * P), sizeof(double));
    int8_t *mask = calloc((size_t)H, 1);
    for (int i = 0; i < H; i += 2)
        mask[i] = 1;
    for (int64_t i = 0; i < b * H * NP; ++i)
        h0[i] = uniform() - 0.5;
    CHECK(oracle_scan(&d, L, Q, &pre, A, D, h0, y, cs, h, NULL, 2) == 0, "scan");
    CHECK(finite_all(y, b * L * H * P) && finite_all(cs, b * nch * H * NP), "scan outputs");
    CHECK(oracle_scan(&d, L, Q, &pre, A, D, NULL, NULL, NULL, h, mask, 0) == 0, "scan, head subset");
    CHECK(oracle_block_step_ex(&d, T, h, &fwd, &rev, A, D, Ar, Dr, yb, yf, yr, NULL, 2) == 0, "block step");
    CHECK(finite_all(yb, b * T * H * P), "block step y");
    CHECK(oracle_block_step_ex(&d, T, h, &fwd, &rev, A, D, NULL, NULL, yb, NULL, NULL, mask, 1) == 0, "block step");
    CHECK(oracle_block_step_dch(&d, T, h, &fwd, &rev, A, Dc, Ar, Dc, yb, NULL, 2) == 0, "per-channel skip");
    CHECK(oracle_commit(&d, T, &fwd, A, D, h, yb, NULL, 2) == 0, "commit");
    CHECK(oracle_full_window(&d, L, &pre, &win_r, A, D, Ar, Dr, yw, NULL, 2) == 0, "full window");
    CHECK(finite_all(yw, b * L * H * P), "full window y");
    /* the convolution, both directions, width 1..4, with and without history and bias */
    const int64_t CH = (int64_t)H * P + 2 * (int64_t)G * N;
    for (int W = 1; W <= 4; ++W) {
        float *w = fill(0, CH * W, -0.5, 0.5), *bias = fill(0, CH, -0.5, 0.5);
        void *hist = fill(dtype, (int64_t)b * (W - 1) * CH + 1, -1, 1);
        void *hout = fill(dtype, (int64_t)b * (W - 1) * CH + 1, 0, 0);
        seq_t out = make_seq(&d, T);
        CHECK(oracle_conv(&d, T, W, 1, 0, w, bias, W > 1 ? hist : NULL, &fwd, &out, W > 1 ? hout : NULL, 2) == 0,
              "conv forward");
        CHECK(oracle_conv(&d, T, W, 0, 1, w, NULL, NULL, &rev, &out, NULL, 1) == 0, "conv reverse");
        free(w);
        free(bias);
        free(hist);
        free(hout);
        free_seq(&out);
    }
    /* arguments the oracle must reject */
    dims_t bad = d;
    bad.ngroups = 3 * H + 1;
    CHECK(oracle_scan(&bad, L, Q, &pre, A, D, NULL, NULL, NULL, h, NULL, 1) != 0, "H % G != 0 rejected");
    CHECK(oracle_commit(&d, 0, &fwd, A, D, h, NULL, NULL, 1) != 0, "T = 0 rejected");
    free(A), free(D), free(Ar), free(Dr), free(Dc), free(h0), free(y), free(cs), free(h), free(yb), free(yf);
    free(yr), free(yw), free(mask);
    free_seq(&pre), free_seq(&fwd), free_seq(&rev), free_seq(&win_r);
    return 0;
}

int main(void)
{
    if (run(0, 2, 4, 16, 16, 2, 100, 16, 13) || run(1, 1, 6, 8, 8, 3, 67, 32, 9) || run(1, 2, 2, 4, 8, 1, 1, 64, 1))
        return 1;
    puts("oracle sanitizer run: ok");
    return 0;
}
