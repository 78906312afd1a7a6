/*
 * Oracle for the bidirectional block-diffusion Mamba state hot path.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously-correct CPU
 * definition that the HIP kernels are checked against. Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it. It shares no code, header,
 * table or helper with the HIP library, and it never includes anything from it.
 *
 * What it computes (all arithmetic in float64; inputs are decoded exactly from the
 * float32 or bfloat16 values the GPU receives):
 *
 *  - The selective state-space recurrence of "Training Hybrid Block Diffusion Language
 *    Models with Partial Bidirectionality", eq. (1): s_i = A_i s_{i-1} + B_i x_i,
 *    y_i = C_i s_i + D x_i, instantiated in the Mamba-2 form with a scalar decay per
 *    head and token:
 *        alpha_t = exp(dt[t,h] * A[h])
 *        S[n][p] <- alpha_t * S[n][p] + dt[t,h] * B[t,g][n] * x[t,h][p]
 *        y[t,h][p] = sum_n C[t,g][n] * S[n][p]  (+ D[h] * x[t,h][p])
 *    with g = h / (H/G) (consecutive heads share a B/C group). S is the boundary state
 *    "after token i" of eq. (1).
 *  - oracle_scan: the prefix scan of eq. (10), s_k = F_fwd(c): the recurrence run over a
 *    prefix from h_init (or zero), emitting y, the state after every chunk of Q tokens
 *    (and after the last token), and the final state.
 *  - oracle_block_step: eqs. (11)-(13). Forward continuation of the cached state into the
 *    active block (eq. 11) without modifying the cached state; a reverse scan over only
 *    the active block, started from a zero state at the block's right end, with outputs
 *    in natural token order (eq. 12: rev(F_rev(rev(b)))); their sum (eq. 13) plus the
 *    skip term D[h] * x_fwd of eq. (1), applied once.
 *  - oracle_block_step_ex: the same with separate parameters for the reverse direction
 *    (eq. 12 gives the reverse scan its own parameters): the reverse recurrence decays
 *    with A_rev[h], and D_rev[h] * x_rev is added to y. Reading: each direction is a full
 *    Mamba-2 scan with its own skip term; the sum of eq. (13) adds both.
 *  - oracle_commit: the "clean forward pass over the new block" that extends the cache
 *    once a block is finalized: the recurrence over the block's clean inputs, updating
 *    the state in place (optionally writing y, with D).
 *
 * Layouts (row-major, contiguous):
 *    x [b][len][H][P], dt [b][len][H], B and C [b][len][G][N],
 *    states [b][H][N][P], chunk states [b][ceil(len/Q)][H][N][P], y [b][len][H][P].
 * Input dtype 0 = float32, 1 = bfloat16 bit patterns (uint16).
 *
 * Independent (stream, head) pairs may run on separate OpenMP threads; each recurrence
 * stays sequential in t.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t batch, nheads, headdim, d_state, ngroups;
    int32_t in_dtype; /* 0 = float32, 1 = bfloat16 bits */
} oracle_dims;

typedef struct {
    const void *x, *dt, *B, *C;
} oracle_seq;

static double val(const void *p, int dtype, int64_t i)
{
    if (dtype == 0)
        return (double)((const float *)p)[i];
    uint32_t bits = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int check(const oracle_dims *d)
{
    if (!d || d->batch < 1 || d->nheads < 1 || d->headdim < 1 || d->d_state < 1 || d->ngroups < 1)
        return 1;
    if (d->nheads % d->ngroups != 0)
        return 1;
    if (d->in_dtype != 0 && d->in_dtype != 1)
        return 1;
    return 0;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * The forward recurrence over `len` tokens of stream b, head h, carrying S (N*P,
 * in/out). If y != NULL, y[b][t][h][:] = C_t . S_t (+ D x_t if with_D). If
 * chunk_states != NULL, the state after tokens chunk-1, 2*chunk-1, ... and after the
 * last token is stored at chunk_states[b][t / chunk][h].
 */
static void forward(const oracle_dims *d, int b, int h, int64_t len, int64_t chunk,
                    const oracle_seq *in, double A, double Dh, int with_D,
                    double *S, double *y, double *chunk_states)
{
    const int H = d->nheads, P = d->headdim, N = d->d_state, G = d->ngroups;
    const int g = h / (H / G);
    const int dty = d->in_dtype;
    const int64_t nch = chunk > 0 ? (len + chunk - 1) / chunk : 0;
    double *xv = malloc(sizeof(double) * P);
    for (int64_t t = 0; t < len; ++t) {
        const int64_t tok = (int64_t)b * len + t;
        const double dt = val(in->dt, dty, tok * H + h);
        const double alpha = exp(dt * A);
        for (int p = 0; p < P; ++p)
            xv[p] = val(in->x, dty, (tok * H + h) * P + p);
        for (int n = 0; n < N; ++n) {
            const double w = dt * val(in->B, dty, (tok * G + g) * N + n);
            double *row = S + (int64_t)n * P;
            for (int p = 0; p < P; ++p)
                row[p] = alpha * row[p] + w * xv[p];
        }
        if (y) {
            double *yo = y + (tok * H + h) * P;
            for (int p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n)
                    acc += val(in->C, dty, (tok * G + g) * N + n) * S[(int64_t)n * P + p];
                yo[p] = with_D ? acc + Dh * xv[p] : acc;
            }
        }
        if (chunk_states && ((t + 1) % chunk == 0 || t == len - 1)) {
            double *dst = chunk_states + (((int64_t)b * nch + t / chunk) * H + h) * (int64_t)N * P;
            memcpy(dst, S, sizeof(double) * (size_t)N * P);
        }
    }
    free(xv);
}

/* Prefix scan (eq. 10). h_init may be NULL (zero state); y and chunk_states may be NULL.
 * head_mask (length H) may be NULL; heads with mask 0 are skipped and their outputs
 * left untouched. Returns 0 on success. */
int oracle_scan(const oracle_dims *d, int64_t len, int64_t chunk, const oracle_seq *in,
                const float *A, const float *D, const double *h_init, double *y,
                double *chunk_states, double *h_out, const int8_t *head_mask, int nthreads)
{
    if (check(d) || len < 1 || !in || !A || !D || !h_out || (chunk_states && chunk < 1))
        return 1;
    set_threads(nthreads);
    const int H = d->nheads;
    const int64_t NP = (int64_t)d->d_state * d->headdim;
    const int pairs = d->batch * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < pairs; ++i) {
        const int b = i / H, h = i % H;
        if (head_mask && !head_mask[h])
            continue;
        double *S = calloc((size_t)NP, sizeof(double));
        if (h_init)
            memcpy(S, h_init + (int64_t)i * NP, sizeof(double) * NP);
        forward(d, b, h, len, chunk, in, A[h], D[h], 1, S, y, chunk_states);
        memcpy(h_out + (int64_t)i * NP, S, sizeof(double) * NP);
        free(S);
    }
    return 0;
}

/* Block step (eqs. 11-13). h_prefix is read only. y = y_fwd + y_rev + D x_fwd.
 * y_fwd and y_rev (without D) are optional extra outputs. The skip weights D (and D_rev) are
 * one per head, [H], or with skip_per_channel one per head and channel, [H][P] (the Mamba-2
 * layer's option of a skip weight per channel of x). */
static int block_step_impl(const oracle_dims *d, int64_t T, const double *h_prefix,
                           const oracle_seq *fwd, const oracle_seq *rev, const float *A,
                           const float *D, const float *A_rev, const float *D_rev,
                           int skip_per_channel, double *y, double *y_fwd, double *y_rev,
                           const int8_t *head_mask, int nthreads)
{
    if (check(d) || T < 1 || !h_prefix || !fwd || !rev || !A || !D || !y)
        return 1;
    const float *Ar = A_rev ? A_rev : A;
    set_threads(nthreads);
    const int H = d->nheads, P = d->headdim, N = d->d_state, G = d->ngroups;
    const int dty = d->in_dtype;
    const int64_t NP = (int64_t)N * P;
    const int pairs = d->batch * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < pairs; ++i) {
        const int b = i / H, h = i % H, g = h / (H / G);
        if (head_mask && !head_mask[h])
            continue;
        double *S = malloc(sizeof(double) * NP);
        double *yf = malloc(sizeof(double) * T * P);
        double *yr = malloc(sizeof(double) * T * P);
        double *xv = malloc(sizeof(double) * P);
        /* eq. (11): forward continuation from a copy of the cached state */
        memcpy(S, h_prefix + (int64_t)i * NP, sizeof(double) * NP);
        for (int64_t t = 0; t < T; ++t) {
            const int64_t tok = (int64_t)b * T + t;
            const double dt = val(fwd->dt, dty, tok * H + h);
            const double alpha = exp(dt * A[h]);
            for (int p = 0; p < P; ++p)
                xv[p] = val(fwd->x, dty, (tok * H + h) * P + p);
            for (int n = 0; n < N; ++n) {
                const double w = dt * val(fwd->B, dty, (tok * G + g) * N + n);
                for (int p = 0; p < P; ++p)
                    S[(int64_t)n * P + p] = alpha * S[(int64_t)n * P + p] + w * xv[p];
            }
            for (int p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n)
                    acc += val(fwd->C, dty, (tok * G + g) * N + n) * S[(int64_t)n * P + p];
                yf[t * P + p] = acc;
            }
        }
        /* eq. (12): reverse scan inside the block only, from a zero state at its right end */
        memset(S, 0, sizeof(double) * NP);
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t tok = (int64_t)b * T + t;
            const double dt = val(rev->dt, dty, tok * H + h);
            const double alpha = exp(dt * Ar[h]);
            for (int p = 0; p < P; ++p)
                xv[p] = val(rev->x, dty, (tok * H + h) * P + p);
            for (int n = 0; n < N; ++n) {
                const double w = dt * val(rev->B, dty, (tok * G + g) * N + n);
                for (int p = 0; p < P; ++p)
                    S[(int64_t)n * P + p] = alpha * S[(int64_t)n * P + p] + w * xv[p];
            }
            for (int p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n)
                    acc += val(rev->C, dty, (tok * G + g) * N + n) * S[(int64_t)n * P + p];
                yr[t * P + p] = acc;
            }
        }
        /* eq. (13) plus the skip term of eq. (1), applied once to the forward input, and
         * the reverse direction's own skip term when it has one */
        for (int64_t t = 0; t < T; ++t) {
            const int64_t tok = (int64_t)b * T + t;
            for (int p = 0; p < P; ++p) {
                const int64_t o = (tok * H + h) * P + p;
                const int64_t w = skip_per_channel ? (int64_t)h * P + p : h;
                y[o] = yf[t * P + p] + yr[t * P + p] + (double)D[w] * val(fwd->x, dty, o);
                if (D_rev)
                    y[o] += (double)D_rev[w] * val(rev->x, dty, o);
                if (y_fwd)
                    y_fwd[o] = yf[t * P + p];
                if (y_rev)
                    y_rev[o] = yr[t * P + p];
            }
        }
        free(S);
        free(yf);
        free(yr);
        free(xv);
    }
    return 0;
}

int oracle_block_step_ex(const oracle_dims *d, int64_t T, const double *h_prefix,
                         const oracle_seq *fwd, const oracle_seq *rev, const float *A,
                         const float *D, const float *A_rev, const float *D_rev, double *y,
                         double *y_fwd, double *y_rev, const int8_t *head_mask, int nthreads)
{
    return block_step_impl(d, T, h_prefix, fwd, rev, A, D, A_rev, D_rev, 0, y, y_fwd, y_rev, head_mask,
                           nthreads);
}

/* The block step with skip weights per head and channel: D and D_rev (when given) are
 * [H][P]. */
int oracle_block_step_dch(const oracle_dims *d, int64_t T, const double *h_prefix,
                          const oracle_seq *fwd, const oracle_seq *rev, const float *A,
                          const float *D, const float *A_rev, const float *D_rev, double *y,
                          const int8_t *head_mask, int nthreads)
{
    return block_step_impl(d, T, h_prefix, fwd, rev, A, D, A_rev, D_rev, 1, y, NULL, NULL, head_mask,
                           nthreads);
}

int oracle_block_step(const oracle_dims *d, int64_t T, const double *h_prefix,
                      const oracle_seq *fwd, const oracle_seq *rev, const float *A,
                      const float *D, double *y, double *y_fwd, double *y_rev,
                      const int8_t *head_mask, int nthreads)
{
    return oracle_block_step_ex(d, T, h_prefix, fwd, rev, A, D, NULL, NULL, y, y_fwd, y_rev,
                                head_mask, nthreads);
}

/*
 * Full-window bidirectional scan: the system the block-local method replaces -- a fully
 * bidirectional Mamba layer over the whole sequence ("DiffuApriel", Sec. 3.2, eqs. (4)-(6):
 * forward and backward scans with their own parameters, summed; the full-sequence
 * baselines of the BDLM page, whose reverse states depend on the active tokens and so cannot
 * be cached). Over one window of len tokens (prefix and active block together) nothing is
 * cached: the forward scan starts from a zero state at token 0 and the reverse scan from a
 * zero state past token len-1, and y = y_fwd + y_rev + D x_fwd (+ D_rev x_rev). That is
 * exactly the block step's pair of scans (eqs. (11)-(13)) taken over the whole window with
 * a zero cached state, which is how it is computed here.
 */
int oracle_full_window(const oracle_dims *d, int64_t len, const oracle_seq *fwd, const oracle_seq *rev,
                       const float *A, const float *D, const float *A_rev, const float *D_rev, double *y,
                       const int8_t *head_mask, int nthreads)
{
    if (check(d) || len < 1)
        return 1;
    const int64_t n = (int64_t)d->batch * d->nheads * d->d_state * d->headdim;
    double *zero = calloc((size_t)n, sizeof(double));
    if (!zero)
        return 1;
    const int rc = oracle_block_step_ex(d, len, zero, fwd, rev, A, D, A_rev, D_rev, y, NULL, NULL, head_mask,
                                        nthreads);
    free(zero);
    return rc;
}

/* Commit: the clean forward pass over a finalized block, advancing h in place.
 * y (with D) is optional. */
int oracle_commit(const oracle_dims *d, int64_t T, const oracle_seq *clean, const float *A,
                  const float *D, double *h, double *y, const int8_t *head_mask, int nthreads)
{
    if (check(d) || T < 1 || !clean || !A || !D || !h)
        return 1;
    set_threads(nthreads);
    const int H = d->nheads;
    const int64_t NP = (int64_t)d->d_state * d->headdim;
    const int pairs = d->batch * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < pairs; ++i) {
        const int b = i / H, hh = i % H;
        if (head_mask && !head_mask[hh])
            continue;
        forward(d, b, hh, T, 0, clean, A[hh], D[hh], 1, h + (int64_t)i * NP, y, NULL);
    }
    return 0;
}

/*
 * Convolution state (the Mamba cache holds "convolution and selective-SSM state", per the
 * cache discussion of "Training Hybrid Block Diffusion Language Models with Partial
 * Bidirectionality"). Reading of what the pages leave open, following the Mamba-2 layer:
 * before the scan, the x, B and C inputs (channels ordered x [H*P], then B [G*N], then C
 * [G*N]: per token, the rows of the three arrays) pass through a depthwise convolution of
 * width W <= 4 with a per-channel bias and then an activation (identity or SiLU). The
 * result is an activation of the input dtype, so it is rounded to that dtype
 * (round-to-nearest-even) before the scan reads it. dt is not convolved.
 *
 *  forward (causal), from the conv state: out_t = bias + sum_k w[k] u_{t-(W-1)+k}, where
 *      u_t for t < 0 is row W-1+t of the conv state (the W-1 raw rows before the segment;
 *      zero when there is none) and the raw input otherwise;
 *  reverse (anti-causal, inside the block only): out_t = bias + sum_k w[k] u_{t+(W-1)-k}
 *      with u_t = 0 past the block's end - the causal convolution of the reversed block
 *      from a zero history, read back in natural order (eq. (12) gives the reverse branch
 *      no state).
 * The conv state after a forward segment is its extended input's last W-1 raw rows.
 *
 * conv state layout: [b][W-1][H*P + 2*G*N], input dtype. w: [H*P + 2*G*N][W] float32,
 * bias: [H*P + 2*G*N] float32 or NULL. act: 0 identity, 1 SiLU (v / (1 + exp(-v))).
 */
static void put(void *p, int dtype, int64_t i, double v)
{
    if (dtype == 0) {
        ((float *)p)[i] = (float)v;
        return;
    }
    /* bfloat16: 8 significant bits, ties to even, straight from float64 */
    double r = v;
    if (v != 0.0 && isfinite(v)) {
        int e;
        frexp(v, &e);
        int qe = e - 8;
        if (qe < -133)
            qe = -133; /* bfloat16 subnormal quantum */
        r = ldexp(nearbyint(ldexp(v, -qe)), qe);
    }
    const float f = (float)r; /* exact */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    ((uint16_t *)p)[i] = (uint16_t)(bits >> 16);
}

/* channel c of token row `tok` of a sequence (x, then B, then C) */
static double chan(const oracle_dims *d, const oracle_seq *s, int64_t tok, int64_t c)
{
    const int64_t HP = (int64_t)d->nheads * d->headdim, GN = (int64_t)d->ngroups * d->d_state;
    if (c < HP)
        return val(s->x, d->in_dtype, tok * HP + c);
    if (c < HP + GN)
        return val(s->B, d->in_dtype, tok * GN + (c - HP));
    return val(s->C, d->in_dtype, tok * GN + (c - HP - GN));
}

static void put_chan(const oracle_dims *d, const oracle_seq *s, int64_t tok, int64_t c, double v)
{
    const int64_t HP = (int64_t)d->nheads * d->headdim, GN = (int64_t)d->ngroups * d->d_state;
    if (c < HP)
        put((void *)s->x, d->in_dtype, tok * HP + c, v);
    else if (c < HP + GN)
        put((void *)s->B, d->in_dtype, tok * GN + (c - HP), v);
    else
        put((void *)s->C, d->in_dtype, tok * GN + (c - HP - GN), v);
}

int oracle_conv(const oracle_dims *d, int64_t len, int32_t width, int32_t act, int32_t reverse,
                const float *w, const float *bias, const void *state_in, const oracle_seq *raw,
                const oracle_seq *out, void *state_out, int nthreads)
{
    if (check(d) || len < 1 || width < 1 || width > 4 || (act != 0 && act != 1) || !w || !raw ||
        !out || (reverse && (state_in || state_out)))
        return 1;
    set_threads(nthreads);
    const int dty = d->in_dtype;
    const int64_t CH = (int64_t)d->nheads * d->headdim + 2 * (int64_t)d->ngroups * d->d_state;
    const int64_t total = (int64_t)d->batch * CH;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        const int64_t b = i / CH, c = i % CH;
        /* the raw input extended by W-1 rows of history (forward) or of zeros (reverse) */
        double *u = malloc(sizeof(double) * (size_t)(len + width - 1));
        for (int k = 0; k < width - 1; ++k) {
            const int64_t hist = reverse ? len + width - 1 - 1 - k : k;
            u[hist] = (!reverse && state_in) ? val(state_in, dty, (b * (width - 1) + k) * CH + c) : 0.0;
        }
        const int64_t off = reverse ? 0 : width - 1;
        for (int64_t t = 0; t < len; ++t)
            u[off + t] = chan(d, raw, b * len + t, c);
        for (int64_t t = 0; t < len; ++t) {
            double v = bias ? (double)bias[c] : 0.0;
            for (int k = 0; k < width; ++k) {
                /* forward: u_{t-(W-1)+k} sits at index t+k; reverse: u_{t+(W-1)-k} at t+W-1-k */
                const int64_t at = reverse ? t + width - 1 - k : t + k;
                v += (double)w[c * width + k] * u[at];
            }
            if (act == 1)
                v = v / (1.0 + exp(-v));
            put_chan(d, out, b * len + t, c, v);
        }
        if (state_out)
            for (int k = 0; k < width - 1; ++k)
                put(state_out, dty, (b * (width - 1) + k) * CH + c, u[len + k]);
        free(u);
    }
    return 0;
}
