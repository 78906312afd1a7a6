/*
 * bdssm.h - C ABI of the bidirectional block-diffusion Mamba state hot path on MI355X.
 *
 * The method ("Training Hybrid Block Diffusion Language Models with Partial
 * Bidirectionality", eqs. (9)-(13) and the cache discussion around them) factors each
 * Mamba layer into a timestep-free prefix operator, which folds the clean prefix into a
 * cached forward state, and an active-block continuation, which runs a forward scan
 * seeded from that state plus a reverse scan confined to the active block. The three
 * calls below are those three operations:
 *
 *   bdssm_prefix_scan  - eq. (10): s_k = F_fwd(c), the forward scan of a prefix,
 *                        returning the boundary state (and optionally y and the state
 *                        after every chunk of the scan).
 *   bdssm_block_step   - eqs. (11)-(13): y = F_fwd(b; s_k) + rev(F_rev(rev(b))) + D x,
 *                        for one denoising step of the active block. The cached state is
 *                        read, never written (the cache must not depend on the step).
 *   bdssm_commit       - the clean forward pass over a finalized block that extends the
 *                        cache: s_{k+1} = F_fwd(b*; s_k), in place.
 *
 * bdssm_decode_graph_* record the calls of one active block (its denoising steps, then its
 * commit) once into a HIP graph and replay it, removing per-call launch latency from a
 * decode loop with static shapes.
 *
 * The scan F is the selective state-space recurrence of eq. (1) in its Mamba-2 form,
 * with one negative scalar A[h] per head:
 *     alpha_t = exp(dt[t,h] * A[h])
 *     S_t     = alpha_t * S_{t-1} + dt[t,h] * B[t,g] x[t,h]^T        (S is N x P)
 *     y[t,h]  = C[t,g] . S_t   (+ D[h] * x[t,h] where stated)
 * with g = h / (H/G): each group of H/G consecutive heads shares B and C. The reverse
 * scan starts from a zero state at the block's right end and runs t = T-1 ... 0 over
 * inputs given in natural token order; its outputs are in natural order too.
 *
 * Layouts (row-major, contiguous, b = stream):
 *     x  [b][len][H][P]     dt [b][len][H]     B, C [b][len][G][N]
 *     state [b][H][N][P] (float32)     chunk states [b][ceil(len/chunk)][H][N][P]
 *     y  [b][len][H][P]     A, D [H] (float32)
 * dt is the final step size (already passed through softplus and any clamp).
 *
 * Conventions for every call:
 *  - Pointers are device pointers (hipMalloc'd, or torch CUDA tensors); the caller owns
 *    every buffer. Base pointers must be 16-byte aligned. The library allocates nothing
 *    (except the graph object of bdssm_decode_graph_create) and never synchronizes.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    asynchronously; the returned status covers argument validation and the launch.
 *    Faults during execution surface at the caller's next synchronization.
 *  - Errors are status codes; nothing is thrown across the ABI. Invalid arguments are
 *    rejected before anything is launched, with no buffer modified.
 *  - Supported shapes: ngroups divides nheads; (d_state, headdim) in {(16,16), (128,64)};
 *    chunk in {16, 32, 64, 128, 256}; block_len in [0, 256]. batch, len and block_len
 *    may be 0 (nothing to do: a prefix scan of zero tokens returns h_init, or zero).
 *  - Thread-safe and re-entrant. Calls on one stream run in order.
 */
#ifndef BDSSM_H
#define BDSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BDSSM_ABI_VERSION 4

typedef enum {
    BDSSM_OK = 0,
    BDSSM_ERR_NULL = 1,        /* a required pointer is NULL */
    BDSSM_ERR_SHAPE = 2,       /* a size is negative or inconsistent (e.g. H % G != 0) */
    BDSSM_ERR_UNSUPPORTED = 3, /* a valid size or dtype with no compiled kernel */
    BDSSM_ERR_ALIGN = 4,       /* a base pointer is not 16-byte aligned */
    BDSSM_ERR_ALIAS = 5,       /* an output overlaps an input it must not overlap */
    BDSSM_ERR_WORKSPACE = 6,   /* workspace missing or smaller than the query returned */
    BDSSM_ERR_HIP = 7,         /* the HIP runtime reported an error at launch */
    BDSSM_ERR_SCRATCH = 8      /* bdssm_prefix_scan_static: more workspace needed than the
                                  static scratch buffer holds */
} bdssm_status;

typedef enum { BDSSM_F32 = 0, BDSSM_BF16 = 1 } bdssm_dtype;

typedef struct {
    int32_t batch;    /* independent streams b */
    int32_t nheads;   /* H */
    int32_t headdim;  /* P */
    int32_t d_state;  /* N */
    int32_t ngroups;  /* G */
    int32_t in_dtype; /* bdssm_dtype of x, dt, B, C */
    int32_t y_dtype;  /* bdssm_dtype of y (F32 for parity checks, BF16 as activations) */
} bdssm_dims;

/* One token segment's inputs (device pointers, layouts above). */
typedef struct {
    const void *x, *dt, *B, *C;
} bdssm_seq;

/* ABI version implemented by the library (BDSSM_ABI_VERSION at build time). */
int bdssm_abi_version(void);

/* Static, human-readable name of a status code; never NULL. */
const char *bdssm_status_str(int status);

/* Bytes of device workspace bdssm_prefix_scan needs for these arguments. with_y and
 * with_chunk_states say whether y and chunk_states will be passed non-NULL. Returns 0
 * when no workspace is needed, and SIZE_MAX for arguments bdssm_prefix_scan would
 * reject. */
size_t bdssm_prefix_scan_workspace(const bdssm_dims *dims, int64_t len, int32_t chunk,
                                   int32_t with_y, int32_t with_chunk_states);

/*
 * Prefix scan: eq. (10), s_k = F_fwd(c^(k)), the forward recurrence over `len` prefix
 * tokens of every stream, computed chunk by chunk (chunk = Q tokens; the last chunk may
 * be shorter).
 *   in            prefix inputs, len tokens
 *   A, D          [H] float32
 *   h_init        [b][H][N][P] float32 starting state, or NULL for zero
 *   y             [b][len][H][P] in dims->y_dtype, y_t = C_t . S_t + D x_t; NULL = state only
 *   chunk_states  [b][ceil(len/Q)][H][N][P] float32: the state after tokens Q-1, 2Q-1, ...
 *                 and after the last token (so the last entry equals h_out); NULL = none
 *   h_out         [b][H][N][P] float32 final state; required; may be the same pointer as
 *                 h_init (updated in place) but must not otherwise overlap anything
 *   workspace     device buffer of at least bdssm_prefix_scan_workspace(...) bytes
 * y and chunk_states must not overlap any input or each other.
 */
bdssm_status bdssm_prefix_scan(const bdssm_dims *dims, int64_t len, int32_t chunk,
                               const bdssm_seq *in, const float *A, const float *D,
                               const float *h_init, void *y, float *chunk_states,
                               float *h_out, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Prefix scan that allocates nothing and takes no workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): bdssm_prefix_scan, bitwise, with the workspace it would need taken
 * from a scratch buffer the library keeps in device memory -- a static array of
 * BDSSM_STATIC_SCRATCH_BYTES (64 MiB) per GPU, held from the library's first use of that
 * GPU until the process ends. Every call on one GPU shares that GPU's buffer and it keeps
 * the last call's contents (each call writes all it reads), so calls that overlap in time
 * on one GPU -- on different streams, or from different threads -- race and give wrong
 * results; calls in order on one stream are safe. On the matrix-core path (bf16 inputs,
 * (d_state, headdim) = (128, 64), chunk >= 64) the largest plan needs about 32 MiB on a
 * 256-CU MI355X, whatever the sizes; other paths need bdssm_prefix_scan_workspace bytes.
 * Arguments, layouts, ownership and errors as bdssm_prefix_scan, plus:
 *   BDSSM_ERR_SCRATCH  the call would need more than BDSSM_STATIC_SCRATCH_BYTES of workspace
 *                      (rejected before anything is launched)
 *   BDSSM_ERR_HIP      the buffer's device address could not be obtained
 */
#define BDSSM_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
bdssm_status bdssm_prefix_scan_static(const bdssm_dims *dims, int64_t len, int32_t chunk,
                                      const bdssm_seq *in, const float *A, const float *D,
                                      const float *h_init, void *y, float *chunk_states,
                                      float *h_out, void *stream);

/*
 * Block step: eqs. (11)-(13), one denoising step of the active block of T = block_len
 * tokens:
 *   y_t = C_t . S_t            (forward scan from h_prefix over fwd, eq. 11)
 *       + C'_t . R_t           (reverse scan over rev from R_T = 0, eq. 12)
 *       + D[h] * x_fwd[t]      (skip term of eq. 1, applied once)
 *   h_prefix  [b][H][N][P] float32 cached state; read only, never written
 *   fwd, rev  the two directions' inputs, T tokens each, natural token order
 *   y         [b][T][H][P] in dims->y_dtype; must not overlap any input
 */
bdssm_status bdssm_block_step(const bdssm_dims *dims, int32_t block_len,
                              const float *h_prefix, const bdssm_seq *fwd,
                              const bdssm_seq *rev, const float *A, const float *D, void *y,
                              void *stream);

/*
 * Block step with separate parameters for the reverse direction (eq. (12) gives the
 * reverse scan its own parameters): the reverse recurrence decays with A_rev[h] instead of
 * A[h], and each direction keeps its own skip term,
 *   y_t = C_t . S_t + C'_t . R_t + D[h] * x_fwd[t] + D_rev[h] * x_rev[t].
 *   A_rev  [H] float32, required (pass A for a shared decay)
 *   D_rev  [H] float32, or NULL for no reverse skip term
 * Everything else as bdssm_block_step, which equals this call with A_rev = A, D_rev = NULL.
 * y must not overlap A_rev or D_rev either.
 */
bdssm_status bdssm_block_step_ex(const bdssm_dims *dims, int32_t block_len,
                                 const float *h_prefix, const bdssm_seq *fwd,
                                 const bdssm_seq *rev, const float *A, const float *D,
                                 const float *A_rev, const float *D_rev, void *y, void *stream);

/*
 * Full-window bidirectional scan: the system the block-local method is compared against, a
 * fully bidirectional Mamba layer over the whole sequence ("DiffuApriel", Sec. 3.2, eqs.
 * (4)-(6): a forward and a backward scan, each with its own parameters, summed; the
 * full-sequence bidirectional baselines of "Training Hybrid Block Diffusion Language Models
 * with Partial Bidirectionality", whose directionality discussion explains why their reverse
 * states cannot be cached). Over one window of len tokens -- the prefix and the active block
 * together -- with nothing cached:
 *   y_t = C_t . S_t             (forward scan from a zero state at token 0, over fwd)
 *       + C'_t . R_t            (reverse scan from a zero state past token len-1, over rev,
 *                                decaying with A_rev)
 *       + D[h] * x_fwd[t] (+ D_rev[h] * x_rev[t] when D_rev is given)
 * for every token of the window. Since the reverse states of prefix tokens depend on the
 * active block, a full-window model recomputes all of this on every denoising step; on the
 * block's own tokens the result equals bdssm_block_step from the prefix's state.
 *   fwd, rev        the two directions' inputs, len tokens each, natural token order
 *   A, D            [H] float32; A_rev [H] float32, required (pass A for a shared decay);
 *                   D_rev [H] float32 or NULL
 *   y               [b][len][H][P] in dims->y_dtype, written (forward half) then added to
 *                   (reverse half, so bf16 y is rounded twice); must not overlap any input
 *   chunk, workspace  as in bdssm_prefix_scan (bdssm_full_window_workspace bytes; both
 *                   directions use the same workspace in turn)
 * Errors as bdssm_prefix_scan.
 */
size_t bdssm_full_window_workspace(const bdssm_dims *dims, int64_t len, int32_t chunk);
bdssm_status bdssm_full_window(const bdssm_dims *dims, int64_t len, int32_t chunk, const bdssm_seq *fwd,
                               const bdssm_seq *rev, const float *A, const float *D, const float *A_rev,
                               const float *D_rev, void *y, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Commit: the clean forward pass over a finalized block of T = block_len tokens that
 * extends the cache, S <- F_fwd(clean; S), in place on h.
 *   clean  the block's clean inputs; clean->C may be NULL when y is NULL
 *   h      [b][H][N][P] float32, read then overwritten with the advanced state
 *   y      NULL, or [b][T][H][P] in dims->y_dtype: y_t = C_t . S_t + D x_t of the pass
 */
bdssm_status bdssm_commit(const bdssm_dims *dims, int32_t block_len, const bdssm_seq *clean,
                          const float *A, const float *D, float *h, void *y, void *stream);

/*
 * Cached state in operand form. The cached state is read by every denoising step of a
 * block and changes only when a block is committed (eqs. (9)-(11): s_k is fixed while
 * block k is denoised), so the re-encoding the block step's matrix-core product needs can
 * be made once per cached state instead of once per step. The operand form of a float32
 * state S is the bf16 pair hi = bf16(S), lo = bf16(S - hi) (round to nearest even; together
 * about 16 significant bits, the same pair bdssm_block_step forms from S on every call), laid
 * out as
 *     ops [b][H][2 (hi, lo)][N/8][P][8] bf16,  ops[..][k][n/8][p][n%8] = k-part of S[n][p],
 * which has the size of the float32 state. Supported for (d_state, headdim) = (128, 64).
 *
 * bdssm_state_ops_bytes: bytes of ops for these dims; SIZE_MAX for invalid or unsupported
 * dims.
 * bdssm_state_ops: writes ops from h [b][H][N][P] float32 (read only); ops must not overlap
 * h. Errors: BDSSM_ERR_NULL, BDSSM_ERR_UNSUPPORTED (other d_state/headdim), BDSSM_ERR_ALIGN,
 * BDSSM_ERR_ALIAS.
 */
size_t bdssm_state_ops_bytes(const bdssm_dims *dims);
bdssm_status bdssm_state_ops(const bdssm_dims *dims, const float *h, void *ops, void *stream);

/*
 * Block step from the cached state in operand form: bdssm_block_step_ex with the state
 * given as h_ops, made by bdssm_state_ops from h_prefix. For block_len <= 32 and
 * batch * nheads < 512 it runs the small-batch kernel of bdssm_block_step_ex and its y is
 * bitwise that call's on h_prefix; otherwise (block_len <= 128) a kernel that copies the
 * operand-form state and x straight into LDS, whose y agrees with bdssm_block_step_ex up to
 * rounding (the same bounds against the exact result). Errors as bdssm_block_step_ex, with
 * BDSSM_ERR_UNSUPPORTED for inputs other than bf16, (d_state, headdim) other than
 * (128, 64), or block_len > 128; y must not overlap h_ops.
 */
bdssm_status bdssm_block_step_ops(const bdssm_dims *dims, int32_t block_len, const void *h_ops,
                                  const bdssm_seq *fwd, const bdssm_seq *rev, const float *A,
                                  const float *D, const float *A_rev, const float *D_rev, void *y,
                                  void *stream);

/*
 * bf16 cached state. The block step reads the whole cached state on every denoising step,
 * so its bytes bound the step at large batch; a bf16 copy halves them at the cost of
 * rounding the state once (relative error 2^-9 per element). The bf16 state of a float32
 * state S is bf16(S), rounded to nearest even -- the operand form's hi part -- laid out as
 *     [b][H][N/8][P][8] bf16,  element (n, p) of a head at index (n/8 * P + p) * 8 + n % 8,
 * made once per cached state (after the prefix scan or a commit, which keep the float32
 * state as the master copy). Supported for d_state a multiple of 8.
 * bdssm_state_bf16_bytes: bytes of the bf16 state; SIZE_MAX for invalid or unsupported dims.
 * bdssm_state_bf16: writes it from h [b][H][N][P] float32 (read only); out must not overlap
 * h. Errors: BDSSM_ERR_NULL, BDSSM_ERR_UNSUPPORTED, BDSSM_ERR_ALIGN, BDSSM_ERR_ALIAS.
 */
size_t bdssm_state_bf16_bytes(const bdssm_dims *dims);
bdssm_status bdssm_state_bf16(const bdssm_dims *dims, const float *h, void *out, void *stream);

/*
 * Block step with every variant of the layer's parameters and of the cached state's form.
 * The reverse scan of eq. (12) has its own parameters (theta_rev): its decay A_rev and its
 * own skip weight D_rev; the skip weights may also be one per channel of x ([H][P], the
 * Mamba-2 layer's per-channel option) instead of one per head:
 *   y_t = C_t . S_t + C'_t . R_t + D (.) x_fwd[t] (+ D_rev (.) x_rev[t])
 * with (.) the per-head scalar or the per-channel product.
 *   state       the cached state in the form state_form:
 *                 BDSSM_STATE_F32   float32 [b][H][N][P] (as bdssm_block_step)
 *                 BDSSM_STATE_OPS   operand form (bdssm_state_ops; bf16 inputs, (d_state,
 *                                   headdim) = (128, 64), block_len <= 128 only)
 *                 BDSSM_STATE_BF16  bf16 state (bdssm_state_bf16)
 *               read only, never written
 *   params      A [H] required; D [H] (or [H][P]) required; A_rev [H] or NULL (= A);
 *               D_rev [H] (or [H][P]) or NULL (none); skip_per_channel 0 or 1
 * With the float32 state and per-head weights this is bdssm_block_step_ex, bitwise; with
 * the operand form, bdssm_block_step_ops. Errors as bdssm_block_step_ex, plus
 * BDSSM_ERR_UNSUPPORTED for an unknown state form or skip layout, or the operand form outside
 * its shapes. y must not overlap the state or any parameter.
 */
enum { BDSSM_STATE_F32 = 0, BDSSM_STATE_OPS = 1, BDSSM_STATE_BF16 = 2 };
typedef struct {
    const float *A, *D, *A_rev, *D_rev;
    int32_t skip_per_channel;
} bdssm_step_params;
bdssm_status bdssm_block_step_variant(const bdssm_dims *dims, int32_t block_len, const void *state,
                                      int32_t state_form, const bdssm_seq *fwd, const bdssm_seq *rev,
                                      const bdssm_step_params *params, void *y, void *stream);

/*
 * Commit with the block step's copy of the state refreshed in the same pass: bdssm_commit,
 * then state_copy <- the advanced state in the form state_form (BDSSM_STATE_OPS: the operand
 * form of bdssm_state_ops; BDSSM_STATE_BF16: the bf16 state of bdssm_state_bf16), bitwise
 * those calls' results. The cached state changes only at a commit (eqs. (9)-(11)), so this
 * is the one place a decode loop needs to re-encode it; with bf16 inputs, (d_state,
 * headdim) = (128, 64) and y == NULL one launch does both (the state walk writes both from
 * its registers), else a commit and an encoding launch.
 *   state_copy  [b][H][2][N/8][P][8] or [b][H][N/8][P][8] bf16; must not overlap h, y or
 *               any input
 * With block_len = 0 the state is unchanged and only the copy is written. Errors as
 * bdssm_commit, plus BDSSM_ERR_UNSUPPORTED for a state form other than those two, or the
 * operand form outside its shape.
 */
bdssm_status bdssm_commit_refresh(const bdssm_dims *dims, int32_t block_len, const bdssm_seq *clean,
                                  const float *A, const float *D, float *h, void *state_copy,
                                  int32_t state_form, void *y, void *stream);

/*
 * Convolution state. A Mamba layer's cache holds convolution state as well as the SSM
 * state (the cache discussion of "Training Hybrid Block Diffusion Language Models with
 * Partial Bidirectionality"); the pages leave the convolution itself open, and these calls
 * take the Mamba-2 layer's: before the scan, each of the CH = H*P + 2*G*N channels of a
 * token (x [H][P], then B [G][N], then C [G][N]) is convolved with its own `width` taps,
 * a bias is added and an activation applied, and the result, rounded to the input dtype,
 * is what the scan reads. dt is not convolved.
 *   forward (causal):   out_t = bias + sum_{k<W} w[k] u_{t-(W-1)+k}, where u_t for t < 0
 *                       comes from the conv state, the W-1 raw (unconvolved) rows that
 *                       precede the segment;
 *   reverse (anti-causal, the block's reverse branch, which has no state, eq. (12)):
 *                       out_t = bias + sum_{k<W} w[k] u_{t+(W-1)-k}, with u_t = 0 past the
 *                       segment's end (the causal convolution of the reversed block).
 * The conv state after a forward segment is the last W-1 rows of the raw input extended by
 * the previous state. Conv state layout: [b][W-1][CH] in dims->in_dtype.
 */
typedef struct {
    int32_t width;       /* W, 1..4 */
    int32_t activation;  /* 0 identity, 1 SiLU (v / (1 + exp(-v))) */
    const float *weight; /* [CH][W] float32, taps w[c][k] */
    const float *bias;   /* [CH] float32, or NULL for none */
} bdssm_conv_params;

/* Bytes of one convolved copy of x, B and C for `len` tokens (each part 256-byte aligned in
 * the buffer): bdssm_block_step_conv needs two, bdssm_commit_conv one. SIZE_MAX for
 * invalid dims or len < 0. */
size_t bdssm_conv_workspace(const bdssm_dims *dims, int64_t len);

/*
 * The convolution of one segment of `len` tokens: out.{x,B,C} <- act(conv(raw.{x,B,C})).
 *   reverse    0 forward (causal), 1 reverse (anti-causal)
 *   state_in   forward: [b][W-1][CH] history before the segment, or NULL for zeros (the
 *              start of a sequence); must be NULL when reverse
 *   raw, out   x, B, C are used (dt is ignored and may be NULL); out must not overlap raw,
 *              the parameters or the states
 *   state_out  forward: [b][W-1][CH] receives the new history, or NULL; it may be the same
 *              pointer as state_in (updated in place) but must not otherwise overlap
 *              anything; must be NULL when reverse
 * A prefix is convolved with this call (forward, state_in NULL, state_out = the cache's
 * conv state) before bdssm_prefix_scan reads it.
 */
bdssm_status bdssm_conv(const bdssm_dims *dims, int64_t len, const bdssm_conv_params *conv,
                        int32_t reverse, const void *state_in, const bdssm_seq *raw,
                        const bdssm_seq *out, void *state_out, void *stream);

/*
 * Block step on unconvolved inputs: the forward branch's x, B, C are convolved causally from
 * the cached conv state (conv_fwd), the reverse branch's anti-causally inside the block
 * (conv_rev, its own parameters; pass conv_fwd's for shared ones), both in one launch into
 * the workspace, then bdssm_block_step_ex runs on the convolved inputs with the raw dt.
 *   conv_state  [b][W_fwd-1][CH] in in_dtype, read only (NULL when W_fwd = 1)
 *   A_rev       as in bdssm_block_step_ex; NULL means A
 *   workspace   at least 2 * bdssm_conv_workspace(dims, block_len) bytes; must not overlap
 *               anything else
 * Everything else as bdssm_block_step_ex.
 */
bdssm_status bdssm_block_step_conv(const bdssm_dims *dims, int32_t block_len,
                                   const bdssm_conv_params *conv_fwd,
                                   const bdssm_conv_params *conv_rev, const float *h_prefix,
                                   const void *conv_state, const bdssm_seq *fwd,
                                   const bdssm_seq *rev, const float *A, const float *D,
                                   const float *A_rev, const float *D_rev, void *y,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * Commit on unconvolved inputs: the clean block is convolved causally from the conv state
 * into the workspace, the conv state is advanced in place, then bdssm_commit advances h.
 *   conv_state  [b][W-1][CH] in in_dtype, read then overwritten (NULL when W = 1)
 *   workspace   at least bdssm_conv_workspace(dims, block_len) bytes
 * Everything else as bdssm_commit, except that clean->C is always required (its raw rows
 * enter the conv state).
 */
bdssm_status bdssm_commit_conv(const bdssm_dims *dims, int32_t block_len,
                               const bdssm_conv_params *conv, const bdssm_seq *clean,
                               const float *A, const float *D, float *h, void *conv_state,
                               void *y, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode loop of one active block as a HIP graph: `steps` calls of bdssm_block_step (step
 * k reads fwd[k], rev[k] and writes y[k], all from the cached state h), followed, when
 * clean is not NULL, by bdssm_commit(clean, h, y_commit). This is the static-shape block
 * buffer of block-diffusion decoding, whose inputs change from step to step in place.
 *   fwd, rev   host arrays of `steps` input descriptors (device pointers)
 *   y          host array of `steps` device output pointers, [b][T][H][P] in y_dtype
 *   h          [b][H][N][P] float32: read by every step, then advanced by the commit
 *   h_ops      NULL, or the cached state in operand form (bdssm_state_ops of h, made by the
 *              caller before the first replay): the steps then read it (bdssm_block_step_ops)
 *              and the commit is followed by bdssm_state_ops(h -> h_ops), so that it holds
 *              the advanced state for the next replay
 *   clean      the commit's inputs, or NULL for steps only; y_commit as in bdssm_commit
 *   stream     the stream the calls are recorded on; must not be NULL (the legacy default
 *              stream cannot be captured). Nothing runs during creation.
 *   out        receives the graph; NULL on error
 * Every call is validated as bdssm_block_step / bdssm_commit validate it; the first
 * failing status is returned and no graph is made. The device pointers are baked into
 * the graph: the buffers must stay allocated, at the same addresses, while it exists.
 * Errors: BDSSM_ERR_NULL (dims, out, fwd, rev, y or stream NULL; steps < 1 with no commit),
 * BDSSM_ERR_SHAPE (steps < 0), the statuses of the recorded calls, BDSSM_ERR_HIP
 * (capture or instantiation failed).
 */
typedef struct bdssm_decode_graph bdssm_decode_graph;
bdssm_status bdssm_decode_graph_create(const bdssm_dims *dims, int32_t block_len, int32_t steps,
                                       float *h, void *h_ops, const bdssm_seq *fwd,
                                       const bdssm_seq *rev,
                                       const float *A, const float *D, void *const *y,
                                       const bdssm_seq *clean, void *y_commit, void *stream,
                                       bdssm_decode_graph **out);

/* Enqueues one replay of the recorded calls on `stream` (NULL = default stream). Runs
 * asynchronously, like the calls it replaces; allocates nothing. */
bdssm_status bdssm_decode_graph_launch(const bdssm_decode_graph *graph, void *stream);

/* Frees the graph (NULL is ignored). Replays already enqueued are not affected. */
void bdssm_decode_graph_destroy(bdssm_decode_graph *graph);

/*
 * Launch-shape override, for tests and launch-shape sweeps only (not for the hot path).
 * Several kernels implement the block step, each one in full and each checked against the
 * same bounds; the library picks one per call from the shapes. This call pins that choice
 * for every later call in the process until it is called again (NULL or all zeros =
 * automatic). Values are read once per call; a change racing with calls on other threads
 * applies to each of them either entirely or not at all.
 *   block_kernel  0 automatic; 1 the small-batch kernel (used where it applies:
 *                 block_len <= 32, bf16 inputs, (d_state, headdim) = (128, 64));
 *                 2 the bandwidth kernels
 *   lat_waves     small-batch kernel: wavefronts per workgroup, 2 or 4 (0 automatic)
 *   bw_heads      bandwidth kernels: heads per workgroup; ignored unless it divides H/G
 *                 (0 automatic)
 *   bw_splits     bandwidth kernel from the float32 state: column splits, 1, 2 or 4
 *                 (0 automatic)
 * Errors: BDSSM_ERR_UNSUPPORTED for values outside these sets (nothing is changed).
 */
typedef struct {
    int32_t block_kernel;
    int32_t lat_waves;
    int32_t bw_heads;
    int32_t bw_splits;
} bdssm_launch_override;
bdssm_status bdssm_set_launch_override(const bdssm_launch_override *o);

#ifdef __cplusplus
}
#endif

#endif /* BDSSM_H */
