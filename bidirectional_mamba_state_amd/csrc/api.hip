// Host side of the C ABI declared in include/bdssm.h: argument validation, the prefix
// scan's work plan and workspace, and kernel dispatch on the caller's stream.
#include <limits.h>
#include <stdlib.h>
#include <stdint.h>

#include <algorithm>

#include "bdssm.h"
#include "internal.h"

using namespace bdssm;

namespace bdssm {

// Compute units of the current device, cached per device (the only global state). Without
// a usable device (for instance a workspace query on a host without GPUs) the MI355X count
// is assumed, so that plans stay deterministic.
int device_cus()
{
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
            (void)hipGetLastError();
            v = 256;
        }
        __atomic_store_n(&cache[dev], v, __ATOMIC_RELAXED);
    }
    return v;
}

}  // namespace bdssm

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

Range rng(const void *p, int64_t bytes)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, p ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool aligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elt(int dtype) { return dtype == BDSSM_BF16 ? 2 : 4; }

bdssm_status check_dims(const bdssm_dims *d, Shape *s)
{
    if (!d)
        return BDSSM_ERR_NULL;
    if (d->batch < 0 || d->nheads < 1 || d->headdim < 1 || d->d_state < 1 || d->ngroups < 1)
        return BDSSM_ERR_SHAPE;
    if (d->nheads % d->ngroups != 0)
        return BDSSM_ERR_SHAPE;
    if ((d->in_dtype != BDSSM_F32 && d->in_dtype != BDSSM_BF16) ||
        (d->y_dtype != BDSSM_F32 && d->y_dtype != BDSSM_BF16))
        return BDSSM_ERR_UNSUPPORTED;
    if (!valu_supported(d->d_state, d->headdim) || d->nheads > 65535 || d->batch > 65535)
        return BDSSM_ERR_UNSUPPORTED;
    *s = Shape{d->batch, d->nheads, d->headdim, d->d_state, d->ngroups, d->in_dtype, d->y_dtype};
    return BDSSM_OK;
}

struct SeqRanges {
    Range x, dt, B, C;
};

// Checks a segment's pointers (C optional when need_c is false) and returns their byte ranges.
bdssm_status check_seq(const bdssm_seq *q, const Shape &s, int64_t len, bool need_c, SeqRanges *out)
{
    if (!q || !q->x || !q->dt || !q->B || (need_c && !q->C))
        return BDSSM_ERR_NULL;
    if (!aligned(q->x) || !aligned(q->dt) || !aligned(q->B) || (q->C && !aligned(q->C)))
        return BDSSM_ERR_ALIGN;
    const int64_t e = elt(s.in_dt), tok = static_cast<int64_t>(s.b) * len;
    out->x = rng(q->x, tok * s.H * s.P * e);
    out->dt = rng(q->dt, tok * s.H * e);
    out->B = rng(q->B, tok * s.G * s.N * e);
    out->C = rng(q->C, tok * s.G * s.N * e);
    return BDSSM_OK;
}

bool hits(Range o, const SeqRanges &q) { return overlap(o, q.x) || overlap(o, q.dt) || overlap(o, q.B) || overlap(o, q.C); }

bool chunk_ok(int32_t chunk)
{
    return chunk == 16 || chunk == 32 || chunk == 64 || chunk == 128 || chunk == 256;
}

// Work plan of one prefix scan.
//  - chunk states or y requested: segments are the Q-token chunks; a chunk-local pass, a
//    state-passing pass, then (for y) a pass that recomputes each chunk from its entering
//    state. Chunk-local states live in chunk_states when given, else in the workspace.
//  - state only: segments of several chunks, just enough of them to fill the GPU; when one
//    segment per (stream, head) already fills it, a single pass runs from h_init to h_out.
struct Plan {
    int64_t seg_len;
    int nseg;
    bool states_in_ws;   // chunk-local states kept in the workspace
    size_t decay_bytes;  // workspace bytes for per-segment decay sums (256-byte rounded)
    size_t ws_bytes;
};

Plan plan_prefix(const Shape &s, int64_t len, int32_t chunk, bool with_y, bool with_cs)
{
    Plan p{};
    const int64_t NP = static_cast<int64_t>(s.N) * s.P;
    if (with_y || with_cs) {
        p.seg_len = chunk;
    } else {
        const int64_t pairs = std::max<int64_t>(1, static_cast<int64_t>(s.b) * s.H);
        const int64_t want = (2048 + pairs - 1) / pairs;  // segments per (stream, head)
        int64_t seg = (len + want - 1) / want;
        seg = (seg + chunk - 1) / chunk * chunk;
        p.seg_len = std::max<int64_t>(seg, chunk);
    }
    p.nseg = static_cast<int>((len + p.seg_len - 1) / p.seg_len);
    const bool single = !with_y && !with_cs && p.nseg == 1;
    p.states_in_ws = !with_cs && !single;
    const int64_t n_bh = static_cast<int64_t>(s.b) * p.nseg * s.H;
    p.decay_bytes = single ? 0 : static_cast<size_t>((n_bh * 4 + 255) / 256 * 256);
    p.ws_bytes = p.decay_bytes + (p.states_in_ws ? static_cast<size_t>(n_bh * NP * 4) : 0);
    return p;
}

bdssm_status launched(hipError_t e) { return e == hipSuccess ? BDSSM_OK : BDSSM_ERR_HIP; }

// Launch-shape override (bdssm_set_launch_override; tests and launch-shape sweeps only):
// block kernel choice, small-batch wavefronts per workgroup, bandwidth-kernel heads per
// workgroup and column splits; 0 = automatic. Read with relaxed atomic loads once per call.
int g_override[4];
int override_of(int i) { return __atomic_load_n(&g_override[i], __ATOMIC_RELAXED); }
enum { OV_KERNEL, OV_LAT_WAVES, OV_BW_HEADS, OV_BW_SPLITS };

void override_block_plan(const Shape &s, int *hpw, int *ps)
{
    const int v = override_of(OV_BW_HEADS);
    if (v >= 1 && (s.H / s.G) % v == 0)
        *hpw = v;
    const int p = override_of(OV_BW_SPLITS);
    if (p == 1 || p == 2 || p == 4)
        *ps = p;
}

// Validates a block step and fills its kernel arguments (nothing is launched).
// state_elt: bytes per state element as stored (4: float32 or operand form, 2: bf16);
// dch: skip weights per head and channel ([H][P]).
bdssm_status prepare_block_step(const bdssm_dims *dims, int32_t block_len, const float *h_prefix,
                                const bdssm_seq *fwd, const bdssm_seq *rev, const float *A,
                                const float *D, const float *A_rev, const float *D_rev, void *y,
                                BlockArgs *out, int state_elt = 4, bool dch = false)
{
    Shape s;
    bdssm_status rc = check_dims(dims, &s);
    if (rc != BDSSM_OK)
        return rc;
    if (block_len < 0)
        return BDSSM_ERR_SHAPE;
    if (block_len > 256)
        return BDSSM_ERR_UNSUPPORTED;
    if (!h_prefix || !A || !D || !A_rev || !y)
        return BDSSM_ERR_NULL;
    SeqRanges qf{}, qr{};
    if ((rc = check_seq(fwd, s, block_len, true, &qf)) != BDSSM_OK)
        return rc;
    if ((rc = check_seq(rev, s, block_len, true, &qr)) != BDSSM_OK)
        return rc;
    if (!aligned(h_prefix) || !aligned(A) || !aligned(D) || !aligned(A_rev) || !aligned(D_rev) ||
        !aligned(y))
        return BDSSM_ERR_ALIGN;
    const int64_t NP = static_cast<int64_t>(s.N) * s.P;
    const int64_t dbytes = (dch ? static_cast<int64_t>(s.H) * s.P : s.H) * 4;
    const Range ry = rng(y, static_cast<int64_t>(s.b) * block_len * s.H * s.P * elt(s.y_dt));
    if (hits(ry, qf) || hits(ry, qr) ||
        overlap(ry, rng(h_prefix, static_cast<int64_t>(s.b) * s.H * NP * state_elt)) ||
        overlap(ry, rng(A, s.H * 4)) || overlap(ry, rng(D, dbytes)) || overlap(ry, rng(A_rev, s.H * 4)) ||
        overlap(ry, rng(D_rev, dbytes)))
        return BDSSM_ERR_ALIAS;
    *out = BlockArgs{s, block_len, h_prefix, Seq{fwd->x, fwd->dt, fwd->B, fwd->C},
                     Seq{rev->x, rev->dt, rev->B, rev->C}, A, D, y, A_rev, D_rev};
    out->d_per_channel = dch ? 1 : 0;
    return BDSSM_OK;
}

// Small batches (fewer (stream, head) pairs than fill the GPU with one workgroup per CU)
// take the latency-ordered kernel, one workgroup per (head, row block, column part); the
// launch-shape override can force either kernel where both apply.
bool use_block_lat(const Shape &s, int T)
{
    if (!block_lat_supported(s, T))
        return false;
    const int k = override_of(OV_KERNEL);
    if (k != 0)
        return k == 1;
    return static_cast<int64_t>(s.b) * s.H < 512;
}

bdssm_status launch_block_step(const BlockArgs &a, hipStream_t st)
{
    if (use_block_lat(a.s, a.T)) {
        return launched(launch_block_step_lat(a, override_of(OV_LAT_WAVES), st));
    }
    if (block_mfma_supported(a.s, a.T)) {
        int hpw, ps;
        block_mfma_plan(a.s, &hpw, &ps);
        override_block_plan(a.s, &hpw, &ps);
        return launched(launch_block_step_mfma(a, hpw, ps, st));
    }
    return launched(launch_block_step_valu(a, st));
}

// Validates a commit (nothing is launched).
bdssm_status prepare_commit(const bdssm_dims *dims, int32_t block_len, const bdssm_seq *clean,
                            const float *A, const float *D, float *h, void *y, Shape *out)
{
    Shape s;
    bdssm_status rc = check_dims(dims, &s);
    if (rc != BDSSM_OK)
        return rc;
    if (block_len < 0)
        return BDSSM_ERR_SHAPE;
    if (block_len > 256)
        return BDSSM_ERR_UNSUPPORTED;
    if (!A || !D || !h)
        return BDSSM_ERR_NULL;
    SeqRanges q{};
    if ((rc = check_seq(clean, s, block_len, y != nullptr, &q)) != BDSSM_OK)
        return rc;
    if (!aligned(A) || !aligned(D) || !aligned(h) || !aligned(y))
        return BDSSM_ERR_ALIGN;
    const int64_t NP = static_cast<int64_t>(s.N) * s.P;
    const Range rh = rng(h, static_cast<int64_t>(s.b) * s.H * NP * 4);
    const Range ry = rng(y, static_cast<int64_t>(s.b) * block_len * s.H * s.P * elt(s.y_dt));
    for (Range o : {rh, ry}) {
        if (hits(o, q) || overlap(o, rng(A, s.H * 4)) || overlap(o, rng(D, s.H * 4)))
            return BDSSM_ERR_ALIAS;
    }
    if (overlap(rh, ry))
        return BDSSM_ERR_ALIAS;
    *out = s;
    return BDSSM_OK;
}

bdssm_status launch_commit(const Shape &s, int32_t block_len, const Seq &seq, const float *A, const float *D,
                           float *h, void *y, hipStream_t st)
{
    // a commit is a prefix scan of the block from h, in place: on the matrix-core prefix
    // path, one segment per (stream, head) (no workspace)
    if (prefix_mfma_supported(s, 64))
        return launched(run_prefix_mfma(s, block_len, 64, seq, A, D, h, y, nullptr, h, nullptr, st, true));
    ForwardArgs f{s, block_len, block_len, 1, seq, A, D, h, nullptr, y, h, nullptr};
    return launched(launch_forward_valu(f, st));
}

// ---- convolution state
struct ConvRanges {
    Range w, b;
};

bdssm_status check_conv(const bdssm_conv_params *c, const Shape &s, ConvRanges *out)
{
    if (!c || !c->weight)
        return BDSSM_ERR_NULL;
    if (c->width < 1 || c->width > 4 || (c->activation != 0 && c->activation != 1))
        return BDSSM_ERR_UNSUPPORTED;
    if ((s.H * s.P) % 8 != 0 || (s.G * s.N) % 8 != 0)
        return BDSSM_ERR_UNSUPPORTED;
    if (!aligned(c->weight) || !aligned(c->bias))
        return BDSSM_ERR_ALIGN;
    const int64_t ch = static_cast<int64_t>(s.H) * s.P + 2 * static_cast<int64_t>(s.G) * s.N;
    out->w = rng(c->weight, ch * c->width * 4);
    out->b = rng(c->bias, ch * 4);
    return BDSSM_OK;
}

int64_t conv_state_bytes(const Shape &s, int width)
{
    const int64_t ch = static_cast<int64_t>(s.H) * s.P + 2 * static_cast<int64_t>(s.G) * s.N;
    return static_cast<int64_t>(s.b) * (width - 1) * ch * elt(s.in_dt);
}

// x, B and C of a segment (dt not needed) with their byte ranges
bdssm_status check_xbc(const bdssm_seq *q, const Shape &s, int64_t len, SeqRanges *out)
{
    if (!q || !q->x || !q->B || !q->C)
        return BDSSM_ERR_NULL;
    if (!aligned(q->x) || !aligned(q->B) || !aligned(q->C))
        return BDSSM_ERR_ALIGN;
    const int64_t e = elt(s.in_dt), tok = static_cast<int64_t>(s.b) * len;
    out->x = rng(q->x, tok * s.H * s.P * e);
    out->dt = rng(nullptr, 0);
    out->B = rng(q->B, tok * s.G * s.N * e);
    out->C = rng(q->C, tok * s.G * s.N * e);
    return BDSSM_OK;
}

// one convolved copy of x, B, C in a workspace: offsets of B and C, total bytes
struct ConvCopy {
    size_t B, C, total;
};

ConvCopy conv_copy_bytes(const Shape &s, int64_t len)
{
    auto r256 = [](int64_t v) { return static_cast<size_t>((v + 255) / 256 * 256); };
    const int64_t e = elt(s.in_dt), tok = static_cast<int64_t>(s.b) * len;
    const size_t xb = r256(tok * s.H * s.P * e), bb = r256(tok * s.G * s.N * e);
    return ConvCopy{xb, xb + bb, xb + 2 * bb};
}

// ---- the static scratch buffer of bdssm_prefix_scan_static: device memory the library
// holds for callers that cannot allocate. Each GPU has its own copy at its own address; in
// host code the array's name is only a stand-in, so the address is taken per device with
// hipGetSymbolAddress (with that device current, on the first call there) and only that
// address is passed to kernels.
constexpr size_t kStaticScratchBytes = BDSSM_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

bdssm_status static_scratch_ptr(void **out)
{
    static void *cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return BDSSM_ERR_HIP;
    }
    void *p = __atomic_load_n(&cache[dev], __ATOMIC_ACQUIRE);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return BDSSM_ERR_HIP;
        }
        __atomic_store_n(&cache[dev], p, __ATOMIC_RELEASE);
    }
    *out = p;
    return BDSSM_OK;
}

// The vector-ALU prefix scan of plan p (workspace already checked). rev: the tokens in
// reverse order, outputs added to y (y required, no chunk states, h_out may be NULL).
bdssm_status run_prefix_valu(const Shape &s, int64_t len, const Plan &p, const Seq &seq, const float *A,
                             const float *D, const float *h_init, void *y, float *chunk_states, float *h_out,
                             void *workspace, bool rev, hipStream_t st)
{
    const bool with_y = y != nullptr, with_cs = chunk_states != nullptr;
    const int64_t NP = static_cast<int64_t>(s.N) * s.P;
    const int r = rev ? 1 : 0;
    bdssm_status rc;
    if (!with_y && !with_cs && p.nseg == 1) {
        // one pass per (stream, head), from h_init straight to h_out (in place is safe:
        // each workgroup reads its whole state before it writes any of it)
        ForwardArgs f{s, len, static_cast<int>(p.seg_len), 1, seq, A, D, h_init, nullptr,
                      nullptr, h_out, nullptr, r};
        return launched(launch_forward_valu(f, st));
    }

    float *decay = static_cast<float *>(workspace);
    float *states = with_cs ? chunk_states
                            : reinterpret_cast<float *>(static_cast<char *>(workspace) + p.decay_bytes);
    // 1. chunk-local states (from zero) and decay sums
    ForwardArgs f1{s, len, static_cast<int>(p.seg_len), p.nseg, seq, A, D, nullptr, nullptr,
                   nullptr, states, decay, r};
    if ((rc = launched(launch_forward_valu(f1, st))) != BDSSM_OK)
        return rc;
    // 2. pass states across segments. With y, h_init must survive until pass 3 reads it,
    //    so h_out is written afterwards from the last chunk state.
    PassArgs pa{s, p.nseg, h_init, states, decay, (with_y || with_cs) ? 1 : 0,
                with_y ? nullptr : h_out};
    if ((rc = launched(launch_state_pass(pa, st))) != BDSSM_OK)
        return rc;
    if (!with_y)
        return BDSSM_OK;
    // 3. outputs: each chunk recomputed from the state entering it
    ForwardArgs f3{s, len, static_cast<int>(p.seg_len), p.nseg, seq, A, D, h_init, states,
                   y, nullptr, nullptr, r};
    if ((rc = launched(launch_forward_valu(f3, st))) != BDSSM_OK)
        return rc;
    for (int b = 0; h_out && b < s.b; ++b) {
        rc = launched(launch_copy_f32(h_out + static_cast<int64_t>(b) * s.H * NP,
                                      states + (static_cast<int64_t>(b) * p.nseg + p.nseg - 1) * s.H * NP,
                                      s.H * NP, st));
        if (rc != BDSSM_OK)
            return rc;
    }
    return BDSSM_OK;
}

// bdssm_prefix_scan and bdssm_prefix_scan_static: with static_scratch the workspace comes
// from the library's static device buffer instead of the caller.
bdssm_status prefix_scan_impl(const bdssm_dims *dims, int64_t len, int32_t chunk, const bdssm_seq *in,
                              const float *A, const float *D, const float *h_init, void *y,
                              float *chunk_states, float *h_out, void *workspace, size_t workspace_bytes,
                              bool static_scratch, void *stream)
{
    Shape s;
    bdssm_status rc = check_dims(dims, &s);
    if (rc != BDSSM_OK)
        return rc;
    if (len < 0)
        return BDSSM_ERR_SHAPE;
    if (!chunk_ok(chunk))
        return BDSSM_ERR_UNSUPPORTED;
    if (!in || !A || !D || !h_out)
        return BDSSM_ERR_NULL;
    SeqRanges q{};
    if ((rc = check_seq(in, s, len, y != nullptr, &q)) != BDSSM_OK)
        return rc;
    if (!aligned(A) || !aligned(D) || !aligned(h_init) || !aligned(y) || !aligned(chunk_states) ||
        !aligned(h_out) || !aligned(workspace))
        return BDSSM_ERR_ALIGN;
    const int64_t NP = static_cast<int64_t>(s.N) * s.P;
    const int64_t state_bytes = static_cast<int64_t>(s.b) * s.H * NP * 4;
    const int64_t nch = (len + chunk - 1) / chunk;
    const Range ry = rng(y, static_cast<int64_t>(s.b) * len * s.H * s.P * elt(s.y_dt));
    const Range rcs = rng(chunk_states, static_cast<int64_t>(s.b) * nch * s.H * NP * 4);
    const Range rho = rng(h_out, state_bytes);
    const Range rhi = rng(h_init, state_bytes);
    const Range rA = rng(A, s.H * 4), rD = rng(D, s.H * 4);
    for (Range o : {ry, rcs, rho}) {
        if (hits(o, q) || overlap(o, rA) || overlap(o, rD))
            return BDSSM_ERR_ALIAS;
    }
    if (overlap(ry, rcs) || overlap(ry, rho) || overlap(rcs, rho) || overlap(ry, rhi) ||
        overlap(rcs, rhi))
        return BDSSM_ERR_ALIAS;
    if (overlap(rho, rhi) && h_out != h_init)
        return BDSSM_ERR_ALIAS;

    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s.b == 0)
        return BDSSM_OK;
    if (len == 0) {  // the scan of no tokens is the identity on the state
        if (h_init == h_out)
            return BDSSM_OK;
        return launched(h_init ? launch_copy_f32(h_out, h_init, state_bytes / 4, st)
                               : launch_fill_f32(h_out, 0.f, state_bytes / 4, st));
    }

    const bool with_y = y != nullptr, with_cs = chunk_states != nullptr;
    const Seq seq{in->x, in->dt, in->B, in->C};
    if (static_scratch) {
        // the plan's workspace from the static buffer (nothing to clear: every byte a kernel
        // reads from it is written earlier in the same call)
        const size_t need = prefix_mfma_supported(s, chunk)
                                ? prefix_mfma_plan(s, len, chunk, with_y || with_cs).ws_bytes
                                : plan_prefix(s, len, chunk, with_y, with_cs).ws_bytes;
        workspace = nullptr;
        workspace_bytes = 0;
        if (need > 0) {
            if (need > kStaticScratchBytes)
                return BDSSM_ERR_SCRATCH;
            if ((rc = static_scratch_ptr(&workspace)) != BDSSM_OK)
                return rc;
            workspace_bytes = kStaticScratchBytes;
        }
    }
    if (prefix_mfma_supported(s, chunk)) {
        const PrefixPlan mp = prefix_mfma_plan(s, len, chunk, with_y || with_cs);
        if (mp.ws_bytes > 0) {
            if (!workspace || workspace_bytes < mp.ws_bytes)
                return BDSSM_ERR_WORKSPACE;
            const Range rws = rng(workspace, static_cast<int64_t>(mp.ws_bytes));
            if (hits(rws, q) || overlap(rws, ry) || overlap(rws, rcs) || overlap(rws, rho) ||
                overlap(rws, rhi) || overlap(rws, rA) || overlap(rws, rD))
                return BDSSM_ERR_ALIAS;
        }
        return launched(run_prefix_mfma(s, len, chunk, seq, A, D, h_init, y, chunk_states, h_out,
                                        workspace, st));
    }
    const Plan p = plan_prefix(s, len, chunk, with_y, with_cs);
    if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes))
        return BDSSM_ERR_WORKSPACE;
    if (p.ws_bytes > 0) {
        const Range rws = rng(workspace, static_cast<int64_t>(p.ws_bytes));
        if (hits(rws, q) || overlap(rws, ry) || overlap(rws, rcs) || overlap(rws, rho) ||
            overlap(rws, rhi) || overlap(rws, rA) || overlap(rws, rD))
            return BDSSM_ERR_ALIAS;
    }

    return run_prefix_valu(s, len, p, seq, A, D, h_init, y, chunk_states, h_out, workspace, false, st);
}

}  // namespace

extern "C" {

int bdssm_abi_version(void) { return BDSSM_ABI_VERSION; }

const char *bdssm_status_str(int status)
{
    switch (status) {
    case BDSSM_OK: return "BDSSM_OK";
    case BDSSM_ERR_NULL: return "BDSSM_ERR_NULL: a required pointer is NULL";
    case BDSSM_ERR_SHAPE: return "BDSSM_ERR_SHAPE: invalid or inconsistent sizes";
    case BDSSM_ERR_UNSUPPORTED: return "BDSSM_ERR_UNSUPPORTED: no kernel for this shape, chunk or dtype";
    case BDSSM_ERR_ALIGN: return "BDSSM_ERR_ALIGN: a pointer is not 16-byte aligned";
    case BDSSM_ERR_ALIAS: return "BDSSM_ERR_ALIAS: an output overlaps an input";
    case BDSSM_ERR_WORKSPACE: return "BDSSM_ERR_WORKSPACE: workspace missing or too small";
    case BDSSM_ERR_HIP: return "BDSSM_ERR_HIP: the HIP runtime reported a launch error";
    case BDSSM_ERR_SCRATCH:
        return "BDSSM_ERR_SCRATCH: the call needs more workspace than the library's static scratch buffer holds";
    default: return "unknown bdssm status";
    }
}

size_t bdssm_prefix_scan_workspace(const bdssm_dims *dims, int64_t len, int32_t chunk,
                                   int32_t with_y, int32_t with_chunk_states)
{
    Shape s;
    if (check_dims(dims, &s) != BDSSM_OK || len < 0 || !chunk_ok(chunk))
        return SIZE_MAX;
    if (len == 0 || s.b == 0)
        return 0;
    if (prefix_mfma_supported(s, chunk))
        return prefix_mfma_plan(s, len, chunk, with_y || with_chunk_states).ws_bytes;
    return plan_prefix(s, len, chunk, with_y != 0, with_chunk_states != 0).ws_bytes;
}

bdssm_status bdssm_prefix_scan(const bdssm_dims *dims, int64_t len, int32_t chunk,
                               const bdssm_seq *in, const float *A, const float *D,
                               const float *h_init, void *y, float *chunk_states,
                               float *h_out, void *workspace, size_t workspace_bytes,
                               void *stream)
{
    return prefix_scan_impl(dims, len, chunk, in, A, D, h_init, y, chunk_states, h_out, workspace,
                            workspace_bytes, false, stream);
}

bdssm_status bdssm_prefix_scan_static(const bdssm_dims *dims, int64_t len, int32_t chunk,
                                      const bdssm_seq *in, const float *A, const float *D,
                                      const float *h_init, void *y, float *chunk_states,
                                      float *h_out, void *stream)
{
    return prefix_scan_impl(dims, len, chunk, in, A, D, h_init, y, chunk_states, h_out, nullptr, 0, true,
                            stream);
}

size_t bdssm_full_window_workspace(const bdssm_dims *dims, int64_t len, int32_t chunk)
{
    // both directions run the prefix scan's plan with outputs, one after the other, in the
    // same workspace
    return bdssm_prefix_scan_workspace(dims, len, chunk, 1, 0);
}

bdssm_status bdssm_full_window(const bdssm_dims *dims, int64_t len, int32_t chunk, const bdssm_seq *fwd,
                               const bdssm_seq *rev, const float *A, const float *D, const float *A_rev,
                               const float *D_rev, void *y, void *workspace, size_t workspace_bytes,
                               void *stream)
{
    Shape s;
    bdssm_status rc = check_dims(dims, &s);
    if (rc != BDSSM_OK)
        return rc;
    if (len < 0)
        return BDSSM_ERR_SHAPE;
    if (!chunk_ok(chunk))
        return BDSSM_ERR_UNSUPPORTED;
    if (!A || !D || !A_rev || !y)
        return BDSSM_ERR_NULL;
    SeqRanges qf{}, qr{};
    if ((rc = check_seq(fwd, s, len, true, &qf)) != BDSSM_OK || (rc = check_seq(rev, s, len, true, &qr)) != BDSSM_OK)
        return rc;
    if (!aligned(A) || !aligned(D) || !aligned(A_rev) || !aligned(D_rev) || !aligned(y) || !aligned(workspace))
        return BDSSM_ERR_ALIGN;
    const Range ry = rng(y, static_cast<int64_t>(s.b) * len * s.H * s.P * elt(s.y_dt));
    const Range rp[4] = {rng(A, s.H * 4), rng(D, s.H * 4), rng(A_rev, s.H * 4), rng(D_rev, s.H * 4)};
    if (hits(ry, qf) || hits(ry, qr))
        return BDSSM_ERR_ALIAS;
    for (const Range &r : rp)
        if (overlap(ry, r))
            return BDSSM_ERR_ALIAS;
    if (s.b == 0 || len == 0)
        return BDSSM_OK;
    const bool mfma = prefix_mfma_supported(s, chunk);
    const size_t need = mfma ? prefix_mfma_plan(s, len, chunk, true).ws_bytes
                             : plan_prefix(s, len, chunk, true, false).ws_bytes;
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return BDSSM_ERR_WORKSPACE;
        const Range rws = rng(workspace, static_cast<int64_t>(need));
        if (hits(rws, qf) || hits(rws, qr) || overlap(rws, ry))
            return BDSSM_ERR_ALIAS;
        for (const Range &r : rp)
            if (overlap(rws, r))
                return BDSSM_ERR_ALIAS;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Seq sf{fwd->x, fwd->dt, fwd->B, fwd->C}, sr{rev->x, rev->dt, rev->B, rev->C};
    if (mfma) {
        // forward from zero over the window (writes y, with D x), then the reverse scan from
        // zero at the window's end (adds its outputs, with D_rev x_rev when given)
        if ((rc = launched(run_prefix_mfma(s, len, chunk, sf, A, D, nullptr, y, nullptr, nullptr, workspace, st)))
            != BDSSM_OK)
            return rc;
        return launched(run_prefix_mfma(s, len, chunk, sr, A_rev, D_rev, nullptr, y, nullptr, nullptr, workspace,
                                        st, false, true));
    }
    const Plan p = plan_prefix(s, len, chunk, true, false);
    if ((rc = run_prefix_valu(s, len, p, sf, A, D, nullptr, y, nullptr, nullptr, workspace, false, st)) != BDSSM_OK)
        return rc;
    return run_prefix_valu(s, len, p, sr, A_rev, D_rev, nullptr, y, nullptr, nullptr, workspace, true, st);
}

bdssm_status bdssm_block_step(const bdssm_dims *dims, int32_t block_len,
                              const float *h_prefix, const bdssm_seq *fwd,
                              const bdssm_seq *rev, const float *A, const float *D, void *y,
                              void *stream)
{
    return bdssm_block_step_ex(dims, block_len, h_prefix, fwd, rev, A, D, A, nullptr, y, stream);
}

bdssm_status bdssm_block_step_ex(const bdssm_dims *dims, int32_t block_len,
                                 const float *h_prefix, const bdssm_seq *fwd,
                                 const bdssm_seq *rev, const float *A, const float *D,
                                 const float *A_rev, const float *D_rev, void *y, void *stream)
{
    BlockArgs a{};
    const bdssm_status rc = prepare_block_step(dims, block_len, h_prefix, fwd, rev, A, D, A_rev, D_rev, y, &a);
    if (rc != BDSSM_OK || a.s.b == 0 || block_len == 0)
        return rc;
    return launch_block_step(a, static_cast<hipStream_t>(stream));
}

bdssm_status bdssm_set_launch_override(const bdssm_launch_override *o)
{
    const bdssm_launch_override z{0, 0, 0, 0};
    const bdssm_launch_override &v = o ? *o : z;
    if (v.block_kernel < 0 || v.block_kernel > 2 || (v.lat_waves != 0 && v.lat_waves != 2 && v.lat_waves != 4) ||
        v.bw_heads < 0 || (v.bw_splits != 0 && v.bw_splits != 1 && v.bw_splits != 2 && v.bw_splits != 4))
        return BDSSM_ERR_UNSUPPORTED;
    __atomic_store_n(&g_override[OV_KERNEL], v.block_kernel, __ATOMIC_RELAXED);
    __atomic_store_n(&g_override[OV_LAT_WAVES], v.lat_waves, __ATOMIC_RELAXED);
    __atomic_store_n(&g_override[OV_BW_HEADS], v.bw_heads, __ATOMIC_RELAXED);
    __atomic_store_n(&g_override[OV_BW_SPLITS], v.bw_splits, __ATOMIC_RELAXED);
    return BDSSM_OK;
}

size_t bdssm_state_ops_bytes(const bdssm_dims *dims)
{
    Shape s;
    if (check_dims(dims, &s) != BDSSM_OK || s.N != 128 || s.P != 64)
        return SIZE_MAX;
    return static_cast<size_t>(s.b) * s.H * s.N * s.P * 4;
}

bdssm_status bdssm_state_ops(const bdssm_dims *dims, const float *h, void *ops, void *stream)
{
    Shape s;
    const bdssm_status rc = check_dims(dims, &s);
    if (rc != BDSSM_OK)
        return rc;
    if (s.N != 128 || s.P != 64)
        return BDSSM_ERR_UNSUPPORTED;
    if (!h || !ops)
        return BDSSM_ERR_NULL;
    if (!aligned(h) || !aligned(ops))
        return BDSSM_ERR_ALIGN;
    const int64_t bytes = static_cast<int64_t>(s.b) * s.H * s.N * s.P * 4;
    if (overlap(rng(ops, bytes), rng(h, bytes)))
        return BDSSM_ERR_ALIAS;
    return launched(launch_state_ops(h, ops, static_cast<int64_t>(s.b) * s.H, static_cast<hipStream_t>(stream)));
}

bdssm_status bdssm_block_step_ops(const bdssm_dims *dims, int32_t block_len, const void *h_ops,
                                  const bdssm_seq *fwd, const bdssm_seq *rev, const float *A,
                                  const float *D, const float *A_rev, const float *D_rev, void *y,
                                  void *stream)
{
    BlockArgs a{};
    // the operand form has the float32 state's size, so the same validation applies
    const bdssm_status rc = prepare_block_step(dims, block_len, static_cast<const float *>(h_ops), fwd, rev, A, D,
                                               A_rev, D_rev, y, &a);
    if (rc != BDSSM_OK)
        return rc;
    if (a.s.b == 0 || block_len == 0)
        return BDSSM_OK;
    a.h_ops = h_ops;
    a.h_prefix = nullptr;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (use_block_lat(a.s, block_len)) {
        return launched(launch_block_step_lat(a, override_of(OV_LAT_WAVES), st));
    }
    if (!block_bw_supported(a.s, block_len))
        return BDSSM_ERR_UNSUPPORTED;
    int hpw = block_bw_plan(a.s), ps = 1;
    override_block_plan(a.s, &hpw, &ps);
    return launched(launch_block_step_bw(a, hpw, st));
}

size_t bdssm_state_bf16_bytes(const bdssm_dims *dims)
{
    Shape s;
    if (check_dims(dims, &s) != BDSSM_OK || s.N % 8 != 0)
        return SIZE_MAX;
    return static_cast<size_t>(s.b) * s.H * s.N * s.P * 2;
}

bdssm_status bdssm_state_bf16(const bdssm_dims *dims, const float *h, void *out, void *stream)
{
    Shape s;
    const bdssm_status rc = check_dims(dims, &s);
    if (rc != BDSSM_OK)
        return rc;
    if (s.N % 8 != 0)
        return BDSSM_ERR_UNSUPPORTED;
    if (!h || !out)
        return BDSSM_ERR_NULL;
    if (!aligned(h) || !aligned(out))
        return BDSSM_ERR_ALIGN;
    const int64_t n = static_cast<int64_t>(s.b) * s.H * s.N * s.P;
    if (overlap(rng(out, n * 2), rng(h, n * 4)))
        return BDSSM_ERR_ALIAS;
    if (n == 0)
        return BDSSM_OK;
    return launched(launch_state_bf16(h, out, static_cast<int64_t>(s.b) * s.H, s.N, s.P,
                                      static_cast<hipStream_t>(stream)));
}

bdssm_status bdssm_block_step_variant(const bdssm_dims *dims, int32_t block_len, const void *state,
                                      int32_t state_form, const bdssm_seq *fwd, const bdssm_seq *rev,
                                      const bdssm_step_params *params, void *y, void *stream)
{
    if (!params)
        return BDSSM_ERR_NULL;
    if (state_form != BDSSM_STATE_F32 && state_form != BDSSM_STATE_OPS && state_form != BDSSM_STATE_BF16)
        return BDSSM_ERR_UNSUPPORTED;
    if (params->skip_per_channel != 0 && params->skip_per_channel != 1)
        return BDSSM_ERR_UNSUPPORTED;
    const bool dch = params->skip_per_channel != 0;
    const float *A_rev = params->A_rev ? params->A_rev : params->A;
    BlockArgs a{};
    const bdssm_status rc = prepare_block_step(dims, block_len, static_cast<const float *>(state), fwd, rev,
                                               params->A, params->D, A_rev, params->D_rev, y, &a,
                                               state_form == BDSSM_STATE_BF16 ? 2 : 4, dch);
    if (rc != BDSSM_OK)
        return rc;
    const Shape &s = a.s;
    const bool mc = s.in_dt == 1 && s.N == 128 && s.P == 64;  // the matrix-core kernels' shapes
    if (state_form == BDSSM_STATE_OPS && (!mc || block_len > 128))
        return BDSSM_ERR_UNSUPPORTED;
    if (state_form == BDSSM_STATE_BF16 && s.N % 8 != 0)
        return BDSSM_ERR_UNSUPPORTED;
    if (s.b == 0 || block_len == 0)
        return BDSSM_OK;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (state_form == BDSSM_STATE_F32)
        return launch_block_step(a, st);
    a.h_ops = state;
    a.h_prefix = nullptr;
    a.ops_hi_only = state_form == BDSSM_STATE_BF16 ? 1 : 0;
    if (use_block_lat(s, block_len))
        return launched(launch_block_step_lat(a, override_of(OV_LAT_WAVES), st));
    if (mc && block_bw_supported(s, block_len)) {
        int hpw = block_bw_plan(s), ps = 1;
        override_block_plan(s, &hpw, &ps);
        return launched(launch_block_step_bw(a, hpw, st));
    }
    // the bf16 state on the vector-ALU kernel (float32 inputs, other shapes, T > 128)
    return launched(launch_block_step_valu(a, st));
}

bdssm_status bdssm_commit(const bdssm_dims *dims, int32_t block_len, const bdssm_seq *clean,
                          const float *A, const float *D, float *h, void *y, void *stream)
{
    Shape s;
    const bdssm_status rc = prepare_commit(dims, block_len, clean, A, D, h, y, &s);
    if (rc != BDSSM_OK || s.b == 0 || block_len == 0)
        return rc;
    return launch_commit(s, block_len, Seq{clean->x, clean->dt, clean->B, clean->C}, A, D, h, y,
                         static_cast<hipStream_t>(stream));
}

bdssm_status bdssm_commit_refresh(const bdssm_dims *dims, int32_t block_len, const bdssm_seq *clean,
                                  const float *A, const float *D, float *h, void *state_copy,
                                  int32_t state_form, void *y, void *stream)
{
    Shape s;
    bdssm_status rc = prepare_commit(dims, block_len, clean, A, D, h, y, &s);
    if (rc != BDSSM_OK)
        return rc;
    if (state_form != BDSSM_STATE_OPS && state_form != BDSSM_STATE_BF16)
        return BDSSM_ERR_UNSUPPORTED;
    if (state_form == BDSSM_STATE_OPS && (s.N != 128 || s.P != 64))
        return BDSSM_ERR_UNSUPPORTED;
    if (state_form == BDSSM_STATE_BF16 && s.N % 8 != 0)
        return BDSSM_ERR_UNSUPPORTED;
    if (!state_copy)
        return BDSSM_ERR_NULL;
    if (!aligned(state_copy))
        return BDSSM_ERR_ALIGN;
    const int64_t n = static_cast<int64_t>(s.b) * s.H * s.N * s.P;
    const Range rc_copy = rng(state_copy, n * (state_form == BDSSM_STATE_OPS ? 4 : 2));
    SeqRanges q{};
    (void)check_seq(clean, s, block_len, y != nullptr, &q);
    if (hits(rc_copy, q) || overlap(rc_copy, rng(h, n * 4)) || overlap(rc_copy, rng(A, s.H * 4)) ||
        overlap(rc_copy, rng(D, s.H * 4)) ||
        overlap(rc_copy, rng(y, static_cast<int64_t>(s.b) * block_len * s.H * s.P * elt(s.y_dt))))
        return BDSSM_ERR_ALIAS;
    if (s.b == 0)
        return BDSSM_OK;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const bool hi_only = state_form == BDSSM_STATE_BF16;
    if (block_len > 0 && !y && prefix_mfma_supported(s, 64)) {
        // one pass: the commit's state walk writes the advanced state and its encoded copy
        return launched(run_prefix_mfma(s, block_len, 64, Seq{clean->x, clean->dt, clean->B, clean->C}, A, D, h,
                                        nullptr, nullptr, h, nullptr, st, true, false, state_copy, hi_only));
    }
    if (block_len > 0 && (rc = launch_commit(s, block_len, Seq{clean->x, clean->dt, clean->B, clean->C}, A, D, h,
                                             y, st)) != BDSSM_OK)
        return rc;
    return launched(hi_only ? launch_state_bf16(h, state_copy, static_cast<int64_t>(s.b) * s.H, s.N, s.P, st)
                            : launch_state_ops(h, state_copy, static_cast<int64_t>(s.b) * s.H, st));
}

size_t bdssm_conv_workspace(const bdssm_dims *dims, int64_t len)
{
    Shape s;
    if (check_dims(dims, &s) != BDSSM_OK || len < 0)
        return SIZE_MAX;
    return conv_copy_bytes(s, len).total;
}

bdssm_status bdssm_conv(const bdssm_dims *dims, int64_t len, const bdssm_conv_params *conv,
                        int32_t reverse, const void *state_in, const bdssm_seq *raw,
                        const bdssm_seq *out, void *state_out, void *stream)
{
    Shape s;
    bdssm_status rc = check_dims(dims, &s);
    if (rc != BDSSM_OK)
        return rc;
    if (len < 0 || (reverse != 0 && reverse != 1))
        return BDSSM_ERR_SHAPE;
    if (reverse && (state_in || state_out))
        return BDSSM_ERR_SHAPE;
    ConvRanges cr{};
    if ((rc = check_conv(conv, s, &cr)) != BDSSM_OK)
        return rc;
    SeqRanges qr{}, qo{};
    if ((rc = check_xbc(raw, s, len, &qr)) != BDSSM_OK || (rc = check_xbc(out, s, len, &qo)) != BDSSM_OK)
        return rc;
    if (!aligned(state_in) || !aligned(state_out))
        return BDSSM_ERR_ALIGN;
    const int64_t sb = conv_state_bytes(s, conv->width);
    const Range rsi = rng(state_in, sb), rso = rng(state_out, sb);
    if (overlap(qo.x, qo.B) || overlap(qo.x, qo.C) || overlap(qo.B, qo.C))
        return BDSSM_ERR_ALIAS;
    for (Range o : {qo.x, qo.B, qo.C}) {
        if (hits(o, qr) || overlap(o, cr.w) || overlap(o, cr.b) || overlap(o, rsi) || overlap(o, rso))
            return BDSSM_ERR_ALIAS;
    }
    if (hits(rso, qr) || overlap(rso, cr.w) || overlap(rso, cr.b) || (overlap(rso, rsi) && state_out != state_in))
        return BDSSM_ERR_ALIAS;
    if (s.b == 0 || len == 0) {
        // no tokens: the history is unchanged
        if (state_out && state_out != state_in && sb > 0) {
            if (state_in)
                return launched(launch_copy_f32(static_cast<float *>(state_out),
                                                static_cast<const float *>(state_in), sb / 4,
                                                static_cast<hipStream_t>(stream)));
            return launched(launch_fill_f32(static_cast<float *>(state_out), 0.f, sb / 4,
                                            static_cast<hipStream_t>(stream)));
        }
        return BDSSM_OK;
    }
    ConvArgs a{};
    a.s = s;
    a.len = len;
    a.act = conv->activation;
    a.q[0] = ConvSeqArgs{raw->x, raw->B, raw->C, const_cast<void *>(out->x), const_cast<void *>(out->B),
                         const_cast<void *>(out->C), conv->weight, conv->bias, state_in, state_out, reverse};
    return launched(launch_conv(a, conv->width, 1, static_cast<hipStream_t>(stream)));
}

bdssm_status bdssm_block_step_conv(const bdssm_dims *dims, int32_t block_len,
                                   const bdssm_conv_params *conv_fwd,
                                   const bdssm_conv_params *conv_rev, const float *h_prefix,
                                   const void *conv_state, const bdssm_seq *fwd,
                                   const bdssm_seq *rev, const float *A, const float *D,
                                   const float *A_rev, const float *D_rev, void *y,
                                   void *workspace, size_t workspace_bytes, void *stream)
{
    Shape s;
    bdssm_status rc = check_dims(dims, &s);
    if (rc != BDSSM_OK)
        return rc;
    if (block_len < 0)
        return BDSSM_ERR_SHAPE;
    if (block_len > 256)
        return BDSSM_ERR_UNSUPPORTED;
    ConvRanges cf{}, cr{};
    if ((rc = check_conv(conv_fwd, s, &cf)) != BDSSM_OK || (rc = check_conv(conv_rev, s, &cr)) != BDSSM_OK)
        return rc;
    if (conv_fwd->width > 1 && !conv_state)
        return BDSSM_ERR_NULL;
    SeqRanges qf{}, qr{};
    if ((rc = check_seq(fwd, s, block_len, true, &qf)) != BDSSM_OK ||
        (rc = check_seq(rev, s, block_len, true, &qr)) != BDSSM_OK)
        return rc;
    if (!aligned(conv_state) || !aligned(workspace))
        return BDSSM_ERR_ALIGN;
    const ConvCopy cc = conv_copy_bytes(s, block_len);
    if (block_len > 0 && s.b > 0 && (!workspace || workspace_bytes < 2 * cc.total))
        return BDSSM_ERR_WORKSPACE;
    const Range rws = rng(workspace, static_cast<int64_t>(2 * cc.total));
    const Range rcs = rng(conv_state, conv_fwd->width > 1 ? conv_state_bytes(s, conv_fwd->width) : 0);
    if (hits(rws, qf) || hits(rws, qr) || overlap(rws, cf.w) || overlap(rws, cf.b) || overlap(rws, cr.w) ||
        overlap(rws, cr.b) || overlap(rws, rcs))
        return BDSSM_ERR_ALIAS;
    // the block step reads the convolved x, B, C from the workspace and the raw dt
    char *w0 = static_cast<char *>(workspace);
    char *w1 = w0 + cc.total;
    const bdssm_seq pf{w0, fwd->dt, w0 + cc.B, w0 + cc.C};
    const bdssm_seq pr{w1, rev->dt, w1 + cc.B, w1 + cc.C};
    BlockArgs a{};
    if ((rc = prepare_block_step(dims, block_len, h_prefix, &pf, &pr, A, D, A_rev ? A_rev : A, D_rev, y, &a)) !=
        BDSSM_OK)
        return rc;
    const Range ry = rng(y, static_cast<int64_t>(s.b) * block_len * s.H * s.P * elt(s.y_dt));
    if (hits(ry, qf) || hits(ry, qr) || overlap(ry, rws) || overlap(ry, rcs) || overlap(ry, cf.w) ||
        overlap(ry, cf.b) || overlap(ry, cr.w) || overlap(ry, cr.b))
        return BDSSM_ERR_ALIAS;
    if (s.b == 0 || block_len == 0)
        return BDSSM_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (conv_fwd->width == conv_rev->width && conv_fwd->activation == conv_rev->activation) {
        // both directions in one launch
        ConvArgs ca{};
        ca.s = s;
        ca.len = block_len;
        ca.act = conv_fwd->activation;
        ca.q[0] = ConvSeqArgs{fwd->x, fwd->B, fwd->C, w0, w0 + cc.B, w0 + cc.C, conv_fwd->weight,
                              conv_fwd->bias, conv_fwd->width > 1 ? conv_state : nullptr, nullptr, 0};
        ca.q[1] = ConvSeqArgs{rev->x, rev->B, rev->C, w1, w1 + cc.B, w1 + cc.C, conv_rev->weight,
                              conv_rev->bias, nullptr, nullptr, 1};
        if ((rc = launched(launch_conv(ca, conv_fwd->width, 2, st))) != BDSSM_OK)
            return rc;
    } else {
        for (int d = 0; d < 2; ++d) {
            const bdssm_conv_params *cp = d ? conv_rev : conv_fwd;
            const bdssm_seq *in = d ? rev : fwd;
            char *w = d ? w1 : w0;
            ConvArgs ca{};
            ca.s = s;
            ca.len = block_len;
            ca.act = cp->activation;
            ca.q[0] = ConvSeqArgs{in->x, in->B, in->C, w, w + cc.B, w + cc.C, cp->weight, cp->bias,
                                  (d == 0 && cp->width > 1) ? conv_state : nullptr, nullptr, d};
            if ((rc = launched(launch_conv(ca, cp->width, 1, st))) != BDSSM_OK)
                return rc;
        }
    }
    return launch_block_step(a, st);
}

bdssm_status bdssm_commit_conv(const bdssm_dims *dims, int32_t block_len,
                               const bdssm_conv_params *conv, const bdssm_seq *clean,
                               const float *A, const float *D, float *h, void *conv_state,
                               void *y, void *workspace, size_t workspace_bytes, void *stream)
{
    Shape s;
    bdssm_status rc = check_dims(dims, &s);
    if (rc != BDSSM_OK)
        return rc;
    if (block_len < 0)
        return BDSSM_ERR_SHAPE;
    if (block_len > 256)
        return BDSSM_ERR_UNSUPPORTED;
    ConvRanges cr{};
    if ((rc = check_conv(conv, s, &cr)) != BDSSM_OK)
        return rc;
    if (conv->width > 1 && !conv_state)
        return BDSSM_ERR_NULL;
    SeqRanges q{};
    if ((rc = check_seq(clean, s, block_len, true, &q)) != BDSSM_OK)
        return rc;
    if (!aligned(conv_state) || !aligned(workspace))
        return BDSSM_ERR_ALIGN;
    const ConvCopy cc = conv_copy_bytes(s, block_len);
    if (block_len > 0 && s.b > 0 && (!workspace || workspace_bytes < cc.total))
        return BDSSM_ERR_WORKSPACE;
    const Range rws = rng(workspace, static_cast<int64_t>(cc.total));
    const Range rcs = rng(conv_state, conv->width > 1 ? conv_state_bytes(s, conv->width) : 0);
    const Range rh = rng(h, static_cast<int64_t>(s.b) * s.H * s.N * s.P * 4);
    const Range ry = rng(y, static_cast<int64_t>(s.b) * block_len * s.H * s.P * elt(s.y_dt));
    for (Range o : {rws, rcs}) {
        if (hits(o, q) || overlap(o, cr.w) || overlap(o, cr.b) || overlap(o, rh) || overlap(o, ry) ||
            overlap(o, rng(A, s.H * 4)) || overlap(o, rng(D, s.H * 4)))
            return BDSSM_ERR_ALIAS;
    }
    if (overlap(rws, rcs))
        return BDSSM_ERR_ALIAS;
    char *w0 = static_cast<char *>(workspace);
    const bdssm_seq pc{w0, clean->dt, w0 + cc.B, w0 + cc.C};
    Shape s2;
    if ((rc = prepare_commit(dims, block_len, &pc, A, D, h, y, &s2)) != BDSSM_OK)
        return rc;
    if (hits(rh, q) || hits(ry, q))
        return BDSSM_ERR_ALIAS;
    if (s.b == 0 || block_len == 0)
        return BDSSM_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    ConvArgs ca{};
    ca.s = s;
    ca.len = block_len;
    ca.act = conv->activation;
    void *cs = conv->width > 1 ? conv_state : nullptr;
    ca.q[0] = ConvSeqArgs{clean->x, clean->B, clean->C, w0, w0 + cc.B, w0 + cc.C, conv->weight, conv->bias,
                          cs, cs, 0};
    if ((rc = launched(launch_conv(ca, conv->width, 1, st))) != BDSSM_OK)
        return rc;
    return launch_commit(s, block_len, Seq{pc.x, pc.dt, pc.B, pc.C}, A, D, h, y, st);
}

}  // extern "C"
