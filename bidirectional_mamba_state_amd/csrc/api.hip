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

// Tuning knobs for launch-shape sweeps: BDSSM_BLOCK_HPW (heads per workgroup, must divide
// the heads of a group) and BDSSM_BLOCK_PS (column splits: 1, 2 or 4). Invalid values are
// ignored.
void override_block_plan(const Shape &s, int *hpw, int *ps)
{
    if (const char *e = getenv("BDSSM_BLOCK_HPW")) {
        const int v = atoi(e);
        if (v >= 1 && (s.H / s.G) % v == 0)
            *hpw = v;
    }
    if (const char *e = getenv("BDSSM_BLOCK_PS")) {
        const int v = atoi(e);
        if (v == 1 || v == 2 || v == 4)
            *ps = v;
    }
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

    if (!with_y && !with_cs && p.nseg == 1) {
        // one pass per (stream, head), from h_init straight to h_out (in place is safe:
        // each workgroup reads its whole state before it writes any of it)
        ForwardArgs f{s, len, static_cast<int>(p.seg_len), 1, seq, A, D, h_init, nullptr,
                      nullptr, h_out, nullptr};
        return launched(launch_forward_valu(f, st));
    }

    float *decay = static_cast<float *>(workspace);
    float *states = with_cs ? chunk_states
                            : reinterpret_cast<float *>(static_cast<char *>(workspace) + p.decay_bytes);
    // 1. chunk-local states (from zero) and decay sums
    ForwardArgs f1{s, len, static_cast<int>(p.seg_len), p.nseg, seq, A, D, nullptr, nullptr,
                   nullptr, states, decay};
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
                   y, nullptr, nullptr};
    if ((rc = launched(launch_forward_valu(f3, st))) != BDSSM_OK)
        return rc;
    for (int b = 0; b < s.b; ++b) {
        rc = launched(launch_copy_f32(h_out + static_cast<int64_t>(b) * s.H * NP,
                                      states + (static_cast<int64_t>(b) * p.nseg + p.nseg - 1) * s.H * NP,
                                      s.H * NP, st));
        if (rc != BDSSM_OK)
            return rc;
    }
    return BDSSM_OK;
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
    const Range ry = rng(y, static_cast<int64_t>(s.b) * block_len * s.H * s.P * elt(s.y_dt));
    if (hits(ry, qf) || hits(ry, qr) || overlap(ry, rng(h_prefix, static_cast<int64_t>(s.b) * s.H * NP * 4)) ||
        overlap(ry, rng(A, s.H * 4)) || overlap(ry, rng(D, s.H * 4)) || overlap(ry, rng(A_rev, s.H * 4)) ||
        overlap(ry, rng(D_rev, s.H * 4)))
        return BDSSM_ERR_ALIAS;
    if (s.b == 0 || block_len == 0)
        return BDSSM_OK;
    BlockArgs a{s, block_len, h_prefix, Seq{fwd->x, fwd->dt, fwd->B, fwd->C},
                Seq{rev->x, rev->dt, rev->B, rev->C}, A, D, y, A_rev, D_rev};
    if (block_mfma_supported(s, block_len)) {
        int hpw, ps;
        block_mfma_plan(s, &hpw, &ps);
        override_block_plan(s, &hpw, &ps);
        return launched(launch_block_step_mfma(a, hpw, ps, static_cast<hipStream_t>(stream)));
    }
    return launched(launch_block_step_valu(a, static_cast<hipStream_t>(stream)));
}

bdssm_status bdssm_commit(const bdssm_dims *dims, int32_t block_len, const bdssm_seq *clean,
                          const float *A, const float *D, float *h, void *y, void *stream)
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
    if (s.b == 0 || block_len == 0)
        return BDSSM_OK;
    const Seq seq{clean->x, clean->dt, clean->B, clean->C};
    // a commit is a prefix scan of the block from h, in place: on the matrix-core prefix
    // path, one segment per (stream, head) (no workspace)
    if (prefix_mfma_supported(s, 64))
        return launched(run_prefix_mfma(s, block_len, 64, seq, A, D, h, y, nullptr, h, nullptr,
                                        static_cast<hipStream_t>(stream), true));
    ForwardArgs f{s, block_len, block_len, 1, seq, A, D, h, nullptr, y, h, nullptr};
    return launched(launch_forward_valu(f, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
