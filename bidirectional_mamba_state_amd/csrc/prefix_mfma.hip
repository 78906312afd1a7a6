// Prefix scan on bf16 matrix cores (gfx950 v_mfma_f32_16x16x32_bf16), d_state 128, headdim 64.
//
// The prefix operator of "Training Hybrid Block Diffusion Language Models with Partial
// Bidirectionality", eq. (10): the forward Mamba-2 recurrence of eq. (1) over the prefix,
// computed in the chunked matrix form. A workgroup owns HPW heads of one B/C group of one
// stream and a segment of consecutive 64-token sub-chunks, and walks them in order with
// the N x P states held in matrix-core accumulators: wavefront w owns columns 16w .. 16w+15
// of every head's state, so the state is at once the operand of C . h and the target of
// the state update, with no trip through LDS. For one sub-chunk with cumulative
// log-decays c_t (relative to its start):
//   state:   h <- exp(c_63) h + sum_s B_s [exp(c_63 - c_s) dt_s x_s]^T
//   output:  y_t = exp(c_t) C_t . h_in + sum_{s<=t} exp(c_t - c_s) dt_s (C_t . B_s) x_s + D x_t
// Outputs are computed transposed (y^T = h^T C^T + X^T M^T) so that a lane holds four
// consecutive columns of one token. The causal C B^T score tiles and their decay weights do
// not depend on the columns: the four wavefronts compute a share each and exchange the
// weighted tiles M through LDS.
// Operands whose contraction runs over tokens are read with the gfx950 transposing LDS load
// (ds_read_b64_tr_b16) from tiles laid out to keep those reads free of bank conflicts.
//
// Passes:
//   STATE  from h_init (or zero): only the state recurrence; writes the segment's end
//          state and its total log-decay (used by the segment scan, or as h_out).
//          k_fold*: the end state as a weighted sum of the segment's tokens, walked from
//          its last sub-chunk to its first, 1, 2 or 4 heads of a B/C group per workgroup.
//   FULL   from the state entering the segment: also y (k_full_*, inputs copied straight
//          into LDS), or only the chunk states (k_scan<1>): the state after every chunk of
//          Q tokens and after the last token, and, for the stream's last segment, the final
//          state.
// Reverse order (REV): k_fold and the full pass also scan a sequence from its last token
// to its first (token t of the scan is token len - 1 - t of the stream), reading the same
// layouts: row r of a sub-chunk holding scan positions t0 .. t0 + n - 1 is stream token
// (len - t0 - n) + (n - 1 - r). The full pass then adds its outputs to y instead of writing
// them (the reverse half of a full-window bidirectional scan, whose forward half wrote y).
// k_scan stages B and x through registers into the fragment-major order of mfma_tiles.h
// (an operand fragment is one contiguous 512-byte read per wavefront).
// The fp32 states and the weighted x~ operand are split into bf16 hi + lo parts, so that
// products against them keep ~16 significant bits; B, C and x are exact in bf16.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "internal.h"
#include "mfma_tiles.h"
#include "wave_ops.h"

namespace bdssm {
namespace {

typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef int v4i32 __attribute__((ext_vector_type(4)));

constexpr int kN = 128, kP = 64, SC = 64;  // d_state, headdim, sub-chunk length
constexpr float kLog2e = 1.4426950408889634f;

enum { TAB_C, TAB_EF, TAB_LG, TAB_COL, TAB_W, NTAB };

struct ScanArgs {
    Shape s;
    int64_t len;         // tokens per stream
    int seg_sub;         // sub-chunks per segment
    int nseg;            // segments per stream
    int chunk_sub;       // sub-chunks per output chunk (chunk / 64)
    int nch;             // output chunks per stream
    Seq in;
    const float *A, *D;
    const float *h_in;   // state entering each segment [b][nseg][H][N][P]; NULL = zero
    float *h_end;        // STATE: end state of each segment [b][nseg][H][N][P]
    float *h_last;       // FULL: final state [b][H][N][P] (written by the last segment), or NULL
    float *tot;          // STATE: natural-log decay of each segment [b][nseg][H], or NULL
    void *y;             // FULL: [b][len][H][P] in s.y_dt, or NULL
    float *chunk_states; // FULL: [b][nch][H][N][P], or NULL
    void *enc;           // STATE, single segment: the end state also encoded for the block
                         // step ([b][H][2][N/8][P][8] operand form, or [b][H][N/8][P][8] bf16),
                         // or NULL
    int enc_hi_only;     // enc holds only the hi parts (the bf16 state)
};

// A lane's four accumulator values, rows n0 .. n0+3 (n0 % 4 == 0) of column p of one head's
// state, encoded for the block step: hi = bf16(S) and lo = bf16(S - hi), both rounded to
// nearest even (the same parts the operand-form pass makes), each four contiguous elements
// of [N/8][P][8]; with hi_only just the hi parts.
__device__ __forceinline__ void store_encoded4(__bf16 *head, bool hi_only, int n0, int p, f32x4 v)
{
    bf16x4 hi, lo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        hi[j] = static_cast<__bf16>(v[j]);
        lo[j] = static_cast<__bf16>(v[j] - static_cast<float>(hi[j]));
    }
    const int o = ((n0 >> 3) * kP + p) * 8 + (n0 & 7);
    *reinterpret_cast<bf16x4 *>(head + o) = hi;
    if (!hi_only)
        *reinterpret_cast<bf16x4 *>(head + kN * kP + o) = lo;
}

template <int HPW>
struct Lds {
    __bf16 B[SC * kN];
    __bf16 X[HPW][SC * kP];
    float tab[2][HPW][NTAB][SC];  // decay tables of sub-chunks k and k+1 (by parity)
    float tot[2][HPW];
};


template <int HPW>
__global__ __launch_bounds__(256, 2) void k_scan(ScanArgs a)
{
    __shared__ __attribute__((aligned(16))) Lds<HPW> L;

    // workgroups of one segment (all heads of a stream) go to the same XCD
    const int nwg = gridDim.x;
    int lid = blockIdx.x;
    if ((nwg & 7) == 0)
        lid = (lid & 7) * (nwg >> 3) + (lid >> 3);
    const int H = a.s.H, G = a.s.G, NGRP = H / HPW;
    const int h0 = (lid % NGRP) * HPW;
    const int sg = (lid / NGRP) % a.nseg;
    const int b = lid / (NGRP * a.nseg);
    const int g = h0 / (H / G);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
    const int p0 = 16 * wave;  // this wavefront's state columns

    const int64_t len = a.len;
    const int64_t seg_t0 = static_cast<int64_t>(sg) * a.seg_sub * SC;
    const int nsub = static_cast<int>(min<int64_t>(a.seg_sub, (len - seg_t0 + SC - 1) / SC));
    const int64_t nsub_all = (len + SC - 1) / SC;
    const int rowBC = G * kN, rowX = H * kP;
    const int64_t tok0 = static_cast<int64_t>(b) * len;
    const __bf16 *Bg = static_cast<const __bf16 *>(a.in.B) + tok0 * rowBC + g * kN;
    const __bf16 *xg = static_cast<const __bf16 *>(a.in.x) + tok0 * rowX + h0 * kP;
    const __bf16 *dtg = static_cast<const __bf16 *>(a.in.dt) + tok0 * H + h0;
    const int64_t NP = static_cast<int64_t>(kN) * kP;
    const int th = min(wave, HPW - 1);  // head whose dt this wavefront stages
    const float Ath = a.A[h0 + th];

    // ---- states: hs[hh][i] holds h[16 i + 4 q + j][p0 + r16] of head h0 + hh
    f32x4 hs[HPW][8];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            hs[hh][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.h_in) {
            const float *hin = a.h_in + ((static_cast<int64_t>(b) * a.nseg + sg) * H + h0 + hh) * NP;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    hs[hh][i][j] = hin[(16 * i + 4 * q + j) * kP + p0 + r16];
        }
    }
    auto store_state = [&](float *base) {  // base: [HPW heads][N][P] with head stride NP
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    base[hh * NP + (16 * i + 4 * q + j) * kP + p0 + r16] = hs[hh][i][j];
    };

    // ---- staging registers, one sub-chunk ahead
    constexpr int BPT = SC * kN / 8 / 256;        // uint4 per thread for B (and C): 4
    constexpr int XPT = SC * kP * HPW / 8 / 256;  // uint4 per thread for x: 2 HPW
    struct Stage {
        uint4 bq[BPT];
        uint4 xq[XPT];
        __bf16 dt;  // dt of sub-chunk k+2, token `lane`, head h0 + min(wave, HPW-1)
    } st;
    // rows past the end are clamped here and zeroed at store time
    auto load_b = [&](int k) {
        const int64_t t0 = seg_t0 + static_cast<int64_t>(k) * SC;
        const int last = static_cast<int>(min<int64_t>(SC, len - t0)) - 1;
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            const int it = tid + 256 * u, row = min(16 * (it >> 8) + (it & 15), last), c16 = (it >> 4) & 15;
            st.bq[u] = *reinterpret_cast<const uint4 *>(Bg + (t0 + row) * rowBC + c16 * 8);
        }
    };
    auto load_x = [&](int k) {
        const int64_t t0 = seg_t0 + static_cast<int64_t>(k) * SC;
        const int last = static_cast<int>(min<int64_t>(SC, len - t0)) - 1;
#pragma unroll
        for (int u = 0; u < XPT; ++u) {
            const int it = tid + 256 * u, c = (it >> 4) % (8 * HPW);
            const int row = min(16 * ((it >> 4) / (8 * HPW)) + (it & 15), last);
            st.xq[u] = *reinterpret_cast<const uint4 *>(xg + (t0 + row) * rowX + c * 8);
        }
    };
    auto load_stage = [&](int k) {
        load_b(k);
        load_x(k);
    };
    // dt two sub-chunks ahead of the stage (clamped to the segment's last sub-chunk)
    auto load_dt = [&](int k) {
        const int64_t t0 = seg_t0 + static_cast<int64_t>(k) * SC;
        const int last = static_cast<int>(min<int64_t>(SC, len - t0)) - 1;
        st.dt = dtg[(t0 + min(lane, last)) * H + th];
    };
    auto store_stage = [&](int k) {
        const int64_t t0 = seg_t0 + static_cast<int64_t>(k) * SC;
        const int nvalid = static_cast<int>(min<int64_t>(SC, len - t0));
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            const int it = tid + 256 * u, row = 16 * (it >> 8) + (it & 15), c16 = (it >> 4) & 15;
            put16<kN>(L.B, row, c16 * 8, sel4(row < nvalid, st.bq[u]));
        }
#pragma unroll
        for (int u = 0; u < XPT; ++u) {
            const int it = tid + 256 * u, c = (it >> 4) % (8 * HPW);
            const int row = 16 * ((it >> 4) / (8 * HPW)) + (it & 15);
            put16<kP>(L.X[c >> 3], row, (c & 7) * 8, sel4(row < nvalid, st.xq[u]));
        }
    };
    // the state update's weights of sub-chunk k for head h0 + wave (wavefronts below HPW),
    // one token per lane, from the dt in st.dt; into table buffer k % 2
    auto tables = [&](int k) {
        if (wave < HPW) {
            const int64_t t0 = seg_t0 + static_cast<int64_t>(k) * SC;
            const int nvalid = static_cast<int>(min<int64_t>(SC, len - t0));
            const float d = lane < nvalid ? bf2f(st.dt) : 0.f;
            const float inc = wave_prefix_sum(d * Ath);
            const float c = inc * kLog2e;
            const float clast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 63));
            L.tab[k & 1][wave][TAB_W][lane] = __builtin_amdgcn_exp2f(clast - c) * d;
            if (lane == 63)
                L.tot[k & 1][wave] = inc;
        }
    };

    float seg_tot[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
        seg_tot[hh] = 0.f;
    // a chunk state is the state after a chunk's last sub-chunk, and after the stream's last;
    // kend: the segment's next chunk end (segment-local sub-chunk), cnext: that chunk
    const int64_t gsub0 = seg_t0 / SC;
    const int kstream_end = gsub0 + nsub == nsub_all ? nsub - 1 : -1;
    int kend = static_cast<int>(a.chunk_sub - 1 - gsub0 % a.chunk_sub);
    int64_t cnext = gsub0 / a.chunk_sub;
    auto emit_chunk_state = [&](int k) {  // after sub-chunk k, for k = 0, 1, .. in turn
        if (k == kend || k == kstream_end)
            store_state(a.chunk_states + ((static_cast<int64_t>(b) * a.nch + cnext) * H + h0) * NP);
        if (k == kend) {
            kend += a.chunk_sub;
            ++cnext;
        }
    };
    load_stage(0);
    load_dt(0);
    __bf16 dt1;  // dt of sub-chunk 1, loaded with the first stage
    {
        const int64_t t1 = seg_t0 + SC * static_cast<int64_t>(min(1, nsub - 1));
        dt1 = dtg[(t1 + min<int64_t>(lane, len - t1 - 1)) * H + th];
    }
    store_stage(0);
    tables(0);
    st.dt = dt1;
    if (nsub > 1)
        tables(1);
    for (int k = 0; k < nsub; ++k) {
        __syncthreads();  // (A) sub-chunk k staged, its tables written
        if (a.chunk_states && k > 0)
            emit_chunk_state(k - 1);
        // the loads of sub-chunk k+1, in flight during sub-chunk k
        const int kn = min(k + 1, nsub - 1);
        load_stage(kn);
        load_dt(min(k + 2, nsub - 1));
        __builtin_amdgcn_sched_barrier(0);  // keep the loads here, ahead of the compute

        // x~ fragments (contraction over tokens, columns p0 .. p0+15), per head and 32-token pair
        bf16x8 xf[HPW][2];
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
            for (int m = 0; m < 2; ++m)
                xf[hh][m] = tr_frag<kP>(L.X[hh], 32 * m, p0, q, r16);

        // ---- state: h <- exp(c_63) h + B^T (w o x), w_s = exp(c_63 - c_s) dt_s
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            const float tot = L.tot[k & 1][hh];
            seg_tot[hh] += tot;
            const float alpha = __expf(tot);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                hs[hh][i] *= alpha;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 bt[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                bt[i] = tr_frag<kN>(L.B, 32 * ks, 16 * i, q, r16);
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                const float4 w0 = *reinterpret_cast<const float4 *>(&L.tab[k & 1][hh][TAB_W][32 * ks + 4 * q]);
                const float4 w1 = *reinterpret_cast<const float4 *>(&L.tab[k & 1][hh][TAB_W][32 * ks + 16 + 4 * q]);
                const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
                float xw[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    xw[e] = bf2f(xf[hh][ks][e]) * wv[e];
                bf16x8 xhi, xlo;
                split8(xw, xhi, xlo);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    hs[hh][i] = mfma(bt[i], xhi, hs[hh][i]);
                    hs[hh][i] = mfma(bt[i], xlo, hs[hh][i]);
                }
            }
        }
        __syncthreads();  // (B) every LDS read for sub-chunk k is done
        // unconditional, so that no path reaches the loop head with loads in flight (after
        // the last sub-chunk it stages data nobody reads)
        store_stage(k + 1);
        // tables of sub-chunk k+2 (its dt was loaded with the stage of k+1, whose wait just
        // passed; at the top of the loop the wait would cover the y stores as well) into the
        // buffer sub-chunk k has finished with; visible after the next barrier (A)
        if (k + 2 < nsub)
            tables(k + 2);
    }
    if (a.chunk_states)
        emit_chunk_state(nsub - 1);

    // ---- end of the segment
    if (a.h_last && sg == a.nseg - 1)
        store_state(a.h_last + (static_cast<int64_t>(b) * H + h0) * NP);
}

// Token mapping of the reverse order: the stream token held by the first memory row of the
// sub-chunk at scan position t0 with nrows valid rows, and the memory row of its scan row
// `row` (rows past the valid ones map past any buffer range). Identities in natural order.
template <bool REV>
__device__ __forceinline__ int64_t first_token(int64_t len, int64_t t0, int nrows)
{
    if constexpr (REV)
        return max<int64_t>(len - t0 - nrows, 0);
    else
        return t0;
}
template <bool REV>
__device__ __forceinline__ int mem_row(int row, int nrows)
{
    if constexpr (REV)
        return row < nrows ? nrows - 1 - row : SC;
    else
        return row;
}

// Segment scan, one thread per four consecutive state elements (16-byte accesses): the end
// states of segments started from zero become the states entering each segment (in place),
// and the final state.
__global__ __launch_bounds__(256) void k_seg_scan(float *buf, const float *tot, int nseg, int H,
                                                  const float *h_init, float *h_out)
{
    const int64_t NP = static_cast<int64_t>(kN) * kP;
    const int64_t e = 4 * (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);
    const int h = blockIdx.y, b = blockIdx.z;
    if (e >= NP)
        return;
    float4 v = h_init ? *reinterpret_cast<const float4 *>(h_init + (static_cast<int64_t>(b) * H + h) * NP + e)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
    // U segments at a time: their loads are issued together, then the recurrence runs
    constexpr int U = 16;
    for (int s0 = 0; s0 < nseg; s0 += U) {
        float4 loc[U];
        float dec[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {  // (past the last segment: the last one, unused)
            const int64_t bh = (static_cast<int64_t>(b) * nseg + min(s0 + u, nseg - 1)) * H + h;
            loc[u] = *reinterpret_cast<const float4 *>(buf + bh * NP + e);
            dec[u] = __expf(tot[bh]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s0 + u < nseg) {
                const int64_t bh = (static_cast<int64_t>(b) * nseg + s0 + u) * H + h;
                *reinterpret_cast<float4 *>(buf + bh * NP + e) = v;
                v.x = fmaf(dec[u], v.x, loc[u].x);
                v.y = fmaf(dec[u], v.y, loc[u].y);
                v.z = fmaf(dec[u], v.z, loc[u].z);
                v.w = fmaf(dec[u], v.w, loc[u].w);
            }
        }
    }
    if (h_out)
        *reinterpret_cast<float4 *>(h_out + (static_cast<int64_t>(b) * H + h) * NP + e) = v;
}


// ---- State-only pass as a weighted sum (segment end states, state-only scans, commits)
//
// The end state of a segment is a weighted sum over its tokens,
//   h_end = exp(R) h_in + sum_t exp(sum_{u > t} a_u) dt_t B_t x_t^T,   a_u = dt_u A, R = sum_u a_u,
// so the segment can be walked from its last sub-chunk to its first with R, the log-decay of
// everything after the current sub-chunk, carried as one number per head: a token's weight is
// then exp2(R + c_63 - c_t) dt_t (c the sub-chunk's inclusive cumulative log2-decay) and the
// state accumulators are never rescaled. Weights of tokens far from the end underflow to zero,
// as their true weights do. Rounding differs from the forward walk of the full pass (sums in
// another order, weights relative to the segment's end).
//
// A workgroup owns HPW heads of one B/C group, in 4 HS wavefronts: wavefront w holds columns
// 16 (w % 4) .. +15 of the HPW / HS heads hb = (w / 4) HPW / HS .. (all 128 rows), so the B^T
// operand it reads serves all its heads and the staged B the whole workgroup. B and the heads'
// x are copied into LDS by buffer loads to LDS in whole lines, NBUF - 1 sub-chunks ahead into
// NBUF buffers. What keeps the matrix cores busy:
//  - no wait for copies in flight: the compiler makes an LDS read wait for the copies it
//    cannot tell apart from it, so each buffer is its own LDS array, the loop is unrolled by
//    NBUF (buffer choice known at compile time) with no branch on the copies' path, and every
//    read address is one step from its array (offsets precomputed, opaque to the optimizer)
//    so that the read keeps its attribution to that array;
//  - the copies of a step are spread over its products: a copy issued while the memory queue
//    is full stalls its wavefront, and with it the wavefront's share of the matrix core;
//  - two wavefronts per SIMD (HS = 2 for 2 and 4 heads), operands read per contraction block;
//  - the token weights of step j + 1 are computed at the end of step j by one wavefront per
//    head and published by the barrier, outside the step's critical path;
//  - tile layouts free of LDS bank conflicts for 32-lane transposing reads (swz_b, swz_x).

// f(integral_constant<int, 0>), .. f(integral_constant<int, N - 1>), in order
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// v unchanged, but opaque to the optimizer (an empty asm statement that may change it)
__device__ __forceinline__ int opaque_int(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// Piece permutation of the fold pass's B tiles: a transposing read of 32 lanes covers 8
// consecutive rows x 32 bytes, and the 16-byte piece c of row t sits at slot c ^ swz_b(t) so
// that those 256 bytes fall in distinct banks (B rows are 256 bytes, one bank period: 8
// distinct piece pairs). x tiles use swz_x.
__device__ __forceinline__ int swz_b(int t) { return 2 * (t & 7); }

template <int HPW, int HS, int NBUF, bool REV>
__device__ __forceinline__ void fold_pass(const ScanArgs &a)
{
    static_assert(NBUF == 3 || NBUF == 4, "three or four staging buffers");
    static_assert(HPW % HS == 0, "heads split evenly over the wavefront groups");
    constexpr int WPG = 4 * HS, HW = HPW / HS;  // wavefronts per workgroup, heads per wavefront
    constexpr int B3 = NBUF > 3 ? SC * kN : 8, X3 = NBUF > 3 ? SC * kP : 8;  // (a stub when unused)
    __shared__ __attribute__((aligned(16))) __bf16 sB0[SC * kN];
    __shared__ __attribute__((aligned(16))) __bf16 sB1[SC * kN];
    __shared__ __attribute__((aligned(16))) __bf16 sB2[SC * kN];
    __shared__ __attribute__((aligned(16))) __bf16 sB3[B3];
    __shared__ __attribute__((aligned(16))) __bf16 sX0[HPW][SC * kP];
    __shared__ __attribute__((aligned(16))) __bf16 sX1[HPW][SC * kP];
    __shared__ __attribute__((aligned(16))) __bf16 sX2[HPW][SC * kP];
    __shared__ __attribute__((aligned(16))) __bf16 sX3[HPW][X3];
    // token weights of walk steps j (by j % 2), per head: written by wavefront hh of head hh
    // at the end of the step before, read by every wavefront of the head after the barrier
    __shared__ __attribute__((aligned(16))) float sW[2][HPW][SC];
    __shared__ float sR[HPW];  // each head's log2-decay over the segment
    auto bufB = [&](auto ph) -> __bf16 * {
        if constexpr (decltype(ph)::value == 0)
            return sB0;
        else if constexpr (decltype(ph)::value == 1)
            return sB1;
        else if constexpr (decltype(ph)::value == 2)
            return sB2;
        else
            return sB3;
    };
    auto bufX = [&](auto ph) -> __bf16 * {  // the HPW heads' tiles, one after the other
        if constexpr (decltype(ph)::value == 0)
            return &sX0[0][0];
        else if constexpr (decltype(ph)::value == 1)
            return &sX1[0][0];
        else if constexpr (decltype(ph)::value == 2)
            return &sX2[0][0];
        else
            return &sX3[0][0];
    };

    // workgroups of one segment (all head groups of a stream) go to the same XCD
    const int nwg = gridDim.x;
    int lid = blockIdx.x;
    if ((nwg & 7) == 0)
        lid = (lid & 7) * (nwg >> 3) + (lid >> 3);
    const int H = a.s.H, G = a.s.G, NGRP = H / HPW;
    const int h0 = (lid % NGRP) * HPW;
    const int sg = (lid / NGRP) % a.nseg;
    const int b = lid / (NGRP * a.nseg);
    const int g = h0 / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p0 = 16 * (wave & 3);  // this wavefront's state columns
    const int hb = (wave >> 2) * HW;  // and its first head (of h0 + hb .. h0 + hb + HW - 1)

    const int64_t len = a.len;
    const int64_t seg_t0 = static_cast<int64_t>(sg) * a.seg_sub * SC;
    const int nsub = static_cast<int>(min<int64_t>(a.seg_sub, (len - seg_t0 + SC - 1) / SC));
    const int rowBC = G * kN, rowX = H * kP;
    const int64_t tok0 = static_cast<int64_t>(b) * len;
    const int64_t NP = static_cast<int64_t>(kN) * kP;
    const __bf16 *Bg = static_cast<const __bf16 *>(a.in.B) + tok0 * rowBC + g * kN;
    const __bf16 *xg = static_cast<const __bf16 *>(a.in.x) + tok0 * rowX + h0 * kP;
    const __bf16 *dtg = static_cast<const __bf16 *>(a.in.dt) + tok0 * H + h0;
    // range-checked buffer over [base, base + bytes), both the same in every lane: built from
    // lane 0's values, so that the descriptor is known to be uniform and stays in scalar
    // registers
    auto mk = [](const void *base, int bytes) {
        const uint64_t p = reinterpret_cast<uint64_t>(base);
        const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
        const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
        return buffer_range(reinterpret_cast<const void *>((static_cast<uint64_t>(hi) << 32) | lo),
                            __builtin_amdgcn_readfirstlane(bytes));
    };
    // wavefront w < HPW computes the token weights of head h0 + w; every wavefront loads the
    // dt of head h0 + w % HPW (the same number of loads in every wavefront keeps the waits
    // of the barriers exact)
    const int hd = wave % HPW;
    const float Aw = a.A[h0 + hd] * kLog2e;  // A in log2 units

    // walk step j handles the segment's sub-chunk nsub - 1 - j; a step past the segment
    // (issued ahead, never used) gets empty ranges, so its copies and dt loads read nothing
    auto sub_of = [&](int j) { return max(nsub - 1 - j, 0); };
    // copies of walk step j into buffer PH: B in 16 pieces of 1 KB (4 rows), x in 8 per head
    // (8 rows); wavefront w takes pieces w, w + WPG, ... of the 16 + 8 HPW
    constexpr int NPIECE = 16 + 8 * HPW, NPW = NPIECE / WPG;
    static_assert(NPIECE % WPG == 0 && 16 % WPG == 0, "pieces split evenly");
    struct Ranges {
        __amdgpu_buffer_rsrc_t rB, rX;
        int nrows;
    };
    auto ranges = [&](int j) {
        const int64_t t0 = seg_t0 + static_cast<int64_t>(sub_of(j)) * SC;
        const int nrows = static_cast<int>(min<int64_t>(SC, len - t0));
        const int64_t f0 = first_token<REV>(len, t0, nrows);
        const bool live = j < nsub;
        return Ranges{mk(Bg + f0 * rowBC, live ? ((nrows - 1) * rowBC + kN) * 2 : 0),
                      mk(xg + f0 * rowX, live ? ((nrows - 1) * rowX + HPW * kP) * 2 : 0), nrows};
    };
    // this wavefront's pieces U0 .. U1 - 1 of walk step j's copies (ranges from ranges(j))
    auto copy_part = [&](auto PH, auto U0, auto U1, const Ranges &g) {
        const auto rB = g.rB;
        const auto rX = g.rX;
        const int nrows = g.nrows;
#pragma unroll
        for (int u = decltype(U0)::value; u < decltype(U1)::value; ++u) {
            const int pc = wave + WPG * u;  // a B piece exactly when u < 16 / WPG
            if (u < 16 / WPG) {
                const int row = 4 * pc + (lane >> 4), c = (lane & 15) ^ swz_b(row);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rB, (__attribute__((address_space(3))) void *)(bufB(PH) + 4 * pc * kN), 16,
                    (mem_row<REV>(row, nrows) * rowBC + 8 * c) * 2, 0, 0, 0);
            } else {
                const int px = pc - 16, hh = px >> 3, row = 8 * (px & 7) + (lane >> 3);
                const int c = (lane & 7) ^ swz_x(row);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rX, (__attribute__((address_space(3))) void *)(bufX(PH) + hh * SC * kP + 8 * (px & 7) * kP), 16,
                    (mem_row<REV>(row, nrows) * rowX + hh * kP + 8 * c) * 2, 0, 0, 0);
            }
        }
    };
    auto copy = [&](auto PH, int j) {
        copy_part(PH, std::integral_constant<int, 0>{}, std::integral_constant<int, NPW>{}, ranges(j));
    };
    auto clear = [&](auto PH) {  // this wavefront's pieces of buffer PH
        const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
            const int pc = wave + WPG * u;
            if (u < 16 / WPG) {
                *reinterpret_cast<uint4 *>(bufB(PH) + 4 * pc * kN + 8 * lane) = z;
            } else {
                const int px = pc - 16;
                *reinterpret_cast<uint4 *>(bufX(PH) + (px >> 3) * SC * kP + 8 * (px & 7) * kP + 8 * lane) = z;
            }
        }
    };
    // dt of walk step j, token `lane`, head h0 + hd (zero past the stream's end)
    auto load_dt = [&](int j, unsigned short &d) {
        const int64_t t0 = seg_t0 + static_cast<int64_t>(sub_of(j)) * SC;
        const int nrows = static_cast<int>(min<int64_t>(SC, len - t0));
        const auto rD = mk(dtg + first_token<REV>(len, t0, nrows) * H, j < nsub ? ((nrows - 1) * H + HPW) * 2 : 0);
        d = __builtin_amdgcn_raw_buffer_load_b16(rD, (mem_row<REV>(lane, nrows) * H + hd) * 2, 0, 0);
    };

    f32x4 acc[HW][8];  // acc[hh][i] holds h[16 i + 4 q + e][p0 + r16] of head h0 + hb + hh
#pragma unroll
    for (int hh = 0; hh < HW; ++hh)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[hh][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float R = 0.f;  // head h0 + hd: log2-decay of the tokens after the weighted sub-chunks
    // weights of walk step j into sW[j % 2][hd] (wavefronts w < HPW): exp2(R + c_63 - c_t) dt_t,
    // lane t
    auto weights = [&](int j, unsigned short dbits) {
        if (wave < HPW) {
            const float d = __uint_as_float(static_cast<uint32_t>(dbits) << 16);
            const float c = wave_prefix_sum(d * Aw);
            const float clast = wave_lane(c, 63);
            sW[j & 1][hd][lane] = __builtin_amdgcn_exp2f(R + (clast - c)) * d;
            R += clast;
        }
    };

    // element offsets of this lane's transposing reads in a buffer, for contraction block ks
    // (tokens 32 ks + 4 q + e and, 16 rows on, 32 ks + 16 + 4 q + e): B^T rows 16 i + r16 and
    // x columns p0 + r16. Each is made opaque to the optimizer once, here: a read's address is
    // then one step from its LDS array, which keeps the compiler's attribution of the read to
    // that array (needed to tell it from the copies in flight) within its search depth.
    int offB[2][8], offX[2][HW];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int tr = 32 * ks + 4 * q + (r16 >> 2);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int col = 16 * i + 4 * (r16 & 3);
            offB[ks][i] = opaque_int(tr * kN + 8 * ((col >> 3) ^ swz_b(tr)) + (col & 7));
        }
        const int col = p0 + 4 * (r16 & 3);
#pragma unroll
        for (int hh = 0; hh < HW; ++hh)
            offX[ks][hh] = opaque_int((hb + hh) * SC * kP + tr * kP + 8 * ((col >> 3) ^ swz_x(tr)) + (col & 7));
    }

    // dt of walk steps j .. j + NBUF - 2, by j % NBUF
    unsigned short dts[NBUF];
    // one walk step j, in buffer PH = j % NBUF, with its dt in dts[PH] (loaded NBUF - 1 steps
    // before); loads the dt of step j + NBUF - 1 into the slot the previous step has left
    auto step = [&](auto PH, int j) {
        constexpr int ph = decltype(PH)::value, phn = (ph + NBUF - 1) % NBUF;
        constexpr int phw = (ph + 1) % NBUF;  // the dt slot of step j + 1
        unsigned short &dn = dts[phn];
        // this wavefront's copies of j have landed once at most those issued after them are in
        // flight: the dt and copies of j + 1 .. j + NBUF - 2; the weights of j are in sW
        workgroup_lds_barrier<(NBUF - 2) * (1 + NPW)>();
        // then walk step j + NBUF - 1 into the buffer j - 1 has left, its dt first, the copies
        // spread over the products below (a copy issued while the memory queue is full stalls
        // the wavefront, and with it its matrix core)
        load_dt(j + NBUF - 1, dn);
        const Ranges g = ranges(j + NBUF - 1);
        constexpr int NG = 2 * HW;  // product groups (ks, hh)
        static_for<2>([&](auto KS) {
            constexpr int ks = decltype(KS)::value;
            // the operands of contraction block ks (tokens 32 ks + 4 q + e and 32 ks + 16 + 4 q
            // + e): B^T (rows 16 i + r16) and x (columns p0 + r16) by transposing reads, and the
            // tokens' weights (a read may follow copies already issued: its address is known to
            // lie in another LDS array)
            bf16x8 bt[8], xf[HW];
            float wv[HW][8];
#pragma unroll
            for (int hh = 0; hh < HW; ++hh) {
                const float4 w0 = *reinterpret_cast<const float4 *>(&sW[j & 1][hb + hh][32 * ks + 4 * q]);
                const float4 w1 = *reinterpret_cast<const float4 *>(&sW[j & 1][hb + hh][32 * ks + 16 + 4 * q]);
                wv[hh][0] = w0.x, wv[hh][1] = w0.y, wv[hh][2] = w0.z, wv[hh][3] = w0.w;
                wv[hh][4] = w1.x, wv[hh][5] = w1.y, wv[hh][6] = w1.z, wv[hh][7] = w1.w;
                const __bf16 *px = bufX(PH) + offX[ks][hh];
                xf[hh] = cat(tr_read(px), tr_read(px + 16 * kP));
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const __bf16 *p = bufB(PH) + offB[ks][i];
                bt[i] = cat(tr_read(p), tr_read(p + 16 * kN));
            }
            __builtin_amdgcn_sched_barrier(0);
            // h += B^T x~ with x~ = w o x split into bf16 hi + lo
            static_for<HW>([&](auto HH) {
                constexpr int hh = decltype(HH)::value, gi = ks * HW + hh;
                copy_part(std::integral_constant<int, phn>{}, std::integral_constant<int, gi * NPW / NG>{},
                          std::integral_constant<int, (gi + 1) * NPW / NG>{}, g);
                __builtin_amdgcn_sched_barrier(0);
                float xw[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    xw[e] = bf2f(xf[hh][e]) * wv[hh][e];
                bf16x8 xhi, xlo;
                split8(xw, xhi, xlo);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    acc[hh][i] = mfma(bt[i], xhi, acc[hh][i]);
                    acc[hh][i] = mfma(bt[i], xlo, acc[hh][i]);
                }
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        // the weights of step j + 1 (its dt was loaded NBUF - 1 steps before it)
        weights(j + 1, dts[phw]);
    };

    // ---- prologue: clear the staging buffers (rows past the stream's end must hold finite
    // values: they are weighted 0), put walk steps 0 .. NBUF - 2 in flight, let them land
    clear(std::integral_constant<int, 0>{});
    clear(std::integral_constant<int, 1>{});
    clear(std::integral_constant<int, 2>{});
    if constexpr (NBUF > 3)
        clear(std::integral_constant<int, 3>{});
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the clears precede the copies
    load_dt(0, dts[0]);
    copy(std::integral_constant<int, 0>{}, 0);
    load_dt(1, dts[1]);
    copy(std::integral_constant<int, 1>{}, 1);
    if constexpr (NBUF > 3) {
        load_dt(2, dts[2]);
        copy(std::integral_constant<int, 2>{}, 2);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    weights(0, dts[0]);
    int j = 0;
    for (; j + NBUF <= nsub; j += NBUF) {  // whole groups: a body with no branch
        step(std::integral_constant<int, 0>{}, j);
        step(std::integral_constant<int, 1>{}, j + 1);
        step(std::integral_constant<int, 2>{}, j + 2);
        if constexpr (NBUF > 3)
            step(std::integral_constant<int, 3>{}, j + 3);
    }
    if (j < nsub)
        step(std::integral_constant<int, 0>{}, j);
    if (j + 1 < nsub)
        step(std::integral_constant<int, 1>{}, j + 1);
    if constexpr (NBUF > 3)
        if (j + 2 < nsub)
            step(std::integral_constant<int, 2>{}, j + 2);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no copy outlives the workgroup

    // ---- the segment's entering state, decayed over the whole segment (R of a head has then
    // also taken the weights of the step past the segment, whose dt are zero)
    if (wave < HPW && lane == 0)
        sR[hd] = R;
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
        const float Rh = sR[hb + hh];
        const float decay = __builtin_amdgcn_exp2f(Rh);
        const int64_t hofs = ((static_cast<int64_t>(b) * a.nseg + sg) * H + h0 + hb + hh) * NP;
        if (a.h_in) {
            const float *hin = a.h_in + hofs;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[hh][i][e] = fmaf(decay, hin[(16 * i + 4 * q + e) * kP + p0 + r16], acc[hh][i][e]);
        }
        if (a.h_end) {
            float *base = a.h_end + hofs;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    base[(16 * i + 4 * q + e) * kP + p0 + r16] = acc[hh][i][e];
        }
        if (a.enc) {  // single segment: the end state is the stream's new state
            const int64_t per = a.enc_hi_only ? NP : 2 * NP;
            __bf16 *head = static_cast<__bf16 *>(a.enc) + (static_cast<int64_t>(b) * H + h0 + hb + hh) * per;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                store_encoded4(head, a.enc_hi_only, 16 * i + 4 * q, p0 + r16, acc[hh][i]);
        }
        if (a.tot && (wave & 3) == 0 && lane == 0)
            a.tot[(static_cast<int64_t>(b) * a.nseg + sg) * H + h0 + hb + hh] = Rh / kLog2e;
    }
}

__global__ __launch_bounds__(256, 2) void k_fold1(ScanArgs a) { fold_pass<1, 1, 3, false>(a); }
__global__ __launch_bounds__(512, 1) void k_fold2(ScanArgs a) { fold_pass<2, 2, 4, false>(a); }
__global__ __launch_bounds__(512, 1) void k_fold4(ScanArgs a) { fold_pass<4, 2, 3, false>(a); }
__global__ __launch_bounds__(256, 2) void k_fold1_rev(ScanArgs a) { fold_pass<1, 1, 3, true>(a); }
__global__ __launch_bounds__(512, 1) void k_fold2_rev(ScanArgs a) { fold_pass<2, 2, 4, true>(a); }
__global__ __launch_bounds__(512, 1) void k_fold4_rev(ScanArgs a) { fold_pass<4, 2, 3, true>(a); }

// ---- FULL pass with outputs, one head per workgroup, inputs copied straight into LDS
//
// The same computation as k_scan<1> with y, with B, C and x copied into LDS by buffer loads
// to LDS in whole lines instead of
// through registers: B and x of sub-chunk k+1 are copied at the start of sub-chunk k into
// the other of two buffers; C, read only before the mid-sub-chunk barrier, has one buffer
// and its next copy is issued right after that barrier. 71.5 KB of LDS: two workgroups per
// CU. B and C rows (256 bytes) hold piece c of row r at slot c ^ swz(r), which keeps three
// read patterns free of bank conflicts: 16-byte operand reads of 16 consecutive rows (score
// tiles), transposing reads of 8 rows x 16 columns per 32 lanes (B in the state update) and
// 8-byte reads of the permuted contraction order (C in the state product); x rows hold
// piece c of row t at slot c ^ swz_x(t) (conflict-free for the transposing reads and the
// output's skip-term reads).
__device__ __forceinline__ int swz(int r)
{
    return ((r & 3) << 2) | ((r & 4) >> 1) | ((r >> 3) & 1);
}

// B and C tiles of the full pass: rows of 256 bytes (pieces permuted by swz) in blocks of 16
// rows, each block followed by 16 bytes of padding. The padding keeps a block's rows in the
// same banks but puts reads of two blocks at a distance no paired read (ds_read2) can encode:
// a pair of the 8-byte fragment reads below, merged into one instruction, conflicts, while
// each alone does not.
constexpr int BC_PAD = 8;  // elements
constexpr int BC_TILE = SC * kN + (SC / 16) * BC_PAD;
__device__ __forceinline__ int bc_row(int row) { return row * kN + (row >> 4) * BC_PAD; }

// The 10 score tiles of a sub-chunk (a causal 4 x 4 grid of 16 x 16 blocks): tile tau is row
// block tile_tb(tau), column block tile_sb(tau) <= tile_tb(tau) (tau = tb (tb + 1) / 2 + sb)
__host__ __device__ constexpr int tile_tb(int tau) { return tau >= 6 ? 3 : tau >= 3 ? 2 : tau >= 1 ? 1 : 0; }
__host__ __device__ constexpr int tile_sb(int tau) { return tau - tile_tb(tau) * (tile_tb(tau) + 1) / 2; }
// whether one of tiles w, w + 4, .. (nt of them) lies in row block tb
__host__ __device__ constexpr bool tile_row_of(int w, int nt, int tb)
{
    return tile_tb(w) == tb || (nt > 1 && tile_tb(w + 4) == tb) || (nt > 2 && tile_tb(w + 8) == tb);
}


// (the body is a device function template with one kernel per output type: a kernel
// template built from generic lambdas loses its host-side launch stub in this compiler)
template <typename Ty, bool REV>
__device__ __forceinline__ void full_pass(const ScanArgs &a)
{
    __shared__ __attribute__((aligned(16))) __bf16 sB0[BC_TILE];
    __shared__ __attribute__((aligned(16))) __bf16 sB1[BC_TILE];
    __shared__ __attribute__((aligned(16))) __bf16 sC[BC_TILE];
    __shared__ __attribute__((aligned(16))) __bf16 sX0[SC * kP];
    __shared__ __attribute__((aligned(16))) __bf16 sX1[SC * kP];
    __shared__ __attribute__((aligned(16))) float sT[2][NTAB][SC];  // decay tables by parity
    __shared__ float sTot[2];
    // the decay-weighted causal score tiles M (row block tb, column block sb <= tb: tile
    // tb (tb + 1) / 2 + sb), each as the 64 lanes' accumulator values in lane order
    __shared__ __attribute__((aligned(16))) __bf16 sM[10][256];
    auto bufB = [&](auto ph) -> __bf16 * {
        if constexpr (decltype(ph)::value == 0)
            return sB0;
        else
            return sB1;
    };
    auto bufX = [&](auto ph) -> __bf16 * {
        if constexpr (decltype(ph)::value == 0)
            return sX0;
        else
            return sX1;
    };

    // workgroups of one segment (all heads of a stream) go to the same XCD
    const int nwg = gridDim.x;
    int lid = blockIdx.x;
    if ((nwg & 7) == 0)
        lid = (lid & 7) * (nwg >> 3) + (lid >> 3);
    const int H = a.s.H, G = a.s.G;
    const int h0 = lid % H;
    const int sg = (lid / H) % a.nseg;
    const int b = lid / (H * a.nseg);
    const int g = h0 / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int64_t len = a.len;
    const int64_t seg_t0 = static_cast<int64_t>(sg) * a.seg_sub * SC;
    const int nsub = static_cast<int>(min<int64_t>(a.seg_sub, (len - seg_t0 + SC - 1) / SC));
    const int64_t nsub_all = (len + SC - 1) / SC;
    const int rowBC = G * kN, rowX = H * kP;
    const int64_t tok0 = static_cast<int64_t>(b) * len;
    const int64_t NP = static_cast<int64_t>(kN) * kP;
    const __bf16 *Bg = static_cast<const __bf16 *>(a.in.B) + tok0 * rowBC + g * kN;
    const __bf16 *Cg = static_cast<const __bf16 *>(a.in.C) + tok0 * rowBC + g * kN;
    const __bf16 *xg = static_cast<const __bf16 *>(a.in.x) + tok0 * rowX + h0 * kP;
    const __bf16 *dtg = static_cast<const __bf16 *>(a.in.dt) + tok0 * H + h0;
    const float Ah = a.A[h0], Dh = (!REV || a.D) ? a.D[h0] : 0.f;
    const auto mk = buffer_range;
    // rows of sub-chunk k of the segment; 0 past the segment (its copies then move nothing)
    auto rows_of = [&](int k) {
        const int64_t t0 = seg_t0 + static_cast<int64_t>(k) * SC;
        return k < nsub ? static_cast<int>(min<int64_t>(SC, len - t0)) : 0;
    };

    // ---- copies of sub-chunk k (range-checked buffers based at its first token: rows past
    // the stream's end read as zero or land nothing). B, C: 16 pieces of 4 rows, wavefront w
    // takes w + 4u; x: 8 pieces of 8 rows, w + 4u.
    auto copy_rows = [&](const __bf16 *base, __bf16 *dst, int k) {
        const int64_t t0 = seg_t0 + static_cast<int64_t>(k) * SC;
        const int nrows = rows_of(k);
        const auto r = mk(base + first_token<REV>(len, t0, nrows) * rowBC, nrows > 0 ? ((nrows - 1) * rowBC + kN) * 2 : 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int pc = wave + 4 * u, row = 4 * pc + (lane >> 4), c = (lane & 15) ^ swz(row);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + bc_row(4 * pc)),
                                                     16, (mem_row<REV>(row, nrows) * rowBC + 8 * c) * 2, 0, 0, 0);
        }
    };
    auto copy_x = [&](__bf16 *dst, int k) {
        const int64_t t0 = seg_t0 + static_cast<int64_t>(k) * SC;
        const int nrows = rows_of(k);
        const auto r = mk(xg + first_token<REV>(len, t0, nrows) * rowX, nrows > 0 ? ((nrows - 1) * rowX + kP) * 2 : 0);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int px = wave + 4 * u, row = 8 * px + (lane >> 3), c = (lane & 7) ^ swz_x(row);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + 8 * px * kP),
                                                     16, (mem_row<REV>(row, nrows) * rowX + 8 * c) * 2, 0, 0, 0);
        }
    };
    // dt of sub-chunk k, token `lane` (zero past the end)
    auto load_dt = [&](int k) {
        const int64_t t0 = seg_t0 + static_cast<int64_t>(k) * SC;
        const int nrows = rows_of(k);
        const auto r = mk(dtg + first_token<REV>(len, t0, nrows) * H, nrows > 0 ? ((nrows - 1) * H + 1) * 2 : 0);
        return __builtin_amdgcn_raw_buffer_load_b16(r, mem_row<REV>(lane, nrows) * H * 2, 0, 0);
    };
    // cumulative log2-decays of a sub-chunk from its dt, into table buffer PH: every wavefront
    // forms the sums and writes its share of the tables
    auto tables = [&](auto Wc, auto PH, unsigned short dbits) {
        constexpr int W = decltype(Wc)::value;
        const float d = __uint_as_float(static_cast<uint32_t>(dbits) << 16);
        const float inc = wave_prefix_sum(d * Ah);
        const float c = inc * kLog2e;
        float(*tb)[SC] = sT[decltype(PH)::value];
        if constexpr (W == 0) {
            tb[TAB_C][lane] = c;
            sTot[decltype(PH)::value] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inc), 63));
        } else if constexpr (W == 1) {
            tb[TAB_EF][lane] = __builtin_amdgcn_exp2f(c);
        } else if constexpr (W == 2) {
            tb[TAB_LG][lane] = __builtin_amdgcn_logf(d) - c;
        } else {
            const float c31 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 31));
            const float clast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 63));
            const float ref = lane < 32 ? c31 : clast;  // end of this token's 32-token pair
            tb[TAB_COL][lane] = __builtin_amdgcn_exp2f(ref - c) * d;
            tb[TAB_W][lane] = __builtin_amdgcn_exp2f(clast - c) * d;
        }
    };

    // ---- operand reads
    // B or C rows 16 blk + r16, contraction n = 32 m + 4 q + e and 32 m + 16 + 4 q + e (e < 4):
    // the order of the state product's h operand, taken by both operands of the score tiles too
    auto k_frag = [&](const __bf16 *T, int blk, int m) {
        const int row = 16 * blk + r16, sw = swz(row);
        const __bf16 *p = T + bc_row(row) + 4 * (q & 1);
        return cat(*reinterpret_cast<const bf16x4 *>(p + 8 * ((4 * m + (q >> 1)) ^ sw)),
                   *reinterpret_cast<const bf16x4 *>(p + 8 * ((4 * m + 2 + (q >> 1)) ^ sw)));
    };
    // B^T: lane (r16, q) gets B[32 ks + 4 q + e][16 i + r16] and B[32 ks + 16 + 4 q + e][..]
    auto bt_frag = [&](const __bf16 *T, int ks, int i) {
        const int tr = 32 * ks + 4 * q + (r16 >> 2), col = 16 * i + 4 * (r16 & 3);
        const __bf16 *p = T + bc_row(tr) + 8 * ((col >> 3) ^ swz(tr)) + (col & 7);
        const __bf16 *p16 = T + bc_row(tr + 16) + 8 * ((col >> 3) ^ swz(tr + 16)) + (col & 7);
        return cat(tr_read(p), tr_read(p16));
    };
    // x~: lane (r16, q) gets x[32 m + 4 q + e][p0 + r16] and x[32 m + 16 + 4 q + e][..]
    auto x_frag = [&](const __bf16 *X, int m, int p0) {
        const int tr = 32 * m + 4 * q + (r16 >> 2), col = p0 + 4 * (r16 & 3), sw = swz_x(tr);
        const __bf16 *p = X + tr * kP + 8 * ((col >> 3) ^ sw) + (col & 7);
        return cat(tr_read(p), tr_read(p + 16 * kP));
    };

    f32x4 hs[8];  // hs[i] holds h[16 i + 4 q + j][p0 + r16]
    auto store_state = [&](float *base, int p0) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                base[(16 * i + 4 * q + j) * kP + p0 + r16] = hs[i][j];
    };
    // a chunk state is the state after a chunk's last sub-chunk, and after the stream's last;
    // kend: the segment's next chunk end (segment-local sub-chunk), cnext: that chunk
    const int64_t gsub0 = seg_t0 / SC;
    const int kstream_end = gsub0 + nsub == nsub_all ? nsub - 1 : -1;
    int kend = static_cast<int>(a.chunk_sub - 1 - gsub0 % a.chunk_sub);
    int64_t cnext = gsub0 / a.chunk_sub;
    auto emit_chunk_state = [&](int k, int p0) {  // after sub-chunk k, for k = 0, 1, .. in turn
        if (k == kend || k == kstream_end)
            store_state(a.chunk_states + ((static_cast<int64_t>(b) * a.nch + cnext) * H + h0) * NP, p0);
        if (k == kend) {
            kend += a.chunk_sub;
            ++cnext;
        }
    };

    // wavefront W owns state columns 16 W .. 16 W + 15 and score tiles W, W + 4, W + 8; it
    // writes its share of the next sub-chunk's tables. Everything below is specialized per
    // wavefront.
    auto body = [&](auto Wc) {
        constexpr int W = decltype(Wc)::value;
        constexpr int p0 = 16 * W;
        unsigned short dnext = 0;  // dt of the sub-chunk after the current one

        // one sub-chunk k, in buffers PH = k % 2
        auto step = [&](auto PH, int k) {
            constexpr int ph = decltype(PH)::value;
            using PN = std::integral_constant<int, 1 - ph>;
            const int64_t t0 = seg_t0 + static_cast<int64_t>(k) * SC;
            const int nvalid = rows_of(k);
            // (A) the copies of k have landed (only the four y stores of k-1 may still be in
            // flight) and its tables are written
            workgroup_lds_barrier<4>();
            if (a.chunk_states && k > 0)
                emit_chunk_state(k - 1, p0);
            // operand reads go out a group ahead of their products: the first two score
            // tiles' (B and C blocks) before the copies and the tables, so that those cover
            // their latency; the C blocks stay for the state product
            constexpr int NT = W < 2 ? 3 : 2;  // score tiles W, W + 4, W + 8 (of 10)
            bf16x8 cf[4][4], bf[2][4], xf[2];
            auto read_c = [&](auto TBc) {
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    cf[decltype(TBc)::value][m] = k_frag(sC, decltype(TBc)::value, m);
            };
            auto read_b = [&](auto SLc, int sb) {
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    bf[decltype(SLc)::value][m] = k_frag(bufB(PH), sb, m);
            };
            read_c(std::integral_constant<int, tile_tb(W)>{});
            read_b(std::integral_constant<int, 0>{}, tile_sb(W));
            if constexpr (!REV) {  // (the reverse order, which holds more, takes it later)
                read_c(std::integral_constant<int, tile_tb(W + 4)>{});
                read_b(std::integral_constant<int, 1>{}, tile_sb(W + 4));
            }
#pragma unroll
            for (int m = 0; m < 2; ++m)
                xf[m] = x_frag(bufX(PH), m, p0);
            auto y_res = [&]() {
                return mk(static_cast<Ty *>(a.y) + (tok0 + first_token<REV>(len, t0, nvalid)) * rowX,
                          static_cast<int64_t>(nvalid) * rowX * sizeof(Ty));
            };
            auto y_off = [&](int tb) {
                const int row = mem_row<REV>(16 * tb + r16, nvalid);
                return ((row * H + h0) * kP + p0 + 4 * q) * static_cast<int>(sizeof(Ty));
            };
            // REV: the forward half's outputs of this wavefront's columns, loaded ahead of the
            // copies so that waiting for them never waits for a copy
            using YRaw = std::conditional_t<sizeof(Ty) == 2, bf16x4, f32x4>;  // as stored
            YRaw yprev[4];
            __amdgpu_buffer_rsrc_t yr;
            if constexpr (REV) {
                yr = y_res();
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    if constexpr (sizeof(Ty) == 2)
                        yprev[tb] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(yr, y_off(tb), 0, 0));
                    else
                        yprev[tb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(yr, y_off(tb), 0, 0));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            const unsigned short dn = load_dt(k + 2);
            copy_rows(Bg, bufB(PN{}), k + 1);
            copy_x(bufX(PN{}), k + 1);
            __builtin_amdgcn_sched_barrier(0);
            tables(Wc, PN{}, dnext);  // sub-chunk k+1, into the table buffer k-1 has left
            dnext = dn;
            if constexpr (!REV)
                yr = y_res();
            const float(*tbl)[SC] = sT[ph];
            // (1) this wavefront's score tiles S[tb][sb] = B_s . C_t, decay-weighted (factored
            // below the diagonal 32-token pair, per element on it), stored for all; the next
            // tile's blocks (after the last, the C blocks no tile read) are read first
            // decay weights of tile i (factored below the diagonal 32-token pair, per element
            // on it) and its store for all
            auto weigh = [&](auto Ic, const f32x4 &S) {
                constexpr int i = decltype(Ic)::value, tau = W + 4 * i, tb = tile_tb(tau), sb = tile_sb(tau);
                // lane (t, q) holds S[s = 16 sb + 4q + j][t]
                const int t = 16 * tb + r16, s0 = 16 * sb + 4 * q;
                constexpr int mp = sb >> 1;
                const float ct = tbl[TAB_C][t];
                float mv[4];
                if constexpr (mp < (tb >> 1)) {  // pair wholly below the row block
                    const float rowf = __builtin_amdgcn_exp2f(ct - tbl[TAB_C][32 * mp + 31]);
                    const float4 cw = *reinterpret_cast<const float4 *>(&tbl[TAB_COL][s0]);
                    mv[0] = S[0] * cw.x * rowf;
                    mv[1] = S[1] * cw.y * rowf;
                    mv[2] = S[2] * cw.z * rowf;
                    mv[3] = S[3] * cw.w * rowf;
                } else {  // the pair holding the row block: masked to s <= t
                    const float4 lg = *reinterpret_cast<const float4 *>(&tbl[TAB_LG][s0]);
                    const float l4[4] = {lg.x, lg.y, lg.z, lg.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        mv[j] = s0 + j <= t ? S[j] * __builtin_amdgcn_exp2f(ct + l4[j]) : 0.f;
                }
                bf16x4 mb;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    mb[j] = static_cast<__bf16>(mv[j]);
                *reinterpret_cast<bf16x4 *>(&sM[tau][4 * lane]) = mb;
            };
            auto read_rest_c = [&]() {  // the C blocks no tile read, for the state product
                if constexpr (!REV)
                    static_for<4>([&](auto Tc) {
                        if constexpr (!tile_row_of(W, NT, decltype(Tc)::value))
                            read_c(Tc);
                    });
            };
            // (1) this wavefront's score tiles S[tb][sb] = B_s . C_t: tiles 0 and 1 with their
            // products interleaved (their blocks were read before the copies; the reverse
            // order: tile 1's read after tile 0's products), then tile 2
            {
                constexpr int tb0 = tile_tb(W), tb1 = tile_tb(W + 4);
                f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
                if constexpr (REV) {
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        S0 = mfma(bf[0][m], cf[tb0][m], S0);
                    read_c(std::integral_constant<int, tb1>{});
                    read_b(std::integral_constant<int, 1>{}, tile_sb(W + 4));
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        S1 = mfma(bf[1][m], cf[tb1][m], S1);
                } else {
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        S0 = mfma(bf[0][m], cf[tb0][m], S0);
                        S1 = mfma(bf[1][m], cf[tb1][m], S1);
                    }
                }
                if constexpr (NT > 2) {
                    read_c(std::integral_constant<int, tile_tb(W + 8)>{});
                    read_b(std::integral_constant<int, 0>{}, tile_sb(W + 8));
                } else {
                    read_rest_c();
                }
                weigh(std::integral_constant<int, 0>{}, S0);
                weigh(std::integral_constant<int, 1>{}, S1);
            }
            if constexpr (NT > 2) {
                constexpr int tb2 = tile_tb(W + 8);
                f32x4 S2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    S2 = mfma(bf[0][m], cf[tb2][m], S2);
                read_rest_c();
                weigh(std::integral_constant<int, 2>{}, S2);
            }
            // (2) the state entering the sub-chunk: y^T[p][t] = sum_n h[n][p] C[t][n], the
            // state as the A operand: rounded to bf16 for a bf16 y (the rounding y takes
            // anyway), split into bf16 hi + lo for an fp32 y
            f32x4 acc[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float hv[8] = {hs[2 * m][0], hs[2 * m][1], hs[2 * m][2], hs[2 * m][3],
                                     hs[2 * m + 1][0], hs[2 * m + 1][1], hs[2 * m + 1][2], hs[2 * m + 1][3]};
                bf16x8 hfh, hfl;
                if constexpr (sizeof(Ty) == 2) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        hfh[e] = static_cast<__bf16>(hv[e]);
                } else {
                    split8(hv, hfh, hfl);
                }
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    // (the reverse order, which also holds the forward outputs, reads C again
                    // rather than keep it)
                    const bf16x8 c = REV ? k_frag(sC, tb, m) : cf[tb][m];
                    acc[tb] = mfma(hfh, c, acc[tb]);
                    if constexpr (sizeof(Ty) != 2)
                        acc[tb] = mfma(hfl, c, acc[tb]);
                }
            }
            workgroup_lds_barrier<63>();  // (A2) the weighted tiles are stored; C is free
            copy_rows(Cg, sC, k + 1);
            // the copies stay ahead of the y stores: barrier (A) counts on exactly four
            // operations after them
            __builtin_amdgcn_sched_barrier(0);
            // the operands of (3), and of the first half of (4), read ahead of the products
            bf16x4 mt[10];  // the weighted tiles, in lane order
#pragma unroll
            for (int tau = 0; tau < 10; ++tau)
                mt[tau] = *reinterpret_cast<const bf16x4 *>(&sM[tau][4 * lane]);
            bf16x4 xv[4];
            float ef[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int t = 16 * tb + r16, pc = p0 + 4 * q;
                xv[tb] = *reinterpret_cast<const bf16x4 *>(bufX(PH) + t * kP + 8 * ((pc >> 3) ^ swz_x(t)) + (pc & 7));
                ef[tb] = tbl[TAB_EF][t];
            }
            bf16x8 bt[2][8];
            float wv[2][8];
            auto read_bt = [&](auto KSc) {
                constexpr int ks = decltype(KSc)::value;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    bt[ks][i] = bt_frag(bufB(PH), ks, i);
                const float4 w0 = *reinterpret_cast<const float4 *>(&tbl[TAB_W][32 * ks + 4 * q]);
                const float4 w1 = *reinterpret_cast<const float4 *>(&tbl[TAB_W][32 * ks + 16 + 4 * q]);
                wv[ks][0] = w0.x, wv[ks][1] = w0.y, wv[ks][2] = w0.z, wv[ks][3] = w0.w;
                wv[ks][4] = w1.x, wv[ks][5] = w1.y, wv[ks][6] = w1.z, wv[ks][7] = w1.w;
            };
            read_bt(std::integral_constant<int, 0>{});
            // (3) + sum_{s<=t} M[t][s] x_s per 32-token pair, + D x_t; the lane holds
            // y[t][p0 + 4q .. p0 + 4q + 3]
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int md = tb >> 1;
                acc[tb] *= ef[tb];
#pragma unroll
                for (int m = 0; m <= md; ++m) {
                    const int lo = tb * (tb + 1) / 2 + 2 * m;  // tile (tb, 2m); (tb, 2m+1) follows
                    acc[tb] = mfma(xf[m], cat(mt[lo], 2 * m + 1 <= tb ? mt[lo + 1] : bf16x4{}), acc[tb]);
                }
                float o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[j] = fmaf(Dh, bf2f(xv[tb][j]), acc[tb][j]);
                if constexpr (REV) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if constexpr (sizeof(Ty) == 2)
                            o[j] += bf2f(yprev[tb][j]);
                        else
                            o[j] += yprev[tb][j];
                    }
                }
                const int off = y_off(tb);
                if constexpr (sizeof(Ty) == 2) {
                    bf16x4 ov;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        ov[j] = static_cast<__bf16>(o[j]);
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2i32, ov), yr, off, 0, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b128(
                        v4i32{__float_as_int(o[0]), __float_as_int(o[1]), __float_as_int(o[2]), __float_as_int(o[3])},
                        yr, off, 0, 0);
                }
            }
            read_bt(std::integral_constant<int, 1>{});
            // (4) state: h <- exp(c_63) h + B^T (w o x), w_s = exp(c_63 - c_s) dt_s
            {
                const float alpha = __expf(sTot[ph]);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    hs[i] *= alpha;
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float xw[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    xw[e] = bf2f(xf[ks][e]) * wv[ks][e];
                bf16x8 xhi, xlo;
                split8(xw, xhi, xlo);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    hs[i] = mfma(bt[ks][i], xhi, hs[i]);
                    hs[i] = mfma(bt[ks][i], xlo, hs[i]);
                }
            }
            // no barrier here: the next step's barrier (A) comes before any buffer or table
            // read in this step is written again
        };

        // ---- prologue: clear the staging buffers when the stream ends inside a sub-chunk
        // (rows past its end must hold finite values: they are weighted 0), put sub-chunk 0
        // in flight, load the entering state, build the tables of 0, let everything land
        if (len % SC != 0) {
            const uint4 z = make_uint4(0, 0, 0, 0);
            for (int i = tid; i < BC_TILE / 8; i += 256) {
                *reinterpret_cast<uint4 *>(sB0 + 8 * i) = z;
                *reinterpret_cast<uint4 *>(sB1 + 8 * i) = z;
                *reinterpret_cast<uint4 *>(sC + 8 * i) = z;
            }
            for (int i = tid; i < SC * kP / 8; i += 256) {
                *reinterpret_cast<uint4 *>(sX0 + 8 * i) = z;
                *reinterpret_cast<uint4 *>(sX1 + 8 * i) = z;
            }
            workgroup_lds_barrier<63>();
        }
        const unsigned short d0 = load_dt(0);
        dnext = load_dt(1);
        copy_rows(Bg, sB0, 0);
        copy_rows(Cg, sC, 0);
        copy_x(sX0, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            hs[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.h_in) {
            const float *hin = a.h_in + ((static_cast<int64_t>(b) * a.nseg + sg) * H + h0) * NP;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    hs[i][j] = hin[(16 * i + 4 * q + j) * kP + p0 + r16];
        }
        tables(Wc, std::integral_constant<int, 0>{}, d0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        int k = 0;
        for (; k + 2 <= nsub; k += 2) {  // pairs of sub-chunks: a body with no branch
            step(std::integral_constant<int, 0>{}, k);
            step(std::integral_constant<int, 1>{}, k + 1);
        }
        if (k < nsub)
            step(std::integral_constant<int, 0>{}, k);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // no copy outlives the workgroup
        if (a.chunk_states)
            emit_chunk_state(nsub - 1, p0);
        if (a.h_last && sg == a.nseg - 1)
            store_state(a.h_last + (static_cast<int64_t>(b) * H + h0) * NP, p0);
    };
    switch (wave) {
    case 0: body(std::integral_constant<int, 0>{}); break;
    case 1: body(std::integral_constant<int, 1>{}); break;
    case 2: body(std::integral_constant<int, 2>{}); break;
    default: body(std::integral_constant<int, 3>{}); break;
    }
}

__global__ __launch_bounds__(256, 2) void k_full_bf16(ScanArgs a) { full_pass<__bf16, false>(a); }
__global__ __launch_bounds__(256, 2) void k_full_f32(ScanArgs a) { full_pass<float, false>(a); }
__global__ __launch_bounds__(256, 2) void k_full_bf16_rev(ScanArgs a) { full_pass<__bf16, true>(a); }
__global__ __launch_bounds__(256, 2) void k_full_f32_rev(ScanArgs a) { full_pass<float, true>(a); }

// The full pass, one head per workgroup: k_full_* with y, k_scan with the chunk states only
template <typename Ty>
hipError_t launch_full(const ScanArgs &a, bool rev, hipStream_t st)
{
    const int nwg = a.s.b * a.nseg * a.s.H;
    if (a.y) {
        if constexpr (sizeof(Ty) == 2) {
            if (rev)
                k_full_bf16_rev<<<dim3(nwg), dim3(256), 0, st>>>(a);
            else
                k_full_bf16<<<dim3(nwg), dim3(256), 0, st>>>(a);
        } else {
            if (rev)
                k_full_f32_rev<<<dim3(nwg), dim3(256), 0, st>>>(a);
            else
                k_full_f32<<<dim3(nwg), dim3(256), 0, st>>>(a);
        }
        return hipGetLastError();
    }
    if (rev)  // the reverse order exists for the passes with y only
        return hipErrorInvalidValue;
    k_scan<1><<<dim3(nwg), dim3(256), 0, st>>>(a);
    return hipGetLastError();
}

template <int HPW>
hipError_t launch_fold(const ScanArgs &a, bool rev, hipStream_t st)
{
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.s.b) * a.nseg * (a.s.H / HPW)));
    const dim3 block(HPW == 1 ? 256 : 512);  // HS = 2 for 2 and 4 heads: eight wavefronts
    if (rev) {
        if constexpr (HPW == 4)
            k_fold4_rev<<<grid, block, 0, st>>>(a);
        else if constexpr (HPW == 2)
            k_fold2_rev<<<grid, block, 0, st>>>(a);
        else
            k_fold1_rev<<<grid, block, 0, st>>>(a);
    } else {
        if constexpr (HPW == 4)
            k_fold4<<<grid, block, 0, st>>>(a);
        else if constexpr (HPW == 2)
            k_fold2<<<grid, block, 0, st>>>(a);
        else
            k_fold1<<<grid, block, 0, st>>>(a);
    }
    return hipGetLastError();
}

// The state-only pass (k_fold, HPW heads per workgroup)
hipError_t launch_state_pass(const ScanArgs &a, int hpw, bool rev, hipStream_t st)
{
    if (hpw == 4)
        return launch_fold<4>(a, rev, st);
    if (hpw == 2)
        return launch_fold<2>(a, rev, st);
    return launch_fold<1>(a, rev, st);
}

// Heads per workgroup of the state-only pass: the largest of 4 and 2 that divides the heads
// of one B/C group (a staged B then serves them all) and still leaves a workgroup for every
// CU with nseg segments per stream; else 1 (two workgroups per CU).
int pick_fold_hpw(const Shape &s, int64_t nseg)
{
    const int hpg = s.H / s.G;
    for (int hpw = 4; hpw > 1; hpw /= 2)
        if (hpg % hpw == 0 && static_cast<int64_t>(s.b) * nseg * (s.H / hpw) >= device_cus())
            return hpw;
    return 1;
}

}  // namespace

bool prefix_mfma_supported(const Shape &s, int chunk)
{
    return s.in_dt == 1 && s.N == kN && s.P == kP && chunk % SC == 0;
}

// Work plan: segments of consecutive sub-chunks, as many (stream, head group, segment)
// workgroups as the GPU holds at once -- a few more would run as a second, mostly empty
// round. The full pass runs one head per workgroup, 2 workgroups per CU. A state-only scan
// takes a single segment when (stream, head group) workgroups already fill the GPU, else
// the largest head group dividing the heads of one B/C group with as many segments as one
// workgroup per CU allows (two per CU with one head each).
PrefixPlan prefix_mfma_plan(const Shape &s, int64_t len, int chunk, bool full, bool single_segment)
{
    (void)chunk;
    PrefixPlan p{};
    const int64_t nsub = std::max<int64_t>(1, (len + SC - 1) / SC);
    const int64_t bh = std::max<int64_t>(1, static_cast<int64_t>(s.b) * s.H);
    int64_t want = 1;
    // a scan of one or two sub-chunks (a commit) is bound by its states' traffic: one head per
    // workgroup puts the most workgroups, and so the most of that traffic, in flight
    int hpw = nsub <= 2 ? 1 : pick_fold_hpw(s, 1);
    if (!single_segment) {
        if (full) {
            want = std::max<int64_t>(1, 2 * device_cus() / bh);
        } else if (bh / hpw < device_cus()) {
            const int hpg = s.H / s.G;
            hpw = hpg % 4 == 0 ? 4 : hpg % 2 == 0 ? 2 : 1;
            want = std::max<int64_t>(1, (hpw > 1 ? 1 : 2) * device_cus() / (bh / hpw));
        }
    }
    const int64_t seg_sub = (nsub + want - 1) / want;
    p.seg_sub = static_cast<int>(seg_sub);
    p.nseg = static_cast<int>((nsub + seg_sub - 1) / seg_sub);
    p.hpw_state = full ? pick_fold_hpw(s, p.nseg) : hpw;
    const int64_t nbh = static_cast<int64_t>(s.b) * p.nseg * s.H;
    p.tot_bytes = p.nseg > 1 ? static_cast<size_t>((nbh * 4 + 255) / 256 * 256) : 0;
    p.ws_bytes = p.nseg > 1 ? p.tot_bytes + static_cast<size_t>(nbh) * kN * kP * 4 : 0;
    return p;
}

hipError_t run_prefix_mfma(const Shape &s, int64_t len, int chunk, const Seq &in, const float *A,
                           const float *D, const float *h_init, void *y, float *chunk_states,
                           float *h_out, void *ws, hipStream_t st, bool single_segment, bool rev,
                           void *enc, bool enc_hi_only)
{
    const bool full = y || chunk_states;
    if (rev && (!y || chunk_states))  // reverse order: y accumulated, nothing else
        return hipErrorInvalidValue;
    if (enc && (full || !single_segment))  // the encoded copy comes from a single state pass
        return hipErrorInvalidValue;
    const PrefixPlan p = prefix_mfma_plan(s, len, chunk, full, single_segment);
    ScanArgs a{};
    a.s = s;
    a.len = len;
    a.seg_sub = p.seg_sub;
    a.nseg = p.nseg;
    a.chunk_sub = chunk / SC;
    a.nch = static_cast<int>((len + chunk - 1) / chunk);
    a.in = in;
    a.A = A;
    a.D = D;
    a.enc = enc;
    a.enc_hi_only = enc_hi_only ? 1 : 0;
    auto run_full = [&]() {
        a.y = y;
        a.chunk_states = chunk_states;
        a.h_last = h_out;
        return s.y_dt ? launch_full<__bf16>(a, rev, st) : launch_full<float>(a, rev, st);
    };
    if (p.nseg == 1) {
        // one segment per (stream, head): a single pass from h_init straight to h_out
        // (the [b][nseg][H] layouts are the [b][H] layouts for nseg == 1)
        a.h_in = h_init;
        if (full)
            return run_full();
        a.h_end = h_out;
        return launch_state_pass(a, p.hpw_state, rev, st);
    }
    hipError_t e;
    float *tot = static_cast<float *>(ws);
    float *segs = reinterpret_cast<float *>(static_cast<char *>(ws) + p.tot_bytes);
    // 1. segment end states from zero
    a.h_in = nullptr;
    a.h_end = segs;
    a.tot = tot;
    if ((e = launch_state_pass(a, p.hpw_state, rev, st)) != hipSuccess)
        return e;
    // 2. states entering each segment (in place); the final state when nothing else follows
    {
        dim3 grid(static_cast<unsigned>((kN * kP / 4 + 255) / 256), s.H, s.b);
        k_seg_scan<<<grid, 256, 0, st>>>(segs, tot, p.nseg, s.H, h_init, full ? nullptr : h_out);
        if ((e = hipGetLastError()) != hipSuccess || !full)
            return e;
    }
    // 3. the full pass from the entering states; the last segment writes h_out
    a.h_in = segs;
    a.h_end = nullptr;
    a.tot = nullptr;
    return run_full();
}

}  // namespace bdssm
