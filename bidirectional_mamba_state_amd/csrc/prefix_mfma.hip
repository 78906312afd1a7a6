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
//          k_state (one head per workgroup, inputs copied straight into LDS) or k_scan<false,
//          2> (two heads per workgroup, inputs staged through registers).
//   FULL   from the state entering the segment: also y (k_full_*, inputs copied straight
//          into LDS), or only the chunk states (k_scan<true, 1>): the state after every
//          chunk of Q tokens and after the last token, and, for the stream's last segment,
//          the final state.
// k_scan stages B and x through registers into the fragment-major order of mfma_tiles.h
// (an operand fragment is one contiguous 512-byte read per wavefront).
// The fp32 states and the weighted x~ operand are split into bf16 hi + lo parts, so that
// products against them keep ~16 significant bits; B, C and x are exact in bf16.
#include <algorithm>
#include <type_traits>

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
};

template <int HPW>
struct Lds {
    __bf16 B[SC * kN];
    __bf16 X[HPW][SC * kP];
    float tab[2][HPW][NTAB][SC];  // decay tables of sub-chunks k and k+1 (by parity)
    float tot[2][HPW];
};


template <bool FULL, int HPW>
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
    auto emit_chunk_state = [&](int k) {  // state after sub-chunk k, at chunk ends and the end
        const int64_t gsub = seg_t0 / SC + k;  // sub-chunk index within the stream
        if ((gsub + 1) % a.chunk_sub == 0 || gsub == nsub_all - 1) {
            const int64_t c = gsub / a.chunk_sub;
            store_state(a.chunk_states + ((static_cast<int64_t>(b) * a.nch + c) * H + h0) * NP);
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
        if (FULL && a.chunk_states && k > 0)
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
    if (FULL && a.chunk_states)
        emit_chunk_state(nsub - 1);

    // ---- end of the segment
    if (!FULL && a.h_end)
        store_state(a.h_end + ((static_cast<int64_t>(b) * a.nseg + sg) * H + h0) * NP);
    if (FULL && a.h_last && sg == a.nseg - 1)
        store_state(a.h_last + (static_cast<int64_t>(b) * H + h0) * NP);
    if (!FULL && a.tot && tid == 0) {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
            a.tot[(static_cast<int64_t>(b) * a.nseg + sg) * H + h0 + hh] = seg_tot[hh];
    }
}

// Segment scan, one thread per state element: the end states of segments started from
// zero become the states entering each segment (in place), and the final state.
__global__ __launch_bounds__(256) void k_seg_scan(float *buf, const float *tot, int nseg, int H,
                                                  const float *h_init, float *h_out)
{
    const int64_t NP = static_cast<int64_t>(kN) * kP;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    if (e >= NP)
        return;
    float v = h_init ? h_init[(static_cast<int64_t>(b) * H + h) * NP + e] : 0.f;
    for (int s = 0; s < nseg; ++s) {
        const int64_t bh = (static_cast<int64_t>(b) * nseg + s) * H + h;
        const float loc = buf[bh * NP + e];
        buf[bh * NP + e] = v;
        v = fmaf(__expf(tot[bh]), v, loc);
    }
    if (h_out)
        h_out[(static_cast<int64_t>(b) * H + h) * NP + e] = v;
}

// State-only pass (segment end states, and the commit): h <- exp(c_63) h + B^T (w o x) per
// 64-token sub-chunk, w_s = exp(c_63 - c_s) dt_s, with the state in the MFMA accumulators of
// wavefront w (columns 16w .. 16w+15) as in k_scan. Its time per sub-chunk is the staging of
// B and x (24 KB per head), so they are copied straight into LDS (gfx950 buffer loads to
// LDS, no registers on the way) in whole 128-byte lines, two sub-chunks ahead into three
// buffers, and read by transposing reads. One head per workgroup (with two, the operands
// do not fit the registers beside the states; those launches keep k_scan).
// The compiler waits for a copy before an LDS read only when it cannot tell that the two
// touch different buffers; it can when each buffer is its own LDS array, the loop is
// unrolled by NBUF (buffer choice known at compile time) and its body has no branch. So:
// the loop runs whole groups of NBUF sub-chunks (the rest after it), every wavefront builds
// its own copy of the decay tables (no wavefront-dependent branch), the staging buffers
// are cleared once before the first copy instead of per sub-chunk (rows past the stream's
// end then hold zeros or an earlier sub-chunk's finite inputs, and weigh 0), and the
// barriers are bare (a memory fence would wait for every copy). Tile layouts, 16-byte
// pieces of a row permuted so that a transposing read (4 rows x 32 bytes per 16 lanes)
// falls in distinct banks:
//   B: 64 rows x 128 bf16, piece c of row t at slot c ^ 2 (t % 4);
//   x: 64 rows x 64 bf16 per head, piece c of row t at slot c ^ 2 (t % 4).
__global__ __launch_bounds__(256, 2) void k_state(ScanArgs a)
{
    constexpr int HPW = 1, NBUF = 3;
    __shared__ __attribute__((aligned(16))) __bf16 sB0[SC * kN];
    __shared__ __attribute__((aligned(16))) __bf16 sB1[SC * kN];
    __shared__ __attribute__((aligned(16))) __bf16 sB2[SC * kN];
    __shared__ __attribute__((aligned(16))) __bf16 sX0[HPW][SC * kP];
    __shared__ __attribute__((aligned(16))) __bf16 sX1[HPW][SC * kP];
    __shared__ __attribute__((aligned(16))) __bf16 sX2[HPW][SC * kP];
    // per wavefront: TAB_W and the total log-decay of sub-chunks k, k+1, k+2 (by k % 3)
    __shared__ __attribute__((aligned(16))) float sW[3][4][HPW][SC];
    __shared__ float sTot[3][4][HPW];
    auto bufB = [&](auto ph) -> __bf16 * {
        if constexpr (decltype(ph)::value == 0)
            return sB0;
        else if constexpr (decltype(ph)::value == 1)
            return sB1;
        else
            return sB2;
    };
    auto bufX = [&](auto ph, int hh) -> __bf16 * {
        if constexpr (decltype(ph)::value == 0)
            return sX0[hh];
        else if constexpr (decltype(ph)::value == 1)
            return sX1[hh];
        else
            return sX2[hh];
    };

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
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p0 = 16 * wave;  // this wavefront's state columns

    const int64_t len = a.len;
    const int64_t seg_t0 = static_cast<int64_t>(sg) * a.seg_sub * SC;
    const int nsub = static_cast<int>(min<int64_t>(a.seg_sub, (len - seg_t0 + SC - 1) / SC));
    const int rowBC = G * kN, rowX = H * kP;
    const int64_t tok0 = static_cast<int64_t>(b) * len;
    const int64_t NP = static_cast<int64_t>(kN) * kP;
    const __bf16 *Bg = static_cast<const __bf16 *>(a.in.B) + tok0 * rowBC + g * kN;
    const __bf16 *xg = static_cast<const __bf16 *>(a.in.x) + tok0 * rowX + h0 * kP;
    const __bf16 *dtg = static_cast<const __bf16 *>(a.in.dt) + tok0 * H + h0;
    // range-checked buffers over the tokens of one sub-chunk (based at its first token, so
    // that offsets stay small however long the stream): rows past the stream's end read as
    // zero
    const auto mk = buffer_range;
    float Ah[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
        Ah[hh] = a.A[h0 + hh];

    // ---- copies of sub-chunk k into buffer PH = k % NBUF: B in 16 pieces of 1 KB (4 rows),
    // x in 8 per head (8 rows); wavefront w takes B pieces w + 4u (u < 4) and x pieces
    // w + 4 (u - 4) (u >= 4)
    constexpr int NPW = 4 + 2 * HPW;  // pieces per wavefront
    auto piece_B = [&](int u) { return wave + 4 * u; };
    auto piece_X = [&](int u) { return wave + 4 * (u - 4); };  // head px / 8, rows 8 (px % 8) ..
    auto copy = [&](auto PH, int k) {
        const int kk = min(k, nsub - 1);  // past the segment: the last sub-chunk again (unused)
        const int64_t t0 = seg_t0 + static_cast<int64_t>(kk) * SC;
        const int nrows = static_cast<int>(min<int64_t>(SC, len - t0));
        const auto rB = mk(Bg + t0 * rowBC, ((nrows - 1) * rowBC + kN) * 2);
        const auto rX = mk(xg + t0 * rowX, ((nrows - 1) * rowX + HPW * kP) * 2);
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
            if (u < 4) {
                const int pc = piece_B(u), row = 4 * pc + (lane >> 4), c = (lane & 15) ^ (2 * (row & 3));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rB, (__attribute__((address_space(3))) void *)(bufB(PH) + 4 * pc * kN), 16,
                    (row * rowBC + 8 * c) * 2, 0, 0, 0);
            } else {
                const int px = piece_X(u), hh = px >> 3, row = 8 * (px & 7) + (lane >> 3);
                const int c = (lane & 7) ^ (2 * (row & 3));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rX, (__attribute__((address_space(3))) void *)(bufX(PH, hh) + 8 * (px & 7) * kP), 16,
                    (row * rowX + hh * kP + 8 * c) * 2, 0, 0, 0);
            }
        }
    };
    auto clear = [&](auto PH) {  // this wavefront's pieces of buffer PH
        const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
            if (u < 4) {
                *reinterpret_cast<uint4 *>(bufB(PH) + 4 * piece_B(u) * kN + 8 * lane) = z;
            } else {
                const int px = piece_X(u);
                *reinterpret_cast<uint4 *>(bufX(PH, px >> 3) + 8 * (px & 7) * kP + 8 * lane) = z;
            }
        }
    };
    // dt of sub-chunk k, token `lane`, every head of the workgroup (zero past the stream's
    // end; k past the segment: its last sub-chunk again)
    auto load_dt = [&](int k, unsigned short (&d)[HPW]) {
        const int kk = min(k, nsub - 1);
        const int64_t t0 = seg_t0 + static_cast<int64_t>(kk) * SC;
        const int nrows = static_cast<int>(min<int64_t>(SC, len - t0));
        const auto rD = mk(dtg + t0 * H, ((nrows - 1) * H + HPW) * 2);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
            d[hh] = __builtin_amdgcn_raw_buffer_load_b16(rD, (lane * H + hh) * 2, 0, 0);
    };
    // TAB_W and the total log-decay of sub-chunk k into this wavefront's own tables
    auto tables = [&](int k, const unsigned short (&dbits)[HPW]) {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            const float d = __uint_as_float(static_cast<uint32_t>(dbits[hh]) << 16);
            const float inc = wave_prefix_sum(d * Ah[hh]);
            const float c = inc * kLog2e;
            const float clast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 63));
            sW[k % 3][wave][hh][lane] = __builtin_amdgcn_exp2f(clast - c) * d;
            sTot[k % 3][wave][hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inc), 63));
        }
    };

    f32x4 hs[HPW][8];  // hs[hh][i] holds h[16 i + 4 q + j][p0 + r16] of head h0 + hh
    float seg_tot[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
        seg_tot[hh] = 0.f;
    // one sub-chunk k, in buffer PH = k % NBUF
    auto step = [&](auto PH, int k) {
        constexpr int ph = decltype(PH)::value, phn = (ph + NBUF - 1) % NBUF;
        // this wavefront's copies of k have landed once at most those issued after them are
        // in flight: dt of k+1 and the copies of k+1
        workgroup_lds_barrier<NPW + HPW>();
        unsigned short dn[HPW];
        {
            // every operand of the sub-chunk into registers first: B^T (contraction over tokens
            // 32 ks + 4q + e and 32 ks + 16 + 4q + e, rows n = 16 i + r16) and x~ (columns
            // p0 + r16) by transposing reads (lane r16 addresses row 4q + r16/4, columns
            // 4 (r16 % 4) .. of a 16-column block), and the weights
            bf16x8 bt[2][8], xf[HPW][2];
            float wv[HPW][2][8];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int tr = 32 * ks + 4 * q + (r16 >> 2), sw = 2 * (tr & 3);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int col = 16 * i + 4 * (r16 & 3);
                    const __bf16 *p = bufB(PH) + tr * kN + 8 * ((col >> 3) ^ sw) + (col & 7);
                    bt[ks][i] = cat(tr_read(p), tr_read(p + 16 * kN));
                }
#pragma unroll
                for (int hh = 0; hh < HPW; ++hh) {
                    const int col = p0 + 4 * (r16 & 3);
                    const __bf16 *px = bufX(PH, hh) + tr * kP + 8 * ((col >> 3) ^ sw) + (col & 7);
                    xf[hh][ks] = cat(tr_read(px), tr_read(px + 16 * kP));
                    const float4 w0 = *reinterpret_cast<const float4 *>(&sW[k % 3][wave][hh][32 * ks + 4 * q]);
                    const float4 w1 = *reinterpret_cast<const float4 *>(&sW[k % 3][wave][hh][32 * ks + 16 + 4 * q]);
                    wv[hh][ks][0] = w0.x, wv[hh][ks][1] = w0.y, wv[hh][ks][2] = w0.z, wv[hh][ks][3] = w0.w;
                    wv[hh][ks][4] = w1.x, wv[hh][ks][5] = w1.y, wv[hh][ks][6] = w1.z, wv[hh][ks][7] = w1.w;
                }
            }
            float tot[HPW];
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh)
                tot[hh] = sTot[k % 3][wave][hh];
            // then sub-chunk k + NBUF - 1 into the buffer k - 1 has left, its dt first (the
            // compiler may make the reads above wait for the copies of k+1, but not for these)
            load_dt(k + 2, dn);
            copy(std::integral_constant<int, phn>{}, k + NBUF - 1);

            // state: h <- exp(c_63) h + B^T (w o x)
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                seg_tot[hh] += tot[hh];
                const float alpha = __expf(tot[hh]);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    hs[hh][i] *= alpha;
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int hh = 0; hh < HPW; ++hh) {
                    float xw[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        xw[e] = bf2f(xf[hh][ks][e]) * wv[hh][ks][e];
                    bf16x8 xhi, xlo;
                    split8(xw, xhi, xlo);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        hs[hh][i] = mfma(bt[ks][i], xhi, hs[hh][i]);
                        hs[hh][i] = mfma(bt[ks][i], xlo, hs[hh][i]);
                    }
                }
            }
        }
        // tables of sub-chunk k+2 into the table buffer k-1 has left
        tables(k + 2, dn);
    };

    // ---- prologue: clear this wavefront's staging pieces, put sub-chunks 0 .. NBUF-2 in
    // flight (each dt ahead of the copies after it, so that waiting for it never waits for
    // them), load the entering state, build the tables of 0 and 1, and let everything land
    // once, so that the waits in the loop can be counted exactly
    clear(std::integral_constant<int, 0>{});
    clear(std::integral_constant<int, 1>{});
    clear(std::integral_constant<int, 2>{});
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the clears precede the copies
    {
        unsigned short d0[HPW], d1[HPW];
        load_dt(0, d0);
        copy(std::integral_constant<int, 0>{}, 0);
        load_dt(1, d1);
        copy(std::integral_constant<int, 1>{}, 1);
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
        tables(0, d0);
        tables(1, d1);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    int k = 0;
    for (; k + NBUF <= nsub; k += NBUF) {  // whole groups: a body with no branch
        step(std::integral_constant<int, 0>{}, k);
        step(std::integral_constant<int, 1>{}, k + 1);
        step(std::integral_constant<int, 2>{}, k + 2);
    }
    if (k < nsub)
        step(std::integral_constant<int, 0>{}, k);
    if (k + 1 < nsub)
        step(std::integral_constant<int, 1>{}, k + 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no copy outlives the workgroup

    // ---- end of the segment
    if (a.h_end) {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            float *base = a.h_end + ((static_cast<int64_t>(b) * a.nseg + sg) * H + h0 + hh) * NP;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    base[(16 * i + 4 * q + j) * kP + p0 + r16] = hs[hh][i][j];
        }
    }
    if (a.tot && tid == 0) {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
            a.tot[(static_cast<int64_t>(b) * a.nseg + sg) * H + h0 + hh] = seg_tot[hh];
    }
}

// ---- FULL pass with outputs, one head per workgroup, inputs copied straight into LDS
//
// The same computation as k_scan<true, true, 1> (and bitwise the same state walk as
// k_state), with B, C and x copied into LDS by buffer loads to LDS in whole lines instead of
// through registers: B and x of sub-chunk k+1 are copied at the start of sub-chunk k into
// the other of two buffers; C, read only before the mid-sub-chunk barrier, has one buffer
// and its next copy is issued right after that barrier. 71.5 KB of LDS: two workgroups per
// CU. B and C rows (256 bytes) hold piece c of row r at slot c ^ swz(r), which keeps three
// read patterns free of bank conflicts: 16-byte operand reads of 16 consecutive rows (score
// tiles), transposing reads of 4 rows x 16 columns per 16 lanes (B in the state update) and
// 8-byte reads of the permuted contraction order (C in the state product); x rows
// (128 bytes) hold piece c of row t at slot c ^ 2 (t % 4), as in k_state.
__device__ __forceinline__ int swz(int r)
{
    return ((r & 3) << 2) | ((r & 4) >> 1) | ((r >> 3) & 1);
}

// (the body is a device function template with one kernel per output type: a kernel
// template built from generic lambdas loses its host-side launch stub in this compiler)
template <typename Ty>
__device__ __forceinline__ void full_pass(const ScanArgs &a)
{
    __shared__ __attribute__((aligned(16))) __bf16 sB0[SC * kN];
    __shared__ __attribute__((aligned(16))) __bf16 sB1[SC * kN];
    __shared__ __attribute__((aligned(16))) __bf16 sC[SC * kN];
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
    const float Ah = a.A[h0], Dh = a.D[h0];
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
        const auto r = mk(base + t0 * rowBC, nrows > 0 ? ((nrows - 1) * rowBC + kN) * 2 : 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int pc = wave + 4 * u, row = 4 * pc + (lane >> 4), c = (lane & 15) ^ swz(row);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + 4 * pc * kN),
                                                     16, (row * rowBC + 8 * c) * 2, 0, 0, 0);
        }
    };
    auto copy_x = [&](__bf16 *dst, int k) {
        const int64_t t0 = seg_t0 + static_cast<int64_t>(k) * SC;
        const int nrows = rows_of(k);
        const auto r = mk(xg + t0 * rowX, nrows > 0 ? ((nrows - 1) * rowX + kP) * 2 : 0);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int px = wave + 4 * u, row = 8 * px + (lane >> 3), c = (lane & 7) ^ (2 * (row & 3));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + 8 * px * kP),
                                                     16, (row * rowX + 8 * c) * 2, 0, 0, 0);
        }
    };
    // dt of sub-chunk k, token `lane` (zero past the end)
    auto load_dt = [&](int k) {
        const int64_t t0 = seg_t0 + static_cast<int64_t>(k) * SC;
        const int nrows = rows_of(k);
        const auto r = mk(dtg + t0 * H, nrows > 0 ? ((nrows - 1) * H + 1) * 2 : 0);
        return __builtin_amdgcn_raw_buffer_load_b16(r, lane * H * 2, 0, 0);
    };
    // cumulative log2-decays of a sub-chunk from its dt, into table buffer PH
    auto tables = [&](auto PH, unsigned short dbits) {
        const float d = __uint_as_float(static_cast<uint32_t>(dbits) << 16);
        const float inc = wave_prefix_sum(d * Ah);
        const float c = inc * kLog2e;
        const float c31 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 31));
        const float clast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 63));
        const float ref = lane < 32 ? c31 : clast;  // end of this token's 32-token pair
        float(*tb)[SC] = sT[decltype(PH)::value];
        tb[TAB_C][lane] = c;
        tb[TAB_EF][lane] = __builtin_amdgcn_exp2f(c);
        tb[TAB_LG][lane] = __builtin_amdgcn_logf(d) - c;
        tb[TAB_COL][lane] = __builtin_amdgcn_exp2f(ref - c) * d;
        tb[TAB_W][lane] = __builtin_amdgcn_exp2f(clast - c) * d;
        sTot[decltype(PH)::value] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inc), 63));
    };

    // ---- operand reads
    // B or C rows 16 blk + r16, contraction n = 32 m + 8 q .. +7 (score tiles)
    auto row_frag = [&](const __bf16 *T, int blk, int m) {
        const int row = 16 * blk + r16;
        return *reinterpret_cast<const bf16x8 *>(T + row * kN + 8 * ((4 * m + q) ^ swz(row)));
    };
    // C rows 16 tb + r16, contraction n = 32 m + 4 q + e and 32 m + 16 + 4 q + e (state product)
    auto c_frag = [&](int tb, int m) {
        const int row = 16 * tb + r16, sw = swz(row);
        const __bf16 *p = sC + row * kN + 4 * (q & 1);
        return cat(*reinterpret_cast<const bf16x4 *>(p + 8 * ((4 * m + (q >> 1)) ^ sw)),
                   *reinterpret_cast<const bf16x4 *>(p + 8 * ((4 * m + 2 + (q >> 1)) ^ sw)));
    };
    // B^T: lane (r16, q) gets B[32 ks + 4 q + e][16 i + r16] and B[32 ks + 16 + 4 q + e][..]
    auto bt_frag = [&](const __bf16 *T, int ks, int i) {
        const int tr = 32 * ks + 4 * q + (r16 >> 2), col = 16 * i + 4 * (r16 & 3);
        const __bf16 *p = T + tr * kN + 8 * ((col >> 3) ^ swz(tr)) + (col & 7);
        const __bf16 *p16 = T + (tr + 16) * kN + 8 * ((col >> 3) ^ swz(tr + 16)) + (col & 7);
        return cat(tr_read(p), tr_read(p16));
    };
    // x~: lane (r16, q) gets x[32 m + 4 q + e][p0 + r16] and x[32 m + 16 + 4 q + e][..]
    auto x_frag = [&](const __bf16 *X, int m, int p0) {
        const int tr = 32 * m + 4 * q + (r16 >> 2), col = p0 + 4 * (r16 & 3), sw = 2 * (tr & 3);
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
    auto emit_chunk_state = [&](int k, int p0) {  // state after sub-chunk k, at chunk ends and the end
        const int64_t gsub = seg_t0 / SC + k;
        if ((gsub + 1) % a.chunk_sub == 0 || gsub == nsub_all - 1) {
            const int64_t c = gsub / a.chunk_sub;
            store_state(a.chunk_states + ((static_cast<int64_t>(b) * a.nch + c) * H + h0) * NP, p0);
        }
    };

    // wavefront W owns state columns 16 W .. 16 W + 15 and score tiles W, W + 4, W + 8;
    // wavefront 0 builds the decay tables. Everything below is specialized per wavefront.
    auto body = [&](auto Wc) {
        constexpr int W = decltype(Wc)::value;
        constexpr int p0 = 16 * W;

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
            bf16x8 xf[2];
#pragma unroll
            for (int m = 0; m < 2; ++m)
                xf[m] = x_frag(bufX(PH), m, p0);
            __builtin_amdgcn_sched_barrier(0);
            unsigned short dn = 0;
            if constexpr (W == 0)
                dn = load_dt(k + 1);
            copy_rows(Bg, bufB(PN{}), k + 1);
            copy_x(bufX(PN{}), k + 1);
            __builtin_amdgcn_sched_barrier(0);
            const __amdgpu_buffer_rsrc_t yr =
                mk(static_cast<Ty *>(a.y) + (tok0 + t0) * rowX, static_cast<int64_t>(nvalid) * rowX * sizeof(Ty));
            const float(*tbl)[SC] = sT[ph];
            // (1) this wavefront's score tiles S[tb][sb] = B_s . C_t, decay-weighted (factored
            // below the diagonal 32-token pair, per element on it), stored for all
#pragma unroll
            for (int rr = 0; rr < 3; ++rr) {
                const int tau = W + 4 * rr;
                if (tau < 10) {
                    const int tb = tau >= 6 ? 3 : tau >= 3 ? 2 : tau >= 1 ? 1 : 0;
                    const int sb = tau - tb * (tb + 1) / 2;
                    f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        S = mfma(row_frag(bufB(PH), sb, m), row_frag(sC, tb, m), S);
                    // lane (t, q) holds S[s = 16 sb + 4q + j][t]
                    const int t = 16 * tb + r16, mp = sb >> 1, s0 = 16 * sb + 4 * q;
                    const float ct = tbl[TAB_C][t];
                    float mv[4];
                    if (mp < (tb >> 1)) {  // pair wholly below the row block
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
                }
            }
            // (2) the state entering the sub-chunk: y^T[p][t] = sum_n h[n][p] C[t][n], the
            // state accumulators split into bf16 hi + lo as the A operand
            f32x4 acc[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float hv[8] = {hs[2 * m][0], hs[2 * m][1], hs[2 * m][2], hs[2 * m][3],
                                     hs[2 * m + 1][0], hs[2 * m + 1][1], hs[2 * m + 1][2], hs[2 * m + 1][3]};
                bf16x8 hfh, hfl;
                split8(hv, hfh, hfl);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const bf16x8 cf = c_frag(tb, m);
                    acc[tb] = mfma(hfh, cf, acc[tb]);
                    acc[tb] = mfma(hfl, cf, acc[tb]);
                }
            }
            workgroup_lds_barrier<63>();  // (A2) the weighted tiles are stored; C is free
            copy_rows(Cg, sC, k + 1);
            // the copies stay ahead of the y stores: barrier (A) counts on exactly four
            // operations after them
            __builtin_amdgcn_sched_barrier(0);
            // (3) + sum_{s<=t} M[t][s] x_s per 32-token pair, + D x_t; the lane holds
            // y[t][p0 + 4q .. p0 + 4q + 3]
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int t = 16 * tb + r16, md = tb >> 1;
                acc[tb] *= tbl[TAB_EF][t];
#pragma unroll
                for (int m = 0; m <= md; ++m) {
                    const int lo = tb * (tb + 1) / 2 + 2 * m;  // tile (tb, 2m); (tb, 2m+1) follows
                    const bf16x4 m0 = *reinterpret_cast<const bf16x4 *>(&sM[lo][4 * lane]);
                    const bf16x4 m1 =
                        2 * m + 1 <= tb ? *reinterpret_cast<const bf16x4 *>(&sM[lo + 1][4 * lane]) : bf16x4{};
                    acc[tb] = mfma(xf[m], cat(m0, m1), acc[tb]);
                }
                const int pc = p0 + 4 * q;
                const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(
                    bufX(PH) + t * kP + 8 * ((pc >> 3) ^ (2 * (t & 3))) + (pc & 7));
                float o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[j] = fmaf(Dh, bf2f(xv[j]), acc[tb][j]);
                const int off = ((t * H + h0) * kP + pc) * static_cast<int>(sizeof(Ty));
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
            // (4) state: h <- exp(c_63) h + B^T (w o x), w_s = exp(c_63 - c_s) dt_s (the same
            // arithmetic as k_state, so that the walk is bitwise the state-only pass's)
            {
                const float tot = sTot[ph];
                const float alpha = __expf(tot);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    hs[i] *= alpha;
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 bt[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    bt[i] = bt_frag(bufB(PH), ks, i);
                const float4 w0 = *reinterpret_cast<const float4 *>(&tbl[TAB_W][32 * ks + 4 * q]);
                const float4 w1 = *reinterpret_cast<const float4 *>(&tbl[TAB_W][32 * ks + 16 + 4 * q]);
                const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
                float xw[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    xw[e] = bf2f(xf[ks][e]) * wv[e];
                bf16x8 xhi, xlo;
                split8(xw, xhi, xlo);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    hs[i] = mfma(bt[i], xhi, hs[i]);
                    hs[i] = mfma(bt[i], xlo, hs[i]);
                }
            }
            workgroup_lds_barrier<63>();  // (B) every LDS read for sub-chunk k is done
            if constexpr (W == 0)
                tables(PN{}, dn);  // sub-chunk k+1, into the table buffer k-1 has left
        };

        // ---- prologue: clear the staging buffers when the stream ends inside a sub-chunk
        // (rows past its end must hold finite values: they are weighted 0), put sub-chunk 0
        // in flight, load the entering state, build the tables of 0, let everything land
        if (len % SC != 0) {
            const uint4 z = make_uint4(0, 0, 0, 0);
            for (int i = tid; i < SC * kN / 8; i += 256) {
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
        unsigned short d0 = 0;
        if constexpr (W == 0)
            d0 = load_dt(0);
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
        if constexpr (W == 0)
            tables(std::integral_constant<int, 0>{}, d0);
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

__global__ __launch_bounds__(256, 2) void k_full_bf16(ScanArgs a) { full_pass<__bf16>(a); }
__global__ __launch_bounds__(256, 2) void k_full_f32(ScanArgs a) { full_pass<float>(a); }

template <bool FULL, int HPW, typename Ty>
hipError_t launch_scan(const ScanArgs &a, hipStream_t st)
{
    const int nwg = a.s.b * a.nseg * (a.s.H / HPW);
    if constexpr (FULL) {
        static_assert(HPW == 1, "the full pass runs one head per workgroup");
        if (a.y) {
            if constexpr (sizeof(Ty) == 2)
                k_full_bf16<<<dim3(nwg), dim3(256), 0, st>>>(a);
            else
                k_full_f32<<<dim3(nwg), dim3(256), 0, st>>>(a);
            return hipGetLastError();
        }
    }
    k_scan<FULL, HPW><<<dim3(nwg), dim3(256), 0, st>>>(a);
    return hipGetLastError();
}

template <bool FULL, typename Ty>
hipError_t launch_scan_hpw(const ScanArgs &a, int hpw, hipStream_t st)
{
    if constexpr (!FULL) {  // the state-only pass
        if (hpw == 2)
            return launch_scan<FULL, 2, Ty>(a, st);
        k_state<<<dim3(static_cast<unsigned>(a.s.b * a.nseg * a.s.H)), dim3(256), 0, st>>>(a);
        return hipGetLastError();
    } else {
        return launch_scan<FULL, 1, Ty>(a, st);
    }
}

// Heads per workgroup: as many as the pass allows (shared B/C staging and scores), but
// no fewer workgroups than CUs when the segment count is fixed at one.
int pick_hpw(const Shape &s, bool full, bool single_segment)
{
    const int hpg = s.H / s.G;
    int hpw = full ? 1 : (static_cast<int64_t>(s.b) * s.H >= 2048 ? 2 : 1);
    while (hpw > 1 && hpg % hpw != 0)
        hpw /= 2;
    if (single_segment)
        while (hpw > 1 && static_cast<int64_t>(s.b) * (s.H / hpw) < 256)
            hpw /= 2;
    return hpw;
}

}  // namespace

bool prefix_mfma_supported(const Shape &s, int chunk)
{
    return s.in_dt == 1 && s.N == kN && s.P == kP && chunk % SC == 0;
}

// Work plan: segments of consecutive sub-chunks, as many (stream, head group, segment)
// workgroups as the GPU holds at once -- a few more would run as a second, mostly empty
// round. The full pass holds 2 workgroups per CU, the state-only pass with one head per
// workgroup 4.
PrefixPlan prefix_mfma_plan(const Shape &s, int64_t len, int chunk, bool full, bool single_segment)
{
    (void)chunk;
    PrefixPlan p{};
    const int hpw = pick_hpw(s, full, single_segment);
    const int64_t groups = std::max<int64_t>(1, static_cast<int64_t>(s.b) * (s.H / hpw));
    const int64_t nsub = std::max<int64_t>(1, (len + SC - 1) / SC);
    const int64_t slots = static_cast<int64_t>(full || hpw > 1 ? 2 : 4) * device_cus();
    const int64_t want = single_segment ? 1 : std::max<int64_t>(1, slots / groups);
    const int64_t seg_sub = (nsub + want - 1) / want;
    p.seg_sub = static_cast<int>(seg_sub);
    p.nseg = static_cast<int>((nsub + seg_sub - 1) / seg_sub);
    const int64_t nbh = static_cast<int64_t>(s.b) * p.nseg * s.H;
    p.tot_bytes = p.nseg > 1 ? static_cast<size_t>((nbh * 4 + 255) / 256 * 256) : 0;
    p.ws_bytes = p.nseg > 1 ? p.tot_bytes + static_cast<size_t>(nbh) * kN * kP * 4 : 0;
    return p;
}

hipError_t run_prefix_mfma(const Shape &s, int64_t len, int chunk, const Seq &in, const float *A,
                           const float *D, const float *h_init, void *y, float *chunk_states,
                           float *h_out, void *ws, hipStream_t st, bool single_segment)
{
    const bool full = y || chunk_states;
    const PrefixPlan p = prefix_mfma_plan(s, len, chunk, full, single_segment);
    const int hpw_full = pick_hpw(s, true, single_segment);
    const int hpw_state = pick_hpw(s, false, single_segment || p.nseg == 1);
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
    auto run_full = [&]() {
        a.y = y;
        a.chunk_states = chunk_states;
        a.h_last = h_out;
        return s.y_dt ? launch_scan_hpw<true, __bf16>(a, hpw_full, st)
                      : launch_scan_hpw<true, float>(a, hpw_full, st);
    };
    if (p.nseg == 1) {
        // one segment per (stream, head): a single pass from h_init straight to h_out
        // (the [b][nseg][H] layouts are the [b][H] layouts for nseg == 1)
        a.h_in = h_init;
        if (full)
            return run_full();
        a.h_end = h_out;
        return launch_scan_hpw<false, float>(a, hpw_state, st);
    }
    hipError_t e;
    float *tot = static_cast<float *>(ws);
    float *segs = reinterpret_cast<float *>(static_cast<char *>(ws) + p.tot_bytes);
    // 1. segment end states from zero
    a.h_in = nullptr;
    a.h_end = segs;
    a.tot = tot;
    if ((e = launch_scan_hpw<false, float>(a, hpw_state, st)) != hipSuccess)
        return e;
    // 2. states entering each segment (in place); the final state when nothing else follows
    {
        dim3 grid(static_cast<unsigned>((kN * kP + 255) / 256), s.H, s.b);
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
