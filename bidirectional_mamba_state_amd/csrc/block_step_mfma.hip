// Block step on bf16 matrix cores (gfx950 v_mfma_f32_16x16x32_bf16), d_state 128, headdim 64.
//
// One denoising step of "Training Hybrid Block Diffusion Language Models with Partial
// Bidirectionality", eqs. (11)-(13), in the matrix ("dual") form of the Mamba-2 scan.
// With a_t = dt_t A and cumulative sums c_t = sum_{k<=t} a_k (forward) and
// r_t = sum_{k>=t} a'_k (reverse), for one head:
//   y_t = exp(c_t) C_t . h_prefix                                   forward, cached state
//       + sum_{s<=t} exp(c_t - c_s) dt_s (C_t . B_s) x_s            forward, inside the block
//       + sum_{s>=t} exp(r_t - r_s) dt'_s (C'_t . B'_s) x'_s        reverse, inside the block
//       + D x_t
// which equals the two recurrences of the eqs. up to rounding.
//
// Work split. A workgroup owns one stream, HPW consecutive heads of one B/C group and a
// slice of P/PS columns. Its wavefronts each own one "unit": a 16-token row block and a
// group of 16-column blocks. The score tiles S = C B^T of both directions depend only on
// the stream's group, so each wavefront computes the NB+1 causal 16x16 tiles of its row
// block once (forward tiles for s-blocks <= its block, reverse tiles for s-blocks >=
// it) and keeps them in registers for all HPW heads. Per head:
//   - the fp32 state is read once from HBM, split into bf16 hi + lo parts and stored
//     transposed in LDS (the matrix-core operand wants 8 consecutive d_state entries per
//     lane); x of both directions is read once and stored transposed in LDS;
//   - the next head's state and x are already being loaded into registers while this
//     head computes (software pipelining across the head loop);
//   - each wavefront accumulates y^T = (h_hi + h_lo)^T C^T on the matrix cores, scales by
//     exp(c_t), builds the decay-masked operands M = S o exp2(..) o dt from its register
//     tiles, accumulates X^T M^T for both directions, adds D x and writes y once. The
//     outputs are transposed so that a lane holds four consecutive columns of one token
//     and stores them as one 8-byte (bf16) or 16-byte (fp32) piece.
// The k-index of the M X products is permuted (lane slots j = 0..3 take s-block 2m, slots
// 4..7 s-block 2m+1) so that the score tiles' accumulator layout is directly the operand
// layout of M^T; the X operand uses the same permutation.
#include "internal.h"
#include "mfma_tiles.h"
#include "wave_ops.h"

namespace bdssm {
namespace {

constexpr int kN = 128, kP = 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 ld16(const void *p) { return *static_cast<const bf16x8 *>(p); }

// Guarded loads without branches (sel8, sel4 of mfma_tiles.h): the address is clamped to a
// valid row and the value replaced by zero afterwards, so that all loads of a phase can be
// in flight together (a branch around a load makes the compiler wait for every outstanding
// load).

__device__ __forceinline__ void store4(float *p, const float (&v)[4])
{
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(__bf16 *p, const float (&v)[4])
{
    bf16x4 b;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        b[j] = static_cast<__bf16>(v[j]);
    *reinterpret_cast<bf16x4 *>(p) = b;
}

template <int NB, int PS>
struct Geo {
    static constexpr int TP = NB * 16;        // padded block length
    static constexpr int PW = kP / PS;        // columns owned by the workgroup
    static constexpr int PBLK = PW / 16;      // 16-column blocks of the workgroup
    static constexpr int PBW = PBLK * NB / 8 > 0 ? PBLK * NB / 8 : 1;  // column blocks per unit
    static constexpr int PGRP = PBLK / PBW;   // column groups per row block
    static constexpr int UNITS = NB * PGRP;   // one per wavefront
    static constexpr int THREADS = 64 * UNITS;
    static constexpr int YW = PBW * 16;       // columns of a unit's output tile
    // LDS row strides (bf16 elements): transposed state [PW][HS] (16-byte operand reads),
    // transposed x [PW][XS] (8-byte operand reads)
    static constexpr int HS = kN + 8;
    static constexpr int XS = TP + 4;
    // global-load items: state = 8 rows x 2 columns, x = 4 tokens x 8 columns
    static constexpr int SITEMS = (kN / 8) * (PW / 2);
    static constexpr int XITEMS = (TP / 4) * (PW / 8);  // per direction
    static constexpr int SPT = (SITEMS + THREADS - 1) / THREADS;      // per thread
    static constexpr int XPT = (2 * XITEMS + THREADS - 1) / THREADS;  // per thread
};

// One head's global data for this thread, held in registers between load and LDS store.
// Values are kept exactly as loaded (no masking or conversion): any use right after the
// load would make the wavefront wait for the whole prefetch.
template <int SPT, int XPT>
struct Stage {
    float2 s[SPT][8];
    uint4 x[XPT][4];
    __bf16 d0, d1;  // dt of tokens 2*lane, 2*lane+1 (wavefronts 0 and 1)
    float A, D;     // the head's A and D
    float Ar, Dr;   // the reverse direction's A and skip weight (0 without one)
};

// per-head decay tables (log2 units), one set per LDS buffer
enum { TAB_CF, TAB_CR, TAB_LGF, TAB_LGR, TAB_COLF, TAB_COLR, TAB_EF, NTAB };

// DCH: skip weights per head and channel ([H][P], read where the outputs are formed)
template <int NB, int PS, typename Ty, bool DCH>
__global__ __launch_bounds__((Geo<NB, PS>::THREADS), 2) void k_block_mfma(BlockArgs a, int hpw, int n_hg)
{
    using Gm = Geo<NB, PS>;
    constexpr int TP = Gm::TP, PW = Gm::PW, PBW = Gm::PBW, PGRP = Gm::PGRP, THREADS = Gm::THREADS,
                  HS = Gm::HS, XS = Gm::XS, YW = Gm::YW, SITEMS = Gm::SITEMS,
                  XITEMS = Gm::XITEMS, SPT = Gm::SPT, XPT = Gm::XPT;
    // two buffers: the next head is staged while the current one is being computed
    __shared__ __attribute__((aligned(16))) __bf16 hT_hi[2][PW * HS];
    __shared__ __attribute__((aligned(16))) __bf16 hT_lo[2][PW * HS];
    __shared__ __attribute__((aligned(16))) __bf16 XTf[2][PW * XS];
    __shared__ __attribute__((aligned(16))) __bf16 XTr[2][PW * XS];
    __shared__ __attribute__((aligned(16))) float tab[2][NTAB][TP];
    __shared__ float hd[2], hdr[2];  // D and the reverse skip weight of the head in each buffer

    // Workgroups sharing a stream (and so its B, C) go to the same XCD: the hardware
    // deals linear workgroup ids round-robin over the 8 XCDs.
    const int nwg = gridDim.x;
    int lid = blockIdx.x;
    if ((nwg & 7) == 0)
        lid = (lid & 7) * (nwg >> 3) + (lid >> 3);
    const int ps = lid % PS;
    const int hg = (lid / PS) % n_hg;
    const int b = lid / (PS * n_hg);

    const int T = a.T, H = a.s.H, G = a.s.G;
    const int h0 = hg * hpw, g = h0 / (H / G);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
    const int pbase = ps * PW;
    const int tb = wave / PGRP, pgrp = wave % PGRP;  // this wavefront's unit
    const int t = tb * 16 + r16;                      // this lane's row as an A operand
    const int md = tb >> 1;                           // the 32-token pair holding row block tb

    // per-stream bases (uniform) and row strides in elements; per-lane offsets fit 32 bits
    const int64_t tok0 = static_cast<int64_t>(b) * T;
    const int rowBC = G * kN, rowX = H * kP;
    const __bf16 *Bf = static_cast<const __bf16 *>(a.fwd.B) + tok0 * rowBC + g * kN;
    const __bf16 *Cf = static_cast<const __bf16 *>(a.fwd.C) + tok0 * rowBC + g * kN;
    const __bf16 *Br = static_cast<const __bf16 *>(a.rev.B) + tok0 * rowBC + g * kN;
    const __bf16 *Cr = static_cast<const __bf16 *>(a.rev.C) + tok0 * rowBC + g * kN;
    const __bf16 *xf = static_cast<const __bf16 *>(a.fwd.x) + tok0 * rowX + pbase;
    const __bf16 *xr = static_cast<const __bf16 *>(a.rev.x) + tok0 * rowX + pbase;
    const __bf16 *dtf = static_cast<const __bf16 *>(a.fwd.dt) + tok0 * H;
    const __bf16 *dtr = static_cast<const __bf16 *>(a.rev.dt) + tok0 * H;
    const float *hp = a.h_prefix + static_cast<int64_t>(b) * H * (kN * kP) + pbase;
    Ty *y = static_cast<Ty *>(a.y) + tok0 * rowX + pbase;

    auto load_state = [&](Stage<SPT, XPT> &st, int h) {
        const float *hs = hp + h * (kN * kP);
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            const int i = tid + k * THREADS;
            if (SITEMS % THREADS == 0 || i < SITEMS) {
                const int p2 = i % (PW / 2), n8 = (i / (PW / 2)) * 8;
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    st.s[k][r] = *reinterpret_cast<const float2 *>(hs + (n8 + r) * kP + 2 * p2);
            }
        }
    };
    auto load_x = [&](Stage<SPT, XPT> &st, int h) {  // x, dt and the head's parameters
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int i = tid + k * THREADS;
            if ((2 * XITEMS) % THREADS == 0 || i < 2 * XITEMS) {
                const bool rv = i >= XITEMS;
                const int ii = rv ? i - XITEMS : i;
                const int p8 = ii % (PW / 8), t4 = (ii / (PW / 8)) * 4;
                const __bf16 *xs = (rv ? xr : xf) + h * kP + p8 * 8;
#pragma unroll
                for (int r = 0; r < 4; ++r)  // rows past T are zeroed at store time
                    st.x[k][r] = *reinterpret_cast<const uint4 *>(xs + min(t4 + r, T - 1) * rowX);
            }
        }
        {   // every wavefront loads (no branch); wavefronts 0 and 1 use them
            const __bf16 *dts = ((wave & 1) ? dtr : dtf) + h;
            st.d0 = dts[min(2 * lane, T - 1) * H];  // masked at store time
            st.d1 = dts[min(2 * lane + 1, T - 1) * H];
        }
        st.A = a.A[h];
        st.D = a.D[h];
        st.Ar = a.A_rev[h];
        st.Dr = a.D_rev ? a.D_rev[h] : 0.f;
    };
    auto load_stage = [&](Stage<SPT, XPT> &st, int h) {
        load_state(st, h);
        load_x(st, h);
    };

    auto store_stage = [&](const Stage<SPT, XPT> &st, int buf) {
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            const int i = tid + k * THREADS;
            if (SITEMS % THREADS == 0 || i < SITEMS) {
                const int p2 = i % (PW / 2), n8 = (i / (PW / 2)) * 8;
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    float f[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r)
                        f[r] = c ? st.s[k][r].y : st.s[k][r].x;
                    bf16x8 hi, lo;
                    split8(f, hi, lo);
                    *reinterpret_cast<bf16x8 *>(&hT_hi[buf][(2 * p2 + c) * HS + n8]) = hi;
                    *reinterpret_cast<bf16x8 *>(&hT_lo[buf][(2 * p2 + c) * HS + n8]) = lo;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int i = tid + k * THREADS;
            if ((2 * XITEMS) % THREADS == 0 || i < 2 * XITEMS) {
                const bool rv = i >= XITEMS;
                const int ii = rv ? i - XITEMS : i;
                const int p8 = ii % (PW / 8), t4 = (ii / (PW / 8)) * 4;
                __bf16 *dst = (rv ? XTr[buf] : XTf[buf]) + p8 * 8 * XS + t4;
                uint32_t w[4][4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint4 v = sel4(t4 + r < T, st.x[k][r]);
                    w[r][0] = v.x;
                    w[r][1] = v.y;
                    w[r][2] = v.z;
                    w[r][3] = v.w;
                }
                // 4 tokens x 8 columns -> 8 columns x 4 tokens (byte permutes)
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                    const uint32_t lo2 = __builtin_amdgcn_perm(w[1][c / 2], w[0][c / 2], sel);
                    const uint32_t hi2 = __builtin_amdgcn_perm(w[3][c / 2], w[2][c / 2], sel);
                    *reinterpret_cast<uint2 *>(dst + c * XS) = make_uint2(lo2, hi2);
                }
            }
        }
        if (tid == 0) {
            hd[buf] = st.D;
            hdr[buf] = st.Dr;
        }
        // decay tables: wavefront 0 forward (prefix sums), wavefront 1 reverse (suffix sums);
        // lane l holds tokens 2l and 2l+1, so 16 lanes cover one 32-token pair
        if (wave < 2) {
            const int t0 = 2 * lane, t1 = t0 + 1;
            const float d0 = t0 < T ? bf2f(st.d0) : 0.f, d1 = t1 < T ? bf2f(st.d1) : 0.f;
            const float Aw = wave == 0 ? st.A : st.Ar;  // the reverse scan has its own decay
            const float a0 = d0 * Aw, a1 = d1 * Aw;
            const float loc = a0 + a1;
            const float inc = wave_prefix_sum(loc);
            const float excl = inc - loc;
            const float total = wave_lane(inc, 63);
            // forward: c_t inclusive prefix sum; reference at the pair's last token
            // reverse: r_t inclusive suffix sum; reference at the pair's first token
            const float c0 = wave == 0 ? (excl + a0) * kLog2e : (total - excl) * kLog2e;
            const float c1 = wave == 0 ? (excl + loc) * kLog2e : (total - excl - a0) * kLog2e;
            // the pair's last token (forward: lane 16k+15) or first token (reverse: lane 16k);
            // the readlanes as separate statements (inside a conditional expression they
            // would become branches), then a per-lane choice
            const int row = lane >> 4;
            const float f15 = wave_lane(c1, 15), f31 = wave_lane(c1, 31), f47 = wave_lane(c1, 47),
                        f63 = wave_lane(c1, 63);
            const float g00 = wave_lane(c0, 0), g16 = wave_lane(c0, 16), g32 = wave_lane(c0, 32),
                        g48 = wave_lane(c0, 48);
            const float reff = row == 0 ? f15 : row == 1 ? f31 : row == 2 ? f47 : f63;
            const float refr = row == 0 ? g00 : row == 1 ? g16 : row == 2 ? g32 : g48;
            const float ref = wave == 0 ? reff : refr;
            if (t0 < TP) {
                float *cc = tab[buf][wave == 0 ? TAB_CF : TAB_CR];
                float *lg = tab[buf][wave == 0 ? TAB_LGF : TAB_LGR];
                float *col = tab[buf][wave == 0 ? TAB_COLF : TAB_COLR];
                cc[t0] = c0;
                cc[t1] = c1;
                lg[t0] = __builtin_amdgcn_logf(d0) - c0;
                lg[t1] = __builtin_amdgcn_logf(d1) - c1;
                col[t0] = __builtin_amdgcn_exp2f(ref - c0) * d0;
                col[t1] = __builtin_amdgcn_exp2f(ref - c1) * d1;
                if (wave == 0) {
                    tab[buf][TAB_EF][t0] = __builtin_amdgcn_exp2f(c0);
                    tab[buf][TAB_EF][t1] = __builtin_amdgcn_exp2f(c1);
                }
            }
        }
    };

    Stage<SPT, XPT> stage;
    load_stage(stage, h0);  // the first head's data is in flight while the score tiles are built

    // ---- score tiles of this wavefront's row block, once per workgroup
    f32x4 S[NB + 1];
    bf16x8 cfw[4];  // C_t fragments of this row block, kept for the cached-state term
    {
        bf16x8 crv[4];
        const int tc = min(t, T - 1);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            cfw[kk] = sel8(t < T, ld16(Cf + tc * rowBC + 32 * kk + 8 * q));
            crv[kk] = sel8(t < T, ld16(Cr + tc * rowBC + 32 * kk + 8 * q));
        }
#pragma unroll
        for (int ut = 0; ut <= NB; ++ut) {
            const bool fwd = ut <= tb;
            const int s = (fwd ? ut : ut - 1) * 16 + r16, sc = min(s, T - 1);
            const __bf16 *Bp = (fwd ? Bf : Br) + sc * rowBC + 8 * q;
            bf16x8 bfrag[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                bfrag[kk] = sel8(s < T, ld16(Bp + 32 * kk));
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = mfma(bfrag[kk], fwd ? cfw[kk] : crv[kk], acc);
            S[ut] = acc;  // S[t = tb*16 + r16][s = sb*16 + 4q + j]
        }
    }
    store_stage(stage, 0);
    if (hpw > 1)
        load_stage(stage, h0 + 1);
    __syncthreads();

    for (int hh = 0; hh < hpw; ++hh) {
        const int h = h0 + hh, cur = hh & 1;
        const __bf16 *hhi = hT_hi[cur], *hlo = hT_lo[cur], *xtf = XTf[cur], *xtr = XTr[cur];
        const float *cf = tab[cur][TAB_CF], *cr = tab[cur][TAB_CR], *lgf = tab[cur][TAB_LGF],
                    *lgr = tab[cur][TAB_LGR], *colf = tab[cur][TAB_COLF], *colr = tab[cur][TAB_COLR],
                    *ef = tab[cur][TAB_EF];

        f32x4 acc[PBW];
#pragma unroll
        for (int pb = 0; pb < PBW; ++pb)
            acc[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // eq. (11), cached-state term: C_t . h, h = hi + lo; the state fragments of
        // contraction block kk + 1 are read while those of kk are multiplied
        bf16x8 hf[2][PBW][2];
        auto read_h = [&](int kk, bf16x8 (&dst)[PBW][2]) {
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb) {
                const int pc = (pgrp * PBW + pb) * 16 + r16;
                dst[pb][0] = ld16(&hhi[pc * HS + 32 * kk + 8 * q]);
                dst[pb][1] = ld16(&hlo[pc * HS + 32 * kk + 8 * q]);
            }
        };
        read_h(0, hf[0]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (kk + 1 < 4)
                read_h(kk + 1, hf[(kk + 1) & 1]);
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb) {
                acc[pb] = mfma(hf[kk & 1][pb][0], cfw[kk], acc[pb]);
                acc[pb] = mfma(hf[kk & 1][pb][1], cfw[kk], acc[pb]);
            }
        }
        // the rest of the next head's loads (its state was issued after the last barrier):
        // spread out rather than queued all at once behind the barrier, and still ahead of
        // this head's y stores
        if (hh >= 1 && hh + 1 < hpw)
            load_x(stage, h + 1);
        {
            const float et = ef[t];  // exp(c_t) of this lane's token
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb)
                acc[pb] *= et;
        }
        // x fragments of the M X rounds, read one round ahead (forward pairs m = 0 ..
        // NB/2 - 1, then reverse pairs; a round the row block skips is read all the same)
        bf16x8 xq[2][PBW];
        auto read_x = [&](const __bf16 *XT, int m, bf16x8 (&dst)[PBW]) {
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb) {
                const int pc = (pgrp * PBW + pb) * 16 + r16;
                const __bf16 *xp = &XT[pc * XS + 32 * m + 4 * q];
                const bf16x4 lo4 = *reinterpret_cast<const bf16x4 *>(xp);
                const bf16x4 hi4 = *reinterpret_cast<const bf16x4 *>(xp + 16);
                dst[pb] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        };
        auto mx = [&](const bf16x8 &af, const bf16x8 (&xf)[PBW]) {
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb)
                acc[pb] = mfma(xf[pb], af, acc[pb]);
        };
        read_x(xtf, 0, xq[0]);
        // eq. (11), inside the block (s <= t). Pairs wholly below the row block use the
        // factored decay exp2(c_t - c_ref) * [exp2(c_ref - c_s) dt_s], c_ref = c at the
        // pair's last token: both factors are <= 1. The pair holding the row block uses
        // exp2(c_t - c_s + log2 dt_s) per element, masked to s <= t.
        const float ctf = cf[t];
#pragma unroll
        for (int m = 0; m < NB / 2; ++m) {
            if (m + 1 < NB / 2)
                read_x(xtf, m + 1, xq[(m + 1) & 1]);
            else
                read_x(xtr, 0, xq[(m + 1) & 1]);
            if (m < md) {
                const float rowf = __builtin_amdgcn_exp2f(ctf - cf[32 * m + 31]);
                const float4 c0 = *reinterpret_cast<const float4 *>(&colf[32 * m + 4 * q]);
                const float4 c1 = *reinterpret_cast<const float4 *>(&colf[32 * m + 16 + 4 * q]);
                const float cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
                float mv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    mv[j] = (j < 4 ? S[2 * m][j] : S[2 * m + 1][j & 3]) * cw[j] * rowf;
                mx(to_bf16x8(mv), xq[m & 1]);
            } else if (m == md) {
                const float4 l0 = *reinterpret_cast<const float4 *>(&lgf[32 * m + 4 * q]);
                const float4 l1 = *reinterpret_cast<const float4 *>(&lgf[32 * m + 16 + 4 * q]);
                const float lg[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                const bool hi_ok = 2 * m + 1 <= tb;
                float mv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int s = 32 * m + (j < 4 ? 0 : 16) + 4 * q + (j & 3);
                    const float sv = j < 4 ? S[2 * m][j] : (hi_ok ? S[2 * m + 1][j & 3] : 0.f);
                    const float w = __builtin_amdgcn_exp2f(ctf + lg[j]);
                    mv[j] = s <= t ? sv * w : 0.f;
                }
                mx(to_bf16x8(mv), xq[m & 1]);
            }
        }
        // eq. (12), reverse inside the block (s >= t); pairs wholly above the row block use
        // the factored decay with the reference at the pair's first token
        const float ctr = cr[t];
#pragma unroll
        for (int m = 0; m < NB / 2; ++m) {
            constexpr int R0 = NB / 2;  // round index of reverse pair 0
            if (m + 1 < NB / 2)
                read_x(xtr, m + 1, xq[(R0 + m + 1) & 1]);
            if (m > md) {
                const float rowr = __builtin_amdgcn_exp2f(ctr - cr[32 * m]);
                const float4 c0 = *reinterpret_cast<const float4 *>(&colr[32 * m + 4 * q]);
                const float4 c1 = *reinterpret_cast<const float4 *>(&colr[32 * m + 16 + 4 * q]);
                const float cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
                float mv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    mv[j] = (j < 4 ? S[2 * m + 1][j] : S[2 * m + 2][j & 3]) * cw[j] * rowr;
                mx(to_bf16x8(mv), xq[(R0 + m) & 1]);
            } else if (m == md) {
                const float4 l0 = *reinterpret_cast<const float4 *>(&lgr[32 * m + 4 * q]);
                const float4 l1 = *reinterpret_cast<const float4 *>(&lgr[32 * m + 16 + 4 * q]);
                const float lg[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                const bool lo_ok = 2 * m >= tb;
                float mv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int s = 32 * m + (j < 4 ? 0 : 16) + 4 * q + (j & 3);
                    const float sv = j < 4 ? (lo_ok ? S[2 * m + 1][j] : 0.f) : S[2 * m + 2][j & 3];
                    const float w = __builtin_amdgcn_exp2f(ctr + lg[j]);
                    mv[j] = s >= t ? sv * w : 0.f;
                }
                mx(to_bf16x8(mv), xq[(R0 + m) & 1]);
            }
        }
        // eq. (13) + D x, written once: the lane holds y[t][pcb + 4q .. pcb + 4q + 3] of each
        // 16-column block pcb and leaves it as one 8-byte (bf16) or 16-byte (fp32) store
        // (+ D_rev x_rev when the reverse direction has its own skip term)
        const float Dh = hd[cur], Dr = hdr[cur];
        const bool with_dr = a.D_rev != nullptr;
        Ty *yh = y + h * kP + pgrp * YW;
#pragma unroll
        for (int pb = 0; pb < PBW; ++pb) {
            const int pcb = (pgrp * PBW + pb) * 16 + 4 * q;
            float o[4];
            float d4[4] = {Dh, Dh, Dh, Dh}, r4[4] = {Dr, Dr, Dr, Dr};
            if constexpr (DCH) {
                const float4 dv = *reinterpret_cast<const float4 *>(a.D + h * kP + pbase + pcb);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    d4[j] = (&dv.x)[j];
                if (with_dr) {
                    const float4 rv = *reinterpret_cast<const float4 *>(a.D_rev + h * kP + pbase + pcb);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        r4[j] = (&rv.x)[j];
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v = fmaf(d4[j], bf2f(xtf[(pcb + j) * XS + t]), acc[pb][j]);
                o[j] = with_dr ? fmaf(r4[j], bf2f(xtr[(pcb + j) * XS + t]), v) : v;
            }
            if (t < T)
                store4(yh + t * rowX + pb * 16 + 4 * q, o);
        }
        // stage the next head into the other buffer (its previous contents were last read
        // before the barrier that ended the previous head), then sync, then prefetch
        if (hh + 1 < hpw)
            store_stage(stage, cur ^ 1);
        __syncthreads();
        if (hh + 2 < hpw)
            load_state(stage, h + 2);
    }
}

template <int NB, int PS, typename Ty>
hipError_t launch_nb(const BlockArgs &a, int hpw, hipStream_t st)
{
    const int n_hg = a.s.H / hpw;
    const int nwg = a.s.b * n_hg * PS;
    if (a.d_per_channel)
        k_block_mfma<NB, PS, Ty, true><<<dim3(nwg), dim3(Geo<NB, PS>::THREADS), 0, st>>>(a, hpw, n_hg);
    else
        k_block_mfma<NB, PS, Ty, false><<<dim3(nwg), dim3(Geo<NB, PS>::THREADS), 0, st>>>(a, hpw, n_hg);
    return hipGetLastError();
}

template <int PS, typename Ty>
hipError_t launch_ps(const BlockArgs &a, int hpw, hipStream_t st)
{
    if (a.T <= 32)
        return launch_nb<2, PS, Ty>(a, hpw, st);
    if (a.T <= 64)
        return launch_nb<4, PS, Ty>(a, hpw, st);
    return launch_nb<8, PS, Ty>(a, hpw, st);
}

template <typename Ty>
hipError_t launch_ty(const BlockArgs &a, int hpw, int ps, hipStream_t st)
{
    switch (ps) {
    case 1: return launch_ps<1, Ty>(a, hpw, st);
    case 2: return launch_ps<2, Ty>(a, hpw, st);
    default: return launch_ps<4, Ty>(a, hpw, st);
    }
}

}  // namespace

bool block_mfma_supported(const Shape &s, int T)
{
    return s.in_dt == 1 && s.N == kN && s.P == kP && T >= 1 && T <= 128;
}

void block_mfma_plan(const Shape &s, int *hpw, int *ps)
{
    const int hpg = s.H / s.G;
    const int64_t pairs = static_cast<int64_t>(s.b) * s.H;
    if (pairs >= 512) {
        // about one workgroup per CU (256 CUs; 8 wavefronts with up to 256 registers each),
        // each running the heads of one group that share its score tiles, with the next
        // head's loads overlapping the current head's matrix work
        int best = 1;
        for (int d = 1; d <= hpg; ++d) {
            if (hpg % d == 0 && pairs / d >= 256)
                best = d;
        }
        *hpw = best;
        *ps = 1;
    } else {
        *hpw = 1;
        *ps = pairs * 4 <= 4096 ? 4 : 2;
    }
}

hipError_t launch_block_step_mfma(const BlockArgs &a, int hpw, int ps, hipStream_t st)
{
    return a.s.y_dt ? launch_ty<__bf16>(a, hpw, ps, st) : launch_ty<float>(a, hpw, ps, st);
}

}  // namespace bdssm
