// Block step for many (stream, head) pairs with the cached state in operand form: the same
// computation as block_step_mfma.hip (eqs. (11)-(13) of "Training Hybrid Block Diffusion
// Language Models with Partial Bidirectionality" in the matrix form of the Mamba-2 scan),
// laid out so that HBM stays busy.
//
// A workgroup of eight wavefronts owns one stream and HPW heads of one B/C group and walks
// them in turn. Wavefront (tb, pgrp) owns the 16-token row block tb and PBW 16-column blocks
// of the outputs, and keeps the NB+1 causal C B^T score tiles of its row block (forward for
// s-blocks <= tb, reverse for s-blocks >= tb) in registers for all heads of the workgroup.
// Per head, the state in operand form ([hi, lo][N/8][P][8] bf16, 32 KB) and x of both
// directions (token-major, the 16-byte pieces of row t permuted by an XOR with swz_x(t)) are
// copied straight into LDS with gfx950 buffer loads to LDS, in whole 1 KB pieces (no
// registers on the way, no conversion), into one of two buffer sets by head parity: the next
// head's copies stream into the other set while the current head is computed (one workgroup
// per CU, two wavefronts per SIMD). Per head:
//   barrier (the head's copies and tables are in; the other set is free) -> the next head's
//   dt loads and copies -> y^T = h^T C^T from the state -> y^T += X^T M^T of both directions
//   (x by transposing reads) -> the next head's decay tables -> D x, y stores.
// Operand reads run one group ahead of their products (the state fragments of the next
// contraction block, the x fragments of the next M X round). Each wavefront's code is
// specialized on its row block, so the causal structure is resolved at compile time and the
// compiler's waits count exactly the copies in flight.
#include <type_traits>

#include "internal.h"
#include "mfma_tiles.h"
#include "wave_ops.h"

namespace bdssm {
namespace {

constexpr int kN = 128, kP = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 8;
constexpr int kOpsElems = 2 * kN * kP;  // one head's state in operand form, bf16 elements

enum { TAB_CF, TAB_CR, TAB_LGF, TAB_LGR, TAB_COLF, TAB_COLR, TAB_EF, NTAB };

// one workgroup per CU: two wavefronts per SIMD
// HI_ONLY: the cached state is its bf16 hi part only (the bf16 cached state): half the state
// copies, one state product instead of two. DCH: skip weights per head and channel.
template <int NB, typename Ty, bool HI_ONLY, bool DCH>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_block_bw(BlockArgs a, int hpw, int n_hg)
{
    constexpr int kStateElems = HI_ONLY ? kOpsElems / 2 : kOpsElems;  // one head's state in HBM
    constexpr int TP = 16 * NB;         // padded block length
    constexpr int PBW = NB / 2;         // 16-column blocks per wavefront (4, 2, 1)
    constexpr int PGRP = 4 / PBW;       // column groups per row block
    static_assert(NB * PGRP == kWaves, "one wavefront per (row block, column group)");
    constexpr int XPD = TP / 8;         // 1 KB x copies per direction (8 rows each)
    constexpr int NX = 2 * XPD / kWaves;               // per wavefront
    constexpr int NS = kStateElems * 2 / 1024 / kWaves;  // state copies per wavefront (4, or 2)

    // two buffer sets, by head parity: the next head's state and x stream in while the
    // current one is computed (set 1 first holds the staged B and C rows)
    __shared__ __attribute__((aligned(16))) __bf16 hop0[kOpsElems];  // the head's state
    __shared__ __attribute__((aligned(16))) __bf16 hop1[kOpsElems];
    __shared__ __attribute__((aligned(16))) __bf16 xf0[TP * kP];     // x, forward
    __shared__ __attribute__((aligned(16))) __bf16 xf1[TP * kP];
    __shared__ __attribute__((aligned(16))) __bf16 xr0[TP * kP];     // x, reverse
    __shared__ __attribute__((aligned(16))) __bf16 xr1[TP * kP];
    // each set its own LDS array, chosen at compile time, so that the compiler can tell the
    // copies into one set from the reads of the other
    auto HOP = [&](auto P) -> __bf16 * {
        if constexpr (decltype(P)::value == 0)
            return hop0;
        else
            return hop1;
    };
    auto XF = [&](auto P) -> __bf16 * {
        if constexpr (decltype(P)::value == 0)
            return xf0;
        else
            return xf1;
    };
    auto XR = [&](auto P) -> __bf16 * {
        if constexpr (decltype(P)::value == 0)
            return xr0;
        else
            return xr1;
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    __shared__ __attribute__((aligned(16))) float tab[2][NTAB][TP]; // decay tables, two heads
    __shared__ float skip[2][2];                                     // D, D_rev of those heads
    __shared__ __attribute__((aligned(16))) float skipc[DCH ? 2 : 1][2][DCH ? kP : 1];  // DCH: per channel

    // Workgroups of one stream (and so of its B, C) go to the same XCD: the hardware deals
    // linear workgroup ids round-robin over the 8 XCDs.
    const int nwg = gridDim.x;
    int lid = blockIdx.x;
    if ((nwg & 7) == 0)
        lid = (lid & 7) * (nwg >> 3) + (lid >> 3);
    const int hg = lid % n_hg, b = lid / n_hg;
    const int T = a.T, H = a.s.H, G = a.s.G;
    const int h0 = hg * hpw, g = h0 / (H / G);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, q = lane >> 4, r16 = lane & 15;

    // range-checked buffers over this stream's T tokens: rows past T read as zero and
    // stores to them are dropped
    const int64_t tok0 = static_cast<int64_t>(b) * T;
    const int rowBC = G * kN, rowX = H * kP;
    const int64_t bc0 = tok0 * rowBC + g * kN, bc_bytes = (static_cast<int64_t>(T - 1) * rowBC + kN) * 2;
    const auto rBf = buffer_range(static_cast<const __bf16 *>(a.fwd.B) + bc0, bc_bytes);
    const auto rCf = buffer_range(static_cast<const __bf16 *>(a.fwd.C) + bc0, bc_bytes);
    const auto rBr = buffer_range(static_cast<const __bf16 *>(a.rev.B) + bc0, bc_bytes);
    const auto rCr = buffer_range(static_cast<const __bf16 *>(a.rev.C) + bc0, bc_bytes);
    const int64_t x_bytes = static_cast<int64_t>(T) * rowX * 2;
    const auto rXf = buffer_range(static_cast<const __bf16 *>(a.fwd.x) + tok0 * rowX, x_bytes);
    const auto rXr = buffer_range(static_cast<const __bf16 *>(a.rev.x) + tok0 * rowX, x_bytes);
    const int64_t dt_bytes = static_cast<int64_t>(T) * H * 2;
    const auto rDf = buffer_range(static_cast<const __bf16 *>(a.fwd.dt) + tok0 * H, dt_bytes);
    const auto rDr = buffer_range(static_cast<const __bf16 *>(a.rev.dt) + tok0 * H, dt_bytes);
    const auto rH = buffer_range(static_cast<const __bf16 *>(a.h_ops) + (static_cast<int64_t>(b) * H + h0) * kStateElems,
                                 static_cast<int64_t>(hpw) * kStateElems * 2);
    const auto rY = buffer_range(static_cast<Ty *>(a.y) + tok0 * rowX, static_cast<int64_t>(T) * rowX * sizeof(Ty));

    // ---- copies into LDS. State: this wavefront's NS pieces of head h0 + hh, in place
    // (hh = hpw reads past the range: nothing moves). x: piece k = 8 rows of one direction;
    // lane l takes row 8 (k % XPD) + l / 8, piece (l % 8) ^ swz_x(row) of it, so that the
    // row's piece c sits at slot c ^ swz_x(row); skip = x_bytes puts a copy past the range.
    auto copy_state = [&](auto P, int hh) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int k = w * NS + i;
            copy_to_lds(rH, HOP(P) + k * 512, (hh * kStateElems + k * 512 + 8 * lane) * 2);
        }
    };
    auto copy_x = [&](auto P, int h, int skip_bytes) {
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int k = w * NX + i, d = k / XPD, j = k % XPD;
            const int tr = 8 * j + (lane >> 3), c = (lane & 7) ^ swz_x(tr);
            copy_to_lds(d ? rXr : rXf, (d ? XR(P) : XF(P)) + 8 * j * kP, (tr * rowX + h * kP + 8 * c) * 2 + skip_bytes);
        }
    };

    // ---- decay tables of one direction (lane l holds tokens 2l and 2l+1; dt past T is 0).
    // A table wavefront loads everything its direction needs of a head -- dt, the decay and
    // the skip weight -- ahead of the copies it issues next, so that using them waits for
    // nothing else (memory operations complete in order).
    struct Head {
        unsigned short d0, d1;  // dt of tokens 2 lane, 2 lane + 1
        float A, D;             // decay and skip weight of the direction (D_rev: 0 if none);
                                // DCH: the skip weight of column `lane`
    };
    auto load_head = [&](int dir, int h, Head &hd) {
        const auto r = dir ? rDr : rDf;
        hd.d0 = __builtin_amdgcn_raw_buffer_load_b16(r, (2 * lane * H + h) * 2, 0, 0);
        hd.d1 = __builtin_amdgcn_raw_buffer_load_b16(r, ((2 * lane + 1) * H + h) * 2, 0, 0);
        const float *asrc = dir ? a.A_rev : a.A;  // the reverse scan has its own decay
        hd.A = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_range(asrc, H * 4), h * 4, 0, 0));
        // the reverse skip weight reads 0 when there is none (a zero-byte range): a select on
        // the loaded value would have to wait for the load before the copies that follow
        const float *dsrc = dir ? a.D_rev : a.D;
        if constexpr (DCH)
            hd.D = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 buffer_range(dsrc, dsrc ? H * kP * 4 : 0), (h * kP + lane) * 4, 0, 0));
        else
            hd.D = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 buffer_range(dsrc, dsrc ? H * 4 : 0), h * 4, 0, 0));
        __builtin_amdgcn_sched_barrier(0);  // all of them ahead of the copies that follow
    };
    auto build_tables = [&](int dir, int buf, const Head &hd) {
        const int t0 = 2 * lane, t1 = t0 + 1;
        const float d0 = __uint_as_float(static_cast<uint32_t>(hd.d0) << 16);
        const float d1 = __uint_as_float(static_cast<uint32_t>(hd.d1) << 16);
        const float Aw = hd.A;
        const float a0 = d0 * Aw, a1 = d1 * Aw, loc = a0 + a1;
        const float inc = wave_prefix_sum(loc), excl = inc - loc, total = wave_lane(inc, 63);
        // forward: c_t inclusive prefix sum, reference at the 32-token pair's last token;
        // reverse: r_t inclusive suffix sum, reference at the pair's first token
        const float c0 = dir ? (total - excl) * kLog2e : (excl + a0) * kLog2e;
        const float c1 = dir ? (total - excl - a0) * kLog2e : (excl + loc) * kLog2e;
        const int row = lane >> 4;
        const float f15 = wave_lane(c1, 15), f31 = wave_lane(c1, 31), f47 = wave_lane(c1, 47), f63 = wave_lane(c1, 63);
        const float g00 = wave_lane(c0, 0), g16 = wave_lane(c0, 16), g32 = wave_lane(c0, 32), g48 = wave_lane(c0, 48);
        const float reff = row == 0 ? f15 : row == 1 ? f31 : row == 2 ? f47 : f63;
        const float refr = row == 0 ? g00 : row == 1 ? g16 : row == 2 ? g32 : g48;
        const float ref = dir ? refr : reff;
        if (t0 < TP) {
            float *cc = tab[buf][dir ? TAB_CR : TAB_CF];
            float *lg = tab[buf][dir ? TAB_LGR : TAB_LGF];
            float *col = tab[buf][dir ? TAB_COLR : TAB_COLF];
            cc[t0] = c0;
            cc[t1] = c1;
            lg[t0] = __builtin_amdgcn_logf(d0) - c0;
            lg[t1] = __builtin_amdgcn_logf(d1) - c1;
            col[t0] = __builtin_amdgcn_exp2f(ref - c0) * d0;
            col[t1] = __builtin_amdgcn_exp2f(ref - c1) * d1;
            if (dir == 0) {
                tab[buf][TAB_EF][t0] = __builtin_amdgcn_exp2f(c0);
                tab[buf][TAB_EF][t1] = __builtin_amdgcn_exp2f(c1);
            }
        }
        if constexpr (DCH)
            skipc[buf][dir][lane] = hd.D;
        else
            skip[buf][dir] = hd.D;  // every lane (a branch would delay the load to here)
    };

    // Rows past T: their copies read past the range and may leave the LDS rows as they
    // were. Weighted 0 they must still be finite, so with a short block the buffers are
    // cleared once, before any copy (later contents are always finite inputs).
    if (T < TP) {
        const uint4 z = make_uint4(0, 0, 0, 0);
        for (int i = threadIdx.x; i < kOpsElems / 8; i += 64 * kWaves) {
            *reinterpret_cast<uint4 *>(hop0 + 8 * i) = z;
            *reinterpret_cast<uint4 *>(hop1 + 8 * i) = z;
        }
        for (int i = threadIdx.x; i < TP * kP / 8; i += 64 * kWaves) {
            *reinterpret_cast<uint4 *>(xf0 + 8 * i) = z;
            *reinterpret_cast<uint4 *>(xr0 + 8 * i) = z;
            *reinterpret_cast<uint4 *>(xf1 + 8 * i) = z;
            *reinterpret_cast<uint4 *>(xr1 + 8 * i) = z;
        }
        workgroup_lds_barrier<63>();
    }

    // ---- B and C rows for the score tiles, staged in LDS before the first head's copies
    // (a matrix-core operand read straight from a row-major tensor touches 16 rows for 64
    // bytes per load, which costs the load path several times what whole lines cost). Rows
    // of N = 128 bf16 in blocks of 16, piece c (8 elements) of row r at slot c ^ (r % 16);
    // C rows go to the state buffer of set 1, B rows to its two x buffers (TP/2 rows each),
    // while the first head's state and x land in set 0.
    constexpr int RPW = TP / 4 / kWaves;  // 1 KB pieces (4 rows) of one tensor per wavefront
    auto copy_rows = [&](__amdgpu_buffer_rsrc_t r, __bf16 *lo_half, __bf16 *hi_half, int k) {
        const int row = 4 * k + (lane >> 4), c = (lane & 15) ^ (row & 15);
        __bf16 *dst = (4 * k < TP / 2 ? lo_half + 4 * k * kN : hi_half + (4 * k - TP / 2) * kN);
        copy_to_lds(r, dst, (row * rowBC + 8 * c) * 2);
    };
    auto copy_bc = [&](int dir) {  // C -> hop1, B -> xf1 | xr1
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            copy_rows(dir ? rCr : rCf, hop1, hop1 + (TP / 2) * kN, w * RPW + i);
            copy_rows(dir ? rBr : rBf, xf1, xr1, w * RPW + i);
        }
    };
    // operand fragment of row 16 blk + r16 of the staged rows: n = 32 kk + 8 q .. +7
    auto row_frag = [&](const __bf16 *lo_half, const __bf16 *hi_half, int blk, int kk) {
        const __bf16 *base = 16 * blk < TP / 2 ? lo_half + 16 * blk * kN : hi_half + (16 * blk - TP / 2) * kN;
        return *reinterpret_cast<const bf16x8 *>(base + 8 * (16 * r16 + ((4 * kk + q) ^ r16)));
    };

    // x operand of M X, pair m of 32 tokens, 16-column block starting at pcol: lane (r16, q)
    // gets column pcol + r16 of tokens 32m + 4q + e (slots 0..3) and 32m + 16 + 4q + e (4..7)
    auto xfrag = [&](const __bf16 *X, int m, int pcol) {
        const int tr = 32 * m + 4 * q + (r16 >> 2), col = pcol + 4 * (r16 & 3);
        const int off = 8 * ((col >> 3) ^ swz_x(tr)) + (col & 7);
        return cat(tr_read(&X[tr * kP + off]), tr_read(&X[(tr + 16) * kP + off]));
    };

    auto body = [&](auto Wc) {
        constexpr int TB = decltype(Wc)::value / PGRP, pgrp = decltype(Wc)::value % PGRP;
        constexpr int MD = TB / 2;                // the 32-token pair holding row block TB
        // table wavefronts: row block 0 forward, row block 1 reverse (column group 0)
        constexpr int DIR = TB < 2 && pgrp == 0 ? TB : -1;
        constexpr bool table_wave = DIR >= 0;
        const int t = 16 * TB + r16;              // this lane's token as an operand row/column

        Head hd{0, 0, 0.f, 0.f};
        if constexpr (table_wave)
            load_head(DIR, h0, hd);
        copy_state(P0{}, 0);
        copy_x(P0{}, h0, 0);

        // ---- score tiles of this row block, once per workgroup: S[ut] lane (r16, q) holds
        // S[t = 16 TB + r16][s = 16 sb + 4q + j]; forward tiles (s-blocks 0..TB) from the
        // staged forward rows, then reverse tiles (s-blocks TB..NB-1) from the reverse rows
        f32x4 S[NB + 1];
        bf16x8 cfw[4];  // C_t fragments, kept for the cached-state term
        copy_bc(0);
        workgroup_lds_barrier<0>();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            cfw[kk] = row_frag(hop1, hop1 + (TP / 2) * kN, TB, kk);
#pragma unroll
        for (int ut = 0; ut <= TB; ++ut) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = mfma(row_frag(xf1, xr1, ut, kk), cfw[kk], acc);
            S[ut] = acc;
        }
        if constexpr (table_wave)
            build_tables(DIR, 0, hd);
        workgroup_lds_barrier<63>();  // everyone's reads of the forward rows are done
        copy_bc(1);
        workgroup_lds_barrier<0>();
        {
            bf16x8 crv[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                crv[kk] = row_frag(hop1, hop1 + (TP / 2) * kN, TB, kk);
#pragma unroll
            for (int ut = TB + 1; ut <= NB; ++ut) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    acc = mfma(row_frag(xf1, xr1, ut - 1, kk), crv[kk], acc);
                S[ut] = acc;
            }
        }

        // one head: its state, x and tables are in set P (copied during the head before); the
        // next head's go to the other set while this one is computed. No branch on the copies'
        // path (after the last head the next head's copies move nothing and its tables are
        // rebuilt for the last one), so that the compiler's waits count exactly the loads and
        // copies in flight.
        auto head = [&](auto P, int hh) {
            constexpr int cur = decltype(P)::value;
            using PN = std::integral_constant<int, 1 - cur>;
            const int h = h0 + hh;
            const bool more = hh + 1 < hpw;
            const int hn = more ? h + 1 : h;
            // the head's copies are in, and every read of the other set (the head before) is
            // done. Memory operations complete in order and the last PBW of this wavefront are
            // the head before's y stores (issued after the copies): those may still be in
            // flight (before the first head, nothing is)
            workgroup_lds_barrier<PBW>();
            if constexpr (table_wave)
                load_head(DIR, hn, hd);
            copy_state(PN{}, hh + 1);
            copy_x(PN{}, hn, more ? 0 : static_cast<int>(x_bytes));
            __builtin_amdgcn_sched_barrier(0);  // the copies stay ahead of the y stores
            const __bf16 *hop = HOP(P);
            const __bf16 *xs0 = XF(P);
            const __bf16 *xs1 = XR(P);
            // eq. (11), cached-state term: y^T = (h_hi + h_lo)^T C^T; the state fragments of
            // contraction block kk + 1 are read while those of kk are multiplied
            constexpr int NH = HI_ONLY ? 1 : 2;  // hi (, lo)
            f32x4 acc[PBW];
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb)
                acc[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
            bf16x8 hf[2][PBW][NH];
            auto read_h = [&](int kk, bf16x8 (&dst)[PBW][NH]) {
#pragma unroll
                for (int pb = 0; pb < PBW; ++pb) {
                    const int pc = (pgrp * PBW + pb) * 16 + r16;
#pragma unroll
                    for (int e = 0; e < NH; ++e)
                        dst[pb][e] = *reinterpret_cast<const bf16x8 *>(&hop[((16 * e + 4 * kk + q) * kP + pc) * 8]);
                }
            };
            read_h(0, hf[0]);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk + 1 < 4)
                    read_h(kk + 1, hf[(kk + 1) & 1]);
#pragma unroll
                for (int pb = 0; pb < PBW; ++pb)
#pragma unroll
                    for (int e = 0; e < NH; ++e)
                        acc[pb] = mfma(hf[kk & 1][pb][e], cfw[kk], acc[pb]);
            }
            {
                const float et = tab[cur][TAB_EF][t];  // exp(c_t)
#pragma unroll
                for (int pb = 0; pb < PBW; ++pb)
                    acc[pb] *= et;
            }
            // x fragments of the M X rounds: forward pairs m = 0 .. MD, then reverse pairs
            // m = MD .. NB/2 - 1; round r + 1's are read while round r is weighted and multiplied
            constexpr int NRF = MD + 1, NR = NRF + NB / 2 - MD;
            bf16x8 xq[2][PBW];
            auto read_x = [&](int r, bf16x8 (&dst)[PBW]) {
                const __bf16 *X = r < NRF ? xs0 : xs1;
                const int m = r < NRF ? r : MD + (r - NRF);
#pragma unroll
                for (int pb = 0; pb < PBW; ++pb)
                    dst[pb] = xfrag(X, m, (pgrp * PBW + pb) * 16);
            };
            read_x(0, xq[0]);
            int rnd = 0;
            auto mx = [&](const bf16x8 &af, const __bf16 *, int) {
                const int cur_r = rnd;
                if (cur_r + 1 < NR)
                    read_x(cur_r + 1, xq[(cur_r + 1) & 1]);
#pragma unroll
                for (int pb = 0; pb < PBW; ++pb)
                    acc[pb] = mfma(xq[cur_r & 1][pb], af, acc[pb]);
                ++rnd;
            };
            const float *cf = tab[cur][TAB_CF], *cr = tab[cur][TAB_CR], *lgf = tab[cur][TAB_LGF],
                        *lgr = tab[cur][TAB_LGR], *colf = tab[cur][TAB_COLF], *colr = tab[cur][TAB_COLR];
            // eq. (11), inside the block (s <= t). Pairs wholly below the row block use the
            // factored decay exp2(c_t - c_ref) * [exp2(c_ref - c_s) dt_s], c_ref = c at the
            // pair's last token (both factors <= 1); the pair holding the row block uses
            // exp2(c_t - c_s + log2 dt_s) per element, masked to s <= t.
            const float ctf = cf[t];
#pragma unroll
            for (int m = 0; m <= MD; ++m) {
                float mv[8];
                if (m < MD) {
                    const float rowf = __builtin_amdgcn_exp2f(ctf - cf[32 * m + 31]);
                    const float4 c0 = *reinterpret_cast<const float4 *>(&colf[32 * m + 4 * q]);
                    const float4 c1 = *reinterpret_cast<const float4 *>(&colf[32 * m + 16 + 4 * q]);
                    const float cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        mv[j] = (j < 4 ? S[2 * m][j] : S[2 * m + 1][j & 3]) * cw[j] * rowf;
                } else {
                    const float4 l0 = *reinterpret_cast<const float4 *>(&lgf[32 * m + 4 * q]);
                    const float4 l1 = *reinterpret_cast<const float4 *>(&lgf[32 * m + 16 + 4 * q]);
                    const float lg[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                    constexpr bool hi_ok = 2 * MD + 1 <= TB;  // here m == MD
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int s = 32 * m + (j < 4 ? 0 : 16) + 4 * q + (j & 3);
                        const float sv = j < 4 ? S[2 * m][j] : (hi_ok ? S[2 * m + 1][j & 3] : 0.f);
                        const float wgt = __builtin_amdgcn_exp2f(ctf + lg[j]);
                        mv[j] = s <= t ? sv * wgt : 0.f;
                    }
                }
                mx(to_bf16x8(mv), xs0, m);
            }
            // eq. (12), reverse inside the block (s >= t); pairs wholly above the row block
            // use the factored decay with the reference at the pair's first token
            const float ctr = cr[t];
#pragma unroll
            for (int m = MD; m < NB / 2; ++m) {
                float mv[8];
                if (m > MD) {
                    const float rowr = __builtin_amdgcn_exp2f(ctr - cr[32 * m]);
                    const float4 c0 = *reinterpret_cast<const float4 *>(&colr[32 * m + 4 * q]);
                    const float4 c1 = *reinterpret_cast<const float4 *>(&colr[32 * m + 16 + 4 * q]);
                    const float cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        mv[j] = (j < 4 ? S[2 * m + 1][j] : S[2 * m + 2][j & 3]) * cw[j] * rowr;
                } else {
                    const float4 l0 = *reinterpret_cast<const float4 *>(&lgr[32 * m + 4 * q]);
                    const float4 l1 = *reinterpret_cast<const float4 *>(&lgr[32 * m + 16 + 4 * q]);
                    const float lg[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                    constexpr bool lo_ok = 2 * MD >= TB;  // here m == MD
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int s = 32 * m + (j < 4 ? 0 : 16) + 4 * q + (j & 3);
                        const float sv = j < 4 ? (lo_ok ? S[2 * m + 1][j] : 0.f) : S[2 * m + 2][j & 3];
                        const float wgt = __builtin_amdgcn_exp2f(ctr + lg[j]);
                        mv[j] = s >= t ? sv * wgt : 0.f;
                    }
                }
                mx(to_bf16x8(mv), xs1, m);
            }
            // the next head's decay tables (its inputs were loaded before the state copies)
            if constexpr (table_wave)
                build_tables(DIR, cur ^ 1, hd);
            // eq. (13) + D x (+ D_rev x_rev), written once: the lane holds y[t][p0 .. p0+3] of
            // each of its column blocks and stores it as one 8- (bf16) or 16-byte (fp32) piece
            const float Dh = skip[cur][0], Dr = skip[cur][1];
            const bool with_dr = a.D_rev != nullptr;
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb) {
                const int p0 = (pgrp * PBW + pb) * 16 + 4 * q;
                const int xo = t * kP + 8 * ((p0 >> 3) ^ swz_x(t)) + (p0 & 7);
                const bf16x4 xf = *reinterpret_cast<const bf16x4 *>(&xs0[xo]);
                const bf16x4 xr = *reinterpret_cast<const bf16x4 *>(&xs1[xo]);
                float o[4];
                if constexpr (DCH) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float v = fmaf(skipc[cur][0][p0 + j], bf2f(xf[j]), acc[pb][j]);
                        o[j] = with_dr ? fmaf(skipc[cur][1][p0 + j], bf2f(xr[j]), v) : v;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float v = fmaf(Dh, bf2f(xf[j]), acc[pb][j]);
                        o[j] = with_dr ? fmaf(Dr, bf2f(xr[j]), v) : v;
                    }
                }
                const int off = (t * rowX + h * kP + p0) * static_cast<int>(sizeof(Ty));
                if constexpr (sizeof(Ty) == 2) {
                    bf16x4 ov;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        ov[j] = static_cast<__bf16>(o[j]);
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u32, ov), rY, off, 0, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b128(
                        v4u32{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])},
                        rY, off, 0, 0);
                }
            }
        };
        int hh = 0;
        for (; hh + 2 <= hpw; hh += 2) {
            head(P0{}, hh);
            head(P1{}, hh + 1);
        }
        if (hh < hpw)
            head(P0{}, hh);
        // no copy into this workgroup's LDS may still be in flight when it ends
        __builtin_amdgcn_s_waitcnt(0);
    };
    // one specialization per wavefront
    switch (w) {
    case 0: body(std::integral_constant<int, 0>{}); break;
    case 1: body(std::integral_constant<int, 1>{}); break;
    case 2: body(std::integral_constant<int, 2>{}); break;
    case 3: body(std::integral_constant<int, 3>{}); break;
    case 4: body(std::integral_constant<int, 4>{}); break;
    case 5: body(std::integral_constant<int, 5>{}); break;
    case 6: body(std::integral_constant<int, 6>{}); break;
    default: body(std::integral_constant<int, 7>{}); break;
    }
}

template <int NB, typename Ty>
hipError_t launch_nb(const BlockArgs &a, int hpw, hipStream_t st)
{
    const int n_hg = a.s.H / hpw;
    const int nwg = a.s.b * n_hg;
    const dim3 grid(nwg), block(64 * kWaves);
    if (a.ops_hi_only)
        a.d_per_channel ? k_block_bw<NB, Ty, true, true><<<grid, block, 0, st>>>(a, hpw, n_hg)
                        : k_block_bw<NB, Ty, true, false><<<grid, block, 0, st>>>(a, hpw, n_hg);
    else
        a.d_per_channel ? k_block_bw<NB, Ty, false, true><<<grid, block, 0, st>>>(a, hpw, n_hg)
                        : k_block_bw<NB, Ty, false, false><<<grid, block, 0, st>>>(a, hpw, n_hg);
    return hipGetLastError();
}

template <typename Ty>
hipError_t launch_ty(const BlockArgs &a, int hpw, hipStream_t st)
{
    if (a.T <= 32)
        return launch_nb<2, Ty>(a, hpw, st);
    if (a.T <= 64)
        return launch_nb<4, Ty>(a, hpw, st);
    return launch_nb<8, Ty>(a, hpw, st);
}

}  // namespace

bool block_bw_supported(const Shape &s, int T)
{
    // byte ranges of the per-stream buffers must fit the 32-bit range of a buffer resource
    return s.in_dt == 1 && s.N == kN && s.P == kP && T >= 1 && T <= 128 &&
           static_cast<int64_t>(T) * s.H * kP * 4 < (int64_t(1) << 31) &&
           static_cast<int64_t>(s.H) * kOpsElems * 2 < (int64_t(1) << 31);
}

int block_bw_plan(const Shape &s)
{
    // heads per workgroup: the largest divisor of the heads per group that still leaves a
    // workgroup for every CU (one per CU: 256), so that the score tiles are shared by as many
    // heads as possible without idling CUs
    const int hpg = s.H / s.G;
    const int64_t pairs = static_cast<int64_t>(s.b) * s.H;
    const int64_t want = static_cast<int64_t>(device_cus());
    int best = 1;
    for (int d = 1; d <= hpg; ++d) {
        if (hpg % d == 0 && pairs / d >= want)
            best = d;
    }
    return best;
}

hipError_t launch_block_step_bw(const BlockArgs &a, int hpw, hipStream_t st)
{
    return a.s.y_dt ? launch_ty<__bf16>(a, hpw, st) : launch_ty<float>(a, hpw, st);
}

}  // namespace bdssm
