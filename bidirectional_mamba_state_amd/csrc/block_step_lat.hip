// Block step for small batches: the same computation as block_step_mfma.hip (eqs. (11)-(13)
// of "Training Hybrid Block Diffusion Language Models with Partial Bidirectionality" in the
// matrix form of the Mamba-2 scan), laid out for latency instead of bandwidth.
//
// With few (stream, head) pairs a launch has about one wavefront per SIMD, and its time is
// the length of one wavefront's chain of dependent steps, not the bytes it moves. A
// workgroup owns one (head, 16-token row block) and its four wavefronts one 16-column
// block each. What dominates that chain is getting the inputs in: a load whose 64 lanes
// touch 16 rows for 64 bytes each costs the L1 several times what the same bytes cost in
// whole 128-byte lines, and the matrix-core operand layouts are of that first kind. So
// every input the workgroup needs -- the B and C rows of its score tiles, the cached fp32
// state of the head and x of both directions -- is copied once, in whole lines, straight
// into LDS (gfx950 buffer loads to LDS, no registers on the way; 19 loads per wavefront,
// each wavefront a quarter of each tile), with the 16-byte pieces of each row permuted
// so that the operand reads that follow are free of bank conflicts:
//   - B and C rows as A/B operands of the C B^T score tiles (16-byte reads);
//   - the state as the B operand of C . h: lane (column p, quarter q) reads h[32k + 8q + e][p],
//     e = 0..7, and splits it into bf16 hi + lo parts in registers (two products, ~16
//     significant bits);
//   - x as the B operand of M X by transposing reads (gfx950 ds_read_b64_tr_b16), giving
//     each lane the tokens of its slots (4q + e, 16 + 4q + e) in its column; the same
//     registers give D x.
// The cumulative log-decays of both directions are a 64-lane DPP scan that every wavefront
// computes for itself into its own small table. The copies are issued in the order of use,
// the state last: after a barrier for B, C and x the score tiles and M X run while the
// state still arrives, and a second barrier precedes C . h; y leaves straight from the
// accumulators. Loads and stores go through range-checked
// buffer resources over the stream's T tokens, so rows past T read as zero and their
// stores are dropped (LDS rows past T are cleared in a branch taken only for short blocks).
#include <type_traits>

#include "internal.h"
#include "mfma_tiles.h"
#include "wave_ops.h"

namespace bdssm {
namespace {

constexpr int kN = 128, kP = 64;
constexpr float kLog2e = 1.4426950408889634f;

// LDS tiles, each filled by whole-line copies (a load that touches few lines in full costs
// the L1 several times less than one that touches many in part), with the 16-byte pieces
// of a row permuted (an XOR of the piece index) so that the operand reads below fall in
// distinct banks:
//   row block: 16 rows of N = 128 bf16 (B or C), piece c of row r at slot c ^ r;
//   state:     N x (the workgroup's 32 or 64 columns) fp32; with 32, row n at LDS row
//              n ^ ((n / 16) % 2) and piece c (4 columns) at slot c ^ 4 ((n / 8) % 2); with
//              64, row n in place and piece c at slot c ^ 4 ((n / 8) % 4);
//   x:         T x P bf16 per direction, piece c (8 columns) of row t at slot c ^ 2 (t % 4);
//   state in operand form (OPS): [hi, lo][N/8][the workgroup's columns][8] bf16 as stored,
//              a lane's operand one 16-byte read, consecutive lanes consecutive pieces.
constexpr int kRowBlk = 16 * 128;

// Operand fragment of row r16 of a row block: n = 32 kk + 8 q .. +7
__device__ __forceinline__ bf16x8 rows_frag(const __bf16 *blk, int kk, int q, int r16)
{
    return *reinterpret_cast<const bf16x8 *>(blk + 8 * (16 * r16 + ((4 * kk + q) ^ r16)));
}

enum { TAB_CF, TAB_CR, TAB_LGF, TAB_LGR, TAB_COLF, TAB_COLR, TAB_EF, NTAB };

// WPG wavefronts per workgroup (2 or 4), each owning one 16-column block of the outputs;
// FORM: the cached state as float32 (0), in operand form (1, k_state_ops) or as its bf16 hi
// part only (2, the bf16 cached state: half the bytes, one product instead of two);
// DCH: skip weights per head and channel ([H][P]) instead of per head
enum { FORM_F32 = 0, FORM_OPS = 1, FORM_BF16 = 2 };
template <typename Ty, int WPG, int FORM, bool DCH>
__global__ __launch_bounds__(64 * WPG) void k_block_lat(BlockArgs a)
{
    constexpr bool OPS = FORM != FORM_F32;
    constexpr int NB = 2, TP = 32;  // one 32-token pair: two 16-token row blocks
    constexpr int CW = 16 * WPG;    // the workgroup's columns
    constexpr int NPH = kP / CW;    // column parts of a head
    // C rows of the row block (forward, reverse), then B rows of its three score tiles
    __shared__ __attribute__((aligned(16))) __bf16 rows[NB + 3][kRowBlk];
    __shared__ __attribute__((aligned(16))) float hst[kN * CW];        // the state, CW columns
    __bf16 *const hops = reinterpret_cast<__bf16 *>(hst);               // ... in operand form
    __shared__ __attribute__((aligned(16))) __bf16 xs[2][TP * kP];      // x, both directions
    __shared__ __attribute__((aligned(16))) float tab[NTAB][TP];        // decay tables

    // every kernel argument the first copies need, loaded in one round: left to itself the
    // compiler loads some of them behind the index arithmetic's branches, a round trip each
    asm volatile("" ::"s"(a.T), "s"(a.s.H), "s"(a.s.G), "s"(a.fwd.x), "s"(a.fwd.dt), "s"(a.fwd.B), "s"(a.fwd.C),
                 "s"(a.rev.x), "s"(a.rev.dt), "s"(a.rev.B), "s"(a.rev.C), "s"(OPS ? a.h_ops : a.h_prefix),
                 "s"(gridDim.x));
    const int T = a.T, H = a.s.H, G = a.s.G;
    // workgroup = (head, row block, column part), grid.y = stream. The hardware deals
    // workgroup ids round-robin over the 8 XCDs; the workgroups of a head read the same B, C
    // and x, so they get consecutive logical ids within one XCD's range and share its L2.
    const int nx = gridDim.x;
    const int wid = (nx & 7) == 0 ? static_cast<int>((blockIdx.x & 7) * (nx >> 3) + (blockIdx.x >> 3))
                                  : static_cast<int>(blockIdx.x);
    const int ph = wid % NPH, tb = (wid / NPH) & 1, h = wid / (2 * NPH), b = blockIdx.y;
    const int g = G == 1 ? 0 : h / (H / G);
    // wavefront w = 16-column block WPG ph + w of the outputs (uniform, so that LDS copy
    // addresses are scalar)
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pblk = WPG * ph + w;
    const int lane = threadIdx.x & 63, q = lane >> 4, r16 = lane & 15;
    const int t = tb * 16 + r16;  // this lane's row as an A operand

    // range-checked buffers over this stream's T tokens: rows past T read as zero
    const int64_t tok0 = static_cast<int64_t>(b) * T;
    const int rowBC = G * kN, rowX = H * kP;
    const int64_t bc_bytes = (static_cast<int64_t>(T - 1) * rowBC + kN) * 2;
    const int64_t bc0 = tok0 * rowBC + g * kN;
    const auto rBf = buffer_range(static_cast<const __bf16 *>(a.fwd.B) + bc0, bc_bytes);
    const auto rCf = buffer_range(static_cast<const __bf16 *>(a.fwd.C) + bc0, bc_bytes);
    const auto rBr = buffer_range(static_cast<const __bf16 *>(a.rev.B) + bc0, bc_bytes);
    const auto rCr = buffer_range(static_cast<const __bf16 *>(a.rev.C) + bc0, bc_bytes);
    const int64_t x0 = tok0 * rowX + h * kP;
    const int64_t x_bytes = (static_cast<int64_t>(T - 1) * rowX + kP) * 2;
    const auto rXf = buffer_range(static_cast<const __bf16 *>(a.fwd.x) + x0, x_bytes);
    const auto rXr = buffer_range(static_cast<const __bf16 *>(a.rev.x) + x0, x_bytes);
    const int64_t dt_bytes = (static_cast<int64_t>(T - 1) * H + 1) * 2;
    const auto rDf = buffer_range(static_cast<const __bf16 *>(a.fwd.dt) + tok0 * H + h, dt_bytes);
    const auto rDr = buffer_range(static_cast<const __bf16 *>(a.rev.dt) + tok0 * H + h, dt_bytes);
    const int64_t bh = static_cast<int64_t>(b) * H + h;
    constexpr int OPS_PARTS = FORM == FORM_BF16 ? 1 : 2;  // bf16 halves per state element
    const auto rH = OPS ? buffer_range(static_cast<const __bf16 *>(a.h_ops) + bh * (OPS_PARTS * kN * kP),
                                       OPS_PARTS * kN * kP * 2)
                        : buffer_range(a.h_prefix + bh * (kN * kP), kN * kP * 4);

    // ---- the workgroup's inputs, each byte copied once, in whole lines, straight into
    // LDS, in the order of use: B and C (score tiles), x (M X), the state (C . h) last, so
    // that the first products overlap the state's arrival. The 28 pieces of B, C and x
    // (1 KB each) are dealt to all wavefronts but the last, which loads dt and builds the
    // decay tables for the workgroup meanwhile (with two wavefronts, it copies x); every
    // wavefront then copies its eighth (WPG = 2) or quarter (4) of the state.
    constexpr int TW = WPG - 1;  // the wavefront that builds the tables
    constexpr int NSTATE = FORM == FORM_BF16 ? 4 : 8;  // state copies per wavefront, its last loads
    auto row0_of = [&](int i) {  // first row of row block i
        return i < 2 ? tb * 16 : (i - 2 <= tb ? i - 2 : i - 3) * 16;
    };
    // piece k < 20: rows 4 (k % 4) .. +3 of row block k / 4; k < 28: x rows 8 (k % 4) .. +7 of
    // direction (k - 20) / 4. Rows past T: zeroed in LDS after the copy has landed.
    auto copy_piece = [&](int k) {
        if (k < 20) {
            const int i = k / 4, j = k % 4;
            const auto r = i == 0 ? rCf : i == 1 ? rCr : (i - 2 <= tb ? rBf : rBr);
            const int rl = 4 * j + (lane >> 4), piece = (lane & 15) ^ rl;
            copy_to_lds(r, &rows[i][4 * j * 128], ((row0_of(i) + rl) * rowBC + 8 * piece) * 2);
        } else {
            const int d = (k - 20) / 4, j = (k - 20) % 4;
            const int tr = 8 * j + (lane >> 3), c = (lane & 7) ^ swz_x(tr);
            copy_to_lds(d ? rXr : rXf, &xs[d][8 * j * kP], (tr * rowX + 8 * c) * 2);
        }
    };
    auto clear_piece = [&](int k) {
        const uint4 z = make_uint4(0, 0, 0, 0);
        if (k < 20) {
            const int i = k / 4, j = k % 4;
            if (row0_of(i) + 4 * j + (lane >> 4) >= T)
                *reinterpret_cast<uint4 *>(&rows[i][4 * j * 128 + 8 * lane]) = z;
        } else {
            const int d = (k - 20) / 4, j = (k - 20) % 4;
            if (8 * j + (lane >> 3) >= T)
                *reinterpret_cast<uint4 *>(&xs[d][8 * j * kP + 8 * lane]) = z;
        }
    };
    // pieces [lo, hi) of wavefront W: WPG = 2: B and C | x; WPG = 4: half of B and C each
    // for 0 and 1, x for 2, none for 3
    auto for_pieces = [&](auto W, auto fn) {
        constexpr int w_ = decltype(W)::value;
        constexpr int lo = WPG == 2 ? (w_ == 0 ? 0 : 20) : (w_ < 2 ? 10 * w_ : w_ == 2 ? 20 : 28);
        constexpr int hi = WPG == 2 ? (w_ == 0 ? 20 : 28) : (w_ < 2 ? 10 * w_ + 10 : 28);
#pragma unroll
        for (int k = lo; k < hi; ++k)
            fn(k);
    };
    auto by_wave = [&](auto fn) {  // fn(integral_constant<w>) for this wavefront's w
        if (w == 0)
            fn(std::integral_constant<int, 0>{});
        else if (w == 1)
            fn(std::integral_constant<int, 1>{});
        else if (WPG == 4 && w == 2)
            fn(std::integral_constant<int, 2>{});
        else if (WPG == 4)
            fn(std::integral_constant<int, 3>{});
    };
    const int t0 = 2 * lane, t1 = t0 + 1;
    // the head's decays and skip weights, read by vector loads issued first in each
    // wavefront's prologue: as scalar loads, the wait that the first copies need for the
    // kernel arguments would also wait for them
    float Ah = 0.f, Dh = 0.f, Ar = 0.f, Dr = 0.f;
    f32x4 Dc = {0.f, 0.f, 0.f, 0.f}, Drc = {0.f, 0.f, 0.f, 0.f};  // DCH: this lane's four columns
    auto load_params = [&](bool decays) {
        if constexpr (DCH) {
            const int pc = 16 * pblk + 4 * q;
            Dc = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(buffer_range(a.D, H * kP * 4),
                                                                                 (h * kP + pc) * 4, 0, 0));
            Drc = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                buffer_range(a.D_rev, a.D_rev ? H * kP * 4 : 0), (h * kP + pc) * 4, 0, 0));
        } else {
            Dh = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_range(a.D, H * 4), h * 4, 0, 0));
            Dr = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_range(a.D_rev, a.D_rev ? H * 4 : 0), h * 4, 0, 0));
        }
        if (decays) {
            Ah = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_range(a.A, H * 4), h * 4, 0, 0));
            Ar = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_range(a.A_rev, H * 4), h * 4, 0, 0));
        }
    };
    auto copy_state = [&]() {  // this wavefront's NSTATE state pieces
#pragma unroll
        for (int m = NSTATE * w; m < NSTATE * w + NSTATE; ++m) {  // LDS state rows 8 m .. 8 m + 7
            if constexpr (OPS) {  // operand rows (hi/lo, n/8) RPC m .. RPC m + RPC - 1, CW pieces each
                constexpr int RPC = 64 / CW;
                const int row = RPC * m + lane / CW, col = lane % CW;
                copy_to_lds(rH, &hops[RPC * m * CW * 8], (row * kP + CW * ph + col) * 16);
            } else if constexpr (WPG == 2) {                       // (32 columns) or 4 m .. 4 m + 3
                const int lr = 8 * m + (lane >> 3), n = lr ^ ((lr >> 4) & 1), c = (lane & 7) ^ (4 * ((n >> 3) & 1));
                copy_to_lds(rH, &hst[8 * m * CW], (n * kP + CW * ph + 4 * c) * 4);
            } else {
                const int n = 4 * m + (lane >> 4), c = (lane & 15) ^ (4 * ((n >> 3) & 3));
                copy_to_lds(rH, &hst[4 * m * CW], (n * kP + 4 * c) * 4);
            }
        }
    };

    // ---- decay tables of both directions (lane l holds tokens 2l and 2l+1; dt past T is 0),
    // built once for the workgroup
    float(*tb_)[TP] = tab;
    auto build_tables = [&](const unsigned short (&dt4)[4]) {  // dt of tokens t0, t1 (fwd, rev)
        const float f0 = __uint_as_float(static_cast<uint32_t>(dt4[0]) << 16);
        const float f1 = __uint_as_float(static_cast<uint32_t>(dt4[1]) << 16);
        const float g0 = __uint_as_float(static_cast<uint32_t>(dt4[2]) << 16);
        const float g1 = __uint_as_float(static_cast<uint32_t>(dt4[3]) << 16);
        // forward: c_t inclusive prefix sum; reference at the pair's last token (lane 15)
        const float a0 = f0 * Ah, a1 = f1 * Ah, loc = a0 + a1;
        const float inc = wave_prefix_sum(loc), excl = inc - loc;
        const float c0 = (excl + a0) * kLog2e, c1 = (excl + loc) * kLog2e;
        // reverse: r_t inclusive suffix sum; reference at the pair's first token (lane 0)
        const float b0 = g0 * Ar, b1 = g1 * Ar, locr = b0 + b1;
        const float incr = wave_prefix_sum(locr), exclr = incr - locr, totr = wave_lane(incr, 63);
        const float r0 = (totr - exclr) * kLog2e, r1 = (totr - exclr - b0) * kLog2e;
        const float reff = wave_lane(c1, 15), refr = wave_lane(r0, 0);
        if (t0 < TP) {
            tb_[TAB_CF][t0] = c0;
            tb_[TAB_CF][t1] = c1;
            tb_[TAB_CR][t0] = r0;
            tb_[TAB_CR][t1] = r1;
            tb_[TAB_LGF][t0] = __builtin_amdgcn_logf(f0) - c0;
            tb_[TAB_LGF][t1] = __builtin_amdgcn_logf(f1) - c1;
            tb_[TAB_LGR][t0] = __builtin_amdgcn_logf(g0) - r0;
            tb_[TAB_LGR][t1] = __builtin_amdgcn_logf(g1) - r1;
            tb_[TAB_COLF][t0] = __builtin_amdgcn_exp2f(reff - c0) * f0;
            tb_[TAB_COLF][t1] = __builtin_amdgcn_exp2f(reff - c1) * f1;
            tb_[TAB_COLR][t0] = __builtin_amdgcn_exp2f(refr - r0) * g0;
            tb_[TAB_COLR][t1] = __builtin_amdgcn_exp2f(refr - r1) * g1;
            tb_[TAB_EF][t0] = __builtin_amdgcn_exp2f(c0);
            tb_[TAB_EF][t1] = __builtin_amdgcn_exp2f(c1);
        }
    };
    // each wavefront's prologue, specialized per wavefront so that every wait counts exactly
    // the loads it must (and no wavefront holds loads it does not use): the table wavefront
    // loads dt first; then its B, C or x pieces; then (table wavefront) the tables; then its
    // state pieces. Its pieces have landed once at most the state copies are in flight.
    by_wave([&](auto W) {
        constexpr bool table_wave = decltype(W)::value == TW;
        unsigned short dt4[4] = {0, 0, 0, 0};
        load_params(table_wave);
        if constexpr (table_wave) {
            dt4[0] = __builtin_amdgcn_raw_buffer_load_b16(rDf, t0 * H * 2, 0, 0);
            dt4[1] = __builtin_amdgcn_raw_buffer_load_b16(rDf, t1 * H * 2, 0, 0);
            dt4[2] = __builtin_amdgcn_raw_buffer_load_b16(rDr, t0 * H * 2, 0, 0);
            dt4[3] = __builtin_amdgcn_raw_buffer_load_b16(rDr, t1 * H * 2, 0, 0);
        }
        for_pieces(W, copy_piece);
        if constexpr (table_wave)
            build_tables(dt4);
        copy_state();
        __builtin_amdgcn_s_waitcnt(0x0F70 | NSTATE);  // vmcnt(NSTATE)
        if (T < TP)  // rows past T: whatever the copies left in LDS there is replaced by zeros
            for_pieces(W, clear_piece);
    });
    workgroup_lds_barrier<NSTATE>();  // (1) everyone's B, C and x, and the tables

    // ---- score tiles of the row block: S[t = tb*16 + r16][s = sb*16 + 4q + j]
    bf16x8 cfw[4], crv[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        cfw[kk] = rows_frag(rows[0], kk, q, r16);
        crv[kk] = rows_frag(rows[1], kk, q, r16);
    }
    f32x4 S[NB + 1];
#pragma unroll
    for (int ut = 0; ut <= NB; ++ut) {
        const bool fwd = ut <= tb;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            acc = mfma(rows_frag(rows[2 + ut], kk, q, r16), fwd ? cfw[kk] : crv[kk], acc);
        S[ut] = acc;
    }

    // x operands: slots 0..3 tokens 4q + j, slots 4..7 tokens 16 + 4q + j, column p, by
    // transposing reads (lane r16 addresses row 4q + r16/4, columns 16 pblk + 4 (r16 % 4) ..)
    bf16x8 xv[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        bf16x4 half[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tr = 16 * u + 4 * q + (r16 >> 2), col = 16 * pblk + 4 * (r16 & 3);
            half[u] = tr_read(&xs[d][tr * kP + 8 * ((col >> 3) ^ swz_x(tr)) + (col & 7)]);
        }
        xv[d] = cat(half[0], half[1]);
    }
    const bf16x8 xvf = xv[0], xvr = xv[1];
    f32x4 acc_x = {0.f, 0.f, 0.f, 0.f};
    // eq. (11), inside the block (s <= t), exp2 per element on the diagonal pair
    {
        const float ctf = tb_[TAB_CF][t];
        const float4 l0 = *reinterpret_cast<const float4 *>(&tb_[TAB_LGF][4 * q]);
        const float4 l1 = *reinterpret_cast<const float4 *>(&tb_[TAB_LGF][16 + 4 * q]);
        const float lg[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const bool hi_ok = 1 <= tb;
        float mv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int s = (j < 4 ? 0 : 16) + 4 * q + (j & 3);
            const float sv = j < 4 ? S[0][j] : (hi_ok ? S[1][j & 3] : 0.f);
            const float w = __builtin_amdgcn_exp2f(ctf + lg[j]);
            mv[j] = s <= t ? sv * w : 0.f;
        }
        acc_x = mfma(xvf, to_bf16x8(mv), acc_x);
    }
    // eq. (12), reverse inside the block (s >= t)
    {
        const float ctr = tb_[TAB_CR][t];
        const float4 l0 = *reinterpret_cast<const float4 *>(&tb_[TAB_LGR][4 * q]);
        const float4 l1 = *reinterpret_cast<const float4 *>(&tb_[TAB_LGR][16 + 4 * q]);
        const float lg[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const bool lo_ok = 0 >= tb;
        float mv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int s = (j < 4 ? 0 : 16) + 4 * q + (j & 3);
            const float sv = j < 4 ? (lo_ok ? S[1][j] : 0.f) : S[2][j & 3];
            const float w = __builtin_amdgcn_exp2f(ctr + lg[j]);
            mv[j] = s >= t ? sv * w : 0.f;
        }
        acc_x = mfma(xvr, to_bf16x8(mv), acc_x);
    }
    // both products are done before the barrier: left to itself the compiler sinks the second
    // one (and its operand) below it, onto the path that waits for the state
    asm volatile("" ::"v"(acc_x));
    workgroup_lds_barrier<0>();  // (2) everyone's state
    // ---- eq. (11), cached-state term: C_t . (h_hi + h_lo), the B operand of column p being
    // h[32kk + 8q + e][p], e = 0..7, split into bf16 halves in registers; two independent chains
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc_lo = {0.f, 0.f, 0.f, 0.f};
    if constexpr (OPS) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 hi = *reinterpret_cast<const bf16x8 *>(&hops[((4 * kk + q) * CW + 16 * w + r16) * 8]);
            acc = mfma(hi, cfw[kk], acc);
            if constexpr (FORM == FORM_OPS) {
                const bf16x8 lo = *reinterpret_cast<const bf16x8 *>(&hops[((16 + 4 * kk + q) * CW + 16 * w + r16) * 8]);
                acc_lo = mfma(lo, cfw[kk], acc_lo);
            }
        }
    } else {
    // 32 columns: row n = 32kk + 8q + e sits at LDS row 32kk + 8q + (e ^ (q / 2)), and local
    // column 16 w + r16 (piece 4 w + r16 / 4) at slot (4 w + r16 / 4) ^ 4 (q % 2), i.e. at
    // 16 (w ^ (q % 2)) + r16. 64 columns: row n in place, column 16 w + r16 at 16 (w ^ q) + r16.
    const float *hq = WPG == 2 ? &hst[8 * q * CW + 16 * (w ^ (q & 1)) + r16] : &hst[8 * q * CW + 16 * (w ^ q) + r16];
    const int sw = WPG == 2 ? (q >> 1) * CW : 0;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const float *hp = hq + 32 * kk * CW;
        float hv[8];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            hv[e] = hp[e * CW + sw];
            hv[e + 1] = hp[(e + 1) * CW - sw];
        }
        bf16x8 hi, lo;
        split8(hv, hi, lo);
        acc = mfma(hi, cfw[kk], acc);
        acc_lo = mfma(lo, cfw[kk], acc_lo);
    }
    }
    // The products were taken with the state and x as A operands, so the accumulators hold
    // y^T: lane (token t = 16 tb + r16, quarter q) has columns p0 .. p0+3 of its token.
    const int p0 = 16 * pblk + 4 * q;
    {
        const float ef = tb_[TAB_EF][t];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[j] = fmaf(acc[j] + acc_lo[j], ef, acc_x[j]);
    }
    // ---- eq. (13) + D x (+ D_rev x_rev), written once: token t, columns p0 .. p0+3, one 8-
    // (bf16) or 16-byte (float32) store. Rows past T fall outside the output buffer's range
    // and are dropped.
    auto x4 = [&](int d) {  // x[t][p0 .. p0+3] of direction d, from the LDS tile
        return *reinterpret_cast<const bf16x4 *>(&xs[d][t * kP + 8 * ((p0 >> 3) ^ swz_x(t)) + (p0 & 7)]);
    };
    float o[4];
    {
        const bf16x4 xf = x4(0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = fmaf(DCH ? Dc[j] : Dh, bf2f(xf[j]), acc[j]);
    }
    if (a.D_rev) {
        const bf16x4 xr = x4(1);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = fmaf(DCH ? Drc[j] : Dr, bf2f(xr[j]), o[j]);
    }
    const auto rY = buffer_range(static_cast<Ty *>(a.y) + x0, (static_cast<int64_t>(T - 1) * rowX + kP) * sizeof(Ty));
    const int off = (t * rowX + p0) * static_cast<int>(sizeof(Ty));
    if constexpr (sizeof(Ty) == 2) {
        bf16x4 ov;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            ov[j] = static_cast<__bf16>(o[j]);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u32, ov), rY, off, 0, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b128(
            v4u32{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])}, rY,
            off, 0, 0);
    }
}

template <typename Ty>
hipError_t launch_ty(const BlockArgs &a, int wpg, hipStream_t st)
{
    // one workgroup per (head, row block, column part), grid.y = stream: two wavefronts (32
    // columns) when that many workgroups still get a compute unit each, else four
    const int64_t pairs = static_cast<int64_t>(a.s.b) * a.s.H;
    if (wpg != 2 && wpg != 4)
        wpg = pairs * 4 <= device_cus() ? 2 : 4;
    const dim3 g2(static_cast<unsigned>(a.s.H * 4), static_cast<unsigned>(a.s.b));
    const dim3 g4(static_cast<unsigned>(a.s.H * 2), static_cast<unsigned>(a.s.b));
    const int form = !a.h_ops ? FORM_F32 : a.ops_hi_only ? FORM_BF16 : FORM_OPS;
    auto go = [&](auto W, auto F, auto C) {
        constexpr int wpg_ = decltype(W)::value;
        k_block_lat<Ty, wpg_, decltype(F)::value, decltype(C)::value>
            <<<wpg_ == 2 ? g2 : g4, dim3(64 * wpg_), 0, st>>>(a);
    };
    auto by_form = [&](auto W, auto C) {
        if (form == FORM_F32)
            go(W, std::integral_constant<int, FORM_F32>{}, C);
        else if (form == FORM_OPS)
            go(W, std::integral_constant<int, FORM_OPS>{}, C);
        else
            go(W, std::integral_constant<int, FORM_BF16>{}, C);
    };
    auto by_dch = [&](auto W) {
        if (a.d_per_channel)
            by_form(W, std::true_type{});
        else
            by_form(W, std::false_type{});
    };
    if (wpg == 2)
        by_dch(std::integral_constant<int, 2>{});
    else
        by_dch(std::integral_constant<int, 4>{});
    return hipGetLastError();
}

// Operand form of cached states: thread (state, n/8, p) reads h[8 (n/8) + e][p], e = 0..7,
// and writes its bf16 hi and lo parts as two 16-byte pieces (the split the block step would
// otherwise make on every call, in the same arithmetic)
__global__ __launch_bounds__(256) void k_state_ops(const float *__restrict__ h, __bf16 *__restrict__ ops, int64_t nbh)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= nbh * (kN / 8) * kP)
        return;
    const int p = static_cast<int>(i % kP), n8 = static_cast<int>((i / kP) % (kN / 8));
    const int64_t bh = i / (kP * (kN / 8));
    const float *src = h + bh * (kN * kP) + 8 * n8 * kP + p;
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        f[e] = src[e * kP];
    bf16x8 hi, lo;
    split8(f, hi, lo);
    __bf16 *dst = ops + bh * (2 * kN * kP) + (static_cast<int64_t>(n8) * kP + p) * 8;
    *reinterpret_cast<bf16x8 *>(dst) = hi;
    *reinterpret_cast<bf16x8 *>(dst + kN * kP) = lo;
}

}  // namespace

bool block_lat_supported(const Shape &s, int T)
{
    // one or two 16-token row blocks: longer blocks need more registers than a wavefront
    // has without spilling, and go to the bandwidth kernel
    return s.in_dt == 1 && s.N == kN && s.P == kP && T >= 1 && T <= 32;
}

hipError_t launch_block_step_lat(const BlockArgs &a, int wpg, hipStream_t st)
{
    return a.s.y_dt ? launch_ty<__bf16>(a, wpg, st) : launch_ty<float>(a, wpg, st);
}

hipError_t launch_state_ops(const float *h, void *ops, int64_t nbh, hipStream_t st)
{
    const int64_t n = nbh * (kN / 8) * kP;
    if (n == 0)
        return hipSuccess;
    k_state_ops<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st>>>(h, static_cast<__bf16 *>(ops), nbh);
    return hipGetLastError();
}

}  // namespace bdssm
