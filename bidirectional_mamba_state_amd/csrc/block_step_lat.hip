// Block step for small batches: the same computation as block_step_mfma.hip (eqs. (11)-(13)
// of "Training Hybrid Block Diffusion Language Models with Partial Bidirectionality" in the
// matrix form of the Mamba-2 scan), laid out for latency instead of bandwidth.
//
// With few (stream, head) pairs a launch has about one wavefront per SIMD, and its time is
// the length of one wavefront's chain of dependent steps, not the bytes it moves. So each
// wavefront is its own workgroup and owns one 16-token row block, one 16-column block and
// one head, and everything it needs goes from global memory straight into registers in the
// layout the matrix cores read:
//   - the cached state as the B operand of C . h: lane (column p, quarter q) loads
//     h[32k + 8q + e][p], e = 0..7, as single dwords -- eight consecutive contraction
//     indices of its column, the bf16 operand layout as loaded -- and splits it into bf16
//     hi + lo parts in registers (two products, ~16 significant bits);
//   - x of both directions as the B operand of M X: 8-byte row pieces transposed 4 x 4
//     (16-bit) across lanes with DPP, giving each lane the tokens of its slots
//     (4q + e, 16 + 4q + e) in its column; the same registers give D x;
//   - the C B^T score tiles as in the bandwidth kernel (B rows as A, C rows as B operand).
// The cumulative log-decays of both directions are a 64-lane DPP scan in the same
// wavefront, shared through a small wavefront-private LDS table. There is no workgroup
// barrier, no state or x staging through LDS, and y leaves straight from the accumulators.
// Loads and stores go through range-checked buffer resources over the stream's T tokens, so
// rows past T read as zero and their stores are dropped, with no clamping or masking code
// (at about one wavefront per SIMD, every vector instruction is on the critical path). All
// loads are issued before the first use, fewer than a wavefront can have in flight (63), so
// the wavefront waits for memory once.
#include "internal.h"
#include "mfma_tiles.h"

namespace bdssm {
namespace {

constexpr int kN = 128, kP = 64;
constexpr float kLog2e = 1.4426950408889634f;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}

// inclusive sum over the 64 lanes: shifts by 1, 2, 4, 8 inside rows of 16 lanes, then the
// last lane of each row is added to the rows after it
__device__ __forceinline__ float wave_inclusive_sum(float v)
{
    v += dpp_move<0x111, 0xf>(v);
    v += dpp_move<0x112, 0xf>(v);
    v += dpp_move<0x114, 0xf>(v);
    v += dpp_move<0x118, 0xf>(v);
    v += dpp_move<0x142, 0xa>(v);
    v += dpp_move<0x143, 0xc>(v);
    return v;
}

__device__ __forceinline__ float lane_value(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <int CTRL>
__device__ __forceinline__ uint32_t quad_move(uint32_t x)
{
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xf, 0xf, false));
}

// 4 x 4 transpose of 16-bit values inside each group of four lanes. Lane i holds row i as
// two dwords (columns 0,1 | 2,3, the lower column in the lower half) and receives column i
// as rows 0,1 | 2,3. First lanes i^2 swap the dword with the other column pair, then lanes
// i^1 swap the 16-bit halves of the other column; v_perm with per-lane selectors puts the
// four rows in order.
__device__ __forceinline__ uint2 quad_transpose16(uint2 v, int i)
{
    const bool b0 = i & 1, b1 = i & 2;
    const uint32_t keep = b1 ? v.y : v.x, send = b1 ? v.x : v.y;
    const uint32_t oth = quad_move<0x4E>(send);  // quad_perm 2,3,0,1: row i^2, same columns
    // column 2*b1 + b0 of rows (i, i^2) is kept, the other column of them is sent to lane i^1
    const uint32_t kept = __builtin_amdgcn_perm(oth, keep, b0 ? 0x07060302u : 0x05040100u);
    const uint32_t snd = __builtin_amdgcn_perm(oth, keep, b0 ? 0x05040100u : 0x07060302u);
    const uint32_t rcv = quad_move<0xB1>(snd);  // quad_perm 1,0,3,2: rows (i^1, i^3)
    // rows (2m, 2m+1): from (kept.lo, rcv.lo) when m == b1, (kept.hi, rcv.hi) otherwise,
    // with the two swapped when b0 is set
    const uint32_t L = __builtin_amdgcn_perm(rcv, kept, b0 ? 0x01000504u : 0x05040100u);
    const uint32_t Hh = __builtin_amdgcn_perm(rcv, kept, b0 ? 0x03020706u : 0x07060302u);
    return make_uint2(b1 ? Hh : L, b1 ? L : Hh);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes)
{
    // raw buffer with range checking: loads past `bytes` return zero, stores are dropped
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ bf16x8 ld_b128(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ void store_y(__amdgpu_buffer_rsrc_t r, int off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void store_y_bf16(__amdgpu_buffer_rsrc_t r, int off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, static_cast<__bf16>(v)), r, off, 0, 0);
}

enum { TAB_CF, TAB_CR, TAB_LGF, TAB_LGR, TAB_COLF, TAB_COLR, TAB_EF, NTAB };

template <typename Ty>
__global__ __launch_bounds__(64) void k_block_lat(BlockArgs a)
{
    constexpr int NB = 2, TP = 32;  // one 32-token pair: two 16-token row blocks
    __shared__ __attribute__((aligned(16))) float tab[NTAB][TP];

    const int T = a.T, H = a.s.H, G = a.s.G;
    // The hardware deals workgroup ids round-robin over the 8 XCDs. The 8 wavefronts of one
    // (stream, head) read the same state and x lines (each a quarter row), so they are given
    // ids that land on one XCD and share its L2: logical id = position within the XCD's
    // consecutive range.
    const int nwg = gridDim.x;
    int wid = blockIdx.x;
    if ((nwg & 7) == 0)
        wid = (wid & 7) * (nwg >> 3) + (wid >> 3);
    const int tb = wid % NB;
    const int pblk = (wid / NB) % (kP / 16);
    const int h = (wid / (NB * (kP / 16))) % H;
    const int b = wid / (NB * (kP / 16) * H);
    const int g = h / (H / G);
    const int lane = threadIdx.x, q = lane >> 4, r16 = lane & 15, i4 = lane & 3;
    const int t = tb * 16 + r16;  // this lane's row as an A operand
    const int p = pblk * 16 + r16;

    // range-checked buffers over this stream's T tokens: rows past T read as zero
    const int64_t tok0 = static_cast<int64_t>(b) * T;
    const int rowBC = G * kN, rowX = H * kP;
    const int64_t bc_bytes = (static_cast<int64_t>(T - 1) * rowBC + kN) * 2;
    const int64_t bc0 = tok0 * rowBC + g * kN;
    const auto rBf = rsrc(static_cast<const __bf16 *>(a.fwd.B) + bc0, bc_bytes);
    const auto rCf = rsrc(static_cast<const __bf16 *>(a.fwd.C) + bc0, bc_bytes);
    const auto rBr = rsrc(static_cast<const __bf16 *>(a.rev.B) + bc0, bc_bytes);
    const auto rCr = rsrc(static_cast<const __bf16 *>(a.rev.C) + bc0, bc_bytes);
    const int64_t x0 = tok0 * rowX + h * kP;
    const int64_t x_bytes = (static_cast<int64_t>(T - 1) * rowX + kP) * 2;
    const auto rXf = rsrc(static_cast<const __bf16 *>(a.fwd.x) + x0, x_bytes);
    const auto rXr = rsrc(static_cast<const __bf16 *>(a.rev.x) + x0, x_bytes);
    const int64_t dt_bytes = (static_cast<int64_t>(T - 1) * H + 1) * 2;
    const auto rDf = rsrc(static_cast<const __bf16 *>(a.fwd.dt) + tok0 * H + h, dt_bytes);
    const auto rDr = rsrc(static_cast<const __bf16 *>(a.rev.dt) + tok0 * H + h, dt_bytes);
    const auto rH = rsrc(a.h_prefix + (static_cast<int64_t>(b) * H + h) * (kN * kP), kN * kP * 4);

    // ---- every load of the wavefront (60, fewer than a wavefront can have in flight),
    // issued before any of them is used
    bf16x8 cfw[4], crv[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        cfw[kk] = ld_b128(rCf, (t * rowBC + 32 * kk + 8 * q) * 2);
        crv[kk] = ld_b128(rCr, (t * rowBC + 32 * kk + 8 * q) * 2);
    }
    bf16x8 bfr[NB + 1][4];
#pragma unroll
    for (int ut = 0; ut <= NB; ++ut) {
        const bool fwd = ut <= tb;
        const int srow = (fwd ? ut : ut - 1) * 16 + r16;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            bfr[ut][kk] = ld_b128(fwd ? rBf : rBr, (srow * rowBC + 32 * kk + 8 * q) * 2);
    }
    // the cached state as B operands of the state product: h[32kk + 8q + e][p]
    float hv[4][8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            hv[kk][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rH, ((32 * kk + 8 * q + e) * kP + p) * 4, 0, 0));
    // x: lane 4c + i loads columns 4c .. 4c+3 of token 4q + i (and 16 + 4q + i); a 16-bit
    // 4 x 4 transpose in each group of four lanes gives tokens 4q .. 4q+3 of its own column
    uint2 xl[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int off = ((16 * u + 4 * q + i4) * rowX + pblk * 16 + (r16 & ~3)) * 2;
        xl[0][u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rXf, off, 0, 0));
        xl[1][u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rXr, off, 0, 0));
    }
    const int t0 = 2 * lane, t1 = t0 + 1;
    const unsigned short df0 = __builtin_amdgcn_raw_buffer_load_b16(rDf, t0 * H * 2, 0, 0);
    const unsigned short df1 = __builtin_amdgcn_raw_buffer_load_b16(rDf, t1 * H * 2, 0, 0);
    const unsigned short dr0 = __builtin_amdgcn_raw_buffer_load_b16(rDr, t0 * H * 2, 0, 0);
    const unsigned short dr1 = __builtin_amdgcn_raw_buffer_load_b16(rDr, t1 * H * 2, 0, 0);
    const float Ah = a.A[h], Dh = a.D[h], Ar = a.A_rev[h];
    const float Dr = a.D_rev ? a.D_rev[h] : 0.f;

    // ---- decay tables of both directions (lane l holds tokens 2l and 2l+1; dt past T is 0)
    {
        const float f0 = __uint_as_float(static_cast<uint32_t>(df0) << 16);
        const float f1 = __uint_as_float(static_cast<uint32_t>(df1) << 16);
        const float g0 = __uint_as_float(static_cast<uint32_t>(dr0) << 16);
        const float g1 = __uint_as_float(static_cast<uint32_t>(dr1) << 16);
        // forward: c_t inclusive prefix sum; reference at the pair's last token (lane 15)
        const float a0 = f0 * Ah, a1 = f1 * Ah, loc = a0 + a1;
        const float inc = wave_inclusive_sum(loc), excl = inc - loc;
        const float c0 = (excl + a0) * kLog2e, c1 = (excl + loc) * kLog2e;
        // reverse: r_t inclusive suffix sum; reference at the pair's first token (lane 0)
        const float b0 = g0 * Ar, b1 = g1 * Ar, locr = b0 + b1;
        const float incr = wave_inclusive_sum(locr), exclr = incr - locr, totr = lane_value(incr, 63);
        const float r0 = (totr - exclr) * kLog2e, r1 = (totr - exclr - b0) * kLog2e;
        const float reff = lane_value(c1, 15), refr = lane_value(r0, 0);
        if (t0 < TP) {
            tab[TAB_CF][t0] = c0;
            tab[TAB_CF][t1] = c1;
            tab[TAB_CR][t0] = r0;
            tab[TAB_CR][t1] = r1;
            tab[TAB_LGF][t0] = __builtin_amdgcn_logf(f0) - c0;
            tab[TAB_LGF][t1] = __builtin_amdgcn_logf(f1) - c1;
            tab[TAB_LGR][t0] = __builtin_amdgcn_logf(g0) - r0;
            tab[TAB_LGR][t1] = __builtin_amdgcn_logf(g1) - r1;
            tab[TAB_COLF][t0] = __builtin_amdgcn_exp2f(reff - c0) * f0;
            tab[TAB_COLF][t1] = __builtin_amdgcn_exp2f(reff - c1) * f1;
            tab[TAB_COLR][t0] = __builtin_amdgcn_exp2f(refr - r0) * g0;
            tab[TAB_COLR][t1] = __builtin_amdgcn_exp2f(refr - r1) * g1;
            tab[TAB_EF][t0] = __builtin_amdgcn_exp2f(c0);
            tab[TAB_EF][t1] = __builtin_amdgcn_exp2f(c1);
        }
    }

    // ---- score tiles of the row block: S[t = tb*16 + r16][s = sb*16 + 4q + j]
    f32x4 S[NB + 1];
#pragma unroll
    for (int ut = 0; ut <= NB; ++ut) {
        const bool fwd = ut <= tb;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            acc = mfma(bfr[ut][kk], fwd ? cfw[kk] : crv[kk], acc);
        S[ut] = acc;
    }

    // ---- eq. (11), cached-state term: C_t . (h_hi + h_lo). The dword loads gave each lane
    // h[32kk + 8q + e][p], e = 0..7: the B operand layout of the bf16 product as loaded, so
    // the state is split in registers; two independent chains
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc_lo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        bf16x8 hi, lo;
        split8(hv[kk], hi, lo);
        acc = mfma(cfw[kk], hi, acc);
        acc_lo = mfma(cfw[kk], lo, acc_lo);
    }
    acc += acc_lo;
    __syncthreads();  // the tables (one wavefront: a wavefront barrier)
    {
        const float4 e4 = *reinterpret_cast<const float4 *>(&tab[TAB_EF][tb * 16 + 4 * q]);
        acc[0] *= e4.x;
        acc[1] *= e4.y;
        acc[2] *= e4.z;
        acc[3] *= e4.w;
    }
    // x operands: slots 0..3 tokens 4q + j, slots 4..7 tokens 16 + 4q + j, column p
    const uint2 f0 = quad_transpose16(xl[0][0], i4), f1 = quad_transpose16(xl[0][1], i4);
    const uint2 v0 = quad_transpose16(xl[1][0], i4), v1 = quad_transpose16(xl[1][1], i4);
    const bf16x8 xvf = __builtin_bit_cast(bf16x8, make_uint4(f0.x, f0.y, f1.x, f1.y));
    const bf16x8 xvr = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
    // eq. (11), inside the block (s <= t), exp2 per element on the diagonal pair
    {
        const float ctf = tab[TAB_CF][t];
        const float4 l0 = *reinterpret_cast<const float4 *>(&tab[TAB_LGF][4 * q]);
        const float4 l1 = *reinterpret_cast<const float4 *>(&tab[TAB_LGF][16 + 4 * q]);
        const float lg[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const bool hi_ok = 1 <= tb;
        bf16x8 af;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int s = (j < 4 ? 0 : 16) + 4 * q + (j & 3);
            const float sv = j < 4 ? S[0][j] : (hi_ok ? S[1][j & 3] : 0.f);
            const float w = __builtin_amdgcn_exp2f(ctf + lg[j]);
            af[j] = static_cast<__bf16>(s <= t ? sv * w : 0.f);
        }
        acc = mfma(af, xvf, acc);
    }
    // eq. (12), reverse inside the block (s >= t)
    {
        const float ctr = tab[TAB_CR][t];
        const float4 l0 = *reinterpret_cast<const float4 *>(&tab[TAB_LGR][4 * q]);
        const float4 l1 = *reinterpret_cast<const float4 *>(&tab[TAB_LGR][16 + 4 * q]);
        const float lg[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const bool lo_ok = 0 >= tb;
        bf16x8 af;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int s = (j < 4 ? 0 : 16) + 4 * q + (j & 3);
            const float sv = j < 4 ? (lo_ok ? S[1][j] : 0.f) : S[2][j & 3];
            const float w = __builtin_amdgcn_exp2f(ctr + lg[j]);
            af[j] = static_cast<__bf16>(s >= t ? sv * w : 0.f);
        }
        acc = mfma(af, xvr, acc);
    }
    // ---- eq. (13) + D x (+ D_rev x_rev), written once: rows tb*16 + 4q + j, column p. The
    // x of those rows are slots (tb & 1) * 4 + j of the operands. Rows past T fall outside
    // the output buffer's range and are dropped.
    const auto rY = rsrc(static_cast<Ty *>(a.y) + x0, (static_cast<int64_t>(T - 1) * rowX + kP) * sizeof(Ty));
    const bool with_dr = a.D_rev != nullptr;
    const bool odd = tb & 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tr = tb * 16 + 4 * q + j;
        const float xa = bf2f(xvf[j]), xb = bf2f(xvf[4 + j]);
        const float ra = bf2f(xvr[j]), rb = bf2f(xvr[4 + j]);
        float v = fmaf(Dh, odd ? xb : xa, acc[j]);
        if (with_dr)
            v = fmaf(Dr, odd ? rb : ra, v);
        if constexpr (sizeof(Ty) == 2)
            store_y_bf16(rY, (tr * rowX + p) * 2, v);
        else
            store_y(rY, (tr * rowX + p) * 4, v);
    }
}

template <typename Ty>
hipError_t launch_ty(const BlockArgs &a, hipStream_t st)
{
    const int64_t nwg = static_cast<int64_t>(a.s.b) * a.s.H * (kP / 16) * 2;
    k_block_lat<Ty><<<dim3(static_cast<unsigned>(nwg)), dim3(64), 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace

bool block_lat_supported(const Shape &s, int T)
{
    // one or two 16-token row blocks: longer blocks need more registers than a wavefront
    // has without spilling, and go to the bandwidth kernel
    return s.in_dt == 1 && s.N == kN && s.P == kP && T >= 1 && T <= 32;
}

hipError_t launch_block_step_lat(const BlockArgs &a, hipStream_t st)
{
    return a.s.y_dt ? launch_ty<__bf16>(a, st) : launch_ty<float>(a, st);
}

}  // namespace bdssm
