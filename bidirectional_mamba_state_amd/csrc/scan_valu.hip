// Recurrence-form kernels (float32 vector ALU) for the selective scan.
//
// These run the Mamba-2 recurrence of "Training Hybrid Block Diffusion Language Models
// with Partial Bidirectionality", eq. (1), token by token, with the N x P state of one
// (stream, head) spread over a 256-thread workgroup: thread (p, r) owns the state column
// p for the d_state rows n = r, r + R, r + 2R, ... (R = 256 / P lanes per column, all in
// one wavefront), so the output C_t . S_t is a partial sum per thread followed by a
// cross-lane reduction over the R lanes of the column.
//
// They serve float32 inputs (where bf16 matrix cores would not meet a 1e-5 error bound)
// and every shape, and are the reference launch configuration for the matrix-core
// kernels.
#include <algorithm>

#include "internal.h"

namespace bdssm {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float load_in(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_in(const uint16_t *p, int64_t i)
{
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// float32 -> bfloat16, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t to_bf16(float v)
{
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ void store_y(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_y(uint16_t *p, int64_t i, float v) { p[i] = to_bf16(v); }
__device__ __forceinline__ float load_y(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_y(const uint16_t *p, int64_t i) { return load_in(p, i); }

template <int N, int P>
struct Lay {
    static constexpr int R = kThreads / P;  // lanes per state column
    static constexpr int NPT = N / R;       // state rows per thread
    static_assert(kThreads % P == 0 && R <= 64 && N % R == 0, "unsupported layout");
};

template <int R>
__device__ __forceinline__ float reduce_lanes(float v)
{
#pragma unroll
    for (int off = 1; off < R; off <<= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// One token: S = alpha S + (dt x_p) B_t over the thread's rows; returns sum_n C_t[n] S[n]
// over those rows (0 when Ct is null).
template <typename Tin, int R, int NPT, bool WANT_Y>
__device__ __forceinline__ float token(float (&S)[NPT], const Tin *Bt, const Tin *Ct,
                                       float alpha, float w, int r)
{
    float part = 0.f;
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
        const int n = r + k * R;
        S[k] = fmaf(alpha, S[k], w * load_in(Bt, n));
        if (WANT_Y)
            part = fmaf(load_in(Ct, n), S[k], part);
    }
    return part;
}

// Forward recurrence over one segment of one (stream, head). grid = (nseg, H, b). With
// a.rev the scan runs over the tokens in reverse (position t is token len - 1 - t) and adds
// its outputs to y.
template <typename Tin, typename Ty, int N, int P, bool WANT_Y>
__global__ __launch_bounds__(kThreads) void k_forward(ForwardArgs a)
{
    using L = Lay<N, P>;
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, p = tid / L::R, r = tid % L::R;
    const int H = a.s.H, G = a.s.G, g = h / (H / G);
    constexpr int64_t NP = static_cast<int64_t>(N) * P;
    const int64_t t0 = static_cast<int64_t>(c) * a.Q;
    const int64_t t1 = min(a.len, t0 + a.Q);

    const float *sin = c == 0 ? a.first_state
                              : (a.prev_states ? a.prev_states +
                                                     ((static_cast<int64_t>(b) * a.nseg + (c - 1)) * H + h) * NP
                                               : nullptr);
    if (c == 0 && sin)
        sin += (static_cast<int64_t>(b) * H + h) * NP;
    float S[L::NPT];
#pragma unroll
    for (int k = 0; k < L::NPT; ++k)
        S[k] = sin ? sin[static_cast<int64_t>(r + k * L::R) * P + p] : 0.f;

    const Tin *x = static_cast<const Tin *>(a.in.x);
    const Tin *dt = static_cast<const Tin *>(a.in.dt);
    const Tin *Bm = static_cast<const Tin *>(a.in.B);
    const Tin *Cm = static_cast<const Tin *>(a.in.C);
    Ty *y = static_cast<Ty *>(a.y);
    const float Ah = a.A[h];
    const float Dh = a.D ? a.D[h] : 0.f;
    float dsum = 0.f;
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t tok = static_cast<int64_t>(b) * a.len + (a.rev ? a.len - 1 - t : t);
        const float dtv = load_in(dt, tok * H + h);
        const float la = dtv * Ah;
        dsum += la;
        const float alpha = expf(la);
        const float xv = load_in(x, (tok * H + h) * P + p);
        const int64_t bc = (tok * G + g) * N;
        float part = token<Tin, L::R, L::NPT, WANT_Y>(S, Bm + bc, WANT_Y ? Cm + bc : nullptr, alpha, dtv * xv, r);
        if (WANT_Y) {
            part = reduce_lanes<L::R>(part);
            if (r == 0) {
                const int64_t o = (tok * H + h) * P + p;
                const float v = fmaf(Dh, xv, part);
                store_y(y, o, a.rev ? v + load_y(y, o) : v);
            }
        }
    }
    if (a.state_out) {
        float *so = a.state_out + ((static_cast<int64_t>(b) * a.nseg + c) * H + h) * NP;
#pragma unroll
        for (int k = 0; k < L::NPT; ++k)
            so[static_cast<int64_t>(r + k * L::R) * P + p] = S[k];
    }
    if (a.decay_out && tid == 0)
        a.decay_out[(static_cast<int64_t>(b) * a.nseg + c) * H + h] = dsum;
}

// Block step: forward from h_prefix over fwd, reverse from zero over rev, y = sum + D x_fwd.
// grid = (H, b); dynamic LDS = T * P floats.
template <typename Tin, typename Ty, int N, int P>
__global__ __launch_bounds__(kThreads) void k_block_step(BlockArgs a)
{
    using L = Lay<N, P>;
    extern __shared__ float ybuf[];
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, p = tid / L::R, r = tid % L::R;
    const int H = a.s.H, G = a.s.G, g = h / (H / G), T = a.T;
    constexpr int64_t NP = static_cast<int64_t>(N) * P;
    const float Ah = a.A[h], Ahr = a.A_rev[h];

    float S[L::NPT];
    if (a.h_prefix) {
        const float *hp = a.h_prefix + (static_cast<int64_t>(b) * H + h) * NP;
#pragma unroll
        for (int k = 0; k < L::NPT; ++k)
            S[k] = hp[static_cast<int64_t>(r + k * L::R) * P + p];
    } else {  // the bf16 cached state, [N/8][P][8]: element (n, p) at (n/8 P + p) 8 + n % 8
        const uint16_t *hb = static_cast<const uint16_t *>(a.h_ops) + (static_cast<int64_t>(b) * H + h) * NP;
#pragma unroll
        for (int k = 0; k < L::NPT; ++k) {
            const int n = r + k * L::R;
            S[k] = load_in(hb, ((n >> 3) * P + p) * 8 + (n & 7));
        }
    }

    {   // eq. (11): forward continuation of the cached state
        const Tin *x = static_cast<const Tin *>(a.fwd.x);
        const Tin *dt = static_cast<const Tin *>(a.fwd.dt);
        const Tin *Bm = static_cast<const Tin *>(a.fwd.B);
        const Tin *Cm = static_cast<const Tin *>(a.fwd.C);
        for (int t = 0; t < T; ++t) {
            const int64_t tok = static_cast<int64_t>(b) * T + t;
            const float dtv = load_in(dt, tok * H + h);
            const float alpha = expf(dtv * Ah);
            const float xv = load_in(x, (tok * H + h) * P + p);
            const int64_t bc = (tok * G + g) * N;
            float part = token<Tin, L::R, L::NPT, true>(S, Bm + bc, Cm + bc, alpha, dtv * xv, r);
            part = reduce_lanes<L::R>(part);
            if (r == 0)
                ybuf[t * P + p] = part;
        }
    }
    {   // eq. (12): reverse scan inside the block, zero state at the right end
#pragma unroll
        for (int k = 0; k < L::NPT; ++k)
            S[k] = 0.f;
        const Tin *x = static_cast<const Tin *>(a.rev.x);
        const Tin *dt = static_cast<const Tin *>(a.rev.dt);
        const Tin *Bm = static_cast<const Tin *>(a.rev.B);
        const Tin *Cm = static_cast<const Tin *>(a.rev.C);
        for (int t = T - 1; t >= 0; --t) {
            const int64_t tok = static_cast<int64_t>(b) * T + t;
            const float dtv = load_in(dt, tok * H + h);
            const float alpha = expf(dtv * Ahr);
            const float xv = load_in(x, (tok * H + h) * P + p);
            const int64_t bc = (tok * G + g) * N;
            float part = token<Tin, L::R, L::NPT, true>(S, Bm + bc, Cm + bc, alpha, dtv * xv, r);
            part = reduce_lanes<L::R>(part);
            if (r == 0)
                ybuf[t * P + p] += part;  // same thread wrote the forward value
        }
    }
    __syncthreads();
    // eq. (13) plus D x_fwd, written once, coalesced along p
    const Tin *xf = static_cast<const Tin *>(a.fwd.x);
    const Tin *xr = static_cast<const Tin *>(a.rev.x);
    Ty *y = static_cast<Ty *>(a.y);
    for (int i = tid; i < T * P; i += kThreads) {
        const int t = i / P, pp = i % P;
        const int64_t o = ((static_cast<int64_t>(b) * T + t) * H + h) * P + pp;
        const int wi = a.d_per_channel ? h * P + pp : h;  // skip weight per head or per channel
        float v = fmaf(a.D[wi], load_in(xf, o), ybuf[i]);
        if (a.D_rev)
            v = fmaf(a.D_rev[wi], load_in(xr, o), v);
        store_y(y, o, v);
    }
}

// bf16 copy of cached states: thread (state, n/8, p) reads h[8 (n/8) + e][p], e = 0..7, and
// writes bf16(h) (round to nearest even) as one 16-byte piece of [N/8][P][8]
__global__ __launch_bounds__(kThreads) void k_state_bf16(const float *__restrict__ h, uint16_t *__restrict__ out,
                                                         int64_t nbh, int N, int P)
{
    const int64_t per = static_cast<int64_t>(N / 8) * P;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= nbh * per)
        return;
    const int64_t st = i / per;
    const int n8 = static_cast<int>((i % per) / P), p = static_cast<int>(i % P);
    const float *src = h + st * N * P + static_cast<int64_t>(8 * n8) * P + p;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2)
        w[e / 2] = static_cast<uint32_t>(to_bf16(src[e * P])) | (static_cast<uint32_t>(to_bf16(src[(e + 1) * P])) << 16);
    *reinterpret_cast<uint4 *>(out + st * N * P + (static_cast<int64_t>(n8) * P + p) * 8) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Inter-chunk state passing, one thread per state element. grid = (ceil(NP/256), H, b).
__global__ __launch_bounds__(kThreads) void k_state_pass(PassArgs a)
{
    const int64_t NP = static_cast<int64_t>(a.s.N) * a.s.P;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int h = blockIdx.y, b = blockIdx.z, H = a.s.H;
    if (e >= NP)
        return;
    float v = a.h_init ? a.h_init[(static_cast<int64_t>(b) * H + h) * NP + e] : 0.f;
    for (int c = 0; c < a.nch; ++c) {
        const int64_t bh = (static_cast<int64_t>(b) * a.nch + c) * H + h;
        v = fmaf(expf(a.decay[bh]), v, a.states[bh * NP + e]);
        if (a.write_all)
            a.states[bh * NP + e] = v;
    }
    if (a.h_out)
        a.h_out[(static_cast<int64_t>(b) * H + h) * NP + e] = v;
}

__global__ void k_copy(float *dst, const float *src, int64_t n)
{
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        dst[i] = src[i];
}

__global__ void k_fill(float *dst, float v, int64_t n)
{
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        dst[i] = v;
}

template <typename Tin, typename Ty, int N, int P>
hipError_t fwd_launch(const ForwardArgs &a, hipStream_t st)
{
    dim3 grid(a.nseg, a.s.H, a.s.b);
    if (a.y)
        k_forward<Tin, Ty, N, P, true><<<grid, kThreads, 0, st>>>(a);
    else
        k_forward<Tin, Ty, N, P, false><<<grid, kThreads, 0, st>>>(a);
    return hipGetLastError();
}

template <typename Tin, typename Ty, int N, int P>
hipError_t blk_launch(const BlockArgs &a, hipStream_t st)
{
    const size_t lds = sizeof(float) * a.T * P;
    k_block_step<Tin, Ty, N, P><<<dim3(a.s.H, a.s.b), kThreads, lds, st>>>(a);
    return hipGetLastError();
}

}  // namespace

bool valu_supported(int N, int P)
{
    return (N == 16 && P == 16) || (N == 128 && P == 64);
}

#define BDSSM_DISPATCH(FN, s, a, st)                                                      \
    do {                                                                                  \
        const int key = ((s).N == 16 ? 0 : 2) + ((s).in_dt ? 4 : 0) + ((s).y_dt ? 1 : 0); \
        switch (key) {                                                                    \
        case 0: return FN<float, float, 16, 16>(a, st);                                   \
        case 1: return FN<float, uint16_t, 16, 16>(a, st);                                \
        case 2: return FN<float, float, 128, 64>(a, st);                                  \
        case 3: return FN<float, uint16_t, 128, 64>(a, st);                               \
        case 4: return FN<uint16_t, float, 16, 16>(a, st);                                \
        case 5: return FN<uint16_t, uint16_t, 16, 16>(a, st);                             \
        case 6: return FN<uint16_t, float, 128, 64>(a, st);                               \
        case 7: return FN<uint16_t, uint16_t, 128, 64>(a, st);                            \
        }                                                                                 \
        return hipErrorInvalidValue;                                                      \
    } while (0)

hipError_t launch_forward_valu(const ForwardArgs &a, hipStream_t st)
{
    BDSSM_DISPATCH(fwd_launch, a.s, a, st);
}

hipError_t launch_block_step_valu(const BlockArgs &a, hipStream_t st)
{
    BDSSM_DISPATCH(blk_launch, a.s, a, st);
}

hipError_t launch_state_pass(const PassArgs &a, hipStream_t st)
{
    const int64_t NP = static_cast<int64_t>(a.s.N) * a.s.P;
    dim3 grid(static_cast<unsigned>((NP + kThreads - 1) / kThreads), a.s.H, a.s.b);
    k_state_pass<<<grid, kThreads, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_state_bf16(const float *h, void *out, int64_t nbh, int N, int P, hipStream_t st)
{
    const int64_t n = nbh * (N / 8) * P;
    k_state_bf16<<<static_cast<unsigned>((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(
        h, static_cast<uint16_t *>(out), nbh, N, P);
    return hipGetLastError();
}

hipError_t launch_copy_f32(float *dst, const float *src, int64_t n, hipStream_t st)
{
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    k_copy<<<static_cast<unsigned>(blocks), 256, 0, st>>>(dst, src, n);
    return hipGetLastError();
}

hipError_t launch_fill_f32(float *dst, float v, int64_t n, hipStream_t st)
{
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    k_fill<<<static_cast<unsigned>(blocks), 256, 0, st>>>(dst, v, n);
    return hipGetLastError();
}

}  // namespace bdssm
