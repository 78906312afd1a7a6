// Depthwise short convolution of the scan's inputs: the convolution state of the Mamba
// cache ("Training Hybrid Block Diffusion Language Models with Partial Bidirectionality",
// the cache discussion: a Mamba layer's cache holds convolution state as well as the
// selective-SSM state).
//
// The x, B and C inputs of a token are one row of CH = H*P + 2*G*N channels (x, then B,
// then C). Each channel c is convolved with its own W taps (W <= 4), a bias is added and
// an activation applied (identity or SiLU); the result, rounded to the input dtype, is
// what the scan reads:
//   forward (causal):   out_t = bias + sum_{j<W} w[W-1-j] u_{t-j},  u_{t<0} from the conv
//                       state (the W-1 raw rows before the segment, or zeros);
//   reverse (anti-causal, inside the block):
//                       out_t = bias + sum_{j<W} w[W-1-j] u_{t+j},  u_{t>=len} = 0.
// The forward pass can also write the new conv state: the last W-1 rows of the raw input
// extended by the old state.
//
// One thread owns 8 consecutive channels of one stream and a run of R tokens. It loads the
// R + W - 1 rows its outputs need (16-byte loads, 64 lanes of a wavefront read 1 KiB of a
// row), so each raw row is read by at most two threads. HBM-bound: the algorithmic bytes are
// the raw rows read once and the convolved rows written once.
//
// The old conv state is read only by the threads of the first run of each channel group,
// and the new state is written by those same threads after they have read the old one, so
// the state may be updated in place.
#include "internal.h"

namespace bdssm {
namespace {

template <typename Ti>
struct Row;

template <>
struct Row<__bf16> {
    uint4 v;
    __device__ __forceinline__ void load(const __bf16 *p) { v = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void store(__bf16 *p) const { *reinterpret_cast<uint4 *>(p) = v; }
    __device__ __forceinline__ float get(int i) const
    {
        const uint32_t word = (i >> 1) == 0 ? v.x : (i >> 1) == 1 ? v.y : (i >> 1) == 2 ? v.z : v.w;
        return __uint_as_float((i & 1) ? (word & 0xffff0000u) : (word << 16));
    }
    __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ void set(const float f[8])
    {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const __bf16 lo = static_cast<__bf16>(f[2 * k]), hi = static_cast<__bf16>(f[2 * k + 1]);
            w[k] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                   (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
        }
        v = make_uint4(w[0], w[1], w[2], w[3]);
    }
};

template <>
struct Row<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p)
    {
        a = *reinterpret_cast<const float4 *>(p);
        b = *reinterpret_cast<const float4 *>(p + 4);
    }
    __device__ __forceinline__ void store(float *p) const
    {
        *reinterpret_cast<float4 *>(p) = a;
        *reinterpret_cast<float4 *>(p + 4) = b;
    }
    __device__ __forceinline__ float get(int i) const
    {
        const float4 &h = i < 4 ? a : b;
        const int k = i & 3;
        return k == 0 ? h.x : k == 1 ? h.y : k == 2 ? h.z : h.w;
    }
    __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void set(const float f[8])
    {
        a = make_float4(f[0], f[1], f[2], f[3]);
        b = make_float4(f[4], f[5], f[6], f[7]);
    }
};

template <typename Ti, int W, int R, bool REV>
__device__ __forceinline__ void conv_run(const Shape &sh, int64_t len, int act, int nrun, const ConvSeqArgs &q)
{
    const int HP = sh.H * sh.P, GN = sh.G * sh.N;
    const int ch8 = (HP + 2 * GN) / 8;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= static_cast<int64_t>(sh.b) * nrun * ch8)
        return;
    const int oct = static_cast<int>(gid % ch8);
    const int64_t rest = gid / ch8;
    const int run = static_cast<int>(rest % nrun);
    const int b = static_cast<int>(rest / nrun);
    const int c = oct * 8;

    // which array the 8 channels live in, and their offset within its token row
    const Ti *src;
    Ti *dst;
    int rowlen, cc;
    if (c < HP) {
        src = static_cast<const Ti *>(q.x), dst = static_cast<Ti *>(q.ox), rowlen = HP, cc = c;
    } else if (c < HP + GN) {
        src = static_cast<const Ti *>(q.B), dst = static_cast<Ti *>(q.oB), rowlen = GN, cc = c - HP;
    } else {
        src = static_cast<const Ti *>(q.C), dst = static_cast<Ti *>(q.oC), rowlen = GN, cc = c - HP - GN;
    }
    src += static_cast<int64_t>(b) * len * rowlen + cc;
    dst += static_cast<int64_t>(b) * len * rowlen + cc;
    const int CH = HP + 2 * GN;
    const Ti *st_in = q.state_in ? static_cast<const Ti *>(q.state_in) + static_cast<int64_t>(b) * (W - 1) * CH + c
                                 : nullptr;

    // taps by distance: wd[j] multiplies u_{t-j} (forward) or u_{t+j} (reverse)
    float wd[W][8], bias[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int k = 0; k < W; ++k)
            wd[W - 1 - k][i] = q.w[(c + i) * W + k];
        bias[i] = q.bias ? q.bias[c + i] : 0.f;
    }

    const int64_t t0 = static_cast<int64_t>(run) * R;
    constexpr int NR = R + W - 1;
    // rows: forward u_{t0-(W-1)} .. u_{t0+R-1}; reverse u_{t0} .. u_{t0+R-1+(W-1)}
    const int64_t first = REV ? t0 : t0 - (W - 1);
    Row<Ti> u[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int64_t idx = first + r;
        const bool in_seq = idx >= 0 && idx < len;
        const bool in_state = idx < 0 && st_in != nullptr;
        // branch-free: the address is always valid, the value selected afterwards
        const Ti *p = in_state ? st_in + (W - 1 + idx) * CH
                               : src + min(max(idx, static_cast<int64_t>(0)), len - 1) * rowlen;
        u[r].load(p);
        if (!in_seq && !in_state)
            u[r].zero();
    }

#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int64_t t = t0 + k;
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float acc = bias[i];
#pragma unroll
            for (int j = W - 1; j >= 0; --j) {  // the oldest input first
                const int r = REV ? k + j : k + (W - 1) - j;
                acc = fmaf(wd[j][i], u[r].get(i), acc);
            }
            if (act == 1)
                acc = acc * __builtin_amdgcn_rcpf(1.f + __expf(-acc));
            v[i] = acc;
        }
        if (t < len) {
            Row<Ti> o;
            o.set(v);
            o.store(dst + t * rowlen);
        }
    }

    // new conv state: rows len-(W-1) .. len-1 of the extended input, written by the
    // threads of the first run (the only ones that read the old state)
    if (!REV && W > 1 && q.state_out && run == 0) {
        Ti *so = static_cast<Ti *>(q.state_out) + static_cast<int64_t>(b) * (W - 1) * CH + c;
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const int64_t idx = len - (W - 1) + j;
            Row<Ti> o;
            if (idx >= 0) {
                o.load(src + idx * rowlen);
            } else {  // still inside the old state: this thread's rows 0 .. W-2 hold it
                o = u[0];
#pragma unroll
                for (int r = 1; r < W - 1; ++r)
                    if (idx + (W - 1) == r)
                        o = u[r];
            }
            o.store(so + j * CH);
        }
    }
}

template <typename Ti, int W, int R>
__global__ __launch_bounds__(256) void k_conv(ConvArgs a)
{
    // the sequence is uniform over the workgroup: its fields are selected, not indexed,
    // so that the argument block is read with scalar loads and never copied
    const ConvSeqArgs q = blockIdx.y ? a.q[1] : a.q[0];
    if (q.reverse)
        conv_run<Ti, W, R, true>(a.s, a.len, a.act, a.nrun, q);
    else
        conv_run<Ti, W, R, false>(a.s, a.len, a.act, a.nrun, q);
}

template <typename Ti, int W>
hipError_t launch_w(const ConvArgs &a, int nseq, bool long_run, hipStream_t st)
{
    const int ch8 = (a.s.H * a.s.P + 2 * a.s.G * a.s.N) / 8;
    const int64_t threads = static_cast<int64_t>(a.s.b) * a.nrun * ch8;
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256), nseq);
    if (long_run)
        hipLaunchKernelGGL((k_conv<Ti, W, 16>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_conv<Ti, W, 4>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

int64_t conv_run_length(int64_t len) { return len > 512 ? 16 : 4; }

hipError_t launch_conv(ConvArgs a, int width, int nseq, hipStream_t st)
{
    const bool long_run = conv_run_length(a.len) == 16;
    a.nrun = static_cast<int>((a.len + conv_run_length(a.len) - 1) / conv_run_length(a.len));
    const bool bf = a.s.in_dt == 1;
    switch (width) {
    case 1: return bf ? launch_w<__bf16, 1>(a, nseq, long_run, st) : launch_w<float, 1>(a, nseq, long_run, st);
    case 2: return bf ? launch_w<__bf16, 2>(a, nseq, long_run, st) : launch_w<float, 2>(a, nseq, long_run, st);
    case 3: return bf ? launch_w<__bf16, 3>(a, nseq, long_run, st) : launch_w<float, 3>(a, nseq, long_run, st);
    default: return bf ? launch_w<__bf16, 4>(a, nseq, long_run, st) : launch_w<float, 4>(a, nseq, long_run, st);
    }
}

}  // namespace bdssm
