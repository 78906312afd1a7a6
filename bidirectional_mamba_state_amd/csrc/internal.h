// Internal declarations shared by the host library and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bdssm {

struct Shape {
    int b, H, P, N, G;
    int in_dt, y_dt;  // 0 = float32, 1 = bfloat16
};

struct Seq {
    const void *x, *dt, *B, *C;
};

// Forward recurrence over segments of one token range (prefix chunks, or a commit block).
// Segment c of stream b covers tokens [c*Q, min(len, (c+1)*Q)).
struct ForwardArgs {
    Shape s;
    int64_t len;          // tokens per stream in `in`
    int Q;                // segment length
    int nseg;             // ceil(len / Q)
    Seq in;
    const float *A, *D;
    const float *first_state;  // state entering segment 0, [b][H][N][P]; NULL = zero
    const float *prev_states;  // state entering segment c>0 = prev_states[b][c-1][h]; NULL = zero
    void *y;                   // [b][len][H][P] in s.y_dt, with D x; NULL = no output
    float *state_out;          // final state of each segment, [b][nseg][H][N][P]; NULL = none
    float *decay_out;          // sum over the segment of dt*A, [b][nseg][H]; NULL = none
    int rev = 0;               // scan token len-1-t at position t, and add the outputs to y
                               // (D may then be NULL: no skip term)
};

// Inter-chunk state passing: h_c = exp(decay_c) h_{c-1} + local_c, in place over `states`.
struct PassArgs {
    Shape s;
    int nch;
    const float *h_init;   // NULL = zero
    float *states;         // [b][nch][H][N][P]: chunk-local states in, chunk states out
    const float *decay;    // [b][nch][H]
    int write_all;         // write every chunk state back (else only the final one)
    float *h_out;          // [b][H][N][P] or NULL
};

struct BlockArgs {
    Shape s;
    int T;
    const float *h_prefix;
    Seq fwd, rev;
    const float *A, *D;
    void *y;
    const float *A_rev;  // decay of the reverse scan (A when the directions share it)
    const float *D_rev;  // skip term of the reverse input, or NULL for none
    const void *h_ops;   // the cached state in operand form (launch_state_ops), read instead
                         // of h_prefix when not NULL
    int ops_hi_only = 0;    // h_ops holds only the hi parts: the bf16 cached state
                            // [b][H][N/8][P][8] (launch_state_bf16)
    int d_per_channel = 0;  // D and D_rev are [H][P] skip weights instead of [H]
};

// Depthwise convolution of one token segment's x, B, C channels (see conv.hip)
struct ConvSeqArgs {
    const void *x, *B, *C;  // raw inputs
    void *ox, *oB, *oC;     // convolved outputs (same layouts and dtype)
    const float *w;         // [CH][W] taps, CH = H*P + 2*G*N
    const float *bias;      // [CH] or NULL
    const void *state_in;   // [b][W-1][CH] history before the segment, or NULL (zeros); forward only
    void *state_out;        // [b][W-1][CH] new history, or NULL; forward only
    int reverse;            // 0 causal, 1 anti-causal with zeros past the end
};

struct ConvArgs {
    Shape s;
    int64_t len;
    int act;   // 0 identity, 1 SiLU
    int nrun;  // token runs per channel group (set by launch_conv)
    ConvSeqArgs q[2];
};

struct PrefixPlan {
    int seg_sub;       // 64-token sub-chunks per segment
    int nseg;          // segments per stream
    int hpw_state;     // heads per workgroup of the state-only pass (1, 2 or 4)
    size_t tot_bytes;  // workspace bytes for segment decays (256-byte rounded)
    size_t ws_bytes;   // total workspace bytes (0 for a single segment)
};

int device_cus();  // compute units of the current device (cached)
bool valu_supported(int N, int P);
bool prefix_mfma_supported(const Shape &s, int chunk);
// full: y or chunk states are wanted; single_segment: one segment per (stream, head), no
// workspace (used by commits)
PrefixPlan prefix_mfma_plan(const Shape &s, int64_t len, int chunk, bool full, bool single_segment = false);
// rev: scan from the last token to the first and add the outputs to y (y required, no chunk
// states; h_out may be NULL when y is given); D may then be NULL (no skip term)
// enc (single segment, state only): h_out also written encoded for the block step, as the
// operand form or (enc_hi_only) the bf16 state
hipError_t run_prefix_mfma(const Shape &s, int64_t len, int chunk, const Seq &in, const float *A,
                           const float *D, const float *h_init, void *y, float *chunk_states,
                           float *h_out, void *ws, hipStream_t st, bool single_segment = false,
                           bool rev = false, void *enc = nullptr, bool enc_hi_only = false);
bool block_mfma_supported(const Shape &s, int T);
void block_mfma_plan(const Shape &s, int *hpw, int *ps);
hipError_t launch_block_step_mfma(const BlockArgs &a, int hpw, int ps, hipStream_t st);
bool block_lat_supported(const Shape &s, int T);
hipError_t launch_block_step_lat(const BlockArgs &a, int wpg, hipStream_t st);  // wpg 2, 4 or 0 (chosen)
// many (stream, head) pairs, state in operand form (a.h_ops): hpw heads per workgroup
bool block_bw_supported(const Shape &s, int T);
int block_bw_plan(const Shape &s);
hipError_t launch_block_step_bw(const BlockArgs &a, int hpw, hipStream_t st);
// Operand form of nbh cached states [nbh][N][P] float32 (N = 128, P = 64): the bf16 pair
// hi = bf16(S), lo = bf16(S - hi) as [nbh][2][N/8][P][8]
hipError_t launch_state_ops(const float *h, void *ops, int64_t nbh, hipStream_t st);
// bf16 copy of nbh cached states [nbh][N][P] float32 (N % 8 == 0): bf16(S) rounded to nearest
// even, as [nbh][N/8][P][8] (the hi part of the operand form)
hipError_t launch_state_bf16(const float *h, void *out, int64_t nbh, int N, int P, hipStream_t st);
hipError_t launch_forward_valu(const ForwardArgs &a, hipStream_t st);
hipError_t launch_block_step_valu(const BlockArgs &a, hipStream_t st);
hipError_t launch_state_pass(const PassArgs &a, hipStream_t st);
hipError_t launch_conv(ConvArgs a, int width, int nseq, hipStream_t st);
hipError_t launch_copy_f32(float *dst, const float *src, int64_t n, hipStream_t st);
hipError_t launch_fill_f32(float *dst, float v, int64_t n, hipStream_t st);

}  // namespace bdssm
