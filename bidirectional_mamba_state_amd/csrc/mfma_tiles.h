// Matrix-core operand helpers shared by the bf16 kernels (gfx950, v_mfma_f32_16x16x32_bf16).
//
// Register layouts of the 16x16x32 product D = A B (+ C), lane l = 16 q + r16:
//   A: row r16, contraction indices 8q .. 8q+7 (as 8 bf16);
//   B: column r16, contraction indices 8q .. 8q+7;
//   D: rows 4q .. 4q+3, column r16 (as 4 floats).
// Any permutation of the contraction index works when both operands use it; the kernels
// use "slots 0..3 = 32m + 4q + e, slots 4..7 = 32m + 16 + 4q + e" for slice m, which is the
// row order of two stacked accumulator tiles, so that accumulators can serve as operands.
#pragma once

#include <hip/hip_runtime.h>

namespace bdssm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float bf2f(__bf16 v) { return static_cast<float>(v); }
__device__ __forceinline__ uint4 sel4(bool ok, uint4 v) { return ok ? v : make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ bf16x8 sel8(bool ok, bf16x8 v) { return ok ? v : bf16x8{}; }
__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi)
{
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// fp32 values as bf16 hi + lo parts (about 16 significant bits together): hi = bf16(f),
// lo = bf16(f - hi), both rounded to nearest even. Written on pairs so that each conversion
// instruction packs two values and the hi parts come back to float32 from the packed word
// (a shift or a mask, exact), instead of being converted a second time one by one.
__device__ __forceinline__ void split8(const float (&f)[8], bf16x8 &hi, bf16x8 &lo)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 hw, lw;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x2 v = {f[2 * k], f[2 * k + 1]};
        const uint32_t p = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
        const f32x2 r = {f[2 * k] - __uint_as_float(p << 16), f[2 * k + 1] - __uint_as_float(p & 0xffff0000u)};
        hw[k] = p;
        lw[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
    }
    hi = __builtin_bit_cast(bf16x8, hw);
    lo = __builtin_bit_cast(bf16x8, lw);
}

// eight floats as bf16 (round to nearest even), converted two per instruction
__device__ __forceinline__ bf16x8 to_bf16x8(const float (&f)[8])
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{f[2 * k], f[2 * k + 1]}), bf16x2));
    return __builtin_bit_cast(bf16x8, w);
}

// Slot permutation of x tiles (token-major rows of 64 bf16 = 128 bytes, two rows per
// 256-byte LDS bank period): the 16-byte piece c of row t sits at slot c ^ swz_x(t). gfx950's
// LDS serves an 8-byte read 32 lanes at a time, and this keeps both of the kernels' 8-byte x
// reads free of bank conflicts: transposing reads of 8 consecutive rows x 32 bytes
// (distinct piece pairs among the even rows and among the odd ones) and reads of 16
// consecutive rows x 16 bytes (distinct pieces among the 8 even rows and among the 8 odd
// ones). Rows t and t + 16 share a permutation.
__device__ __forceinline__ int swz_x(int t) { return 2 * ((t >> 1) & 3) + ((t >> 3) & 1); }

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): in each 16-lane group, lanes 4r .. 4r+3
// address row r (four consecutive elements each) and lane j receives column j of the four
// rows.
__device__ __forceinline__ bf16x4 tr_read(const __bf16 *p)
{
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// Fragment-major LDS tiles. A tile of R rows (a multiple of 16) x K columns is cut into
// 8-byte pieces (4 columns); the piece holding columns c .. c+3 of row r lives in the
// 512-byte region of (16-row block r/16, 32-column slice c/32, 16-column half (c/16)%2), at
// slot 16 q + (r%16 ^ 4q) with q = (c/4)%4. An operand fragment (lane (r16, q): row
// 16 blk + r16, columns 32m + 4q + e and 32m + 16 + 4q + e) is then two contiguous 512-byte
// reads, and a transposing read (4 rows x 16 columns per 16 lanes) touches 16 distinct
// 8-byte bank slots. (Measured on gfx950: contiguous 8-byte reads run at about 100 B/clk
// per CU, row-strided ones at about 60.)
template <int K>
__device__ __forceinline__ int f8_off(int r, int c)  // in bf16 elements; c a multiple of 4
{
    const int blk = r >> 4, r16 = r & 15, m = c >> 5, hf = (c >> 4) & 1, q = (c >> 2) & 3;
    return ((((blk * (K / 32) + m) * 2 + hf) * 64) + 16 * q + (r16 ^ (4 * q))) * 4;
}

// Operand fragment with the contraction along rows 16 blk + r16 of a tile: columns
// 32m + 4q + e (slots e = 0..3) and 32m + 16 + 4q + e (slots 4..7).
template <int K>
__device__ __forceinline__ bf16x8 frag(const __bf16 *T, int blk, int m, int q, int r16)
{
    const __bf16 *p = T + f8_off<K>(16 * blk + r16, 32 * m + 4 * q);
    return cat(*reinterpret_cast<const bf16x4 *>(p), *reinterpret_cast<const bf16x4 *>(p + 256));
}

// Operand fragment with the contraction over rows of a tile: lane (r16, q) gets column
// col0 + r16 of rows row0 + 4q + e (slots e = 0..3) and row0 + 16 + 4q + e (slots 4..7).
// row0 and col0: multiples of 16.
template <int K>
__device__ __forceinline__ bf16x8 tr_frag(const __bf16 *T, int row0, int col0, int q, int r16)
{
    const __bf16 *p = T + f8_off<K>(row0 + 4 * q + (r16 >> 2), col0 + 4 * (r16 & 3));
    return cat(tr_read(p), tr_read(p + (K / 32) * 2 * 64 * 4));  // the next 16-row block
}

// A 16-byte piece of row r (columns c .. c+7, c a multiple of 8) into a fragment-major tile
template <int K>
__device__ __forceinline__ void put16(__bf16 *T, int r, int c, uint4 v)
{
    *reinterpret_cast<uint2 *>(T + f8_off<K>(r, c)) = make_uint2(v.x, v.y);
    *reinterpret_cast<uint2 *>(T + f8_off<K>(r, c + 4)) = make_uint2(v.z, v.w);
}

}  // namespace bdssm
