// Wavefront-level helpers shared by the gfx950 kernels: 64-lane scans by DPP moves,
// range-checked buffer resources, copies from global memory straight into LDS, and a
// workgroup barrier that does not wait for those copies.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace bdssm {

typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float wave_dpp_move(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}

// inclusive sum over the 64 lanes: shifts by 1, 2, 4, 8 inside rows of 16 lanes, then the
// last lane of each row is added to the rows after it
__device__ __forceinline__ float wave_prefix_sum(float v)
{
    v += wave_dpp_move<0x111, 0xf>(v);
    v += wave_dpp_move<0x112, 0xf>(v);
    v += wave_dpp_move<0x114, 0xf>(v);
    v += wave_dpp_move<0x118, 0xf>(v);
    v += wave_dpp_move<0x142, 0xa>(v);
    v += wave_dpp_move<0x143, 0xc>(v);
    return v;
}

__device__ __forceinline__ float wave_lane(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// raw buffer over [base, base + bytes) with range checking: loads past the end return zero,
// stores past it are dropped (bytes < 2^31)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_range(const void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// Copies 1 KB of global memory into LDS without passing through registers (gfx950 buffer
// load to LDS): lane l's 16 bytes from byte offset `off` land at dst + 16 l.
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t r, void *dst, int off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, off, 0, 0, 0);
}

// Workgroup barrier over LDS: waits until at most INFLIGHT of this wavefront's vector
// memory operations are outstanding (INFLIGHT = 63: no wait) and its LDS accesses are done,
// then synchronizes. A memory fence here would also wait for every copy into LDS.
template <int INFLIGHT>
__device__ __forceinline__ void workgroup_lds_barrier()
{
    static_assert(INFLIGHT >= 0 && INFLIGHT < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    // vmcnt(INFLIGHT) (bits 3:0 and 15:14), expcnt unchanged (7), lgkmcnt(0)
    __builtin_amdgcn_s_waitcnt((INFLIGHT & 15) | ((INFLIGHT >> 4) << 14) | 0x0070);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace bdssm
