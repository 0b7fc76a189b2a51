// chunk_common.h -- device helpers shared by the chunked kernels: bf16 MFMA
// fragments and their LDS reads, DPP lane moves, LDS-only synchronisation.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace lam {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4 bf4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A or B operand of a 16x16x32 product from a row-major bf16 LDS matrix:
// rows r0..r0+15, reduction columns c0..c0+31 taken in accumulator order
// (c0 + 4g .. +3 and c0 + 16 + 4g .. +3 for lane group g), read as two
// independent 8-byte LDS loads.  The loads are volatile, so the compiler keeps them as single ds_read_b64 with
// immediate offsets instead of fusing the pair into ds_read2_b64: on gfx950 a
// conflict-free ds_read_b64 takes about 2 cycles, while ds_read2_b64 of the
// same bytes takes 7.5 (14.8 at these row strides).
typedef __attribute__((address_space(3))) volatile const bf16x4 vlds_bf16x4_t;
__device__ __forceinline__ bf16x8 row_frag2(const __bf16 *m, int stride, int r0, int c0, int lane) {
    const auto p = reinterpret_cast<__attribute__((address_space(3))) const __bf16 *>(
        (__attribute__((address_space(3))) const void *)(m + (r0 + (lane & 15)) * stride + c0 + 4 * (lane >> 4)));
    return cat8(*reinterpret_cast<vlds_bf16x4_t *>(p), *reinterpret_cast<vlds_bf16x4_t *>(p + 16));
}
// Column gather with the gfx950 LDS transpose read.  Within each 16-lane
// group g, lane m supplies the 8-byte piece m[r0 + 4g + m/4][c0 + 4(m%4) ..]
// and lane i receives m[r0 + 4g + j][c0 + i] in slot j = 0..3: four
// consecutive rows of one column, i.e. the accumulator-order operand of a
// reduction over rows, read from a row-major tile.
__device__ __forceinline__ bf16x4 col_gather4(const __bf16 *m, int stride, int r0, int c0, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const __bf16 *p = m + (r0 + 4 * g + (i >> 2)) * stride + c0 + 4 * (i & 3);
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}
// A operand of a 16x16x32 product contracting over rows r0..r0+31 of a
// row-major tile, for output rows = columns c0..c0+15 (accumulator order).
__device__ __forceinline__ bf16x8 col_frag(const __bf16 *m, int stride, int r0, int c0, int lane) {
    return cat8(col_gather4(m, stride, r0, c0, lane), col_gather4(m, stride, r0 + 16, c0, lane));
}
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that orders LDS only: outstanding global loads (the
// producers' prefetch) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (fixed order of additions, so it is bitwise reproducible).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_shift(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp_shift<0x111, 0xf>(x);  // row_shr:1
    x += dpp_shift<0x112, 0xf>(x);  // row_shr:2
    x += dpp_shift<0x114, 0xf>(x);  // row_shr:4
    x += dpp_shift<0x118, 0xf>(x);  // row_shr:8
    x += dpp_shift<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_shift<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}
// Value of lane N of this lane's quad (DPP quad_perm [N, N, N, N]).
template <int N>
__device__ __forceinline__ float quad_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), N * 0x55, 0xf, 0xf, false));
}
template <int I>
using ic = std::integral_constant<int, I>;
// Calls f(ic<I>) for I = 0 .. N-1.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &f) {
    if constexpr (I < N) {
        f(ic<I>{});
        static_for<N, I + 1>(f);
    }
}

// Order this wave's LDS writes before its later LDS reads of other lanes'
// data.  A wave's LDS instructions complete in issue order, so this only
// stops the compiler from moving accesses across it.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
}
// Publish: make this wave's LDS writes visible, then count one arrival.
__device__ __forceinline__ void lds_arrive(unsigned int *cnt, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Bounded wait until `*cnt` reaches `target`.  Every wave leaves the loop
// after at most 2^22 polls, so a lost arrival can never hang the kernel; a
// wave that runs out ORs LAM_DEVICE_WAIT_TIMEOUT (bit 0) into the call's
// device status word (word 0 of the workspace) with a vector atomic, so the
// host can tell that this call's outputs are not to be trusted.
__device__ __forceinline__ void lds_wait(unsigned int *cnt, unsigned int target, unsigned int *status) {
    for (int it = 0; it < (1 << 22); ++it) {
        if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace lam
