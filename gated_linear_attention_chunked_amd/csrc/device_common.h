// device_common.h -- small device helpers shared by the gfx950 kernels:
// storage-dtype loads/stores, lane reductions and the XCD-aware block map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lam {

// ---------------------------------------------------------------- storage
// bf16 is carried as its raw 16-bit pattern; widening is exact.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
// Round to nearest, ties to even; NaN stays NaN (quiet bit forced).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

struct IoF32 {
    using T = float;
    static __device__ __forceinline__ float ld(const void *p, int64_t i) {
        return static_cast<const float *>(p)[i];
    }
    static __device__ __forceinline__ void st(void *p, int64_t i, float x) {
        static_cast<float *>(p)[i] = x;
    }
    // elements i .. i + 3 (i a multiple of 4 in a 16-byte aligned tensor)
    static __device__ __forceinline__ float4 ld4(const void *p, int64_t i) {
        return *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
    }
};
struct IoBF16 {
    using T = uint16_t;
    static __device__ __forceinline__ float ld(const void *p, int64_t i) {
        return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    }
    static __device__ __forceinline__ void st(void *p, int64_t i, float x) {
        static_cast<uint16_t *>(p)[i] = f32_to_bf16_bits(x);
    }
    // elements i .. i + 3 (i a multiple of 4 in an 8-byte aligned tensor)
    static __device__ __forceinline__ float4 ld4(const void *p, int64_t i) {
        const uint2 x = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i);
        return make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                           __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u));
    }
};

// log2 of a decay, floored at -200 so a zero decay (log2 = -inf) becomes a
// finite full erase; a NaN decay stays NaN (fmaxf would drop it) and so
// propagates through the chain as it does token by token.
__device__ __forceinline__ float log2_decay(float alpha) {
    const float l = __builtin_amdgcn_logf(alpha);
    return l != l ? l : fmaxf(l, -200.f);
}

// ------------------------------------------------------------- reductions
// Sum over aligned groups of W lanes (W in {1, 2, 4, 8, 16, 64}); every lane
// of the group receives the group's sum.  Within a 16-lane row the partial
// sums move by DPP (quad swaps, then the 8- and 16-lane mirrors), which stay
// in the vector ALU; a whole-wave sum then adds the four row sums read out
// with readlane.  Each step adds a lane and its partner in both orders, so
// every lane of a group ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int W>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 64, "group width");
    if constexpr (W >= 2) x += dpp_mov<0xb1>(x);   // quad_perm [1,0,3,2]: partner lane ^ 1
    if constexpr (W >= 4) x += dpp_mov<0x4e>(x);   // quad_perm [2,3,0,1]: partner lane ^ 2
    if constexpr (W >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror: lane 7 - i of the 8
    if constexpr (W >= 16) x += dpp_mov<0x140>(x); // row_mirror: lane 15 - i of the row
    if constexpr (W == 64) {
        const int xi = __float_as_int(x);
        x = (__int_as_float(__builtin_amdgcn_readlane(xi, 0)) + __int_as_float(__builtin_amdgcn_readlane(xi, 16))) +
            (__int_as_float(__builtin_amdgcn_readlane(xi, 32)) + __int_as_float(__builtin_amdgcn_readlane(xi, 48)));
    }
    return x;
}

// --------------------------------------------------------------- mapping
// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X, so ids
// congruent mod 8 share an XCD (and its L2).  Given `groups` groups of `per`
// workgroups that read the same data, return (group, member) such that all
// members of a group land on one XCD.  Falls back to the plain order when the
// group count is not a multiple of 8.
__device__ __forceinline__ void xcd_group_map(int bid, int groups, int per, int &group,
                                              int &member) {
    if ((groups & 7) == 0) {
        const int xcd = bid & 7, local = bid >> 3;
        group = (local / per) * 8 + xcd;
        member = local % per;
    } else {
        group = bid / per;
        member = bid % per;
    }
}

}  // namespace lam
