// delta_step.hip -- one-token decode step of the delta-rule family for many
// concurrent streams, memory updated in place.
//
// The rule ("Mechanisms, trade-offs and cross-layer routing of
// linear-attention architectures", "Technical details"), for one token of
// one (stream, head): the memory is decayed (scalar alpha, or per key channel
// for Kimi Delta), the residual of the decayed memory's prediction is written
// along k scaled by beta, and the query reads the updated memory.  The
// streaming, fixed-size state is what makes decoding need no cache of past
// tokens ("Technical summary: Variational Linear Attention (VLA)", section 5).
//
// With a per-column decay d (alpha, alpha_c or 1), read key e (k, or b * k for
// Gated DeltaNet-2) and target z (v, or w * v), each row W_i of the memory
// takes, in one pass over it:
//   p = sum_c W_ic d_c e_c,  o = sum_c W_ic d_c q_c,  r = z_i - p,
//   y_i = o + beta r (k . q),  W_ic <- d_c W_ic + beta r k_c,
// which is the rule with y read after the write (y = W_new q).
//
// The step moves the whole state twice (read and write, fp32) and touches
// each token input once, so it is bound by HBM.  One wave owns 8 rows of one
// (stream, head): each row is dk/4 lanes x one float4 (32 lanes at dk = 128,
// so a load instruction covers 2 rows; 16 or 8 lanes at dk = 64 or 32), and
// the row sums reduce within those lanes (DPP inside 16-lane rows, then one
// swizzle across two of them at dk = 128).  dk = 96 takes the token-recurrent
// kernel.
#include "device_common.h"
#include "lam_internal.h"

namespace lam {
namespace {

constexpr int kStepWaves = 4;   // waves per workgroup
constexpr int kStepRows = 8;    // memory rows per wave

template <int VARIANT, typename IO, int DK>
__global__ __launch_bounds__(64 * kStepWaves) void delta_step_kernel(DeltaArgs a) {
    constexpr int LPR = DK / 4;           // lanes per row (one float4 each)
    constexpr int RPI = 64 / LPR;         // rows per load instruction
    constexpr int NI = kStepRows / RPI;   // load instructions per wave
    constexpr bool kChan = VARIANT == kKimiDelta;
    constexpr bool kScalar = VARIANT == kGatedDeltaNet || VARIANT == kGatedDeltaNet2;
    constexpr bool kGates2 = VARIANT == kGatedDeltaNet2;
    static_assert(LPR <= 32 && 64 % LPR == 0, "row layout");

    const int H = static_cast<int>(a.H), dv = a.dv;
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * kStepWaves + (threadIdx.x >> 6);
    const int wpr = dv / kStepRows;  // waves per (stream, head)
    const int64_t head = wave / wpr;  // n * H + h
    if (head >= a.B * a.H) return;
    const int r0 = (wave % wpr) * kStepRows;
    const int sub = lane / LPR, cl = lane % LPR;  // row within an instruction, float4 column
    const int c0 = 4 * cl;

    // token inputs of this (stream, head): [N, H, dk] and [N, H, dv]
    const int64_t kbase = head * DK + c0;
    float kk[4], qq[4], ee[4], dd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        kk[j] = IO::ld(a.k, kbase + j);
        qq[j] = IO::ld(a.q, kbase + j);
        ee[j] = kGates2 ? kk[j] * IO::ld(a.erase_b, kbase + j) : kk[j];
        dd[j] = 1.f;
    }
    if constexpr (kChan) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dd[j] = IO::ld(a.alpha, kbase + j);
    }
    if constexpr (kScalar) {
        const float al = IO::ld(a.alpha, head);
#pragma unroll
        for (int j = 0; j < 4; ++j) dd[j] = al;
    }
    const float beta = IO::ld(a.beta, head);
    // k . q over the whole key: the LPR lanes of each row hold all of it once
    float kq = kk[0] * qq[0] + kk[1] * qq[1] + kk[2] * qq[2] + kk[3] * qq[3];
    auto row_sum = [&](float x) {  // sum over the LPR lanes of a row
        if constexpr (LPR <= 16) {
            x = group_sum<LPR>(x);
        } else {
            x = group_sum<16>(x);
            x += __shfl_xor(x, 16, 64);
        }
        return x;
    };
    kq = row_sum(kq);

    float *Wp = a.state_out;  // in place: state_in == state_out
    const float *Win = a.state_in;
#pragma unroll
    for (int it = 0; it < NI; ++it) {
        const int row = r0 + RPI * it + sub;
        const int64_t wo = (head * dv + row) * DK + c0;
        float4 w4 = Win ? *reinterpret_cast<const float4 *>(Win + wo) : make_float4(0.f, 0.f, 0.f, 0.f);
        float w[4] = {w4.x, w4.y, w4.z, w4.w};
        float p = 0.f, o = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float wd = w[j] * dd[j];
            p = fmaf(wd, ee[j], p);
            o = fmaf(wd, qq[j], o);
        }
        p = row_sum(p);
        o = row_sum(o);
        const int64_t vo = head * dv + row;
        float z = IO::ld(a.v, vo);
        if constexpr (kGates2) z *= IO::ld(a.write_w, vo);
        const float br = beta * (z - p);
        if (cl == 0) IO::st(a.out, vo, fmaf(br, kq, o));
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = fmaf(br, kk[j], w[j] * dd[j]);
        if (Wp) *reinterpret_cast<float4 *>(Wp + wo) = make_float4(w[0], w[1], w[2], w[3]);
    }
}

template <int VARIANT, typename IO>
hipError_t launch_var_io(const DeltaArgs &a, hipStream_t stream) {
    const int64_t waves = a.B * a.H * (a.dv / kStepRows);
    const unsigned blocks = static_cast<unsigned>((waves + kStepWaves - 1) / kStepWaves);
    switch (a.dk) {
        case 32: delta_step_kernel<VARIANT, IO, 32><<<blocks, 64 * kStepWaves, 0, stream>>>(a); break;
        case 64: delta_step_kernel<VARIANT, IO, 64><<<blocks, 64 * kStepWaves, 0, stream>>>(a); break;
        case 128: delta_step_kernel<VARIANT, IO, 128><<<blocks, 64 * kStepWaves, 0, stream>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_io(const DeltaArgs &a, hipStream_t stream) {
    switch (a.variant) {
        case kDeltaNet: return launch_var_io<kDeltaNet, IO>(a, stream);
        case kGatedDeltaNet: return launch_var_io<kGatedDeltaNet, IO>(a, stream);
        case kKimiDelta: return launch_var_io<kKimiDelta, IO>(a, stream);
        case kGatedDeltaNet2: return launch_var_io<kGatedDeltaNet2, IO>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool delta_step_supported(const DeltaArgs &a) {
    return (a.dk == 32 || a.dk == 64 || a.dk == 128) && a.dv % kStepRows == 0;
}

hipError_t launch_delta_step(const DeltaArgs &a, hipStream_t stream) {
    if (!delta_step_supported(a)) return hipErrorNotSupported;
    return a.dtype == kBF16 ? launch_io<IoBF16>(a, stream) : launch_io<IoF32>(a, stream);
}

}  // namespace lam
