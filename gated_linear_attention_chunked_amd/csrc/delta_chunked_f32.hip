// delta_chunked_f32.hip -- fp32 chunked scan of the delta-rule family
// (DeltaNet, Gated DeltaNet, Gated DeltaNet-2) on gfx950 fp32 matrix cores,
// for fp32 storage and for the head sizes the bf16 schedule does not take.
//
// The rule ("Mechanisms, trade-offs and cross-layer routing of
// linear-attention architectures", "Technical details"): W_t = a_t W_{t-1} +
// beta_t r_t k_t^T with r_t = z_t - a_t W_{t-1} e_t and y_t = W_t q_t (e = k,
// z = v except for Gated DeltaNet-2's erase/write gates; a = 1 for DeltaNet).
// Over a chunk of VC = 16 tokens (rows = tokens, S = memory at the chunk
// start, g_t = sum_{j<=t} log2 a_j, gamma_t = 2^{g_t}, Gamma_ts = 2^{g_t - g_s}
// for s <= t), the residuals R of the chunk satisfy
//   R = (I + N diag(beta))^{-1} (Z - diag(gamma) E S^T),  N = strict(E K^T * Gamma),
//   Y = diag(gamma) Q S^T + lower(Q K^T * Gamma) diag(beta) R,
//   S' = gamma_C S + R^T diag(beta gamma_C / gamma) K,
// the same residual form as the bf16 chunked schedule.  With
// Tc = (I + N diag(beta))^{-1} and Aq = lower(Q K^T * Gamma) diag(beta) it is
// the state step of chunk_f32.h:
//   U = R = Tc Z - Ktil S^T,      Ktil = Tc diag(gamma) E,
//   Y = Qtil S^T + (Aq Tc) Z,     Qtil = diag(gamma) Q - Aq Ktil,
//   S^T <- gamma_C S^T + Ahat^T U, Ahat = diag(beta gamma_C / gamma) K.
// Every exponent is a difference g_t - g_s with s <= t (or g_C - g_t), so no
// factor exceeds one.  Nothing here crosses chunks, so the derivation runs
// for every chunk at once; the state kernel then walks the chunks.
#include "chunk_f32.h"

namespace lam {
namespace {

template <int DK, bool GATES2>
struct DeriveF32Lds {
    static constexpr int RS = DK + 4;  // row stride of the token-row tiles
    alignas(16) float k[VC * RS], q[VC * RS];
    alignas(16) float e[GATES2 ? VC * RS : 4];  // erase-gated keys b * k (Gated DeltaNet-2)
    alignas(16) float lt[VC * VLTS];  // N diag(beta), strictly lower, by column
    alignas(16) float am[VC][VC + 1]; // Aq, row-major
    alignas(16) f32x4 top[64];        // Tc, A-operand order
    float g[VC], gm[VC], sc[VC], bt[VC];
};

// Inclusive prefix sum over lanes 0..15 of a 16-lane group (every group does
// its own; fixed order of additions).
__device__ __forceinline__ float prefix16(float x, int i) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
        const float y = __shfl_up(x, off, 16);
        x += i >= off ? y : 0.f;
    }
    return x;
}

// One wave per (b, h, chunk of 16 tokens): the chunk record for the state
// kernel.  Lane (g, i): g = lane / 16, i = lane % 16.
template <typename IO, int VARIANT, int DK>
__global__ __launch_bounds__(64) void delta_f32_derive_kernel(DeltaArgs a, ChunkRec<DK> *__restrict__ rec,
                                                              unsigned int *status) {
    constexpr bool kDecay = VARIANT != kDeltaNet;
    constexpr bool kGates2 = VARIANT == kGatedDeltaNet2;
    using L = DeriveF32Lds<DK, kGates2>;
    constexpr int RS = L::RS;
    __shared__ L s;
    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H);
    const int nch = (T + VC - 1) / VC;
    const int head = blockIdx.x / nch, c = blockIdx.x % nch;
    const int b = head / H, h = head % H;
    const int lane = threadIdx.x, g = lane >> 4, i = lane & 15;
    const int t0 = c * VC, n = min(VC, T - t0);
    if (blockIdx.x == 0 && lane == 0) *status = 0u;  // first kernel of the call
    const float *E = kGates2 ? s.e : s.k;

    // ---- token rows (past the end: zero) and gates (past the end: no decay, beta 0)
    const int64_t tk = (static_cast<int64_t>(b) * T + t0) * H + h;  // token index of row 0
    // Four elements a lane per load, every load issued before the first wait;
    // loads read clamped rows inside the sequence, padding rows are zeroed.
    constexpr int Q4 = DK / 4, NL = VC * Q4 / 64;  // 4-element groups per row, per lane
    float4 kr[NL], qr[NL], br[kGates2 ? NL : 1];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
        const int e = lane + 64 * u, t = e / Q4, j = 4 * (e % Q4);
        const int64_t gi = (tk + static_cast<int64_t>(min(t, n - 1)) * H) * DK + j;
        kr[u] = IO::ld4(a.k, gi);
        qr[u] = IO::ld4(a.q, gi);
        if constexpr (kGates2) br[u] = IO::ld4(a.erase_b, gi);
    }
    if (lane < VC) {
        const bool ok = lane < n;
        const int64_t ti = tk + static_cast<int64_t>(min(lane, n - 1)) * H;
        float la = 0.f;
        if constexpr (kDecay) {
            const float av = IO::ld(a.alpha, ti);
            la = ok ? log2_decay(av) : 0.f;
        }
        const float gl = prefix16(la, lane);
        const float gC = __shfl(gl, VC - 1, 16);
        const float bl = IO::ld(a.beta, ti);
        const float bv = ok ? bl : 0.f;
        s.g[lane] = gl;
        s.gm[lane] = exp2f(gl);
        s.bt[lane] = bv;
        s.sc[lane] = bv * exp2f(gC - gl);
        if (lane == 0) rec[blockIdx.x].gc = f32x4{exp2f(gC), exp2f(gC), exp2f(gC), exp2f(gC)};
    }
    // (selected component by component: a select of whole vectors becomes a
    // select of their addresses in private memory)
    auto keep = [](bool ok, float4 x) {
        return make_float4(ok ? x.x : 0.f, ok ? x.y : 0.f, ok ? x.z : 0.f, ok ? x.w : 0.f);
    };
#pragma unroll
    for (int u = 0; u < NL; ++u) {
        const int e = lane + 64 * u, t = e / Q4, j = 4 * (e % Q4);
        const bool ok = t < n;
        *reinterpret_cast<float4 *>(&s.k[t * RS + j]) = keep(ok, kr[u]);
        *reinterpret_cast<float4 *>(&s.q[t * RS + j]) = keep(ok, qr[u]);
        if constexpr (kGates2) {
            const float4 ke = make_float4(kr[u].x * br[u].x, kr[u].y * br[u].y, kr[u].z * br[u].z, kr[u].w * br[u].w);
            *reinterpret_cast<float4 *>(&s.e[t * RS + j]) = keep(ok, ke);
        }
    }
    __syncthreads();

    // ---- E K^T and Q K^T (lane (g, i): [t = 4g + r][s = i]), two chains each
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 ek2[2] = {zero4, zero4}, qk2[2] = {zero4, zero4};
#pragma unroll
    for (int q4 = 0; q4 < DK / 16; ++q4) {
        const f32x4 er = lds4(&E[i * RS + 16 * q4 + 4 * g]);
        const f32x4 qr = lds4(&s.q[i * RS + 16 * q4 + 4 * g]);
        const f32x4 kr = lds4(&s.k[i * RS + 16 * q4 + 4 * g]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            ek2[m & 1] = mfma4(er[m], kr[m], ek2[m & 1]);
            qk2[m & 1] = mfma4(qr[m], kr[m], qk2[m & 1]);
        }
    }
    const f32x4 ek = ek2[0] + ek2[1], qk = qk2[0] + qk2[1];
    // N diag(beta) (strict) by column s = i, and Aq (s <= t) row-major
    {
        const float gs = s.g[i], bs = s.bt[i];
        f32x4 nl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * g + r;
            const float dec = kDecay ? exp2f(fminf(s.g[t] - gs, 0.f)) : 1.f;
            nl[r] = i < t ? ek[r] * dec * bs : 0.f;
            s.am[t][i] = i <= t ? qk[r] * dec * bs : 0.f;
        }
        *reinterpret_cast<f32x4 *>(&s.lt[i * VLTS + 4 * g]) = nl;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    unit_lower_inverse(s.lt, s.top, lane);  // Tc = (I + N diag(beta))^{-1}
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    ChunkRec<DK> &R = rec[blockIdx.x];
    const f32x4 tc = s.top[lane];  // A-operand order: Tc[i][4g + m]
    f32x4 aqa;                     // Aq in A-operand order: Aq[i][4g + m]
#pragma unroll
    for (int m = 0; m < 4; ++m) aqa[m] = s.am[i][4 * g + m];
    f32x4 gmv, scv;  // gamma and beta gamma_C / gamma of tokens 4g + m
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        gmv[m] = s.gm[4 * g + m];
        scv[m] = s.sc[4 * g + m];
    }
#pragma unroll
    for (int j = 0; j < DK / 16; ++j) {
        const int col = 16 * j + i;
        // Ktil = Tc (diag(gamma) E): B operand at step m = gamma_{4g+m} E[4g + m][col]
        f32x4 k0 = zero4, k1 = zero4;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float bm = gmv[m] * E[(4 * g + m) * RS + col];
            if (m & 1) k1 = mfma4(tc[m], bm, k1);
            else k0 = mfma4(tc[m], bm, k0);
        }
        const f32x4 kt = k0 + k1;  // lane (g, i): Ktil[4g + r][col], the B operand of Aq Ktil
        // Qtil = diag(gamma) Q - Aq Ktil
        f32x4 q0, q1 = zero4;
#pragma unroll
        for (int r = 0; r < 4; ++r) q0[r] = gmv[r] * s.q[(4 * g + r) * RS + col];
        q0 = mfma4(-aqa[0], kt[0], q0);
        q1 = mfma4(-aqa[1], kt[1], q1);
        q0 = mfma4(-aqa[2], kt[2], q0);
        q1 = mfma4(-aqa[3], kt[3], q1);
        const f32x4 qt = q0 + q1;
        // Ahat^T tile j, A-operand order: lane (g, i) step m holds Ahat[4g + m][col]
        f32x4 ah;
#pragma unroll
        for (int m = 0; m < 4; ++m) ah[m] = scv[m] * s.k[(4 * g + m) * RS + col];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            R.kt[(4 * g + r) * DK + col] = kt[r];
            R.qt[(4 * g + r) * DK + col] = qt[r];
        }
        R.aht[j][lane] = ah;
    }
    R.top[lane] = tc;
    // Aq Tc in A-operand order, as (Aq Tc)^T = Tc^T Aq^T: A operand Tc^T
    // (lane (g, i) step m: Tc[4g + m][i]), B operand Aq^T (step m: Aq[i][4g + m])
    {
        const float *tf = reinterpret_cast<const float *>(s.top);
        f32x4 a0 = zero4, a1 = zero4;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float tcm = tf[((i >> 2) * 16 + 4 * g + m) * 4 + (i & 3)];
            if (m & 1) a1 = mfma4(tcm, aqa[m], a1);
            else a0 = mfma4(tcm, aqa[m], a0);
        }
        R.aqt[lane] = a0 + a1;
    }
}

template <typename IO, int VARIANT, int DK>
hipError_t launch_kd(const DeltaArgs &a, hipStream_t stream) {
    constexpr bool kDecay = VARIANT != kDeltaNet;
    constexpr bool kGates2 = VARIANT == kGatedDeltaNet2;
    const int64_t nch = (a.T + VC - 1) / VC;
    unsigned int *status = static_cast<unsigned int *>(a.ws);
    ChunkRec<DK> *rec = reinterpret_cast<ChunkRec<DK> *>(static_cast<char *>(a.ws) + kStatusBytes);
    delta_f32_derive_kernel<IO, VARIANT, DK><<<static_cast<unsigned>(a.B * a.H * nch), 64, 0, stream>>>(a, rec, status);
    ScanArgs sa{};
    sa.B = a.B;
    sa.T = a.T;
    sa.H = a.H;
    sa.dv = a.dv;
    sa.v = a.v;
    sa.w = kGates2 ? a.write_w : nullptr;
    sa.out = a.out;
    sa.S_in = a.state_in;
    sa.S_out = a.state_out;
    sa.side = a.side;
    sa.side_kind = a.side ? a.side_kind : kSideNone;
    chunk_state_kernel<IO, DK, kDecay, kGates2>
        <<<static_cast<unsigned>(a.B * a.H * (a.dv / 16)), 64 * state_waves<DK>(), 0, stream>>>(sa, rec);
    return hipGetLastError();
}

template <typename IO, int VARIANT>
hipError_t launch_v(const DeltaArgs &a, hipStream_t stream) {
    switch (a.dk) {
        case 32: return launch_kd<IO, VARIANT, 32>(a, stream);
        case 64: return launch_kd<IO, VARIANT, 64>(a, stream);
        case 96: return launch_kd<IO, VARIANT, 96>(a, stream);
        case 128: return launch_kd<IO, VARIANT, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <typename IO>
hipError_t launch_io(const DeltaArgs &a, hipStream_t stream) {
    switch (a.variant) {
        case kDeltaNet: return launch_v<IO, kDeltaNet>(a, stream);
        case kGatedDeltaNet: return launch_v<IO, kGatedDeltaNet>(a, stream);
        case kGatedDeltaNet2: return launch_v<IO, kGatedDeltaNet2>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int DK>
size_t rec_bytes() { return sizeof(ChunkRec<DK>); }

}  // namespace

bool delta_f32_chunked_supported(const DeltaArgs &a) {
    return a.variant != kKimiDelta && (a.dk == 32 || a.dk == 64 || a.dk == 96 || a.dk == 128) && a.dv % 16 == 0 &&
           a.dv > 0;
}

bool delta_f32_chunked_workspace(const DeltaArgs &a, size_t *bytes) {
    size_t per;
    switch (a.dk) {
        case 32: per = rec_bytes<32>(); break;
        case 64: per = rec_bytes<64>(); break;
        case 96: per = rec_bytes<96>(); break;
        case 128: per = rec_bytes<128>(); break;
        default: return false;
    }
    const int64_t tasks = a.B * a.H * ((a.T + VC - 1) / VC);
    if (tasks > 0x7fffffff || a.B * a.H * (a.dv / 16) > 0x7fffffff) return false;
    *bytes = kStatusBytes + static_cast<size_t>(tasks) * per;
    return true;
}

hipError_t launch_delta_f32_chunked(const DeltaArgs &a, hipStream_t stream) {
    if (!delta_f32_chunked_supported(a)) return hipErrorNotSupported;
    return a.dtype == kBF16 ? launch_io<IoBF16>(a, stream) : launch_io<IoF32>(a, stream);
}

}  // namespace lam
