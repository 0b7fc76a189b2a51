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
//
// The backward pass of the same rule (the gradients of sum <dY, Y> +
// <dS_T, S_T>) is here too: the derivation with the adjoint records, the
// forward again keeping the states it needs, the adjoint scan of
// chunk_f32.h in reverse, and a chunk-parallel kernel for the gradients
// (below, "backward").
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
// BWD: also the adjoint scan's record (Tc^T Ahat, the transposed decayed
// queries and erase keys, (Aq Tc)^T) for the backward pass.
template <typename IO, int VARIANT, int DK, bool BWD>
__global__ __launch_bounds__(64) void delta_f32_derive_kernel(DeltaArgs a, ChunkRec<DK> *__restrict__ rec,
                                                              AdjRec<DK> *__restrict__ arec, unsigned int *status) {
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
        if (lane == 0) {
            rec[blockIdx.x].gc = f32x4{exp2f(gC), exp2f(gC), exp2f(gC), exp2f(gC)};
            if constexpr (BWD) arec[blockIdx.x].gc = f32x4{exp2f(gC), exp2f(gC), exp2f(gC), exp2f(gC)};
        }
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
    // Tc as a B operand (lane (g, i) step m: Tc[4g + m][i]), i.e. Tc^T as an A operand
    f32x4 tcb;
    {
        const float *tf = reinterpret_cast<const float *>(s.top);
#pragma unroll
        for (int m = 0; m < 4; ++m) tcb[m] = tf[((i >> 2) * 16 + 4 * g + m) * 4 + (i & 3)];
    }
#pragma unroll
    for (int j = 0; j < DK / 16; ++j) {
        const int col = 16 * j + i;
        // Ktil = Tc (diag(gamma) E): B operand at step m = gamma_{4g+m} E[4g + m][col]
        f32x4 k0 = zero4, k1 = zero4, ge;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float bm = gmv[m] * E[(4 * g + m) * RS + col];
            ge[m] = bm;
            if (m & 1) k1 = mfma4(tc[m], bm, k1);
            else k0 = mfma4(tc[m], bm, k0);
        }
        const f32x4 kt = k0 + k1;  // lane (g, i): Ktil[4g + r][col], the B operand of Aq Ktil
        // Qtil = diag(gamma) Q - Aq Ktil (not for the backward: its forward
        // recompute forms no output)
        f32x4 q0, q1 = zero4;
#pragma unroll
        for (int r = 0; r < 4; ++r) q0[r] = gmv[r] * s.q[(4 * g + r) * RS + col];
        if constexpr (BWD) {  // (gamma Q)^T and (gamma E)^T tiles: the same values in A-operand order
            arec[blockIdx.x].gqt[j][lane] = q0;
            arec[blockIdx.x].get[j][lane] = ge;
        } else {
            q0 = mfma4(-aqa[0], kt[0], q0);
            q1 = mfma4(-aqa[1], kt[1], q1);
            q0 = mfma4(-aqa[2], kt[2], q0);
            q1 = mfma4(-aqa[3], kt[3], q1);
        }
        const f32x4 qt = q0 + q1;
        // Ahat^T tile j, A-operand order: lane (g, i) step m holds Ahat[4g + m][col]
        f32x4 ah;
#pragma unroll
        for (int m = 0; m < 4; ++m) ah[m] = scv[m] * s.k[(4 * g + m) * RS + col];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            R.kt[(4 * g + r) * DK + col] = kt[r];
            if constexpr (!BWD) R.qt[(4 * g + r) * DK + col] = qt[r];
        }
        R.aht[j][lane] = ah;
        if constexpr (BWD) {  // Ahat' = Tc^T Ahat: A operand Tc^T, B operand Ahat (step m: Ahat[4g + m][col])
            f32x4 p0 = zero4, p1 = zero4;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (m & 1) p1 = mfma4(tcb[m], ah[m], p1);
                else p0 = mfma4(tcb[m], ah[m], p0);
            }
            const f32x4 ap = p0 + p1;
#pragma unroll
            for (int r = 0; r < 4; ++r) arec[blockIdx.x].ap[(4 * g + r) * DK + col] = ap[r];
        }
    }
    R.top[lane] = tc;
    // Aq Tc in A-operand order, as (Aq Tc)^T = Tc^T Aq^T: A operand Tc^T
    // (lane (g, i) step m: Tc[4g + m][i]), B operand Aq^T (step m: Aq[i][4g + m])
    if constexpr (!BWD) {
        f32x4 a0 = zero4, a1 = zero4;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (m & 1) a1 = mfma4(tcb[m], aqa[m], a1);
            else a0 = mfma4(tcb[m], aqa[m], a0);
        }
        R.aqt[lane] = a0 + a1;
    }
    if constexpr (BWD) {  // (Aq Tc)^T in A-operand order = Aq Tc in accumulator order: A Aq, B Tc
        f32x4 a0 = zero4, a1 = zero4;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (m & 1) a1 = mfma4(aqa[m], tcb[m], a1);
            else a0 = mfma4(aqa[m], tcb[m], a0);
        }
        arec[blockIdx.x].aqtt[lane] = a0 + a1;
    }
}

template <typename IO, int VARIANT, int DK>
hipError_t launch_kd(const DeltaArgs &a, hipStream_t stream) {
    constexpr bool kDecay = VARIANT != kDeltaNet;
    constexpr bool kGates2 = VARIANT == kGatedDeltaNet2;
    const int64_t nch = (a.T + VC - 1) / VC;
    unsigned int *status = static_cast<unsigned int *>(a.ws);
    ChunkRec<DK> *rec = reinterpret_cast<ChunkRec<DK> *>(static_cast<char *>(a.ws) + kStatusBytes);
    delta_f32_derive_kernel<IO, VARIANT, DK, false>
        <<<static_cast<unsigned>(a.B * a.H * nch), 64, 0, stream>>>(a, rec, nullptr, status);
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

// ------------------------------------------------------------ backward
// The gradients of one chunk from the chunk-start state S0, the cotangent
// G' of the state after the chunk, the residuals U and dX (from the forward
// recompute and the adjoint scan): in the residual form above, with
// Nm = strict(E K^T * Gamma), Am = lower(Q K^T * Gamma), Kc = diag(sc) K,
// sc = beta gamma_C / gamma,
//   dQ  = diag(gamma) dY S0 + dQK K,         dQK = (dY U^T * lower) diag(beta) * Gamma
//   dE  = -diag(gamma) dX S0 + dEK K,        dEK = -(dX U^T * strict) diag(beta) * Gamma
//   dK  = dEK^T E + dQK^T Q + diag(sc) U G' (+ dE, or b * dE when E = b * K)
//   dbeta_s = sum_t (dA_ts Am_ts + dL_ts Nm_ts) + dsc_s gamma_C / gamma_s,   dsc = rowsum(U G' * K)
//   d log gamma_t = rowsum(gw) - colsum(gw) + dg_t gamma_t - dsc_t sc_t
//                   (+ <G', S0> gamma_C + sum_s dsc_s sc_s at the last token),
//   gw = (dNm * E K^T + dAm * Q K^T) * Gamma,  dg = rowsum(Q * dY S0) - rowsum(E * dX S0),
// and d alpha_j = sum_{t >= j} d log gamma_t / alpha_j.  The three products
// over the value dimension and the 16 x 16 Gram blocks run on the matrix
// cores; the rest is per-element.
template <int DK, bool G2>
struct GradLds {
    static constexpr int RS = DK + 4;
    alignas(16) float q[VC * RS], k[VC * RS];
    alignas(16) float e[G2 ? VC * RS : 4];
    float ek[VC][VC + 1], qk[VC][VC + 1], dyu[VC][VC + 1], dxu[VC][VC + 1];
    float dek[VC][VC + 1], dqk[VC][VC + 1], gw[VC][VC + 1], bc[VC][VC + 1];
    float l2[VC], gm[VC], bt[VC], sc[VC];
    float pdg[4][VC], pdsc[4][VC];  // per wave: its key tiles' part of dg_t and dsc_t
    float dgc[4];
};

struct BwdWs {
    const float *s_chunks, *ds_chunks, *u, *dx;  // states per pair of chunks; U and dX per token
    const void *rec, *arec;                      // the chunk records and adjoint records
};

template <typename IO, int VARIANT, int DK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void delta_f32_grad_kernel(DeltaBwdArgs ga, BwdWs wp) {
    constexpr bool kDecay = VARIANT != kDeltaNet;
    constexpr bool kGates2 = VARIANT == kGatedDeltaNet2;
    using L = GradLds<DK, kGates2>;
    constexpr int RS = L::RS;
    __shared__ L s;
    const DeltaArgs &a = ga.f;
    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H), DV = a.dv;
    const int nch = (T + VC - 1) / VC;
    const int head = blockIdx.x / nch, c = blockIdx.x % nch;
    const int b = head / H, h = head % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int t0 = c * VC, n = min(VC, T - t0);
    const int64_t tk = (static_cast<int64_t>(b) * T + t0) * H + h;  // token index of row 0
    const float *E = kGates2 ? s.e : s.k;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    auto keep = [](bool ok, float4 x) {
        return make_float4(ok ? x.x : 0.f, ok ? x.y : 0.f, ok ? x.z : 0.f, ok ? x.w : 0.f);
    };

    // ---- the chunk's q, k (and b * k) rows, zero past the end; gates
    constexpr int Q4 = DK / 4;
    for (int e = tid; e < VC * Q4; e += 256) {
        const int t = e / Q4, j = 4 * (e % Q4);
        const int64_t gi = (tk + static_cast<int64_t>(min(t, n - 1)) * H) * DK + j;
        const bool ok = t < n;
        const float4 kv = IO::ld4(a.k, gi), qv = IO::ld4(a.q, gi);
        *reinterpret_cast<float4 *>(&s.k[t * RS + j]) = keep(ok, kv);
        *reinterpret_cast<float4 *>(&s.q[t * RS + j]) = keep(ok, qv);
        if constexpr (kGates2) {
            const float4 bv = IO::ld4(a.erase_b, gi);
            *reinterpret_cast<float4 *>(&s.e[t * RS + j]) =
                keep(ok, make_float4(kv.x * bv.x, kv.y * bv.y, kv.z * bv.z, kv.w * bv.w));
        }
    }
    if (tid < VC) {  // the same decay logarithms and scales as the derivation
        const bool ok = tid < n;
        const int64_t ti = tk + static_cast<int64_t>(min(tid, n - 1)) * H;
        float la = 0.f;
        if constexpr (kDecay) {
            const float av = IO::ld(a.alpha, ti);
            la = ok ? log2_decay(av) : 0.f;
        }
        const float gl = prefix16(la, tid);
        const float gC = __shfl(gl, VC - 1, 16);
        const float bl = IO::ld(a.beta, ti);
        const float bv = ok ? bl : 0.f;
        s.l2[tid] = gl;
        s.gm[tid] = exp2f(gl);
        s.bt[tid] = bv;
        s.sc[tid] = bv * exp2f(gC - gl);
    }
    __syncthreads();

    // ---- products over the value dimension: lane (g, i) reads row i (token
    // t0 + i, zero past the end), values 16 vt + 4g .. + 3
    // The states are kept per pair of chunks: S at the start of the even
    // chunk, G' at the end of the odd one (or of the last chunk).  An odd
    // chunk forms its S0 = gC_prev S + U_prev^T Ahat_prev from its
    // predecessor; an even chunk with a successor forms its
    // G' = gC_next G'_next + dY_next^T (gamma Q)_next - dX_next^T (gamma E)_next.
    // Both come out in the order the products below read them (lane (g, i):
    // value 4g + m of the tile, key i).
    constexpr int KT = DK / 16, MT = (KT + 3) / 4;
    const int np = (nch + 1) / 2;
    const bool odd = c & 1, from_next = !odd && c + 1 < nch;
    const float *S0 = wp.s_chunks + (static_cast<int64_t>(head) * np + (c >> 1)) * DK * DV;   // S^T rows
    const float *G1 = wp.ds_chunks + (static_cast<int64_t>(head) * np + (c >> 1)) * DK * DV;  // G'^T rows
    // B operands of the update, per key tile (odd: Ahat_prev; even: (gamma
    // Q)_next and (gamma E)_next), and its decay
    f32x4 b1[MT], b2[MT];
    float g_nb = 1.f;
    if (odd) {
        const ChunkRec<DK> &Rp = static_cast<const ChunkRec<DK> *>(wp.rec)[static_cast<int64_t>(head) * nch + c - 1];
        g_nb = Rp.gc[0];
#pragma unroll
        for (int jt = 0; jt < MT; ++jt)
            if (w + 4 * jt < KT) b1[jt] = Rp.aht[w + 4 * jt][lane];
    } else if (from_next) {
        const AdjRec<DK> &An = static_cast<const AdjRec<DK> *>(wp.arec)[static_cast<int64_t>(head) * nch + c + 1];
        g_nb = An.gc[0];
#pragma unroll
        for (int jt = 0; jt < MT; ++jt)
            if (w + 4 * jt < KT) {
                b1[jt] = An.gqt[w + 4 * jt][lane];
                b2[jt] = An.get[w + 4 * jt][lane];
            }
    }
    const int n_next = min(VC, T - t0 - VC);  // rows of the next chunk (when there is one)
    const bool rok = i < n;
    const int64_t rowi = (tk + static_cast<int64_t>(min(i, n - 1)) * H) * DV + 4 * g;
    auto row_f32 = [&](const float *base, int vt) {
        const float4 x = keep(rok, *reinterpret_cast<const float4 *>(base + rowi + 16 * vt));
        return f32x4{x.x, x.y, x.z, x.w};
    };
    auto row_dy = [&](int vt) {
        const float4 x = keep(rok, IO::ld4(ga.dout, rowi + 16 * vt));
        return f32x4{x.x, x.y, x.z, x.w};
    };
    // One pass over the value tiles, a tile's loads then its products: at
    // about 112 registers a lane four workgroups share a compute unit, and
    // their waves cover each other's load latency (holding the next tile's
    // loads in flight instead needs about 180 registers and halves that).
    // This wave's key tiles kt = w + 4 jt take dY S0, dX S0 and U G'; waves
    // 0 and 1 also take dY U^T and dX U^T from the same rows.  KIND: 0 an odd
    // chunk (S0 rebuilt from its predecessor), 1 an even chunk with a
    // successor (G' rebuilt), 2 the last chunk when it is even (both as
    // stored).
    f32x4 a1[MT], a2[MT], a3[MT];
#pragma unroll
    for (int jt = 0; jt < MT; ++jt) a1[jt] = a2[jt] = a3[jt] = zero4;
    f32x4 cc0 = zero4, cc1 = zero4;
    float dgc = 0.f;
    struct Tile {
        f32x4 yr, xr, ur, sv[MT], gv[MT];
        f32x4 a_1, a_2;  // A operands of the rebuild: lane (g, i) step m holds token 4g + m, value 16 vt + i
    };
    auto load_tile = [&](auto kind, int vt, Tile &o) {
        constexpr int K = decltype(kind)::value;
        o.yr = row_dy(vt);
        o.xr = row_f32(wp.dx, vt);
        o.ur = row_f32(wp.u, vt);
#pragma unroll
        for (int jt = 0; jt < MT; ++jt) {
            const int kt = w + 4 * jt;
            if (kt < KT) {
                const int64_t so = static_cast<int64_t>(16 * kt + i) * DV + 16 * vt + 4 * g;
                const float4 s4 = *reinterpret_cast<const float4 *>(S0 + so);
                const float4 g4 = *reinterpret_cast<const float4 *>(G1 + so);
                o.sv[jt] = f32x4{s4.x, s4.y, s4.z, s4.w};
                o.gv[jt] = f32x4{g4.x, g4.y, g4.z, g4.w};
            }
        }
        if constexpr (K == 0) {  // the previous chunk is whole
#pragma unroll
            for (int m = 0; m < 4; ++m)
                o.a_1[m] = wp.u[(tk + static_cast<int64_t>(4 * g + m - VC) * H) * DV + 16 * vt + i];
        } else if constexpr (K == 1) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 4 * g + m;
                const int64_t off = (tk + static_cast<int64_t>(VC + min(r, n_next - 1)) * H) * DV + 16 * vt + i;
                const float yv = IO::ld(ga.dout, off), xv = wp.dx[off];
                o.a_1[m] = r < n_next ? yv : 0.f;
                o.a_2[m] = r < n_next ? -xv : 0.f;
            }
        }
    };
    auto use_tile = [&](auto kind, Tile &o) {
        constexpr int K = decltype(kind)::value;
#pragma unroll
        for (int jt = 0; jt < MT; ++jt) {
            if (w + 4 * jt < KT) {
                if constexpr (K == 0) {
                    f32x4 acc = o.sv[jt] * g_nb;
#pragma unroll
                    for (int m = 0; m < 4; ++m) acc = mfma4(o.a_1[m], b1[jt][m], acc);
                    o.sv[jt] = acc;
                } else if constexpr (K == 1) {
                    f32x4 acc = o.gv[jt] * g_nb;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        acc = mfma4(o.a_1[m], b1[jt][m], acc);
                        acc = mfma4(o.a_2[m], b2[jt][m], acc);
                    }
                    o.gv[jt] = acc;
                }
            }
        }
#pragma unroll
        for (int jt = 0; jt < MT; ++jt) {
            if (w + 4 * jt < KT) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    a1[jt] = mfma4(o.yr[m], o.sv[jt][m], a1[jt]);
                    a2[jt] = mfma4(o.xr[m], o.sv[jt][m], a2[jt]);
                    a3[jt] = mfma4(o.ur[m], o.gv[jt][m], a3[jt]);
                    dgc = fmaf(o.sv[jt][m], o.gv[jt][m], dgc);
                }
            }
        }
        if (w < 2) {
            const f32x4 ar = w == 0 ? o.yr : o.xr;
            cc0 = mfma4(ar[0], o.ur[0], cc0);
            cc1 = mfma4(ar[1], o.ur[1], cc1);
            cc0 = mfma4(ar[2], o.ur[2], cc0);
            cc1 = mfma4(ar[3], o.ur[3], cc1);
        }
    };
    auto run = [&](auto kind) {
        const int nt = DV / 16;
        for (int vt = 0; vt < nt; ++vt) {
            Tile ta;
            load_tile(kind, vt, ta);
            use_tile(kind, ta);
        }
    };
    if (odd) run(icst<0>{});
    else if (from_next) run(icst<1>{});
    else run(icst<2>{});
    // this wave's part of the per-token sums over the key dimension,
    // dg_t = <Q_t, (dY S0)_t> - <E_t, (dX S0)_t> and dsc_t = <(U G')_t, K_t>
    // (zero for a wave without key tiles)
    {
        float pg[4] = {0.f, 0.f, 0.f, 0.f}, ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jt = 0; jt < MT; ++jt) {
            const int kt = w + 4 * jt;
            if (kt < KT) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int o = (4 * g + r) * RS + 16 * kt + i;
                    pg[r] = fmaf(s.q[o], a1[jt][r], pg[r]);
                    pg[r] = fmaf(-E[o], a2[jt][r], pg[r]);
                    ps[r] = fmaf(a3[jt][r], s.k[o], ps[r]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pg[r] = group_sum<16>(pg[r]);
            ps[r] = group_sum<16>(ps[r]);
        }
        if (i == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s.pdg[w][4 * g + r] = pg[r];
                s.pdsc[w][4 * g + r] = ps[r];
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dgc += __shfl_xor(dgc, off);
    if (lane == 0) s.dgc[w] = dgc;
    // ---- the 16 x 16 blocks: dY U^T (wave 0) and dX U^T (wave 1) from the
    // pass above, E K^T (wave 2) and Q K^T (wave 3) from LDS
    {
        if (w >= 2) {
            const float *X = w == 2 ? E : s.q;
#pragma unroll
            for (int q4 = 0; q4 < DK / 16; ++q4) {
                const f32x4 xr = lds4(&X[i * RS + 16 * q4 + 4 * g]);
                const f32x4 kr = lds4(&s.k[i * RS + 16 * q4 + 4 * g]);
                cc0 = mfma4(xr[0], kr[0], cc0);
                cc1 = mfma4(xr[1], kr[1], cc1);
                cc0 = mfma4(xr[2], kr[2], cc0);
                cc1 = mfma4(xr[3], kr[3], cc1);
            }
        }
        const f32x4 acc = cc0 + cc1;
        float(*dst)[VC + 1] = w == 0 ? s.dyu : w == 1 ? s.dxu : w == 2 ? s.ek : s.qk;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[4 * g + r][i] = acc[r];
    }
    __syncthreads();

    // ---- per (t, s): the adjoints through Aq and the solve
    {
        const int t = tid >> 4, u = tid & 15;
        const bool tri = u <= t, str = u < t;
        const float G = tri ? (kDecay ? exp2f(s.l2[t] - s.l2[u]) : 1.f) : 0.f;
        const float ek = s.ek[t][u], qk = s.qk[t][u];
        const float nm = str ? ek * G : 0.f, am = tri ? qk * G : 0.f;
        const float dA = tri ? s.dyu[t][u] : 0.f, dL = str ? -s.dxu[t][u] : 0.f;
        s.bc[t][u] = dA * am + dL * nm;
        const float dAm = dA * s.bt[u], dNm = dL * s.bt[u];
        s.dek[t][u] = dNm * G;
        s.dqk[t][u] = dAm * G;
        s.gw[t][u] = (dNm * ek + dAm * qk) * G;
    }
    __syncthreads();

    // ---- per token: dbeta and the decay's adjoint (wave 0, lanes 0 .. 15)
    if (tid < VC) {
        const int t = tid;
        const float dg = (s.pdg[0][t] + s.pdg[1][t]) + (s.pdg[2][t] + s.pdg[3][t]);
        const float dsc = (s.pdsc[0][t] + s.pdsc[1][t]) + (s.pdsc[2][t] + s.pdsc[3][t]);
        float dbe = 0.f;
        for (int u = 0; u < VC; ++u) dbe += s.bc[u][t];
        const float gC = s.gm[VC - 1];
        dbe = fmaf(dsc, exp2f(s.l2[VC - 1] - s.l2[t]), dbe);
        const int64_t ti = tk + static_cast<int64_t>(min(t, n - 1)) * H;
        if (t < n) ga.dbeta[ti] = dbe;
        if constexpr (kDecay) {
            // d log alpha_j = sum_{t >= j} d log gamma_t, summed in the form
            // without cancellation: the Gamma terms with both indices >= j
            // cancel (only gw_ab, a >= j > b, remain), and so do the sc terms
            // of tokens >= j against the last token's sum:
            //   sum_{a >= j, b < j} gw_ab + sum_{t >= j} dg_t gamma_t
            //   + <G', S0> gamma_C + sum_{s < j} dsc_s sc_s
            float dlog = 0.f;
            for (int aa = t; aa < VC; ++aa)
                for (int bb = 0; bb < t; ++bb) dlog += s.gw[aa][bb];
            float dgs = dg * s.gm[t];  // suffix sum over t' >= t
            float scp = dsc * s.sc[t];  // prefix sum over t' <= t, made exclusive below
            const float own = scp;
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                const float y = __shfl_down(dgs, off, 16), z = __shfl_up(scp, off, 16);
                dgs += t + off < 16 ? y : 0.f;
                scp += t >= off ? z : 0.f;
            }
            dlog += dgs + (s.dgc[0] + s.dgc[1] + s.dgc[2] + s.dgc[3]) * gC + (scp - own);
            if (t < n) ga.dalpha[ti] = dlog / IO::ld(a.alpha, ti);
        }
    }

    // ---- per (t, key): dQ, dE, dK on the matrix cores (16 x 16 by 16 x 16 per key tile)
    // (the same lanes hold the same key tile's dY S0, dX S0 and U G' rows
    // from the pass over the value tiles, so those stay in registers)
#pragma unroll
    for (int jt = 0; jt < MT; ++jt) {
        const int kt = w + 4 * jt;
        if (kt >= KT) continue;
        const int col = 16 * kt + i;
        f32x4 aq = zero4, ae = zero4, ak0 = zero4, ak1 = zero4;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int u = 4 * g + m;
            aq = mfma4(s.dqk[i][u], s.k[u * RS + col], aq);   // dQK K
            ae = mfma4(s.dek[i][u], s.k[u * RS + col], ae);   // dEK K
            ak0 = mfma4(s.dek[u][i], E[u * RS + col], ak0);   // dEK^T E
            ak1 = mfma4(s.dqk[u][i], s.q[u * RS + col], ak1); // dQK^T Q
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * g + r;
            if (t < n) {
                const int o = t * RS + col;
                const float dq = fmaf(s.gm[t], a1[jt][r], aq[r]);
                const float dE = fmaf(-s.gm[t], a2[jt][r], ae[r]);
                float dk = fmaf(s.sc[t], a3[jt][r], ak0[r] + ak1[r]);
                const int64_t gi = (tk + static_cast<int64_t>(t) * H) * DK + col;
                if constexpr (kGates2) {
                    ga.derase_b[gi] = s.k[o] * dE;
                    dk = fmaf(IO::ld(a.erase_b, gi), dE, dk);
                } else {
                    dk += dE;
                }
                ga.dq[gi] = dq;
                ga.dk[gi] = dk;
            }
        }
    }
}

template <int DK>
struct BwdLayout {
    size_t rec_off, arec_off, s_off, ds_off, u_off, dx_off, bytes;
};
template <int DK>
bool bwd_layout(const DeltaArgs &a, BwdLayout<DK> *L) {
    const int64_t nch = (a.T + VC - 1) / VC, tasks = a.B * a.H * nch;
    if (tasks > 0x7fffffff || a.B * a.H * (a.dv / 16) > 0x7fffffff) return false;
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    const size_t st = static_cast<size_t>(a.B * a.H * ((nch + 1) / 2)) * DK * a.dv * sizeof(float);  // per pair of chunks
    const size_t rows = static_cast<size_t>(a.B * a.T * a.H) * a.dv * sizeof(float);
    L->rec_off = kStatusBytes;
    L->arec_off = up(L->rec_off + static_cast<size_t>(tasks) * sizeof(ChunkRec<DK>));
    L->s_off = up(L->arec_off + static_cast<size_t>(tasks) * sizeof(AdjRec<DK>));
    L->ds_off = up(L->s_off + st);
    L->u_off = up(L->ds_off + st);
    L->dx_off = up(L->u_off + rows);
    L->bytes = L->dx_off + rows;
    return true;
}

template <typename IO, int VARIANT, int DK>
hipError_t launch_bwd_kd(const DeltaBwdArgs &g, hipStream_t stream) {
    constexpr bool kDecay = VARIANT != kDeltaNet;
    constexpr bool kGates2 = VARIANT == kGatedDeltaNet2;
    const DeltaArgs &a = g.f;
    BwdLayout<DK> L;
    if (!bwd_layout<DK>(a, &L)) return hipErrorInvalidValue;
    char *ws = static_cast<char *>(a.ws);
    const int64_t nch = (a.T + VC - 1) / VC, tasks = a.B * a.H * nch;
    unsigned int *status = reinterpret_cast<unsigned int *>(ws);
    ChunkRec<DK> *rec = reinterpret_cast<ChunkRec<DK> *>(ws + L.rec_off);
    AdjRec<DK> *arec = reinterpret_cast<AdjRec<DK> *>(ws + L.arec_off);
    float *s_chunks = reinterpret_cast<float *>(ws + L.s_off);
    float *ds_chunks = reinterpret_cast<float *>(ws + L.ds_off);
    float *u = reinterpret_cast<float *>(ws + L.u_off);
    float *dx = reinterpret_cast<float *>(ws + L.dx_off);
    const unsigned scan_grid = static_cast<unsigned>(a.B * a.H * (a.dv / 16));
    delta_f32_derive_kernel<IO, VARIANT, DK, true><<<static_cast<unsigned>(tasks), 64, 0, stream>>>(a, rec, arec, status);
    ScanArgs sa{};  // the forward again, keeping each chunk's start state and U
    sa.B = a.B;
    sa.T = a.T;
    sa.H = a.H;
    sa.dv = a.dv;
    sa.v = a.v;
    sa.w = kGates2 ? a.write_w : nullptr;
    sa.S_in = a.state_in;
    sa.side_kind = kSideNone;
    sa.s_chunks = s_chunks;
    sa.u_f32 = u;
    chunk_state_kernel<IO, DK, kDecay, kGates2, true><<<scan_grid, 64 * state_waves<DK>(), 0, stream>>>(sa, rec);
    AdjArgs aa{};
    aa.B = a.B;
    aa.T = a.T;
    aa.H = a.H;
    aa.dv = a.dv;
    aa.dy = g.dout;
    aa.v = kGates2 ? a.v : nullptr;
    aa.w = kGates2 ? a.write_w : nullptr;
    aa.dS_in = g.dstate_out;
    aa.dS_out = g.dstate_in;
    aa.ds_chunks = ds_chunks;
    aa.dx = dx;
    aa.dv_out = g.dv;
    aa.dw_out = kGates2 ? g.dwrite_w : nullptr;
    chunk_adjoint_kernel<IO, DK, kDecay, kGates2><<<scan_grid, 64 * state_waves<DK>(), 0, stream>>>(aa, arec);
    delta_f32_grad_kernel<IO, VARIANT, DK>
        <<<static_cast<unsigned>(tasks), 256, 0, stream>>>(g, BwdWs{s_chunks, ds_chunks, u, dx, rec, arec});
    return hipGetLastError();
}

template <typename IO, int VARIANT>
hipError_t launch_bwd_v(const DeltaBwdArgs &g, hipStream_t stream) {
    switch (g.f.dk) {
        case 32: return launch_bwd_kd<IO, VARIANT, 32>(g, stream);
        case 64: return launch_bwd_kd<IO, VARIANT, 64>(g, stream);
        case 96: return launch_bwd_kd<IO, VARIANT, 96>(g, stream);
        case 128: return launch_bwd_kd<IO, VARIANT, 128>(g, stream);
    }
    return hipErrorInvalidValue;
}

template <typename IO>
hipError_t launch_bwd_io(const DeltaBwdArgs &g, hipStream_t stream) {
    switch (g.f.variant) {
        case kDeltaNet: return launch_bwd_v<IO, kDeltaNet>(g, stream);
        case kGatedDeltaNet: return launch_bwd_v<IO, kGatedDeltaNet>(g, stream);
        case kGatedDeltaNet2: return launch_bwd_v<IO, kGatedDeltaNet2>(g, stream);
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

bool delta_f32_backward_workspace(const DeltaArgs &a, size_t *bytes) {
    if (!delta_f32_chunked_supported(a)) return false;
    bool ok = false;
    switch (a.dk) {
        case 32: { BwdLayout<32> L; ok = bwd_layout<32>(a, &L); *bytes = L.bytes; break; }
        case 64: { BwdLayout<64> L; ok = bwd_layout<64>(a, &L); *bytes = L.bytes; break; }
        case 96: { BwdLayout<96> L; ok = bwd_layout<96>(a, &L); *bytes = L.bytes; break; }
        case 128: { BwdLayout<128> L; ok = bwd_layout<128>(a, &L); *bytes = L.bytes; break; }
    }
    return ok;
}

hipError_t launch_delta_f32_backward(const DeltaBwdArgs &g, hipStream_t stream) {
    if (!delta_f32_chunked_supported(g.f) || g.f.T <= 0) return hipErrorNotSupported;
    return g.f.dtype == kBF16 ? launch_bwd_io<IoBF16>(g, stream) : launch_bwd_io<IoF32>(g, stream);
}

hipError_t launch_delta_f32_chunked(const DeltaArgs &a, hipStream_t stream) {
    if (!delta_f32_chunked_supported(a)) return hipErrorNotSupported;
    return a.dtype == kBF16 ? launch_io<IoBF16>(a, stream) : launch_io<IoF32>(a, stream);
}

}  // namespace lam
