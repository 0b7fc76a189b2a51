// vla_chunked.hip -- chunked VLA scan on gfx950 fp32 matrix cores.
//
// The rules ("Technical summary: Variational Linear Attention (VLA)",
// sections 2.2-2.3): per token the inverse penalty takes a rank-1
// Sherman-Morrison downdate A <- A - z z^T / (1 + p.z) with z = A p, the gate
// is the unit vector along A khat, and the state writes its residual along
// the gate, S <- S + (v - S khat) alphahat^T; keys and queries pass through
// ELU+1 and unit normalisation; y = S qhat.
//
// Chunked form over C = 16 tokens (rows = tokens; A, S at the chunk start):
//   Pa = P A^T, KA = Khat A^T, F = Z X^T with X = [P; Khat] (16 x 32):
//     F_t = (Pa X^T)_t - sum_{s<t} c_ts F_s,  c_ts = F_s[p_t] / D_s,
//     D_t = 1 + F_t[p_t]                     (z_t = A_{t-1} p_t, D_t = 1 + p_t.z_t)
//   Z = (I + C)^{-1} Pa,  N = KA - E Z with E_ts = F_s[khat_t] / D_s (s <= t),
//   alphahat_t = N_t / |N_t|,  A <- A - Z^T D^{-1} Z,
//   U = (I + strict(Khat Ahat^T))^{-1} (V - Khat S^T),
//   Y = Qhat S^T + lower(Qhat Ahat^T) U,  S <- S + U^T Ahat.
// The sequential part is the 16-step recurrence for F (one wave, lanes over
// its 32 columns) and two 16x16 unit-lower inverses; everything else is
// 16x16x4 fp32 MFMA products.
//
// Schedule: one workgroup of D/16 waves per (b, h) chain.  Wave w keeps
// column tile w of A^T and of S^T as fp32 accumulator tiles in registers,
// so every product against the state and every state update is local to
// the wave; chunk tiles move between waves through LDS, one barrier per
// phase.
#include "device_common.h"
#include "lam_internal.h"

namespace lam {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int VC = 16;    // chunk length
constexpr int VLTS = 20;  // column stride (floats) of a 16x16 matrix stored by column

// fp32 16x16x4 product.  Operand layout (lane = 16 g + i): A supplies row i,
// column g; B supplies row g, column i; the accumulator holds rows 4g..4g+3 of
// column i.  Contractions over 16 run as four steps with k = 4g + m at step
// m, so each lane's operands for the four steps are four consecutive floats.
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 lds4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
template <int I>
struct icst {
    static constexpr int value = I;
};
// f(icst<0>) ... f(icst<14>)
template <int I = 0, typename F>
__device__ __forceinline__ void static_for15(F &f) {
    if constexpr (I < 15) {
        f(icst<I>{});
        static_for15<I + 1>(f);
    }
}
__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }

template <int D>
struct VlaLds {
    static constexpr int DS = D + 4;  // row stride of the token-row tiles
    static constexpr int TS = VC + 4; // row stride of the transposed tiles
    // token-row tiles, double-buffered: chunk c is consumed while chunk c + 1
    // is staged and its features are computed
    alignas(16) float p[2][VC * DS], kh[2][VC * DS], qh[2][VC * DS], v[2][VC * DS];
    alignas(16) float pa[VC * DS];      // P A^T
    alignas(16) float ah[VC * DS];      // alphahat rows
    alignas(16) float zt[D * TS];       // Z^T
    alignas(16) float at[D * TS];       // alphahat^T
    alignas(16) float g0t[2 * VC * TS]; // (Pa X^T)^T: column c of Pa X^T as a row
    alignas(16) float e[VC * TS];       // E, rows t
    alignas(16) float lt[VC * VLTS];    // strictly lower matrix by column (C, then strict(Khat Ahat^T))
    alignas(16) f32x4 wop[64];          // (I + C)^{-1}, A-operand order
    alignas(16) f32x4 top[64];          // (I + strict(Khat Ahat^T))^{-1}, A-operand order
    alignas(16) f32x4 aq[64];           // lower(Qhat Ahat^T), A-operand order
    alignas(16) float rd[VC];           // 1 / D_t
    alignas(16) float part[D / 16][VC]; // per-wave partial |N_t|^2
};

// Value of lane N of this lane's quad (DPP quad_perm [N, N, N, N]).
template <int N>
__device__ __forceinline__ float quad_lane(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), N * 0x55, 0xf, 0xf, false));
}

// (I + L)^{-1} for strictly lower L given by columns, written in A-operand
// order (element (row, col) at out[(col / 4) * 16 + row][col % 4]).  One wave:
// lane = (col = lane / 4, row quad q = lane % 4), forward substitution in
// fp32; X[j][col] comes from the quad by DPP, and the columns of L, which do
// not depend on X, are read two steps ahead.
__device__ __forceinline__ void unit_lower_inverse(const float *lt, f32x4 *out, int lane) {
    const int col = lane >> 2, q = lane & 3;
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (4 * q + r == col) ? 1.f : 0.f;
    f32x4 lw[3];
    lw[0] = lds4(lt + 4 * q);
    lw[1] = lds4(lt + VLTS + 4 * q);
    auto step = [&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if constexpr (j + 2 < 15) lw[(j + 2) % 3] = lds4(lt + (j + 2) * VLTS + 4 * q);
        const f32x4 lj = lw[j % 3];                  // L[4q + r][j]
        const float xj = quad_lane<j / 4>(x[j % 4]);  // X[j][col]
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = fmaf(-lj[r], xj, x[r]);
    };
    static_for15(step);
    float *o = reinterpret_cast<float *>(out);
#pragma unroll
    for (int r = 0; r < 4; ++r) o[((col >> 2) * 16 + 4 * q + r) * 4 + (col & 3)] = x[r];
}

template <typename IO, int D>
__global__ __launch_bounds__(64 * (D / 16)) void vla_chunked_kernel(VlaArgs a) {
    constexpr int NW = D / 16, NT = 64 * NW, NQ = D / 16;
    constexpr int DS = VlaLds<D>::DS, TS = VlaLds<D>::TS;
    __shared__ VlaLds<D> s;

    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H);
    const int b = blockIdx.x / H, h = blockIdx.x % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int64_t sb = (static_cast<int64_t>(b) * H + h) * D * D;
    const int col = 16 * w + i;  // this lane's column of the wave's tiles

    // A^T and S^T column tile w: AT[q] = A^T[16q + 4g + r][col] = A[col][16q + 4g + r]
    f32x4 AT[NQ], ST[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if (a.A_in) {
            const float4 x = *reinterpret_cast<const float4 *>(a.A_in + sb + static_cast<int64_t>(col) * D + 16 * q + 4 * g);
            AT[q] = f32x4{x.x, x.y, x.z, x.w};
        } else {
            f32x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = (16 * q + 4 * g + r == col) ? 1.f : 0.f;
            AT[q] = x;
        }
    }
    if (a.S_in) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const float4 x = *reinterpret_cast<const float4 *>(a.S_in + sb + static_cast<int64_t>(col) * D + 16 * q + 4 * g);
            ST[q] = f32x4{x.x, x.y, x.z, x.w};
        }
    } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q) ST[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // raw inputs of one chunk staged in registers: element e = tid + NT * u of
    // each 16 x D tile (token e / D, channel e % D)
    constexpr int EPT = VC * D / NT;  // = 4
    float rq[EPT], rk[EPT], rv[EPT], rp[EPT];
    auto tok = [&](int t) { return ((static_cast<int64_t>(b) * T + t) * H + h) * D; };
    // this thread's elements sit at fixed offsets from the chunk's first row
    uint32_t eoff[EPT];
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
        const int e = tid + NT * u;
        eoff[u] = static_cast<uint32_t>((e / D) * H * D + e % D);
    }
    auto fetch = [&](int c0) {  // past the end: the last chunk again (never used)
        const int cc = min(c0, ((T - 1) / VC) * VC);
        const int n = min(VC, T - cc);
        const int64_t base = tok(cc);
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = tid + NT * u, t = e / D;
            // rows past the end reread the last row (never used)
            const uint32_t o = t < n ? eoff[u] : static_cast<uint32_t>((n - 1) * H * D + e % D);
            rq[u] = IO::ld(a.q, base + o);
            rk[u] = IO::ld(a.k, base + o);
            rv[u] = IO::ld(a.v, base + o);
            rp[u] = IO::ld(a.p, base + o);
        }
    };
    // staged registers into buffer bi (rows past n: p = v = 0, features zeroed)
    auto stage = [&](int bi, int n) {
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = tid + NT * u, t = e / D, j = e % D;
            const bool ok = t < n;
            s.p[bi][t * DS + j] = ok ? rp[u] : 0.f;
            s.v[bi][t * DS + j] = ok ? rv[u] : 0.f;
            s.kh[bi][t * DS + j] = rk[u];
            s.qh[bi][t * DS + j] = rq[u];
        }
    };
    // khat, qhat = unit(ELU(x) + 1) in place in buffer bi, zero past row n.
    // NWF waves share the rows (this wave is the wi-th: rows wi, wi + NWF, ...),
    // all of its rows at once.
    auto features = [&](auto nwf, int bi, int n, int wi) {
        constexpr int NWF = decltype(nwf)::value;
        constexpr int PER = (D + 63) / 64, RPW = (VC + NWF - 1) / NWF;
        float *KH = s.kh[bi], *QH = s.qh[bi];
        float fk[RPW][PER], fq[RPW][PER], ssk[RPW], ssq[RPW];
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
            const int t = wi + NWF * rr;
            ssk[rr] = ssq[rr] = 0.f;
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                // read a valid element unconditionally and mask the value,
                // so the reads of all rows go out together
                const int j = lane + 64 * u;
                const float okf = (t < VC && j < D) ? 1.f : 0.f;
                const int o = min(t, VC - 1) * DS + min(j, D - 1);
                fk[rr][u] = elu1(KH[o]) * okf;
                fq[rr][u] = elu1(QH[o]) * okf;
                ssk[rr] = fmaf(fk[rr][u], fk[rr][u], ssk[rr]);
                ssq[rr] = fmaf(fq[rr][u], fq[rr][u], ssq[rr]);
            }
        }
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
            ssk[rr] = group_sum<64>(ssk[rr]);
            ssq[rr] = group_sum<64>(ssq[rr]);
        }
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
            const int t = wi + NWF * rr;
            const float ik = t < n ? __builtin_amdgcn_rsqf(ssk[rr]) : 0.f;
            const float iq = t < n ? __builtin_amdgcn_rsqf(ssq[rr]) : 0.f;
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int j = lane + 64 * u;
                if (t < VC && j < D) {
                    KH[t * DS + j] = fk[rr][u] * ik;
                    QH[t * DS + j] = fq[rr][u] * iq;
                }
            }
        }
    };
    if (T > 0) {
        fetch(0);
        stage(0, min(VC, T));
        fetch(VC);
        __syncthreads();
        features(icst<NW>{}, 0, min(VC, T), w);
    }

    for (int c0 = 0; c0 < T; c0 += VC) {
        const int n = min(VC, T - c0), n1 = min(VC, T - c0 - VC);  // rows of this chunk, of the next
        const int cb = (c0 / VC) & 1, nb = cb ^ 1;
        const float *P = s.p[cb], *KH = s.kh[cb], *QH = s.qh[cb], *V = s.v[cb];
        // ---- stage chunk c + 1 into the other buffer, refill the registers
        stage(nb, n1);
        fetch(c0 + 2 * VC);
        __syncthreads();
        // ---- products against the chunk-start state (tile w of each):
        // Pa = P A^T, KA = Khat A^T, KS = Khat S^T, QS = Qhat S^T
        f32x4 pa = {0.f, 0.f, 0.f, 0.f}, ka = pa, ks = pa, qs = pa;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const f32x4 pr = lds4(&P[i * DS + 16 * q + 4 * g]);
            const f32x4 kr = lds4(&KH[i * DS + 16 * q + 4 * g]);
            const f32x4 qr = lds4(&QH[i * DS + 16 * q + 4 * g]);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                pa = mfma4(pr[m], AT[q][m], pa);
                ka = mfma4(kr[m], AT[q][m], ka);
                ks = mfma4(kr[m], ST[q][m], ks);
                qs = mfma4(qr[m], ST[q][m], qs);
            }
        }
        // R = V - Khat S^T (tile w, accumulator order)
        f32x4 rr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            rr[r] = V[(4 * g + r) * DS + col] - ks[r];
            s.pa[(4 * g + r) * DS + col] = pa[r];
        }
        __syncthreads();
        // ---- Pa X^T (16 x 32), waves 0 and 1: column c of it stored as row c of g0t
        if (w < 2) {
            const float *xs = w == 0 ? P : KH;
            f32x4 g0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 ar = lds4(&s.pa[i * DS + 16 * q + 4 * g]);
                const f32x4 br = lds4(&xs[i * DS + 16 * q + 4 * g]);
#pragma unroll
                for (int m = 0; m < 4; ++m) g0 = mfma4(ar[m], br[m], g0);
            }
            // g0 lane (g, i): (Pa X^T)[t = 4g + r][16w + i]
            *reinterpret_cast<f32x4 *>(&s.g0t[(16 * w + i) * TS + 4 * g]) = g0;
        }
        __syncthreads();
        // ---- wave 0: the recurrence for F, then Z's coefficients inverted
        if (w == 0) {
            // lane c < 32 keeps column c of F: F[s] = F_s[c]
            const int c = lane & 31;
            float gcol[VC], F[VC], rdv[VC];
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                const f32x4 x = lds4(&s.g0t[c * TS + 4 * t4]);
#pragma unroll
                for (int r = 0; r < 4; ++r) gcol[4 * t4 + r] = x[r];
            }
#pragma unroll
            for (int t = 0; t < VC; ++t) {
                // c_ts = F_s[p_t] / D_s: column t of row s, held by lane t;
                // four partial sums keep the chain short
                float acc[4] = {gcol[t], 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < t; ++s2) {
                    const float cts = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(F[s2]), t)) * rdv[s2];
                    acc[s2 & 3] = fmaf(-cts, F[s2], acc[s2 & 3]);
                }
                const float f = (acc[0] + acc[1]) + (acc[2] + acc[3]);
                F[t] = f;
                const float dt = 1.f + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), t));
                rdv[t] = __builtin_amdgcn_rcpf(dt);
            }
            // C (strictly lower, by column s): C_ts = F_s[t] / D_s, lanes t < 16
            // E (rows t): E_ts = F_s[16 + t] / D_s for s <= t, lanes 16 + t
            if (lane < VC) {
#pragma unroll
                for (int s2 = 0; s2 < VC; ++s2) s.lt[s2 * VLTS + lane] = s2 < lane ? F[s2] * rdv[s2] : 0.f;
            } else if (lane < 2 * VC) {
                const int t = lane - VC;
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    f32x4 x;
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[r] = 4 * s4 + r <= t ? F[4 * s4 + r] * rdv[4 * s4 + r] : 0.f;
                    *reinterpret_cast<f32x4 *>(&s.e[t * TS + 4 * s4]) = x;
                }
            }
            if (lane < VC) s.rd[lane] = rdv[lane];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            unit_lower_inverse(s.lt, s.wop, lane);
        } else {
            // meanwhile the other waves map the features of chunk c + 1
            features(icst<NW - 1>{}, nb, n1, w - 1);
        }
        __syncthreads();
        // ---- Z = (I + C)^{-1} Pa, N = KA - E Z (tile w); Z^T to LDS; |N_t|^2 partials
        f32x4 z = {0.f, 0.f, 0.f, 0.f}, nn = ka;
        {
            const f32x4 wa = s.wop[lane];
            const f32x4 ea = lds4(&s.e[i * TS + 4 * g]);
#pragma unroll
            for (int m = 0; m < 4; ++m) z = mfma4(wa[m], pa[m], z);
#pragma unroll
            for (int m = 0; m < 4; ++m) nn = mfma4(-ea[m], z[m], nn);
        }
        *reinterpret_cast<f32x4 *>(&s.zt[col * TS + 4 * g]) = z;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float sq = group_sum<16>(nn[r] * nn[r]);
            if (i == 0) s.part[w][4 * g + r] = sq;
        }
        __syncthreads();
        // ---- alphahat (tile w) to LDS by rows and by columns; A^T -= Z^T D^{-1} Z
        f32x4 ah;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * g + r;
            float ss = 0.f;
#pragma unroll
            for (int u = 0; u < NW; ++u) ss += s.part[u][t];
            ah[r] = nn[r] * (t < n ? __builtin_amdgcn_rsqf(ss) : 0.f);
            s.ah[t * DS + col] = ah[r];
        }
        *reinterpret_cast<f32x4 *>(&s.at[col * TS + 4 * g]) = ah;
        {
            const f32x4 rd4 = lds4(&s.rd[4 * g]);
            f32x4 zd;
#pragma unroll
            for (int r = 0; r < 4; ++r) zd[r] = -z[r] * rd4[r];
            // B operand at step m: (D^{-1} Z)[4g + m][col] -- held by lane (g, i) as zd[m]
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 za = lds4(&s.zt[(16 * q + i) * TS + 4 * g]);
#pragma unroll
                for (int m = 0; m < 4; ++m) AT[q] = mfma4(za[m], zd[m], AT[q]);
            }
        }
        __syncthreads();
        // ---- wave 0: strict(Khat Ahat^T) by column, inverted; wave 1: lower(Qhat Ahat^T)
        if (w == 0) {
            f32x4 km = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 kr = lds4(&KH[i * DS + 16 * q + 4 * g]);
                const f32x4 ar = lds4(&s.ah[i * DS + 16 * q + 4 * g]);
#pragma unroll
                for (int m = 0; m < 4; ++m) km = mfma4(kr[m], ar[m], km);
            }
            // km lane (g, i): (Khat Ahat^T)[t = 4g + r][s = i]; column s = i of the strict part
            f32x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = i < 4 * g + r ? km[r] : 0.f;
            *reinterpret_cast<f32x4 *>(&s.lt[i * VLTS + 4 * g]) = x;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            unit_lower_inverse(s.lt, s.top, lane);
        } else if (w == 1) {
            f32x4 aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 ar = lds4(&s.ah[i * DS + 16 * q + 4 * g]);
                const f32x4 qr = lds4(&QH[i * DS + 16 * q + 4 * g]);
#pragma unroll
                for (int m = 0; m < 4; ++m) aq = mfma4(ar[m], qr[m], aq);
            }
            // aq lane (g, i): (Ahat Qhat^T)[s = 4g + r][t = i] = (Qhat Ahat^T)[t = i][s = 4g + r]:
            // already the A operand of Y = Aq U; keep s <= t
#pragma unroll
            for (int r = 0; r < 4; ++r) aq[r] = 4 * g + r <= i ? aq[r] : 0.f;
            s.aq[lane] = aq;
        }
        __syncthreads();
        // ---- U = (I + strict(Khat Ahat^T))^{-1} R, Y = QS + Aq U, S^T += Ahat^T U (tile w)
        {
            const f32x4 ta = s.top[lane], qa = s.aq[lane];
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) u = mfma4(ta[m], rr[m], u);
            f32x4 y = qs;
#pragma unroll
            for (int m = 0; m < 4; ++m) y = mfma4(qa[m], u[m], y);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g + r;
                if (t < n) IO::st(a.out, tok(c0 + t) + col, y[r]);
            }
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 aa = lds4(&s.at[(16 * q + i) * TS + 4 * g]);
#pragma unroll
                for (int m = 0; m < 4; ++m) ST[q] = mfma4(aa[m], u[m], ST[q]);
            }
        }
        __syncthreads();  // chunk tiles free for the next chunk
    }

#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if (a.A_out)
            *reinterpret_cast<float4 *>(a.A_out + sb + static_cast<int64_t>(col) * D + 16 * q + 4 * g) =
                make_float4(AT[q][0], AT[q][1], AT[q][2], AT[q][3]);
        if (a.S_out)
            *reinterpret_cast<float4 *>(a.S_out + sb + static_cast<int64_t>(col) * D + 16 * q + 4 * g) =
                make_float4(ST[q][0], ST[q][1], ST[q][2], ST[q][3]);
    }
}

template <typename IO, int D>
hipError_t launch_d(const VlaArgs &a, hipStream_t stream) {
    const unsigned blocks = static_cast<unsigned>(a.B * a.H);
    vla_chunked_kernel<IO, D><<<dim3(blocks), dim3(64 * (D / 16)), 0, stream>>>(a);
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_io(const VlaArgs &a, hipStream_t stream) {
    switch (a.d) {
        case 32: return launch_d<IO, 32>(a, stream);
        case 64: return launch_d<IO, 64>(a, stream);
        case 96: return launch_d<IO, 96>(a, stream);
        case 128: return launch_d<IO, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool vla_chunked_supported(const VlaArgs &a) {
    return a.d == 32 || a.d == 64 || a.d == 96 || a.d == 128;
}

// The single-kernel schedule keeps every intermediate in LDS and registers.
bool vla_chunked_workspace(const VlaArgs &, size_t *bytes) {
    *bytes = 0;
    return true;
}

hipError_t launch_vla_chunked(const VlaArgs &a, hipStream_t stream) {
    if (!vla_chunked_supported(a)) return hipErrorNotSupported;
    return a.dtype == kBF16 ? launch_io<IoBF16>(a, stream) : launch_io<IoF32>(a, stream);
}

}  // namespace lam
